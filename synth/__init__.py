"""Seeded synthetic workloads shared by the oracle tests, the GPU tests,
``smoke()`` and ``bench.py``.

This module only draws random numbers and names shapes, formats and seeds; it
holds none of the method's arithmetic (no rotation, codebook, quantization or
attention).  Both the HIP path and the oracle receive exactly these arrays.

Every cache stream (batch row b, KV head h, tensor K or V) is drawn from its
own ``numpy`` generator keyed by (workload seed, tensor, b, h), so any stream
can be regenerated alone at any size -- the full-size tests sample a few
streams without drawing the rest.

Workloads (the pages measure only on real models and corpora; these seeded
inputs with the same shapes stand in for them):

c1  single head, d = 128, 512 keys/values, rows N(0, I) rescaled to an L2
    norm drawn from U[0.8, 1.2]; 4-bit PQ4 keys and values; seed 0.
c2  turbo3 (PQ3) keys and values; B = 1, 32 query / 8 KV heads, d = 128,
    context 4096; N(0, 1) entries times a per-channel scale exp(U[ln 0.5,
    ln 2]) drawn per (tensor, KV head, channel); seed 1.
c3  TQ3K keys (2-bit MSE + 1-bit QJL) with GQ2V values; B = 1, 40 / 8
    heads, d = 128, context 30,000; N(0, 1) entries; seed 2.
c4  PQ4 keys and values, B = 8, 32 / 8 heads, d = 128, context 65,536
    (65,535 prefilled plus one token appended per decode step); N(0, 1)
    entries with 10 (KV head, channel) pairs per tensor -- 1% of the
    8 x 128 channels -- scaled by 8; seed 3.
c5  d = 256 PQ4: bulk compression of 131,072 tokens x 4 KV heads, then
    decode with B = 32, 16 / 2 heads, context 8,192, the same bytes viewed
    as [32][2][8192]; entries Student-t with 4 degrees of freedom divided by
    sqrt(d * 4 / 2) so that E|x|^2 = 1; seed 4.

Queries: q ~ N(0, I) * c_h with c_h = 2 sqrt(d) / sqrt(E|k|^2) for the KV
head h the query head reads, so that the exact logits q.k/sqrt(d) have a
standard deviation near 2 (a non-trivial softmax).
"""

from dataclasses import dataclass, field, replace

import numpy as np

PQ4, PQ3, TQ3K, GQ2V, GQ4V = 1, 2, 3, 4, 5
QUANTILE_MEAN, LLOYD_MAX = 0, 1
K_TENSOR, V_TENSOR, Q_TENSOR, APPEND = 0, 1, 2, 3


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    context: int
    capacity: int
    k_format: int
    v_format: int
    k_bits: int
    v_bits: int
    k_kind: int
    v_kind: int
    seed: int
    dist: str
    rot_seed_k: int = 0
    rot_seed_v: int = 0
    qjl_seed: int = 0
    prefill: int = 0  # tokens written before the decode steps (c4: context - 1)
    extra: dict = field(default_factory=dict)

    @property
    def group(self):
        return self.n_q_heads // self.n_kv_heads


def _seeds(seed):
    return dict(rot_seed_k=1000 + seed, rot_seed_v=2000 + seed, qjl_seed=3000 + seed)


C1 = Workload("c1", 1, 1, 1, 128, 512, 512, PQ4, PQ4, 4, 4, QUANTILE_MEAN, QUANTILE_MEAN, 0, "unit_norm_gaussian",
              prefill=512, **_seeds(0))
C2 = Workload("c2", 1, 32, 8, 128, 4096, 4096, PQ3, PQ3, 3, 3, QUANTILE_MEAN, QUANTILE_MEAN, 1, "channel_scaled",
              prefill=4096, **_seeds(1))
C3 = Workload("c3", 1, 40, 8, 128, 30000, 30016, TQ3K, GQ2V, 2, 2, LLOYD_MAX, LLOYD_MAX, 2, "gaussian",
              prefill=30000, **_seeds(2))
C4 = Workload("c4", 8, 32, 8, 128, 65536, 65536, PQ4, PQ4, 4, 4, QUANTILE_MEAN, QUANTILE_MEAN, 3, "outlier_channels",
              prefill=65535, **_seeds(3))
C5 = Workload("c5", 32, 16, 2, 256, 8192, 8192, PQ4, PQ4, 4, 4, QUANTILE_MEAN, QUANTILE_MEAN, 4, "student_t4",
              prefill=8192, extra={"prefill_tokens": 131072, "prefill_kv_heads": 4}, **_seeds(4))

WORKLOADS = {w.name: w for w in (C1, C2, C3, C4, C5)}


def scaled(w, **changes):
    """The same workload (distribution, formats, seeds) at other sizes."""
    return replace(w, **changes)


def _rng(w, *key):
    return np.random.default_rng([w.seed, *key])


def _channel_scale(w, tensor, h):
    """Per-channel standard deviation of stream (tensor, h), float64 [d]."""
    d = w.head_dim
    if w.dist == "channel_scaled":
        r = _rng(w, 100 + tensor, h)
        return np.exp(r.uniform(np.log(0.5), np.log(2.0), size=d))
    if w.dist == "outlier_channels":
        r = _rng(w, 200 + tensor)
        pick = r.choice(w.n_kv_heads * d, size=int(round(0.01 * w.n_kv_heads * d)), replace=False)
        sc = np.ones(w.n_kv_heads * d)
        sc[pick] = 8.0
        return sc.reshape(w.n_kv_heads, d)[h]
    if w.dist == "student_t4":
        return np.full(d, 1.0 / np.sqrt(2.0 * d))  # variance of t_4 is 2
    return np.ones(d)


def stream(w, tensor, b, h, start, count):
    """fp16 rows [count, d] of tokens start..start+count-1 of one cache stream.

    Rows of one stream are drawn in blocks of 4096 tokens from generators
    keyed by the block number, so any token range can be drawn alone.
    """
    d = w.head_dim
    out = np.empty((count, d), dtype=np.float16)
    sc = _channel_scale(w, tensor, h).astype(np.float32)
    blk = 4096
    t = start
    while t < start + count:
        bi = t // blk
        lo = bi * blk
        r = _rng(w, tensor, b, h, bi)
        if w.dist == "student_t4":
            x = r.standard_t(4, size=(blk, d)).astype(np.float32)
        else:
            x = r.standard_normal(size=(blk, d), dtype=np.float32)
        if w.dist == "unit_norm_gaussian":
            nrm = np.linalg.norm(x.astype(np.float64), axis=1)
            target = r.uniform(0.8, 1.2, size=blk)
            x = (x.astype(np.float64) * (target / nrm)[:, None]).astype(np.float32)
        else:
            x = x * sc[None, :]
        a, e = t - lo, min(start + count, lo + blk) - lo
        out[t - start:t - start + (e - a)] = x[a:e].astype(np.float16)
        t = lo + e
    return out


def appended(w, tensor, b, h, step):
    """fp16 row [d] appended to stream (b, h) at decode step ``step``."""
    r = _rng(w, APPEND, tensor, b, h, step)
    sc = _channel_scale(w, tensor, h).astype(np.float32)
    if w.dist == "student_t4":
        x = r.standard_t(4, size=w.head_dim).astype(np.float32)
    else:
        x = r.standard_normal(size=w.head_dim, dtype=np.float32)
    if w.dist == "unit_norm_gaussian":
        x = (x / np.linalg.norm(x) * r.uniform(0.8, 1.2)).astype(np.float32)
    else:
        x = x * sc
    return x.astype(np.float16)


def key_energy(w, h):
    """E|k|^2 of KV head h's key rows (input statistics, used to scale q)."""
    if w.dist == "unit_norm_gaussian":
        return 1.0 + 0.4 ** 2 / 12.0  # E[U^2] for U ~ U[0.8, 1.2]
    return float(np.sum(_channel_scale(w, K_TENSOR, h) ** 2))


def queries(w, step=0, batch=None):
    """fp32 queries [B, Hq, d] for decode step ``step``."""
    B = w.batch if batch is None else batch
    d = w.head_dim
    r = _rng(w, Q_TENSOR, step)
    q = r.standard_normal(size=(B, w.n_q_heads, d))
    for g in range(w.n_q_heads):
        c = 2.0 * np.sqrt(d) / np.sqrt(key_energy(w, g // w.group))
        q[:, g] *= c
    return q.astype(np.float32)


def batch_rows(w, tensor, b, start, count):
    """fp16 [count, Hkv, d]: tokens of sequence b for every KV head, the
    [T][Hkv][d] layout the append call takes."""
    return np.stack([stream(w, tensor, b, h, start, count) for h in range(w.n_kv_heads)], axis=1)


def rotated_unit_rows(seed, n, d):
    """fp32 [n, d] rows of unit-norm-like coordinates with the N(0, 1/d) law
    of rotated unit vectors, for the test that feeds both sides identical
    rotated coordinates (values only; no rotation is applied here)."""
    r = np.random.default_rng([seed, 77])
    y = r.standard_normal(size=(n, d)) / np.sqrt(d)
    return y.astype(np.float32)
