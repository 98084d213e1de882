"""Sparse V on the GPU (tq_decode_partial_sparse_v), through the C ABI.

* Threshold 0 writes the same split records as tq_decode_partial, bit for bit.
* Two-level keys: every eighth token holds key A, the others key B, and each
  query puts the logit of A exactly Delta = ln(1 / tau) + 0.25 above that of B.
  Every tile (32 or 64 tokens, starting at a multiple of 32) starts with an A
  token, so the running maximum is the A logit when any B token is weighed:
  each B weight is e^-Delta < tau and each A weight is 1.  The result is then fixed whatever the visiting order: the
  softmax over all tokens with only the A tokens' values (the oracle's
  sparse_v_output), which differs from full attention by far more than the
  tolerance.
* Random needles: the output lies in the oracle's interval for the threshold
  (sparse_v_interval), i.e. between the extremes of every order.

Every kernel family is covered: the sparse matrix-core kernel (G 4 with one
or two tables, G 8), the bf16 matrix-core kernel (d 256, and G 8 with two
tables) and the generic kernel (PQ3; TQ3K keys with GQ2V values).
"""

import math

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

tq = pytest.importorskip("compressed_domain_attention_kv_amd")
P = pytest.importorskip("parity")
from oracle import attention as oatt  # noqa: E402

CASES = {
    "c4": synth.scaled(synth.C4, batch=2, n_q_heads=8, n_kv_heads=2, context=1300, capacity=1344),
    "c4_lloyd_v": synth.scaled(synth.C4, v_kind=synth.LLOYD_MAX, batch=2, n_q_heads=8, n_kv_heads=2, context=777,
                               capacity=832),
    "c4_g8": synth.scaled(synth.C4, batch=1, n_q_heads=16, n_kv_heads=2, context=1234, capacity=1280),
    "c4_g8_lloyd_v": synth.scaled(synth.C4, v_kind=synth.LLOYD_MAX, batch=1, n_q_heads=16, n_kv_heads=2,
                                  context=900, capacity=960),
    "c5": synth.scaled(synth.C5, batch=2, n_q_heads=16, n_kv_heads=2, context=700, capacity=704),
    "c5_g4": synth.scaled(synth.C5, batch=2, n_q_heads=8, n_kv_heads=2, context=600, capacity=640),
    "c5_lloyd_v": synth.scaled(synth.C5, v_kind=synth.LLOYD_MAX, batch=1, n_q_heads=16, n_kv_heads=2, context=500,
                               capacity=512),
    "c2": synth.scaled(synth.C2, batch=2, n_q_heads=8, n_kv_heads=2, context=777, capacity=832),
    "c3": synth.scaled(synth.C3, batch=1, n_q_heads=10, n_kv_heads=2, context=999, capacity=1024),
}


def _say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    yield


def _lens(w):
    return [max(1, w.context - 97 * b) for b in range(w.batch)]


def _encode(st, w, lens, two_level=False):
    """Oracle-encoded streams (optionally keys A/B: token 0 / token 1 of the stream
    repeated, A at every eighth position) and their dequantized rows."""
    kb, vb, kdq, vdq = {}, {}, [], []
    for b in range(w.batch):
        kdq.append([])
        vdq.append([])
        for h in range(w.n_kv_heads):
            ek = st.oracle_encode(synth.K_TENSOR, synth.stream(w, synth.K_TENSOR, b, h, 0, lens[b]))
            ev = st.oracle_encode(synth.V_TENSOR, synth.stream(w, synth.V_TENSOR, b, h, 0, lens[b]))
            kblk = ek.blocks
            if two_level:
                n = lens[b]
                kblk = np.where((np.arange(n) % 8 == 0)[:, None], kblk[0][None, :], kblk[1][None, :])
                kblk = np.ascontiguousarray(kblk.astype(np.uint8))
            kb[(b, h)], vb[(b, h)] = kblk, ev.blocks
            kdq[b].append(st.oracle_dequant(synth.K_TENSOR, kblk))
            vdq[b].append(st.oracle_dequant(synth.V_TENSOR, ev.blocks))
    return kb, vb, kdq, vdq


def _run(st, L, q, kc, vc, lens, tau, split_tokens=0, plain=False):
    """Rotate the queries, run one partial entry and the combine; returns (out, workspace bytes)."""
    w = st.w
    qd = torch.from_numpy(np.ascontiguousarray(q, np.float32)).cuda()
    q_rot = torch.empty_like(qd)
    q_sk = torch.empty_like(qd) if w.k_format == synth.TQ3K else None
    tq.rotate_sketch_query(L, st.cbk, st.S_dev, qd, q_rot, q_sk)
    ws = torch.zeros(tq.decode_workspace_bytes(L, split_tokens), dtype=torch.uint8, device="cuda")
    sl = torch.tensor(np.asarray(lens, np.int32), device="cuda")
    if plain:
        tq.decode_partial(L, st.cbk, st.cbv, q_rot, q_sk, kc, vc, sl, ws, split_tokens=split_tokens)
    else:
        tq.decode_partial_sparse_v(L, st.cbk, st.cbv, q_rot, q_sk, kc, vc, sl, ws, tau, split_tokens=split_tokens)
    out = torch.full((L.batch, L.n_q_heads, w.head_dim), float("nan"), device="cuda")
    tq.decode_combine(L, st.cbv, ws, out, split_tokens=split_tokens)
    torch.cuda.synchronize()
    return out.cpu().numpy(), ws.cpu().numpy()


def _caches(st, L, kb, vb):
    return P.place_streams(st, L, synth.K_TENSOR, kb), P.place_streams(st, L, synth.V_TENSOR, vb)


@pytest.mark.parametrize("name", list(CASES))
def test_threshold_zero_is_the_plain_partial(name):
    w = CASES[name]
    st = P.Setup(w)
    L = st.layout()
    lens = _lens(w)
    _say(f"sparse V tau=0 {name} lens={lens}")
    kb, vb, _, _ = _encode(st, w, lens)
    kc, vc = _caches(st, L, kb, vb)
    q = synth.queries(w)
    for split in (0, 256):
        o0, ws0 = _run(st, L, q, kc, vc, lens, 0.0, split, plain=True)
        o1, ws1 = _run(st, L, q, kc, vc, lens, 0.0, split)
        assert np.array_equal(ws0, ws1), f"{name} split {split}: records differ"
        assert np.array_equal(o0, o1, equal_nan=True)


def _two_level_queries(w, kdq, tau, seed):
    """Per query head: logit(A) - logit(B) = ln(1/tau) + 0.25 exactly, plus a random part orthogonal to A - B."""
    d = w.head_dim
    delta = math.log(1.0 / tau) + 0.25
    r = np.random.default_rng([seed, 99])
    q = np.zeros((w.batch, w.n_q_heads, d))
    for b in range(w.batch):
        for g in range(w.n_q_heads):
            kd = kdq[b][g // w.group]
            u = kd[0] - kd[1]
            x = r.standard_normal(d) * np.sqrt(d) / np.linalg.norm(u)
            x -= (x @ u) / (u @ u) * u
            q[b, g] = x + delta * np.sqrt(d) * u / (u @ u)
    return q


@pytest.mark.parametrize("name", list(CASES))
def test_two_level_keys_give_the_order_free_result(name):
    tau = 0.05
    w = CASES[name]
    st = P.Setup(w)
    L = st.layout()
    lens = _lens(w)
    _say(f"sparse V two-level {name} tau={tau} lens={lens}")
    kb, vb, kdq, vdq = _encode(st, w, lens, two_level=True)
    kc, vc = _caches(st, L, kb, vb)
    q = _two_level_queries(w, kdq, tau, w.seed)
    for split in (0, 256):
        out, _ = _run(st, L, q, kc, vc, lens, tau, split)
        worst = 0.0
        for b in range(w.batch):
            n = lens[b]
            keep = np.arange(n) % 8 == 0
            for g in range(w.n_q_heads):
                h = g // w.group
                want = oatt.sparse_v_output(q[b, g].astype(np.float32), kdq[b][h], vdq[b][h], keep)
                full, _ = oatt.softmax_attention(q[b, g].astype(np.float32), kdq[b][h], vdq[b][h])
                # the construction matters: leaving the B values out moves the output well past the tolerance
                assert P.rel_err_rows(full, want) > 10 * P.OUT_TOL, f"{name} b={b} g={g}: construction too weak"
                e = float(P.rel_err_rows(out[b, g], want))
                worst = max(worst, e)
                assert e <= P.OUT_TOL, f"{name} split {split} b={b} g={g}: {e:.3g}"
        _say(f"  split {split}: worst output err {worst:.2e}")


@pytest.mark.parametrize("name", ["c4", "c4_g8_lloyd_v", "c5", "c3"])
def test_random_needles_stay_in_the_oracle_interval(name):
    """Each query head points at one random key (a needle) on top of its usual query."""
    tau = 1e-3
    w = CASES[name]
    st = P.Setup(w)
    L = st.layout()
    lens = _lens(w)
    kb, vb, kdq, vdq = _encode(st, w, lens)
    kc, vc = _caches(st, L, kb, vb)
    q = synth.queries(w).astype(np.float64)
    r = np.random.default_rng([w.seed, 98])
    for b in range(w.batch):
        for g in range(w.n_q_heads):
            k = kdq[b][g // w.group][r.integers(lens[b])]
            q[b, g] += 12.0 * np.sqrt(w.head_dim) * k / (k @ k)
    _say(f"sparse V needles {name} tau={tau}")
    out, _ = _run(st, L, q, kc, vc, lens, tau)
    ref, _ = _run(st, L, q, kc, vc, lens, 0.0)
    moved = 0.0
    for b in range(w.batch):
        for g in range(w.n_q_heads):
            h = g // w.group
            lo, hi = oatt.sparse_v_interval(q[b, g].astype(np.float32), kdq[b][h], vdq[b][h], tau, margin=1e-3)
            tol = P.OUT_TOL * max(np.max(np.abs(lo)), np.max(np.abs(hi)))
            assert np.all(out[b, g] >= lo - tol) and np.all(out[b, g] <= hi + tol), f"{name} b={b} g={g}"
            moved = max(moved, float(np.max(np.abs(out[b, g] - ref[b, g]))))
    _say(f"  largest change against threshold 0: {moved:.3g}")


def test_threshold_out_of_range_is_refused():
    w = CASES["c4"]
    st = P.Setup(w)
    L = st.layout()
    d = w.head_dim
    q = torch.zeros((L.batch, L.n_q_heads, d), device="cuda")
    kc = torch.zeros(tq.cache_bytes(L)[0], dtype=torch.uint8, device="cuda")
    sl = torch.zeros(L.batch, dtype=torch.int32, device="cuda")
    ws = torch.zeros(tq.decode_workspace_bytes(L), dtype=torch.uint8, device="cuda")
    for bad in (-0.1, 1.5, float("nan")):
        with pytest.raises(tq.TQError) as e:
            tq.decode_partial_sparse_v(L, st.cbk, st.cbv, q, None, kc, kc, sl, ws, bad)
        assert e.value.status == -1
