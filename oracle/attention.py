"""Textbook decode attention over dequantized caches, in float64.

What the fused compressed-domain kernel reaches is exactly softmax attention
over the dequantized cache: the unfused nine-step path of the "TurboQuant
Triton deep dive" (section "nine-step path": unpack, look up, rotate back,
scale by the norm, dot with the query) followed by softmax(q k^T / sqrt(d)) v
("PolarQuant-KV", section 3.3; the 1/sqrt(d) logit scale also in "turbo4
post-mortem", section 9).  The oracle therefore dequantizes every cached
vector, forms the logits, takes a max-subtracted softmax and the weighted sum
of dequantized values.

Grouped-query attention: query head g reads KV head g // (Hq / Hkv).

``hybrid_attention`` is the same softmax over the compressed history and the
exact tokens of the capture ring taken together.

Sparse V ("turbo4 post-mortem", section 9, lists a sparse-V mode without a rule
or threshold; the reading here: a token's value is left out when its weight is
negligible).  ``sparse_v_output`` is the softmax with every token in the
denominator but only a chosen set of tokens in the value sum;
``sparse_v_interval`` bounds, per output coordinate, every result that keeps
at least the tokens whose softmax weight reaches the threshold.

Besides the plain path, two helpers restate the identities the fast path
relies on, so that tests can pin them:

* ``compressed_scores``: the logit evaluated on the codes with a query that
  was rotated once, <Pi q, n c[idx]> ("TurboQuant Triton deep dive", trick 1:
  <q, Pi^T y> = <Pi q, y>), plus the QJL term <S q, 2b - 1> (trick 2);
* ``split_records`` / ``combine_records``: the online-softmax state
  (m, l, acc) of any partition of the keys and its merge (trick 3).
"""

import numpy as np

from . import formats, rotation


def softmax_attention(q, khat, vhat):
    """o = softmax(q khat^T / sqrt(d)) vhat for one query vector; returns (o, logits)."""
    q = np.asarray(q, dtype=np.float64)
    d = q.shape[-1]
    if khat.shape[0] == 0:
        return np.zeros(vhat.shape[1]), np.zeros(0)
    s = khat @ q / np.sqrt(d)
    p = np.exp(s - s.max())
    p /= p.sum()
    return p @ vhat, s


def hybrid_attention(q, khat, vhat, k_exact, v_exact):
    """Hybrid read of one query: the compressed history (dequantized khat,
    vhat) and the exact recent tokens of the capture ring (k_exact, v_exact,
    their stored fp16 values as they are) form one key set ("TurboQuant Triton
    deep dive": the write path keeps the newest tokens exact in a ring buffer;
    the hybrid mode in its limits section reads both).  Returns (o, logits)."""
    d = np.asarray(q).shape[-1]
    k = np.concatenate([np.asarray(khat, np.float64).reshape(-1, d), np.asarray(k_exact, np.float64).reshape(-1, d)])
    v = np.concatenate([np.asarray(vhat, np.float64).reshape(-1, d), np.asarray(v_exact, np.float64).reshape(-1, d)])
    return softmax_attention(q, k, v)


def decode_attention(q, kv_k, kv_v, seq_lens, G):
    """Attention for q [B, Hq, d] over dequantized caches kv_k/kv_v [B][Hkv] -> [N, d].

    Returns (out [B, Hq, d], logits: list of per-(b, g) arrays).
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    out = np.zeros((B, Hq, d))
    logits = [[None] * Hq for _ in range(B)]
    for b in range(B):
        n = int(seq_lens[b])
        for g in range(Hq):
            h = g // G
            o, s = softmax_attention(q[b, g], kv_k[b][h][:n], kv_v[b][h][:n])
            out[b, g] = o
            logits[b][g] = s
    return out, logits


def compressed_scores(q, blocks, fmt, d, tabs, signs, S=None):
    """Logits evaluated in the compressed domain for one query vector.

    PQ4/PQ3: s_i = sum over blocks of n_blk * <Pi q, c[idx]> / sqrt(d).
    TQ3K:    s_i = n * (<Pi q, c[idx]> + sqrt(pi/2)/d * gamma * <S q, 2b-1>) / sqrt(d).
    """
    q = np.asarray(q, dtype=np.float64)
    q_rot = rotation.rotate(q[None, :], signs)[0]
    cent = tabs.centroids.astype(np.float64)
    if fmt in (formats.PQ4, formats.PQ3):
        if fmt == formats.PQ4:
            norms, idx = formats.unpack_pq4(blocks, d)
        else:
            norms, idx = formats.unpack_pq3(blocks, d)
        bs = formats.block_size_of(fmt)
        s = np.zeros(blocks.shape[0])
        for blk in range(d // bs):
            sl = slice(bs * blk, bs * (blk + 1))
            s += norms[:, blk] * (cent[idx[:, sl]] @ q_rot[sl])
        return s / np.sqrt(d)
    if fmt == formats.TQ3K:
        n16, g16, idx, bits = formats.unpack_tq3k(blocks, d)
        q_sk = np.asarray(S, dtype=np.float64) @ q
        mse = cent[idx] @ q_rot
        qjl = (2.0 * bits - 1.0) @ q_sk
        return n16 * (mse + formats.QJL_CONST / d * g16 * qjl) / np.sqrt(d)
    raise ValueError("compressed scores are defined for key formats")


def split_records(s, vhat, bounds):
    """Online-softmax state of each part [bounds[k], bounds[k+1]) of the keys.

    m = max logit of the part (-inf if empty), l = sum exp(s - m),
    acc = sum exp(s - m) v.
    """
    recs = []
    for a, b in zip(bounds[:-1], bounds[1:]):
        if b <= a:
            recs.append((-np.inf, 0.0, np.zeros(vhat.shape[1])))
            continue
        m = s[a:b].max()
        e = np.exp(s[a:b] - m)
        recs.append((m, e.sum(), e @ vhat[a:b]))
    return recs


def combine_records(recs):
    """Merge (m, l, acc) parts: rescale each by exp(m_p - M) and normalize."""
    ms = np.array([r[0] for r in recs])
    if not np.isfinite(ms).any():
        return np.zeros(recs[0][2].shape[0])
    M = ms.max()
    w = np.where(np.isfinite(ms), np.exp(np.where(np.isfinite(ms), ms - M, 0.0)), 0.0)
    L = sum(wi * r[1] for wi, r in zip(w, recs))
    acc = sum(wi * r[2] for wi, r in zip(w, recs))
    return acc / L


def sparse_v_output(q, khat, vhat, keep):
    """Softmax attention of one query in which every token's weight enters the
    denominator but only tokens with keep[t] add their value:
    o = sum_{t kept} p_t vhat_t with p = softmax(q khat^T / sqrt(d))."""
    q = np.asarray(q, dtype=np.float64)
    if khat.shape[0] == 0:
        return np.zeros(vhat.shape[1])
    s = khat @ q / np.sqrt(q.shape[-1])
    p = np.exp(s - s.max())
    p /= p.sum()
    return (p * np.asarray(keep, dtype=np.float64)) @ vhat


def sparse_v_interval(q, khat, vhat, tau, margin=0.0):
    """Per-coordinate range [lo, hi] of sparse_v_output over every keep set that
    contains each token with p_t >= tau (1 + margin), the others optional.

    A token left out by the threshold rule has weight e^(s_t - m) < tau against
    a running maximum m that never exceeds the true maximum M, so its softmax
    weight p_t <= e^(s_t - M) < tau: such sets cover every visiting order.
    margin > 0 also lets tokens just above tau drop, for a decision taken in
    finite precision.  Coordinate j: lo = sure_j + sum_opt min(0, p_t v_tj),
    hi = sure_j + sum_opt max(0, p_t v_tj)."""
    q = np.asarray(q, dtype=np.float64)
    if khat.shape[0] == 0:
        z = np.zeros(vhat.shape[1])
        return z, z.copy()
    s = khat @ q / np.sqrt(q.shape[-1])
    p = np.exp(s - s.max())
    p /= p.sum()
    sure = p >= tau * (1.0 + margin)
    contrib = p[:, None] * np.asarray(vhat, dtype=np.float64)
    base = contrib[sure].sum(axis=0)
    opt = contrib[~sure]
    return base + np.minimum(opt, 0.0).sum(axis=0), base + np.maximum(opt, 0.0).sum(axis=0)
