"""Pins of the oracle's attention: identities, special cases, brute force."""

import math

import numpy as np
import pytest
from scipy.special import softmax

from oracle import attention as A
from oracle import codebook as cb
from oracle import formats as F
from oracle import prng, rotation


def _setup(fmt, d, seed=0):
    bits = {F.PQ4: 4, F.PQ3: 3, F.TQ3K: 2}[fmt]
    kind = cb.LLOYD_MAX if fmt == F.TQ3K else cb.QUANTILE_MEAN
    t = cb.tables(d, bits, kind)
    s = prng.rotation_signs(seed + 1, d)
    S = prng.qjl_matrix(seed + 2, d) if fmt == F.TQ3K else None
    return t, s, S


@pytest.mark.parametrize("fmt,d", [(F.PQ4, 128), (F.PQ4, 256), (F.PQ3, 128), (F.PQ3, 32), (F.TQ3K, 128), (F.TQ3K, 16)])
def test_compressed_domain_score_equals_dot_with_dequantized_key(fmt, d):
    """<q, k_hat> computed as <Pi q, n c[idx]> (+ QJL term) equals the plain
    dot product with the fully dequantized key (rotate-the-query identity)."""
    t, s, S = _setup(fmt, d)
    rng = np.random.default_rng(3)
    x = rng.normal(size=(8, d)).astype(np.float16)
    if fmt == F.TQ3K:
        enc = F.encode_tq3k(x, t, s, S)
    else:
        enc = F.encode_rotated(x, fmt, t, s)
    khat = F.dequant(enc.blocks, fmt, d, t, s, S)
    q = rng.normal(size=d)
    fast = A.compressed_scores(q, enc.blocks, fmt, d, t, s, S)
    plain = khat @ q / np.sqrt(d)
    assert np.max(np.abs(fast - plain)) < 1e-12 * max(1, np.abs(plain).max())


def test_tq3k_brute_force_pure_python_tiny():
    """d = 16, element by element in Python floats: the decoded key and the
    score from the page's formula sqrt(pi/2)/d * gamma * <S q, 2b - 1>."""
    d = 16
    t, s, S = _setup(F.TQ3K, d, seed=4)
    rng = np.random.default_rng(5)
    x = rng.normal(size=(3, d)).astype(np.float16)
    q = rng.normal(size=d)
    enc = F.encode_tq3k(x, t, s, S)
    n16, g16, idx, bits = F.unpack_tq3k(enc.blocks, d)
    H = rotation.hadamard(d)
    for v in range(3):
        # Pi^T c = diag(s) H c / sqrt(d), coordinate by coordinate
        k = []
        for i in range(d):
            mse = sum(float(H[i, j]) * float(t.centroids[idx[v, j]]) for j in range(d)) * s[i] / math.sqrt(d)
            qjl = sum(float(S[j, i]) * (2 * int(bits[v, j]) - 1) for j in range(d))
            k.append(float(n16[v]) * (mse + math.sqrt(math.pi / 2) / d * float(g16[v]) * qjl))
        score = sum(k[i] * q[i] for i in range(d)) / math.sqrt(d)
        fast = A.compressed_scores(q, enc.blocks[v:v + 1], F.TQ3K, d, t, s, S)[0]
        assert abs(score - fast) < 1e-12
        assert np.allclose(F.dequant(enc.blocks[v:v + 1], F.TQ3K, d, t, s, S)[0], k, atol=1e-13)


def test_single_key_returns_its_value():
    rng = np.random.default_rng(0)
    v = rng.normal(size=(1, 128))
    o, _ = A.softmax_attention(rng.normal(size=128), rng.normal(size=(1, 128)), v)
    assert np.allclose(o, v[0], atol=1e-15)


def test_identical_keys_average_values():
    rng = np.random.default_rng(1)
    k = np.repeat(rng.normal(size=(1, 64)), 7, axis=0)
    v = rng.normal(size=(7, 64))
    o, _ = A.softmax_attention(rng.normal(size=64), k, v)
    assert np.allclose(o, v.mean(0), atol=1e-14)


def test_two_keys_logistic_weights():
    d = 4
    q = np.array([1.0, 0, 0, 0])
    k = np.array([[2.0, 0, 0, 0], [0.0, 0, 0, 0]])
    v = np.array([[1.0, 0, 0, 0], [0.0, 1, 0, 0]])
    o, s = A.softmax_attention(q, k, v)
    w = 1 / (1 + math.exp(-(2.0 / math.sqrt(d))))
    assert np.allclose(o, [w, 1 - w, 0, 0], atol=1e-15)
    assert np.allclose(s, [1.0, 0.0])


def test_softmax_matches_scipy():
    rng = np.random.default_rng(2)
    q = rng.normal(size=128) * 3
    k = rng.normal(size=(300, 128))
    v = rng.normal(size=(300, 128))
    o, s = A.softmax_attention(q, k, v)
    assert np.allclose(o, softmax(k @ q / np.sqrt(128)) @ v, atol=1e-13)


@pytest.mark.parametrize("bounds", [[0, 1000], [0, 64, 1000], [0, 0, 500, 500, 1000], [0, 1, 999, 1000],
                                    list(range(0, 1001, 37)) + [1000]])
def test_any_split_combines_to_the_same_output(bounds):
    rng = np.random.default_rng(4)
    s = rng.normal(size=1000) * 4
    v = rng.normal(size=(1000, 16))
    ref = softmax(s) @ v
    out = A.combine_records(A.split_records(s, v, sorted(bounds)))
    assert np.allclose(out, ref, atol=1e-13)


def test_empty_context_outputs_zero():
    assert np.all(A.combine_records(A.split_records(np.zeros(0), np.zeros((0, 8)), [0, 0, 0])) == 0)
    out, _ = A.decode_attention(np.ones((1, 2, 8)), [[np.zeros((0, 8))]], [[np.zeros((0, 8))]], [0], 2)
    assert np.all(out == 0)


def test_gqa_head_mapping():
    rng = np.random.default_rng(6)
    B, Hq, Hkv, d, N = 2, 6, 2, 8, 5
    q = rng.normal(size=(B, Hq, d))
    K = [[rng.normal(size=(N, d)) for _ in range(Hkv)] for _ in range(B)]
    V = [[rng.normal(size=(N, d)) for _ in range(Hkv)] for _ in range(B)]
    out, _ = A.decode_attention(q, K, V, [N, 3], Hq // Hkv)
    for b, n in ((0, N), (1, 3)):
        for g in range(Hq):
            h = g // 3
            ref = softmax(K[b][h][:n] @ q[b, g] / np.sqrt(d)) @ V[b][h][:n]
            assert np.allclose(out[b, g], ref, atol=1e-14)


def test_tq3k_key_inner_product_unbiased_over_qjl_matrices():
    """Over independent Gaussian S the TQ3K key is an unbiased estimate of the
    original key in inner products: E <q, k_hat> = n16/n * <q, x>.  A residual
    taken in the wrong (rotated) space or a missing S^T product breaks it."""
    d = 64
    t = cb.tables(d, 2, cb.LLOYD_MAX)
    s = prng.rotation_signs(31, d)
    rng = np.random.default_rng(32)
    x = rng.normal(size=(1, d)).astype(np.float16)
    q = rng.normal(size=d)
    vals = []
    for _ in range(4000):
        S = rng.standard_normal(size=(d, d)).astype(np.float32)
        enc = F.encode_tq3k(x, t, s, S)
        vals.append(F.dequant(enc.blocks, F.TQ3K, d, t, s, S)[0] @ q)
    vals = np.array(vals)
    xf = x[0].astype(np.float64)
    n = np.linalg.norm(xf)
    target = float(np.float16(n)) / n * (xf @ q)
    assert abs(vals.mean() - target) < 3 * vals.std() / np.sqrt(len(vals))
    # the MSE stage alone is biased for this key; the QJL term removes it
    mse_only = float(np.float16(n)) * rotation.unrotate(
        t.centroids.astype(np.float64)[F.encode_tq3k(x, t, s, S).idx], s)[0] @ q
    assert abs(mse_only - target) > 3 * vals.std() / np.sqrt(len(vals))


# ---------------------------------------------------------------------------
# sparse V


def _tiny(n, d, seed, peak=0.0):
    rng = np.random.default_rng(seed)
    k = rng.normal(size=(n, d))
    v = rng.normal(size=(n, d))
    q = rng.normal(size=d) + peak * k[0]
    return q, k, v


def test_sparse_v_output_keep_all_and_keep_none():
    q, k, v = _tiny(9, 8, 1)
    o, _ = A.softmax_attention(q, k, v)
    assert np.allclose(A.sparse_v_output(q, k, v, np.ones(9, bool)), o, rtol=0, atol=1e-15)
    assert np.all(A.sparse_v_output(q, k, v, np.zeros(9, bool)) == 0.0)


def test_sparse_v_output_is_softmax_weighted_partial_sum():
    """Against scipy's softmax: the kept tokens' p_t v_t summed, by a loop."""
    q, k, v = _tiny(7, 4, 2)
    keep = np.array([1, 0, 1, 1, 0, 0, 1], bool)
    p = softmax(k @ q / 2.0)  # sqrt(4)
    want = np.zeros(4)
    for t in range(7):
        if keep[t]:
            want += p[t] * v[t]
    assert np.allclose(A.sparse_v_output(q, k, v, keep), want, rtol=0, atol=1e-14)


@pytest.mark.parametrize("seed,tau,peak", [(3, 0.05, 0.0), (4, 0.1, 1.0), (5, 0.02, 2.0), (6, 0.2, 3.0)])
def test_sparse_v_interval_is_attained_by_brute_force(seed, tau, peak):
    """Every keep set that holds the tokens with p >= tau: its output lies in
    [lo, hi], and per coordinate some such set reaches lo and another hi."""
    n, d = 10, 6
    q, k, v = _tiny(n, d, seed, peak)
    lo, hi = A.sparse_v_interval(q, k, v, tau)
    p = softmax(k @ q / math.sqrt(d))
    must = p >= tau
    opt = np.flatnonzero(~must)
    assert 0 < len(opt) < n
    outs = []
    for mask in range(1 << len(opt)):
        keep = must.copy()
        for i, t in enumerate(opt):
            if mask >> i & 1:
                keep[t] = True
        outs.append(A.sparse_v_output(q, k, v, keep))
    outs = np.array(outs)
    assert np.all(outs >= lo - 1e-14) and np.all(outs <= hi + 1e-14)
    assert np.allclose(outs.min(axis=0), lo, atol=1e-14) and np.allclose(outs.max(axis=0), hi, atol=1e-14)


def test_sparse_v_interval_threshold_zero_is_exact_attention():
    q, k, v = _tiny(12, 5, 7)
    o, _ = A.softmax_attention(q, k, v)
    lo, hi = A.sparse_v_interval(q, k, v, 0.0)
    assert np.allclose(lo, o, atol=1e-15) and np.allclose(hi, o, atol=1e-15)


def test_sparse_v_interval_margin_widens_only():
    q, k, v = _tiny(10, 6, 8, 1.5)
    lo0, hi0 = A.sparse_v_interval(q, k, v, 0.05)
    lo1, hi1 = A.sparse_v_interval(q, k, v, 0.05, margin=10.0)
    assert np.all(lo1 <= lo0 + 1e-15) and np.all(hi1 >= hi0 - 1e-15)
    o, _ = A.softmax_attention(q, k, v)
    assert np.all(lo0 <= o + 1e-14) and np.all(o <= hi0 + 1e-14)
