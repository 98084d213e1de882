"""Pins of the oracle's block formats, encoders and decoders."""

import numpy as np
import pytest

from oracle import codebook as cb
from oracle import formats as F
from oracle import prng, rotation


def _page_pq4_code(blk, j):
    # extraction printed on the turbo4 page (section 5), byte offsets of qs
    # inside the 68-byte block start at 4
    qs = blk[4:]
    return (int(qs[j // 2]) >> ((j % 2) * 4)) & 0xF


def _page_pq3_code(blk, j):
    # 2+1 extraction printed on the turbo4 page (section 4) for one 14-byte
    # block: qs at bytes 2..9, signs at bytes 10..13
    qs, signs = blk[2:10], blk[10:14]
    idx = (int(qs[j // 4]) >> ((j % 4) * 2)) & 0x3
    if int(signs[j // 8]) & (1 << (j % 8)):
        idx |= 4
    return idx


def test_block_sizes_match_the_pages():
    assert F.vector_bytes(F.PQ4, 128) == 68
    assert F.vector_bytes(F.PQ4, 128) * 8 / 128 == 4.25  # bits per value
    assert round(256 / 68, 2) == 3.76  # compression against fp16
    assert F.vector_bytes(F.PQ3, 128) * 8 / 128 == 3.5
    assert F.vector_bytes(F.TQ3K, 128) == 52
    assert F.vector_bytes(F.GQ2V, 128) == 48
    assert F.vector_bytes(F.PQ4, 256) == 136


def test_pq4_pack_matches_page_extraction_all_codes():
    rng = np.random.default_rng(0)
    idx = rng.integers(0, 16, size=(9, 256))
    idx[0] = np.arange(256) % 16
    n16 = rng.uniform(0.1, 3, size=9).astype(np.float16)
    blocks = F.pack_pq4(n16, idx)
    for v in range(9):
        for blk in range(2):
            b = blocks[v, 68 * blk:68 * (blk + 1)]
            assert b[2] == 0 and b[3] == 0
            assert (int(b[0]) | (int(b[1]) << 8)) == int(n16[v].view(np.uint16))
            for j in range(128):
                assert _page_pq4_code(b, j) == idx[v, 128 * blk + j]
    norms, back = F.unpack_pq4(blocks, 256)
    assert np.array_equal(back, idx)
    assert np.array_equal(norms[:, 0], n16.astype(np.float64))


def test_pq3_pack_matches_page_extraction_all_codes():
    rng = np.random.default_rng(1)
    idx = rng.integers(0, 8, size=(7, 128))
    idx[0] = np.arange(128) % 8
    n16 = rng.uniform(0.1, 3, size=7).astype(np.float16)
    blocks = F.pack_pq3(n16, idx)
    for v in range(7):
        for blk in range(4):
            b = blocks[v, 14 * blk:14 * (blk + 1)]
            for j in range(32):
                assert _page_pq3_code(b, j) == idx[v, 32 * blk + j]
    norms, back = F.unpack_pq3(blocks, 128)
    assert np.array_equal(back, idx)
    assert np.all(norms == n16.astype(np.float64)[:, None])


def test_tq3k_and_gq2v_bit_layouts_round_trip():
    rng = np.random.default_rng(2)
    idx = rng.integers(0, 4, size=(5, 128))
    bits = rng.integers(0, 2, size=(5, 128))
    blocks = F._tq3k_pack(np.ones(5, np.float16), np.full(5, 0.5, np.float16), idx, bits)
    n16, g16, i2, b2 = F.unpack_tq3k(blocks, 128)
    assert np.array_equal(i2, idx) and np.array_equal(b2, bits)
    assert np.all(n16 == 1.0) and np.all(g16 == 0.5)
    # explicit bit positions for one vector
    for j in range(128):
        assert (blocks[0, 4 + j // 4] >> (2 * (j % 4))) & 3 == idx[0, j]
        assert (blocks[0, 36 + j // 8] >> (j % 8)) & 1 == bits[0, j]


@pytest.mark.parametrize("kind,bits,fmt,d", [
    (cb.QUANTILE_MEAN, 4, F.PQ4, 128),
    (cb.QUANTILE_MEAN, 4, F.PQ4, 256),
    (cb.LLOYD_MAX, 4, F.PQ4, 128),
    (cb.QUANTILE_MEAN, 3, F.PQ3, 128),
])
def test_basis_vector_closed_form(kind, bits, fmt, d):
    """x = n e_m: every rotated coordinate is +-1/sqrt(d), so each one takes
    the centroid c* nearest 1/sqrt(d) with the sign of y, and the decoded
    vector is exactly n16 * c* * sqrt(d) * e_m because H H = d I."""
    t = cb.tables(d, bits, kind)
    s = prng.rotation_signs(21, d)
    cstar = t.centroids[np.argmin(np.abs(t.centroids.astype(np.float64) - 1 / np.sqrt(d)))]
    for m in (0, 5, d - 1):
        for n in (1.0, 0.37, 20.0):
            x = np.zeros((1, d), np.float16)
            x[0, m] = n
            enc = F.encode_rotated(x, fmt, t, s)
            khat = F.dequant(enc.blocks, fmt, d, t, s)[0]
            ref = np.zeros(d)
            ref[m] = float(np.float16(n)) * float(cstar) * np.sqrt(d)
            assert np.max(np.abs(khat - ref)) < 1e-12 * max(1.0, n)
    if kind == cb.QUANTILE_MEAN and bits == 4:
        # the gain c* sqrt(d) of the page's construction
        assert abs(float(cstar) * np.sqrt(d) - 1.01289) < 1e-4


def test_zero_vector_decodes_to_zero():
    t = cb.tables(128, 4)
    s = prng.rotation_signs(1, 128)
    enc = F.encode_rotated(np.zeros((1, 128), np.float16), F.PQ4, t, s)
    assert enc.blocks[0, 0] == 0 and enc.blocks[0, 1] == 0
    assert np.all(enc.idx == 7)
    assert np.all(F.dequant(enc.blocks, F.PQ4, 128, t, s) == 0)


def test_norm_saturates_at_fp16_max():
    t = cb.tables(128, 4)
    s = prng.rotation_signs(1, 128)
    x = np.full((1, 128), 60000, np.float16)
    enc = F.encode_rotated(x, F.PQ4, t, s)
    assert np.float16(65504).view(np.uint16) == (enc.blocks[0, 0] | (enc.blocks[0, 1].astype(np.uint16) << 8))


@pytest.mark.parametrize("fmt,bits", [(F.PQ4, 4), (F.PQ3, 3)])
def test_encode_decode_error_matches_quantizer_mse(fmt, bits):
    """Relative reconstruction error of random unit vectors equals the scalar
    quantizer's MSE times d (each of d rotated coordinates contributes)."""
    from test_oracle_codebook import _mse_by_quadrature
    d = 128
    t = cb.tables(d, bits)
    s = prng.rotation_signs(4, d)
    x = np.random.default_rng(5).normal(size=(3000, d))
    x = (x / np.linalg.norm(x, axis=1, keepdims=True)).astype(np.float16)
    enc = F.encode_rotated(x, fmt, t, s)
    khat = F.dequant(enc.blocks, fmt, d, t, s)
    xf = x.astype(np.float64)
    u = xf / np.linalg.norm(xf, axis=1, keepdims=True)
    n16 = enc.blocks[:, :2].copy().view(np.float16).astype(np.float64)
    rel = np.sum((khat / n16 - u) ** 2, axis=1)
    ref = _mse_by_quadrature(t.centroids64, 1 / np.sqrt(d)) * d
    assert abs(rel.mean() - ref) < 0.05 * ref


def test_gq2v_error_bound_and_extremes():
    rng = np.random.default_rng(6)
    v = rng.normal(size=(200, 128)).astype(np.float16)
    v[0, :32] = 1.5  # constant group
    v[1, 32:64] = 0.0  # zero group
    enc = F.encode_gq2v(v)
    vhat = F.dequant(enc.blocks, F.GQ2V, 128)
    scale, zero, q = F.unpack_gq2v(enc.blocks, 128)
    err = np.abs(vhat - v.astype(np.float64))
    bound = np.repeat(scale, 32, axis=1) / 2 + 2e-3 * (np.abs(v.astype(np.float64)) + np.repeat(scale, 32, axis=1))
    assert np.all(err <= bound)
    assert np.all(vhat[0, :32] == 1.5) and np.all(vhat[1, 32:64] == 0.0)
    for g in range(4):
        grp = v[2:, 32 * g:32 * (g + 1)].astype(np.float64)
        qq = q[2:, 32 * g:32 * (g + 1)]
        assert np.all(qq[np.arange(len(grp)), grp.argmin(1)] == 0)
        assert np.all(qq[np.arange(len(grp)), grp.argmax(1)] == 3)


def test_gq4v_error_bound_extremes_and_nibble_layout():
    """GQ4V: the 4-bit sibling of GQ2V.  |v - v_hat| <= scale/2 (+ fp16 rounding of the
    stored scale and zero); constant and zero groups decode exactly; each group's minimum
    takes code 0 and its maximum code 15; the codes sit in the bytes as the nibble
    extraction printed for the PQ4 block reads them, (q[j/2] >> ((j%2)*4)) & 0xF, after a
    [fp16 scale][fp16 zero] header per 32-channel group."""
    rng = np.random.default_rng(16)
    v = rng.normal(size=(300, 128)).astype(np.float16)
    v[0, :32] = -0.75  # constant group
    v[1, 96:] = 0.0  # zero group
    v[2, 32:64] = np.linspace(-1, 1, 32)  # evenly spread: every code in use
    enc = F.encode_gq4v(v)
    assert enc.blocks.shape == (300, 80) and F.vector_bytes(F.GQ4V, 128) == 80 and F.vector_bytes(F.GQ4V, 256) == 160
    vhat = F.dequant(enc.blocks, F.GQ4V, 128)
    scale, zero, q = F.unpack_gq4v(enc.blocks, 128)
    # bytes read by the printed nibble formula and the fp16 header, independently of unpack_gq4v
    for g in range(4):
        hdr = enc.blocks[:, 20 * g:20 * g + 4].copy().view(np.float16).astype(np.float64)
        qs = enc.blocks[:, 20 * g + 4:20 * g + 20].astype(np.int64)
        for j in range(32):
            assert np.array_equal((qs[:, j // 2] >> ((j % 2) * 4)) & 0xF, enc.idx[:, 32 * g + j])
        assert np.array_equal(hdr[:, 0], scale[:, g]) and np.array_equal(hdr[:, 1], zero[:, g])
    assert np.array_equal(q, enc.idx)
    err = np.abs(vhat - v.astype(np.float64))
    sc = np.repeat(scale, 32, axis=1)
    assert np.all(err <= sc / 2 + 2e-3 * (np.abs(v.astype(np.float64)) + sc))
    assert np.all(vhat[0, :32] == -0.75) and np.all(vhat[1, 96:] == 0.0)
    assert sorted(set(q[2, 32:64].tolist())) == list(range(16))
    for g in range(4):
        grp = v[3:, 32 * g:32 * (g + 1)].astype(np.float64)
        qq = q[3:, 32 * g:32 * (g + 1)]
        assert np.all(qq[np.arange(len(grp)), grp.argmin(1)] == 0)
        assert np.all(qq[np.arange(len(grp)), grp.argmax(1)] == 15)
    # the step is (max - min) / 15 against GQ2V's / 3: the squared error falls about 25-fold
    e2 = np.mean((F.dequant(F.encode_gq2v(v).blocks, F.GQ2V, 128) - v.astype(np.float64)) ** 2)
    e4 = np.mean(err ** 2)
    assert 15 < e2 / e4 < 35


def test_qjl_estimator_is_unbiased_with_closed_form_variance():
    """E[<y, r_hat>] = <y, r> over Gaussian S; the variance is
    [(pi/2) |r|^2 |y|^2 - <r, y>^2] / d, and E|r_hat|^2 = (pi/2 + (d-1)/d)|r|^2."""
    d = 128
    rng = np.random.default_rng(2024)
    r = rng.normal(size=d)
    y = 0.6 * r / np.linalg.norm(r) + rng.normal(size=d) / np.sqrt(d)
    gamma = np.linalg.norm(r)
    trials, chunk = 100_000, 2_000
    est, energy = [], []
    for _ in range(trials // chunk):
        S = rng.standard_normal(size=(chunk, d, d))
        bits, _ = F.qjl_sign_bits(r[None, :], S)
        rhat = F.qjl_reconstruct(bits, np.full(chunk, gamma), S)
        est.append(rhat @ y)
        energy.append(np.sum(rhat * rhat, axis=1))
    est = np.concatenate(est)
    energy = np.concatenate(energy)
    true = r @ y
    se = est.std() / np.sqrt(trials)
    assert abs(est.mean() - true) < 3 * se
    var_cf = ((np.pi / 2) * gamma ** 2 * (y @ y) - true ** 2) / d
    assert abs(est.var() / var_cf - 1) < 0.03
    e_cf = (np.pi / 2 + (d - 1) / d) * gamma ** 2
    assert abs(energy.mean() / e_cf - 1) < 3 * energy.std() / np.sqrt(trials) / e_cf + 1e-9


def test_tq3k_residual_is_in_unrotated_normalized_space():
    d = 128
    t = cb.tables(d, 2, cb.LLOYD_MAX)
    s = prng.rotation_signs(8, d)
    S = prng.qjl_matrix(9, d)
    x = np.random.default_rng(7).normal(size=(20, d)).astype(np.float16)
    enc = F.encode_tq3k(x, t, s, S)
    xf = x.astype(np.float64)
    u = xf / np.linalg.norm(xf, axis=1, keepdims=True)
    mse = rotation.unrotate(t.centroids.astype(np.float64)[enc.idx], s)
    r = u - mse
    assert np.allclose(enc.extra["gamma"], np.linalg.norm(r, axis=1), atol=1e-12)
    assert np.array_equal(enc.extra["bits"], (r @ S.astype(np.float64).T >= 0).astype(np.int64))
    # the residual norm equals the rotated-domain quantization error
    yq = rotation.rotate(u, s) - t.centroids.astype(np.float64)[enc.idx]
    assert np.allclose(enc.extra["gamma"], np.linalg.norm(yq, axis=1), atol=1e-12)
