"""Helpers of the GPU parity tests (imported by tests/test_gpu_*.py).

Write side: the HIP encoder and the oracle encode the same seeded fp16 rows;
the bytes must match except for codes whose oracle coordinate lies within
1e-6 of a decision boundary (fp32 summation order of the rotation differs),
fp16 norms one ulp apart when the float64 norm sits on an fp16 rounding
midpoint, and -- TQ3K only -- QJL sign bits whose projection is within
rounding of zero.  Every such difference is counted and returned.

Read side: the HIP decoder reads bytes the *oracle* wrote, so that both
sides attend over identical codes; scores must agree to 1e-4 and outputs to
1e-3 (max abs error over the row / max abs value of the row; for scores the
denominator is at least a tenth of the row's Cauchy-Schwarz scale, see
score_err).

GPU output bytes are parsed here with the pages' extraction formulas; the
oracle's own unpackers are never applied to GPU data.
"""

import numpy as np
import torch

import compressed_domain_attention_kv_amd as tq
import synth
from oracle import attention as oatt
from oracle import codebook as ocb
from oracle import formats as ofmt
from oracle import prng as oprng

SCORE_TOL = 1e-4
OUT_TOL = 1e-3
BOUNDARY_EPS = 1e-6


class Setup:
    """Codebooks of one workload, built independently by each side."""

    def __init__(self, w):
        self.w = w
        d = w.head_dim
        tq3k = w.k_format == synth.TQ3K
        self.cbk, S = tq.build_codebook(d, w.k_bits, w.k_kind, w.rot_seed_k, w.qjl_seed, want_qjl_matrix=tq3k)
        self.cbv, _ = tq.build_codebook(d, w.v_bits, w.v_kind, w.rot_seed_v, w.qjl_seed + 1)
        self.S_dev = torch.from_numpy(S).cuda() if tq3k else None
        self.tk = ocb.tables(d, w.k_bits, w.k_kind)
        self.tv = ocb.tables(d, w.v_bits, w.v_kind)
        self.sk = oprng.rotation_signs(w.rot_seed_k, d)
        self.sv = oprng.rotation_signs(w.rot_seed_v, d)
        self.S_o = oprng.qjl_matrix(w.qjl_seed, d) if tq3k else None
        self.vbk = tq.vector_bytes(w.k_format, d)
        self.vbv = tq.vector_bytes(w.v_format, d)

    def layout(self, batch=None, capacity=None):
        w = self.w
        return tq.Layout(w.batch if batch is None else batch, w.n_q_heads, w.n_kv_heads, w.head_dim,
                         w.capacity if capacity is None else capacity, w.k_format, w.v_format)

    # --- oracle encoders
    def oracle_encode(self, tensor, x16):
        w = self.w
        fmt = w.k_format if tensor == synth.K_TENSOR else w.v_format
        tabs = self.tk if tensor == synth.K_TENSOR else self.tv
        signs = self.sk if tensor == synth.K_TENSOR else self.sv
        if fmt in (ofmt.PQ4, ofmt.PQ3):
            return ofmt.encode_rotated(x16, fmt, tabs, signs)
        if fmt == ofmt.TQ3K:
            return ofmt.encode_tq3k(x16, tabs, signs, self.S_o)
        if fmt == ofmt.GQ4V:
            return ofmt.encode_gq4v(x16)
        return ofmt.encode_gq2v(x16)

    def oracle_dequant(self, tensor, blocks):
        w = self.w
        if tensor == synth.K_TENSOR:
            return ofmt.dequant(blocks, w.k_format, w.head_dim, self.tk, self.sk, self.S_o)
        return ofmt.dequant(blocks, w.v_format, w.head_dim, self.tv, self.sv, self.S_o)


# ---------------------------------------------------------------------------
# parsing GPU bytes (page formulas)


def _u16(lo, hi):
    return lo.astype(np.uint16) | (hi.astype(np.uint16) << 8)


def parse_codes(fmt, blocks, d):
    """-> (fp16 norm bits per block [n, nblk], codes [n, d], extra dict)."""
    n = blocks.shape[0]
    if fmt == synth.PQ4:
        nb = d // 128
        norms = np.stack([_u16(blocks[:, 68 * k], blocks[:, 68 * k + 1]) for k in range(nb)], 1)
        codes = np.zeros((n, d), np.int64)
        for k in range(nb):
            qs = blocks[:, 68 * k + 4:68 * k + 68].astype(np.int64)
            for j in range(128):
                codes[:, 128 * k + j] = (qs[:, j // 2] >> ((j % 2) * 4)) & 0xF
        return norms, codes, {"reserved": blocks[:, [68 * k + r for k in range(nb) for r in (2, 3)]]}
    if fmt == synth.PQ3:
        nb = d // 32
        norms = np.stack([_u16(blocks[:, 14 * k], blocks[:, 14 * k + 1]) for k in range(nb)], 1)
        codes = np.zeros((n, d), np.int64)
        for k in range(nb):
            qs = blocks[:, 14 * k + 2:14 * k + 10].astype(np.int64)
            sg = blocks[:, 14 * k + 10:14 * k + 14].astype(np.int64)
            for j in range(32):
                idx = (qs[:, j // 4] >> ((j % 4) * 2)) & 0x3
                idx |= ((sg[:, j // 8] >> (j % 8)) & 1) << 2
                codes[:, 32 * k + j] = idx
        return norms, codes, {}
    if fmt == synth.TQ3K:
        norms = _u16(blocks[:, 0], blocks[:, 1])[:, None]
        gam = _u16(blocks[:, 2], blocks[:, 3])
        qs = blocks[:, 4:4 + d // 4].astype(np.int64)
        qj = blocks[:, 4 + d // 4:].astype(np.int64)
        codes = np.zeros((n, d), np.int64)
        bits = np.zeros((n, d), np.int64)
        for j in range(d):
            codes[:, j] = (qs[:, j // 4] >> (2 * (j % 4))) & 3
            bits[:, j] = (qj[:, j // 8] >> (j % 8)) & 1
        return norms, codes, {"gamma": gam, "bits": bits}
    raise ValueError(fmt)


def _fp16_neighbor_ok(bits_a, bits_b, x64):
    """fp16 encodings one ulp apart with x on (or within 1e-6 of) their midpoint."""
    a = bits_a.view(np.float16).astype(np.float64)
    b = bits_b.view(np.float16).astype(np.float64)
    one_ulp = np.abs(bits_a.astype(np.int64) - bits_b.astype(np.int64)) == 1
    mid = 0.5 * (a + b)
    return one_ulp & (np.abs(x64 - mid) <= 1e-6 * np.maximum(np.abs(x64), 1e-30))


def compare_write(setup, tensor, gpu_blocks, enc):
    """Check GPU blocks against the oracle encoding of the same rows.

    Returns counts of tolerated differences; raises AssertionError otherwise.
    """
    w = setup.w
    d = w.head_dim
    fmt = w.k_format if tensor == synth.K_TENSOR else w.v_format
    tabs = setup.tk if tensor == synth.K_TENSOR else setup.tv
    stats = {"vectors": gpu_blocks.shape[0], "code_flips": 0, "norm_flips": 0, "gamma_flips": 0, "qjl_flips": 0,
             "bytes_equal": bool(np.array_equal(gpu_blocks, enc.blocks))}
    if fmt in (synth.GQ2V, synth.GQ4V):
        assert np.array_equal(gpu_blocks, enc.blocks), "group-quantized value blocks must be bit-exact"
        return stats
    if stats["bytes_equal"]:
        return stats
    gn, gc, gx = parse_codes(fmt, gpu_blocks, d)
    on, oc, ox = parse_codes(fmt, enc.blocks, d)
    if fmt == synth.PQ4:
        assert np.all(gx["reserved"] == 0)
    # codes: only adjacent codes across a boundary the oracle's coordinate touches
    diff = gc != oc
    if diff.any():
        v, j = np.nonzero(diff)
        assert np.all(np.abs(gc[v, j] - oc[v, j]) == 1), "non-adjacent code mismatch"
        k = np.minimum(gc[v, j], oc[v, j])
        dist = np.abs(enc.y[v, j] - tabs.bounds[k].astype(np.float64))
        assert np.all(dist <= BOUNDARY_EPS), f"code mismatch {dist.max():.3g} from a boundary"
        stats["code_flips"] = int(diff.sum())
    ndiff = gn != on
    if ndiff.any():
        v, _ = np.nonzero(ndiff)
        ok = _fp16_neighbor_ok(gn[ndiff], on[ndiff], np.minimum(enc.norm[v], 65504.0))
        assert np.all(ok), "norm mismatch beyond an fp16 rounding tie"
        stats["norm_flips"] = int(ndiff.sum())
    if fmt == synth.TQ3K:
        flipped_vec = diff.any(axis=1)
        gd = (gx["gamma"] != ox["gamma"]) & ~flipped_vec
        if gd.any():
            ok = _fp16_neighbor_ok(gx["gamma"][gd], ox["gamma"][gd], enc.extra["gamma"][gd])
            assert np.all(ok), "residual norm mismatch beyond an fp16 rounding tie"
            stats["gamma_flips"] = int(gd.sum())
        bd = (gx["bits"] != ox["bits"]) & ~flipped_vec[:, None]
        if bd.any():
            v, i = np.nonzero(bd)
            proj = enc.extra["proj"][v, i]
            rowscale = np.linalg.norm(setup.S_o.astype(np.float64), axis=1)[i] * enc.extra["gamma"][v]
            assert np.all(np.abs(proj) <= 1e-5 * rowscale), "QJL sign mismatch away from zero"
            stats["qjl_flips"] = int(bd.sum())
        stats["vectors_with_code_flips"] = int(flipped_vec.sum())
    return stats


# ---------------------------------------------------------------------------
# read side


def cs_scale(q_row, kd):
    """|q| max_i |k_hat_i| / sqrt(d): the largest score any of these keys could give q
    (Cauchy-Schwarz), the natural scale of a row of scores."""
    if kd.shape[0] == 0:
        return 0.0
    return float(np.linalg.norm(np.asarray(q_row, np.float64)) * np.max(np.linalg.norm(kd, axis=1))
                 / np.sqrt(kd.shape[1]))


def score_err(got, ref, cs):
    """max_i |got_i - ref_i| over max(max_i |ref_i|, cs / 10).  The plain max_i |ref_i|
    of the output tolerance is ill-conditioned when every score of a row nearly cancels
    (a one-token row whose score is 0.0075 with cs = 27); a tenth of the row's
    Cauchy-Schwarz scale bounds the denominator away from zero and leaves ordinary rows,
    whose largest score is far above it, unchanged."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = max(float(np.max(np.abs(ref))), 0.1 * cs)
    num = float(np.max(np.abs(got - ref)))
    return num / den if den > 0 else num


def rel_err_rows(got, ref):
    """max_j |got - ref| / max_j |ref| per row (last axis)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.max(np.abs(ref), axis=-1)
    num = np.max(np.abs(got - ref), axis=-1)
    return np.where(den > 0, num / np.where(den > 0, den, 1), num)


def gpu_decode(setup, L, q, k_cache, v_cache, seq_lens, split_tokens=0, want_scores=True, partial_only=False):
    """Rotate/sketch the queries and run the fused decode; returns numpy arrays."""
    w = setup.w
    d = w.head_dim
    qd = torch.from_numpy(np.ascontiguousarray(q, np.float32)).cuda()
    q_rot = torch.empty_like(qd)
    q_sk = torch.empty_like(qd) if w.k_format == synth.TQ3K else None
    tq.rotate_sketch_query(L, setup.cbk, setup.S_dev, qd, q_rot, q_sk)
    out = torch.full((L.batch, L.n_q_heads, d), float("nan"), device="cuda")
    ws = tq.decode_workspace(L, split_tokens)
    scores = torch.full((L.batch, L.n_q_heads, L.capacity), float("nan"), device="cuda") if want_scores else None
    sl = torch.tensor(np.asarray(seq_lens, np.int32), device="cuda")
    tq.decode_attention(L, setup.cbk, setup.cbv, q_rot, q_sk, k_cache, v_cache, sl, out, ws, scores=scores,
                        split_tokens=split_tokens)
    torch.cuda.synchronize()
    return (out.cpu().numpy(), None if scores is None else scores.cpu().numpy(), q_rot.cpu().numpy(),
            None if q_sk is None else q_sk.cpu().numpy())


def oracle_decode(setup, q, kdq, vdq, seq_lens):
    """Oracle attention over dequantized streams kdq[b][h], vdq[b][h] ([N, d])."""
    return oatt.decode_attention(q, kdq, vdq, seq_lens, setup.w.group)


def check_read(setup, q, kdq, vdq, seq_lens, out, scores, capacity):
    """Compare GPU outputs/scores with the oracle; returns (worst score err, worst out err)."""
    ref_out, ref_logits = oracle_decode(setup, q, kdq, vdq, seq_lens)
    B, Hq = q.shape[:2]
    worst_s, worst_o = 0.0, 0.0
    for b in range(B):
        n = int(seq_lens[b])
        for g in range(Hq):
            if n == 0:
                assert np.all(out[b, g] == 0), "empty context must give a zero output"
                continue
            if scores is not None:
                es = score_err(scores[b, g, :n], ref_logits[b][g], cs_scale(q[b, g], kdq[b][g // setup.w.group]))
                worst_s = max(worst_s, float(es))
                assert es <= SCORE_TOL, f"scores b={b} g={g}: {es:.3g}"
            eo = rel_err_rows(out[b, g], ref_out[b, g])
            worst_o = max(worst_o, float(eo))
            assert eo <= OUT_TOL, f"output b={b} g={g}: {eo:.3g}"
    return worst_s, worst_o


def place_streams(setup, L, tensor, blocks_by_stream):
    """Device cache of layout L holding the given per-(b, h) byte rows at positions 0..N-1."""
    vb = setup.vbk if tensor == synth.K_TENSOR else setup.vbv
    host = np.zeros((L.batch, L.n_kv_heads, L.capacity, vb), np.uint8)
    for (b, h), blk in blocks_by_stream.items():
        host[b, h, :blk.shape[0]] = blk
    return torch.from_numpy(host.reshape(-1)).cuda()
