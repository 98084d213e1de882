"""Per-token score error of the matrix-core decode kernels against the analytic bound of
their bf16 hi/lo operands.

Every fp32 operand x of the score products (the scaled rotated query, the centroids) enters
as hi = bf16(x) and lo = bf16(x - hi), so |x - hi - lo| <= 2^-16 |x|; all four cross terms
are summed, products are exact in fp32 and sums are fp32.  For a token whose coordinate j
lies in a block of norm n_b(j) and has centroid c_j:

    |s_gpu - s| <= (2^-15 + d 2^-24 + 2e-6) sum_j n_b(j) |q_j| |c_j| / sqrt(d)

(2^-15: the operand splits; d 2^-24: the fp32 sums; 2e-6: the fp32 query rotation, the norm
products and the scale back to natural-log units).  The keys are chosen to stress the bound:
every eighth token has a norm of 1000 and a quarter of the tokens have codes picked so that
their score against the first query head nearly cancels.  The oracle packs the bytes (PQ4,
and PQ3 with a different norm per 32-coordinate block), both sides attend over them, and
the check holds for every token and query head.  Kernels: the 2:4-sparse one (PQ4 at four
and eight query heads per KV head, PQ3 keys) and the dense one (PQ4 at d 256).  TQ3K keys
(a second, sign-sketch term) are not covered here."""

import numpy as np
import pytest
import torch

import synth
from oracle import formats as ofmt
from oracle import rotation as orot

pytestmark = pytest.mark.gpu

tq = pytest.importorskip("compressed_domain_attention_kv_amd")
P = pytest.importorskip("parity")

CASES = {
    "pq4_g4": synth.scaled(synth.C4, batch=1, n_q_heads=4, n_kv_heads=1, context=512, capacity=512),
    "pq4_g8": synth.scaled(synth.C4, batch=1, n_q_heads=8, n_kv_heads=1, context=512, capacity=512),
    "pq4_d256": synth.scaled(synth.C5, batch=1, n_q_heads=8, n_kv_heads=1, context=512, capacity=512),
    "pq3_g4": synth.scaled(synth.C2, batch=1, n_q_heads=4, n_kv_heads=1, context=512, capacity=512),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    yield


def _near_cancelling_codes(rng, qr, cent, levels, nblk):
    """Codes [d] whose sum_j qr_j cent[code_j] (per block weight nblk[j]) nearly cancels:
    coordinates in random order, each taking the level that brings the partial sum
    closest to zero, then a second pass over all coordinates."""
    d = qr.shape[0]
    code = rng.integers(0, levels, size=d)
    total = float(np.sum(nblk * qr * cent[code]))
    for _ in range(2):
        for j in rng.permutation(d):
            rest = total - nblk[j] * qr[j] * cent[code[j]]
            cand = rest + nblk[j] * qr[j] * cent[:levels]
            best = int(np.argmin(np.abs(cand)))
            code[j] = best
            total = float(cand[best])
    return code


@pytest.mark.parametrize("name", list(CASES))
def test_scores_within_the_hi_lo_bound(name):
    w = CASES[name]
    st = P.Setup(w)
    L = st.layout()
    d, N = w.head_dim, w.context
    fmt = w.k_format
    levels = 1 << w.k_bits
    blk = 128 if fmt == synth.PQ4 else 32
    nb = d // blk
    rng = np.random.default_rng(11)
    q = synth.queries(w)                                  # [1, Hq, d]
    qr = orot.rotate(q[0].astype(np.float64), st.sk)     # rotated queries [Hq, d]
    cent = st.tk.centroids.astype(np.float64)
    # block norms: U[0.8, 1.2], every eighth token 1000 (PQ4 at d 256 stores one norm per vector)
    norms = rng.uniform(0.8, 1.2, size=(N, nb))
    norms[::8] = 1000.0
    if fmt == synth.PQ4:
        norms[:, :] = norms[:, :1]
    norms16 = norms.astype(np.float16)
    nb64 = norms16.astype(np.float64)
    codes = rng.integers(0, levels, size=(N, d))
    for t in range(1, N, 4):  # a quarter of the tokens: near-cancelling against query head 0
        nj = np.repeat(nb64[t], blk)
        codes[t] = _near_cancelling_codes(rng, qr[0], cent, levels, nj)
    if fmt == synth.PQ4:
        kbytes = ofmt.pack_pq4(norms16[:, 0], codes)
    else:
        kbytes = np.concatenate([ofmt.pack_pq3(norms16[:, b], codes[:, blk * b:blk * (b + 1)]) for b in range(nb)],
                                axis=1)
    vrows = synth.stream(w, synth.V_TENSOR, 0, 0, 0, N)
    vbytes = st.oracle_encode(synth.V_TENSOR, vrows).blocks
    kc = P.place_streams(st, L, synth.K_TENSOR, {(0, 0): kbytes})
    vc = P.place_streams(st, L, synth.V_TENSOR, {(0, 0): vbytes})
    _, scores, _, _ = P.gpu_decode(st, L, q, kc, vc, [N])
    kd = st.oracle_dequant(synth.K_TENSOR, kbytes)       # [N, d], unrotated
    exact = (q[0].astype(np.float64) @ kd.T) / np.sqrt(d)  # [Hq, N]
    got = scores[0, :, :N].astype(np.float64)
    # the bound's sum: sum_j n_b(j) |q_j| |c_j| / sqrt(d), per head and token
    nj = np.repeat(nb64, blk, axis=1)                    # [N, d]
    mag = (np.abs(qr)[:, None, :] * (nj * np.abs(cent[codes]))[None, :, :]).sum(axis=2) / np.sqrt(d)
    bound = (2.0 ** -15 + d * 2.0 ** -24 + 2e-6) * mag
    err = np.abs(got - exact)
    ratio = err / bound
    cancel = np.abs(exact[0, 1::4]) / mag[0, 1::4]
    print(f"{name}: worst error / bound {ratio.max():.3f}, median {np.median(ratio):.4f}; "
          f"near-cancelling |s| / scale median {np.median(cancel):.1e}", flush=True)
    assert np.all(np.isfinite(got))
    assert np.all(err <= bound), f"score error beyond the hi/lo bound: worst ratio {ratio.max():.3f}"
    assert np.median(cancel) < 1e-3  # the construction does cancel
