"""Decode at the longest stream a layout accepts.

One (batch row, KV head) stream holds the largest capacity the layout check
allows, so the decode kernels' byte offsets into the stream reach within a few
thousand vectors of 2^31.  Every token but the last 64 carries one key/value
pair (k0, v0) and the rest carry (k1, v1): either the last 64, with k1 along the
query so that its score leads by about 40 (natural-log units: the tail decides
the output), or the second half of the stream, with k1 of the size of k0 (the
two halves weigh about the same, so every token counts, and the small scores
keep the score rounding out of the comparison).
With two distinct tokens the softmax has a closed form over the oracle's
dequantization of the GPU-written blocks:

    o = (n0 e^(s0) v0 + n1 e^(s1) v1) / (n0 e^(s0) + n1 e^(s1)),

which the output must match to the output tolerance; a mis-addressed tail
(offsets wrapped, or read as zeros past a truncated range) would pull the
output towards v0.
"""

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

tq = pytest.importorskip("compressed_domain_attention_kv_amd")
P = pytest.importorskip("parity")

SLACK = 4096  # tokens the layout check keeps free past a stream's end
TAIL = 64


def _say(msg):
    print(msg, flush=True)


def _max_capacity(kf, vf, d):
    vb = max(tq.vector_bytes(kf, d), tq.vector_bytes(vf, d))
    cap = ((2**31 - 1) // vb - SLACK) // 64 * 64
    while (cap + SLACK) * vb > 2**31 - 1:
        cap -= 64
    return cap


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    yield


# the kernel families: the 2:4-sparse PQ4 kernel (four query heads per KV head), its PQ3 path,
# the d 256 byte-pair kernel (eight heads), the TQ3K-key kernel (five heads, GQ2V values), and
# the generic kernel (one head)
CASES = {
    "pq4_d128_g4": (synth.C4, 4, 128),
    "tq3k_gq2v_d128_g5": (synth.C3, 5, 128),
    "pq3_d128_g4": (synth.C2, 4, 128),
    "pq4_d256_g8": (synth.C5, 8, 256),
    "pq4_d128_g1": (synth.C1, 1, 128),
}


@pytest.mark.parametrize("balanced", [False, True], ids=["tail", "balanced"])
@pytest.mark.parametrize("name", list(CASES))
def test_decode_at_the_longest_accepted_stream(name, balanced):
    base, G, d = CASES[name]
    cap = _max_capacity(base.k_format, base.v_format, d)
    w = synth.scaled(base, batch=1, n_q_heads=G, n_kv_heads=1, head_dim=d, context=cap, capacity=cap)
    st = P.Setup(w)
    L = st.layout()
    kb, vb = tq.cache_bytes(L)
    _say(f"max stream {name}: capacity {cap}, K {kb / 2**30:.2f} GiB, V {vb / 2**30:.2f} GiB")

    # the two key/value rows, encoded by the library on a one-tile layout
    rng = np.random.default_rng(17 + d + G)
    q = np.zeros((1, G, d), np.float32)
    q[0, :] = rng.standard_normal(d).astype(np.float32)  # one query for every head of the group
    qn = q[0, 0] / np.linalg.norm(q[0, 0])
    k0 = (0.3 * rng.standard_normal(d)).astype(np.float16)
    n1 = cap // 2 // 64 * 64 if balanced else TAIL
    if balanced:
        k1 = (0.3 * rng.standard_normal(d)).astype(np.float16)
    else:
        k1 = (qn * (40.0 * np.sqrt(d) / np.linalg.norm(q[0, 0])) + 0.05 * rng.standard_normal(d)).astype(np.float16)
    v0 = rng.standard_normal(d).astype(np.float16)
    v1 = (rng.standard_normal(d) + 3.0).astype(np.float16)
    Ls = tq.Layout(1, G, 1, d, 64, w.k_format, w.v_format)
    kbs, vbs = tq.cache_bytes(Ls)
    kc_s = torch.zeros(kbs, dtype=torch.uint8, device="cuda")
    vc_s = torch.zeros(vbs, dtype=torch.uint8, device="cuda")
    tq.quantize_append(Ls, st.cbk, st.cbv, st.S_dev, torch.from_numpy(np.stack([k0, k1])[:, None]).cuda(),
                       torch.from_numpy(np.stack([v0, v1])[:, None]).cuda(),
                       torch.tensor([0, 1], dtype=torch.int32, device="cuda"), kc_s, vc_s)
    kblk = kc_s.view(64, st.vbk)[:2].clone()
    vblk = vc_s.view(64, st.vbv)[:2].clone()
    del kc_s, vc_s

    # the long stream: n0 copies of (k0, v0), then n1 copies of (k1, v1)
    n0 = cap - n1
    kc = torch.empty(kb, dtype=torch.uint8, device="cuda")
    vc = torch.empty(vb, dtype=torch.uint8, device="cuda")
    kc.view(cap, st.vbk)[:n0] = kblk[0]
    kc.view(cap, st.vbk)[n0:] = kblk[1]
    vc.view(cap, st.vbv)[:n0] = vblk[0]
    vc.view(cap, st.vbv)[n0:] = vblk[1]

    qd = torch.from_numpy(q).cuda()
    q_rot = torch.empty_like(qd)
    q_sk = torch.empty_like(qd) if w.k_format == synth.TQ3K else None
    tq.rotate_sketch_query(L, st.cbk, st.S_dev, qd, q_rot, q_sk)
    out = torch.full((1, G, d), float("nan"), device="cuda")
    # the balanced case on 8192-token splits: with the automatic split a wavefront may sum some
    # 20,000 equal terms (TQ3K keys, one split per 161,000 tokens), whose fp32 sums drift by up
    # to that count times 2^-24, about 1e-3, beside the output tolerance
    split = 8192 if balanced else 0
    ws = tq.decode_workspace(L, split)
    sl = torch.tensor([cap], dtype=torch.int32, device="cuda")
    tq.decode_attention(L, st.cbk, st.cbv, q_rot, q_sk, kc, vc, sl, out, ws, split_tokens=split)
    torch.cuda.synchronize()
    got = out.cpu().numpy()[0]
    del kc, vc, ws
    torch.cuda.empty_cache()

    # closed form over the oracle's dequantization of the GPU-written blocks
    khat = st.oracle_dequant(synth.K_TENSOR, kblk.cpu().numpy())
    vhat = st.oracle_dequant(synth.V_TENSOR, vblk.cpu().numpy())
    qq = q[0, 0].astype(np.float64)
    s = khat @ qq / np.sqrt(d)
    lead = s[1] - s[0]
    wts = np.array([n0 * np.exp(s[0] - s[1]), n1 * 1.0])
    ref = (wts[0] * vhat[0] + wts[1] * vhat[1]) / wts.sum()
    _say(f"  score lead {lead:.1f}, weight of the n0 tokens {wts[0] / wts.sum():.2e}")
    share = wts[0] / wts.sum()
    assert (0.05 < share < 0.95) if balanced else lead > 30.0
    for g in range(G):
        err = P.rel_err_rows(got[g], ref)
        assert err <= P.OUT_TOL, f"head {g}: relative error {err:.3g}"


@pytest.mark.parametrize("fmt_d", [(synth.PQ4, 128), (synth.PQ4, 256), (synth.PQ3, 128)], ids=["pq4_d128", "pq4_d256",
                                                                                                "pq3_d128"])
def test_append_at_the_end_of_the_longest_accepted_stream(fmt_d):
    """Rows appended at the last positions of the longest stream land there, byte for byte as
    the same rows encoded into a one-tile cache, and nothing else in the stream changes; at
    PQ4 d 128 also through the decode step, whose partial kernel writes the step's token."""
    fmt, d = fmt_d
    cap = _max_capacity(fmt, fmt, d)
    bits = 4 if fmt == synth.PQ4 else 3
    cbk, _ = tq.build_codebook(d, bits, 0, 5, 6)
    cbv, _ = tq.build_codebook(d, bits, 0, 7, 8)
    L = tq.Layout(1, 4, 1, d, cap, fmt, fmt)
    Ls = tq.Layout(1, 4, 1, d, 64, fmt, fmt)
    vb = tq.vector_bytes(fmt, d)
    kb, _ = tq.cache_bytes(L)
    _say(f"append at the end: fmt {fmt} d {d} capacity {cap} ({kb / 2**30:.2f} GiB per cache)")
    rng = np.random.default_rng(d + fmt)
    rows_k = rng.standard_normal((3, 1, d)).astype(np.float16)
    rows_v = rng.standard_normal((3, 1, d)).astype(np.float16)
    # reference bytes: the same rows at positions 0..2 of a one-tile cache
    ks = torch.zeros(tq.cache_bytes(Ls)[0], dtype=torch.uint8, device="cuda")
    vs = torch.zeros(tq.cache_bytes(Ls)[1], dtype=torch.uint8, device="cuda")
    tq.quantize_append(Ls, cbk, cbv, None, torch.from_numpy(rows_k).cuda(), torch.from_numpy(rows_v).cuda(),
                       torch.tensor([0, 1, 2], dtype=torch.int32, device="cuda"), ks, vs)
    ref_k = ks.view(64, vb)[:3].cpu().numpy()
    ref_v = vs.view(64, vb)[:3].cpu().numpy()

    kc = torch.full((kb,), 0xEE, dtype=torch.uint8, device="cuda")
    vc = torch.full((kb,), 0xEE, dtype=torch.uint8, device="cuda")
    pos = [cap - 3, cap - 2, cap - 1]
    tq.quantize_append(L, cbk, cbv, None, torch.from_numpy(rows_k).cuda(), torch.from_numpy(rows_v).cuda(),
                       torch.tensor(pos, dtype=torch.int32, device="cuda"), kc, vc)
    torch.cuda.synchronize()
    for cache, ref, nm in ((kc, ref_k, "k"), (vc, ref_v, "v")):
        tail = cache.view(cap, vb)[cap - 4:].cpu().numpy()
        assert np.all(tail[0] == 0xEE), f"{nm}: the row before the appended ones changed"
        assert np.array_equal(tail[1:], ref), f"{nm}: appended rows differ from the one-tile encoding"
        head = cache.view(cap, vb)[: cap - 4]
        assert bool((head == 0xEE).all()), f"{nm}: a row outside the appended ones changed"

    if fmt == synth.PQ4 and d == 128:
        # the decode step appends its token at the last position from inside the partial kernel
        kc.view(cap, vb)[cap - 1] = 0xEE
        vc.view(cap, vb)[cap - 1] = 0xEE
        q = torch.from_numpy(rng.standard_normal((1, 4, d)).astype(np.float32)).cuda()
        scratch = torch.empty_like(q)
        ws = tq.decode_workspace(L)
        sl = torch.tensor([cap], dtype=torch.int32, device="cuda")
        tq.decode_step(L, cbk, cbv, torch.from_numpy(rows_k[2:3]).cuda().view(1, 1, d),
                       torch.from_numpy(rows_v[2:3]).cuda().view(1, 1, d),
                       torch.tensor([cap - 1], dtype=torch.int32, device="cuda"), q, scratch, kc, vc, sl, ws)
        torch.cuda.synchronize()
        assert np.array_equal(kc.view(cap, vb)[cap - 1].cpu().numpy(), ref_k[2]), "decode step: key row"
        assert np.array_equal(vc.view(cap, vb)[cap - 1].cpu().numpy(), ref_v[2]), "decode step: value row"
        assert np.array_equal(kc.view(cap, vb)[cap - 3:cap - 1].cpu().numpy(), ref_k[:2])
    del kc, vc
    torch.cuda.empty_cache()
