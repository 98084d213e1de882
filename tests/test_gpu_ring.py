"""GPU parity of the capture ring and the hybrid read, through the C ABI.

The ring keeps the newest tokens exact (fp16) and a flush quantizes its
oldest batch into the compressed cache ("TurboQuant Triton deep dive", write
path); the hybrid read attends over the compressed history and the exact
ring tokens together (same page, limits section).  Ring placement: the token
at absolute position pos of a sequence lives in slot pos % ring_cap.
"""

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

tq = pytest.importorskip("compressed_domain_attention_kv_amd")
P = pytest.importorskip("parity")

NAN16 = 0x7E00  # fp16 NaN: every ring slot the kernels must not read holds it

WORKLOADS = {
    "c4": synth.scaled(synth.C4, batch=4, n_q_heads=8, n_kv_heads=2, context=600, capacity=640),
    "c2": synth.scaled(synth.C2, batch=2, n_q_heads=8, n_kv_heads=2, context=500, capacity=512),
    "c3": synth.scaled(synth.C3, batch=2, n_q_heads=10, n_kv_heads=2, context=400, capacity=448),
    "c5": synth.scaled(synth.C5, batch=2, n_q_heads=16, n_kv_heads=2, context=300, capacity=320),
    "c4_g8": synth.scaled(synth.C4, batch=2, n_q_heads=16, n_kv_heads=2, context=300, capacity=320),
    "c3_h3": synth.scaled(synth.C3, batch=3, n_q_heads=12, n_kv_heads=3, context=600, capacity=640),
}


def _say(msg):
    print(msg, flush=True)


def _rows(w, tensor, b, h, start, count):
    return synth.stream(w, tensor, b, h, start, count)


def _ring_host(w, cap, comp, n):
    """Ring tensors holding tokens comp[b] .. comp[b]+n[b]-1 at slot pos % cap, NaN elsewhere."""
    kr = np.full((w.batch, w.n_kv_heads, cap, w.head_dim), NAN16, np.uint16)
    vr = kr.copy()
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            slots = (comp[b] + np.arange(n[b])) % cap
            kr[b, h, slots] = _rows(w, synth.K_TENSOR, b, h, comp[b], n[b]).view(np.uint16)
            vr[b, h, slots] = _rows(w, synth.V_TENSOR, b, h, comp[b], n[b]).view(np.uint16)
    return kr, vr


@pytest.mark.parametrize("cap", [1, 64, 96, 256])
def test_ring_append_places_rows_at_pos_mod_cap(cap):
    w = WORKLOADS["c4"]
    L = P.Setup(w).layout()
    kr = torch.full((tq.ring_bytes(L, cap) // 2,), NAN16, dtype=torch.int16, device="cuda")
    vr = torch.full_like(kr, NAN16)
    ref_k = np.full((w.batch, w.n_kv_heads, cap, w.head_dim), NAN16, np.uint16)
    ref_v = ref_k.copy()
    rng = np.random.default_rng(cap)
    for step in range(3):
        pos = rng.integers(0, 5000, w.batch).astype(np.int32)
        pos[step % w.batch] = -1  # skipped sequence
        kn = rng.integers(0, 0x7C00, (w.batch, w.n_kv_heads, w.head_dim)).astype(np.uint16)
        vn = rng.integers(0, 0x7C00, (w.batch, w.n_kv_heads, w.head_dim)).astype(np.uint16)
        tq.ring_append(L, cap, torch.from_numpy(kn.view(np.int16)).cuda(), torch.from_numpy(vn.view(np.int16)).cuda(),
                       torch.from_numpy(pos).cuda(), kr, vr)
        for b in range(w.batch):
            if pos[b] >= 0:
                ref_k[b, :, pos[b] % cap] = kn[b]
                ref_v[b, :, pos[b] % cap] = vn[b]
    torch.cuda.synchronize()
    assert np.array_equal(kr.cpu().numpy().view(np.uint16).reshape(ref_k.shape), ref_k)
    assert np.array_equal(vr.cpu().numpy().view(np.uint16).reshape(ref_v.shape), ref_v)


@pytest.mark.parametrize("name", ["c4", "c2", "c3", "c5", "c3_h3"])
def test_ring_flush_writes_what_append_would(name):
    """Flushing count ring tokens (wrapping around the ring) writes the blocks the
    oracle encodes for those rows, at their absolute positions, and nothing else."""
    w = WORKLOADS[name]
    st = P.Setup(w)
    L = st.layout()
    cap, count = 96, 80
    first = [37 + 101 * b for b in range(w.batch)]  # ring slots wrap for every sequence
    kr, vr = _ring_host(w, cap, first, [cap] * w.batch)
    kc_bytes, vc_bytes = tq.cache_bytes(L)
    kc = torch.full((kc_bytes,), 0xEE, dtype=torch.uint8, device="cuda")
    vc = torch.full((vc_bytes,), 0xEE, dtype=torch.uint8, device="cuda")
    tq.ring_flush(L, st.cbk, st.cbv, st.S_dev, cap, torch.from_numpy(kr.view(np.int16)).cuda(),
                  torch.from_numpy(vr.view(np.int16)).cuda(), torch.tensor(first, dtype=torch.int32, device="cuda"),
                  count, kc, vc)
    torch.cuda.synchronize()
    kh = kc.cpu().numpy().reshape(w.batch, w.n_kv_heads, w.capacity, st.vbk)
    vh = vc.cpu().numpy().reshape(w.batch, w.n_kv_heads, w.capacity, st.vbv)
    flips = vectors = 0
    for b in range(w.batch):
        lo, hi = first[b], min(first[b] + count, w.capacity)
        outside = np.ones(w.capacity, bool)
        outside[lo:hi] = False
        assert np.all(kh[b][:, outside] == 0xEE) and np.all(vh[b][:, outside] == 0xEE)
        for h in range(w.n_kv_heads):
            for tensor, cache in ((synth.K_TENSOR, kh), (synth.V_TENSOR, vh)):
                enc = st.oracle_encode(tensor, _rows(w, tensor, b, h, lo, hi - lo))
                s = P.compare_write(st, tensor, cache[b, h, lo:hi], enc)
                flips += int(s.get("code_flips", 0))
                vectors += int(s["vectors"])
    _say(f"flush {name}: {vectors} vectors, {flips} tolerated code flips")
    assert flips <= max(2, 1e-4 * vectors * w.head_dim)


def _hybrid_case(name, comp, n, cap, split=0):
    w = WORKLOADS[name]
    st = P.Setup(w)
    L = st.layout()
    _say(f"hybrid {name} cap={cap} comp={comp} ring={n} split={split}")
    host_k = np.full((w.batch, w.n_kv_heads, w.capacity, st.vbk), 0xFF, np.uint8)
    host_v = np.full((w.batch, w.n_kv_heads, w.capacity, st.vbv), 0xFF, np.uint8)
    kdq, vdq = {}, {}
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            ek = st.oracle_encode(synth.K_TENSOR, _rows(w, synth.K_TENSOR, b, h, 0, max(comp[b], 1)))
            ev = st.oracle_encode(synth.V_TENSOR, _rows(w, synth.V_TENSOR, b, h, 0, max(comp[b], 1)))
            host_k[b, h, :comp[b]] = ek.blocks[:comp[b]]
            host_v[b, h, :comp[b]] = ev.blocks[:comp[b]]
            kdq[(b, h)] = st.oracle_dequant(synth.K_TENSOR, ek.blocks)[:comp[b]]
            vdq[(b, h)] = st.oracle_dequant(synth.V_TENSOR, ev.blocks)[:comp[b]]
    kr, vr = _ring_host(w, cap, comp, n)
    q = synth.queries(w)
    qd = torch.from_numpy(q).cuda()
    q_rot = torch.empty_like(qd)
    q_sk = torch.empty_like(qd) if w.k_format == synth.TQ3K else None
    tq.rotate_sketch_query(L, st.cbk, st.S_dev, qd, q_rot, q_sk)
    out = torch.full_like(qd, float("nan"))
    ws = torch.empty(tq.decode_hybrid_workspace_bytes(L, split), dtype=torch.uint8, device="cuda")
    tq.decode_attention_hybrid(L, st.cbk, st.cbv, q_rot, q_sk, torch.from_numpy(host_k.reshape(-1)).cuda(),
                               torch.from_numpy(host_v.reshape(-1)).cuda(),
                               torch.tensor(comp, dtype=torch.int32, device="cuda"), cap,
                               torch.from_numpy(kr.view(np.int16)).cuda(), torch.from_numpy(vr.view(np.int16)).cuda(),
                               torch.tensor(n, dtype=torch.int32, device="cuda"), out, ws, split_tokens=split)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    worst = 0.0
    for b in range(w.batch):
        for g in range(w.n_q_heads):
            h = g // w.group
            kx = _rows(w, synth.K_TENSOR, b, h, comp[b], n[b]).astype(np.float64)
            vx = _rows(w, synth.V_TENSOR, b, h, comp[b], n[b]).astype(np.float64)
            ref, _ = P.oatt.hybrid_attention(q[b, g], kdq[(b, h)], vdq[(b, h)], kx, vx)
            if comp[b] + n[b] == 0:
                assert np.all(o[b, g] == 0.0)
                continue
            e = float(P.rel_err_rows(o[b, g], ref))
            worst = max(worst, e)
            assert e <= P.OUT_TOL, (b, g, e)
    _say(f"  worst output err {worst:.2e}")


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_hybrid_matches_oracle(name):
    w = WORKLOADS[name]
    cap = 128
    comp = [w.context - 128 - 41 * b for b in range(w.batch)]
    n = [128 - 37 * b for b in range(w.batch)]
    _hybrid_case(name, comp, n, cap)


@pytest.mark.parametrize("name,cap", [("c4", 256), ("c4", 201), ("c5", 256), ("c5", 130)])
def test_hybrid_long_rings(name, cap):
    """Rings longer than 128 tokens (the 256-token kernels; at d = 256 and 256
    tokens the value rows are staged after the scores), full and partial,
    with lengths that are not multiples of four."""
    w = WORKLOADS[name]
    comp = [w.context - cap - 11 * b for b in range(w.batch)]
    n = [cap - 37 * b for b in range(w.batch)]
    _hybrid_case(name, comp, n, cap)


def test_hybrid_edge_lengths():
    """Empty ring, empty compressed part, both empty, a full ring that wraps,
    and a single ring token, in one batch of six sequences."""
    base = WORKLOADS["c4"]
    WORKLOADS["c4_edges"] = synth.scaled(base, batch=6)
    try:
        comp = [300, 0, 0, 511, 5, 257]
        n = [0, 64, 0, 64, 1, 64]
        _hybrid_case("c4_edges", comp, n, 64)
        _hybrid_case("c4_edges", comp, n, 64, split=256)
    finally:
        del WORKLOADS["c4_edges"]


def test_ring_lifecycle_append_flush_read():
    """A decode loop: every step appends one token per sequence to the ring;
    when a ring is full its oldest half is flushed into the compressed cache;
    the hybrid read after each step matches the oracle over the same split of
    tokens (compressed rows encoded by the oracle from the same fp16 rows)."""
    w = WORKLOADS["c4"]
    st = P.Setup(w)
    L = st.layout()
    cap, half = 32, 16
    B, H, d = w.batch, w.n_kv_heads, w.head_dim
    start = [100 + 30 * b for b in range(B)]
    kc = torch.zeros(tq.cache_bytes(L)[0], dtype=torch.uint8, device="cuda")
    vc = torch.zeros(tq.cache_bytes(L)[1], dtype=torch.uint8, device="cuda")
    for b in range(B):  # compressed prefix of every sequence, through the HIP encoder
        rows_k = np.stack([_rows(w, synth.K_TENSOR, b, h, 0, start[b]) for h in range(H)], axis=1)
        rows_v = np.stack([_rows(w, synth.V_TENSOR, b, h, 0, start[b]) for h in range(H)], axis=1)
        dst = torch.arange(b * w.capacity, b * w.capacity + start[b], dtype=torch.int32, device="cuda")
        tq.quantize_append(L, st.cbk, st.cbv, None, torch.from_numpy(rows_k).cuda(), torch.from_numpy(rows_v).cuda(),
                           dst, kc, vc)
    kr = torch.full((tq.ring_bytes(L, cap) // 2,), NAN16, dtype=torch.int16, device="cuda")
    vr = torch.full_like(kr, NAN16)
    comp, n = list(start), [0] * B
    q = synth.queries(w)
    qd = torch.from_numpy(q).cuda()
    q_rot = torch.empty_like(qd)
    tq.rotate_sketch_query(L, st.cbk, None, qd, q_rot, None)
    ws = torch.empty(tq.decode_hybrid_workspace_bytes(L), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(qd)
    for step in range(40):
        pos = [comp[b] + n[b] for b in range(B)]
        kn = np.stack([np.stack([_rows(w, synth.K_TENSOR, b, h, pos[b], 1)[0] for h in range(H)]) for b in range(B)])
        vn = np.stack([np.stack([_rows(w, synth.V_TENSOR, b, h, pos[b], 1)[0] for h in range(H)]) for b in range(B)])
        tq.ring_append(L, cap, torch.from_numpy(kn).cuda(), torch.from_numpy(vn).cuda(),
                       torch.tensor(pos, dtype=torch.int32, device="cuda"), kr, vr)
        n = [x + 1 for x in n]
        if n[0] == cap:  # all sequences fill together: flush the oldest half
            tq.ring_flush(L, st.cbk, st.cbv, None, cap, kr, vr, torch.tensor(comp, dtype=torch.int32, device="cuda"),
                          half, kc, vc)
            comp = [x + half for x in comp]
            n = [x - half for x in n]
        if step % 13 == 12 or step == 39:
            tq.decode_attention_hybrid(L, st.cbk, st.cbv, q_rot, None, kc, vc,
                                       torch.tensor(comp, dtype=torch.int32, device="cuda"), cap, kr, vr,
                                       torch.tensor(n, dtype=torch.int32, device="cuda"), out, ws)
            torch.cuda.synchronize()
            o = out.cpu().numpy()
            gk = kc.view(B, H, w.capacity, st.vbk).cpu().numpy()
            gv = vc.view(B, H, w.capacity, st.vbv).cpu().numpy()
            flips = 0
            for b in range(B):
                for h in range(H):
                    # the GPU encoder wrote the compressed rows (prefill and flushes): checked
                    # against the oracle's encoding of the same fp16 rows, then decoded by the
                    # oracle from the GPU's own bytes, so the read bound holds unchanged
                    ek = st.oracle_encode(synth.K_TENSOR, _rows(w, synth.K_TENSOR, b, h, 0, comp[b]))
                    ev = st.oracle_encode(synth.V_TENSOR, _rows(w, synth.V_TENSOR, b, h, 0, comp[b]))
                    sk = P.compare_write(st, synth.K_TENSOR, gk[b, h, :comp[b]], ek)
                    sv = P.compare_write(st, synth.V_TENSOR, gv[b, h, :comp[b]], ev)
                    flips += sk["code_flips"] + sv["code_flips"]
                    kd = st.oracle_dequant(synth.K_TENSOR, gk[b, h, :comp[b]])
                    vd = st.oracle_dequant(synth.V_TENSOR, gv[b, h, :comp[b]])
                    for g in range(h * w.group, (h + 1) * w.group):
                        ref, _ = P.oatt.hybrid_attention(
                            q[b, g], kd, vd, _rows(w, synth.K_TENSOR, b, h, comp[b], n[b]).astype(np.float64),
                            _rows(w, synth.V_TENSOR, b, h, comp[b], n[b]).astype(np.float64))
                        assert P.rel_err_rows(o[b, g], ref) <= P.OUT_TOL, (step, b, g)
            _say(f"  step {step}: comp={comp} ring={n} ok (boundary code flips {flips})")
