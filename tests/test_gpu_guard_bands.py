"""Guard bands around every buffer a call writes, and unchanged inputs.

Each device buffer an entry point writes is the middle of a larger allocation
whose first and last 4 KiB hold a known byte; after the call those bytes must
be intact, so no kernel stores before or after the buffer it was given.  The
buffers a call only reads are compared with copies taken before it.  An
out-of-bounds store is the failure [P1] section 7 ("turbo4" revival) reports
finding by review (a 48-entry array written with 64 entries); these checks
catch that class of fault for every kernel family, at ragged lengths that
include an empty sequence, a one-token one, and one that fills the cache.
Values are checked by the parity tests, not here.
"""

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

tq = pytest.importorskip("compressed_domain_attention_kv_amd")

GUARD = 4096  # bytes on each side; keeps the buffer 256-byte aligned
FILL = 0x5A

# one workload per kernel family: the generic kernel (one query head), the
# matrix-core PQ3 and PQ3/PQ4 kernels, TQ3K keys with 2- and 4-bit values at
# d 128 and 256, PQ4 at four and eight heads per KV head with one and two
# centroid tables, and the d 256 PQ4 kernels
WORKLOADS = {
    "c1": synth.C1,
    "c2": synth.scaled(synth.C2, batch=2, n_q_heads=8, n_kv_heads=2, context=300, capacity=320),
    "pq3k_pq4v": synth.scaled(synth.C2, v_format=synth.PQ4, v_bits=4, batch=2, n_q_heads=4, n_kv_heads=1,
                              context=200, capacity=256),
    "c3": synth.scaled(synth.C3, batch=2, n_q_heads=10, n_kv_heads=2, context=300, capacity=320),
    "c3_gq4v_d256": synth.scaled(synth.C3, v_format=synth.GQ4V, v_bits=4, head_dim=256, batch=2, n_q_heads=8,
                                 n_kv_heads=2, context=200, capacity=256),
    "c4": synth.scaled(synth.C4, batch=3, n_q_heads=8, n_kv_heads=2, context=600, capacity=640),
    "c4_g8": synth.scaled(synth.C4, batch=2, n_q_heads=16, n_kv_heads=2, context=300, capacity=320),
    "c4_g8_lloyd_v": synth.scaled(synth.C4, v_kind=synth.LLOYD_MAX, batch=2, n_q_heads=16, n_kv_heads=2,
                                  context=300, capacity=320),
    "c5": synth.scaled(synth.C5, batch=3, n_q_heads=16, n_kv_heads=2, context=400, capacity=448),
    "c5_g4": synth.scaled(synth.C5, batch=2, n_q_heads=8, n_kv_heads=2, context=300, capacity=320),
    "c5_lloyd_v": synth.scaled(synth.C5, v_kind=synth.LLOYD_MAX, batch=2, n_q_heads=16, n_kv_heads=2,
                               context=300, capacity=320),
}


def _say(msg):
    print(msg, flush=True)


class Guarded:
    """A device buffer of nbytes (viewed as dtype) inside guard bands."""

    def __init__(self, nbytes, dtype=torch.uint8, fill=None):
        self.n = nbytes
        self.big = torch.full((nbytes + 2 * GUARD,), FILL, dtype=torch.uint8, device="cuda")
        if fill is not None:
            self.big[GUARD:GUARD + nbytes] = fill
        self.t = self.big[GUARD:GUARD + nbytes].view(dtype)

    def check(self, what):
        h = self.big.cpu().numpy()
        lo, hi = h[:GUARD], h[GUARD + self.n:]
        bad_lo, bad_hi = np.flatnonzero(lo != FILL), np.flatnonzero(hi != FILL)
        assert bad_lo.size == 0, f"{what}: {bad_lo.size} bytes written before the buffer (first at -{GUARD - bad_lo[0]})"
        assert bad_hi.size == 0, f"{what}: {bad_hi.size} bytes written after the buffer (first at +{bad_hi[0]})"


def _same(before, after, what):
    assert torch.equal(before, after), f"{what} was modified by a call that only reads it"


def _new_rows(w, tensor, step):
    """fp16 [B, Hkv, d]: the row each (sequence, KV head) stream appends at a decode step."""
    rows = [[synth.appended(w, tensor, b, h, step) for h in range(w.n_kv_heads)] for b in range(w.batch)]
    return torch.from_numpy(np.ascontiguousarray(np.array(rows, dtype=np.float16))).cuda()


def _lens(w):
    # an empty sequence, a one-token one, a full cache, and ragged ones
    pick = [0, 1, w.capacity] + [max(1, w.context - 97 * b) for b in range(w.batch)]
    return pick[:w.batch] if w.batch > 1 else [w.capacity]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    yield


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_guard_bands_and_read_only_inputs(name):
    w = WORKLOADS[name]
    d, B, Hq, Hkv, cap = w.head_dim, w.batch, w.n_q_heads, w.n_kv_heads, w.capacity
    tq3k = w.k_format == synth.TQ3K
    cbk, S = tq.build_codebook(d, w.k_bits, w.k_kind, w.rot_seed_k, w.qjl_seed, want_qjl_matrix=tq3k)
    cbv, _ = tq.build_codebook(d, w.v_bits, w.v_kind, w.rot_seed_v, w.qjl_seed + 1)
    S_dev = torch.from_numpy(S).cuda() if tq3k else None
    L = tq.Layout(B, Hq, Hkv, d, cap, w.k_format, w.v_format)
    kb, vb = tq.cache_bytes(L)
    lens = _lens(w)
    _say(f"guard bands {name} lens={lens}")

    # --- bulk append of every position, into guarded caches
    kc, vc = Guarded(kb), Guarded(vb)
    k_rows = np.concatenate([synth.batch_rows(w, synth.K_TENSOR, b, 0, cap) for b in range(B)])
    v_rows = np.concatenate([synth.batch_rows(w, synth.V_TENSOR, b, 0, cap) for b in range(B)])
    k_new, v_new = torch.from_numpy(k_rows).cuda(), torch.from_numpy(v_rows).cuda()
    dst = torch.arange(B * cap, dtype=torch.int32, device="cuda")
    ins = [t.clone() for t in (k_new, v_new, dst)]
    tq.quantize_append(L, cbk, cbv, S_dev, k_new, v_new, dst, kc.t, vc.t)
    torch.cuda.synchronize()
    kc.check("quantize_append k_cache")
    vc.check("quantize_append v_cache")
    for a, b_, nm in zip(ins, (k_new, v_new, dst), ("k_new", "v_new", "dst_row")):
        _same(a, b_, f"quantize_append {nm}")

    # --- quantize_rotated, one format per side
    for fmt, cb in ((w.k_format, cbk), (w.v_format, cbv)):
        if fmt not in (synth.PQ4, synth.PQ3, synth.TQ3K):
            continue
        n = 777
        y = torch.from_numpy(synth.rotated_unit_rows(11 + fmt, n, d)).cuda()
        n16 = torch.full((n,), 1.5, dtype=torch.float16, device="cuda")
        blocks = Guarded(n * tq.vector_bytes(fmt, d))
        tq.quantize_rotated(fmt, cb, S_dev if fmt == synth.TQ3K else None, y, n16, blocks.t)
        torch.cuda.synchronize()
        blocks.check(f"quantize_rotated fmt {fmt} blocks")

    # --- query rotation
    q = torch.from_numpy(np.ascontiguousarray(synth.queries(w), np.float32)).cuda()
    nq = B * Hq * d * 4
    q_rot = Guarded(nq, torch.float32)
    q_sk = Guarded(nq, torch.float32) if tq3k else None
    q0 = q.clone()
    tq.rotate_sketch_query(L, cbk, S_dev, q, q_rot.t, q_sk.t if q_sk else None)
    torch.cuda.synchronize()
    q_rot.check("rotate_sketch_query q_rot")
    if q_sk:
        q_sk.check("rotate_sketch_query q_sketch")
    _same(q0, q, "rotate_sketch_query q")
    qr, qs = q_rot.t.view(B, Hq, d), (q_sk.t.view(B, Hq, d) if q_sk else None)

    sl = torch.tensor(np.asarray(lens, np.int32), device="cuda")
    reads = [kc.t.clone(), vc.t.clone(), qr.clone(), sl.clone()] + ([qs.clone()] if qs is not None else [])

    def unchanged(what):
        now = [kc.t, vc.t, qr, sl] + ([qs] if qs is not None else [])
        for a, b_, nm in zip(reads, now, ("k_cache", "v_cache", "q_rot", "seq_lens", "q_sketch")):
            _same(a, b_, f"{what} {nm}")

    for split in (0, 256):
        wsb = tq.decode_workspace_bytes(L, split)
        _say(f"  decode calls, split {split}: workspace {wsb} bytes")

        # full decode with scores
        ws, out = Guarded(wsb), Guarded(nq, torch.float32)
        scores = Guarded(B * Hq * cap * 4, torch.float32)
        tq.decode_workspace_init(L, ws.t, split)
        tq.decode_attention(L, cbk, cbv, qr, qs, kc.t, vc.t, sl, out.t.view(B, Hq, d), ws.t,
                            scores=scores.t.view(B, Hq, cap), split_tokens=split)
        torch.cuda.synchronize()
        for g, nm in ((ws, "ws"), (out, "out"), (scores, "scores")):
            g.check(f"decode_attention {nm}")
        unchanged("decode_attention")

        # partial + combine, and sparse V
        ws2, out2 = Guarded(wsb), Guarded(nq, torch.float32)
        tq.decode_workspace_init(L, ws2.t, split)
        tq.decode_partial(L, cbk, cbv, qr, qs, kc.t, vc.t, sl, ws2.t, split_tokens=split)
        tq.decode_combine(L, cbv, ws2.t, out2.t.view(B, Hq, d), split_tokens=split)
        tq.decode_partial_sparse_v(L, cbk, cbv, qr, qs, kc.t, vc.t, sl, ws2.t, 1e-3, split_tokens=split)
        torch.cuda.synchronize()
        ws2.check("decode_partial / decode_combine / decode_partial_sparse_v ws")
        out2.check("decode_combine out")
        unchanged("decode_partial")

        # the entry point on the library's own scratch
        out3 = Guarded(nq, torch.float32)
        tq.decode_attention_static(L, cbk, cbv, qr, qs, kc.t, vc.t, sl, out3.t.view(B, Hq, d), split_tokens=split)
        torch.cuda.synchronize()
        out3.check("decode_attention_static out")
        unchanged("decode_attention_static")

        if tq3k:
            continue  # the unrotated-query calls take no sketch
        # partial from the unrotated query
        ws4, scr = Guarded(wsb), Guarded(nq, torch.float32)
        sc4 = Guarded(B * Hq * cap * 4, torch.float32)
        tq.decode_workspace_init(L, ws4.t, split)
        tq.decode_partial_from_query(L, cbk, cbv, q, scr.t.view(B, Hq, d), kc.t, vc.t, sl, ws4.t,
                                     scores=sc4.t.view(B, Hq, cap), split_tokens=split)
        torch.cuda.synchronize()
        for g, nm in ((ws4, "ws"), (scr, "q_rot_scratch"), (sc4, "scores")):
            g.check(f"decode_partial_from_query {nm}")
        unchanged("decode_partial_from_query")
        _same(q0, q, "decode_partial_from_query q")

        # decode step: appends at each sequence's next free position (the full
        # sequence's position is the capacity, which the step skips)
        kcs, vcs = Guarded(kb, fill=kc.t), Guarded(vb, fill=vc.t)
        ws5, scr5, out5 = Guarded(wsb), Guarded(nq, torch.float32), Guarded(nq, torch.float32)
        sc5 = Guarded(B * Hq * cap * 4, torch.float32)
        tq.decode_workspace_init(L, ws5.t, split)
        kn, vn = _new_rows(w, synth.K_TENSOR, 0), _new_rows(w, synth.V_TENSOR, 0)
        pos = torch.tensor(np.asarray(lens, np.int32), device="cuda")
        sl5 = torch.tensor(np.asarray([min(n + 1, cap) for n in lens], np.int32), device="cuda")
        tq.decode_step(L, cbk, cbv, kn, vn, pos, q, scr5.t.view(B, Hq, d), kcs.t,
                       vcs.t, sl5, ws5.t, out=out5.t.view(B, Hq, d), scores=sc5.t.view(B, Hq, cap),
                       split_tokens=split)
        torch.cuda.synchronize()
        for g, nm in ((kcs, "k_cache"), (vcs, "v_cache"), (ws5, "ws"), (scr5, "q_rot_scratch"), (out5, "out"),
                      (sc5, "scores")):
            g.check(f"decode_step {nm}")
        _same(q0, q, "decode_step q")

    # --- capture ring: append, flush into guarded caches, hybrid read
    for ring_cap in (64, 256):
        rb = tq.ring_bytes(L, ring_cap)
        kr, vr = Guarded(rb, torch.float16, fill=0), Guarded(rb, torch.float16, fill=0)
        for step in range(3):
            kn, vn = _new_rows(w, synth.K_TENSOR, step), _new_rows(w, synth.V_TENSOR, step)
            pos = torch.tensor([ring_cap - 2 + step + 5 * b for b in range(B)], dtype=torch.int32, device="cuda")
            tq.ring_append(L, ring_cap, kn, vn, pos, kr.t, vr.t)
        torch.cuda.synchronize()
        kr.check(f"ring_append k_ring (cap {ring_cap})")
        vr.check(f"ring_append v_ring (cap {ring_cap})")

        kcf, vcf = Guarded(kb, fill=kc.t), Guarded(vb, fill=vc.t)
        rings = (kr.t.clone(), vr.t.clone())
        first = torch.tensor([cap - 3 + b for b in range(B)], dtype=torch.int32, device="cuda")
        tq.ring_flush(L, cbk, cbv, S_dev, ring_cap, kr.t, vr.t, first, min(ring_cap, 8), kcf.t, vcf.t)
        torch.cuda.synchronize()
        kcf.check(f"ring_flush k_cache (cap {ring_cap})")
        vcf.check(f"ring_flush v_cache (cap {ring_cap})")
        _same(rings[0], kr.t, "ring_flush k_ring")
        _same(rings[1], vr.t, "ring_flush v_ring")

        comp = torch.tensor([max(0, n - 3) for n in lens], dtype=torch.int32, device="cuda")
        rl = torch.tensor([min(3, n) for n in lens], dtype=torch.int32, device="cuda")
        ws6 = Guarded(tq.decode_hybrid_workspace_bytes(L))
        out6 = Guarded(nq, torch.float32)
        tq.decode_attention_hybrid(L, cbk, cbv, qr, qs, kc.t, vc.t, comp, ring_cap, kr.t, vr.t, rl,
                                   out6.t.view(B, Hq, d), ws6.t)
        torch.cuda.synchronize()
        ws6.check(f"decode_attention_hybrid ws (cap {ring_cap})")
        out6.check(f"decode_attention_hybrid out (cap {ring_cap})")
        unchanged("decode_attention_hybrid")
        _same(rings[0], kr.t, "decode_attention_hybrid k_ring")
        _same(rings[1], vr.t, "decode_attention_hybrid v_ring")


def test_guard_check_sees_writes_next_to_the_buffer():
    """The check itself: a byte changed just before or just after the buffer
    (by a plain device fill, inside the larger allocation) is reported."""
    for where in (GUARD - 1, GUARD + 100):
        g = Guarded(100)
        g.big[where] = 0
        with pytest.raises(AssertionError):
            g.check("planted")
    g = Guarded(100)
    g.t.fill_(0)  # the buffer itself may be written
    g.check("inside")
