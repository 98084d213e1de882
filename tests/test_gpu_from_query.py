"""tq_decode_partial_from_query on the GPU, through the C ABI: the partial from the
unrotated query writes the same split records as tq_rotate_sketch_query followed by
tq_decode_partial, bit for bit -- where the kernel rotates the query in its
prologue (PQ4, d 128, four query heads per KV head, one table) and where the
rotation runs as its own launch (every other case) -- and its output matches the
oracle."""

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

tq = pytest.importorskip("compressed_domain_attention_kv_amd")
P = pytest.importorskip("parity")

CASES = {
    "c4": synth.scaled(synth.C4, batch=3, n_q_heads=8, n_kv_heads=2, context=1300, capacity=1344),
    "c4_lloyd_v": synth.scaled(synth.C4, v_kind=synth.LLOYD_MAX, batch=2, n_q_heads=8, n_kv_heads=2, context=777,
                               capacity=832),
    "c4_g8": synth.scaled(synth.C4, batch=1, n_q_heads=16, n_kv_heads=2, context=1234, capacity=1280),
    "c5": synth.scaled(synth.C5, batch=2, n_q_heads=16, n_kv_heads=2, context=700, capacity=704),
    "c2": synth.scaled(synth.C2, batch=2, n_q_heads=8, n_kv_heads=2, context=777, capacity=832),
}


def _say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    yield


def _cache(st, w, L, lens):
    kb, vb, kdq, vdq = {}, {}, [], []
    for b in range(w.batch):
        kdq.append([])
        vdq.append([])
        for h in range(w.n_kv_heads):
            ek = st.oracle_encode(synth.K_TENSOR, synth.stream(w, synth.K_TENSOR, b, h, 0, max(lens[b], 1)))
            ev = st.oracle_encode(synth.V_TENSOR, synth.stream(w, synth.V_TENSOR, b, h, 0, max(lens[b], 1)))
            kb[(b, h)], vb[(b, h)] = ek.blocks[:lens[b]], ev.blocks[:lens[b]]
            kdq[b].append(st.oracle_dequant(synth.K_TENSOR, ek.blocks)[:lens[b]])
            vdq[b].append(st.oracle_dequant(synth.V_TENSOR, ev.blocks)[:lens[b]])
    return (P.place_streams(st, L, synth.K_TENSOR, kb), P.place_streams(st, L, synth.V_TENSOR, vb), kdq, vdq)


def _both(st, L, q, kc, vc, lens, split):
    """(records, out) of rotate + partial and of the from-query call (timed), plus the event time."""
    w = st.w
    qd = torch.from_numpy(np.ascontiguousarray(q, np.float32)).cuda()
    sl = torch.tensor(np.asarray(lens, np.int32), device="cuda")
    nbytes = tq.decode_workspace_bytes(L, split)
    q_rot = torch.empty_like(qd)
    ws0 = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    tq.rotate_sketch_query(L, st.cbk, None, qd, q_rot, None)
    tq.decode_partial(L, st.cbk, st.cbv, q_rot, None, kc, vc, sl, ws0, split_tokens=split)
    scratch = torch.full_like(qd, float("nan"))
    ws1 = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    e1.record()
    tq.decode_partial_from_query(L, st.cbk, st.cbv, qd, scratch, kc, vc, sl, ws1, split_tokens=split,
                                 events=(e0.cuda_event, e1.cuda_event))
    out = torch.full((L.batch, L.n_q_heads, w.head_dim), float("nan"), device="cuda")
    tq.decode_combine(L, st.cbv, ws1, out, split_tokens=split)
    torch.cuda.synchronize()
    return ws0.cpu().numpy(), ws1.cpu().numpy(), out.cpu().numpy(), scratch.cpu().numpy(), q_rot.cpu().numpy(), \
        e0.elapsed_time(e1)


@pytest.mark.parametrize("name", list(CASES))
def test_from_query_equals_rotate_then_partial(name):
    w = CASES[name]
    st = P.Setup(w)
    L = st.layout()
    lens = [max(1, w.context - 97 * b) for b in range(w.batch)]
    kc, vc, kdq, vdq = _cache(st, w, L, lens)
    q = synth.queries(w)
    fused = w.k_format == synth.PQ4 and w.head_dim == 128 and w.group == 4 and w.k_kind == w.v_kind
    _say(f"from query {name} lens={lens} rotated in the kernel: {fused}")
    for split in (0, 256):
        ws0, ws1, out, scratch, q_rot, ms = _both(st, L, q, kc, vc, lens, split)
        assert np.array_equal(ws0, ws1), f"{name} split {split}: records differ"
        assert ms > 0.0
        if fused:
            assert np.all(np.isnan(scratch)), "the fused kernel must leave the scratch untouched"
        else:
            assert np.array_equal(scratch, q_rot)
        P.check_read(st, q, kdq, vdq, lens, out, None, w.capacity)


def test_from_query_edge_lengths():
    """Zero, one, one tile, tile + 1 and full-capacity contexts in one batch, rotated in the kernel."""
    w = synth.scaled(synth.C4, batch=6, n_q_heads=8, n_kv_heads=2, capacity=640, context=640)
    st = P.Setup(w)
    L = st.layout()
    lens = [0, 1, 64, 65, 639, 640]
    kc, vc, kdq, vdq = _cache(st, w, L, lens)
    q = synth.queries(w)
    for split in (0, 256, 512):
        ws0, ws1, out, _, _, _ = _both(st, L, q, kc, vc, lens, split)
        assert np.array_equal(ws0, ws1)
        assert np.all(out[0] == 0.0)
        P.check_read(st, q, kdq, vdq, lens, out, None, w.capacity)


STEP_CASES = {
    # rotated and appended in the kernel; sequence 2's new token lies in a wavefront's first tile
    "c4": (synth.scaled(synth.C4, batch=5, n_q_heads=8, n_kv_heads=2, context=1300, capacity=1344),
           [1300, 1203, 70, 1025, 640], [1299, 1202, 69, -1, 1344]),
    "c5": (synth.scaled(synth.C5, batch=3, n_q_heads=16, n_kv_heads=2, context=700, capacity=704),
           [700, 603, 33], [699, 602, 32]),
    "c2": (synth.scaled(synth.C2, batch=2, n_q_heads=8, n_kv_heads=2, context=777, capacity=832),
           [777, 680], [776, 679]),
}


@pytest.mark.parametrize("name", list(STEP_CASES))
def test_decode_step_equals_flush_then_partial(name):
    """tq_decode_step writes the same cache bytes and split records as a one-slot ring
    flush followed by the partial from the query (sequences with a negative position or
    one past the capacity are skipped)."""
    w, lens, pos = STEP_CASES[name]
    st = P.Setup(w)
    L = st.layout()
    kc0, vc0, _, _ = _cache(st, w, L, [max(0, n - 1) for n in lens])
    k_new = torch.from_numpy(np.stack([synth.batch_rows(w, synth.K_TENSOR, b, 5000, 1)[0]
                                       for b in range(w.batch)])).cuda()
    v_new = torch.from_numpy(np.stack([synth.batch_rows(w, synth.V_TENSOR, b, 5000, 1)[0]
                                       for b in range(w.batch)])).cuda()
    new_pos = torch.tensor(pos, dtype=torch.int32, device="cuda")
    sl = torch.tensor(np.asarray(lens, np.int32), device="cuda")
    qd = torch.from_numpy(np.ascontiguousarray(synth.queries(w), np.float32)).cuda()
    _say(f"decode step {name} lens={lens} pos={pos}")
    for split in (0, 256):
        nbytes = tq.decode_workspace_bytes(L, split)
        kc1, vc1, kc2, vc2 = kc0.clone(), vc0.clone(), kc0.clone(), vc0.clone()
        ws1 = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
        ws2 = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
        s1, s2 = torch.empty_like(qd), torch.empty_like(qd)
        tq.decode_step(L, st.cbk, st.cbv, k_new, v_new, new_pos, qd, s1, kc1, vc1, sl, ws1, split_tokens=split)
        tq.ring_flush(L, st.cbk, st.cbv, None, 1, k_new, v_new, new_pos, 1, kc2, vc2)
        tq.decode_partial_from_query(L, st.cbk, st.cbv, qd, s2, kc2, vc2, sl, ws2, split_tokens=split)
        torch.cuda.synchronize()
        assert torch.equal(kc1, kc2) and torch.equal(vc1, vc2), f"{name} split {split}: cache bytes differ"
        assert torch.equal(ws1, ws2), f"{name} split {split}: records differ"
        # the appended rows landed where asked, and nowhere else changed
        changed = (kc1 != kc0).view(w.batch, w.n_kv_heads, w.capacity, -1).any(-1).cpu().numpy()
        for b in range(w.batch):
            want = np.zeros(w.capacity, bool)
            if 0 <= pos[b] < w.capacity:
                want[pos[b]] = True
            for h in range(w.n_kv_heads):
                assert np.all(changed[b, h] <= want), f"{name} b={b} h={h}: bytes changed elsewhere"
