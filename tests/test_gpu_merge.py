"""The one-launch decode (tq_decode_step with an output), which merges each
(batch row, KV head) stream's split records in the partial launch itself (the
workgroup that finishes a stream last merges it), on the GPU through the C ABI:

* its output equals tq_decode_partial_from_query followed by tq_decode_combine bit
  for bit at four query heads per KV head (the merge repeats the combine's order
  of operations), and to fp32 rounding at eight;
* its split records equal the partial's;
* the arrival counters are zero again after every call, so calls can follow each
  other on one workspace;
* with an appended token, cache bytes and output equal those of the step without
  an output followed by the combine;
* every output agrees with the oracle at the output tolerance.
The 2:4-sparse kernel merges (PQ4 at four or eight heads, PQ3 keys at four); layouts
whose kernel does not (d 256, five heads) run the combine after the partial and must give
the same results too."""

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
    "c4_g8": synth.scaled(synth.C4, batch=2, n_q_heads=16, n_kv_heads=2, context=1234, capacity=1280),
    "c5": synth.scaled(synth.C5, batch=2, n_q_heads=16, n_kv_heads=2, context=700, capacity=704),
    "c2": synth.scaled(synth.C2, batch=2, n_q_heads=8, n_kv_heads=2, context=777, capacity=832),
}


def _say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    yield


def _round_up(x, a):
    return (x + a - 1) // a * a


def ws_regions(L, split):
    """Byte offsets (acc, arrivals, total) of the workspace layout tq.h documents."""
    recs = L.batch * L.n_q_heads * tq.decode_splits(L, split)
    acc = _round_up(recs * 8, 256)
    cnt = acc + _round_up(recs * L.head_dim * 4, 256)
    return acc, cnt, cnt + _round_up(L.batch * L.n_kv_heads * 4, 256)


def _arrivals(ws, L, split):
    _, cnt, _ = ws_regions(L, split)
    return ws[cnt:cnt + 4 * L.batch * L.n_kv_heads].cpu().numpy().view(np.uint32)


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


def _merged_and_split(st, L, q, kc, vc, lens, split, ws_merged):
    """Outputs of the one-launch step on ws_merged (no token appended), and of the
    partial from the query followed by the combine; the latter's workspace."""
    w = st.w
    qd = torch.from_numpy(np.ascontiguousarray(q, np.float32)).cuda()
    sl = torch.tensor(np.asarray(lens, np.int32), device="cuda")
    rows = torch.zeros(L.batch, L.n_kv_heads, w.head_dim, dtype=torch.float16, device="cuda")
    skip = torch.full((L.batch,), -1, dtype=torch.int32, device="cuda")  # no sequence appends
    out1 = torch.full((L.batch, L.n_q_heads, w.head_dim), float("nan"), device="cuda")
    tq.decode_step(L, st.cbk, st.cbv, rows, rows, skip, qd, torch.empty_like(qd), kc, vc, sl, ws_merged, out=out1,
                   split_tokens=split)
    ws2 = torch.zeros(tq.decode_workspace_bytes(L, split), dtype=torch.uint8, device="cuda")
    out2 = torch.full_like(out1, float("nan"))
    tq.decode_partial_from_query(L, st.cbk, st.cbv, qd, torch.empty_like(qd), kc, vc, sl, ws2, split_tokens=split)
    tq.decode_combine(L, st.cbv, ws2, out2, split_tokens=split)
    torch.cuda.synchronize()
    return out1.cpu().numpy(), out2.cpu().numpy(), ws2


def _check_pair(st, L, split, out1, out2, ws1, ws2):
    w = st.w
    merges = w.k_format == synth.PQ4 and w.head_dim == 128 and (w.group == 4 or (w.group == 8 and w.k_kind == w.v_kind))
    if w.group == 8 and merges:  # the merge groups the splits differently from the combine at eight heads
        assert np.all(P.rel_err_rows(out1, out2) <= 1e-6), "merged output differs beyond fp32 rounding"
    else:
        assert np.array_equal(out1, out2), "merged output differs from partial + combine"
    acc, cnt, _ = ws_regions(L, split)
    recs = L.batch * L.n_q_heads * tq.decode_splits(L, split)
    assert torch.equal(ws1[:8 * recs], ws2[:8 * recs]), "(m, l) records differ"
    assert torch.equal(ws1[acc:acc + 4 * L.head_dim * recs], ws2[acc:acc + 4 * L.head_dim * recs]), "sums differ"
    assert np.all(_arrivals(ws1, L, split) == 0), "arrival counters not cleared"


@pytest.mark.parametrize("name", list(CASES))
def test_merged_decode_equals_partial_then_combine(name):
    w = CASES[name]
    st = P.Setup(w)
    L = st.layout()
    lens = [max(1, w.context - 97 * b) for b in range(w.batch)]
    kc, vc, kdq, vdq = _cache(st, w, L, lens)
    q = synth.queries(w)
    for split in (0, 256, 1024):
        ws = tq.decode_workspace(L, split)
        _say(f"merged decode {name} split {split}: {tq.decode_splits(L, split)} splits, lens {lens}")
        out1, out2, ws2 = _merged_and_split(st, L, q, kc, vc, lens, split, ws)
        _check_pair(st, L, split, out1, out2, ws, ws2)
        P.check_read(st, q, kdq, vdq, lens, out1, None, w.capacity)


def test_merged_decode_repeated_calls_and_edge_lengths():
    """Zero, one, one tile, tile + 1 and full-capacity contexts; three calls in a row on one
    workspace with different queries, each against the oracle."""
    w = synth.scaled(synth.C4, batch=6, n_q_heads=8, n_kv_heads=2, capacity=640, context=640)
    st = P.Setup(w)
    L = st.layout()
    lens = [0, 1, 64, 65, 639, 640]
    kc, vc, kdq, vdq = _cache(st, w, L, lens)
    for split in (0, 256, 512):
        ws = tq.decode_workspace(L, split)
        for step in range(3):
            q = synth.queries(w, step=step)
            out1, out2, ws2 = _merged_and_split(st, L, q, kc, vc, lens, split, ws)
            _check_pair(st, L, split, out1, out2, ws, ws2)
            assert np.all(out1[0] == 0.0)
            P.check_read(st, q, kdq, vdq, lens, out1, None, w.capacity)


def test_merged_decode_odd_record_count():
    """An odd number of records per workspace (one row of five query heads, one split):
    the regions stay aligned and the two-launch path serves the layout."""
    w = synth.scaled(synth.C4, batch=1, n_q_heads=5, n_kv_heads=1, capacity=256, context=200)
    st = P.Setup(w)
    L = st.layout()
    lens = [200]
    kc, vc, kdq, vdq = _cache(st, w, L, lens)
    q = synth.queries(w)
    ws = tq.decode_workspace(L, 256)
    out1, out2, ws2 = _merged_and_split(st, L, q, kc, vc, lens, 256, ws)
    assert np.array_equal(out1, out2)
    P.check_read(st, q, kdq, vdq, lens, out1, None, w.capacity)


STEP_CASES = {
    "c4": (synth.scaled(synth.C4, batch=5, n_q_heads=8, n_kv_heads=2, context=1300, capacity=1344),
           [1300, 1203, 70, 1025, 640], [1299, 1202, 69, -1, 1344]),
    "c5": (synth.scaled(synth.C5, batch=3, n_q_heads=16, n_kv_heads=2, context=700, capacity=704),
           [700, 603, 33], [699, 602, 32]),
}


@pytest.mark.parametrize("name", list(STEP_CASES))
def test_decode_step_with_output(name):
    """tq_decode_step with an output: the same cache bytes and records as the step without
    one, and the output of tq_decode_combine over those records (bit for bit)."""
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
    for split in (0, 256):
        _say(f"decode step with output {name} split {split}")
        kc1, vc1, kc2, vc2 = kc0.clone(), vc0.clone(), kc0.clone(), vc0.clone()
        ws1 = tq.decode_workspace(L, split)
        ws2 = torch.zeros_like(ws1)
        out1 = torch.full_like(qd, float("nan"))
        out2 = torch.full_like(qd, float("nan"))
        tq.decode_step(L, st.cbk, st.cbv, k_new, v_new, new_pos, qd, torch.empty_like(qd), kc1, vc1, sl, ws1,
                       out=out1, split_tokens=split)
        tq.decode_step(L, st.cbk, st.cbv, k_new, v_new, new_pos, qd, torch.empty_like(qd), kc2, vc2, sl, ws2,
                       split_tokens=split)
        tq.decode_combine(L, st.cbv, ws2, out2, split_tokens=split)
        torch.cuda.synchronize()
        assert torch.equal(kc1, kc2) and torch.equal(vc1, vc2), "cache bytes differ"
        _check_pair(st, L, split, out1.cpu().numpy(), out2.cpu().numpy(), ws1, ws2)
