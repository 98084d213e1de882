"""tq_decode_attention_static, the decode that allocates nothing (its split records
live in the library's own device array), on the GPU through the C ABI: two calls
in a row, the second with a smaller input, each equal bit for bit to
tq_decode_attention on a caller workspace (same kernels, same arithmetic) and
within the output tolerance of the oracle."""

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

tq = pytest.importorskip("compressed_domain_attention_kv_amd")
P = pytest.importorskip("parity")


def _say(msg):
    print(msg, flush=True)


def _run(w, lens, split):
    st = P.Setup(w)
    L = st.layout()
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
    kc, vc = P.place_streams(st, L, synth.K_TENSOR, kb), P.place_streams(st, L, synth.V_TENSOR, vb)
    q = synth.queries(w)
    qd = torch.from_numpy(np.ascontiguousarray(q, np.float32)).cuda()
    q_rot = torch.empty_like(qd)
    q_sk = torch.empty_like(qd) if w.k_format == synth.TQ3K else None
    tq.rotate_sketch_query(L, st.cbk, st.S_dev, qd, q_rot, q_sk)
    sl = torch.tensor(np.asarray(lens, np.int32), device="cuda")
    assert tq.decode_workspace_bytes(L, split) <= tq.STATIC_SCRATCH_BYTES
    out_ws = torch.full_like(qd, float("nan"))
    ws = torch.empty(tq.decode_workspace_bytes(L, split), dtype=torch.uint8, device="cuda")
    tq.decode_attention(L, st.cbk, st.cbv, q_rot, q_sk, kc, vc, sl, out_ws, ws, split_tokens=split)
    out_st = torch.full_like(qd, float("nan"))
    tq.decode_attention_static(L, st.cbk, st.cbv, q_rot, q_sk, kc, vc, sl, out_st, split_tokens=split)
    torch.cuda.synchronize()
    a, b_ = out_ws.cpu().numpy(), out_st.cpu().numpy()
    assert np.array_equal(a, b_), "static-scratch output differs from the workspace decode"
    _, worst = P.check_read(st, q, kdq, vdq, lens, b_, None, w.capacity)
    _say(f"  {w.name} batch {w.batch} lens {lens}: bit-equal to the workspace decode, oracle err {worst:.2e}")


def test_static_scratch_decode_two_calls_second_smaller():
    # first call: c4 layout (the 2:4-sparse PQ4 kernel), 4 x 8 streams
    big = synth.scaled(synth.C4, batch=4, n_q_heads=32, n_kv_heads=8, context=3000, capacity=3008)
    _run(big, [3000, 2900, 1500, 7], 0)
    # second call, smaller: fewer sequences, shorter contexts, other split length (the array
    # still holds the first call's records, which the second must not read)
    small = synth.scaled(synth.C4, batch=2, n_q_heads=8, n_kv_heads=2, context=500, capacity=512)
    _run(small, [500, 0], 256)


def test_static_scratch_decode_other_formats():
    # the generic kernel (TQ3K keys with GQ2V values) and the d 256 kernel share the array too
    _run(synth.scaled(synth.C3, batch=1, n_q_heads=10, n_kv_heads=2, context=900, capacity=960), [900], 0)
    _run(synth.scaled(synth.C5, batch=2, n_q_heads=16, n_kv_heads=2, context=700, capacity=704), [700, 333], 0)
