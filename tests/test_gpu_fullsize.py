"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark uses (automatic split count, full batch).

Each (sequence, KV head) stream is independent, so the oracle checks sampled
streams: it encodes their rows itself (write-side check of the GPU bytes),
its bytes then replace the GPU's for those streams, and the outputs of every
query head reading them are compared with the oracle's attention.  Outputs of
the other streams are checked for finiteness and the convexity bound
|o_j| <= max_t |v_hat_tj| that any softmax average obeys.
"""

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

tq = pytest.importorskip("compressed_domain_attention_kv_amd")
P = pytest.importorskip("parity")


def _say(msg):
    print(msg, flush=True)


def _gen_rows(w, tensor, count, batch=None):
    from concurrent.futures import ThreadPoolExecutor
    B = w.batch if batch is None else batch
    with ThreadPoolExecutor(16) as ex:
        return list(ex.map(lambda b: synth.batch_rows(w, tensor, b, 0, count), range(B)))


def _cache_view(t, L, vb):
    return t.view(L.batch, L.n_kv_heads, L.capacity, vb)


def _run_full(w, sample, append_step=None):
    """Prefill (and optionally one appended token) through the HIP encoder,
    check sampled streams against the oracle on both sides."""
    st = P.Setup(w)
    L = st.layout()
    d = w.head_dim
    kb_, vb_ = tq.cache_bytes(L)
    kc = torch.empty(kb_, dtype=torch.uint8, device="cuda")
    vc = torch.empty(vb_, dtype=torch.uint8, device="cuda")
    _say(f"{w.name}: generating and encoding {w.batch}x{w.n_kv_heads}x{w.prefill} rows")
    krows = _gen_rows(w, synth.K_TENSOR, w.prefill)
    vrows = _gen_rows(w, synth.V_TENSOR, w.prefill)
    for b in range(w.batch):
        dst = torch.arange(b * w.capacity, b * w.capacity + w.prefill, dtype=torch.int32, device="cuda")
        tq.quantize_append(L, st.cbk, st.cbv, st.S_dev, torch.from_numpy(krows[b]).cuda(),
                           torch.from_numpy(vrows[b]).cuda(), dst, kc, vc)
    lens = [w.prefill] * w.batch
    appended = {}
    if append_step is not None:
        kn = np.stack([np.stack([synth.appended(w, synth.K_TENSOR, b, h, append_step) for h in range(w.n_kv_heads)])
                       for b in range(w.batch)])
        vn = np.stack([np.stack([synth.appended(w, synth.V_TENSOR, b, h, append_step) for h in range(w.n_kv_heads)])
                       for b in range(w.batch)])
        dst = torch.tensor([b * w.capacity + w.prefill for b in range(w.batch)], dtype=torch.int32, device="cuda")
        tq.quantize_append(L, st.cbk, st.cbv, st.S_dev, torch.from_numpy(kn).cuda(), torch.from_numpy(vn).cuda(),
                           dst, kc, vc)
        lens = [w.prefill + 1] * w.batch
        appended = {(b, h): (kn[b, h], vn[b, h]) for b in range(w.batch) for h in range(w.n_kv_heads)}
    torch.cuda.synchronize()
    kview, vview = _cache_view(kc, L, st.vbk), _cache_view(vc, L, st.vbv)
    kdq, vdq = {}, {}
    for (b, h) in sample:
        n = lens[b]
        xk, xv = krows[b][:, h], vrows[b][:, h]
        if (b, h) in appended:
            xk = np.concatenate([xk, appended[(b, h)][0][None]])
            xv = np.concatenate([xv, appended[(b, h)][1][None]])
        ek, ev = st.oracle_encode(synth.K_TENSOR, xk), st.oracle_encode(synth.V_TENSOR, xv)
        sk = P.compare_write(st, synth.K_TENSOR, kview[b, h, :n].cpu().numpy(), ek)
        sv = P.compare_write(st, synth.V_TENSOR, vview[b, h, :n].cpu().numpy(), ev)
        _say(f"  stream {(b, h)} write side: K {sk} V {sv}")
        # the oracle's bytes replace the GPU's for this stream
        kview[b, h, :n].copy_(torch.from_numpy(ek.blocks))
        vview[b, h, :n].copy_(torch.from_numpy(ev.blocks))
        kdq[(b, h)] = st.oracle_dequant(synth.K_TENSOR, ek.blocks)
        vdq[(b, h)] = st.oracle_dequant(synth.V_TENSOR, ev.blocks)
    q = synth.queries(w, step=0 if append_step is None else append_step)
    out, scores, _, _ = P.gpu_decode(st, L, q, kc, vc, lens, split_tokens=0, want_scores=True)
    assert np.all(np.isfinite(out))
    worst_s = worst_o = 0.0
    for (b, h) in sample:
        for g in range(h * w.group, (h + 1) * w.group):
            ref, logits = P.oatt.softmax_attention(q[b, g], kdq[(b, h)], vdq[(b, h)])
            es = P.rel_err_rows(scores[b, g, :lens[b]], logits)
            eo = P.rel_err_rows(out[b, g], ref)
            worst_s, worst_o = max(worst_s, float(es)), max(worst_o, float(eo))
            assert es <= P.SCORE_TOL and eo <= P.OUT_TOL, (b, g, es, eo)
    _say(f"  sampled streams: worst score err {worst_s:.2e}, worst output err {worst_o:.2e}")
    return st, L, out, kc, vc, lens


def _check_unsampled_bounds(st, w, out, vc, L, lens, probe):
    """|o_j| <= max_t |v_hat_tj| for a few unsampled streams (values decoded by the oracle
    from the bytes the oracle itself writes for those rows)."""
    for (b, h) in probe:
        vrows = synth.stream(w, synth.V_TENSOR, b, h, 0, w.prefill)
        ev = st.oracle_encode(synth.V_TENSOR, vrows)
        vmax = np.abs(st.oracle_dequant(synth.V_TENSOR, ev.blocks)).max(axis=0)
        for g in range(h * w.group, (h + 1) * w.group):
            assert np.all(np.abs(out[b, g]) <= vmax * (1 + 1e-2) + 1e-3), (b, g)


def test_c4_full_size_with_append():
    w = synth.C4
    st, L, out, kc, vc, lens = _run_full(w, sample=[(0, 0), (7, 5), (3, 2)], append_step=0)
    assert tq.decode_splits(L) >= 16  # split-K: one single-round grid of 16 splits per stream


def test_c2_full_size():
    w = synth.C2
    st, L, out, kc, vc, lens = _run_full(w, sample=[(0, h) for h in range(w.n_kv_heads)])


def test_c3_full_size():
    w = synth.C3
    st, L, out, kc, vc, lens = _run_full(w, sample=[(0, 0), (0, 3), (0, 7)])
    _check_unsampled_bounds(st, w, out, vc, L, lens, [(0, 5)])


def test_c5_bulk_prefill_then_decode():
    """131,072 tokens x 4 KV heads compressed in one call, then decoded as
    [32][2][8192] over the same bytes."""
    w = synth.C5
    st = P.Setup(w)
    d = w.head_dim
    T, Hp = w.extra["prefill_tokens"], w.extra["prefill_kv_heads"]
    Lp = tq.Layout(1, Hp, Hp, d, T, w.k_format, w.v_format)
    kb_, vb_ = tq.cache_bytes(Lp)
    kc = torch.empty(kb_, dtype=torch.uint8, device="cuda")
    vc = torch.empty(vb_, dtype=torch.uint8, device="cuda")
    wp = synth.scaled(w, batch=1, n_q_heads=Hp, n_kv_heads=Hp, capacity=T, context=T, prefill=T)
    _say("c5: generating 131072 x 4 x 256 K and V rows")
    k = synth.batch_rows(wp, synth.K_TENSOR, 0, 0, T)
    v = synth.batch_rows(wp, synth.V_TENSOR, 0, 0, T)
    tq.quantize_append(Lp, st.cbk, st.cbv, None, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                       torch.arange(T, dtype=torch.int32, device="cuda"), kc, vc)
    torch.cuda.synchronize()
    # decode view: stream (b, h) of [32][2][8192] is prefill head p = (2b + h) // 16, tokens 8192 * ((2b + h) % 16) + ...
    L = st.layout()
    assert tq.cache_bytes(L) == (kb_, vb_)
    kview, vview = kc.view(w.batch, w.n_kv_heads, w.capacity, st.vbk), vc.view(w.batch, w.n_kv_heads, w.capacity, st.vbv)
    sample = [(0, 0), (13, 1), (31, 1)]
    kdq, vdq = {}, {}
    for (b, h) in sample:
        flat = b * w.n_kv_heads + h
        p, part = flat // (T // w.capacity), flat % (T // w.capacity)
        rows_k = k[part * w.capacity:(part + 1) * w.capacity, p]
        rows_v = v[part * w.capacity:(part + 1) * w.capacity, p]
        ek, ev = st.oracle_encode(synth.K_TENSOR, rows_k), st.oracle_encode(synth.V_TENSOR, rows_v)
        sk = P.compare_write(st, synth.K_TENSOR, kview[b, h].cpu().numpy(), ek)
        sv = P.compare_write(st, synth.V_TENSOR, vview[b, h].cpu().numpy(), ev)
        _say(f"  stream {(b, h)} write side: K {sk} V {sv}")
        kview[b, h].copy_(torch.from_numpy(ek.blocks))
        vview[b, h].copy_(torch.from_numpy(ev.blocks))
        kdq[(b, h)] = st.oracle_dequant(synth.K_TENSOR, ek.blocks)
        vdq[(b, h)] = st.oracle_dequant(synth.V_TENSOR, ev.blocks)
    q = synth.queries(w)
    lens = [w.context] * w.batch
    out, scores, _, _ = P.gpu_decode(st, L, q, kc, vc, lens)
    assert np.all(np.isfinite(out))
    for (b, h) in sample:
        for g in range(h * w.group, (h + 1) * w.group):
            ref, logits = P.oatt.softmax_attention(q[b, g], kdq[(b, h)], vdq[(b, h)])
            assert P.rel_err_rows(scores[b, g], logits) <= P.SCORE_TOL
            assert P.rel_err_rows(out[b, g], ref) <= P.OUT_TOL


def _last_row(e):
    """The oracle encoding of the last row alone."""
    import dataclasses
    return dataclasses.replace(e, blocks=e.blocks[-1:], norm=e.norm[-1:], y=e.y[-1:], idx=e.idx[-1:])


def test_c4_full_size_fused_step():
    """The benchmark's launch: tq_decode_step at c4's full size (the kernel appends token
    65,535 of every stream and rotates the query in its prologue), then the combine.  The
    prefix of the sampled streams holds the oracle's bytes; the appended rows the kernel
    wrote are checked against the oracle's encoding, and the outputs against the oracle's
    attention over its own encoding of every row."""
    w = synth.C4
    st = P.Setup(w)
    L = st.layout()
    d, n0 = w.head_dim, w.prefill
    kb_, vb_ = tq.cache_bytes(L)
    kc = torch.empty(kb_, dtype=torch.uint8, device="cuda")
    vc = torch.empty(vb_, dtype=torch.uint8, device="cuda")
    _say(f"{w.name} fused step: generating and encoding {w.batch}x{w.n_kv_heads}x{n0} rows")
    krows = _gen_rows(w, synth.K_TENSOR, n0)
    vrows = _gen_rows(w, synth.V_TENSOR, n0)
    for b in range(w.batch):
        dst = torch.arange(b * w.capacity, b * w.capacity + n0, dtype=torch.int32, device="cuda")
        tq.quantize_append(L, st.cbk, st.cbv, None, torch.from_numpy(krows[b]).cuda(),
                           torch.from_numpy(vrows[b]).cuda(), dst, kc, vc)
    step = 1
    kn = np.stack([np.stack([synth.appended(w, synth.K_TENSOR, b, h, step) for h in range(w.n_kv_heads)])
                   for b in range(w.batch)])
    vn = np.stack([np.stack([synth.appended(w, synth.V_TENSOR, b, h, step) for h in range(w.n_kv_heads)])
                   for b in range(w.batch)])
    torch.cuda.synchronize()
    kview, vview = _cache_view(kc, L, st.vbk), _cache_view(vc, L, st.vbv)
    sample = [(0, 0), (5, 7), (2, 3)]
    enc = {}
    for (b, h) in sample:
        ek = st.oracle_encode(synth.K_TENSOR, np.concatenate([krows[b][:, h], kn[b, h][None]]))
        ev = st.oracle_encode(synth.V_TENSOR, np.concatenate([vrows[b][:, h], vn[b, h][None]]))
        kview[b, h, :n0].copy_(torch.from_numpy(ek.blocks[:n0]))
        vview[b, h, :n0].copy_(torch.from_numpy(ev.blocks[:n0]))
        enc[(b, h)] = (ek, ev)
    q = synth.queries(w, step=step)
    qd = torch.from_numpy(q).cuda()
    out = torch.full((w.batch, w.n_q_heads, d), float("nan"), device="cuda")
    ws = torch.empty(tq.decode_workspace_bytes(L), dtype=torch.uint8, device="cuda")
    tq.decode_step(L, st.cbk, st.cbv, torch.from_numpy(kn).cuda(), torch.from_numpy(vn).cuda(),
                   torch.full((w.batch,), n0, dtype=torch.int32, device="cuda"), qd, torch.empty_like(qd), kc, vc,
                   torch.full((w.batch,), n0 + 1, dtype=torch.int32, device="cuda"), ws)
    tq.decode_combine(L, st.cbv, ws, out)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    assert np.all(np.isfinite(out))
    worst = 0.0
    for (b, h), (ek, ev) in enc.items():
        sk = P.compare_write(st, synth.K_TENSOR, kview[b, h, n0:n0 + 1].cpu().numpy(), _last_row(ek))
        sv = P.compare_write(st, synth.V_TENSOR, vview[b, h, n0:n0 + 1].cpu().numpy(), _last_row(ev))
        _say(f"  stream {(b, h)} appended row: K {sk} V {sv}")
        kd, vd = st.oracle_dequant(synth.K_TENSOR, ek.blocks), st.oracle_dequant(synth.V_TENSOR, ev.blocks)
        for g in range(h * w.group, (h + 1) * w.group):
            ref, _ = P.oatt.softmax_attention(q[b, g], kd, vd)
            e = float(P.rel_err_rows(out[b, g], ref))
            worst = max(worst, e)
            assert e <= P.OUT_TOL, (b, g, e)
    _say(f"  sampled streams: worst output err {worst:.2e}")
