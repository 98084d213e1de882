"""GPU parity of the HIP path against the oracle, through the C ABI.

Sizes are chosen so the oracle finishes in seconds while every kernel still
spans several 64-token tiles, several context splits and a ragged tail.
"""

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

tq = pytest.importorskip("compressed_domain_attention_kv_amd")
P = pytest.importorskip("parity")

# reduced versions of the five workloads (same distributions, formats, seeds)
REDUCED = {
    "c1": synth.C1,
    "c2": synth.scaled(synth.C2, batch=2, n_q_heads=8, n_kv_heads=2, context=777, capacity=832),
    "c3": synth.scaled(synth.C3, batch=1, n_q_heads=10, n_kv_heads=2, context=999, capacity=1024),
    "c4": synth.scaled(synth.C4, batch=3, n_q_heads=8, n_kv_heads=2, context=1300, capacity=1344),
    "c5": synth.scaled(synth.C5, batch=2, n_q_heads=16, n_kv_heads=2, context=700, capacity=704),
    "pq3k_pq4v": synth.scaled(synth.C2, v_format=synth.PQ4, v_bits=4, batch=1, n_q_heads=4, n_kv_heads=1,
                              context=500, capacity=512),
    # PQ4 with K and V on different centroid tables (the matrix-core kernel
    # that reads two tables) and PQ4 with eight query heads per KV head
    "c4_lloyd_v": synth.scaled(synth.C4, v_kind=synth.LLOYD_MAX, batch=2, n_q_heads=8, n_kv_heads=2, context=1111,
                               capacity=1152),
    "c4_g8": synth.scaled(synth.C4, batch=2, n_q_heads=16, n_kv_heads=2, context=1234, capacity=1280),
    "c4_g8_lloyd_v": synth.scaled(synth.C4, v_kind=synth.LLOYD_MAX, batch=1, n_q_heads=16, n_kv_heads=2,
                                  context=900, capacity=960),
    # TQ3K keys with 4-bit group-quantized values, at d 128 and 256
    "c3_gq4v": synth.scaled(synth.C3, v_format=synth.GQ4V, v_bits=4, batch=2, n_q_heads=10, n_kv_heads=2,
                            context=999, capacity=1024),
    "c3_gq4v_d256": synth.scaled(synth.C3, v_format=synth.GQ4V, v_bits=4, head_dim=256, batch=1, n_q_heads=8,
                                 n_kv_heads=2, context=600, capacity=640),
}


def _lens(w):
    return [max(1, w.context - 97 * b) for b in range(w.batch)]


def _say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    yield


# ---------------------------------------------------------------------------
# write side


@pytest.mark.parametrize("fmt,d", [(synth.PQ4, 128), (synth.PQ4, 256), (synth.PQ3, 128), (synth.PQ3, 256),
                                   (synth.TQ3K, 128), (synth.TQ3K, 256)])
def test_codes_bit_exact_on_identical_rotated_inputs(fmt, d):
    """Both sides quantize the same fp32 rotated coordinates: codes and norms
    must agree bit for bit (TQ3K: codes exact; residual norm and QJL signs,
    which the kernel computes in fp32, agree up to counted rounding ties)."""
    from oracle import codebook as ocb, formats as ofmt, prng as oprng
    bits, kind = {synth.PQ4: (4, 0), synth.PQ3: (3, 0), synth.TQ3K: (2, 1)}[fmt]
    _say(f"quantize_rotated fmt={fmt} d={d}")
    n = 3000
    y = synth.rotated_unit_rows(5 + d + fmt, n, d)
    # exact boundary values and zeros exercise the tie rule
    cb, S = tq.build_codebook(d, bits, kind, 77, 78, want_qjl_matrix=(fmt == synth.TQ3K))
    tabs = ocb.tables(d, bits, kind)
    y[0, : len(tabs.bounds)] = tabs.bounds
    y[1, :] = 0.0
    y[2, : len(tabs.bounds)] = np.nextafter(tabs.bounds, np.float32(1), dtype=np.float32)
    n16 = np.random.default_rng(d).uniform(0.1, 5, n).astype(np.float16)
    blocks = torch.zeros(n * tq.vector_bytes(fmt, d), dtype=torch.uint8, device="cuda")
    S_dev = torch.from_numpy(S).cuda() if S is not None else None
    tq.quantize_rotated(fmt, cb, S_dev, torch.from_numpy(y).cuda(),
                        torch.from_numpy(n16).cuda(), blocks)
    torch.cuda.synchronize()
    got = blocks.cpu().numpy().reshape(n, -1)
    if fmt in (synth.PQ4, synth.PQ3):
        ref, _ = ofmt.pack_rotated(y, n16, fmt, tabs)
        assert np.array_equal(got, ref)
        return
    S_o = oprng.qjl_matrix(78, d)
    ref, idx, gamma, proj, bits_o = ofmt.pack_rotated_tq3k(y, n16, tabs, oprng.rotation_signs(77, d), S_o)
    gn, gc, gx = P.parse_codes(fmt, got, d)
    on, oc, ox = P.parse_codes(fmt, ref, d)
    assert np.array_equal(gc, oc) and np.array_equal(gn, on)
    gd = gx["gamma"] != ox["gamma"]
    assert np.all(P._fp16_neighbor_ok(gx["gamma"][gd], ox["gamma"][gd], gamma[gd]))
    bd = gx["bits"] != ox["bits"]
    v, i = np.nonzero(bd)
    scale = np.linalg.norm(S_o.astype(np.float64), axis=1)[i] * gamma[v]
    assert np.all(np.abs(proj[v, i]) <= 1e-5 * scale)
    _say(f"  gamma ties {int(gd.sum())}, qjl ties {int(bd.sum())} of {n * d}")


@pytest.mark.parametrize("name", list(REDUCED))
def test_append_matches_oracle(name):
    w = REDUCED[name]
    st = P.Setup(w)
    L = st.layout()
    lens = _lens(w)
    _say(f"append {name} lens={lens}")
    k_rows = [synth.batch_rows(w, synth.K_TENSOR, b, 0, lens[b]) for b in range(w.batch)]
    v_rows = [synth.batch_rows(w, synth.V_TENSOR, b, 0, lens[b]) for b in range(w.batch)]
    dst = np.concatenate([b * w.capacity + np.arange(lens[b]) for b in range(w.batch)]).astype(np.int32)
    kc_bytes, vc_bytes = tq.cache_bytes(L)
    kc = torch.full((kc_bytes,), 0xEE, dtype=torch.uint8, device="cuda")
    vc = torch.full((vc_bytes,), 0xEE, dtype=torch.uint8, device="cuda")
    tq.quantize_append(L, st.cbk, st.cbv, st.S_dev, torch.from_numpy(np.concatenate(k_rows)).cuda(),
                       torch.from_numpy(np.concatenate(v_rows)).cuda(), torch.from_numpy(dst).cuda(), kc, vc)
    torch.cuda.synchronize()
    kh = kc.cpu().numpy().reshape(w.batch, w.n_kv_heads, w.capacity, st.vbk)
    vh = vc.cpu().numpy().reshape(w.batch, w.n_kv_heads, w.capacity, st.vbv)
    totals = {}
    for b in range(w.batch):
        # rows past the written ones are untouched
        assert np.all(kh[b, :, lens[b]:] == 0xEE) and np.all(vh[b, :, lens[b]:] == 0xEE)
        for h in range(w.n_kv_heads):
            for tensor, cache, rows in ((synth.K_TENSOR, kh, k_rows), (synth.V_TENSOR, vh, v_rows)):
                enc = st.oracle_encode(tensor, rows[b][:, h])
                s = P.compare_write(st, tensor, cache[b, h, :lens[b]], enc)
                for k_, v_ in s.items():
                    if isinstance(v_, (int, np.integer)) and not isinstance(v_, bool):
                        totals[k_] = totals.get(k_, 0) + int(v_)
    _say(f"  tolerated differences: {totals}")
    # flips must stay rare: at most 1 in 10^4 coordinates
    assert totals.get("code_flips", 0) <= max(2, 1e-4 * totals["vectors"] * w.head_dim)


def test_append_skips_out_of_range_rows():
    w = REDUCED["c4"]
    st = P.Setup(w)
    L = st.layout(batch=1, capacity=128)
    rows = synth.batch_rows(w, synth.K_TENSOR, 0, 0, 4)
    dst = torch.tensor([5, -1, 128, 7], dtype=torch.int32, device="cuda")  # 2 invalid rows
    kc = torch.full((tq.cache_bytes(L)[0],), 0xAB, dtype=torch.uint8, device="cuda")
    vc = torch.full((tq.cache_bytes(L)[1],), 0xAB, dtype=torch.uint8, device="cuda")
    x = torch.from_numpy(rows).cuda()
    tq.quantize_append(L, st.cbk, st.cbv, None, x, x, dst, kc, vc)
    torch.cuda.synchronize()
    kh = kc.cpu().numpy().reshape(w.n_kv_heads, 128, st.vbk)
    written = {5, 7}
    for pos in range(128):
        assert (pos in written) == (not np.all(kh[:, pos] == 0xAB))


@pytest.mark.parametrize("case", ["pq4_d128", "pq4_d256", "pq3", "tq3k_gq2v", "tq3k_gq4v_d256"])
def test_append_odd_shapes_and_scattered_rows(case):
    """Appends whose row arithmetic divides by no power of two (3 sequences, 3 KV heads, a
    capacity of 960 = 15 x 64 tokens), of 300 tokens whose destinations are scattered in-range rows
    mixed with -1 and rows past batch x capacity: every written row equals the oracle's
    encoding of its source row (up to the tolerated boundary flips), every other row keeps its
    fill."""
    base = {"pq4_d128": synth.C4, "pq4_d256": synth.C5, "pq3": synth.C2, "tq3k_gq2v": synth.C3,
            "tq3k_gq4v_d256": synth.scaled(synth.C3, v_format=synth.GQ4V, v_bits=4, head_dim=256)}[case]
    w = synth.scaled(base, batch=3, n_q_heads=12, n_kv_heads=3, context=960, capacity=960)
    st = P.Setup(w)
    L = st.layout()
    d, T, cap = w.head_dim, 300, 960
    rng = np.random.default_rng(5)
    rows = {t: (rng.standard_normal((T, 3, d)) * rng.uniform(0.05, 3.0, size=(T, 3, 1))).astype(np.float16)
            for t in (synth.K_TENSOR, synth.V_TENSOR)}
    dst = rng.permutation(3 * cap)[:T].astype(np.int32)
    bad = rng.choice(T, size=40, replace=False)
    dst[bad[:20]] = -1
    dst[bad[20:]] = 3 * cap + rng.integers(0, 5000, size=20)
    kb, vb = tq.cache_bytes(L)
    kc = torch.full((kb,), 0xEE, dtype=torch.uint8, device="cuda")
    vc = torch.full((vb,), 0xEE, dtype=torch.uint8, device="cuda")
    tq.quantize_append(L, st.cbk, st.cbv, st.S_dev, torch.from_numpy(rows[synth.K_TENSOR]).cuda(),
                       torch.from_numpy(rows[synth.V_TENSOR]).cuda(), torch.from_numpy(dst).cuda(), kc, vc)
    torch.cuda.synchronize()
    valid = np.nonzero((dst >= 0) & (dst < 3 * cap))[0]
    flips = 0
    for tensor, cache, vbytes in ((synth.K_TENSOR, kc, st.vbk), (synth.V_TENSOR, vc, st.vbv)):
        host = cache.cpu().numpy().reshape(3, 3, cap, vbytes)
        touched = np.zeros((3, 3, cap), dtype=bool)
        for h in range(3):
            got = host[dst[valid] // cap, h, dst[valid] % cap]
            stats = P.compare_write(st, tensor, got, st.oracle_encode(tensor, rows[tensor][valid, h]))
            flips += stats["code_flips"]
            touched[dst[valid] // cap, h, dst[valid] % cap] = True
        assert np.all(host[~touched] == 0xEE), "a row outside the valid destinations was written"
    _say(f"append {case}: {len(valid)} of {T} tokens written, code flips {flips}")
    assert flips <= max(2, 1e-4 * 2 * 3 * len(valid) * d)


@pytest.mark.parametrize("name", ["c4", "c5", "c2"])
def test_append_special_vectors(name):
    """Zero vectors (decode to exactly 0), norms above the fp16 range (saturate),
    tiny norms, and basis vectors n e_m, whose coordinates all land on the centroid
    nearest 1/sqrt(d) with the signs of column m of the rotation, against the
    oracle's encoding of the same rows."""
    w = REDUCED[name]
    st = P.Setup(w)
    d = w.head_dim
    L = st.layout(batch=1, capacity=64)
    rng = np.random.default_rng(77)
    rows = []
    rows.append(np.zeros(d))
    rows.append(rng.standard_normal(d) * (70000.0 / np.sqrt(d)) * 1.5)  # norm ~ 1e5 > 65504
    rows.append(rng.standard_normal(d) * 1e-3)
    for m in (0, 1, d // 2 + 3, d - 1):
        e = np.zeros(d)
        e[m] = 3.0
        rows.append(e)
    rows.append(-rows[-1])
    x = np.stack(rows).astype(np.float16)
    T = x.shape[0]
    xh = np.repeat(x[:, None, :], w.n_kv_heads, axis=1)  # [T, Hkv, d]
    dst = torch.arange(T, dtype=torch.int32, device="cuda")
    kc = torch.zeros(tq.cache_bytes(L)[0], dtype=torch.uint8, device="cuda")
    vc = torch.zeros(tq.cache_bytes(L)[1], dtype=torch.uint8, device="cuda")
    xd = torch.from_numpy(xh).cuda()
    tq.quantize_append(L, st.cbk, st.cbv, st.S_dev, xd, xd, dst, kc, vc)
    torch.cuda.synchronize()
    kh = kc.cpu().numpy().reshape(w.n_kv_heads, 64, st.vbk)
    vh = vc.cpu().numpy().reshape(w.n_kv_heads, 64, st.vbv)
    for tensor, cache in ((synth.K_TENSOR, kh), (synth.V_TENSOR, vh)):
        enc = st.oracle_encode(tensor, x)
        for h in range(w.n_kv_heads):
            P.compare_write(st, tensor, cache[h, :T], enc)
        dq = st.oracle_dequant(tensor, cache[0, :T])
        assert np.all(dq[0] == 0.0)  # the zero vector
        assert np.all(np.isfinite(dq))


# ---------------------------------------------------------------------------
# query rotation / sketch


@pytest.mark.parametrize("name", ["c3", "c4", "c5"])
def test_rotate_sketch_query_matches_oracle(name):
    from oracle import rotation as orot
    w = REDUCED[name]
    st = P.Setup(w)
    L = st.layout()
    q = synth.queries(w)
    qd = torch.from_numpy(q).cuda()
    q_rot = torch.empty_like(qd)
    q_sk = torch.empty_like(qd) if w.k_format == synth.TQ3K else None
    tq.rotate_sketch_query(L, st.cbk, st.S_dev, qd, q_rot, q_sk)
    torch.cuda.synchronize()
    ref = orot.rotate(q.reshape(-1, w.head_dim), st.sk).reshape(q.shape)
    assert np.max(P.rel_err_rows(q_rot.cpu().numpy(), ref)) < 1e-5
    if q_sk is not None:
        ref_sk = q.reshape(-1, w.head_dim).astype(np.float64) @ st.S_o.astype(np.float64).T
        assert np.max(P.rel_err_rows(q_sk.cpu().numpy().reshape(ref_sk.shape), ref_sk)) < 1e-5


# ---------------------------------------------------------------------------
# read side


def _oracle_cache(st, w, lens):
    """Oracle-encoded streams and their dequantized rows."""
    kb, vb, kdq, vdq = {}, {}, [], []
    for b in range(w.batch):
        kdq.append([])
        vdq.append([])
        for h in range(w.n_kv_heads):
            ek = st.oracle_encode(synth.K_TENSOR, synth.stream(w, synth.K_TENSOR, b, h, 0, lens[b]))
            ev = st.oracle_encode(synth.V_TENSOR, synth.stream(w, synth.V_TENSOR, b, h, 0, lens[b]))
            kb[(b, h)], vb[(b, h)] = ek.blocks, ev.blocks
            kdq[b].append(st.oracle_dequant(synth.K_TENSOR, ek.blocks))
            vdq[b].append(st.oracle_dequant(synth.V_TENSOR, ev.blocks))
    return kb, vb, kdq, vdq


def _garbage_cache(st, L, tensor, streams):
    """Oracle bytes at 0..N-1, 0xFF (NaN norms) everywhere else."""
    vb = st.vbk if tensor == synth.K_TENSOR else st.vbv
    host = np.full((L.batch, L.n_kv_heads, L.capacity, vb), 0xFF, np.uint8)
    for (b, h), blk in streams.items():
        host[b, h, :blk.shape[0]] = blk
    return torch.from_numpy(host.reshape(-1)).cuda()


@pytest.mark.parametrize("split", [0, 256])
@pytest.mark.parametrize("name", list(REDUCED))
def test_decode_matches_oracle_on_identical_bytes(name, split):
    w = REDUCED[name]
    st = P.Setup(w)
    L = st.layout()
    lens = _lens(w)
    _say(f"decode {name} split={split} lens={lens} splits={tq.decode_splits(L, split)}")
    kb, vb, kdq, vdq = _oracle_cache(st, w, lens)
    kc = _garbage_cache(st, L, synth.K_TENSOR, kb)
    vc = _garbage_cache(st, L, synth.V_TENSOR, vb)
    q = synth.queries(w)
    out, scores, _, _ = P.gpu_decode(st, L, q, kc, vc, lens, split_tokens=split)
    ws, wo = P.check_read(st, q, kdq, vdq, lens, out, scores, w.capacity)
    _say(f"  worst score err {ws:.2e}, worst output err {wo:.2e}")


def test_decode_edge_lengths():
    """Zero, one, one tile, tile + 1 and full-capacity contexts in one batch."""
    base = REDUCED["c4"]
    w = synth.scaled(base, batch=6, capacity=640, context=640)
    st = P.Setup(w)
    L = st.layout()
    lens = [0, 1, 64, 65, 639, 640]
    kb, vb, kdq, vdq = _oracle_cache(st, w, [max(n, 1) for n in lens])
    kc = _garbage_cache(st, L, synth.K_TENSOR, {k: v[:lens[k[0]]] for k, v in kb.items()})
    vc = _garbage_cache(st, L, synth.V_TENSOR, {k: v[:lens[k[0]]] for k, v in vb.items()})
    kdq = [[x[:lens[b]] for x in row] for b, row in enumerate(kdq)]
    vdq = [[x[:lens[b]] for x in row] for b, row in enumerate(vdq)]
    q = synth.queries(w)
    for split in (0, 256, 512):
        out, scores, _, _ = P.gpu_decode(st, L, q, kc, vc, lens, split_tokens=split)
        assert np.all(out[0] == 0.0)
        P.check_read(st, q, kdq, vdq, lens, out, scores, w.capacity)
        # scores are written only below the context length
        for b, n in enumerate(lens):
            assert np.all(np.isnan(scores[b, :, n:]))


@pytest.mark.parametrize("vfmt", [synth.GQ2V, synth.GQ4V])
@pytest.mark.parametrize("G", [1, 2, 4, 5, 8])
def test_tq3k_keys_every_group_size_and_ragged_lengths(G, vfmt):
    """TQ3K keys with group-quantized values at d 128 for every group size the matrix-core
    kernel is built for: contexts of 0, 1, a token block, a tile, one past it, one split,
    one past a split and the full capacity, with the automatic and a 256-token split."""
    w = synth.scaled(synth.C3, v_format=vfmt, v_bits=2 if vfmt == synth.GQ2V else 4, batch=8, n_q_heads=2 * G,
                     n_kv_heads=2, context=1024, capacity=1024)
    st = P.Setup(w)
    L = st.layout()
    lens = [0, 1, 16, 33, 255, 257, 700, 1024]
    kb, vb, kdq, vdq = _oracle_cache(st, w, lens)
    kc = _garbage_cache(st, L, synth.K_TENSOR, kb)
    vc = _garbage_cache(st, L, synth.V_TENSOR, vb)
    q = synth.queries(w)
    for split in (0, 256):
        out, scores, _, _ = P.gpu_decode(st, L, q, kc, vc, lens, split_tokens=split)
        es, eo = P.check_read(st, q, kdq, vdq, lens, out, scores, w.capacity)
        assert np.all(out[0] == 0.0)
        for b, n in enumerate(lens):  # scores are written only below the context length
            assert np.all(np.isnan(scores[b, :, n:]))
        _say(f"tq3k G={G} v={vfmt} split={split}: score err {es:.2e}, output err {eo:.2e}")


@pytest.mark.parametrize("pair", ["pq3_pq3", "pq3_pq4", "pq3_pq3_two_tables"])
def test_pq3_keys_ragged_lengths(pair):
    """turbo3 keys on the 2:4-sparse kernel (PQ3 values of the same table, PQ4 values) and on
    the generic kernel (PQ3 values of another table): contexts of 0, 1, a token block, a tile,
    one past it, one split, one past a split and the full capacity over garbage-filled caches,
    with the automatic and a 256-token split."""
    vf, vb, vk = {"pq3_pq3": (synth.PQ3, 3, synth.QUANTILE_MEAN), "pq3_pq4": (synth.PQ4, 4, synth.QUANTILE_MEAN),
                  "pq3_pq3_two_tables": (synth.PQ3, 3, synth.LLOYD_MAX)}[pair]
    w = synth.scaled(synth.C2, v_format=vf, v_bits=vb, v_kind=vk, batch=8, n_q_heads=8, n_kv_heads=2, context=1024,
                     capacity=1024)
    st = P.Setup(w)
    L = st.layout()
    lens = [0, 1, 16, 33, 255, 257, 700, 1024]
    kb, vbytes, kdq, vdq = _oracle_cache(st, w, lens)
    kc = _garbage_cache(st, L, synth.K_TENSOR, kb)
    vc = _garbage_cache(st, L, synth.V_TENSOR, vbytes)
    q = synth.queries(w)
    for split in (0, 256):
        out, scores, _, _ = P.gpu_decode(st, L, q, kc, vc, lens, split_tokens=split)
        es, eo = P.check_read(st, q, kdq, vdq, lens, out, scores, w.capacity)
        assert np.all(out[0] == 0.0)
        for b, n in enumerate(lens):  # scores are written only below the context length
            assert np.all(np.isnan(scores[b, :, n:]))
        _say(f"pq3 keys {pair} split={split}: score err {es:.2e}, output err {eo:.2e}")


@pytest.mark.parametrize("case", ["g4", "g8", "g4_two_tables"])
def test_pq4_sparse_ragged_lengths(case):
    """PQ4 on the 2:4-sparse kernel: four and eight query heads per KV head (values staged in
    LDS a tile ahead; at eight heads in stages of exactly a tile, weights one token block at a
    time) and four heads with the values' own centroid table (values through registers):
    contexts of 0, 1, a token block, a tile, one past it, one split, one past a split and the
    full capacity over garbage-filled caches, with the automatic and a 256-token split."""
    G, vk = {"g4": (4, synth.QUANTILE_MEAN), "g8": (8, synth.QUANTILE_MEAN),
             "g4_two_tables": (4, synth.LLOYD_MAX)}[case]
    w = synth.scaled(synth.C4, v_kind=vk, batch=8, n_q_heads=2 * G, n_kv_heads=2, context=1024, capacity=1024)
    st = P.Setup(w)
    L = st.layout()
    lens = [0, 1, 16, 33, 255, 257, 700, 1024]
    kb, vbytes, kdq, vdq = _oracle_cache(st, w, lens)
    kc = _garbage_cache(st, L, synth.K_TENSOR, kb)
    vc = _garbage_cache(st, L, synth.V_TENSOR, vbytes)
    q = synth.queries(w)
    for split in (0, 256):
        out, scores, _, _ = P.gpu_decode(st, L, q, kc, vc, lens, split_tokens=split)
        es, eo = P.check_read(st, q, kdq, vdq, lens, out, scores, w.capacity)
        assert np.all(out[0] == 0.0)
        for b, n in enumerate(lens):  # scores are written only below the context length
            assert np.all(np.isnan(scores[b, :, n:]))
        _say(f"pq4 sparse {case} split={split}: score err {es:.2e}, output err {eo:.2e}")


@pytest.mark.parametrize("case", ["g4", "g8", "g8_two_tables"])
def test_pq4_d256_ragged_lengths(case):
    """PQ4 at d 256: the byte-pair kernel (one table for keys and values) at four and eight
    query heads per KV head, and the dense kernel at eight with the values' own centroids:
    contexts of 0, 1, a token block, a tile, one past it, one past a split and the full
    capacity over garbage-filled caches, with the automatic split and splits of 256 and 512
    tokens (one or two tiles per wavefront, wavefronts without tokens, a last tile partly past
    the end)."""
    G, vk = {"g4": (4, synth.QUANTILE_MEAN), "g8": (8, synth.QUANTILE_MEAN),
             "g8_two_tables": (8, synth.LLOYD_MAX)}[case]
    w = synth.scaled(synth.C5, v_kind=vk, batch=8, n_q_heads=2 * G, n_kv_heads=2, context=1024, capacity=1024)
    st = P.Setup(w)
    L = st.layout()
    lens = [0, 1, 16, 32, 33, 300, 700, 1024]
    kb, vbytes, kdq, vdq = _oracle_cache(st, w, lens)
    kc = _garbage_cache(st, L, synth.K_TENSOR, kb)
    vc = _garbage_cache(st, L, synth.V_TENSOR, vbytes)
    q = synth.queries(w)
    for split in (0, 256, 512):
        out, scores, _, _ = P.gpu_decode(st, L, q, kc, vc, lens, split_tokens=split)
        es, eo = P.check_read(st, q, kdq, vdq, lens, out, scores, w.capacity)
        assert np.all(out[0] == 0.0)
        for b, n in enumerate(lens):  # scores are written only below the context length
            assert np.all(np.isnan(scores[b, :, n:]))
        _say(f"pq4 d256 {case} split={split}: score err {es:.2e}, output err {eo:.2e}")


def test_timed_partial_matches_untimed():
    """tq_decode_partial_timed writes the same records as tq_decode_partial and
    its events span a positive kernel time."""
    w = REDUCED["c4"]
    st = P.Setup(w)
    L = st.layout()
    lens = _lens(w)
    kb, vb, _, _ = _oracle_cache(st, w, lens)
    kc = _garbage_cache(st, L, synth.K_TENSOR, kb)
    vc = _garbage_cache(st, L, synth.V_TENSOR, vb)
    q_rot = torch.empty((L.batch, L.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    tq.rotate_sketch_query(L, st.cbk, None, torch.from_numpy(synth.queries(w)).cuda(), q_rot, None)
    sl = torch.tensor(np.asarray(lens, np.int32), device="cuda")
    wss = [torch.zeros(tq.decode_workspace_bytes(L), dtype=torch.uint8, device="cuda") for _ in range(2)]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    e1.record()
    tq.decode_partial(L, st.cbk, st.cbv, q_rot, None, kc, vc, sl, wss[0])
    tq.decode_partial(L, st.cbk, st.cbv, q_rot, None, kc, vc, sl, wss[1], events=(e0.cuda_event, e1.cuda_event))
    torch.cuda.synchronize()
    assert torch.equal(wss[0], wss[1])
    assert e0.elapsed_time(e1) > 0.0


def test_single_key_returns_its_value_on_gpu():
    w = synth.scaled(REDUCED["c4"], batch=1, capacity=64, context=1)
    st = P.Setup(w)
    L = st.layout()
    kb, vb, kdq, vdq = _oracle_cache(st, w, [1])
    kc = _garbage_cache(st, L, synth.K_TENSOR, kb)
    vc = _garbage_cache(st, L, synth.V_TENSOR, vb)
    q = synth.queries(w)
    out, _, _, _ = P.gpu_decode(st, L, q, kc, vc, [1])
    for g in range(w.n_q_heads):
        h = g // w.group
        assert P.rel_err_rows(out[0, g], vdq[0][h][0]) < 1e-5


def test_c1_end_to_end():
    """Workload c1 at its full size: append through the HIP encoder, decode,
    compare with the oracle.  The GPU's bytes are first checked against the
    oracle's encoding of the same rows (codes may differ only on a decision
    boundary, counted); the oracle then decodes the GPU's own bytes, so the
    read side holds the output tolerance whatever ties the encoder met."""
    w = synth.C1
    st = P.Setup(w)
    L = st.layout()
    k = synth.batch_rows(w, synth.K_TENSOR, 0, 0, 512)
    v = synth.batch_rows(w, synth.V_TENSOR, 0, 0, 512)
    kc = torch.zeros(tq.cache_bytes(L)[0], dtype=torch.uint8, device="cuda")
    vc = torch.zeros(tq.cache_bytes(L)[1], dtype=torch.uint8, device="cuda")
    tq.quantize_append(L, st.cbk, st.cbv, None, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                       torch.arange(512, dtype=torch.int32, device="cuda"), kc, vc)
    q = synth.queries(w)
    out, scores, _, _ = P.gpu_decode(st, L, q, kc, vc, [512])
    ek = st.oracle_encode(synth.K_TENSOR, k[:, 0])
    ev = st.oracle_encode(synth.V_TENSOR, v[:, 0])
    gk, gv = kc.cpu().numpy().reshape(512, 68), vc.cpu().numpy().reshape(512, 68)
    sk = P.compare_write(st, synth.K_TENSOR, gk, ek)
    sv = P.compare_write(st, synth.V_TENSOR, gv, ev)
    _say(f"c1 write: {sk} {sv}")
    kdq = [[st.oracle_dequant(synth.K_TENSOR, gk)]]  # validated above: the oracle decodes the GPU's bytes
    vdq = [[st.oracle_dequant(synth.V_TENSOR, gv)]]
    ws, wo = P.check_read(st, q, kdq, vdq, [512], out, scores, 512)
    _say(f"c1 read: worst score err {ws:.2e}, output err {wo:.2e}; code flips K {sk['code_flips']} "
         f"V {sv['code_flips']}")


@pytest.mark.parametrize("d", [128, 256])
def test_small_and_bulk_pq4_appends_write_the_same_bytes(d):
    """The PQ4 write kernel takes one pass per workgroup for small launches (an append of a
    token per stream) and four for bulk writes; the bytes are the same either way."""
    base = REDUCED["c4"] if d == 128 else REDUCED["c5"]
    w = synth.scaled(base, batch=1, n_q_heads=8, n_kv_heads=8, capacity=1152, context=1100)
    st = P.Setup(w)
    L = st.layout()
    T = w.context
    assert 2 * T * w.n_kv_heads > 8192  # one bulk launch
    k_rows = torch.from_numpy(synth.batch_rows(w, synth.K_TENSOR, 0, 0, T)).cuda()
    v_rows = torch.from_numpy(synth.batch_rows(w, synth.V_TENSOR, 0, 0, T)).cuda()
    dst = torch.arange(T, dtype=torch.int32, device="cuda")
    kcb, vcb = tq.cache_bytes(L)
    caches = []
    for chunk in (T, 97):  # 97 tokens x 8 heads x 2 tensors: small launches
        kc = torch.full((kcb,), 0xEE, dtype=torch.uint8, device="cuda")
        vc = torch.full((vcb,), 0xEE, dtype=torch.uint8, device="cuda")
        for t0 in range(0, T, chunk):
            t1 = min(T, t0 + chunk)
            tq.quantize_append(L, st.cbk, st.cbv, None, k_rows[t0:t1].contiguous(), v_rows[t0:t1].contiguous(),
                               dst[t0:t1].contiguous(), kc, vc)
        torch.cuda.synchronize()
        caches.append((kc.cpu().numpy(), vc.cpu().numpy()))
    assert np.array_equal(caches[0][0], caches[1][0]) and np.array_equal(caches[0][1], caches[1][1])
