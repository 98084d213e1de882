"""CPU-only checks of the C ABI: the library loads, exports every declared
symbol, and its host-side logic (codebooks, sizes, validation) is right.
No call here enqueues GPU work."""

import ctypes
import os
import re

import numpy as np
import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "tq.h")

tq = pytest.importorskip("compressed_domain_attention_kv_amd")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tq_[a-z_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = _declared_functions()
    assert len(names) >= 13
    for n in names:
        assert hasattr(tq.lib, n), n
        assert ctypes.cast(getattr(tq.lib, n), ctypes.c_void_p).value


def test_struct_sizes_match_header():
    assert ctypes.sizeof(tq.Codebook) == 192
    assert ctypes.sizeof(tq.Layout) == 32


@pytest.mark.parametrize("d", [128, 256])
@pytest.mark.parametrize("bits,kind", [(4, 0), (3, 0), (2, 0), (4, 1), (3, 1), (2, 1), (1, 0)])
def test_codebook_tables_equal_the_oracle(d, bits, kind):
    from oracle import codebook as cb
    from oracle import prng
    c, S = tq.build_codebook(d, bits, kind, 1234, 5678, want_qjl_matrix=(bits == 2))
    t = cb.tables(d, bits, kind)
    assert np.array_equal(c.centroid_array(), t.centroids)
    assert np.array_equal(c.bound_array(), t.bounds)
    assert np.array_equal(c.sign_array(), prng.rotation_signs(1234, d))
    assert c.n_levels == 1 << bits and c.head_dim == d
    if S is not None:
        S_o = prng.qjl_matrix(5678, d)
        # Box-Muller through libm on both sides: agree to 1 ulp, in practice exactly
        assert np.max(np.abs(S - S_o) / np.maximum(np.abs(S_o), 1e-30)) <= 2 ** -23
        assert np.mean(S == S_o) > 0.999


def test_codebook_argument_errors():
    c = tq.Codebook()
    f = tq.lib.tq_build_codebook
    assert f(100, 4, 0, 1, 2, ctypes.byref(c), None) == -2
    assert f(128, 5, 0, 1, 2, ctypes.byref(c), None) == -2
    assert f(128, 4, 7, 1, 2, ctypes.byref(c), None) == -2
    assert f(128, 4, 0, 1, 2, None, None) == -1


def test_vector_and_cache_bytes():
    assert tq.vector_bytes(tq.FMT_PQ4, 128) == 68
    assert tq.vector_bytes(tq.FMT_PQ4, 256) == 136
    assert tq.vector_bytes(tq.FMT_PQ3, 128) == 56
    assert tq.vector_bytes(tq.FMT_TQ3K, 128) == 52
    assert tq.vector_bytes(tq.FMT_GQ2V, 128) == 48
    assert tq.vector_bytes(tq.FMT_GQ4V, 128) == 80 and tq.vector_bytes(tq.FMT_GQ4V, 256) == 160
    assert tq.cache_bytes(tq.Layout(1, 5, 1, 128, 64, tq.FMT_TQ3K, tq.FMT_GQ4V)) == (64 * 52, 64 * 80)
    assert tq.vector_bytes(tq.FMT_PQ4, 64) == 0
    L = tq.Layout(8, 32, 8, 128, 65536, tq.FMT_PQ4, tq.FMT_PQ4)
    k, v = tq.cache_bytes(L)
    assert k == v == 8 * 8 * 65536 * 68
    assert k + v == 570_425_344


def test_layout_validation_codes():
    ok = tq.Layout(1, 4, 2, 128, 128, tq.FMT_PQ4, tq.FMT_PQ4)
    tq.cache_bytes(ok)
    for bad, code in [
        (tq.Layout(1, 3, 2, 128, 128, tq.FMT_PQ4, tq.FMT_PQ4), -1),  # Hq not a multiple of Hkv
        (tq.Layout(1, 4, 2, 128, 100, tq.FMT_PQ4, tq.FMT_PQ4), -1),  # capacity not a multiple of 64
        (tq.Layout(0, 4, 2, 128, 128, tq.FMT_PQ4, tq.FMT_PQ4), -1),
        (tq.Layout(1, 4, 2, 96, 128, tq.FMT_PQ4, tq.FMT_PQ4), -2),  # head dim
        (tq.Layout(1, 4, 2, 128, 128, tq.FMT_GQ2V, tq.FMT_PQ4), -2),  # format pair
        (tq.Layout(1, 4, 2, 128, 128, tq.FMT_TQ3K, tq.FMT_PQ4), -2),
        (tq.Layout(1, 4, 2, 128, 128, tq.FMT_PQ4, tq.FMT_GQ4V), -2),
        (tq.Layout(1, 4, 2, 128, 128, tq.FMT_GQ4V, tq.FMT_GQ4V), -2),
    ]:
        with pytest.raises(tq.TQError) as e:
            tq.cache_bytes(bad)
        assert e.value.status == code


def test_stream_length_limit_of_32_bit_stream_offsets():
    """One (b, kv-head) stream must stay addressable with 32-bit byte offsets, with room for
    the tiles a kernel requests past its end: (capacity + 4096) * vector bytes < 2^31.  The
    longest accepted stream and the next multiple of 64 tokens, per format pair and d."""
    for kf, vf, d in [(tq.FMT_PQ4, tq.FMT_PQ4, 128), (tq.FMT_PQ4, tq.FMT_PQ4, 256), (tq.FMT_PQ3, tq.FMT_PQ4, 128),
                      (tq.FMT_TQ3K, tq.FMT_GQ2V, 128), (tq.FMT_TQ3K, tq.FMT_GQ4V, 256)]:
        vb = max(tq.vector_bytes(kf, d), tq.vector_bytes(vf, d))
        cap = ((2**31 - 1) // vb - 4096) // 64 * 64
        while (cap + 4096) * vb > 2**31 - 1:
            cap -= 64
        k_bytes, v_bytes = tq.cache_bytes(tq.Layout(1, 1, 1, d, cap, kf, vf))
        assert k_bytes == cap * tq.vector_bytes(kf, d) and v_bytes == cap * tq.vector_bytes(vf, d)
        with pytest.raises(tq.TQError) as e:
            tq.cache_bytes(tq.Layout(1, 1, 1, d, cap + 64, kf, vf))
        assert e.value.status == -4
    # the old bound alone (2^31 - 1 vectors) would have accepted a 24M-token d 256 stream
    with pytest.raises(tq.TQError) as e:
        tq.cache_bytes(tq.Layout(1, 1, 1, 256, 24 * 2**20, tq.FMT_PQ4, tq.FMT_PQ4))
    assert e.value.status == -4


def test_splits_and_workspace_arithmetic():
    L = tq.Layout(8, 32, 8, 128, 65536, tq.FMT_PQ4, tq.FMT_PQ4)
    s = tq.decode_splits(L)
    assert s >= 1 and 8 * 8 * s >= 1024  # PQ4, d 128, G 4: four splits per workgroup, one per CU
    pq3 = tq.Layout(8, 32, 8, 128, 65536, tq.FMT_PQ3, tq.FMT_PQ3)
    assert 8 * 8 * tq.decode_splits(pq3) >= 1024  # PQ3 keys, d 128, G 4: the same 2:4-sparse kernel
    other = tq.Layout(8, 40, 8, 128, 65536, tq.FMT_PQ3, tq.FMT_PQ3)
    assert 8 * 8 * tq.decode_splits(other) >= 2048  # one split per workgroup elsewhere
    # (m, l) records, value sums and one arrival counter per stream, each region 256-byte aligned
    recs = 8 * 32 * s
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    assert tq.decode_workspace_bytes(L) == up(8 * recs) + up(4 * 128 * recs) + up(4 * 8 * 8)
    odd = tq.Layout(1, 5, 1, 128, 256, tq.FMT_PQ4, tq.FMT_PQ4)  # 5 records: the value sums still start aligned
    assert tq.decode_workspace_bytes(odd, 256) == 256 + up(5 * 512) + 256
    assert tq.decode_splits(L, 1024) == 64
    assert tq.decode_splits(L, 1000) == 0  # not a multiple of 256
    small = tq.Layout(1, 1, 1, 128, 512, tq.FMT_PQ4, tq.FMT_PQ4)
    assert tq.decode_splits(small, 256) == 2


def test_device_calls_reject_bad_arguments_before_any_launch():
    """Null pointers and short workspaces are refused on the host (no GPU here)."""
    L = tq.Layout(1, 4, 2, 128, 128, tq.FMT_PQ4, tq.FMT_PQ4)
    cb, _ = tq.build_codebook(128, 4, 0, 1, 2)
    r = ctypes.byref
    assert tq.lib.tq_quantize_append(r(L), r(cb), r(cb), None, None, None, None, 3, None, None, None) == -1
    assert tq.lib.tq_quantize_append(r(L), r(cb), r(cb), None, None, None, None, 0, None, None, None) == 0
    assert tq.lib.tq_quantize_append(r(L), r(cb), r(cb), None, None, None, None, -1, None, None, None) == -1
    cb3, _ = tq.build_codebook(128, 3, 0, 1, 2)  # wrong bit width for PQ4
    assert tq.lib.tq_quantize_append(r(L), r(cb3), r(cb), None, ctypes.c_void_p(16), ctypes.c_void_p(16),
                                     ctypes.c_void_p(16), 1, ctypes.c_void_p(16), ctypes.c_void_p(16), None) == -1
    assert tq.lib.tq_rotate_sketch_query(r(L), r(cb), None, None, None, None, None) == -1
    fake = ctypes.c_void_p(1 << 20)
    need = tq.decode_workspace_bytes(L)
    assert tq.lib.tq_decode_partial(r(L), r(cb), r(cb), fake, None, fake, fake, fake, None, 0, fake,
                                    need - 1, None) == -3
    assert tq.lib.tq_decode_partial(r(L), r(cb), r(cb), fake, None, fake, fake, fake, None, 100, fake,
                                    need, None) == -1
    misaligned = ctypes.c_void_p((1 << 20) + 4)
    assert tq.lib.tq_decode_partial(r(L), r(cb), r(cb), fake, None, misaligned, fake, fake, None, 0, fake,
                                    need, None) == -1
    Lg = tq.Layout(1, 6, 2, 128, 128, tq.FMT_PQ4, tq.FMT_PQ4)  # G = 3 not built
    assert tq.lib.tq_decode_partial(r(Lg), r(cb), r(cb), fake, None, fake, fake, fake, None, 0, fake,
                                    1 << 30, None) == -2
    assert tq.lib.tq_decode_combine(r(L), r(cb), 0, fake, need - 1, fake, None) == -3
    # the timed variant needs both events, and checks its arguments like the plain call
    assert tq.lib.tq_decode_partial_timed(r(L), r(cb), r(cb), fake, None, fake, fake, fake, None, 0, fake,
                                          need, None, None, fake) == -1
    assert tq.lib.tq_decode_partial_timed(r(L), r(cb), r(cb), fake, None, fake, fake, fake, None, 0, fake,
                                          need - 1, None, fake, fake) == -3
    assert tq.lib.tq_quantize_rotated(9, r(cb), None, fake, fake, 1, fake, None) == -2
    # the partial from the unrotated query: its own arguments first, then those of the partial
    fq = tq.lib.tq_decode_partial_from_query
    assert fq(r(L), r(cb), r(cb), None, fake, fake, fake, fake, None, 0, fake, need, None, None, None) == -1
    assert fq(r(L), r(cb), r(cb), misaligned, fake, fake, fake, fake, None, 0, fake, need, None, None, None) == -1
    assert fq(r(L), r(cb), r(cb), fake, None, fake, fake, fake, None, 0, fake, need, None, None, None) == -1
    assert fq(r(L), r(cb), r(cb), fake, fake, fake, fake, fake, None, 0, fake, need, None, fake, None) == -1
    assert fq(r(L), r(cb), r(cb), fake, fake, fake, fake, fake, None, 0, fake, need - 1, None, None, None) == -3
    Lt = tq.Layout(1, 4, 2, 128, 128, tq.FMT_TQ3K, tq.FMT_GQ2V)
    assert fq(r(Lt), r(cb), r(cb), fake, fake, fake, fake, fake, None, 0, fake, need, None, None, None) == -2
    # one decode step: the new rows and positions, then the arguments of the partial from the query
    ds = tq.lib.tq_decode_step
    assert ds(r(L), r(cb), r(cb), None, fake, fake, fake, fake, fake, fake, fake, None, None, 0, fake, need, None,
              None, None) == -1
    odd = ctypes.c_void_p((1 << 20) + 2)  # not 4-byte aligned
    assert ds(r(L), r(cb), r(cb), fake, fake, odd, fake, fake, fake, fake, fake, None, None, 0, fake, need, None,
              None, None) == -1
    assert ds(r(L), r(cb), r(cb), fake, fake, fake, fake, fake, fake, fake, fake, odd, None, 0, fake, need, None,
              None, None) == -1  # a misaligned output
    assert ds(r(L), r(cb), r(cb), fake, misaligned, fake, fake, fake, fake, fake, fake, None, None, 0, fake, need,
              None, None, None) == -1
    assert ds(r(L), r(cb), r(cb), fake, fake, fake, fake, fake, fake, fake, fake, fake, None, 0, fake, need - 1,
              None, None, None) == -3
    assert ds(r(Lt), r(cb), r(cb), fake, fake, fake, fake, fake, fake, fake, fake, None, None, 0, fake, need, None,
              None, None) == -2
    # the sparse-V variant checks its arguments like the plain call, and the threshold range
    sv = tq.lib.tq_decode_partial_sparse_v
    assert sv(r(L), r(cb), r(cb), fake, None, fake, fake, fake, None, 0, 0.0, fake, need - 1, None) == -3
    assert sv(r(L), r(cb), r(cb), fake, None, misaligned, fake, fake, None, 0, 0.0, fake, need, None) == -1
    for bad in (-1e-3, 1.0001, float("nan"), float("inf")):
        assert sv(r(L), r(cb), r(cb), fake, None, fake, fake, fake, None, 0, bad, fake, need, None) == -1
    # clearing a workspace's arrival counters: layout, split length, pointer and size first
    wi = tq.lib.tq_decode_workspace_init
    assert wi(r(L), 0, None, need, None) == -1
    assert wi(r(L), 0, misaligned, need, None) == -1
    assert wi(r(L), 100, fake, need, None) == -1
    assert wi(r(L), 0, fake, need - 1, None) == -3
    assert wi(r(Lg), 0, fake, need - 1, None) == -3  # the layout itself is valid; G is checked by the decodes
    assert tq.strerror(-3).startswith("workspace")


def test_ring_calls_check_their_arguments_before_any_launch():
    L = tq.Layout(2, 8, 2, 128, 256, tq.FMT_PQ4, tq.FMT_PQ4)
    cb, _ = tq.build_codebook(128, 4, 0, 1, 2)
    r = ctypes.byref
    fake = ctypes.c_void_p(1 << 20)
    assert tq.ring_bytes(L, 128) == 2 * 2 * 128 * 128 * 2
    assert tq.ring_bytes(L, 0) == 0 and tq.ring_bytes(L, tq.RING_CAP_MAX + 1) == 0
    assert tq.lib.tq_ring_append(r(L), 0, fake, fake, fake, fake, fake, None) == -1
    assert tq.lib.tq_ring_append(r(L), 64, None, fake, fake, fake, fake, None) == -1
    assert tq.lib.tq_ring_append(r(L), 64, fake, fake, fake, ctypes.c_void_p((1 << 20) + 8), fake, None) == -1
    assert tq.lib.tq_ring_flush(r(L), r(cb), r(cb), None, 64, fake, fake, fake, 65, fake, fake, None) == -1
    assert tq.lib.tq_ring_flush(r(L), r(cb), r(cb), None, 64, fake, fake, fake, -1, fake, fake, None) == -1
    assert tq.lib.tq_ring_flush(r(L), r(cb), r(cb), None, 64, None, None, None, 0, None, None, None) == 0
    need = tq.decode_hybrid_workspace_bytes(L)
    assert need == tq.decode_workspace_bytes(L)  # the ring is merged in the combine, with no record of its own
    args = [r(L), r(cb), r(cb), fake, None, fake, fake, fake]
    assert tq.lib.tq_decode_attention_hybrid(*args, 0, fake, fake, fake, fake, 0, fake, need, None) == -1
    assert tq.lib.tq_decode_attention_hybrid(*args, 64, None, fake, fake, fake, 0, fake, need, None) == -1
    assert tq.lib.tq_decode_attention_hybrid(*args, 64, fake, fake, fake, fake, 0, fake, need - 1, None) == -3


def test_ring_capacity_limit_matches_the_header():
    text = open(HEADER).read()
    m = re.search(r"#define TQ_RING_CAP_MAX (\d+)", text)
    assert m and int(m.group(1)) == tq.RING_CAP_MAX


def test_binding_refuses_bad_tensors_before_the_library():
    """The binding checks what the C ABI cannot see (device, dtype, layout, size); on the
    CPU every device argument is refused as not being a GPU tensor."""
    import torch
    L = tq.Layout(1, 4, 2, 128, 128, tq.FMT_PQ4, tq.FMT_PQ4)
    cb, _ = tq.build_codebook(128, 4, 0, 1, 2)
    cpu = torch.zeros(1 << 16, dtype=torch.uint8)
    q = torch.zeros(1, 4, 128)
    with pytest.raises(tq.TQError, match="k_cache must be a GPU tensor") as e:
        tq.decode_attention(L, cb, cb, q, None, cpu, cpu, torch.zeros(1, dtype=torch.int32), q, cpu)
    assert e.value.status == -1
    with pytest.raises(tq.TQError, match="must be a torch tensor"):
        tq.decode_combine(L, cb, bytearray(1 << 16), q)
    with pytest.raises(tq.TQError, match="ws is required"):
        tq.decode_workspace_init(L, None)
    with pytest.raises(tq.TQError, match="dst_row must be a 1-D int32 tensor"):
        tq.quantize_append(L, cb, cb, None, None, None, [0, 1], cpu, cpu)
    with pytest.raises(tq.TQError, match="invalid layout or ring_cap"):
        tq.ring_append(L, 0, None, None, None, cpu, cpu)


def test_static_decode_refuses_layouts_beyond_its_scratch():
    """tq_decode_attention_static checks the workspace its layout needs against the size
    of the library's device array before any device call (none happens here)."""
    r = ctypes.byref
    cb, _ = tq.build_codebook(128, 4, 0, 1, 2)
    fake = ctypes.c_void_p(1 << 20)
    big = tq.Layout(8, 64, 8, 128, 65536, tq.FMT_PQ4, tq.FMT_PQ4)
    assert tq.decode_workspace_bytes(big, 256) > tq.STATIC_SCRATCH_BYTES
    f = tq.lib.tq_decode_attention_static
    assert f(r(big), r(cb), r(cb), fake, None, fake, fake, fake, fake, 256, None) == -3
    assert f(r(big), r(cb), r(cb), fake, None, fake, fake, fake, fake, 100, None) == -1  # split not a multiple of 256
    bad = tq.Layout(1, 3, 2, 128, 128, tq.FMT_PQ4, tq.FMT_PQ4)
    assert f(r(bad), r(cb), r(cb), fake, None, fake, fake, fake, fake, 0, None) == -1
    text = open(HEADER).read()
    m = re.search(r"#define TQ_STATIC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == tq.STATIC_SCRATCH_BYTES
