"""ctypes declarations of libtq's C ABI and torch-tensor marshalling.

Names and semantics follow ``include/tq.h`` one to one; each wrapper passes
``tensor.data_ptr()`` and the current HIP stream and raises ``TQError`` on a
non-zero status.  No arithmetic of the method happens here.
"""

import ctypes
import os

import numpy as np

FMT_PQ4, FMT_PQ3, FMT_TQ3K, FMT_GQ2V = 1, 2, 3, 4
CB_QUANTILE_MEAN, CB_LLOYD_MAX = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libtq.so")

if not os.path.exists(library_path):
    raise ImportError(
        f"{library_path} is missing: build it with `python compressed_domain_attention_kv_amd/build.py`")

# torch ships its own HIP runtime with the same SONAME (libamdhip64.so.7) as
# the system one libtq links against.  Loading torch first makes the dynamic
# linker bind libtq to torch's copy, so the process holds a single HIP
# runtime and torch's streams and allocations are valid handles for libtq.
import torch  # noqa: E402,F401

lib = ctypes.CDLL(library_path)


class Codebook(ctypes.Structure):
    """Mirror of ``tq_codebook``."""

    _fields_ = [
        ("head_dim", ctypes.c_int32),
        ("bits", ctypes.c_int32),
        ("kind", ctypes.c_int32),
        ("n_levels", ctypes.c_int32),
        ("centroids", ctypes.c_float * 16),
        ("bounds", ctypes.c_float * 16),
        ("sign_bits", ctypes.c_uint32 * 8),
        ("rot_seed", ctypes.c_uint64),
        ("qjl_seed", ctypes.c_uint64),
    ]

    def centroid_array(self):
        return np.array(self.centroids[: self.n_levels], dtype=np.float32)

    def bound_array(self):
        return np.array(self.bounds[: self.n_levels - 1], dtype=np.float32)

    def sign_array(self):
        """+-1 rotation signs as float64 [head_dim]."""
        words = np.array(self.sign_bits, dtype=np.uint32)
        j = np.arange(self.head_dim)
        bit = (words[j >> 5] >> (j & 31).astype(np.uint32)) & 1
        return np.where(bit == 1, -1.0, 1.0)


class Layout(ctypes.Structure):
    """Mirror of ``tq_layout``."""

    _fields_ = [
        ("batch", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("capacity", ctypes.c_int32),
        ("k_format", ctypes.c_int32),
        ("v_format", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]

    def __init__(self, batch, n_q_heads, n_kv_heads, head_dim, capacity, k_format, v_format):
        super().__init__(batch, n_q_heads, n_kv_heads, head_dim, capacity, k_format, v_format, 0)


_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.c_size_t
_PL = ctypes.POINTER(Layout)
_PC = ctypes.POINTER(Codebook)

lib.tq_version.restype = ctypes.c_char_p
lib.tq_version.argtypes = []
lib.tq_strerror.restype = ctypes.c_char_p
lib.tq_strerror.argtypes = [_I]
lib.tq_build_codebook.restype = _I
lib.tq_build_codebook.argtypes = [_I, _I, _I, ctypes.c_uint64, ctypes.c_uint64, _PC, _P]
lib.tq_vector_bytes.restype = _SZ
lib.tq_vector_bytes.argtypes = [_I, _I]
lib.tq_cache_bytes.restype = _I
lib.tq_cache_bytes.argtypes = [_PL, ctypes.POINTER(_SZ), ctypes.POINTER(_SZ)]
lib.tq_quantize_append.restype = _I
lib.tq_quantize_append.argtypes = [_PL, _PC, _PC, _P, _P, _P, _P, _I, _P, _P, _P]
lib.tq_quantize_rotated.restype = _I
lib.tq_quantize_rotated.argtypes = [_I, _PC, _P, _P, _P, _I, _P, _P]
lib.tq_rotate_sketch_query.restype = _I
lib.tq_rotate_sketch_query.argtypes = [_PL, _PC, _P, _P, _P, _P, _P]
lib.tq_decode_splits.restype = _I
lib.tq_decode_splits.argtypes = [_PL, _I]
lib.tq_decode_workspace_bytes.restype = _SZ
lib.tq_decode_workspace_bytes.argtypes = [_PL, _I]
lib.tq_decode_attention.restype = _I
lib.tq_decode_attention.argtypes = [_PL, _PC, _PC, _P, _P, _P, _P, _P, _P, _P, _I, _P, _SZ, _P]
lib.tq_decode_partial.restype = _I
lib.tq_decode_partial.argtypes = [_PL, _PC, _PC, _P, _P, _P, _P, _P, _P, _I, _P, _SZ, _P]
lib.tq_decode_partial_timed.restype = _I
lib.tq_decode_partial_timed.argtypes = [_PL, _PC, _PC, _P, _P, _P, _P, _P, _P, _I, _P, _SZ, _P, _P, _P]
lib.tq_decode_combine.restype = _I
lib.tq_decode_partial_from_query.restype = _I
lib.tq_decode_partial_from_query.argtypes = [_PL, _PC, _PC, _P, _P, _P, _P, _P, _P, _I, _P, _SZ, _P, _P, _P]
lib.tq_decode_step.restype = _I
lib.tq_decode_step.argtypes = [_PL, _PC, _PC, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _P, _SZ, _P, _P, _P]
lib.tq_decode_partial_sparse_v.restype = _I
lib.tq_decode_partial_sparse_v.argtypes = [_PL, _PC, _PC, _P, _P, _P, _P, _P, _P, _I, ctypes.c_float, _P, _SZ, _P]
lib.tq_decode_combine.argtypes = [_PL, _PC, _I, _P, _SZ, _P, _P]
lib.tq_ring_bytes.restype = _SZ
lib.tq_ring_bytes.argtypes = [_PL, _I]
lib.tq_ring_append.restype = _I
lib.tq_ring_append.argtypes = [_PL, _I, _P, _P, _P, _P, _P, _P]
lib.tq_ring_flush.restype = _I
lib.tq_ring_flush.argtypes = [_PL, _PC, _PC, _P, _I, _P, _P, _P, _I, _P, _P, _P]
lib.tq_decode_hybrid_workspace_bytes.restype = _SZ
lib.tq_decode_hybrid_workspace_bytes.argtypes = [_PL, _I]
lib.tq_decode_attention_hybrid.restype = _I
lib.tq_decode_attention_hybrid.argtypes = [_PL, _PC, _PC, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P, _I, _P, _SZ, _P]

RING_CAP_MAX = 256


class TQError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {strerror(status)} ({status})")


def strerror(status):
    return lib.tq_strerror(status).decode()


def version():
    return lib.tq_version().decode()


def _check(status, where):
    if status != 0:
        raise TQError(status, where)


def _ptr(t):
    """Device (or host) address of a tensor, or None."""
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(stream)
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def build_codebook(head_dim, bits, kind, rot_seed, qjl_seed, want_qjl_matrix=False):
    """-> (Codebook, S as float32 numpy [d, d] or None).  Host only."""
    cb = Codebook()
    S = np.zeros((head_dim, head_dim), dtype=np.float32) if want_qjl_matrix else None
    _check(lib.tq_build_codebook(head_dim, bits, kind, rot_seed, qjl_seed, ctypes.byref(cb),
                                 None if S is None else S.ctypes.data_as(ctypes.c_void_p)),
           "tq_build_codebook")
    return cb, S


def vector_bytes(fmt, head_dim):
    return int(lib.tq_vector_bytes(fmt, head_dim))


def cache_bytes(L):
    k, v = _SZ(), _SZ()
    _check(lib.tq_cache_bytes(ctypes.byref(L), ctypes.byref(k), ctypes.byref(v)), "tq_cache_bytes")
    return k.value, v.value


def quantize_append(L, cbk, cbv, S_dev, k_new, v_new, dst_row, k_cache, v_cache, stream=None):
    """k_new/v_new: fp16 [T, Hkv, d]; dst_row: int32 [T]; caches: uint8 tensors."""
    T = int(dst_row.shape[0])
    _check(lib.tq_quantize_append(ctypes.byref(L), ctypes.byref(cbk), ctypes.byref(cbv), _ptr(S_dev),
                                  _ptr(k_new), _ptr(v_new), _ptr(dst_row), T, _ptr(k_cache), _ptr(v_cache),
                                  _stream(stream)), "tq_quantize_append")


def quantize_rotated(fmt, cb, S_dev, y, norm16, blocks, stream=None):
    """y: fp32 [n, d]; norm16: fp16 [n]; blocks: uint8 [n * vector_bytes]."""
    n = int(y.shape[0])
    _check(lib.tq_quantize_rotated(fmt, ctypes.byref(cb), _ptr(S_dev), _ptr(y), _ptr(norm16), n, _ptr(blocks),
                                   _stream(stream)), "tq_quantize_rotated")


def rotate_sketch_query(L, cbk, S_dev, q, q_rot, q_sketch=None, stream=None):
    _check(lib.tq_rotate_sketch_query(ctypes.byref(L), ctypes.byref(cbk), _ptr(S_dev), _ptr(q), _ptr(q_rot),
                                      _ptr(q_sketch), _stream(stream)), "tq_rotate_sketch_query")


def decode_splits(L, split_tokens=0):
    return int(lib.tq_decode_splits(ctypes.byref(L), split_tokens))


def decode_workspace_bytes(L, split_tokens=0):
    return int(lib.tq_decode_workspace_bytes(ctypes.byref(L), split_tokens))


def decode_attention(L, cbk, cbv, q_rot, q_sketch, k_cache, v_cache, seq_lens, out, ws, scores=None,
                     split_tokens=0, stream=None):
    _check(lib.tq_decode_attention(ctypes.byref(L), ctypes.byref(cbk), ctypes.byref(cbv), _ptr(q_rot),
                                   _ptr(q_sketch), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens), _ptr(out),
                                   _ptr(scores), split_tokens, _ptr(ws), ws.numel() * ws.element_size(),
                                   _stream(stream)), "tq_decode_attention")


def decode_partial(L, cbk, cbv, q_rot, q_sketch, k_cache, v_cache, seq_lens, ws, scores=None, split_tokens=0,
                   stream=None, events=None):
    """events: optional (start, stop) raw hipEvent_t handles, recorded at the
    kernel's own start and end (tq_decode_partial_timed)."""
    args = (ctypes.byref(L), ctypes.byref(cbk), ctypes.byref(cbv), _ptr(q_rot), _ptr(q_sketch), _ptr(k_cache),
            _ptr(v_cache), _ptr(seq_lens), _ptr(scores), split_tokens, _ptr(ws), ws.numel() * ws.element_size(),
            _stream(stream))
    if events is None:
        _check(lib.tq_decode_partial(*args), "tq_decode_partial")
    else:
        start, stop = events
        _check(lib.tq_decode_partial_timed(*args, ctypes.c_void_p(start), ctypes.c_void_p(stop)),
               "tq_decode_partial_timed")


def decode_partial_from_query(L, cbk, cbv, q, q_rot_scratch, k_cache, v_cache, seq_lens, ws, scores=None,
                              split_tokens=0, stream=None, events=None):
    """events: optional (start, stop) raw hipEvent_t handles for the partial kernel's dispatch."""
    start, stop = events if events is not None else (None, None)
    _check(lib.tq_decode_partial_from_query(ctypes.byref(L), ctypes.byref(cbk), ctypes.byref(cbv), _ptr(q),
                                            _ptr(q_rot_scratch), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens),
                                            _ptr(scores), split_tokens, _ptr(ws), ws.numel() * ws.element_size(),
                                            _stream(stream), ctypes.c_void_p(start), ctypes.c_void_p(stop)),
           "tq_decode_partial_from_query")


def decode_step(L, cbk, cbv, k_new, v_new, new_pos, q, q_rot_scratch, k_cache, v_cache, seq_lens, ws, scores=None,
                split_tokens=0, stream=None, events=None):
    """events: optional (start, stop) raw hipEvent_t handles for the partial kernel's dispatch."""
    start, stop = events if events is not None else (None, None)
    _check(lib.tq_decode_step(ctypes.byref(L), ctypes.byref(cbk), ctypes.byref(cbv), _ptr(k_new), _ptr(v_new),
                              _ptr(new_pos), _ptr(q), _ptr(q_rot_scratch), _ptr(k_cache), _ptr(v_cache),
                              _ptr(seq_lens), _ptr(scores), split_tokens, _ptr(ws), ws.numel() * ws.element_size(),
                              _stream(stream), ctypes.c_void_p(start), ctypes.c_void_p(stop)), "tq_decode_step")


def decode_partial_sparse_v(L, cbk, cbv, q_rot, q_sketch, k_cache, v_cache, seq_lens, ws, v_threshold,
                            scores=None, split_tokens=0, stream=None):
    _check(lib.tq_decode_partial_sparse_v(ctypes.byref(L), ctypes.byref(cbk), ctypes.byref(cbv), _ptr(q_rot),
                                          _ptr(q_sketch), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens),
                                          _ptr(scores), split_tokens, float(v_threshold), _ptr(ws),
                                          ws.numel() * ws.element_size(), _stream(stream)),
           "tq_decode_partial_sparse_v")


def decode_combine(L, cbv, ws, out, split_tokens=0, stream=None):
    _check(lib.tq_decode_combine(ctypes.byref(L), ctypes.byref(cbv), split_tokens, _ptr(ws),
                                 ws.numel() * ws.element_size(), _ptr(out), _stream(stream)), "tq_decode_combine")


def ring_bytes(L, ring_cap):
    return int(lib.tq_ring_bytes(ctypes.byref(L), ring_cap))


def ring_append(L, ring_cap, k_new, v_new, pos, k_ring, v_ring, stream=None):
    _check(lib.tq_ring_append(ctypes.byref(L), ring_cap, _ptr(k_new), _ptr(v_new), _ptr(pos), _ptr(k_ring),
                              _ptr(v_ring), _stream(stream)), "tq_ring_append")


def ring_flush(L, cbk, cbv, S_dev, ring_cap, k_ring, v_ring, first, count, k_cache, v_cache, stream=None):
    _check(lib.tq_ring_flush(ctypes.byref(L), ctypes.byref(cbk), ctypes.byref(cbv), _ptr(S_dev), ring_cap,
                             _ptr(k_ring), _ptr(v_ring), _ptr(first), count, _ptr(k_cache), _ptr(v_cache),
                             _stream(stream)), "tq_ring_flush")


def decode_hybrid_workspace_bytes(L, split_tokens=0):
    return int(lib.tq_decode_hybrid_workspace_bytes(ctypes.byref(L), split_tokens))


def decode_attention_hybrid(L, cbk, cbv, q_rot, q_sketch, k_cache, v_cache, comp_lens, ring_cap, k_ring, v_ring,
                            ring_lens, out, ws, split_tokens=0, stream=None):
    _check(lib.tq_decode_attention_hybrid(ctypes.byref(L), ctypes.byref(cbk), ctypes.byref(cbv), _ptr(q_rot),
                                          _ptr(q_sketch), _ptr(k_cache), _ptr(v_cache), _ptr(comp_lens), ring_cap,
                                          _ptr(k_ring), _ptr(v_ring), _ptr(ring_lens), _ptr(out), split_tokens,
                                          _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "tq_decode_attention_hybrid")
