"""ctypes declarations of libtq's C ABI and torch-tensor marshalling.

Names and semantics follow ``include/tq.h`` one to one; each wrapper passes
``tensor.data_ptr()`` and the current HIP stream and raises ``TQError`` on a
non-zero status.  No arithmetic of the method happens here.

The C ABI takes raw device pointers and cannot see buffer sizes, so every
wrapper checks its tensors first: a GPU tensor on the current device, the
expected dtype, contiguous, aligned as the header requires, and at least as
many bytes as the layout needs (caches from ``cache_bytes``, queries and
outputs B*Hq*d fp32, per-sequence arrays B int32, and so on).  A bad argument
raises ``TQError`` with status TQ_ERR_INVALID before the library is called.
"""

import ctypes
import os

import numpy as np

FMT_PQ4, FMT_PQ3, FMT_TQ3K, FMT_GQ2V, FMT_GQ4V = 1, 2, 3, 4, 5
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
lib.tq_decode_workspace_init.restype = _I
lib.tq_decode_workspace_init.argtypes = [_PL, _I, _P, _SZ, _P]
lib.tq_decode_attention.restype = _I
lib.tq_decode_attention.argtypes = [_PL, _PC, _PC, _P, _P, _P, _P, _P, _P, _P, _I, _P, _SZ, _P]
lib.tq_decode_attention_static.restype = _I
lib.tq_decode_attention_static.argtypes = [_PL, _PC, _PC, _P, _P, _P, _P, _P, _P, _I, _P]
lib.tq_decode_partial.restype = _I
lib.tq_decode_partial.argtypes = [_PL, _PC, _PC, _P, _P, _P, _P, _P, _P, _I, _P, _SZ, _P]
lib.tq_decode_partial_timed.restype = _I
lib.tq_decode_partial_timed.argtypes = [_PL, _PC, _PC, _P, _P, _P, _P, _P, _P, _I, _P, _SZ, _P, _P, _P]
lib.tq_decode_combine.restype = _I
lib.tq_decode_partial_from_query.restype = _I
lib.tq_decode_partial_from_query.argtypes = [_PL, _PC, _PC, _P, _P, _P, _P, _P, _P, _I, _P, _SZ, _P, _P, _P]
lib.tq_decode_step.restype = _I
lib.tq_decode_step.argtypes = [_PL, _PC, _PC, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _P, _SZ, _P, _P, _P]
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
STATIC_SCRATCH_BYTES = 8 << 20


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


ERR_INVALID = -1

_F32 = (torch.float32,)
_I32 = (torch.int32,)
_F16 = (torch.float16, torch.int16)  # fp16 values, or their bit patterns
_ANY = None


def _bad(where, what):
    raise TQError(ERR_INVALID, f"{where}: {what}")


def _dev(t, name, where, nbytes, dtypes=_ANY, align=4, optional=False):
    """The address of a device tensor after the checks the C ABI cannot make."""
    if t is None:
        if optional:
            return None
        _bad(where, f"{name} is required")
    if not isinstance(t, torch.Tensor):
        _bad(where, f"{name} must be a torch tensor, not {type(t).__name__}")
    if not t.is_cuda:
        _bad(where, f"{name} must be a GPU tensor (got {t.device})")
    if t.device.index != torch.cuda.current_device():
        _bad(where, f"{name} is on {t.device}, the current device is cuda:{torch.cuda.current_device()}")
    if dtypes is not None and t.dtype not in dtypes:
        _bad(where, f"{name} must be {' or '.join(str(d) for d in dtypes)}, not {t.dtype}")
    if not t.is_contiguous():
        _bad(where, f"{name} must be contiguous")
    have = t.numel() * t.element_size()
    if have < nbytes:
        _bad(where, f"{name} holds {have} bytes, the call needs {nbytes}")
    if t.data_ptr() % align:
        _bad(where, f"{name} must be {align}-byte aligned")
    return ctypes.c_void_p(t.data_ptr())


def _rows(L):
    return L.batch * L.n_q_heads * L.head_dim * 4  # fp32 [B][Hq][d]


def _caches(L, k_cache, v_cache, where):
    kb, vb = cache_bytes(L)
    return (_dev(k_cache, "k_cache", where, kb, align=16), _dev(v_cache, "v_cache", where, vb, align=16))


def _qjl(L, S_dev, where):
    need = L.k_format == FMT_TQ3K
    return _dev(S_dev, "S_dev", where, L.head_dim * L.head_dim * 4, _F32, 16, optional=not need)


def _nbytes(t):
    return t.numel() * t.element_size()


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
    w = "tq_quantize_append"
    if not isinstance(dst_row, torch.Tensor) or dst_row.dim() != 1:
        _bad(w, "dst_row must be a 1-D int32 tensor")
    T = int(dst_row.shape[0])
    rows = T * L.n_kv_heads * L.head_dim * 2
    kc, vc = _caches(L, k_cache, v_cache, w)
    args = (_qjl(L, S_dev, w), _dev(k_new, "k_new", w, rows, _F16, 16), _dev(v_new, "v_new", w, rows, _F16, 16),
            _dev(dst_row, "dst_row", w, T * 4, _I32), T, kc, vc)
    _check(lib.tq_quantize_append(ctypes.byref(L), ctypes.byref(cbk), ctypes.byref(cbv), *args, _stream(stream)), w)


def quantize_rotated(fmt, cb, S_dev, y, norm16, blocks, stream=None):
    """y: fp32 [n, d]; norm16: fp16 [n]; blocks: uint8 [n * vector_bytes]."""
    w = "tq_quantize_rotated"
    if not isinstance(y, torch.Tensor) or y.dim() != 2:
        _bad(w, "y must be a 2-D fp32 tensor [n, d]")
    n, d = int(y.shape[0]), cb.head_dim
    S = _dev(S_dev, "S_dev", w, d * d * 4, _F32, 16, optional=fmt != FMT_TQ3K)
    _check(lib.tq_quantize_rotated(fmt, ctypes.byref(cb), S, _dev(y, "y", w, n * d * 4, _F32, 16),
                                   _dev(norm16, "norm16", w, n * 2, _F16, 2),
                                   n, _dev(blocks, "blocks", w, n * vector_bytes(fmt, d), align=16), _stream(stream)), w)


def rotate_sketch_query(L, cbk, S_dev, q, q_rot, q_sketch=None, stream=None):
    w = "tq_rotate_sketch_query"
    n = _rows(L)
    sk = L.k_format == FMT_TQ3K
    _check(lib.tq_rotate_sketch_query(ctypes.byref(L), ctypes.byref(cbk), _qjl(L, S_dev, w),
                                      _dev(q, "q", w, n, _F32, 16), _dev(q_rot, "q_rot", w, n, _F32, 16),
                                      _dev(q_sketch, "q_sketch", w, n, _F32, 16, optional=not sk), _stream(stream)), w)


def decode_splits(L, split_tokens=0):
    return int(lib.tq_decode_splits(ctypes.byref(L), split_tokens))


def decode_workspace_bytes(L, split_tokens=0):
    return int(lib.tq_decode_workspace_bytes(ctypes.byref(L), split_tokens))


def decode_workspace_init(L, ws, split_tokens=0, stream=None):
    """Clear the workspace's arrival counters (needed once after allocation)."""
    w = "tq_decode_workspace_init"
    _check(lib.tq_decode_workspace_init(ctypes.byref(L), split_tokens,
                                        _dev(ws, "ws", w, decode_workspace_bytes(L, split_tokens), align=16),
                                        _nbytes(ws), _stream(stream)), w)


def decode_workspace(L, split_tokens=0, device=None):
    """A device workspace for decodes of layout L, its arrival counters cleared."""
    nbytes = decode_workspace_bytes(L, split_tokens)
    if nbytes == 0:
        _bad("decode_workspace", "invalid layout or split length")
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=device if device is not None else "cuda")
    decode_workspace_init(L, ws, split_tokens)
    return ws


def _ws(L, ws, split_tokens, where):
    return _dev(ws, "ws", where, decode_workspace_bytes(L, split_tokens), align=16), _nbytes(ws)


def _decode_common(L, q_rot, q_sketch, k_cache, v_cache, seq_lens, scores, where):
    n = _rows(L)
    kc, vc = _caches(L, k_cache, v_cache, where)
    sk = L.k_format == FMT_TQ3K
    return (_dev(q_rot, "q_rot", where, n, _F32), _dev(q_sketch, "q_sketch", where, n, _F32, optional=not sk), kc, vc,
            _dev(seq_lens, "seq_lens", where, L.batch * 4, _I32))


def _scores(L, scores, where):
    return _dev(scores, "scores", where, L.batch * L.n_q_heads * L.capacity * 4, _F32, optional=True)


def decode_attention(L, cbk, cbv, q_rot, q_sketch, k_cache, v_cache, seq_lens, out, ws, scores=None,
                     split_tokens=0, stream=None):
    w = "tq_decode_attention"
    common = _decode_common(L, q_rot, q_sketch, k_cache, v_cache, seq_lens, scores, w)
    _check(lib.tq_decode_attention(ctypes.byref(L), ctypes.byref(cbk), ctypes.byref(cbv), *common,
                                   _dev(out, "out", w, _rows(L), _F32), _scores(L, scores, w), split_tokens,
                                   *_ws(L, ws, split_tokens, w), _stream(stream)), w)


def decode_attention_static(L, cbk, cbv, q_rot, q_sketch, k_cache, v_cache, seq_lens, out, split_tokens=0,
                            stream=None):
    """tq_decode_attention with the library's own device scratch instead of a workspace."""
    w = "tq_decode_attention_static"
    common = _decode_common(L, q_rot, q_sketch, k_cache, v_cache, seq_lens, None, w)
    _check(lib.tq_decode_attention_static(ctypes.byref(L), ctypes.byref(cbk), ctypes.byref(cbv), *common,
                                          _dev(out, "out", w, _rows(L), _F32), split_tokens, _stream(stream)), w)


def decode_partial(L, cbk, cbv, q_rot, q_sketch, k_cache, v_cache, seq_lens, ws, scores=None, split_tokens=0,
                   stream=None, events=None):
    """events: optional (start, stop) raw hipEvent_t handles, recorded at the
    kernel's own start and end (tq_decode_partial_timed)."""
    w = "tq_decode_partial"
    args = (ctypes.byref(L), ctypes.byref(cbk), ctypes.byref(cbv),
            *_decode_common(L, q_rot, q_sketch, k_cache, v_cache, seq_lens, scores, w), _scores(L, scores, w),
            split_tokens, *_ws(L, ws, split_tokens, w), _stream(stream))
    if events is None:
        _check(lib.tq_decode_partial(*args), w)
    else:
        start, stop = events
        _check(lib.tq_decode_partial_timed(*args, ctypes.c_void_p(start), ctypes.c_void_p(stop)),
               "tq_decode_partial_timed")


def decode_partial_from_query(L, cbk, cbv, q, q_rot_scratch, k_cache, v_cache, seq_lens, ws, scores=None,
                              split_tokens=0, stream=None, events=None):
    """events: optional (start, stop) raw hipEvent_t handles for the partial kernel's dispatch."""
    w = "tq_decode_partial_from_query"
    start, stop = events if events is not None else (None, None)
    n = _rows(L)
    kc, vc = _caches(L, k_cache, v_cache, w)
    _check(lib.tq_decode_partial_from_query(ctypes.byref(L), ctypes.byref(cbk), ctypes.byref(cbv),
                                            _dev(q, "q", w, n, _F32, 16),
                                            _dev(q_rot_scratch, "q_rot_scratch", w, n, _F32, 16), kc, vc,
                                            _dev(seq_lens, "seq_lens", w, L.batch * 4, _I32), _scores(L, scores, w),
                                            split_tokens, *_ws(L, ws, split_tokens, w), _stream(stream),
                                            ctypes.c_void_p(start), ctypes.c_void_p(stop)), w)


def decode_step(L, cbk, cbv, k_new, v_new, new_pos, q, q_rot_scratch, k_cache, v_cache, seq_lens, ws, out=None,
                scores=None, split_tokens=0, stream=None, events=None):
    """events: optional (start, stop) raw hipEvent_t handles for the partial kernel's dispatch;
    out: optional fp32 [B, Hq, d] attention output (the workspace's counters must be clear)."""
    w = "tq_decode_step"
    start, stop = events if events is not None else (None, None)
    n = _rows(L)
    rows = L.batch * L.n_kv_heads * L.head_dim * 2
    kc, vc = _caches(L, k_cache, v_cache, w)
    _check(lib.tq_decode_step(ctypes.byref(L), ctypes.byref(cbk), ctypes.byref(cbv),
                              _dev(k_new, "k_new", w, rows, _F16, 16), _dev(v_new, "v_new", w, rows, _F16, 16),
                              _dev(new_pos, "new_pos", w, L.batch * 4, _I32), _dev(q, "q", w, n, _F32, 16),
                              _dev(q_rot_scratch, "q_rot_scratch", w, n, _F32, 16), kc, vc,
                              _dev(seq_lens, "seq_lens", w, L.batch * 4, _I32),
                              _dev(out, "out", w, n, _F32, optional=True), _scores(L, scores, w), split_tokens,
                              *_ws(L, ws, split_tokens, w), _stream(stream), ctypes.c_void_p(start),
                              ctypes.c_void_p(stop)), w)


def decode_partial_sparse_v(L, cbk, cbv, q_rot, q_sketch, k_cache, v_cache, seq_lens, ws, v_threshold,
                            scores=None, split_tokens=0, stream=None):
    w = "tq_decode_partial_sparse_v"
    _check(lib.tq_decode_partial_sparse_v(ctypes.byref(L), ctypes.byref(cbk), ctypes.byref(cbv),
                                          *_decode_common(L, q_rot, q_sketch, k_cache, v_cache, seq_lens, scores, w),
                                          _scores(L, scores, w), split_tokens, float(v_threshold),
                                          *_ws(L, ws, split_tokens, w), _stream(stream)), w)


def decode_combine(L, cbv, ws, out, split_tokens=0, stream=None):
    w = "tq_decode_combine"
    _check(lib.tq_decode_combine(ctypes.byref(L), ctypes.byref(cbv), split_tokens, *_ws(L, ws, split_tokens, w),
                                 _dev(out, "out", w, _rows(L), _F32), _stream(stream)), w)


def ring_bytes(L, ring_cap):
    return int(lib.tq_ring_bytes(ctypes.byref(L), ring_cap))


def _rings(L, ring_cap, k_ring, v_ring, where):
    nb = ring_bytes(L, ring_cap)
    if nb == 0:
        _bad(where, f"invalid layout or ring_cap {ring_cap}")
    return _dev(k_ring, "k_ring", where, nb, _F16, 16), _dev(v_ring, "v_ring", where, nb, _F16, 16)


def ring_append(L, ring_cap, k_new, v_new, pos, k_ring, v_ring, stream=None):
    w = "tq_ring_append"
    rows = L.batch * L.n_kv_heads * L.head_dim * 2
    kr, vr = _rings(L, ring_cap, k_ring, v_ring, w)
    _check(lib.tq_ring_append(ctypes.byref(L), ring_cap, _dev(k_new, "k_new", w, rows, _F16, 16),
                              _dev(v_new, "v_new", w, rows, _F16, 16), _dev(pos, "pos", w, L.batch * 4, _I32),
                              kr, vr, _stream(stream)), w)


def ring_flush(L, cbk, cbv, S_dev, ring_cap, k_ring, v_ring, first, count, k_cache, v_cache, stream=None):
    w = "tq_ring_flush"
    kc, vc = _caches(L, k_cache, v_cache, w)
    _check(lib.tq_ring_flush(ctypes.byref(L), ctypes.byref(cbk), ctypes.byref(cbv), _qjl(L, S_dev, w), ring_cap,
                             *_rings(L, ring_cap, k_ring, v_ring, w), _dev(first, "first", w, L.batch * 4, _I32),
                             count, kc, vc, _stream(stream)), w)


def decode_hybrid_workspace_bytes(L, split_tokens=0):
    return int(lib.tq_decode_hybrid_workspace_bytes(ctypes.byref(L), split_tokens))


def decode_attention_hybrid(L, cbk, cbv, q_rot, q_sketch, k_cache, v_cache, comp_lens, ring_cap, k_ring, v_ring,
                            ring_lens, out, ws, split_tokens=0, stream=None):
    w = "tq_decode_attention_hybrid"
    common = _decode_common(L, q_rot, q_sketch, k_cache, v_cache, comp_lens, None, w)
    _check(lib.tq_decode_attention_hybrid(ctypes.byref(L), ctypes.byref(cbk), ctypes.byref(cbv), *common, ring_cap,
                                          *_rings(L, ring_cap, k_ring, v_ring, w),
                                          _dev(ring_lens, "ring_lens", w, L.batch * 4, _I32),
                                          _dev(out, "out", w, _rows(L), _F32), split_tokens,
                                          *_ws(L, ws, split_tokens, w), _stream(stream)), w)
