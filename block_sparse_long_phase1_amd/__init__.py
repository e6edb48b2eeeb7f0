"""Star Attention two-phase hot path on one AMD Instinct MI355X (gfx950).

Thin ctypes binding over ``libstarattn.so``; the entry points keep the C ABI's
names (see ``include/star_attn.h``).  PyTorch supplies device memory and the
current HIP stream; every step of the computation runs in the library's HIP
kernels.  There is no fallback: if the library is missing or a call fails, the
call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

from .configs import CONFIGS, StarConfig, n_blocks, shard_bounds  # noqa: F401

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libstarattn.so")

STAR_OK, STAR_ERR_INVALID_ARG, STAR_ERR_UNSUPPORTED, STAR_ERR_HIP, STAR_ERR_WORKSPACE = range(5)
STAR_F32, STAR_BF16 = 0, 1

_lib = None
_lock = threading.Lock()


class StarError(RuntimeError):
    def __init__(self, status: int, func: str, msg: str):
        super().__init__("%s failed with %s: %s" % (func, _status_name(status), msg))
        self.status = status


def _status_name(status: int) -> str:
    return load_library().star_status_str(status).decode()


def load_library(path: str | None = None, make_default: bool = False):
    """Load libstarattn.so (built in-tree by block_sparse_long_phase1_amd.build).  With `path`,
    load that build of the library instead (the profiling build, say); `make_default` then makes
    every binding below call it."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise RuntimeError("libstarattn.so not found at %s; build it with "
                               "`python -m block_sparse_long_phase1_amd.build`" % p)
        lib = ctypes.CDLL(p)
        vp, i64, i32, f32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
        lib.star_status_str.argtypes = [ctypes.c_int]
        lib.star_status_str.restype = ctypes.c_char_p
        lib.star_last_error.argtypes = []
        lib.star_last_error.restype = ctypes.c_char_p
        lib.star_version.argtypes = []
        lib.star_version.restype = ctypes.c_char_p
        lib.star_phase1_encode.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, i32, ctypes.c_int, f32, vp]
        lib.star_phase1_encode.restype = ctypes.c_int
        lib.star_phase2_workspace_bytes.argtypes = [i32, i64, i32, i32, i32]
        lib.star_phase2_workspace_bytes.restype = sz
        lib.star_phase2_partial.argtypes = [vp, i32, vp, vp, i64, i64, i64, i32, i32, i32, ctypes.c_int, f32,
                                            vp, vp, vp, vp, sz, vp]
        lib.star_phase2_partial.restype = ctypes.c_int
        lib.star_phase2_partial_kv8.argtypes = [vp, i32, vp, vp, vp, vp, i64, i64, i64, i32, i32, i32, ctypes.c_int,
                                                f32, vp, vp, vp, vp, sz, vp]
        lib.star_phase2_partial_kv8.restype = ctypes.c_int
        lib.star_softmax_merge.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp, ctypes.c_int, vp, vp]
        lib.star_softmax_merge.restype = ctypes.c_int
        lib.star_phase2_query_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
        lib.star_phase2_query_workspace_bytes.restype = sz
        lib.star_phase2_query.argtypes = [vp, i32, vp, vp, i64, vp, i32, vp, vp, i64, i64, i32, i32, i32,
                                          ctypes.c_int, f32, vp, vp, vp, sz, vp]
        lib.star_phase2_query.restype = ctypes.c_int
        lib.star_decode_workspace_bytes.argtypes = [i64, i64, i32, i32, i32, i32]
        lib.star_decode_workspace_bytes.restype = sz
        lib.star_decode_step.argtypes = [vp, vp, vp, vp, vp, i64, vp, i32, vp, vp, i64, i64, i32, i32, i32,
                                         ctypes.c_int, f32, vp, vp, vp, sz, vp]
        lib.star_decode_step.restype = ctypes.c_int
        lib.star_decode_step_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, vp, i32, vp, vp, i64, i64, i32, i32,
                                                 i32, ctypes.c_int, f32, vp, vp, vp]
        lib.star_decode_step_noalloc.restype = ctypes.c_int
        lib.star_kv_fp8_scales.argtypes = [vp, i64, i32, i32, ctypes.c_int, vp, vp]
        lib.star_kv_fp8_scales.restype = ctypes.c_int
        lib.star_kv_quantize_fp8.argtypes = [vp, i64, i32, i32, ctypes.c_int, vp, vp, vp]
        lib.star_kv_quantize_fp8.restype = ctypes.c_int
        lib.star_decode_step_kv8.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, vp, i32, vp, vp, i64, i64, i32, i32,
                                             i32, ctypes.c_int, f32, vp, vp, vp, sz, vp]
        lib.star_decode_step_kv8.restype = ctypes.c_int
        lib.star_phase2_query_kv8.argtypes = [vp, i32, vp, vp, vp, vp, i64, vp, i32, vp, vp, i64, i64, i32, i32,
                                              i32, ctypes.c_int, f32, vp, vp, vp, sz, vp]
        lib.star_phase2_query_kv8.restype = ctypes.c_int
        if path is None or make_default:
            _lib = lib
        return lib


def _check(status: int, func: str):
    if status != STAR_OK:
        lib = load_library()
        raise StarError(status, func, lib.star_last_error().decode())


# ----------------------------------------------------------------------------- marshalling
def _torch():
    import torch
    return torch


def _dt(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return STAR_BF16
    if t.dtype == torch.float32:
        return STAR_F32
    raise TypeError("tensors must be bfloat16 or float32, got %s" % t.dtype)


def _dev(t, name):
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return ctypes.c_void_p(t.data_ptr())


def _opt(t, name):
    return ctypes.c_void_p(0) if t is None else _dev(t, name)


def _f32(t, name, shape=None):
    """fp32 device tensor of the given shape (statistics, partials, LSE outputs)."""
    torch = _torch()
    if t.dtype != torch.float32:
        raise TypeError("%s must be float32, got %s" % (name, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    return _dev(t, name)


def _same(t, ref, name, shape):
    if t.dtype != ref.dtype:
        raise TypeError("%s must be %s, got %s" % (name, ref.dtype, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    return _dev(t, name)


def _u8(t, name, shape):
    """uint8 device tensor of the given shape (E4M3 codes)."""
    torch = _torch()
    if t.dtype != torch.uint8:
        raise TypeError("%s must be uint8 (E4M3 codes), got %s" % (name, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    return _dev(t, name)


def _stream(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _scale(d, scale):
    return float(1.0 / d ** 0.5) if scale is None else float(scale)


# ----------------------------------------------------------------------------- entry points
def star_phase1_encode(q, k, v, block: int, anchor: int, o=None, lse=None, scale=None,
                       want_lse: bool = True, stream=None):
    """Phase-1 anchored blockwise-local encoding.  q [Hq,L,d], k/v [Hkv,L,d] -> (o, lse)."""
    torch = _torch()
    hq, L, d = q.shape
    hkv = k.shape[0]
    if o is None:
        o = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((hq, L), dtype=torch.float32, device=q.device)
    st = load_library().star_phase1_encode(
        _dev(q, "q"), _same(k, q, "k", (hkv, L, d)), _same(v, q, "v", (hkv, L, d)),
        _same(o, q, "o", (hq, L, d)), ctypes.c_void_p(0) if lse is None else _f32(lse, "lse", (hq, L)),
        L, block, anchor, hq, hkv, d, _dt(q), _scale(d, scale), _stream(stream))
    _check(st, "star_phase1_encode")
    return o, lse


def star_phase2_workspace_bytes(rows: int, n_kv: int, hq: int, hkv: int, d: int) -> int:
    return int(load_library().star_phase2_workspace_bytes(rows, n_kv, hq, hkv, d))


def _kv_view(t, q, name, hkv, d):
    """Base pointer of a (possibly strided) partition view [Hkv, n, d] of a bigger cache."""
    if t is None:
        return ctypes.c_void_p(0)
    if not t.is_cuda or t.dtype != q.dtype or t.shape[0] != hkv or t.shape[-1] != d or t.stride(-1) != 1:
        raise ValueError("%s must be a device [Hkv, n, d] view with unit last stride and q's dtype" % name)
    return ctypes.c_void_p(t.data_ptr())


def _partition_stride(k, v, n_kv: int, kv_head_stride, d: int) -> int:
    """The element stride between kv heads of a partition view pair, checked against both
    views: k and v must share it, hold n_kv tokens per head and, from their first element,
    reach (hkv - 1) * stride + n_kv * d elements inside their storage."""
    hkv = k.shape[0]
    stride = k.stride(0) if kv_head_stride is None else int(kv_head_stride)
    if v.shape[0] != hkv:
        raise ValueError("k and v views must have the same number of kv heads")
    for t, name in ((k, "k"), (v, "v")):
        if t.dim() != 3 or t.shape[-1] != d or (t.shape[1] > 1 and t.stride(1) != d):
            raise ValueError("%s must be a [Hkv, n, %d] view whose tokens are %d elements apart" % (name, d, d))
    if hkv > 1 and (k.stride(0) != stride or v.stride(0) != stride):
        raise ValueError("kv_head_stride %d must equal k.stride(0) (%d) and v.stride(0) (%d)"
                         % (stride, k.stride(0), v.stride(0)))
    if n_kv > 0:
        for t, name in ((k, "k"), (v, "v")):
            if t.shape[1] < n_kv:
                raise ValueError("%s view holds %d tokens, n_kv is %d" % (name, t.shape[1], n_kv))
            avail = t.untyped_storage().nbytes() // t.element_size() - t.storage_offset()
            if (hkv - 1) * stride + n_kv * d > avail:
                raise ValueError("%s view: %d kv heads of %d tokens at stride %d run past its storage"
                                 % (name, hkv, n_kv, stride))
    return stride


def _kv8_view(t, name, hkv, d):
    """Base pointer of a (possibly strided) uint8 E4M3 partition view [Hkv, n, d]."""
    torch = _torch()
    if t is None:
        return ctypes.c_void_p(0)
    if not t.is_cuda or t.dtype != torch.uint8 or t.shape[0] != hkv or t.shape[-1] != d or t.stride(-1) != 1:
        raise ValueError("%s must be a device uint8 [Hkv, n, d] view with unit last stride" % name)
    return ctypes.c_void_p(t.data_ptr())


def star_phase2_partial(q, k, v, kv_head_stride, n_kv: int, causal_offset: int = -1,
                        a_out=None, m_out=None, l_out=None, workspace=None, scale=None, stream=None):
    """Local attention of q [Hq,rows,d] over one KV partition.

    k/v are device views [Hkv, >=n_kv, d] whose first element is partition token 0 of kv
    head 0 (e.g. ``k_ctx[:, lo:]``), with ``kv_head_stride`` elements between kv heads (None:
    k.stride(0); it must equal both views' stride).  Returns fp32 (A [Hq,rows,d], m [Hq,rows],
    l [Hq,rows]).
    """
    torch = _torch()
    hq, rows, d = q.shape
    hkv = k.shape[0]
    dev = q.device
    if a_out is None:
        a_out = torch.empty((hq, rows, d), dtype=torch.float32, device=dev)
    if m_out is None:
        m_out = torch.empty((hq, rows), dtype=torch.float32, device=dev)
    if l_out is None:
        l_out = torch.empty((hq, rows), dtype=torch.float32, device=dev)
    kv_head_stride = _partition_stride(k, v, n_kv, kv_head_stride, d)
    need = star_phase2_workspace_bytes(rows, n_kv, hq, hkv, d)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else ctypes.c_void_p(0)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = load_library().star_phase2_partial(
        _dev(q, "q"), rows, _kv_view(k, q, "k", hkv, d), _kv_view(v, q, "v", hkv, d), kv_head_stride,
        n_kv, causal_offset, hq, hkv, d, _dt(q), _scale(d, scale), _f32(a_out, "a_out", (hq, rows, d)),
        _f32(m_out, "m_out", (hq, rows)), _f32(l_out, "l_out", (hq, rows)), ws_ptr, ws_bytes, _stream(stream))
    _check(st, "star_phase2_partial")
    return a_out, m_out, l_out


def star_phase2_partial_kv8(q, k8, v8, k_scale, v_scale, kv_head_stride, n_kv: int, causal_offset: int = -1,
                            a_out=None, m_out=None, l_out=None, workspace=None, scale=None, stream=None):
    """star_phase2_partial over a partition of E4M3 codes: k8/v8 are uint8 device views
    [Hkv, >=n_kv, d] (e.g. ``k8_ctx[:, lo:]``) with fp32 scales [Hkv]; q is bf16.
    kv_head_stride as in star_phase2_partial (None: k8.stride(0))."""
    torch = _torch()
    hq, rows, d = q.shape
    hkv = k8.shape[0]
    dev = q.device
    if a_out is None:
        a_out = torch.empty((hq, rows, d), dtype=torch.float32, device=dev)
    if m_out is None:
        m_out = torch.empty((hq, rows), dtype=torch.float32, device=dev)
    if l_out is None:
        l_out = torch.empty((hq, rows), dtype=torch.float32, device=dev)
    kv_head_stride = _partition_stride(k8, v8, n_kv, kv_head_stride, d)
    need = star_phase2_workspace_bytes(rows, n_kv, hq, hkv, d)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else ctypes.c_void_p(0)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = load_library().star_phase2_partial_kv8(
        _dev(q, "q"), rows, _kv8_view(k8, "k8", hkv, d), _kv8_view(v8, "v8", hkv, d),
        _f32(k_scale, "k_scale", (hkv,)), _f32(v_scale, "v_scale", (hkv,)), kv_head_stride, n_kv, causal_offset,
        hq, hkv, d, _dt(q), _scale(d, scale), _f32(a_out, "a_out", (hq, rows, d)), _f32(m_out, "m_out", (hq, rows)),
        _f32(l_out, "l_out", (hq, rows)), ws_ptr, ws_bytes, _stream(stream))
    _check(st, "star_phase2_partial_kv8")
    return a_out, m_out, l_out


def star_softmax_merge(a, m, l, o=None, lse=None, out_dtype=None, want_lse: bool = True, stream=None):
    """Merge partials a [P,Hq,rows,d], m/l [P,Hq,rows] -> (o [Hq,rows,d], lse [Hq,rows])."""
    torch = _torch()
    P, hq, rows, d = a.shape
    out_dtype = out_dtype or torch.float32
    if o is None:
        o = torch.empty((hq, rows, d), dtype=out_dtype, device=a.device)
    if lse is None and want_lse:
        lse = torch.empty((hq, rows), dtype=torch.float32, device=a.device)
    if tuple(o.shape) != (hq, rows, d):
        raise ValueError("o must have shape %s" % ((hq, rows, d),))
    st = load_library().star_softmax_merge(
        _f32(a, "a"), _f32(m, "m", (P, hq, rows)), _f32(l, "l", (P, hq, rows)), P, hq, rows, d,
        _dev(o, "o"), _dt(o), ctypes.c_void_p(0) if lse is None else _f32(lse, "lse", (hq, rows)),
        _stream(stream))
    _check(st, "star_softmax_merge")
    return o, lse


def star_decode_workspace_bytes(L: int, tail_cap: int, n_shards: int, hq: int, hkv: int, d: int) -> int:
    return int(load_library().star_decode_workspace_bytes(L, tail_cap, n_shards, hq, hkv, d))


def decode_workspace(L: int, tail_cap: int, n_shards: int, hq: int, hkv: int, d: int, device):
    """A zero-filled decode workspace (reusable across steps on one stream)."""
    torch = _torch()
    need = star_decode_workspace_bytes(L, tail_cap, n_shards, hq, hkv, d)
    return torch.zeros(max(need, 16), dtype=torch.uint8, device=device)


def star_phase2_query_workspace_bytes(rows: int, n_shards: int, hq: int, hkv: int, d: int) -> int:
    return int(load_library().star_phase2_query_workspace_bytes(rows, n_shards, hq, hkv, d))


def star_phase2_query(q, k_ctx, v_ctx, bounds, k_tail, v_tail, tail_len: int, o=None, lse=None,
                      workspace=None, scale=None, want_lse: bool = True, stream=None):
    """Query encoding on the query host: q [Hq,rows,d] are the last `rows` of the tail's
    tail_len valid tokens; caches [Hkv,L,d] and [Hkv,tail_cap,d]; bounds: S+1 host ints."""
    torch = _torch()
    hq, rows, d = q.shape
    hkv, L, _ = k_ctx.shape
    tail_cap = k_tail.shape[1]
    n_shards = len(bounds) - 1
    if o is None:
        o = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((hq, rows), dtype=torch.float32, device=q.device)
    if workspace is None:
        nb = star_phase2_query_workspace_bytes(rows, n_shards, hq, hkv, d)
        workspace = torch.empty(max(nb, 16), dtype=torch.uint8, device=q.device)
    b = (ctypes.c_int64 * (n_shards + 1))(*[int(x) for x in bounds])
    st = load_library().star_phase2_query(
        _dev(q, "q"), rows, _same(k_ctx, q, "k_ctx", (hkv, L, d)), _same(v_ctx, q, "v_ctx", (hkv, L, d)), L, b,
        n_shards, _same(k_tail, q, "k_tail", (hkv, tail_cap, d)), _same(v_tail, q, "v_tail", (hkv, tail_cap, d)),
        tail_len, tail_cap, hq, hkv, d, _dt(q), _scale(d, scale), _same(o, q, "o", (hq, rows, d)),
        ctypes.c_void_p(0) if lse is None else _f32(lse, "lse", (hq, rows)),
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "star_phase2_query")
    return o, lse


def star_decode_step(q_new, k_new, v_new, k_ctx, v_ctx, bounds, k_tail, v_tail, tail_len: int,
                     o=None, lse=None, workspace=None, scale=None, want_lse: bool = True, stream=None):
    """One generated token: q_new [Hq,d], k_new/v_new [Hkv,d]; caches [Hkv,L,d] and
    [Hkv,tail_cap,d]; bounds: S+1 host ints.  Appends k_new/v_new at tail_len."""
    torch = _torch()
    hq, d = q_new.shape
    hkv, L, _ = k_ctx.shape
    tail_cap = k_tail.shape[1]
    n_shards = len(bounds) - 1
    if o is None:
        o = torch.empty((hq, d), dtype=q_new.dtype, device=q_new.device)
    if lse is None and want_lse:
        lse = torch.empty((hq,), dtype=torch.float32, device=q_new.device)
    if workspace is None:
        workspace = decode_workspace(L, tail_cap, n_shards, hq, hkv, d, q_new.device)
    b = (ctypes.c_int64 * (n_shards + 1))(*[int(x) for x in bounds])
    st = load_library().star_decode_step(
        _dev(q_new, "q_new"), _same(k_new, q_new, "k_new", (hkv, d)), _same(v_new, q_new, "v_new", (hkv, d)),
        _same(k_ctx, q_new, "k_ctx", (hkv, L, d)), _same(v_ctx, q_new, "v_ctx", (hkv, L, d)), L, b, n_shards,
        _same(k_tail, q_new, "k_tail", (hkv, tail_cap, d)), _same(v_tail, q_new, "v_tail", (hkv, tail_cap, d)),
        tail_len, tail_cap, hq, hkv, d, _dt(q_new), _scale(d, scale), _same(o, q_new, "o", (hq, d)),
        ctypes.c_void_p(0) if lse is None else _f32(lse, "lse", (hq,)),
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "star_decode_step")
    return o, lse


def star_decode_step_noalloc(q_new, k_new, v_new, k_ctx, v_ctx, bounds, k_tail, v_tail, tail_len: int,
                             o, lse=None, scale=None, stream=None):
    """star_decode_step without a workspace: the library keeps the chunk partials in its own
    static device scratch (calls on one GPU must not overlap).  The caller passes the
    outputs o [Hq,d] (and optionally lse [Hq]); nothing is allocated here either."""
    hq, d = q_new.shape
    hkv, L, _ = k_ctx.shape
    tail_cap = k_tail.shape[1]
    n_shards = len(bounds) - 1
    b = (ctypes.c_int64 * (n_shards + 1))(*[int(x) for x in bounds])
    st = load_library().star_decode_step_noalloc(
        _dev(q_new, "q_new"), _same(k_new, q_new, "k_new", (hkv, d)), _same(v_new, q_new, "v_new", (hkv, d)),
        _same(k_ctx, q_new, "k_ctx", (hkv, L, d)), _same(v_ctx, q_new, "v_ctx", (hkv, L, d)), L, b, n_shards,
        _same(k_tail, q_new, "k_tail", (hkv, tail_cap, d)), _same(v_tail, q_new, "v_tail", (hkv, tail_cap, d)),
        tail_len, tail_cap, hq, hkv, d, _dt(q_new), _scale(d, scale), _same(o, q_new, "o", (hq, d)),
        ctypes.c_void_p(0) if lse is None else _f32(lse, "lse", (hq,)), _stream(stream))
    _check(st, "star_decode_step_noalloc")
    return o, lse


def star_kv_fp8_scales(x, scale=None, stream=None):
    """Per-kv-head E4M3 scales of a context cache x [Hkv, tokens, d] (bf16 or fp32):
    max |x[g]| / 448 (1 for an all-zero head), fp32 [Hkv]."""
    torch = _torch()
    hkv, n, d = x.shape
    if scale is None:
        scale = torch.empty((hkv,), dtype=torch.float32, device=x.device)
    st = load_library().star_kv_fp8_scales(_dev(x, "x"), n, hkv, d, _dt(x), _f32(scale, "scale", (hkv,)),
                                           _stream(stream))
    _check(st, "star_kv_fp8_scales")
    return scale


def star_kv_quantize_fp8(x, scale, out=None, stream=None):
    """E4M3 codes (uint8 [Hkv, tokens, d]) of x [Hkv, tokens, d] / scale[g]."""
    torch = _torch()
    hkv, n, d = x.shape
    if out is None:
        out = torch.empty((hkv, n, d), dtype=torch.uint8, device=x.device)
    st = load_library().star_kv_quantize_fp8(_dev(x, "x"), n, hkv, d, _dt(x), _f32(scale, "scale", (hkv,)),
                                             _u8(out, "out", (hkv, n, d)), _stream(stream))
    _check(st, "star_kv_quantize_fp8")
    return out


def star_decode_step_kv8(q_new, k_new, v_new, k_ctx8, v_ctx8, k_scale, v_scale, bounds, k_tail, v_tail,
                         tail_len: int, o=None, lse=None, workspace=None, scale=None, want_lse: bool = True,
                         stream=None):
    """star_decode_step over an E4M3 context cache: k_ctx8/v_ctx8 uint8 [Hkv,L,d] with fp32
    scales [Hkv]; everything else bf16 as in star_decode_step."""
    torch = _torch()
    hq, d = q_new.shape
    hkv, L, _ = k_ctx8.shape
    tail_cap = k_tail.shape[1]
    n_shards = len(bounds) - 1
    if o is None:
        o = torch.empty((hq, d), dtype=q_new.dtype, device=q_new.device)
    if lse is None and want_lse:
        lse = torch.empty((hq,), dtype=torch.float32, device=q_new.device)
    if workspace is None:
        workspace = decode_workspace(L, tail_cap, n_shards, hq, hkv, d, q_new.device)
    b = (ctypes.c_int64 * (n_shards + 1))(*[int(x) for x in bounds])
    st = load_library().star_decode_step_kv8(
        _dev(q_new, "q_new"), _same(k_new, q_new, "k_new", (hkv, d)), _same(v_new, q_new, "v_new", (hkv, d)),
        _u8(k_ctx8, "k_ctx8", (hkv, L, d)), _u8(v_ctx8, "v_ctx8", (hkv, L, d)),
        _f32(k_scale, "k_scale", (hkv,)), _f32(v_scale, "v_scale", (hkv,)), L, b, n_shards,
        _same(k_tail, q_new, "k_tail", (hkv, tail_cap, d)), _same(v_tail, q_new, "v_tail", (hkv, tail_cap, d)),
        tail_len, tail_cap, hq, hkv, d, _dt(q_new), _scale(d, scale), _same(o, q_new, "o", (hq, d)),
        ctypes.c_void_p(0) if lse is None else _f32(lse, "lse", (hq,)),
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "star_decode_step_kv8")
    return o, lse


def star_phase2_query_kv8(q, k_ctx8, v_ctx8, k_scale, v_scale, bounds, k_tail, v_tail, tail_len: int, o=None,
                          lse=None, workspace=None, scale=None, want_lse: bool = True, stream=None):
    """star_phase2_query over an E4M3 context cache: k_ctx8/v_ctx8 uint8 [Hkv,L,d] with fp32
    scales [Hkv]; everything else bf16 as in star_phase2_query."""
    torch = _torch()
    hq, rows, d = q.shape
    hkv, L, _ = k_ctx8.shape
    tail_cap = k_tail.shape[1]
    n_shards = len(bounds) - 1
    if o is None:
        o = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((hq, rows), dtype=torch.float32, device=q.device)
    if workspace is None:
        nb = star_phase2_query_workspace_bytes(rows, n_shards, hq, hkv, d)
        workspace = torch.empty(max(nb, 16), dtype=torch.uint8, device=q.device)
    b = (ctypes.c_int64 * (n_shards + 1))(*[int(x) for x in bounds])
    st = load_library().star_phase2_query_kv8(
        _dev(q, "q"), rows, _u8(k_ctx8, "k_ctx8", (hkv, L, d)), _u8(v_ctx8, "v_ctx8", (hkv, L, d)),
        _f32(k_scale, "k_scale", (hkv,)), _f32(v_scale, "v_scale", (hkv,)), L, b, n_shards,
        _same(k_tail, q, "k_tail", (hkv, tail_cap, d)), _same(v_tail, q, "v_tail", (hkv, tail_cap, d)),
        tail_len, tail_cap, hq, hkv, d, _dt(q), _scale(d, scale), _same(o, q, "o", (hq, rows, d)),
        ctypes.c_void_p(0) if lse is None else _f32(lse, "lse", (hq, rows)),
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "star_phase2_query_kv8")
    return o, lse


__all__ = [
    "CONFIGS", "StarConfig", "n_blocks", "shard_bounds", "load_library", "StarError",
    "star_phase1_encode", "star_phase2_workspace_bytes", "star_phase2_partial", "star_softmax_merge",
    "star_phase2_query_workspace_bytes", "star_phase2_query",
    "star_decode_workspace_bytes", "star_decode_step", "decode_workspace", "STAR_F32", "STAR_BF16",
    "star_kv_fp8_scales", "star_kv_quantize_fp8", "star_decode_step_kv8", "star_phase2_query_kv8",
    "star_phase2_partial_kv8", "star_decode_step_noalloc",
]
