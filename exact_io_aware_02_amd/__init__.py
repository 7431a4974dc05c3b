"""Exact attention on MI355X: Python binding of libfa.so.

Thin ctypes marshalling over the C ABI in ``include/fa.h``.  The functions
named like the C entry points (``fa_fwd``, ``fa_fwd_strided``, ``fa_fwd_ex``,
``fa_fwd_splitk``, ``fa_fwd_fp8``, ``fa_bwd``, ``fa_bwd_strided``, ``fa_bwd_stages``, ``fa_bwd_ex``,
``fa_bwd_noalloc``, the workspace-size queries, ``fa_status_string``, ``fa_last_error_message``)
take torch tensors, read their sizes and strides,
and call the library on the tensors' device and current stream.  Every step
of the computation runs in the library's HIP kernels; there is no other
implementation here, and nothing falls back: if libfa.so is missing or the
device is not gfx950, calls raise.

``attention_fwd`` / ``attention_bwd`` / ``attention_fwd_fp8`` are conveniences that allocate the
outputs (and the backward workspace) with torch, then call the entry points.
"""
import ctypes
import math
import os

import torch

__all__ = [
    "FA_OK", "FA_ERR_INVALID_ARG", "FA_ERR_UNSUPPORTED", "FA_ERR_DEVICE", "FA_ERR_LAUNCH",
    "FA_FP16", "FA_BF16", "FaError", "lib_path", "load_library",
    "fa_fwd", "fa_fwd_strided", "fa_fwd_ex", "fa_fwd_fp8", "fa_bwd", "fa_bwd_strided", "fa_bwd_stages",
    "fa_bwd_ex", "fa_bwd_workspace_bytes", "fa_bwd_ex_workspace_bytes", "fa_bwd_noalloc",
    "fa_fwd_splitk", "fa_fwd_splitk_workspace_bytes",
    "FA_BWD_NOALLOC_SCRATCH_BYTES",
    "FA_BWD_PREP", "FA_BWD_DKDV", "FA_BWD_DQ", "FA_BWD_ALL",
    "fa_status_string", "fa_last_error_message", "fa_abi_version",
    "attention_fwd", "attention_bwd", "attention_fwd_fp8", "EXPORTED_SYMBOLS",
]

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_DEVICE, FA_ERR_LAUNCH = 0, 1, 2, 3, 4
FA_FP16, FA_BF16 = 0, 1
FA_BWD_PREP, FA_BWD_DKDV, FA_BWD_DQ, FA_BWD_ALL = 1, 2, 4, 7

EXPORTED_SYMBOLS = (
    "fa_fwd", "fa_fwd_strided", "fa_fwd_ex", "fa_bwd_workspace_bytes", "fa_bwd", "fa_bwd_strided", "fa_bwd_stages",
    "fa_bwd_ex", "fa_fwd_fp8", "fa_bwd_ex_workspace_bytes", "fa_bwd_noalloc", "fa_fwd_splitk",
    "fa_fwd_splitk_workspace_bytes", "fa_status_string", "fa_last_error_message", "fa_abi_version",
)
FA_BWD_NOALLOC_SCRATCH_BYTES = 8 << 20

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_u64, _u32 = ctypes.c_uint64, ctypes.c_uint32
_I64x3 = ctypes.c_int64 * 3


_STATUS_NAMES = {FA_OK: "FA_OK", FA_ERR_INVALID_ARG: "FA_ERR_INVALID_ARG", FA_ERR_UNSUPPORTED: "FA_ERR_UNSUPPORTED",
                 FA_ERR_DEVICE: "FA_ERR_DEVICE", FA_ERR_LAUNCH: "FA_ERR_LAUNCH"}


class FaError(RuntimeError):
    """A nonzero status from libfa.so, or an argument the binding rejects
    before calling it (with the status the library uses for such errors)."""

    def __init__(self, status, detail):
        self.status = status
        super().__init__("%s: %s" % (_STATUS_NAMES.get(status, "FA_UNKNOWN_STATUS"), detail))


def lib_path():
    """The in-tree libfa.so, or the file EXACT_IO_AWARE_FA_LIB names (the
    sanitizer build of the host code uses this)."""
    return os.environ.get("EXACT_IO_AWARE_FA_LIB") or os.path.join(_HERE, "libfa.so")


def load_library():
    """Load libfa.so (built in-tree by ``python -m exact_io_aware_02_amd.build``)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError("libfa.so is not built (%s); run: python -m exact_io_aware_02_amd.build" % path)
    lib = ctypes.CDLL(path)
    lib.fa_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _i, _vp]
    lib.fa_fwd.restype = _i
    lib.fa_fwd_strided.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _i,
                                   _I64x3, _I64x3, _I64x3, _I64x3, _vp]
    lib.fa_fwd_strided.restype = _i
    lib.fa_bwd_workspace_bytes.argtypes = [_i, _i, _i, _i, _i, _i]
    lib.fa_bwd_workspace_bytes.restype = _sz
    lib.fa_bwd_ex_workspace_bytes.argtypes = [_i, _i, _i, _i, _i, _i, _i]
    lib.fa_bwd_ex_workspace_bytes.restype = _sz
    lib.fa_bwd.argtypes = [_vp] * 9 + [_i] * 5 + [_f, _i, _i, _vp, _sz, _vp]
    lib.fa_bwd.restype = _i
    lib.fa_bwd_strided.argtypes = [_vp] * 9 + [_i] * 5 + [_f, _i, _i] + [_I64x3] * 8 + [_vp, _sz, _vp]
    lib.fa_bwd_strided.restype = _i
    lib.fa_bwd_stages.argtypes = [_vp] * 9 + [_i] * 5 + [_f, _i, _i] + [_I64x3] * 8 + [_vp, _sz, _i, _vp]
    lib.fa_bwd_stages.restype = _i
    lib.fa_fwd_ex.argtypes = [_vp] * 5 + [_i] * 6 + [_f, _i, _i, _i, _f, _u64, _u32, _i] + [_I64x3] * 4 + [_vp]
    lib.fa_fwd_ex.restype = _i
    lib.fa_bwd_ex.argtypes = ([_vp] * 9 + [_i] * 6 + [_f, _i, _i, _i, _f, _u64, _u32, _i] + [_I64x3] * 8 +
                              [_vp, _sz, _i, _vp])
    lib.fa_bwd_ex.restype = _i
    lib.fa_fwd_fp8.argtypes = [_vp] * 5 + [_i] * 6 + [_f, _i, _i, _i, _f, _f, _f] + [_I64x3] * 4 + [_vp]
    lib.fa_fwd_fp8.restype = _i
    lib.fa_bwd_noalloc.argtypes = [_vp] * 9 + [_i] * 5 + [_f, _i, _i, _vp]
    lib.fa_bwd_noalloc.restype = _i
    lib.fa_fwd_splitk.argtypes = ([_vp] * 5 + [_i] * 6 + [_f, _i, _i, _i, _f, _u64, _u32, _i] + [_I64x3] * 4 +
                                  [_vp, _sz, _vp])
    lib.fa_fwd_splitk.restype = _i
    lib.fa_fwd_splitk_workspace_bytes.argtypes = [_i] * 8
    lib.fa_fwd_splitk_workspace_bytes.restype = _sz
    lib.fa_status_string.argtypes = [_i]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_last_error_message.argtypes = []
    lib.fa_last_error_message.restype = ctypes.c_char_p
    lib.fa_abi_version.argtypes = []
    lib.fa_abi_version.restype = _i
    _LIB = lib
    return lib


def fa_status_string(status):
    return load_library().fa_status_string(int(status)).decode()


def fa_last_error_message():
    return load_library().fa_last_error_message().decode()


def fa_abi_version():
    return load_library().fa_abi_version()


def _check(status):
    if status != FA_OK:
        raise FaError(status, fa_last_error_message())


def _dtype_code(t):
    if t.dtype == torch.float16:
        return FA_FP16
    if t.dtype == torch.bfloat16:
        return FA_BF16
    raise FaError(FA_ERR_UNSUPPORTED, "dtype %s unsupported (float16 or bfloat16; fp32 is not supported)" % t.dtype)


def _on_device(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise FaError(FA_ERR_INVALID_ARG, "tensors must live on a HIP device (got %s)" % t.device)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t, stream):
    if stream is not None:
        return ctypes.c_void_p(stream if isinstance(stream, int) else stream.cuda_stream)
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


_AXES = {"bhsd": (0, 1, 2, 3), "bshd": (0, 2, 1, 3)}


def _axes(layout):
    try:
        return _AXES[layout]
    except KeyError:
        raise ValueError("layout must be 'bhsd' or 'bshd'") from None


def _dims(t, layout):
    """(B, H, N, d) of a 4-D tensor in the given layout."""
    ab, ah, as_, ad = _axes(layout)
    if t.dim() != 4:
        raise FaError(FA_ERR_INVALID_ARG, "expected a 4-D tensor, got shape %r" % (tuple(t.shape),))
    return t.shape[ab], t.shape[ah], t.shape[as_], t.shape[ad]


# ---------------------------------------------------------------- validation
# Every extent the library uses comes from q's and k's sizes, so each other
# tensor is checked against them here, before the call: a smaller v, dO or
# dV, an lse that is not fp32 [B, H, Nq], or a mixed fp16/bf16 set would
# otherwise be read or written out of bounds, or reinterpreted.

def _bad(msg):
    raise FaError(FA_ERR_INVALID_ARG, msg)


def _want_shape(name, t, shape):
    if tuple(t.shape) != tuple(shape):
        _bad("%s has shape %r, expected %r" % (name, tuple(t.shape), tuple(shape)))


def _want_dtype(dtype, **ts):
    for name, t in ts.items():
        if t.dtype != dtype:
            _bad("%s is %s, expected %s" % (name, t.dtype, dtype))


def _want_contiguous(**ts):
    for name, t in ts.items():
        if not t.is_contiguous():
            _bad("%s must be contiguous for this entry point (use the _strided/_ex variant)" % name)


def _want_lse(lse, B, H, Nq):
    if lse.dtype != torch.float32:
        _bad("lse is %s, expected torch.float32" % lse.dtype)
    _want_shape("lse", lse, (B, H, Nq))
    if not lse.is_contiguous():
        _bad("lse must be a contiguous [B, H, Nq] array")


def _want_device(q, **ts):
    if not q.is_cuda:
        _bad("tensors must live on a HIP device (q is on %s)" % q.device)
    for name, t in ts.items():
        if not t.is_cuda:
            _bad("tensors must live on a HIP device (%s is on %s)" % (name, t.device))
        if t.device != q.device:
            _bad("%s is on %s, q on %s" % (name, t.device, q.device))


def _check_fwd(q, k, v, o, lse, layout, contiguous=False, same_heads=True, out_dtype=None, device=True):
    """Validate a forward call; returns (B, H, H_kv, Nq, Nk, d)."""
    B, H, Nq, d = _dims(q, layout)
    Bk, Hkv, Nk, dk = _dims(k, layout)
    _want_dtype(q.dtype, k=k, v=v)
    _want_dtype(q.dtype if out_dtype is None else out_dtype, o=o)
    if Bk != B or dk != d or (same_heads and Hkv != H):
        _bad("k has %s dims (B, H, N, d) = %r, incompatible with q's %r" % (layout, (Bk, Hkv, Nk, dk), (B, H, Nq, d)))
    _want_shape("v", v, k.shape)
    _want_shape("o", o, q.shape)
    _want_lse(lse, B, H, Nq)
    if contiguous:
        _want_contiguous(q=q, k=k, v=v, o=o)
    if device:
        _want_device(q, k=k, v=v, o=o, lse=lse)
    return B, H, Hkv, Nq, Nk, d


def _check_bwd(q, k, v, o, lse, do, dq, dk, dv, workspace, layout, contiguous=False, same_heads=True):
    """Validate a backward call; returns (B, H, H_kv, Nq, Nk, d)."""
    dims = _check_fwd(q, k, v, o, lse, layout, contiguous, same_heads, device=False)
    _want_dtype(q.dtype, do=do, dq=dq, dk=dk, dv=dv)
    _want_shape("dout", do, q.shape)
    _want_shape("dq", dq, q.shape)
    _want_shape("dk", dk, k.shape)
    _want_shape("dv", dv, k.shape)
    if contiguous:
        _want_contiguous(do=do, dq=dq, dk=dk, dv=dv)
    if not workspace.is_contiguous():
        _bad("workspace must be contiguous")
    _want_device(q, k=k, v=v, o=o, lse=lse, do=do, dq=dq, dk=dk, dv=dv, workspace=workspace)
    return dims


def _strides(t, layout):
    ab, ah, as_, ad = _axes(layout)
    if t.shape[ad] > 1 and t.stride(ad) != 1:
        raise FaError(FA_ERR_INVALID_ARG, "the d dimension must be contiguous")
    return _I64x3(t.stride(ab), t.stride(ah), t.stride(as_))


def _default_scale(d, scale):
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def fa_fwd(q, k, v, o, lse, scale, causal, stream=None):
    """C ``fa_fwd`` on contiguous BHSD tensors: q/o [B,H,Nq,d], k/v [B,H,Nk,d],
    lse fp32 [B,H,Nq].  Enqueues on ``stream`` (default: current stream)."""
    dt = _dtype_code(q)
    B, H, _, Nq, Nk, d = _check_fwd(q, k, v, o, lse, "bhsd", contiguous=True)
    with torch.cuda.device(q.device):
        _check(load_library().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Nq, Nk, d,
                                     float(scale), int(bool(causal)), dt, _stream(q, stream)))


def fa_fwd_strided(q, k, v, o, lse, scale, causal, layout="bshd", stream=None):
    """C ``fa_fwd_strided``: the tensors' own strides, read in ``layout``."""
    dt = _dtype_code(q)
    B, H, _, Nq, Nk, d = _check_fwd(q, k, v, o, lse, layout)
    with torch.cuda.device(q.device):
        _check(load_library().fa_fwd_strided(
            _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Nq, Nk, d, float(scale), int(bool(causal)),
            dt, _strides(q, layout), _strides(k, layout), _strides(v, layout), _strides(o, layout),
            _stream(q, stream)))


def fa_bwd_workspace_bytes(B, H, Nq, Nk, d, dtype):
    return int(load_library().fa_bwd_workspace_bytes(B, H, Nq, Nk, d, dtype))


def fa_bwd_ex_workspace_bytes(B, H, H_kv, Nq, Nk, d, dtype):
    """C ``fa_bwd_ex_workspace_bytes``: the workspace that lets ``fa_bwd_ex``
    split the dK/dV stage when there are fewer K/V heads."""
    return int(load_library().fa_bwd_ex_workspace_bytes(B, H, H_kv, Nq, Nk, d, dtype))


def fa_bwd(q, k, v, o, lse, do, dq, dk, dv, scale, causal, workspace, stream=None):
    """C ``fa_bwd`` on contiguous BHSD tensors; ``workspace`` is a device
    tensor of at least ``fa_bwd_workspace_bytes`` bytes."""
    dt = _dtype_code(q)
    B, H, _, Nq, Nk, d = _check_bwd(q, k, v, o, lse, do, dq, dk, dv, workspace, "bhsd", contiguous=True)
    nbytes = workspace.numel() * workspace.element_size()
    with torch.cuda.device(q.device):
        _check(load_library().fa_bwd(
            _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv),
            B, H, Nq, Nk, d, float(scale), int(bool(causal)), dt, _ptr(workspace), nbytes,
            _stream(q, stream)))


def fa_bwd_noalloc(q, k, v, o, lse, do, dq, dk, dv, scale, causal, stream=None):
    """C ``fa_bwd_noalloc``: ``fa_bwd`` with the library's own scratch as the
    workspace (no allocation; calls that overlap on one GPU race)."""
    dt = _dtype_code(q)
    B, H, _, Nq, Nk, d = _check_fwd(q, k, v, o, lse, "bhsd", contiguous=True, device=False)
    _want_dtype(q.dtype, do=do, dq=dq, dk=dk, dv=dv)
    _want_shape("dout", do, q.shape)
    _want_shape("dq", dq, q.shape)
    _want_shape("dk", dk, k.shape)
    _want_shape("dv", dv, k.shape)
    _want_contiguous(do=do, dq=dq, dk=dk, dv=dv)
    _want_device(q, k=k, v=v, o=o, lse=lse, do=do, dq=dq, dk=dk, dv=dv)
    with torch.cuda.device(q.device):
        _check(load_library().fa_bwd_noalloc(
            _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv),
            B, H, Nq, Nk, d, float(scale), int(bool(causal)), dt, _stream(q, stream)))


def fa_bwd_strided(q, k, v, o, lse, do, dq, dk, dv, scale, causal, workspace, layout="bshd", stream=None):
    """C ``fa_bwd_strided``: every d-major tensor's own strides, read in ``layout``."""
    dt = _dtype_code(q)
    B, H, _, Nq, Nk, d = _check_bwd(q, k, v, o, lse, do, dq, dk, dv, workspace, layout)
    nbytes = workspace.numel() * workspace.element_size()
    st = [_strides(t, layout) for t in (q, k, v, o, do, dq, dk, dv)]
    with torch.cuda.device(q.device):
        _check(load_library().fa_bwd_strided(
            _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv),
            B, H, Nq, Nk, d, float(scale), int(bool(causal)), dt, *st, _ptr(workspace), nbytes,
            _stream(q, stream)))


def fa_bwd_stages(q, k, v, o, lse, do, dq, dk, dv, scale, causal, workspace, stages, layout="bhsd", stream=None):
    """C ``fa_bwd_stages``: run the selected backward stages (OR of FA_BWD_*)."""
    dt = _dtype_code(q)
    B, H, _, Nq, Nk, d = _check_bwd(q, k, v, o, lse, do, dq, dk, dv, workspace, layout)
    nbytes = workspace.numel() * workspace.element_size()
    st = [_strides(t, layout) for t in (q, k, v, o, do, dq, dk, dv)]
    with torch.cuda.device(q.device):
        _check(load_library().fa_bwd_stages(
            _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv),
            B, H, Nq, Nk, d, float(scale), int(bool(causal)), dt, *st, _ptr(workspace), nbytes, int(stages),
            _stream(q, stream)))


def _window(window):
    left, right = (-1, -1) if window is None else window
    return int(left), int(right)


def _dropout(dropout):
    p, seed, offset = (0.0, 0, 0) if dropout is None else dropout
    return float(p), int(seed), int(offset)


def fa_fwd_ex(q, k, v, o, lse, scale, causal, window=(-1, -1), layout="bhsd", stream=None, dropout=None):
    """C ``fa_fwd_ex``: k, v may have fewer heads than q (it must divide q's);
    ``window`` = (left, right), a negative side unbounded; ``dropout`` =
    (p, seed, offset) or None."""
    dt = _dtype_code(q)
    B, H, Hkv, Nq, Nk, d = _check_fwd(q, k, v, o, lse, layout, same_heads=False)
    wl, wr = _window(window)
    dp, seed, off = _dropout(dropout)
    with torch.cuda.device(q.device):
        _check(load_library().fa_fwd_ex(
            _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Hkv, Nq, Nk, d, float(scale), int(bool(causal)),
            wl, wr, dp, seed, off, dt, _strides(q, layout), _strides(k, layout), _strides(v, layout),
            _strides(o, layout), _stream(q, stream)))


def fa_fwd_splitk_workspace_bytes(B, H, Nq, Nk, d, causal, window=(-1, -1)):
    """C ``fa_fwd_splitk_workspace_bytes`` (0: the sizes need no workspace)."""
    wl, wr = _window(window)
    return int(load_library().fa_fwd_splitk_workspace_bytes(B, H, Nq, Nk, d, int(bool(causal)), wl, wr))


def fa_fwd_splitk(q, k, v, o, lse, scale, causal, workspace, window=(-1, -1), layout="bhsd", stream=None,
                  dropout=None):
    """C ``fa_fwd_splitk``: ``fa_fwd_ex`` with the keys of heavy query blocks
    split over workgroups; ``workspace`` is a device tensor of at least
    ``fa_fwd_splitk_workspace_bytes`` bytes, or None when that is 0."""
    dt = _dtype_code(q)
    B, H, Hkv, Nq, Nk, d = _check_fwd(q, k, v, o, lse, layout, same_heads=False, device=False)
    if workspace is not None and not workspace.is_contiguous():
        _bad("workspace must be contiguous")
    _want_device(q, k=k, v=v, o=o, lse=lse, **({} if workspace is None else {"workspace": workspace}))
    wl, wr = _window(window)
    dp, seed, off = _dropout(dropout)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    with torch.cuda.device(q.device):
        _check(load_library().fa_fwd_splitk(
            _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Hkv, Nq, Nk, d, float(scale), int(bool(causal)),
            wl, wr, dp, seed, off, dt, _strides(q, layout), _strides(k, layout), _strides(v, layout),
            _strides(o, layout), _ptr(workspace), nbytes, _stream(q, stream)))


def fa_bwd_ex(q, k, v, o, lse, do, dq, dk, dv, scale, causal, workspace, window=(-1, -1), stages=FA_BWD_ALL,
              layout="bhsd", stream=None, dropout=None):
    """C ``fa_bwd_ex``: the backward of ``fa_fwd_ex`` (dk, dv shaped like k,
    v; the same ``window`` and ``dropout``)."""
    dt = _dtype_code(q)
    B, H, Hkv, Nq, Nk, d = _check_bwd(q, k, v, o, lse, do, dq, dk, dv, workspace, layout, same_heads=False)
    wl, wr = _window(window)
    dp, seed, off = _dropout(dropout)
    nbytes = workspace.numel() * workspace.element_size()
    st = [_strides(t, layout) for t in (q, k, v, o, do, dq, dk, dv)]
    with torch.cuda.device(q.device):
        _check(load_library().fa_bwd_ex(
            _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv),
            B, H, Hkv, Nq, Nk, d, float(scale), int(bool(causal)), wl, wr, dp, seed, off, dt, *st,
            _ptr(workspace), nbytes, int(stages), _stream(q, stream)))


def _fp8_input(*ts):
    for t in ts:
        if t.dtype not in (torch.float8_e4m3fn, torch.uint8):
            raise FaError(FA_ERR_UNSUPPORTED, "fp8 inputs must be float8_e4m3fn (or its bytes as uint8), got %s"
                          % t.dtype)


def fa_fwd_fp8(q, k, v, o, lse, scale, causal, window=(-1, -1), descale=(1.0, 1.0, 1.0), layout="bhsd",
               stream=None):
    """C ``fa_fwd_fp8``: q, k, v float8_e4m3fn (k, v may have fewer heads),
    o bf16 shaped like q, lse fp32 [B,H,Nq]; ``descale`` = (q, k, v)
    per-tensor factors."""
    _fp8_input(q, k, v)
    if o.dtype != torch.bfloat16:
        raise FaError(FA_ERR_UNSUPPORTED, "fp8 forward writes a bfloat16 o, got %s" % o.dtype)
    B, H, Hkv, Nq, Nk, d = _check_fwd(q, k, v, o, lse, layout, same_heads=False, out_dtype=torch.bfloat16)
    wl, wr = _window(window)
    qd, kd, vd = (float(x) for x in descale)
    with torch.cuda.device(q.device):
        _check(load_library().fa_fwd_fp8(
            _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Hkv, Nq, Nk, d, float(scale), int(bool(causal)),
            wl, wr, qd, kd, vd, _strides(q, layout), _strides(k, layout), _strides(v, layout),
            _strides(o, layout), _stream(q, stream)))


def attention_fwd_fp8(q, k, v, causal=False, scale=None, layout="bhsd", stream=None, window=None,
                      descale=(1.0, 1.0, 1.0)):
    """Forward on float8_e4m3fn q, k, v; allocates o (bf16, q's shape) and
    lse (fp32 [B,H,Nq]); returns (o, lse).  No backward exists for fp8."""
    _fp8_input(q, k, v)
    _on_device(q, k, v)
    B, H, Nq, d = _dims(q, layout)
    s = _default_scale(d, scale)
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    fa_fwd_fp8(q, k, v, o, lse, s, causal, window, descale, layout, stream)
    return o, lse


def attention_fwd(q, k, v, causal=False, scale=None, layout="bhsd", stream=None, window=None, dropout=None,
                  splitk=True):
    """O = softmax(scale Q K^T) V (top-left causal mask if ``causal``).

    Allocates o (like q) and lse (fp32 [B,H,Nq]); returns (o, lse).  ``scale``
    defaults to 1/sqrt(d).  k and v may carry fewer heads than q (dividing
    them); ``window`` = (left, right) restricts query i to keys
    i - left .. i + right (negative: unbounded); ``dropout`` = (p, seed,
    offset) drops attention weights (see ``include/fa.h``).  ``splitk``:
    for grids too small to fill the chip, allocate the workspace of
    ``fa_fwd_splitk`` and split heavy query blocks' keys over workgroups
    (False: the C ``fa_fwd`` family, without a workspace).
    """
    _dtype_code(q)
    _on_device(q, k, v)
    B, H, Nq, d = _dims(q, layout)
    s = _default_scale(d, scale)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if splitk:
        Nk = _dims(k, layout)[2]
        nbytes = fa_fwd_splitk_workspace_bytes(B, H, Nq, Nk, d, causal, _window(window))
        if nbytes > 0:
            ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
            fa_fwd_splitk(q, k, v, o, lse, s, causal, ws, _window(window), layout, stream, dropout)
            return o, lse
    if _dims(k, layout)[1] != H or window is not None or dropout is not None:
        fa_fwd_ex(q, k, v, o, lse, s, causal, window, layout, stream, dropout)
    elif layout == "bhsd" and q.is_contiguous() and k.is_contiguous() and v.is_contiguous():
        fa_fwd(q, k, v, o, lse, s, causal, stream)
    else:
        fa_fwd_strided(q, k, v, o, lse, s, causal, layout, stream)
    return o, lse


def attention_bwd(q, k, v, o, lse, do, causal=False, scale=None, layout="bhsd", stream=None, window=None,
                  dropout=None):
    """Gradients (dq, dk, dv) of sum(O * dO), recomputing P from ``lse``
    (fewer K/V heads, ``window`` and ``dropout`` as in ``attention_fwd``)."""
    _on_device(q, k, v, o, lse, do)
    B, H, Nq, d = _dims(q, layout)
    Hkv, Nk = _dims(k, layout)[1:3]
    s = _default_scale(d, scale)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    # the workspace that lets the dK/dV stage split its key blocks' steps
    # (fewer K/V heads, or a grid too small for the chip)
    nbytes = fa_bwd_ex_workspace_bytes(B, H, Hkv, Nq, Nk, d, _dtype_code(q))
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=q.device)
    contiguous = all(t.is_contiguous() for t in (q, k, v, o, do))
    if Hkv != H or window is not None or dropout is not None:
        fa_bwd_ex(q, k, v, o, lse, do, dq, dk, dv, s, causal, ws, window, FA_BWD_ALL, layout, stream, dropout)
    elif layout == "bhsd" and contiguous:
        fa_bwd(q, k, v, o, lse, do, dq, dk, dv, s, causal, ws, stream)
    else:
        fa_bwd_strided(q, k, v, o, lse, do, dq, dk, dv, s, causal, ws, layout, stream)
    return dq, dk, dv
