"""Thin Python binding of libw4a16.so, the gfx950 W4A16 / ternary small-M
linear-layer library (C ABI declared in include/w4a16.h).

Every function here has the same name and argument order as its C entry
point and only marshals arguments: tensors (anything with ``data_ptr()``) or
raw integer device pointers go in as pointers, the stream defaults to torch's
current HIP stream, and a negative status raises :class:`W4A16Error`.  All
computation happens in the library's HIP kernels; if the library has not been
built, importing this package fails loudly (build it with
``python -m bit_weight_only_03_amd.build``).
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libw4a16.so")

W4A16_F16, W4A16_BF16, W4A16_F32 = 0, 1, 2
_DTYPES = {"f16": W4A16_F16, "bf16": W4A16_BF16, "f32": W4A16_F32}


class W4A16Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        detail = f", HIP: {w4a16_last_error()}" if status == -7 else ""
        super().__init__(f"{fn} failed: status {status} ({w4a16_status_string(status)}{detail})")


_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.c_size_t
_PSZ = ctypes.POINTER(ctypes.c_size_t)

_SIGS = {
    "w4a16_packed_sizes": [_I, _I, _I, _PSZ, _PSZ, _PSZ],
    "w4a16_pack": [_P, _P, _P, _P, _P, _P, _I, _I, _I, _P],
    "w4a16_unpack": [_P, _P, _P, _P, _P, _P, _I, _I, _I, _P],
    "w4a16_workspace_bytes": [_I, _I, _I, _I, _PSZ],
    "w4a16_gemv": [_P, _I, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _SZ, _P],
    "w4a16_gemv_noalloc": [_P, _I, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P],
    "w4a16_gemv_add": [_P, _I, _P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _P, _SZ, _P],
    "w16a16_workspace_bytes": [_I, _I, _I, _PSZ],
    "w16a16_gemv": [_P, _P, _I, _P, _I, _I, _I, _I, _P, _SZ, _P],
    "w4a16_dequant": [_P, _P, _P, _P, _I, _I, _I, _P],
    "mxfp4_packed_sizes": [_I, _I, _PSZ, _PSZ],
    "mxfp4_pack": [_P, _P, _P, _P, _I, _I, _P],
    "mxfp4_unpack": [_P, _P, _P, _P, _I, _I, _P],
    "mxfp4_workspace_bytes": [_I, _I, _I, _PSZ],
    "mxfp4_gemv": [_P, _I, _P, _P, _P, _I, _I, _I, _I, _P, _SZ, _P],
    "mxfp4_dequant": [_P, _P, _P, _I, _I, _P],
    "w2t_packed_sizes": [_I, _I, _I, _PSZ, _PSZ],
    "w2t_pack": [_P, _P, _P, _P, _I, _I, _I, _P],
    "w2t_unpack": [_P, _P, _P, _P, _I, _I, _I, _P],
    "w2t_workspace_bytes": [_I, _I, _I, _I, _PSZ],
    "w2t_gemv": [_P, _I, _P, _P, _P, _I, _I, _I, _I, _I, _P, _SZ, _P],
    "w2t_dequant": [_P, _P, _P, _I, _I, _I, _P],
    "w4a16_bw_probe": [_P, _SZ, _P, _P],
    "w4a16_bw_probe_sink_floats": [],
    "w4a16_status_string": [_I],
    "w4a16_last_variant": [],
    "w4a16_plan_variant": [_I, _I, _I, _I, _I, ctypes.c_char_p, _SZ],
    "w4a16_last_error": [],
}
_STR_RESULT = ("w4a16_status_string", "w4a16_last_variant", "w4a16_last_error")

_lib_handle = None


def _lib_get():
    """Load libw4a16.so on first use; there is no other implementation, so a
    missing library is an error."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m bit_weight_only_03_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            f = getattr(lib, name)
            f.argtypes = args
            f.restype = ctypes.c_char_p if name in _STR_RESULT else _I
        _lib_handle = lib
    return _lib_handle


class _LazyLib:
    def __getattr__(self, name):
        return getattr(_lib_get(), name)


_lib = _LazyLib()

EXPORTED = tuple(_SIGS)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dt(d):
    return _DTYPES[d] if isinstance(d, str) else int(d)


def _check(fn: str, rc: int):
    if rc != 0:
        raise W4A16Error(fn, rc)


def w4a16_status_string(status: int) -> str:
    return _lib.w4a16_status_string(status).decode()


def w4a16_last_variant() -> str:
    return _lib.w4a16_last_variant().decode()


def w4a16_plan_variant(M: int, N: int, K: int, group: int, x_dtype="f16") -> str:
    buf = ctypes.create_string_buffer(256)
    _check("w4a16_plan_variant", _lib.w4a16_plan_variant(M, N, K, group, _dt(x_dtype), buf,
                                                         len(buf)))
    return buf.value.decode()


def w4a16_last_error() -> str:
    return _lib.w4a16_last_error().decode()


def w4a16_packed_sizes(N: int, K: int, group: int):
    q, s, z = _SZ(), _SZ(), _SZ()
    _check("w4a16_packed_sizes", _lib.w4a16_packed_sizes(N, K, group, ctypes.byref(q),
                                                        ctypes.byref(s), ctypes.byref(z)))
    return q.value, s.value, z.value


def w4a16_pack(qweight_canon, scales_canon, zeros_canon, qweight, scales, zeros, N, K, group,
               stream=None):
    _check("w4a16_pack", _lib.w4a16_pack(_ptr(qweight_canon), _ptr(scales_canon), _ptr(zeros_canon),
                                         _ptr(qweight), _ptr(scales), _ptr(zeros), N, K, group,
                                         _stream(stream)))


def w4a16_unpack(qweight, scales, zeros, qweight_canon, scales_canon, zeros_canon, N, K, group,
                 stream=None):
    _check("w4a16_unpack", _lib.w4a16_unpack(_ptr(qweight), _ptr(scales), _ptr(zeros),
                                             _ptr(qweight_canon), _ptr(scales_canon),
                                             _ptr(zeros_canon), N, K, group, _stream(stream)))


def w4a16_workspace_bytes(M: int, N: int, K: int, group: int) -> int:
    b = _SZ()
    _check("w4a16_workspace_bytes", _lib.w4a16_workspace_bytes(M, N, K, group, ctypes.byref(b)))
    return b.value


def w4a16_gemv(x, x_dtype, qweight, scales, zeros, y, y_dtype, M, N, K, group, workspace=None,
               workspace_bytes=0, stream=None):
    _check("w4a16_gemv", _lib.w4a16_gemv(_ptr(x), _dt(x_dtype), _ptr(qweight), _ptr(scales),
                                         _ptr(zeros), _ptr(y), _dt(y_dtype), M, N, K, group,
                                         _ptr(workspace), workspace_bytes, _stream(stream)))


def w4a16_gemv_noalloc(x, x_dtype, qweight, scales, zeros, y, y_dtype, M, N, K, group,
                       stream=None):
    _check("w4a16_gemv_noalloc", _lib.w4a16_gemv_noalloc(
        _ptr(x), _dt(x_dtype), _ptr(qweight), _ptr(scales), _ptr(zeros), _ptr(y), _dt(y_dtype),
        M, N, K, group, _stream(stream)))


W4A16_NOALLOC_SCRATCH_BYTES = 16 << 20
# Arrival counters at the start of every workspace: zero before its first use.
W4A16_WORKSPACE_HEAD_BYTES = 64 << 10


def w4a16_gemv_add(x, x_dtype, qweight, scales, zeros, residual, residual_dtype, y, y_dtype, M, N, K,
                   group, workspace=None, workspace_bytes=0, stream=None):
    _check("w4a16_gemv_add", _lib.w4a16_gemv_add(
        _ptr(x), _dt(x_dtype), _ptr(qweight), _ptr(scales), _ptr(zeros), _ptr(residual),
        _dt(residual_dtype), _ptr(y), _dt(y_dtype), M, N, K, group, _ptr(workspace),
        workspace_bytes, _stream(stream)))


def w16a16_workspace_bytes(M: int, N: int, K: int) -> int:
    b = ctypes.c_size_t(0)
    _check("w16a16_workspace_bytes", _lib.w16a16_workspace_bytes(M, N, K, ctypes.byref(b)))
    return b.value


def w16a16_gemv(x, w, dtype, y, y_dtype, M, N, K, workspace=None, workspace_bytes=0, stream=None):
    _check("w16a16_gemv", _lib.w16a16_gemv(_ptr(x), _ptr(w), _dt(dtype), _ptr(y), _dt(y_dtype),
                                           M, N, K, _ptr(workspace), workspace_bytes,
                                           _stream(stream)))


def w4a16_dequant(qweight, scales, zeros, w, N, K, group, stream=None):
    _check("w4a16_dequant", _lib.w4a16_dequant(_ptr(qweight), _ptr(scales), _ptr(zeros), _ptr(w),
                                               N, K, group, _stream(stream)))


def mxfp4_packed_sizes(N: int, K: int):
    q, s = _SZ(), _SZ()
    _check("mxfp4_packed_sizes", _lib.mxfp4_packed_sizes(N, K, ctypes.byref(q), ctypes.byref(s)))
    return q.value, s.value


def mxfp4_pack(qweight_canon, scales_canon, qweight, scales, N, K, stream=None):
    _check("mxfp4_pack", _lib.mxfp4_pack(_ptr(qweight_canon), _ptr(scales_canon), _ptr(qweight),
                                         _ptr(scales), N, K, _stream(stream)))


def mxfp4_unpack(qweight, scales, qweight_canon, scales_canon, N, K, stream=None):
    _check("mxfp4_unpack", _lib.mxfp4_unpack(_ptr(qweight), _ptr(scales), _ptr(qweight_canon),
                                             _ptr(scales_canon), N, K, _stream(stream)))


def mxfp4_workspace_bytes(M: int, N: int, K: int) -> int:
    b = _SZ()
    _check("mxfp4_workspace_bytes", _lib.mxfp4_workspace_bytes(M, N, K, ctypes.byref(b)))
    return b.value


def mxfp4_gemv(x, x_dtype, qweight, scales, y, y_dtype, M, N, K, workspace=None, workspace_bytes=0,
               stream=None):
    _check("mxfp4_gemv", _lib.mxfp4_gemv(_ptr(x), _dt(x_dtype), _ptr(qweight), _ptr(scales), _ptr(y),
                                         _dt(y_dtype), M, N, K, _ptr(workspace), workspace_bytes,
                                         _stream(stream)))


def mxfp4_dequant(qweight, scales, w, N, K, stream=None):
    _check("mxfp4_dequant", _lib.mxfp4_dequant(_ptr(qweight), _ptr(scales), _ptr(w), N, K,
                                               _stream(stream)))


def w2t_packed_sizes(N: int, K: int, group: int):
    q, s = _SZ(), _SZ()
    _check("w2t_packed_sizes", _lib.w2t_packed_sizes(N, K, group, ctypes.byref(q), ctypes.byref(s)))
    return q.value, s.value


def w2t_pack(codes_canon, scales_canon, qweight, scales, N, K, group, stream=None):
    _check("w2t_pack", _lib.w2t_pack(_ptr(codes_canon), _ptr(scales_canon), _ptr(qweight),
                                     _ptr(scales), N, K, group, _stream(stream)))


def w2t_unpack(qweight, scales, codes_canon, scales_canon, N, K, group, stream=None):
    _check("w2t_unpack", _lib.w2t_unpack(_ptr(qweight), _ptr(scales), _ptr(codes_canon),
                                         _ptr(scales_canon), N, K, group, _stream(stream)))


def w2t_workspace_bytes(M: int, N: int, K: int, group: int) -> int:
    b = _SZ()
    _check("w2t_workspace_bytes", _lib.w2t_workspace_bytes(M, N, K, group, ctypes.byref(b)))
    return b.value


def w2t_gemv(x, x_dtype, qweight, scales, y, y_dtype, M, N, K, group, workspace=None,
             workspace_bytes=0, stream=None):
    _check("w2t_gemv", _lib.w2t_gemv(_ptr(x), _dt(x_dtype), _ptr(qweight), _ptr(scales), _ptr(y),
                                     _dt(y_dtype), M, N, K, group, _ptr(workspace), workspace_bytes,
                                     _stream(stream)))


def w2t_dequant(qweight, scales, w, N, K, group, stream=None):
    _check("w2t_dequant", _lib.w2t_dequant(_ptr(qweight), _ptr(scales), _ptr(w), N, K, group,
                                           _stream(stream)))


def w4a16_bw_probe_sink_floats() -> int:
    return _lib.w4a16_bw_probe_sink_floats()


def w4a16_bw_probe(buf, nbytes: int, sink, stream=None):
    _check("w4a16_bw_probe", _lib.w4a16_bw_probe(_ptr(buf), nbytes, _ptr(sink), _stream(stream)))
