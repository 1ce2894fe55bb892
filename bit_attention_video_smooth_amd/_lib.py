"""ctypes binding of libvcattn.so (C ABI in include/vc_attention.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of the library.  PyTorch supplies device memory and the stream.
Functions keep the C names; a negative return code raises VCError with the
library's own message.  There is no fallback: without the built library
every call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libvcattn.so")

VC_OK = 0
VC_ERR_INVALID = -1
VC_ERR_UNSUPPORTED = -2
VC_ERR_WORKSPACE = -3
VC_ERR_HIP = -4

EXPORTS = ["vc_version", "vc_last_error", "vc_prepared_sizes", "vsmooth_workspace_bytes",
           "vsmooth_prepare", "vsmooth_prepare_warm", "vsmooth_prepare_noalloc", "vc_attention_fwd",
           "vc_attention_fwd_dump",
           "vc_attention_fwd_bf16", "vc_sage_prepared_sizes", "vc_sage_workspace_bytes",
           "vc_sage_prepare", "vc_sage_attention_fwd", "vc_sage_attention_fwd_dump",
           "vc_debug_expcast", "vc_debug_e4m3_encode", "vc_debug_mfma_fp8", "vc_debug_mfma_rate"]

VC_SAGE_QK_INT8 = 0
VC_SAGE_QK_FP8 = 1


class VCError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("vc error %d: %s" % (code, msg))
        self.code = code


class vc_shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("L", ctypes.c_int32),
                ("d", ctypes.c_int32)]


class vsmooth_params(ctypes.Structure):
    _fields_ = [("block", ctypes.c_int32), ("kmeans_k", ctypes.c_int32),
                ("kmeans_iters", ctypes.c_int32), ("smooth_k", ctypes.c_int32),
                ("v_scale_mode", ctypes.c_int32), ("v_format", ctypes.c_int32),
                ("seed", ctypes.c_uint64)]


class vc_prepared(ctypes.Structure):
    _fields_ = [("q8", ctypes.c_void_p), ("k8", ctypes.c_void_p), ("v8", ctypes.c_void_p),
                ("q_scale", ctypes.c_void_p), ("k_scale", ctypes.c_void_p),
                ("v_scale", ctypes.c_void_p), ("v_mean", ctypes.c_void_p),
                ("perm", ctypes.c_void_p), ("kmeans_obj", ctypes.c_void_p)]


class vc_attn_params(ctypes.Structure):
    _fields_ = [("z_off", ctypes.c_int32), ("out_dtype", ctypes.c_int32), ("skip_lambda", ctypes.c_float),
                ("prob_cast", ctypes.c_int32), ("v_format", ctypes.c_int32)]


class vc_sage_params(ctypes.Structure):
    _fields_ = [("qk_dtype", ctypes.c_int32), ("v_dtype", ctypes.c_int32), ("q_block_size", ctypes.c_int32),
                ("k_block_size", ctypes.c_int32), ("v_block_size", ctypes.c_int32), ("smooth_k", ctypes.c_int32)]


class vc_sage_prepared(ctypes.Structure):
    _fields_ = [("q8", ctypes.c_void_p), ("k8", ctypes.c_void_p), ("v8", ctypes.c_void_p),
                ("q_scale", ctypes.c_void_p), ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p)]


_lock = threading.Lock()
_lib = None


def load():
    """Load libvcattn.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libvcattn.so is not built (run python -m "
                               "bit_attention_video_smooth_amd.build); no fallback exists")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        S, VP, PR, AP = (ctypes.POINTER(vc_shape), ctypes.POINTER(vsmooth_params),
                         ctypes.POINTER(vc_prepared), ctypes.POINTER(vc_attn_params))
        L.vc_version.restype = ctypes.c_int
        L.vc_last_error.restype = ctypes.c_char_p
        L.vc_prepared_sizes.argtypes = [S, ctypes.POINTER(sz)]
        L.vsmooth_workspace_bytes.argtypes = [S, VP, ctypes.POINTER(sz)]
        L.vsmooth_prepare.argtypes = [S, VP, P, P, P, P, PR, P, sz, P]
        L.vsmooth_prepare_warm.argtypes = [S, VP, P, P, P, P, P, PR, P, sz, P]
        L.vsmooth_prepare_noalloc.argtypes = [S, VP, P, P, P, P, PR, P]
        L.vc_attention_fwd.argtypes = [S, AP, PR, P, P]
        L.vc_attention_fwd_dump.argtypes = [S, AP, PR, P, i32, i32, P, P, P]
        L.vc_attention_fwd_bf16.argtypes = [S, P, P, P, P, i32, P]
        SP, SR = ctypes.POINTER(vc_sage_params), ctypes.POINTER(vc_sage_prepared)
        L.vc_sage_prepared_sizes.argtypes = [S, ctypes.POINTER(sz)]
        L.vc_sage_workspace_bytes.argtypes = [S, ctypes.POINTER(sz)]
        L.vc_sage_prepare.argtypes = [S, SP, P, P, P, SR, P, sz, P]
        L.vc_sage_attention_fwd.argtypes = [S, SP, AP, SR, P, P]
        L.vc_sage_attention_fwd_dump.argtypes = [S, SP, AP, SR, P, i32, i32, P, P, P]
        L.vc_debug_expcast.argtypes = [P, P, P, i64, P, P]
        L.vc_debug_e4m3_encode.argtypes = [P, i64, P, P]
        L.vc_debug_mfma_fp8.argtypes = [P, P, P, i32, P]
        L.vc_debug_mfma_rate.argtypes = [i32, i32, P, P]
        for n in EXPORTS:
            getattr(L, n).restype = ctypes.c_int if n != "vc_last_error" else ctypes.c_char_p
        _lib = L
        return L


def _check(rc: int):
    if rc != VC_OK:
        raise VCError(rc, load().vc_last_error().decode())


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


def shape_of(B, H, L, d) -> vc_shape:
    return vc_shape(B, H, L, d)


def make_params(kmeans_k=0, kmeans_iters=8, seed=0, smooth_k=1, v_scale_mode=0, v_format=0) -> vsmooth_params:
    return vsmooth_params(128, kmeans_k, kmeans_iters, smooth_k, v_scale_mode, v_format, seed & (2**64 - 1))


# ---------------------------------------------------------------- C names --

def vc_version() -> int:
    return load().vc_version()


def vc_last_error() -> str:
    return load().vc_last_error().decode()


def vc_prepared_sizes(shape: vc_shape):
    arr = (ctypes.c_size_t * 9)()
    _check(load().vc_prepared_sizes(ctypes.byref(shape), arr))
    return list(arr)


def vsmooth_workspace_bytes(shape: vc_shape, params: vsmooth_params) -> int:
    n = ctypes.c_size_t()
    _check(load().vsmooth_workspace_bytes(ctypes.byref(shape), ctypes.byref(params), ctypes.byref(n)))
    return n.value


def vsmooth_prepare(shape, params, q, k, v, perm_in, out: vc_prepared, ws, ws_bytes, stream=None):
    _check(load().vsmooth_prepare(ctypes.byref(shape), ctypes.byref(params), _ptr(q), _ptr(k), _ptr(v),
                                  _ptr(perm_in), ctypes.byref(out), _ptr(ws), ws_bytes, _stream(stream)))


def vsmooth_prepare_noalloc(shape, params, q, k, v, perm_in, out: vc_prepared, stream=None):
    _check(load().vsmooth_prepare_noalloc(ctypes.byref(shape), ctypes.byref(params), _ptr(q), _ptr(k), _ptr(v),
                                          _ptr(perm_in), ctypes.byref(out), _stream(stream)))


def vsmooth_prepare_warm(shape, params, q, k, v, centroids_in, centroids_out, out: vc_prepared, ws, ws_bytes,
                         stream=None):
    _check(load().vsmooth_prepare_warm(ctypes.byref(shape), ctypes.byref(params), _ptr(q), _ptr(k), _ptr(v),
                                       _ptr(centroids_in), _ptr(centroids_out), ctypes.byref(out), _ptr(ws),
                                       ws_bytes, _stream(stream)))


def vc_attention_fwd(shape, params: vc_attn_params, prep: vc_prepared, out, stream=None):
    _check(load().vc_attention_fwd(ctypes.byref(shape), ctypes.byref(params), ctypes.byref(prep),
                                   _ptr(out), _stream(stream)))


def vc_attention_fwd_dump(shape, params, prep, out, bh, q_tile, s_dump, p_dump, stream=None):
    _check(load().vc_attention_fwd_dump(ctypes.byref(shape), ctypes.byref(params), ctypes.byref(prep),
                                        _ptr(out), bh, q_tile, _ptr(s_dump), _ptr(p_dump),
                                        _stream(stream)))


def vc_attention_fwd_bf16(shape, q, k, v, out, out_dtype=0, stream=None):
    _check(load().vc_attention_fwd_bf16(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                        out_dtype, _stream(stream)))


def make_sage_params(qk_dtype=VC_SAGE_QK_INT8, smooth_k=1) -> vc_sage_params:
    """The recipe's fixed fields: v_dtype FP8 E4M3, q/k/v block sizes 1/16/1."""
    return vc_sage_params(qk_dtype, 0, 1, 16, 1, smooth_k)


def vc_sage_prepared_sizes(shape: vc_shape):
    arr = (ctypes.c_size_t * 6)()
    _check(load().vc_sage_prepared_sizes(ctypes.byref(shape), arr))
    return list(arr)


def vc_sage_workspace_bytes(shape: vc_shape) -> int:
    n = ctypes.c_size_t()
    _check(load().vc_sage_workspace_bytes(ctypes.byref(shape), ctypes.byref(n)))
    return n.value


def vc_sage_prepare(shape, params: vc_sage_params, q, k, v, out: vc_sage_prepared, ws, ws_bytes, stream=None):
    _check(load().vc_sage_prepare(ctypes.byref(shape), ctypes.byref(params), _ptr(q), _ptr(k), _ptr(v),
                                  ctypes.byref(out), _ptr(ws), ws_bytes, _stream(stream)))


def vc_sage_attention_fwd(shape, sage: vc_sage_params, params: vc_attn_params, prep: vc_sage_prepared, out,
                          stream=None):
    _check(load().vc_sage_attention_fwd(ctypes.byref(shape), ctypes.byref(sage), ctypes.byref(params),
                                        ctypes.byref(prep), _ptr(out), _stream(stream)))


def vc_sage_attention_fwd_dump(shape, sage, params, prep, out, bh, q_tile, s_dump, p_dump, stream=None):
    _check(load().vc_sage_attention_fwd_dump(ctypes.byref(shape), ctypes.byref(sage), ctypes.byref(params),
                                             ctypes.byref(prep), _ptr(out), bh, q_tile, _ptr(s_dump),
                                             _ptr(p_dump), _stream(stream)))


def vc_debug_expcast(S, c8, krow, n, out, stream=None):
    _check(load().vc_debug_expcast(_ptr(S), _ptr(c8), _ptr(krow), n, _ptr(out), _stream(stream)))


def vc_debug_e4m3_encode(x, n, out, stream=None):
    _check(load().vc_debug_e4m3_encode(_ptr(x), n, _ptr(out), _stream(stream)))


def vc_debug_mfma_fp8(a, b, c, n_tiles, stream=None):
    _check(load().vc_debug_mfma_fp8(_ptr(a), _ptr(b), _ptr(c), n_tiles, _stream(stream)))


def vc_debug_mfma_rate(blocks, iters, out, stream=None):
    _check(load().vc_debug_mfma_rate(blocks, iters, _ptr(out), _stream(stream)))
