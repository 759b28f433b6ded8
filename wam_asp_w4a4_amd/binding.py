"""ctypes binding of libasp's C entry points (argument marshalling only).

Every function has the name and argument order of its C counterpart in
``include/asp.h``.  Array arguments may be torch tensors (device or host,
contiguous) or NumPy arrays (host); ``None`` passes NULL.  The stream argument
defaults to torch's current stream on the tensors' device.  A non-zero status
raises :class:`ASPError` with the library's own message.

The library is loaded on first use; a missing build raises at once -- there is
no fallback implementation.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

ABI_VERSION = 8
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libasp.so")

ASP_F32 = 0
ASP_BF16 = 1
DTYPES = {"f32": ASP_F32, "bf16": ASP_BF16}

# name -> (restype, argtypes); mirrors include/asp.h
_i32, _i64, _sz, _p = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p
_psz = ctypes.POINTER(ctypes.c_size_t)
SIGNATURES = {
    "asp_abi_version": (_i32, []),
    "asp_source_digest": (ctypes.c_char_p, []),
    "asp_status_string": (ctypes.c_char_p, [_i32]),
    "asp_last_error": (ctypes.c_char_p, []),
    "asp_gemm_kernel_name": (ctypes.c_char_p, [_i64, _i64, _i64]),
    "asp_packed_sizes": (_i32, [_i64, _i64, _i32, _psz, _psz, _psz]),
    "asp_pack_weight": (_i32, [_i64, _i64, _i32, _p, _p, _p, _p, _p, _p, _p, _i32]),
    "asp_pack_weight_shared": (_i32, [_i64, _i64, _i32, _p, _p, _p, _p, _p, _p, _p, _i32]),
    "asp_quantize_nvfp4_host": (_i32, [_p, _i64, _i64, _p, _p]),
    "asp_prep_pack_bytes": (_i32, [_i64, _i32, _psz]),
    "asp_pack_prep": (_i32, [_i64, _i32, _p, _p, _p]),
    "asp_quantize_nvfp4": (_i32, [_p, _i64, _i64, _p, _p, _p]),
    "asp_dequantize_nvfp4": (_i32, [_p, _p, _i64, _i64, _p, _p]),
    "asp_act_prep_workspace_bytes": (_i32, [_i64, _i64, _i32, _psz]),
    "asp_act_prep": (_i32, [_p, _i32, _i64, _i64, _i32, _p, _p, _p, _p, _p, _p, _sz, _p]),
    "asp_act_prep_u": (_i32, [_p, _i32, _i64, _i64, _i32, _p, _p, _sz, _p]),
    "asp_act_prep_q": (_i32, [_p, _i32, _i64, _i64, _i32, _p, _p, _p, _p, _p, _p, _sz, _p]),
    "asp_gemm_lowrank": (_i32, [_p, _p, _p, _i64, _i64, _i64, _i32, _p, _p, _p, _p, _p, _i32, _p]),
    "asp_workspace_bytes": (_i32, [_i64, _i64, _i64, _i32, _psz]),
    "asp_forward": (_i32, [_p, _i32, _i64, _i64, _i64, _i32, _p, _p, _p, _p, _p, _p, _i32,
                           _p, _sz, _p]),
    "asp_smoothing_search_workspace_bytes": (_i32, [_i64, _i64, _i64, _i32, _i32, _psz]),
    "asp_smoothing_search": (_i32, [_p, _i32, _i64, _i64, _p, _p, _i64, _p, _i32, _p, _p, _i32,
                                    _p, _p, _p, _sz, _p]),
    "asp_top_eigenspace_workspace_bytes": (_i32, [_i64, _i32, _i32, _psz]),
    "asp_top_eigenspace_slices": (_i32, [_i64, _i32, ctypes.POINTER(ctypes.c_int32)]),
    "asp_metric_product_partials": (_i32, [_p, _i64, _p, _i32, _p, _p]),
    "asp_top_eigenspace": (_i32, [_p, _i64, _p, _i32, _i32, _i32, _p, _p, _p, _p, _sz, _p]),
    "asp_svdq_packed_sizes": (_i32, [_i64, _i64, _i32, _psz, _psz, _psz, _psz]),
    "asp_svdq_gram": (_i32, [_i64, _i64, _p, _p, _p]),
    "asp_svdq_pack_weight": (_i32, [_i64, _i64, _i32, _p, _p, _p, _p, _p, _p, _p]),
    "asp_svdq_workspace_bytes": (_i32, [_i64, _i64, _i64, _i32, _psz]),
    "asp_svdq_act_quant": (_i32, [_p, _i32, _i64, _i64, _p, _p, _p, _p]),
    "asp_svdq_gemm": (_i32, [_p, _p, _p, _i64, _i64, _i64, _i32, _p, _p, _p, _p, _p, _i32, _p]),
    "asp_svdq_forward": (_i32, [_p, _i32, _i64, _i64, _i32, _p, _p, _p, _p, _p, _i64, _p, _i32,
                                _p, _sz, _p]),
    "asp_forward_noalloc": (_i32, [_p, _i32, _i64, _i64, _i64, _i32, _p, _p, _p, _p, _p, _p,
                                   _i32, _p]),
    "asp_forward_group": (_i32, [_i32, _p, _i32, _i64, _i64, _i32, _p, _p, _p, _p, _p, _p, _p,
                                 _i32, _p, _p, _p]),
    "asp_forward_group_stages": (_i32, [_i32, _i32, _p, _i32, _i64, _i64, _i32, _p, _p, _p, _p,
                                        _p, _p, _p, _i32, _p, _p, _p]),
}

_lib = None


class ASPError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded libasp.  Raises if it has not been built, if its ABI
    revision differs from this binding's, or if it was built from sources
    other than the ones beside it (a stale build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m wam_asp_w4a4_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        if handle.asp_abi_version() != ABI_VERSION:
            raise RuntimeError("libasp ABI version mismatch")
        from .build import source_digest
        built, current = handle.asp_source_digest().decode(), source_digest()
        if built != current:
            raise RuntimeError(f"{LIB_PATH} was built from other sources (digest {built}, "
                               f"sources {current}): rebuild it with "
                               "`python -m wam_asp_w4a4_amd.build`")
        _lib = handle
    return _lib


def _check(status: int):
    if status != 0:
        msg = lib().asp_last_error().decode()
        raise ASPError(status, msg)


def _ptr(a):
    if a is None:
        return None
    if isinstance(a, np.ndarray):
        if not a.flags["C_CONTIGUOUS"]:
            raise ValueError("NumPy arrays must be C-contiguous")
        return a.ctypes.data
    if not a.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return a.data_ptr()


def _stream(stream, *tensors):
    if stream is not None:
        return stream
    import torch
    for t in tensors:
        if isinstance(t, torch.Tensor) and t.is_cuda:
            return torch.cuda.current_stream(t.device).cuda_stream
    return None


# ------------------------------------------------------------------- host


def asp_abi_version() -> int:
    return lib().asp_abi_version()


def asp_source_digest() -> str:
    return lib().asp_source_digest().decode()


def asp_status_string(status: int) -> str:
    return lib().asp_status_string(status).decode()


def asp_last_error() -> str:
    return lib().asp_last_error().decode()


def asp_packed_sizes(N: int, K: int, r: int):
    c, s, w = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().asp_packed_sizes(N, K, r, ctypes.byref(c), ctypes.byref(s), ctypes.byref(w)))
    return c.value, s.value, w.value


def asp_workspace_bytes(M: int, N: int, K: int, r: int) -> int:
    b = ctypes.c_size_t()
    _check(lib().asp_workspace_bytes(M, N, K, r, ctypes.byref(b)))
    return b.value


def asp_prep_pack_bytes(K: int, r: int) -> int:
    b = ctypes.c_size_t()
    _check(lib().asp_prep_pack_bytes(K, r, ctypes.byref(b)))
    return b.value


def asp_pack_prep(K, r, s, v, prep_pack):
    _check(lib().asp_pack_prep(K, r, _ptr(s), _ptr(v), _ptr(prep_pack)))


def asp_pack_weight(N, K, r, w, s, v, w_codes, w_scales, wv, w_prequant=None, n_threads=0):
    _check(lib().asp_pack_weight(N, K, r, _ptr(w), _ptr(s), _ptr(v), _ptr(w_codes),
                                 _ptr(w_scales), _ptr(wv), _ptr(w_prequant), n_threads))


def asp_pack_weight_shared(N, K, r, w, s, v, w_codes, w_scales, wv, w_prequant=None,
                           n_threads=0):
    _check(lib().asp_pack_weight_shared(N, K, r, _ptr(w), _ptr(s), _ptr(v), _ptr(w_codes),
                                        _ptr(w_scales), _ptr(wv), _ptr(w_prequant), n_threads))


def asp_quantize_nvfp4_host(inp, rows, cols, codes, scales):
    _check(lib().asp_quantize_nvfp4_host(_ptr(inp), rows, cols, _ptr(codes), _ptr(scales)))


# ----------------------------------------------------------------- device


def asp_quantize_nvfp4(inp, rows, cols, codes, scales, stream=None):
    _check(lib().asp_quantize_nvfp4(_ptr(inp), rows, cols, _ptr(codes), _ptr(scales),
                                    _stream(stream, inp)))


def asp_dequantize_nvfp4(codes, scales, rows, cols, out, stream=None):
    _check(lib().asp_dequantize_nvfp4(_ptr(codes), _ptr(scales), rows, cols, _ptr(out),
                                      _stream(stream, out)))


def asp_act_prep_workspace_bytes(M: int, K: int, r: int) -> int:
    b = ctypes.c_size_t()
    _check(lib().asp_act_prep_workspace_bytes(M, K, r, ctypes.byref(b)))
    return b.value


def asp_act_prep(x, x_dtype, M, K, r, prep_pack, x_codes, x_scales, u, prequant=None,
                 workspace=None, workspace_bytes=0, stream=None):
    _check(lib().asp_act_prep(_ptr(x), x_dtype, M, K, r, _ptr(prep_pack), _ptr(x_codes),
                              _ptr(x_scales), _ptr(u), _ptr(prequant), _ptr(workspace),
                              workspace_bytes, _stream(stream, x)))


def asp_gemm_kernel_name(M, N, K):
    return lib().asp_gemm_kernel_name(M, N, K).decode()


def asp_act_prep_u(x, x_dtype, M, K, r, prep_pack, workspace=None, workspace_bytes=0,
                   stream=None):
    _check(lib().asp_act_prep_u(_ptr(x), x_dtype, M, K, r, _ptr(prep_pack), _ptr(workspace),
                                workspace_bytes, _stream(stream, x)))


def asp_act_prep_q(x, x_dtype, M, K, r, prep_pack, x_codes, x_scales, u, prequant=None,
                   workspace=None, workspace_bytes=0, stream=None):
    _check(lib().asp_act_prep_q(_ptr(x), x_dtype, M, K, r, _ptr(prep_pack), _ptr(x_codes),
                                _ptr(x_scales), _ptr(u), _ptr(prequant), _ptr(workspace),
                                workspace_bytes, _stream(stream, x)))


def asp_gemm_lowrank(x_codes, x_scales, u, M, N, K, r, w_codes, w_scales, wv, bias, y, y_dtype,
                     stream=None):
    _check(lib().asp_gemm_lowrank(_ptr(x_codes), _ptr(x_scales), _ptr(u), M, N, K, r,
                                  _ptr(w_codes), _ptr(w_scales), _ptr(wv), _ptr(bias), _ptr(y),
                                  y_dtype, _stream(stream, y)))


def asp_smoothing_search_workspace_bytes(M, N, K, r, n_candidates):
    out = ctypes.c_size_t(0)
    _check(lib().asp_smoothing_search_workspace_bytes(M, N, K, r, n_candidates, ctypes.byref(out)))
    return out.value


def asp_smoothing_search(x, x_dtype, M, K, w, bias, N, v, r, alphas, betas, workspace,
                         workspace_bytes, stream=None):
    """Returns (mse per candidate as a NumPy float64 array, best index)."""
    # converted copies are held in locals until the call returns
    alphas = np.ascontiguousarray(alphas, np.float32)
    betas = np.ascontiguousarray(betas, np.float32)
    w = np.ascontiguousarray(w, np.float32)
    bias = None if bias is None else np.ascontiguousarray(bias, np.float32)
    v = None if v is None else np.ascontiguousarray(v, np.float32)
    n = len(alphas)
    mse = np.empty(n, np.float64)
    best = ctypes.c_int32(0)
    _check(lib().asp_smoothing_search(
        _ptr(x), x_dtype, M, K, _ptr(w), _ptr(bias), N, _ptr(v), r, _ptr(alphas), _ptr(betas), n,
        _ptr(mse), ctypes.cast(ctypes.byref(best), ctypes.c_void_p).value, _ptr(workspace),
        workspace_bytes, _stream(stream, x)))
    return mse, int(best.value)


def asp_top_eigenspace_workspace_bytes(K, p, r):
    out = ctypes.c_size_t(0)
    _check(lib().asp_top_eigenspace_workspace_bytes(K, p, r, ctypes.byref(out)))
    return out.value


def asp_top_eigenspace_slices(K, p):
    out = ctypes.c_int32(0)
    _check(lib().asp_top_eigenspace_slices(K, p, ctypes.byref(out)))
    return int(out.value)


def asp_metric_product_partials(g, K, v, p, yp, stream=None):
    _check(lib().asp_metric_product_partials(_ptr(g), K, _ptr(v), p, _ptr(yp),
                                             _stream(stream, g)))


def asp_top_eigenspace(g, K, v0, p, r, iters, v, evals, resid, workspace, workspace_bytes,
                       stream=None):
    _check(lib().asp_top_eigenspace(_ptr(g), K, _ptr(v0), p, r, iters, _ptr(v), _ptr(evals),
                                    _ptr(resid), _ptr(workspace), workspace_bytes,
                                    _stream(stream, g)))


def asp_svdq_packed_sizes(N, K, r):
    """(code bytes, scale bytes, L1 bytes, prep-pack bytes) of one packed layer."""
    out = [ctypes.c_size_t(0) for _ in range(4)]
    _check(lib().asp_svdq_packed_sizes(N, K, r, *[ctypes.byref(o) for o in out]))
    return tuple(o.value for o in out)


def asp_svdq_gram(N, K, w, s, g):
    _check(lib().asp_svdq_gram(N, K, _ptr(w), _ptr(s), _ptr(g)))


def asp_svdq_pack_weight(N, K, r, w, s, v, codes, scales, l1, prep):
    _check(lib().asp_svdq_pack_weight(N, K, r, _ptr(w), _ptr(s), _ptr(v), _ptr(codes),
                                      _ptr(scales), _ptr(l1), _ptr(prep)))


def asp_svdq_workspace_bytes(M, N, K, r):
    out = ctypes.c_size_t(0)
    _check(lib().asp_svdq_workspace_bytes(M, N, K, r, ctypes.byref(out)))
    return out.value


def asp_svdq_act_quant(x, x_dtype, M, K, prep_pack, x_codes, x_scales, stream=None):
    _check(lib().asp_svdq_act_quant(_ptr(x), x_dtype, M, K, _ptr(prep_pack), _ptr(x_codes),
                                    _ptr(x_scales), _stream(stream, x)))


def asp_svdq_gemm(x_codes, x_scales, u, M, N, K, r, w_codes, w_scales, l1, bias, y, y_dtype,
                  stream=None):
    _check(lib().asp_svdq_gemm(_ptr(x_codes), _ptr(x_scales), _ptr(u), M, N, K, r, _ptr(w_codes),
                               _ptr(w_scales), _ptr(l1), _ptr(bias), _ptr(y), y_dtype,
                               _stream(stream, y)))


def asp_svdq_forward(x, x_dtype, M, K, r, prep_pack, w_codes, w_scales, l1, bias, N, y, y_dtype,
                     workspace, workspace_bytes, stream=None):
    _check(lib().asp_svdq_forward(_ptr(x), x_dtype, M, K, r, _ptr(prep_pack), _ptr(w_codes),
                                  _ptr(w_scales), _ptr(l1), _ptr(bias), N, _ptr(y), y_dtype,
                                  _ptr(workspace), workspace_bytes, _stream(stream, x)))


def _ptr_array(items):
    """A host array of device pointers (NULL entries for None); None for a None list."""
    if items is None:
        return None, None
    arr = (ctypes.c_void_p * len(items))(*[_ptr(a) for a in items])
    return arr, ctypes.cast(arr, ctypes.c_void_p).value


def asp_forward_group(x, x_dtype, M, K, r, prep_pack, w_codes, w_scales, wv, bias, N, y, y_dtype,
                      workspace, workspace_bytes, stream=None):
    """Per-layer arguments are equal-length lists (bias and wv may be None)."""
    asp_forward_group_stages(7, x, x_dtype, M, K, r, prep_pack, w_codes, w_scales, wv, bias, N, y,
                             y_dtype, workspace, workspace_bytes, stream)


def asp_forward_group_stages(stages, x, x_dtype, M, K, r, prep_pack, w_codes, w_scales, wv, bias,
                             N, y, y_dtype, workspace, workspace_bytes, stream=None):
    n = len(y)
    keep = []  # the ctypes arrays must outlive the call

    def arr(items):
        a, p = _ptr_array(items)
        keep.append(a)
        return p

    nn = (ctypes.c_int64 * n)(*N)
    nb = (ctypes.c_size_t * n)(*workspace_bytes)
    keep += [nn, nb]
    _check(lib().asp_forward_group_stages(
        stages, n, arr(x), x_dtype, M, K, r, arr(prep_pack), arr(w_codes), arr(w_scales), arr(wv),
        arr(bias), ctypes.cast(nn, ctypes.c_void_p).value, arr(y), y_dtype, arr(workspace),
        ctypes.cast(nb, ctypes.c_void_p).value, _stream(stream, *y)))


def asp_forward_noalloc(x, x_dtype, M, N, K, r, prep_pack, w_codes, w_scales, wv, bias, y,
                        y_dtype, stream=None):
    _check(lib().asp_forward_noalloc(_ptr(x), x_dtype, M, N, K, r, _ptr(prep_pack),
                                     _ptr(w_codes), _ptr(w_scales), _ptr(wv), _ptr(bias), _ptr(y),
                                     y_dtype, _stream(stream, y)))


def asp_forward(x, x_dtype, M, N, K, r, prep_pack, w_codes, w_scales, wv, bias, y, y_dtype,
                workspace, workspace_bytes, stream=None):
    _check(lib().asp_forward(_ptr(x), x_dtype, M, N, K, r, _ptr(prep_pack), _ptr(w_codes),
                             _ptr(w_scales), _ptr(wv), _ptr(bias), _ptr(y), y_dtype,
                             _ptr(workspace), workspace_bytes, _stream(stream, y)))
