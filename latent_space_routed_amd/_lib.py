"""ctypes binding of liblmoe.so: the calls of include/lmoe.h under the same names.

Argument marshalling only: tensors are passed as device pointers, the current HIP stream is passed
as the stream, and a non-OK status raises ``LmoeError``. Nothing here computes; if the library
is missing the import of any call fails loudly (there is no fallback).
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblmoe.so")

LMOE_OK, LMOE_ERR_INVALID_ARGUMENT, LMOE_ERR_UNSUPPORTED, LMOE_ERR_WORKSPACE, LMOE_ERR_HIP = range(5)
LMOE_F32, LMOE_BF16 = 0, 1
LMOE_CALL_ROUTE, LMOE_CALL_PERMUTE, LMOE_CALL_GROUPED_GLU, LMOE_CALL_COMBINE_NORM_UP = 0, 1, 2, 3
LMOE_CALL_GROUPED_GLU_MX = 32
LMOE_CALL_BWD_UP, LMOE_CALL_BWD_COMBINE_NORM, LMOE_CALL_BWD_EXPERTS, LMOE_CALL_BWD_DOWN, LMOE_CALL_BWD_SHARED = \
    16, 17, 18, 19, 20

# every symbol include/lmoe.h declares
EXPORTS = ("lmoe_workspace_bytes", "lmoe_status_string", "lmoe_split_router", "lmoe_route", "lmoe_qb_histogram",
           "lmoe_qb_update", "lmoe_permute", "lmoe_grouped_situ_glu", "lmoe_grouped_situ_glu_noalloc",
           "lmoe_pack_shared", "lmoe_combine_norm_up", "lmoe_combine_norm", "lmoe_up_project",
           "lmoe_bwd_transpose_weights", "lmoe_bwd_up",
           "lmoe_bwd_combine_norm", "lmoe_bwd_router", "lmoe_bwd_experts", "lmoe_bwd_down", "lmoe_bwd_shared",
           "lmoe_mx_quantize", "lmoe_grouped_situ_glu_mx", "lmoe_profile_enable", "lmoe_profile_only",
           "lmoe_profile_reset", "lmoe_profile_collect", "lmoe_profile_get")


class LmoeError(RuntimeError):
    def __init__(self, call: str, status: int):
        super().__init__(f"{call} failed: {status_string(status)} ({status})")
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d_model", ctypes.c_int32), ("d_latent", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("n_shared", ctypes.c_int32), ("inter_shared", ctypes.c_int32), ("n_bins", ctypes.c_int32),
                ("beta1", ctypes.c_float), ("beta2", ctypes.c_float), ("rms_eps", ctypes.c_float),
                ("act_dtype", ctypes.c_int32)]


def make_shape(cfg, T: int | None = None) -> Shape:
    """lmoe_shape from any object with the layer-shape attributes (T overridable)."""
    return Shape(cfg.T if T is None else T, cfg.d_model, cfg.d_latent, cfg.n_experts, cfg.top_k, cfg.inter,
                 cfg.n_shared, cfg.inter_shared, cfg.n_bins, cfg.beta1, cfg.beta2, cfg.rms_eps,
                 LMOE_BF16 if cfg.act_dtype == "bf16" else LMOE_F32)


_lib = None
_P = ctypes.c_void_p
_S = ctypes.POINTER(Shape)


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m latent_space_routed_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        sigs = {
            "lmoe_workspace_bytes": (ctypes.c_size_t, [_S, ctypes.c_int]),
            "lmoe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
            "lmoe_split_router": (ctypes.c_int, [_S, _P, _P, _P]),
            "lmoe_route": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
            "lmoe_qb_histogram": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _P]),
            "lmoe_qb_update": (ctypes.c_int, [_S, _P, ctypes.c_int64, _P, _P]),
            "lmoe_permute": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
            "lmoe_grouped_situ_glu": (ctypes.c_int, [_S, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                     ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_int32, _P, _P,
                                                     _P, _P, _P, _P, ctypes.c_int32, _P, ctypes.c_size_t, _P]),
            "lmoe_grouped_situ_glu_noalloc": (ctypes.c_int, [_S, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                             ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_int32, _P,
                                                             _P, _P, _P, _P, _P, ctypes.c_int32, _P]),
            "lmoe_pack_shared": (ctypes.c_int, [_S, _P, _P, _P, _P, _P]),
            "lmoe_combine_norm_up": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_int32,
                                                    _P, ctypes.c_size_t, _P]),
            "lmoe_combine_norm": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _P]),
            "lmoe_up_project": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _P, ctypes.c_int32, _P, ctypes.c_size_t, _P]),
            "lmoe_bwd_transpose_weights": (ctypes.c_int, [_S] + [_P] * 9),
            "lmoe_bwd_up": (ctypes.c_int, [_S] + [_P] * 10 + [ctypes.c_size_t, _P]),
            "lmoe_bwd_combine_norm": (ctypes.c_int, [_S] + [_P] * 12 + [ctypes.c_size_t, _P]),
            "lmoe_bwd_router": (ctypes.c_int, [_S] + [_P] * 10),
            "lmoe_bwd_experts": (ctypes.c_int, [_S] + [_P] * 13 + [ctypes.c_size_t, _P]),
            "lmoe_bwd_down": (ctypes.c_int, [_S] + [_P] * 8 + [ctypes.c_size_t, _P]),
            "lmoe_bwd_shared": (ctypes.c_int, [_S] + [_P] * 8 + [ctypes.c_size_t, _P]),
            "lmoe_mx_quantize": (ctypes.c_int, [_S, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, _P, _P, _P, _P]),
            "lmoe_grouped_situ_glu_mx": (ctypes.c_int, [_S, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                         ctypes.c_int32, ctypes.c_int32, _P, _P, ctypes.c_int32, _P,
                                                         _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
            "lmoe_profile_enable": (None, [ctypes.c_int]),
            "lmoe_profile_only": (None, [ctypes.c_char_p]),
            "lmoe_profile_reset": (None, []),
            "lmoe_profile_collect": (ctypes.c_int, []),
            "lmoe_profile_get": (ctypes.c_int, [ctypes.c_char_p, ctypes.POINTER(ctypes.c_int64),
                                                ctypes.POINTER(ctypes.c_double)]),
        }
        for name, (res, args) in sigs.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().lmoe_status_string(status).decode()


def _ptr(t: torch.Tensor | None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError("lmoe calls take device tensors")
    if not t.is_contiguous():
        raise ValueError("lmoe calls take contiguous tensors")
    return t.data_ptr()


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _check(name: str, status: int) -> None:
    if status != LMOE_OK:
        raise LmoeError(name, status)


def _nbytes(t: torch.Tensor | None) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def workspace_bytes(shape: Shape, which: int) -> int:
    return int(lib().lmoe_workspace_bytes(ctypes.byref(shape), which))


def lmoe_split_router(shape, w_router, w_router_split, stream=None):
    _check("lmoe_split_router", lib().lmoe_split_router(ctypes.byref(shape), _ptr(w_router), _ptr(w_router_split),
                                                        _stream(stream)))


def lmoe_route(shape, x, w_router, bias, logit_offset, scores, topk_idx, topk_w, thresh, workspace, stream=None,
               w_router_split=None):
    """w_router_split (optional, bf16 layers): the lmoe_split_router output, so the call does not
    split the router weights again."""
    _check("lmoe_route", lib().lmoe_route(ctypes.byref(shape), _ptr(x), _ptr(w_router), _ptr(w_router_split),
                                          _ptr(bias), _ptr(logit_offset), _ptr(scores), _ptr(topk_idx),
                                          _ptr(topk_w), _ptr(thresh), _ptr(workspace), _nbytes(workspace),
                                          _stream(stream)))


def lmoe_qb_histogram(shape, scores, bias, topk_idx, thresh, hist, stream=None):
    _check("lmoe_qb_histogram", lib().lmoe_qb_histogram(ctypes.byref(shape), _ptr(scores), _ptr(bias),
                                                        _ptr(topk_idx), _ptr(thresh), _ptr(hist), _stream(stream)))


def lmoe_qb_update(shape, hist, n_acc: int, bias, stream=None):
    _check("lmoe_qb_update", lib().lmoe_qb_update(ctypes.byref(shape), _ptr(hist), int(n_acc), _ptr(bias),
                                                  _stream(stream)))


def lmoe_permute(shape, x, w_down, topk_idx, x_lat, expert_offsets, sorted_token, slot_of_pair, x_perm, workspace,
                 stream=None):
    _check("lmoe_permute", lib().lmoe_permute(ctypes.byref(shape), _ptr(x), _ptr(w_down), _ptr(topk_idx),
                                              _ptr(x_lat), _ptr(expert_offsets), _ptr(sorted_token),
                                              _ptr(slot_of_pair), _ptr(x_perm), _ptr(workspace),
                                              _nbytes(workspace), _stream(stream)))


def lmoe_grouped_situ_glu(shape, n_groups: int, rows: int, K: int, inter: int, n_out: int, a, group_offsets, w1, w2,
                          h, y, workspace, a_row_index=None, stream=None):
    """a_row_index (optional): GEMM row r reads a[a_row_index[r]]; w2/y None stops after h."""
    y_dtype = LMOE_F32 if (y is not None and y.dtype == torch.float32) else LMOE_BF16
    a_rows = a.shape[0] if a_row_index is not None else rows
    _check("lmoe_grouped_situ_glu",
           lib().lmoe_grouped_situ_glu(ctypes.byref(shape), n_groups, rows, K, inter, n_out, _ptr(a), a_rows,
                                       _ptr(a_row_index), _ptr(group_offsets), _ptr(w1), _ptr(w2), _ptr(h), _ptr(y),
                                       y_dtype, _ptr(workspace), _nbytes(workspace), _stream(stream)))


def lmoe_grouped_situ_glu_noalloc(shape, n_groups: int, rows: int, K: int, inter: int, n_out: int, a, group_offsets,
                                  w1, w2, h, y, a_row_index=None, stream=None):
    """lmoe_grouped_situ_glu without a workspace (the library's own per-device scratch array)."""
    y_dtype = LMOE_F32 if (y is not None and y.dtype == torch.float32) else LMOE_BF16
    a_rows = a.shape[0] if a_row_index is not None else rows
    _check("lmoe_grouped_situ_glu_noalloc",
           lib().lmoe_grouped_situ_glu_noalloc(ctypes.byref(shape), n_groups, rows, K, inter, n_out, _ptr(a), a_rows,
                                               _ptr(a_row_index), _ptr(group_offsets), _ptr(w1), _ptr(w2), _ptr(h),
                                               _ptr(y), y_dtype, _stream(stream)))


def lmoe_pack_shared(shape, w1s, w2s, w1s_packed, w2s_packed, stream=None):
    _check("lmoe_pack_shared", lib().lmoe_pack_shared(ctypes.byref(shape), _ptr(w1s), _ptr(w2s), _ptr(w1s_packed),
                                                      _ptr(w2s_packed), _stream(stream)))


def lmoe_combine_norm_up(shape, y_perm, slot_of_pair, topk_w, gamma, w_up, y_shared, n_out, out, h_shared=None,
                         w2_shared=None, workspace=None, stream=None):
    out_dtype = LMOE_F32 if out.dtype == torch.float32 else LMOE_BF16
    _check("lmoe_combine_norm_up",
           lib().lmoe_combine_norm_up(ctypes.byref(shape), _ptr(y_perm), _ptr(slot_of_pair), _ptr(topk_w),
                                      _ptr(gamma), _ptr(w_up), _ptr(y_shared), _ptr(h_shared), _ptr(w2_shared),
                                      _ptr(n_out), _ptr(out), out_dtype, _ptr(workspace), _nbytes(workspace),
                                      _stream(stream)))


def lmoe_combine_norm(shape, y_perm, slot_of_pair, topk_w, gamma, n_out, stream=None):
    _check("lmoe_combine_norm",
           lib().lmoe_combine_norm(ctypes.byref(shape), _ptr(y_perm), _ptr(slot_of_pair), _ptr(topk_w), _ptr(gamma),
                                   _ptr(n_out), _stream(stream)))


def lmoe_up_project(shape, n, w_up, y_shared, out, h_shared=None, w2_shared=None, workspace=None, stream=None):
    out_dtype = LMOE_F32 if out.dtype == torch.float32 else LMOE_BF16
    _check("lmoe_up_project",
           lib().lmoe_up_project(ctypes.byref(shape), _ptr(n), _ptr(w_up), _ptr(y_shared), _ptr(h_shared),
                                 _ptr(w2_shared), _ptr(out), out_dtype, _ptr(workspace), _nbytes(workspace),
                                 _stream(stream)))


def _call(name: str, shape, *args):
    """Calls a backward entry point: tensors and None become pointers; a (tensor, 'ws') pair becomes
    the workspace pointer and its size."""
    cargs = [ctypes.byref(shape)]
    for a in args:
        if isinstance(a, tuple):
            cargs += [_ptr(a[0]), _nbytes(a[0])]
        else:
            cargs.append(_ptr(a))
    cargs.append(_stream(None))
    _check(name, getattr(lib(), name)(*cargs))


def lmoe_bwd_transpose_weights(shape, w_up, w2s_packed, w1s_packed, w_down, w_up_t, w2s_t, w1s_t, w_down_t):
    _call("lmoe_bwd_transpose_weights", shape, w_up, w2s_packed, w1s_packed, w_down, w_up_t, w2s_t, w1s_t, w_down_t)


def lmoe_bwd_up(shape, dout, n, h_shared, w_up_t, w2s_t, dn, dh_shared, dw_up, dw2_shared, workspace):
    _call("lmoe_bwd_up", shape, dout, n, h_shared, w_up_t, w2s_t, dn, dh_shared, dw_up, dw2_shared, (workspace, "ws"))


def lmoe_bwd_combine_norm(shape, dn, y_perm, slot_of_pair, topk_idx, scores, topk_w, gamma, dy_perm, dlogit,
                          dlogit_sorted, dgamma, workspace):
    _call("lmoe_bwd_combine_norm", shape, dn, y_perm, slot_of_pair, topk_idx, scores, topk_w, gamma, dy_perm, dlogit,
          dlogit_sorted, dgamma, (workspace, "ws"))


def lmoe_bwd_router(shape, x, w_router, dlogit, dlogit_sorted, topk_idx, expert_offsets, sorted_token, dw_router, dx):
    _call("lmoe_bwd_router", shape, x, w_router, dlogit, dlogit_sorted, topk_idx, expert_offsets, sorted_token,
          dw_router, dx)


def lmoe_bwd_experts(shape, x_lat, sorted_token, expert_offsets, w1, w2, h, dy_perm, dh, dgu, dx_perm, dw1, dw2,
                     workspace):
    _call("lmoe_bwd_experts", shape, x_lat, sorted_token, expert_offsets, w1, w2, h, dy_perm, dh, dgu, dx_perm, dw1,
          dw2, (workspace, "ws"))


def lmoe_bwd_down(shape, x, dx_perm, slot_of_pair, w_down_t, dx_lat, dw_down, dx, workspace):
    _call("lmoe_bwd_down", shape, x, dx_perm, slot_of_pair, w_down_t, dx_lat, dw_down, dx, (workspace, "ws"))


def lmoe_bwd_shared(shape, x, w1s_packed, w1s_t, dh_shared, dgu_shared, dw1s_packed, dx, workspace):
    _call("lmoe_bwd_shared", shape, x, w1s_packed, w1s_t, dh_shared, dgu_shared, dw1s_packed, dx, (workspace, "ws"))


LMOE_MX_FP4, LMOE_MX_FP8 = 4, 8


def lmoe_mx_quantize(shape, fmt: int, rows: int, K: int, x, codes, scales, stream=None):
    _check("lmoe_mx_quantize", lib().lmoe_mx_quantize(ctypes.byref(shape), int(fmt), int(rows), int(K), _ptr(x),
                                                      _ptr(codes), _ptr(scales), _stream(stream)))


def lmoe_grouped_situ_glu_mx(shape, G, rows, K, inter, n_out, a_codes, a_scales, a_rows, a_row_index, group_offsets,
                             w1_codes, w1_scales, w2_codes, w2_scales, h, y, workspace, stream=None):
    _check("lmoe_grouped_situ_glu_mx", lib().lmoe_grouped_situ_glu_mx(
        ctypes.byref(shape), int(G), int(rows), int(K), int(inter), int(n_out), _ptr(a_codes), _ptr(a_scales),
        int(a_rows), _ptr(a_row_index), _ptr(group_offsets), _ptr(w1_codes), _ptr(w1_scales), _ptr(w2_codes),
        _ptr(w2_scales), _ptr(h), _ptr(y), _ptr(workspace), _nbytes(workspace), _stream(stream)))


def profile_enable(on: bool) -> None:
    lib().lmoe_profile_enable(1 if on else 0)


def profile_only(name: str | None) -> None:
    """Time only the kernels named ``name`` (None: every kernel)."""
    lib().lmoe_profile_only(name.encode() if name else None)


def profile_reset() -> None:
    lib().lmoe_profile_reset()


def profile_collect() -> None:
    _check("lmoe_profile_collect", lib().lmoe_profile_collect())


def profile_get(name: str):
    n, ms = ctypes.c_int64(0), ctypes.c_double(0.0)
    if not lib().lmoe_profile_get(name.encode(), ctypes.byref(n), ctypes.byref(ms)):
        return 0, 0.0
    return int(n.value), float(ms.value)
