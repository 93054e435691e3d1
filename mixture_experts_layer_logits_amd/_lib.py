"""ctypes binding of libmoe.so: the C ABI of include/moe.h, one Python
function per entry point with the same name.

Tensors are passed as device pointers (``t.data_ptr()``) and the stream is
torch's current HIP stream; nothing else crosses the boundary.  Every step of
the layer runs in the library's HIP kernels.  Loading fails loudly when the
library has not been built; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_WORKSPACE = -3
MOE_ERR_HIP = -4

MOE_DTYPE_F32 = 0
MOE_DTYPE_BF16 = 1
MOE_SCORE_SOFTMAX = 0
MOE_SCORE_SIGMOID = 1
(MOE_OP_ROUTE, MOE_OP_PERMUTE, MOE_OP_FFN, MOE_OP_COMBINE, MOE_OP_BACKWARD,
 MOE_OP_FFN_MXFP8, MOE_OP_BACKWARD_RECOMPUTE, MOE_OP_FFN_COMBINE,
 MOE_OP_BACKWARD_MXFP8) = range(9)

EXPORTED = ("moe_workspace_size", "moe_route_topk", "moe_permute",
            "moe_grouped_ffn", "moe_unpermute_combine", "moe_ffn_backward",
            "moe_status_string", "moe_mx_quantize", "moe_grouped_ffn_mxfp8",
            "moe_grouped_ffn_combine", "moe_mx_quantize_t", "moe_ffn_backward_mxfp8",
            "moe_grouped_ffn_mxfp8_combine", "moe_set_phase_events", "moe_permute_noalloc")
(MOE_PHASE_FC1, MOE_PHASE_FC2, MOE_PHASE_BWD_DISPATCH, MOE_PHASE_BWD_DH,
 MOE_PHASE_BWD_DW_DOWN, MOE_PHASE_BWD_DX, MOE_PHASE_BWD_DW_GATE_UP,
 MOE_PHASE_BWD_GATHER, MOE_PHASE_COUNT) = range(9)
PHASE_NAMES = ("fc1", "fc2", "bwd_dispatch", "bwd_dh", "bwd_dw_down", "bwd_dx",
               "bwd_dw_gate_up", "bwd_gather")


class MoeShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("T", "d", "E", "k", "F", "F_shared", "n_groups",
                 "topk_groups", "score", "renorm", "dtype", "wgrad_dtype", "wgrad_mx")]


class MoeError(RuntimeError):
    def __init__(self, status: int, fn: str):
        self.status = status
        super().__init__(f"{fn}: {status_string(status)} ({status})")


_lib: Optional[ctypes.CDLL] = None


def load() -> ctypes.CDLL:
    """Loads libmoe.so (raises if it is missing: build it first)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m mixture_experts_layer_logits_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    sp = ctypes.POINTER(MoeShape)
    lib.moe_workspace_size.argtypes = [sp, ctypes.c_int, ctypes.POINTER(sz)]
    lib.moe_route_topk.argtypes = [sp] + [vp] * 7 + [vp, sz, vp]
    lib.moe_permute.argtypes = [sp] + [vp] * 8 + [vp, sz, vp]
    lib.moe_permute_noalloc.argtypes = [sp] + [vp] * 8 + [vp]
    lib.moe_grouped_ffn.argtypes = [sp] + [vp] * 13 + [vp, sz, vp]
    lib.moe_unpermute_combine.argtypes = [sp] + [vp] * 5 + [vp, sz, vp]
    lib.moe_grouped_ffn_combine.argtypes = [sp] + [vp] * 12 + [vp, sz, vp]
    lib.moe_mx_quantize_t.argtypes = [vp, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.c_int32, vp, vp, vp]
    lib.moe_ffn_backward_mxfp8.argtypes = [sp] + [vp] * 28 + [vp, sz, vp]
    lib.moe_grouped_ffn_mxfp8_combine.argtypes = [sp] + [vp] * 18 + [vp, sz, vp]
    lib.moe_ffn_backward.argtypes = [sp] + [vp] * 26 + [vp, sz, vp]
    lib.moe_mx_quantize.argtypes = [vp, ctypes.c_int64, ctypes.c_int32, vp, vp, vp]
    lib.moe_grouped_ffn_mxfp8.argtypes = [sp] + [vp] * 18 + [vp, sz, vp]
    lib.moe_set_phase_events.argtypes = [ctypes.POINTER(vp), ctypes.c_int]
    lib.moe_status_string.argtypes = [ctypes.c_int]
    lib.moe_status_string.restype = ctypes.c_char_p
    for name in EXPORTED:
        if name != "moe_status_string":
            getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().moe_status_string(int(status)).decode()


def make_shape(cfg) -> MoeShape:
    """A moe_shape from an object with the layer's fields (e.g. MoEConfig)."""
    return MoeShape(cfg.T, cfg.d, cfg.E, cfg.k, cfg.F, cfg.F_shared,
                    cfg.n_groups, cfg.topk_groups, cfg.score, cfg.renorm,
                    cfg.dtype, getattr(cfg, "wgrad_dtype", MOE_DTYPE_F32),
                    getattr(cfg, "wgrad_mx", 0))


_I32, _F32, _U8 = torch.int32, torch.float32, torch.uint8


def _act(shape):
    """Storage type of x, the weights and the activations of ``shape``."""
    return torch.bfloat16 if shape.dtype == MOE_DTYPE_BF16 else torch.float32


def _wgt(shape):
    """Storage type of the weight gradients of ``shape``."""
    return torch.bfloat16 if shape.wgrad_dtype == MOE_DTYPE_BF16 else torch.float32


def _p(t, dtype=None) -> Optional[int]:
    """The device address of a tensor argument (an int passes through as an
    address).  The library reads every tensor as a dense row-major array of
    the type its declaration states, on the current device: a host tensor,
    a strided view or a tensor of another type is refused here instead of
    being misread (an empty tensor carries no data, so its type is free)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError(f"expected a device tensor, got one on {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"expected a contiguous tensor, got strides {t.stride()}")
    if dtype is not None and t.numel() > 0 and t.dtype != dtype:
        raise TypeError(f"expected a {dtype} tensor, got {t.dtype}")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, fn: str) -> int:
    if status != MOE_OK:
        raise MoeError(status, fn)
    return status


def moe_workspace_size(shape: MoeShape, op: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load().moe_workspace_size(ctypes.byref(shape), op, ctypes.byref(n)),
           "moe_workspace_size")
    return n.value


def moe_route_topk(shape, x, w_router, router_bias, logits, score_bias,
                   topk_idx, topk_w, ws=None, ws_bytes=0, stream=None,
                   check=True):
    st = load().moe_route_topk(
        ctypes.byref(shape), _p(x, _act(shape)), _p(w_router, _act(shape)),
        _p(router_bias, _F32), _p(logits, _F32), _p(score_bias, _F32),
        _p(topk_idx, _I32), _p(topk_w, _F32), _p(ws), ws_bytes,
        _stream(stream))
    return _check(st, "moe_route_topk") if check else st


def moe_permute(shape, x, topk_idx, topk_w, expert_offsets, row_token,
                token_row, row_gate, x_perm, ws=None, ws_bytes=0, stream=None,
                check=True):
    st = load().moe_permute(
        ctypes.byref(shape), _p(x, _act(shape)), _p(topk_idx, _I32), _p(topk_w, _F32),
        _p(expert_offsets, _I32), _p(row_token, _I32), _p(token_row, _I32),
        _p(row_gate, _F32), _p(x_perm, _act(shape)), _p(ws), ws_bytes, _stream(stream))
    return _check(st, "moe_permute") if check else st


def moe_permute_noalloc(shape, x, topk_idx, topk_w, expert_offsets, row_token,
                        token_row, row_gate, x_perm, stream=None, check=True):
    st = load().moe_permute_noalloc(
        ctypes.byref(shape), _p(x, _act(shape)), _p(topk_idx, _I32), _p(topk_w, _F32),
        _p(expert_offsets, _I32), _p(row_token, _I32), _p(token_row, _I32),
        _p(row_gate, _F32), _p(x_perm, _act(shape)), _stream(stream))
    return _check(st, "moe_permute_noalloc") if check else st


def moe_grouped_ffn(shape, x_perm, row_token, expert_offsets, w_gate, w_up,
                    w_down, x, ws_gate, ws_up, ws_down, y_perm, y_shared,
                    gu_save, ws=None, ws_bytes=0, stream=None, check=True):
    a = _act(shape)
    st = load().moe_grouped_ffn(
        ctypes.byref(shape), _p(x_perm, a), _p(row_token, _I32), _p(expert_offsets, _I32),
        _p(w_gate, a), _p(w_up, a), _p(w_down, a), _p(x, a), _p(ws_gate, a), _p(ws_up, a),
        _p(ws_down, a), _p(y_perm, a), _p(y_shared, a), _p(gu_save, a), _p(ws), ws_bytes,
        _stream(stream))
    return _check(st, "moe_grouped_ffn") if check else st


def moe_grouped_ffn_combine(shape, x_perm, row_token, row_gate, expert_offsets,
                            w_gate, w_up, w_down, x, ws_gate, ws_up, ws_down, y,
                            ws=None, ws_bytes=0, stream=None, check=True):
    a = _act(shape)
    st = load().moe_grouped_ffn_combine(
        ctypes.byref(shape), _p(x_perm, a), _p(row_token, _I32), _p(row_gate, _F32),
        _p(expert_offsets, _I32), _p(w_gate, a), _p(w_up, a), _p(w_down, a), _p(x, a),
        _p(ws_gate, a), _p(ws_up, a), _p(ws_down, a), _p(y, _F32), _p(ws), ws_bytes,
        _stream(stream))
    return _check(st, "moe_grouped_ffn_combine") if check else st


def moe_grouped_ffn_mxfp8_combine(shape, xq, xs, row_token, row_gate, expert_offsets,
                                  w_gate_q, w_gate_s, w_up_q, w_up_s, w_down_q, w_down_s,
                                  ws_gate_q, ws_gate_s, ws_up_q, ws_up_s, ws_down_q,
                                  ws_down_s, y, ws=None, ws_bytes=0, stream=None, check=True):
    st = load().moe_grouped_ffn_mxfp8_combine(
        ctypes.byref(shape), _p(xq, _U8), _p(xs, _U8), _p(row_token, _I32),
        _p(row_gate, _F32), _p(expert_offsets, _I32), *(_p(t, _U8) for t in (
            w_gate_q, w_gate_s, w_up_q, w_up_s, w_down_q, w_down_s, ws_gate_q, ws_gate_s,
            ws_up_q, ws_up_s, ws_down_q, ws_down_s)), _p(y, _F32), _p(ws), ws_bytes,
        _stream(stream))
    return _check(st, "moe_grouped_ffn_mxfp8_combine") if check else st


def moe_mx_quantize_t(src, batches, rows, cols, ldq, q, scales, stream=None, check=True):
    st = load().moe_mx_quantize_t(_p(src, torch.bfloat16), batches, rows, cols, ldq,
                                  _p(q, _U8), _p(scales, _U8), _stream(stream))
    return _check(st, "moe_mx_quantize_t") if check else st


def moe_ffn_backward_mxfp8(shape, dy, x_perm, gu_save, y_perm, expert_offsets,
                           row_token, token_row, topk_idx, topk_w, logits,
                           w_down_tq, w_down_ts, w_gu_tq, w_gu_ts, x,
                           ws_down_tq, ws_down_ts, ws_gu_tq, ws_gu_ts, dx,
                           dw_gate, dw_up, dw_down, dws_gate, dws_up, dws_down,
                           d_gate, d_logits, ws=None, ws_bytes=0, stream=None,
                           check=True):
    a, g = _act(shape), _wgt(shape)
    st = load().moe_ffn_backward_mxfp8(
        ctypes.byref(shape), _p(dy, a), _p(x_perm, a), _p(gu_save, a), _p(y_perm, a),
        _p(expert_offsets, _I32), _p(row_token, _I32), _p(token_row, _I32),
        _p(topk_idx, _I32), _p(topk_w, _F32), _p(logits, _F32), _p(w_down_tq, _U8),
        _p(w_down_ts, _U8), _p(w_gu_tq, _U8), _p(w_gu_ts, _U8), _p(x, a),
        _p(ws_down_tq, _U8), _p(ws_down_ts, _U8), _p(ws_gu_tq, _U8), _p(ws_gu_ts, _U8),
        _p(dx, _F32), _p(dw_gate, g), _p(dw_up, g), _p(dw_down, g), _p(dws_gate, g),
        _p(dws_up, g), _p(dws_down, g), _p(d_gate, _F32), _p(d_logits, _F32),
        _p(ws), ws_bytes, _stream(stream))
    return _check(st, "moe_ffn_backward_mxfp8") if check else st


def moe_unpermute_combine(shape, y_perm, token_row, topk_w, y_shared, y,
                          ws=None, ws_bytes=0, stream=None, check=True):
    st = load().moe_unpermute_combine(
        ctypes.byref(shape), _p(y_perm, _act(shape)), _p(token_row, _I32),
        _p(topk_w, _F32), _p(y_shared, _act(shape)), _p(y, _F32), _p(ws), ws_bytes,
        _stream(stream))
    return _check(st, "moe_unpermute_combine") if check else st


def moe_ffn_backward(shape, dy, x_perm, gu_save, y_perm, expert_offsets,
                     row_token, token_row, topk_idx, topk_w, logits, w_gate,
                     w_up, w_down, x, ws_gate, ws_up, ws_down, dx, dw_gate,
                     dw_up, dw_down, dws_gate, dws_up, dws_down, d_gate,
                     d_logits, ws=None, ws_bytes=0, stream=None, check=True):
    a, g = _act(shape), _wgt(shape)
    st = load().moe_ffn_backward(
        ctypes.byref(shape), _p(dy, a), _p(x_perm, a), _p(gu_save, a), _p(y_perm, a),
        _p(expert_offsets, _I32), _p(row_token, _I32), _p(token_row, _I32),
        _p(topk_idx, _I32), _p(topk_w, _F32), _p(logits, _F32), _p(w_gate, a),
        _p(w_up, a), _p(w_down, a), _p(x, a), _p(ws_gate, a), _p(ws_up, a),
        _p(ws_down, a), _p(dx, _F32), _p(dw_gate, g), _p(dw_up, g), _p(dw_down, g),
        _p(dws_gate, g), _p(dws_up, g), _p(dws_down, g), _p(d_gate, _F32),
        _p(d_logits, _F32), _p(ws), ws_bytes, _stream(stream))
    return _check(st, "moe_ffn_backward") if check else st


def moe_mx_quantize(src, rows, cols, q, scales, stream=None, check=True):
    st = load().moe_mx_quantize(_p(src, torch.bfloat16), int(rows), int(cols), _p(q, _U8),
                                _p(scales, _U8), _stream(stream))
    return _check(st, "moe_mx_quantize") if check else st


def moe_grouped_ffn_mxfp8(shape, xq, xs, row_token, expert_offsets, w_gate_q,
                          w_gate_s, w_up_q, w_up_s, w_down_q, w_down_s,
                          ws_gate_q, ws_gate_s, ws_up_q, ws_up_s, ws_down_q,
                          ws_down_s, y_perm, y_shared, ws=None, ws_bytes=0,
                          stream=None, check=True):
    st = load().moe_grouped_ffn_mxfp8(
        ctypes.byref(shape), _p(xq, _U8), _p(xs, _U8), _p(row_token, _I32),
        _p(expert_offsets, _I32), *(_p(t, _U8) for t in (
            w_gate_q, w_gate_s, w_up_q, w_up_s, w_down_q, w_down_s, ws_gate_q, ws_gate_s,
            ws_up_q, ws_up_s, ws_down_q, ws_down_s)), _p(y_perm, torch.bfloat16),
        _p(y_shared, torch.bfloat16), _p(ws), ws_bytes, _stream(stream))
    return _check(st, "moe_grouped_ffn_mxfp8") if check else st


def moe_set_phase_events(events) -> None:
    """Records the given hipEvent_t handles (a ctypes c_void_p array of
    2 * MOE_PHASE_COUNT entries, or None to stop) around each phase's
    kernels in later calls on this thread; the array must stay alive while
    set."""
    if events is None:
        _check(load().moe_set_phase_events(None, 0), "moe_set_phase_events")
    else:
        _check(load().moe_set_phase_events(events, len(events)), "moe_set_phase_events")
