"""ctypes binding of libmep.so.  Argument marshalling only: every step of the path runs in the
HIP kernels behind the C ABI (include/mep.h).  PyTorch supplies device memory and the stream.

The functions named like the C entry points take preallocated tensors; the convenience
helpers ``route``, ``build_layout`` and ``plan`` allocate outputs and workspaces with torch.
There is no CPU fallback: if the library is missing or no GPU is present, calls raise.
"""
from __future__ import annotations

import ctypes
import os
import threading
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmep.so")

MEP_OK, MEP_ERR_INVALID_ARG, MEP_ERR_UNSUPPORTED, MEP_ERR_CAPACITY, MEP_ERR_DEVICE = 0, 1, 2, 3, 4
MEP_F32, MEP_BF16 = 0, 1
MEP_SOFTMAX, MEP_SIGMOID = 0, 1


class MepError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__("%s failed: %s (%d)" % (where, status_string(code), code))
        self.code = code


class RouteParams(ctypes.Structure):
    _fields_ = [("score_fn", ctypes.c_int), ("renormalize", ctypes.c_int),
                ("n_group", ctypes.c_int), ("topk_group", ctypes.c_int),
                ("group_topn", ctypes.c_int), ("scale", ctypes.c_float)]


class PlanOutputs(ctypes.Structure):
    _fields_ = [("is_token_in_rank", ctypes.c_void_p), ("num_tokens_per_rank", ctypes.c_void_p),
                ("num_tokens_per_expert", ctypes.c_void_p), ("rank_prefix_matrix", ctypes.c_void_p),
                ("channel_prefix_matrix", ctypes.c_void_p), ("recv_tokens", ctypes.c_void_p),
                ("recv_cu_seqlens", ctypes.c_void_p), ("recv_zero_fill", ctypes.c_void_p),
                ("dst", ctypes.c_void_p), ("dup_counts", ctypes.c_void_p),
                ("dup_offsets", ctypes.c_void_p), ("dup_groups", ctypes.c_void_p),
                ("cap_groups", ctypes.c_int64), ("dup_loffs", ctypes.c_void_p),
                ("cap_dups", ctypes.c_int64)]


BALANCED_FIELDS = ("group_tokens", "z", "alloc", "alloc_cumsum", "experts_to_copy", "remote_stats",
                   "cu_seqlens", "zero_fill", "expert_offsets", "dst")


class BalancedOutputs(ctypes.Structure):
    _fields_ = [(f, ctypes.c_void_p) for f in BALANCED_FIELDS]


EXPORTS = ("mep_route_topk", "mep_route_topk_timed", "mep_build_layout", "mep_layout_workspace_size", "mep_plan",
           "mep_plan_workspace_size", "mep_layout_plan", "mep_route_layout_plan",
           "mep_route_layout_plan_timed", "mep_route_layout_plan_noalloc", "mep_tile_map",
           "mep_plan_balanced", "mep_permute_rows",
           "mep_combine_rows", "mep_sigmoid_eval", "mep_status_string")

_lib = None
_lock = threading.Lock()


def lib():
    """Load libmep.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise RuntimeError("libmep.so is not built; run python -m expert_dispatch_layout_amd.build")
                L = ctypes.CDLL(LIB_PATH)
                P, I64, I, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
                L.mep_route_topk.argtypes = [P, I, I64, I, I, P, ctypes.POINTER(RouteParams), P, P, P]
                L.mep_route_topk.restype = I
                L.mep_route_topk_timed.argtypes = [P, I, I64, I, I, P, ctypes.POINTER(RouteParams),
                                                   P, P, P, P, P]
                L.mep_route_topk_timed.restype = I
                L.mep_build_layout.argtypes = [P, I64, I, I, I, P, P, P, P, I64, P, P, SZ, P]
                L.mep_build_layout.restype = I
                L.mep_layout_workspace_size.argtypes = [I64, I, I]
                L.mep_layout_workspace_size.restype = SZ
                L.mep_plan.argtypes = [P, P, P, I64, I, I, I, I, I, I, I64,
                                       ctypes.POINTER(PlanOutputs), P, SZ, P]
                L.mep_plan.restype = I
                L.mep_plan_workspace_size.argtypes = [I64, I, I, I, I]
                L.mep_plan_workspace_size.restype = SZ
                L.mep_layout_plan.argtypes = [P, I64, I, I, I, P, P, P, P, I64, P,
                                              I, I, I, I64, ctypes.POINTER(PlanOutputs), P, SZ, P]
                L.mep_layout_plan.restype = I
                L.mep_tile_map.argtypes = [P, I, I64, I, P, P, I64, P, P, P]
                L.mep_tile_map.restype = I
                L.mep_route_layout_plan.argtypes = [P, I, I64, I, I, P, ctypes.POINTER(RouteParams), P, P,
                                                    I, P, P, P, P, I64, P, I, I, I, I64,
                                                    ctypes.POINTER(PlanOutputs), P, SZ, P]
                L.mep_route_layout_plan.restype = I
                L.mep_route_layout_plan_timed.argtypes = L.mep_route_layout_plan.argtypes + [P, P, P, P]
                L.mep_route_layout_plan_timed.restype = I
                L.mep_route_layout_plan_noalloc.argtypes = L.mep_route_layout_plan.argtypes[:21] + [P]
                L.mep_route_layout_plan_noalloc.restype = I
                L.mep_plan_balanced.argtypes = [P, P, P, P, I64, I, I, I, I, I, I64, I64,
                                                ctypes.POINTER(BalancedOutputs), P]
                L.mep_plan_balanced.restype = I
                L.mep_permute_rows.argtypes = [P, I, I64, I64, I, P, P, I, P, I64, P]
                L.mep_permute_rows.restype = I
                L.mep_combine_rows.argtypes = [P, I, I64, I64, I, P, P, I64, P, P]
                L.mep_combine_rows.restype = I
                L.mep_sigmoid_eval.argtypes = [P, I64, P, P, P, P]
                L.mep_sigmoid_eval.restype = I
                L.mep_status_string.argtypes = [I]
                L.mep_status_string.restype = ctypes.c_char_p
                _lib = L
    return _lib


def status_string(code: int) -> str:
    return lib().mep_status_string(code).decode()


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check(rc: int, where: str):
    if rc != MEP_OK:
        raise MepError(rc, where)


def _require_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("device tensors are required")


# ---------------------------------------------------------------------------------------------
# Entry points with the C names (preallocated outputs)
# ---------------------------------------------------------------------------------------------

def mep_route_topk(logits, K, bias, params: RouteParams, topk_ids, topk_weights=None, stream=None):
    _require_cuda(logits, bias, topk_ids, topk_weights)
    dtype = MEP_BF16 if logits.dtype == torch.bfloat16 else MEP_F32
    if logits.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("logits must be float32 or bfloat16")
    N, E = logits.shape
    rc = lib().mep_route_topk(_ptr(logits), dtype, N, E, K, _ptr(bias), ctypes.byref(params),
                              _ptr(topk_ids), _ptr(topk_weights), _stream(stream))
    _check(rc, "mep_route_topk")


def mep_sigmoid_eval(x, cr_out=None, filter_out=None, weight_out=None, stream=None):
    """The routing kernels' sigmoid evaluations of float32 device tensor `x` into the given
    outputs (float32, float32, float64; any may be None)."""
    _require_cuda(x, cr_out, filter_out, weight_out)
    if x.dtype != torch.float32 or not x.is_contiguous():
        raise ValueError("x must be a contiguous float32 tensor")
    for t, dt in ((cr_out, torch.float32), (filter_out, torch.float32), (weight_out, torch.float64)):
        if t is not None and (t.dtype != dt or t.numel() < x.numel() or not t.is_contiguous()):
            raise ValueError("outputs must be contiguous, of the input's size and of their dtype")
    rc = lib().mep_sigmoid_eval(_ptr(x), x.numel(), _ptr(cr_out), _ptr(filter_out), _ptr(weight_out),
                                _stream(stream))
    _check(rc, "mep_sigmoid_eval")


def mep_build_layout(topk_ids, E, alignment, tokens_per_expert, cu_seqlens, expanded_to_permuted,
                     permuted_to_expanded, zero_fill, ws, stream=None):
    _require_cuda(topk_ids, tokens_per_expert, cu_seqlens, expanded_to_permuted,
                  permuted_to_expanded, zero_fill, ws)
    N, K = topk_ids.shape
    cap = permuted_to_expanded.numel() if permuted_to_expanded is not None else 0
    rc = lib().mep_build_layout(_ptr(topk_ids), N, E, K, alignment, _ptr(tokens_per_expert),
                                _ptr(cu_seqlens), _ptr(expanded_to_permuted),
                                _ptr(permuted_to_expanded), cap, _ptr(zero_fill), _ptr(ws),
                                ws.numel() * ws.element_size(), _stream(stream))
    _check(rc, "mep_build_layout")


def mep_plan(topk_ids, cu_seqlens, expanded_to_permuted, E, alignment, R, num_src, num_channels,
             NvS, outputs: "PlanTensors", ws, stream=None):
    _require_cuda(topk_ids, cu_seqlens, expanded_to_permuted, ws)
    N, K = topk_ids.shape
    po = outputs.as_struct()
    rc = lib().mep_plan(_ptr(topk_ids), _ptr(cu_seqlens), _ptr(expanded_to_permuted), N, E, K,
                        alignment, R, num_src, num_channels, NvS, ctypes.byref(po), _ptr(ws),
                        ws.numel() * ws.element_size(), _stream(stream))
    _check(rc, "mep_plan")


# ---------------------------------------------------------------------------------------------
# Prepared calls: the same entry points with their arguments converted once, for loops that
# issue the same call many times (a zero-argument callable per call; each call checks the
# return code).  Tensors must stay alive and in place while the callable is used.
# ---------------------------------------------------------------------------------------------

def tile_map_capacity(num_slots: int, E: int, tile: int) -> int:
    """Tiles that `num_slots` slots over E experts can need at most (the bound mep_tile_map
    checks cap_ctas against)."""
    return (num_slots + min(E, num_slots) * (tile - 1)) // tile


def mep_tile_map(tokens_per_expert, num_slots, tile, cta_to_expert=None, cta_mn_limit=None,
                 permuted_idx_size=None, num_ctas=None, stream=None):
    _require_cuda(tokens_per_expert, cta_to_expert, cta_mn_limit, permuted_idx_size, num_ctas)
    E = tokens_per_expert.numel()
    caps = [t.numel() for t in (cta_to_expert, cta_mn_limit) if t is not None]
    cap = min(caps) if caps else 0
    rc = lib().mep_tile_map(_ptr(tokens_per_expert), E, num_slots, tile, _ptr(cta_to_expert),
                            _ptr(cta_mn_limit), cap, _ptr(permuted_idx_size), _ptr(num_ctas),
                            _stream(stream))
    _check(rc, "mep_tile_map")


def _row_dtype(t):
    if t.dtype == torch.bfloat16:
        return MEP_BF16
    if t.dtype == torch.float32:
        return MEP_F32
    raise ValueError("rows must be float32 or bfloat16")


def _permute_args(x, expanded_to_permuted, K, zero_fill, x_permuted, stream):
    _require_cuda(x, expanded_to_permuted, zero_fill, x_permuted)
    if x.dtype != x_permuted.dtype:
        raise ValueError("x and x_permuted must have the same dtype")
    N, H = x.shape
    E = zero_fill.shape[0] if zero_fill is not None else 0
    return (_ptr(x), _row_dtype(x), N, H, K, _ptr(expanded_to_permuted), _ptr(zero_fill), E,
            _ptr(x_permuted), x_permuted.shape[0], _stream(stream))


def _combine_args(y_permuted, expanded_to_permuted, K, topk_weights, out, stream):
    _require_cuda(y_permuted, expanded_to_permuted, topk_weights, out)
    if y_permuted.dtype != out.dtype:
        raise ValueError("y_permuted and out must have the same dtype")
    N, H = out.shape
    return (_ptr(y_permuted), _row_dtype(out), N, H, K, _ptr(expanded_to_permuted),
            _ptr(topk_weights), y_permuted.shape[0], _ptr(out), _stream(stream))


def mep_permute_rows(x, expanded_to_permuted, K, zero_fill, x_permuted, stream=None):
    _check(lib().mep_permute_rows(*_permute_args(x, expanded_to_permuted, K, zero_fill, x_permuted,
                                                 stream)), "mep_permute_rows")


def mep_combine_rows(y_permuted, expanded_to_permuted, K, topk_weights, out, stream=None):
    _check(lib().mep_combine_rows(*_combine_args(y_permuted, expanded_to_permuted, K, topk_weights,
                                                 out, stream)), "mep_combine_rows")


def bound_permute_rows(x, expanded_to_permuted, K, zero_fill, x_permuted, stream=None):
    return _bound("mep_permute_rows",
                  _permute_args(x, expanded_to_permuted, K, zero_fill, x_permuted, stream),
                  "mep_permute_rows")


def bound_combine_rows(y_permuted, expanded_to_permuted, K, topk_weights, out, stream=None):
    return _bound("mep_combine_rows",
                  _combine_args(y_permuted, expanded_to_permuted, K, topk_weights, out, stream),
                  "mep_combine_rows")


def bound_tile_map(tokens_per_expert, num_slots, tile, cta_to_expert=None, cta_mn_limit=None,
                   permuted_idx_size=None, num_ctas=None, stream=None):
    _require_cuda(tokens_per_expert, cta_to_expert, cta_mn_limit, permuted_idx_size, num_ctas)
    caps = [t.numel() for t in (cta_to_expert, cta_mn_limit) if t is not None]
    return _bound("mep_tile_map", (_ptr(tokens_per_expert), tokens_per_expert.numel(), num_slots,
                                   tile, _ptr(cta_to_expert), _ptr(cta_mn_limit),
                                   min(caps) if caps else 0, _ptr(permuted_idx_size),
                                   _ptr(num_ctas), _stream(stream)), "mep_tile_map")


def _bound(fn_name, args, where):
    fn = getattr(lib(), fn_name)
    args = tuple(args)

    def call():
        rc = fn(*args)
        if rc != MEP_OK:
            raise MepError(rc, where)
    return call


def bound_route_topk(logits, K, bias, params: RouteParams, topk_ids, topk_weights=None, stream=None,
                     timer: "KernelTimer" = None):
    """With `timer`, the call is mep_route_topk_timed: the routing kernel's own launch updates
    the timer's two events with its start and end."""
    _require_cuda(logits, bias, topk_ids, topk_weights)
    if logits.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("logits must be float32 or bfloat16")
    dtype = MEP_BF16 if logits.dtype == torch.bfloat16 else MEP_F32
    N, E = logits.shape
    args = (_ptr(logits), dtype, N, E, K, _ptr(bias), ctypes.byref(params), _ptr(topk_ids),
            _ptr(topk_weights), _stream(stream))
    if timer is None:
        return _bound("mep_route_topk", args, "mep_route_topk")
    return _bound("mep_route_topk_timed", args + (timer.start, timer.stop), "mep_route_topk_timed")


class KernelTimer:
    """Two HIP events (created through the HIP runtime that torch and libmep share) for
    mep_route_topk_timed; elapsed_ms() is hipEventElapsedTime once the work has completed.
    The events are timing-only (hipEventDisableSystemFence): recording them performs no
    system-scope cache write-back, which would otherwise delay the work that follows."""

    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence

    def __init__(self, flags: int = DISABLE_SYSTEM_FENCE):
        if KernelTimer._hip is None:
            h = ctypes.CDLL("libamdhip64.so.7")
            h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                              ctypes.c_void_p]
            h.hipEventDestroy.argtypes = [ctypes.c_void_p]
            KernelTimer._hip = h
        self.start = ctypes.c_void_p()
        self.stop = ctypes.c_void_p()
        for e in (self.start, self.stop):
            rc = KernelTimer._hip.hipEventCreateWithFlags(ctypes.byref(e), flags)
            if rc != 0:
                raise RuntimeError("hipEventCreateWithFlags failed (%d)" % rc)

    def elapsed_ms(self) -> float:
        ms = ctypes.c_float()
        rc = KernelTimer._hip.hipEventElapsedTime(ctypes.byref(ms), self.start, self.stop)
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed (%d)" % rc)
        return ms.value

    def __del__(self):
        h = type(self)._hip  # not the module global, which interpreter shutdown may clear first
        if h is not None:
            for e in (self.start, self.stop):
                if e:
                    h.hipEventDestroy(e)


def event_elapsed_ms(start, stop) -> float:
    """hipEventElapsedTime between two events (ctypes handles, e.g. of two KernelTimers)."""
    if KernelTimer._hip is None:
        KernelTimer(0)
    ms = ctypes.c_float()
    rc = KernelTimer._hip.hipEventElapsedTime(ctypes.byref(ms), start, stop)
    if rc != 0:
        raise RuntimeError("hipEventElapsedTime failed (%d)" % rc)
    return ms.value


def bound_build_layout(topk_ids, E, alignment, tokens_per_expert, cu_seqlens, expanded_to_permuted,
                       permuted_to_expanded, zero_fill, ws, stream=None):
    _require_cuda(topk_ids, tokens_per_expert, cu_seqlens, expanded_to_permuted,
                  permuted_to_expanded, zero_fill, ws)
    N, K = topk_ids.shape
    cap = permuted_to_expanded.numel() if permuted_to_expanded is not None else 0
    return _bound("mep_build_layout", (_ptr(topk_ids), N, E, K, alignment, _ptr(tokens_per_expert),
                                       _ptr(cu_seqlens), _ptr(expanded_to_permuted),
                                       _ptr(permuted_to_expanded), cap, _ptr(zero_fill), _ptr(ws),
                                       ws.numel() * ws.element_size(), _stream(stream)),
                  "mep_build_layout")


def bound_plan(topk_ids, cu_seqlens, expanded_to_permuted, E, alignment, R, num_src, num_channels,
               NvS, outputs: "PlanTensors", ws, stream=None):
    _require_cuda(topk_ids, cu_seqlens, expanded_to_permuted, ws)
    N, K = topk_ids.shape
    po = outputs.as_struct()
    call = _bound("mep_plan", (_ptr(topk_ids), _ptr(cu_seqlens), _ptr(expanded_to_permuted), N, E, K,
                               alignment, R, num_src, num_channels, NvS, ctypes.byref(po), _ptr(ws),
                               ws.numel() * ws.element_size(), _stream(stream)), "mep_plan")
    call.outputs = po  # keeps the struct referenced by the byref alive
    return call


def _layout_plan_args(topk_ids, E, alignment, layout, R, num_src, num_channels, NvS, po, ws, stream):
    N, K = topk_ids.shape
    cap = layout.permuted_to_expanded.numel() if layout.permuted_to_expanded is not None else 0
    return (_ptr(topk_ids), N, E, K, alignment, _ptr(layout.tokens_per_expert), _ptr(layout.cu_seqlens),
            _ptr(layout.expanded_to_permuted), _ptr(layout.permuted_to_expanded), cap,
            _ptr(layout.zero_fill), R, num_src, num_channels, NvS, ctypes.byref(po), _ptr(ws),
            ws.numel() * ws.element_size(), _stream(stream))


def _route_layout_plan_args(logits, K, bias, params, topk_ids, topk_weights, alignment, layout, R,
                            num_src, num_channels, NvS, po, ws, stream):
    _require_cuda(logits, bias, topk_ids, topk_weights, ws)
    ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    if logits.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("logits must be float32 or bfloat16")
    dtype = MEP_BF16 if logits.dtype == torch.bfloat16 else MEP_F32
    N, E = logits.shape
    cap = layout.permuted_to_expanded.numel() if layout.permuted_to_expanded is not None else 0
    return (_ptr(logits), dtype, N, E, K, _ptr(bias), ctypes.byref(params), _ptr(topk_ids),
            _ptr(topk_weights), alignment, _ptr(layout.tokens_per_expert), _ptr(layout.cu_seqlens),
            _ptr(layout.expanded_to_permuted), _ptr(layout.permuted_to_expanded), cap,
            _ptr(layout.zero_fill), R, num_src, num_channels, NvS, ctypes.byref(po), _ptr(ws),
            ws_bytes, _stream(stream))


def mep_route_layout_plan(logits, K, bias, params, topk_ids, topk_weights, alignment,
                          layout: "LayoutTensors", R, num_src, num_channels, NvS,
                          outputs: "PlanTensors", ws, stream=None):
    """Routing, layout and plan in one call (one kernel for small batches)."""
    po = outputs.as_struct()
    rc = lib().mep_route_layout_plan(*_route_layout_plan_args(
        logits, K, bias, params, topk_ids, topk_weights, alignment, layout, R, num_src,
        num_channels, NvS, po, ws, stream))
    _check(rc, "mep_route_layout_plan")


def mep_route_layout_plan_noalloc(logits, K, bias, params, topk_ids, topk_weights, alignment,
                                  layout: "LayoutTensors", R, num_src, num_channels, NvS,
                                  outputs: "PlanTensors", stream=None):
    """mep_route_layout_plan with the library's own per-GPU workspace (allocates nothing)."""
    po = outputs.as_struct()
    args = _route_layout_plan_args(logits, K, bias, params, topk_ids, topk_weights, alignment,
                                   layout, R, num_src, num_channels, NvS, po, None, stream)
    rc = lib().mep_route_layout_plan_noalloc(*(args[:21] + args[23:]))
    _check(rc, "mep_route_layout_plan_noalloc")


def bound_route_layout_plan(logits, K, bias, params, topk_ids, topk_weights, alignment,
                            layout: "LayoutTensors", R, num_src, num_channels, NvS,
                            outputs: "PlanTensors", ws, stream=None,
                            route_timer: "KernelTimer" = None, plan_timer: "KernelTimer" = None):
    """With a timer, the call is mep_route_layout_plan_timed: the routing kernel's launch stamps
    route_timer's events, the plan-tile kernel's launch plan_timer's."""
    po = outputs.as_struct()
    args = _route_layout_plan_args(logits, K, bias, params, topk_ids, topk_weights, alignment,
                                   layout, R, num_src, num_channels, NvS, po, ws, stream)
    if route_timer is None and plan_timer is None:
        call = _bound("mep_route_layout_plan", args, "mep_route_layout_plan")
    else:
        ev = (route_timer.start if route_timer else None, route_timer.stop if route_timer else None,
              plan_timer.start if plan_timer else None, plan_timer.stop if plan_timer else None)
        call = _bound("mep_route_layout_plan_timed", args + ev, "mep_route_layout_plan_timed")
    call.keep = po
    return call


def mep_layout_plan(topk_ids, E, alignment, layout: "LayoutTensors", R, num_src, num_channels, NvS,
                    outputs: "PlanTensors", ws, stream=None):
    """mep_build_layout + mep_plan in one call; `ws` is a plan workspace."""
    _require_cuda(topk_ids, ws)
    po = outputs.as_struct()
    rc = lib().mep_layout_plan(*_layout_plan_args(topk_ids, E, alignment, layout, R, num_src,
                                                  num_channels, NvS, po, ws, stream))
    _check(rc, "mep_layout_plan")


def bound_layout_plan(topk_ids, E, alignment, layout: "LayoutTensors", R, num_src, num_channels,
                      NvS, outputs: "PlanTensors", ws, stream=None):
    _require_cuda(topk_ids, ws)
    po = outputs.as_struct()
    call = _bound("mep_layout_plan", _layout_plan_args(topk_ids, E, alignment, layout, R, num_src,
                                                       num_channels, NvS, po, ws, stream),
                  "mep_layout_plan")
    call.outputs = po
    return call


def layout_workspace_size(N, E, K) -> int:
    return int(lib().mep_layout_workspace_size(N, E, K))


def plan_workspace_size(N, E, K, R, num_src) -> int:
    return int(lib().mep_plan_workspace_size(N, E, K, R, num_src))


# ---------------------------------------------------------------------------------------------
# Allocating helpers
# ---------------------------------------------------------------------------------------------

def alloc_workspace(nbytes: int, device=None) -> torch.Tensor:
    """Zero-filled workspace (the library requires zero on first use and keeps it valid)."""
    return torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device or "cuda")


def route_params(score_fn=MEP_SOFTMAX, renormalize=True, n_group=1, topk_group=1, group_topn=2,
                 scale=1.0) -> RouteParams:
    return RouteParams(score_fn, int(renormalize), n_group, topk_group, group_topn, float(scale))


def route(logits, K, *, bias=None, score_fn=MEP_SOFTMAX, renormalize=True, n_group=1,
          topk_group=1, group_topn=2, scale=1.0, stream=None):
    N = logits.shape[0]
    ids = torch.empty((N, K), dtype=torch.int32, device=logits.device)
    w = torch.empty((N, K), dtype=torch.float32, device=logits.device)
    mep_route_topk(logits, K, bias, route_params(score_fn, renormalize, n_group, topk_group,
                                                 group_topn, scale), ids, w, stream)
    return ids, w


@dataclass
class LayoutTensors:
    tokens_per_expert: torch.Tensor
    cu_seqlens: torch.Tensor
    expanded_to_permuted: torch.Tensor
    permuted_to_expanded: torch.Tensor  # capacity-sized; first cu_seqlens[E] rows are valid
    zero_fill: torch.Tensor


def permuted_capacity(N, E, K, alignment) -> int:
    nk = N * K
    return nk + min(E, nk) * (alignment - 1)


def alloc_layout(N, E, K, alignment, device="cuda") -> LayoutTensors:
    cap = max(permuted_capacity(N, E, K, alignment), 1)
    i32 = dict(dtype=torch.int32, device=device)
    return LayoutTensors(torch.empty(E, **i32), torch.empty(E + 1, **i32),
                         torch.empty(max(N * K, 1), **i32)[:N * K], torch.empty(cap, **i32),
                         torch.empty((E, 2), **i32))


def build_layout(topk_ids, E, alignment, *, out: LayoutTensors | None = None, ws=None,
                 stream=None) -> LayoutTensors:
    N, K = topk_ids.shape
    out = out or alloc_layout(N, E, K, alignment, topk_ids.device)
    ws = ws if ws is not None else alloc_workspace(layout_workspace_size(N, E, K), topk_ids.device)
    mep_build_layout(topk_ids, E, alignment, out.tokens_per_expert, out.cu_seqlens,
                     out.expanded_to_permuted, out.permuted_to_expanded, out.zero_fill, ws, stream)
    return out


@dataclass
class PlanTensors:
    is_token_in_rank: torch.Tensor | None
    num_tokens_per_rank: torch.Tensor | None
    num_tokens_per_expert: torch.Tensor | None
    rank_prefix_matrix: torch.Tensor | None
    channel_prefix_matrix: torch.Tensor | None
    recv_tokens: torch.Tensor | None
    recv_cu_seqlens: torch.Tensor | None
    recv_zero_fill: torch.Tensor | None
    dst: torch.Tensor | None
    dup_counts: torch.Tensor | None
    dup_offsets: torch.Tensor | None
    dup_groups: torch.Tensor | None
    dup_loffs: torch.Tensor | None

    def as_struct(self) -> PlanOutputs:
        cap_g = self.dup_groups.shape[0] if self.dup_groups is not None else 0
        cap_d = self.dup_loffs.shape[0] if self.dup_loffs is not None else 0
        return PlanOutputs(*(_addr(t) for t in (
            self.is_token_in_rank, self.num_tokens_per_rank, self.num_tokens_per_expert,
            self.rank_prefix_matrix, self.channel_prefix_matrix, self.recv_tokens,
            self.recv_cu_seqlens, self.recv_zero_fill, self.dst, self.dup_counts,
            self.dup_offsets, self.dup_groups)), cap_g, _addr(self.dup_loffs), cap_d)


def _addr(t):
    return None if t is None else t.data_ptr()


@dataclass
class BalancedTensors:
    group_tokens: "torch.Tensor"
    z: "torch.Tensor"
    alloc: "torch.Tensor"
    alloc_cumsum: "torch.Tensor"
    experts_to_copy: "torch.Tensor"
    remote_stats: "torch.Tensor"
    cu_seqlens: "torch.Tensor"
    zero_fill: "torch.Tensor"
    expert_offsets: "torch.Tensor"
    dst: "torch.Tensor"

    def as_struct(self) -> BalancedOutputs:
        return BalancedOutputs(*[getattr(self, f).data_ptr() if getattr(self, f).numel() else None
                                 for f in BALANCED_FIELDS])


def balanced_nvs(N, E, K, R, num_copies, token_padding, capacity) -> int:
    """The smallest per-rank row stride mep_plan_balanced accepts."""
    epn = E // R
    return max(N * min(K, epn), capacity) + (E + num_copies) * (token_padding - 1)


def alloc_balanced(N, E, K, R, num_copies, device="cuda") -> BalancedTensors:
    i32 = dict(dtype=torch.int32, device=device)
    G = E + num_copies
    return BalancedTensors(torch.empty(R, **i32), torch.empty((R, R), **i32),
                           torch.empty((R, E), **i32), torch.empty((E, R), **i32),
                           torch.empty((R, num_copies), **i32), torch.empty((R, 2), **i32),
                           torch.empty((R, G), **i32), torch.empty((R, G, 2), **i32),
                           torch.empty((R, E), **i32), torch.empty(N * K, **i32))


def _balanced_args(topk_ids, layout, E, R, num_copies, token_padding, capacity, NvS, out, stream):
    _require_cuda(topk_ids, layout.tokens_per_expert, layout.cu_seqlens, layout.expanded_to_permuted)
    N, K = topk_ids.shape
    st = out.as_struct()
    return ((_ptr(topk_ids), _ptr(layout.tokens_per_expert), _ptr(layout.cu_seqlens),
             _ptr(layout.expanded_to_permuted), N, E, K, R, num_copies, token_padding, capacity, NvS,
             ctypes.byref(st), _stream(stream)), st)


def mep_plan_balanced(topk_ids, layout, E, R, num_copies, token_padding, capacity, NvS,
                      out: BalancedTensors, stream=None):
    args, _keep = _balanced_args(topk_ids, layout, E, R, num_copies, token_padding, capacity, NvS,
                                 out, stream)
    _check(lib().mep_plan_balanced(*args), "mep_plan_balanced")


def bound_plan_balanced(topk_ids, layout, E, R, num_copies, token_padding, capacity, NvS,
                        out: BalancedTensors, stream=None):
    args, keep = _balanced_args(topk_ids, layout, E, R, num_copies, token_padding, capacity, NvS,
                                out, stream)
    call = _bound("mep_plan_balanced", args, "mep_plan_balanced")
    call.keep = keep  # the output table must outlive the prepared call
    return call


def default_nvs(N, E, K, R, alignment) -> int:
    epn = E // R
    return N * min(K, epn) + epn * (alignment - 1)


def dedup_capacity(N, E, K, R):
    epn = E // R
    g = N * min(K // 2, R) if epn >= 2 else 0
    d = N * (K - (K + epn - 1) // epn)
    return g, d


def alloc_plan(N, E, K, R, num_src, num_channels, device="cuda") -> PlanTensors:
    epn = E // R
    i32 = dict(dtype=torch.int32, device=device)
    cap_g, cap_d = dedup_capacity(N, E, K, R)
    return PlanTensors(
        torch.empty((max(N, 1), R), dtype=torch.uint8, device=device)[:N],
        torch.empty((num_src, R), **i32), torch.empty((num_src, E), **i32),
        torch.empty((num_src, R), **i32), torch.empty((num_src, R, num_channels), **i32),
        torch.empty(R, **i32), torch.empty((R, epn + 1), **i32), torch.empty((E, 2), **i32),
        torch.empty(max(N * K, 1), **i32)[:N * K], torch.empty((R, 2), **i32),
        torch.empty((R + 1, 2), **i32), torch.empty((max(cap_g, 1), 3), **i32),
        torch.empty(max(cap_d, 1), **i32))


def plan(topk_ids, cu_seqlens, expanded_to_permuted, E, alignment, R, num_src, num_channels, *,
         NvS=None, out: PlanTensors | None = None, ws=None, stream=None) -> PlanTensors:
    N, K = topk_ids.shape
    NvS = NvS if NvS is not None else default_nvs(N, E, K, R, alignment)
    out = out or alloc_plan(N, E, K, R, num_src, num_channels, topk_ids.device)
    ws = ws if ws is not None else alloc_workspace(plan_workspace_size(N, E, K, R, num_src),
                                                   topk_ids.device)
    mep_plan(topk_ids, cu_seqlens, expanded_to_permuted, E, alignment, R, num_src, num_channels,
             NvS, out, ws, stream)
    return out
