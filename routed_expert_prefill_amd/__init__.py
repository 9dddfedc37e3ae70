"""Grouped routed-MoE prefill on gfx950: Python binding of the C ABI.

The three calls mirror include/moe_prefill.h one to one; every step runs in
the HIP library.  This module only checks tensor placement/dtypes, passes raw
device pointers and the current HIP stream, and allocates outputs and
workspaces with torch.  There is no CPU fallback: if the library is missing,
every call raises.
"""
from __future__ import annotations

import ctypes
from typing import NamedTuple, Optional

from . import _lib
from ._lib import (MOE_ACT_BF16, MOE_ACT_FP8_E4M3_ROW, MOE_W_BF16, MOE_W_FP8_E4M3_B128,
                   LibraryNotBuilt, MoeFfnDesc)

__all__ = [
    "route_topk", "route_build", "route_build_noalloc", "grouped_ffn", "combine", "combine_shared", "quant_rows_fp8", "MoEPrefill", "RouteTable",
    "ffn_desc", "ffn_plan", "ffn_gate_up", "ffn_down", "LibraryNotBuilt", "load_library",
]


def load_library():
    return _lib.load()


class RouteTable(NamedTuple):
    counts: "torch.Tensor"  # int32 [E+1]
    offsets: "torch.Tensor"  # int32 [E+2]
    sorted_routes: "torch.Tensor"  # int32 [T*k]
    route_rows: "torch.Tensor"  # int32 [T*k]


def _torch():
    import torch

    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    torch = _torch()
    return torch.cuda.current_stream().cuda_stream


def _need(t, name, dtype, ndim=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def route_topk(logits, k: int, bias=None, topk_ids=None, topk_w=None):
    """moe_route_topk: top-k experts (descending, ties to the lower index) and
    renormalised gates from fp32 router logits [T, E]."""
    torch = _torch()
    lib = _lib.load()
    _need(logits, "logits", torch.float32, 2)
    T, E = logits.shape
    if bias is not None:
        _need(bias, "bias", torch.float32, 1)
        if bias.numel() != E:
            raise ValueError("bias must have E entries")
    if topk_ids is None:
        topk_ids = torch.empty(T, k, dtype=torch.int32, device=logits.device)
    if topk_w is None:
        topk_w = torch.empty(T, k, dtype=torch.float32, device=logits.device)
    _need(topk_ids, "topk_ids", torch.int32, 2)
    _need(topk_w, "topk_w", torch.float32, 2)
    rc = lib.moe_route_topk(_ptr(logits), _ptr(bias), T, E, k, _ptr(topk_ids), _ptr(topk_w),
                            _stream())
    _lib.check(rc, "moe_route_topk")
    return topk_ids, topk_w


def route_build(topk_ids, route_mask, E: int, out: Optional[RouteTable] = None,
                workspace=None) -> RouteTable:
    """moe_route_build: histogram, prefix and stable scatter of the routes."""
    torch = _torch()
    lib = _lib.load()
    _need(topk_ids, "topk_ids", torch.int32, 2)
    if route_mask is not None:
        _need(route_mask, "route_mask", torch.uint8, 2)
    T, k = topk_ids.shape
    dev = topk_ids.device
    if out is None:
        out = RouteTable(
            counts=torch.empty(E + 1, dtype=torch.int32, device=dev),
            offsets=torch.empty(E + 2, dtype=torch.int32, device=dev),
            sorted_routes=torch.empty(T * k, dtype=torch.int32, device=dev),
            route_rows=torch.empty(T * k, dtype=torch.int32, device=dev),
        )
    wsb = lib.moe_route_build_workspace(T, k, E)
    if workspace is None:
        workspace = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)
    rc = lib.moe_route_build(_ptr(topk_ids), _ptr(route_mask), T, k, E, _ptr(out.counts),
                             _ptr(out.offsets), _ptr(out.sorted_routes), _ptr(out.route_rows),
                             _ptr(workspace), workspace.numel(), _stream())
    _lib.check(rc, "moe_route_build")
    return out


def route_build_noalloc(topk_ids, route_mask, E: int, out: Optional[RouteTable] = None) -> RouteTable:
    """moe_route_build_noalloc: the route build on the library's own device
    scratch (no workspace); at most MOE_ROUTE_NOALLOC_MAX_ROUTES routes.  The
    outputs are allocated here unless given; the C call allocates nothing."""
    torch = _torch()
    lib = _lib.load()
    _need(topk_ids, "topk_ids", torch.int32, 2)
    if route_mask is not None:
        _need(route_mask, "route_mask", torch.uint8, 2)
    T, k = topk_ids.shape
    dev = topk_ids.device
    if out is None:
        out = RouteTable(
            counts=torch.empty(E + 1, dtype=torch.int32, device=dev),
            offsets=torch.empty(E + 2, dtype=torch.int32, device=dev),
            sorted_routes=torch.empty(T * k, dtype=torch.int32, device=dev),
            route_rows=torch.empty(T * k, dtype=torch.int32, device=dev),
        )
    rc = lib.moe_route_build_noalloc(_ptr(topk_ids), _ptr(route_mask), T, k, E, _ptr(out.counts),
                                     _ptr(out.offsets), _ptr(out.sorted_routes),
                                     _ptr(out.route_rows), _stream())
    _lib.check(rc, "moe_route_build_noalloc")
    return out


def ffn_desc(T: int, k: int, E: int, d: int, f: int, fp8: bool = False) -> MoeFfnDesc:
    return MoeFfnDesc(T, k, E, d, f, MOE_W_FP8_E4M3_B128 if fp8 else MOE_W_BF16,
                      MOE_ACT_FP8_E4M3_ROW if fp8 else MOE_ACT_BF16)


def grouped_ffn(x, offsets, sorted_routes, w_gate, w_up, w_down, k: int, s_gate=None,
                s_up=None, s_down=None, y=None, workspace=None):
    """moe_grouped_ffn: y[i] = Wd . bf16(silu(Wg . x) * (Wu . x)) per sorted row i."""
    torch = _torch()
    lib = _lib.load()
    fp8 = w_gate.dtype == torch.uint8
    _need(x, "x", torch.bfloat16, 2)
    wdt = torch.uint8 if fp8 else torch.bfloat16
    for name, w in (("w_gate", w_gate), ("w_up", w_up), ("w_down", w_down)):
        _need(w, name, wdt, 3)
    _need(offsets, "offsets", torch.int32, 1)
    _need(sorted_routes, "sorted_routes", torch.int32, 1)
    if fp8:
        for name, s in (("s_gate", s_gate), ("s_up", s_up), ("s_down", s_down)):
            _need(s, name, torch.float32, 3)
    T, d = x.shape
    E, f, d2 = w_gate.shape
    if d2 != d or tuple(w_up.shape) != (E, f, d) or tuple(w_down.shape) != (E, d, f):
        raise ValueError("weight shapes must be w_gate/w_up [E,f,d] and w_down [E,d,f]")
    if offsets.numel() != E + 2 or sorted_routes.numel() != T * k:
        raise ValueError("offsets must have E+2 entries and sorted_routes T*k")
    desc = ffn_desc(T, k, E, d, f, fp8)
    if y is None:
        y = torch.empty(T * k, d, dtype=torch.float32, device=x.device)
    _need(y, "y", torch.float32, 2)
    wsb = lib.moe_grouped_ffn_workspace(ctypes.byref(desc))
    if workspace is None:
        workspace = torch.empty(max(wsb, 256), dtype=torch.uint8, device=x.device)
    rc = lib.moe_grouped_ffn(ctypes.byref(desc), _ptr(x), _ptr(offsets), _ptr(sorted_routes),
                             _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(s_gate), _ptr(s_up),
                             _ptr(s_down), _ptr(y), _ptr(workspace), workspace.numel(), _stream())
    _lib.check(rc, "moe_grouped_ffn")
    return y


def _ffn_ws(desc, device, workspace):
    torch = _torch()
    lib = _lib.load()
    need = lib.moe_grouped_ffn_workspace(ctypes.byref(desc))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    return workspace


def ffn_plan(desc: MoeFfnDesc, x, offsets, workspace):
    """moe_ffn_plan: tile schedule from offsets (fp8: also quantises x)."""
    lib = _lib.load()
    rc = lib.moe_ffn_plan(ctypes.byref(desc), _ptr(x), _ptr(offsets), _ptr(workspace),
                          workspace.numel(), _stream())
    _lib.check(rc, "moe_ffn_plan")


def ffn_gate_up(desc: MoeFfnDesc, x, sorted_routes, w_gate, w_up, s_gate, s_up, workspace):
    """moe_ffn_gate_up: gate/up GEMM with the SwiGLU epilogue, h into the workspace."""
    lib = _lib.load()
    rc = lib.moe_ffn_gate_up(ctypes.byref(desc), _ptr(x), _ptr(sorted_routes), _ptr(w_gate),
                             _ptr(w_up), _ptr(s_gate), _ptr(s_up), _ptr(workspace),
                             workspace.numel(), _stream())
    _lib.check(rc, "moe_ffn_gate_up")


def ffn_down(desc: MoeFfnDesc, offsets, w_down, s_down, y, workspace):
    """moe_ffn_down: (fp8: per-row quantisation of h) down GEMM into y."""
    lib = _lib.load()
    rc = lib.moe_ffn_down(ctypes.byref(desc), _ptr(offsets), _ptr(w_down), _ptr(s_down), _ptr(y),
                          _ptr(workspace), workspace.numel(), _stream())
    _lib.check(rc, "moe_ffn_down")


def _row_limit(row_limit):
    """The combine's row bound: a one-element int32 device tensor (for
    instance ``offsets[E:E + 1]`` of a route table) or None."""
    torch = _torch()
    if row_limit is None:
        return None
    if not isinstance(row_limit, torch.Tensor) or row_limit.dtype != torch.int32 or \
            row_limit.numel() != 1 or row_limit.device.type != "cuda":
        raise TypeError("row_limit must be a one-element int32 GPU tensor")
    return row_limit.data_ptr()


def combine(y, route_rows, topk_w, route_mask, out=None, row_limit=None):
    """moe_combine: out[t] = sum over read j of w[t,j] * y[route_rows[t*k+j]] (fp32).

    Route r is read when its mask is set and, with row_limit (offsets[E:E+1]
    of the route table), its row lies below offsets[E]."""
    torch = _torch()
    lib = _lib.load()
    _need(y, "y", torch.float32, 2)
    _need(route_rows, "route_rows", torch.int32, 1)
    _need(topk_w, "topk_w", torch.float32, 2)
    if route_mask is not None:
        _need(route_mask, "route_mask", torch.uint8, 2)
    lim = _row_limit(row_limit)
    T, k = topk_w.shape
    d = y.shape[1]
    if out is None:
        out = torch.empty(T, d, dtype=torch.float32, device=y.device)
    _need(out, "out", torch.float32, 2)
    rc = lib.moe_combine(_ptr(y), _ptr(route_rows), _ptr(topk_w), _ptr(route_mask), lim, T, k,
                         d, _ptr(out), _stream())
    _lib.check(rc, "moe_combine")
    return out


def combine_shared(y, route_rows, topk_w, route_mask, shared=None, out=None, out_bf16=None,
                   want_fp32=True, want_bf16=False, row_limit=None):
    """moe_combine_shared: routed combine plus the shared-expert rows, as fp32
    and/or bf16 (round to nearest even)."""
    torch = _torch()
    lib = _lib.load()
    _need(y, "y", torch.float32, 2)
    _need(route_rows, "route_rows", torch.int32, 1)
    _need(topk_w, "topk_w", torch.float32, 2)
    if route_mask is not None:
        _need(route_mask, "route_mask", torch.uint8, 2)
    lim = _row_limit(row_limit)
    T, k = topk_w.shape
    d = y.shape[1]
    if shared is not None:
        _need(shared, "shared", torch.float32, 2)
        if tuple(shared.shape) != (T, d):
            raise ValueError("shared must be [T, d]")
    if out is None and want_fp32:
        out = torch.empty(T, d, dtype=torch.float32, device=y.device)
    if out_bf16 is None and want_bf16:
        out_bf16 = torch.empty(T, d, dtype=torch.bfloat16, device=y.device)
    if out is not None:
        _need(out, "out", torch.float32, 2)
    if out_bf16 is not None:
        _need(out_bf16, "out_bf16", torch.bfloat16, 2)
    rc = lib.moe_combine_shared(_ptr(y), _ptr(route_rows), _ptr(topk_w), _ptr(route_mask), lim,
                                _ptr(shared), T, k, d, _ptr(out), _ptr(out_bf16), _stream())
    _lib.check(rc, "moe_combine_shared")
    return out, out_bf16


def quant_rows_fp8(x, q=None, s=None):
    """moe_quant_rows_fp8: per-row E4M3 codes and fp32 scales of a bf16 matrix."""
    torch = _torch()
    lib = _lib.load()
    _need(x, "x", torch.bfloat16, 2)
    rows, cols = x.shape
    if q is None:
        q = torch.empty(rows, cols, dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty(rows, dtype=torch.float32, device=x.device)
    rc = lib.moe_quant_rows_fp8(_ptr(x), rows, cols, _ptr(q), _ptr(s), _stream())
    _lib.check(rc, "moe_quant_rows_fp8")
    return q, s


class MoEPrefill:
    """The whole path -- route build, grouped FFN, combine -- with buffers kept
    across calls (nothing is allocated per call after construction)."""

    def __init__(self, T: int, k: int, E: int, d: int, f: int, fp8: bool = False, device="cuda"):
        torch = _torch()
        lib = _lib.load()
        self.T, self.k, self.E, self.d, self.f, self.fp8 = T, k, E, d, f, fp8
        dev = torch.device(device)
        R = T * k
        self.rt = RouteTable(
            counts=torch.empty(E + 1, dtype=torch.int32, device=dev),
            offsets=torch.empty(E + 2, dtype=torch.int32, device=dev),
            sorted_routes=torch.empty(R, dtype=torch.int32, device=dev),
            route_rows=torch.empty(R, dtype=torch.int32, device=dev),
        )
        self.rb_ws = torch.empty(max(lib.moe_route_build_workspace(T, k, E), 256),
                                 dtype=torch.uint8, device=dev)
        self.desc = ffn_desc(T, k, E, d, f, fp8)
        self.ffn_ws = _ffn_ws(self.desc, dev, None)
        self.y = torch.empty(R, d, dtype=torch.float32, device=dev)
        self.out = torch.empty(T, d, dtype=torch.float32, device=dev)
        # offsets[E]: rows of y the FFN writes.  The combine reads no route at
        # or past it, so active routes whose ids lie outside [0, E) -- which
        # the route build sends to the trailing bin -- add exact zeros, as
        # masked ones do.
        self.row_limit = self.rt.offsets[E:E + 1]

    def __call__(self, x, topk_ids, topk_w, route_mask, w_gate, w_up, w_down, s_gate=None,
                 s_up=None, s_down=None, stage_events=None):
        """One pass of the path.  stage_events: optional torch events recorded
        on the current stream: 2 events around the gate/up stage, or 6 --
        before the route build and after each of route build, FFN plan,
        gate/up, down and combine."""
        ev = stage_events
        if ev is not None and len(ev) == 2:
            ev = [None, None, ev[0], ev[1], None, None]  # around ffn_gate_up
        if ev is not None and ev[0] is not None:
            ev[0].record()
        rt = route_build(topk_ids, route_mask, self.E, out=self.rt, workspace=self.rb_ws)
        if ev is None:
            grouped_ffn(x, rt.offsets, rt.sorted_routes, w_gate, w_up, w_down, self.k, s_gate,
                        s_up, s_down, y=self.y, workspace=self.ffn_ws)
            return combine(self.y, rt.route_rows, topk_w, route_mask, out=self.out,
                           row_limit=self.row_limit)
        def mark(i):
            if ev[i] is not None:
                ev[i].record()

        mark(1)
        ffn_plan(self.desc, x, rt.offsets, self.ffn_ws)
        mark(2)
        ffn_gate_up(self.desc, x, rt.sorted_routes, w_gate, w_up, s_gate, s_up, self.ffn_ws)
        mark(3)
        ffn_down(self.desc, rt.offsets, w_down, s_down, self.y, self.ffn_ws)
        mark(4)
        out = combine(self.y, rt.route_rows, topk_w, route_mask, out=self.out,
                      row_limit=self.row_limit)
        mark(5)
        return out
