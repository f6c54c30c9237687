"""Torch-facing binding of the C ABI: same names as include/coli_moe.h.

PyTorch provides device memory and streams only. Every function checks the
tensor shapes/dtypes it marshals, passes raw pointers to the library and
raises ColiError on a non-zero status.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional, Tuple

import numpy as np
import torch

from . import _lib
from ._lib import (CDense, CLayer, CWsLayout, COLI_ACCUMULATE, COLI_PATH_GEMV, COLI_PATH_GROUPED, ColiError,
                   check, lib)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dev(t: torch.Tensor, dtype, name: str):
    if not t.is_cuda or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} device tensor")


@dataclass
class MoELayer:
    """Device tensors of one MoE layer plus the C struct that points at them."""
    H: int
    I: int
    E: int
    top_k: int
    has_shared: int
    n_group: int
    topk_group: int
    route_scale: float
    router_w: torch.Tensor   # [E][H] f32
    router_b: torch.Tensor   # [E] f32
    gate_q: torch.Tensor     # [E+s][I][H/2] u8 (int4), [E+s][I][H] i8 (int8) or [E+s][I][H/4] u8 (int2)
    up_q: torch.Tensor
    down_q: torch.Tensor     # [E+s][H][I/2] u8 (int4), [E+s][H][I] i8 (int8) or [E+s][H][I/4] u8 (int2)
    gate_s: torch.Tensor     # [E+s][I] f32 ([E+s][I][H/G] with group scales)
    up_s: torch.Tensor
    down_s: torch.Tensor     # [E+s][H] f32 ([E+s][H][I/G])
    weight_bits: int = 4
    group_size: int = 0      # int4 only: > 0 gives one scale per group of that many columns

    @classmethod
    def empty(cls, H, I, E, top_k, has_shared=1, n_group=1, topk_group=1, route_scale=1.0, device="cuda",
              weight_bits=4, group_size=0):
        n = E + has_shared
        f32 = torch.float32
        qt, div = {8: (torch.int8, 1), 2: (torch.uint8, 4)}.get(weight_bits, (torch.uint8, 2))
        if group_size:
            if weight_bits == 8:
                raise ValueError("group scales are an int4 format")
            G = group_size
            return cls(H, I, E, top_k, has_shared, n_group, topk_group, route_scale,
                       torch.empty((E, H), dtype=f32, device=device), torch.empty(E, dtype=f32, device=device),
                       torch.empty((n, I, H // 2), dtype=qt, device=device),
                       torch.empty((n, I, H // 2), dtype=qt, device=device),
                       torch.empty((n, H, I // 2), dtype=qt, device=device),
                       torch.empty((n, I, H // G), dtype=f32, device=device),
                       torch.empty((n, I, H // G), dtype=f32, device=device),
                       torch.empty((n, H, I // G), dtype=f32, device=device), weight_bits, group_size)
        return cls(H, I, E, top_k, has_shared, n_group, topk_group, route_scale,
                   torch.empty((E, H), dtype=f32, device=device), torch.empty(E, dtype=f32, device=device),
                   torch.empty((n, I, H // div), dtype=qt, device=device),
                   torch.empty((n, I, H // div), dtype=qt, device=device),
                   torch.empty((n, H, I // div), dtype=qt, device=device),
                   torch.empty((n, I), dtype=f32, device=device), torch.empty((n, I), dtype=f32, device=device),
                   torch.empty((n, H), dtype=f32, device=device), weight_bits)

    def c(self) -> CLayer:
        return CLayer(self.H, self.I, self.E, self.top_k, self.n_group, self.topk_group, self.has_shared,
                      self.route_scale, *(t.data_ptr() for t in (
                          self.router_w, self.router_b, self.gate_q, self.up_q, self.down_q,
                          self.gate_s, self.up_s, self.down_s)), self.weight_bits, self.group_size)

    @property
    def expert_bytes(self) -> int:
        codes = 3 * self.H * self.I * self.weight_bits // 8
        if self.group_size:
            return codes + 4 * 3 * self.H * self.I // self.group_size
        return codes + 4 * (2 * self.I + self.H)


@dataclass
class DenseMLP:
    """Device tensors of one dense SwiGLU MLP plus the C struct that points at them."""
    H: int
    I: int
    gate_q: torch.Tensor     # [I][H/2] u8 (int4) or [I][H] i8 (int8)
    up_q: torch.Tensor
    down_q: torch.Tensor     # [H][I/2] u8 (int4) or [H][I] i8 (int8)
    gate_s: torch.Tensor     # [I] f32
    up_s: torch.Tensor
    down_s: torch.Tensor     # [H] f32
    weight_bits: int = 4

    @classmethod
    def empty(cls, H, I, device="cuda", weight_bits=4):
        f32 = torch.float32
        qt, div = (torch.int8, 1) if weight_bits == 8 else (torch.uint8, 2)
        return cls(H, I, torch.empty((I, H // div), dtype=qt, device=device),
                   torch.empty((I, H // div), dtype=qt, device=device),
                   torch.empty((H, I // div), dtype=qt, device=device),
                   torch.empty(I, dtype=f32, device=device), torch.empty(I, dtype=f32, device=device),
                   torch.empty(H, dtype=f32, device=device), weight_bits)

    def c(self) -> CDense:
        return CDense(self.H, self.I, self.weight_bits, *(t.data_ptr() for t in (
            self.gate_q, self.up_q, self.down_q, self.gate_s, self.up_s, self.down_s)))

    @property
    def nbytes(self) -> int:
        return 3 * self.H * self.I * self.weight_bits // 8 + 4 * (2 * self.I + self.H)


def dense_workspace(mlp: DenseMLP, T: int, stream=None) -> torch.Tensor:
    cm = mlp.c()
    n = lib().coli_dense_workspace_bytes(ctypes.byref(cm), T)
    if n == 0:
        raise ColiError("coli_dense_workspace_bytes", _lib.COLI_EINVAL)
    ws = torch.empty(n, dtype=torch.uint8, device=mlp.gate_q.device)
    check("coli_moe_workspace_init", lib().coli_moe_workspace_init(_ptr(ws), n, _stream(stream)))
    return ws


def dense_forward(mlp: DenseMLP, x: torch.Tensor, ws: torch.Tensor, y: Optional[torch.Tensor] = None,
                  flags: int = 0, gamma: Optional[torch.Tensor] = None, eps: float = 1e-6, stream=None,
                  c_mlp: Optional[CDense] = None) -> torch.Tensor:
    """y (+)= MLP(x), or MLP(RMSNorm(x) * gamma) when gamma is given (y may be x)."""
    _dev(x, torch.float32, "x")
    if gamma is not None:
        _dev(gamma, torch.float32, "gamma")
    T = x.shape[0]
    if y is None:
        y = torch.empty_like(x)
    cm = c_mlp if c_mlp is not None else mlp.c()
    check("coli_dense_forward", lib().coli_dense_forward(ctypes.byref(cm), _ptr(x), _ptr(gamma), eps, T, _ptr(y),
                                                         flags, _ptr(ws), ws.numel(), _stream(stream)))
    return y


def version() -> str:
    return lib().coli_version().decode()


def quant_act_q8(x: torch.Tensor, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    _dev(x, torch.float32, "x")
    T, H = x.shape
    xq = torch.empty((T, H), dtype=torch.int8, device=x.device)
    xs = torch.empty((T, H // 32), dtype=torch.float32, device=x.device)
    check("coli_quant_act_q8", lib().coli_quant_act_q8(_ptr(x), T, H, _ptr(xq), _ptr(xs), _stream(stream)))
    return xq, xs


def workspace_bytes(layer: MoELayer, T: int) -> int:
    cl = layer.c()
    return int(lib().coli_moe_workspace_bytes(ctypes.byref(cl), T))


def workspace(layer: MoELayer, T: int, stream=None) -> torch.Tensor:
    n = workspace_bytes(layer, T)
    if n == 0:
        raise ColiError("coli_moe_workspace_bytes", -1)
    ws = torch.empty(n, dtype=torch.uint8, device=layer.router_w.device)
    check("coli_moe_workspace_init", lib().coli_moe_workspace_init(_ptr(ws), n, _stream(stream)))
    return ws


def workspace_layout(layer: MoELayer, T: int, flags: int = 0) -> CWsLayout:
    cl = layer.c()
    out = CWsLayout()
    check("coli_moe_workspace_layout", lib().coli_moe_workspace_layout(ctypes.byref(cl), T, flags, ctypes.byref(out)))
    return out


def moe_route(layer: MoELayer, x: torch.Tensor, ws: torch.Tensor, stream=None):
    _dev(x, torch.float32, "x")
    T = x.shape[0]
    idx = torch.empty((T, layer.top_k), dtype=torch.int32, device=x.device)
    w = torch.empty((T, layer.top_k), dtype=torch.float32, device=x.device)
    cl = layer.c()
    check("coli_moe_route", lib().coli_moe_route(ctypes.byref(cl), _ptr(x), T, _ptr(idx), _ptr(w), _ptr(ws),
                                                 ws.numel(), _stream(stream)))
    return idx, w


def moe_forward(layer: MoELayer, x: torch.Tensor, ws: torch.Tensor, y: Optional[torch.Tensor] = None,
                flags: int = 0, stream=None, c_layer: Optional[CLayer] = None) -> torch.Tensor:
    _dev(x, torch.float32, "x")
    T = x.shape[0]
    if y is None:
        y = torch.empty_like(x)
    cl = c_layer if c_layer is not None else layer.c()
    check("coli_moe_forward", lib().coli_moe_forward(ctypes.byref(cl), _ptr(x), T, _ptr(y), flags, _ptr(ws),
                                                     ws.numel(), _stream(stream)))
    return y


def moe_forward_noalloc(layer: MoELayer, x: torch.Tensor, y: torch.Tensor, flags: int = 0, stream=None,
                        c_layer: Optional[CLayer] = None) -> torch.Tensor:
    """coli_moe_forward on the library's own device scratch (no workspace, no
    allocation: the caller passes the output y)."""
    _dev(x, torch.float32, "x"); _dev(y, torch.float32, "y")
    cl = c_layer if c_layer is not None else layer.c()
    check("coli_moe_forward_noalloc", lib().coli_moe_forward_noalloc(ctypes.byref(cl), _ptr(x), x.shape[0], _ptr(y),
                                                                     flags, _stream(stream)))
    return y


def moe_forward_rms(layer: MoELayer, x: torch.Tensor, gamma: torch.Tensor, eps: float, ws: torch.Tensor,
                    y: Optional[torch.Tensor] = None, flags: int = 0, stream=None,
                    c_layer: Optional[CLayer] = None) -> torch.Tensor:
    """y (+)= MoE(RMSNorm(x) * gamma) in one call (y may be x: the residual add in place)."""
    _dev(x, torch.float32, "x"); _dev(gamma, torch.float32, "gamma")
    T = x.shape[0]
    if y is None:
        y = torch.empty_like(x)
    cl = c_layer if c_layer is not None else layer.c()
    check("coli_moe_forward_rms", lib().coli_moe_forward_rms(ctypes.byref(cl), _ptr(x), _ptr(gamma), eps, T,
                                                             _ptr(y), flags, _ptr(ws), ws.numel(),
                                                             _stream(stream)))
    return y


class KernelEvents:
    """Start/stop event pairs (HIP events with timing) for coli_moe_forward_timed."""

    def __init__(self, n: int = 16):
        self._hip = ctypes.CDLL("libamdhip64.so")
        self._hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self._hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self._hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.n = n
        self.start = (ctypes.c_void_p * n)()
        self.stop = (ctypes.c_void_p * n)()
        for arr in (self.start, self.stop):
            for i in range(n):
                e = ctypes.c_void_p()
                if self._hip.hipEventCreate(ctypes.byref(e)) != 0:
                    raise RuntimeError("hipEventCreate failed")
                arr[i] = e
        self.names = (ctypes.c_char_p * n)()
        self.count = ctypes.c_int(0)

    def durations_ms(self):
        """(kernel name, ms) of each timed launch of the last call (waits for them)."""
        out = []
        for i in range(min(self.n, self.count.value)):
            self._hip.hipEventSynchronize(self.stop[i])
            f = ctypes.c_float()
            if self._hip.hipEventElapsedTime(ctypes.byref(f), self.start[i], self.stop[i]) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            out.append((self.names[i].decode(), f.value))
        return out

    def __del__(self):
        try:
            for arr in (self.start, self.stop):
                for e in arr:
                    if e:
                        self._hip.hipEventDestroy(e)
        except Exception:
            pass


class kernel_timer:
    """Context manager: every library launch inside the block records its own
    start/stop in `events` (coli_timer_begin / coli_timer_end)."""

    def __init__(self, events: KernelEvents):
        self.events = events

    def __enter__(self):
        check("coli_timer_begin", lib().coli_timer_begin(self.events.start, self.events.stop, self.events.n,
                                                         self.events.names))
        return self.events

    def __exit__(self, *exc):
        check("coli_timer_end", lib().coli_timer_end(ctypes.byref(self.events.count)))
        return False


def moe_forward_timed(layer: MoELayer, x: torch.Tensor, ws: torch.Tensor, events: KernelEvents,
                      y: Optional[torch.Tensor] = None, flags: int = 0, stream=None,
                      c_layer: Optional[CLayer] = None, gamma: Optional[torch.Tensor] = None,
                      eps: float = 1e-6) -> torch.Tensor:
    """moe_forward (or moe_forward_rms with gamma) with every launch's own
    start/stop in `events` (events.durations_ms() reads them after the stream
    has run)."""
    _dev(x, torch.float32, "x")
    if gamma is not None:
        _dev(gamma, torch.float32, "gamma")
    T = x.shape[0]
    if y is None:
        y = torch.empty_like(x)
    cl = c_layer if c_layer is not None else layer.c()
    check("coli_moe_forward_timed",
          lib().coli_moe_forward_timed(ctypes.byref(cl), _ptr(x), _ptr(gamma), eps, T, _ptr(y), flags, _ptr(ws),
                                       ws.numel(),
                                       _stream(stream), events.start, events.stop, events.n,
                                       ctypes.byref(events.count), events.names))
    return y


def moe_experts(layer: MoELayer, xq: torch.Tensor, xs: torch.Tensor, idx: torch.Tensor, w: torch.Tensor,
                ws: torch.Tensor, y: Optional[torch.Tensor] = None, flags: int = 0, stream=None) -> torch.Tensor:
    _dev(xq, torch.int8, "xq"); _dev(xs, torch.float32, "xs")
    _dev(idx, torch.int32, "idx"); _dev(w, torch.float32, "w")
    T = xq.shape[0]
    if y is None:
        y = torch.empty((T, layer.H), dtype=torch.float32, device=xq.device)
    cl = layer.c()
    check("coli_moe_experts", lib().coli_moe_experts(ctypes.byref(cl), _ptr(xq), _ptr(xs), _ptr(idx), _ptr(w), T,
                                                     _ptr(y), flags, _ptr(ws), ws.numel(), _stream(stream)))
    return y


def rmsnorm(x: torch.Tensor, gamma: torch.Tensor, eps: float = 1e-6, out: Optional[torch.Tensor] = None,
            stream=None) -> torch.Tensor:
    _dev(x, torch.float32, "x"); _dev(gamma, torch.float32, "gamma")
    T, H = x.shape
    if out is None:
        out = torch.empty_like(x)
    check("coli_rmsnorm", lib().coli_rmsnorm(_ptr(x), _ptr(gamma), T, H, eps, _ptr(out), _stream(stream)))
    return out


def pack_int4_rows(w: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Host packer (synchronous, host memory)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, cols = w.shape
    q = np.empty((rows, cols // 2), dtype=np.uint8)
    s = np.empty(rows, dtype=np.float32)
    check("coli_pack_int4_rows", lib().coli_pack_int4_rows(ctypes.c_void_p(w.ctypes.data), rows, cols,
                                                           ctypes.c_void_p(q.ctypes.data),
                                                           ctypes.c_void_p(s.ctypes.data)))
    return q, s


def pack_int4_rows_dev(w: torch.Tensor, q: torch.Tensor, s: torch.Tensor, stream=None) -> None:
    _dev(w, torch.float32, "w")
    rows, cols = w.shape
    check("coli_pack_int4_rows_dev", lib().coli_pack_int4_rows_dev(_ptr(w), rows, cols, _ptr(q), _ptr(s),
                                                                   _stream(stream)))


def pack_int2_rows_dev(w: torch.Tensor, q: torch.Tensor, s: torch.Tensor, stream=None) -> None:
    """int2 codes (the library's column order, four per byte) and f32 row scales (device)."""
    _dev(w, torch.float32, "w")
    rows, cols = w.shape
    check("coli_pack_int2_rows_dev", lib().coli_pack_int2_rows_dev(_ptr(w), rows, cols, _ptr(q), _ptr(s),
                                                                   _stream(stream)))


def pack_int4_groups_dev(w: torch.Tensor, group: int, q: torch.Tensor, s: torch.Tensor, stream=None) -> None:
    """int4 codes and one f32 scale per group of `group` columns of each row (device)."""
    _dev(w, torch.float32, "w")
    rows, cols = w.shape
    check("coli_pack_int4_groups_dev", lib().coli_pack_int4_groups_dev(_ptr(w), rows, cols, group, _ptr(q), _ptr(s),
                                                                       _stream(stream)))


def pack_int8_rows(w: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Host int8 packer (synchronous, host memory); the library's int8 layout."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, cols = w.shape
    q = np.empty((rows, cols), dtype=np.int8)
    s = np.empty(rows, dtype=np.float32)
    check("coli_pack_int8_rows", lib().coli_pack_int8_rows(ctypes.c_void_p(w.ctypes.data), rows, cols,
                                                           ctypes.c_void_p(q.ctypes.data),
                                                           ctypes.c_void_p(s.ctypes.data)))
    return q, s


def pack_int8_rows_dev(w: torch.Tensor, q: torch.Tensor, s: torch.Tensor, stream=None) -> None:
    _dev(w, torch.float32, "w")
    rows, cols = w.shape
    check("coli_pack_int8_rows_dev", lib().coli_pack_int8_rows_dev(_ptr(w), rows, cols, _ptr(q), _ptr(s),
                                                                   _stream(stream)))


def debug_block_dots(q4: torch.Tensor, q8: torch.Tensor, stream=None) -> torch.Tensor:
    _dev(q4, torch.uint8, "q4"); _dev(q8, torch.int8, "q8")
    rows, half = q4.shape
    S = torch.empty((rows, 2 * half // 32), dtype=torch.int32, device=q4.device)
    check("coli_debug_block_dots", lib().coli_debug_block_dots(_ptr(q4), _ptr(q8), rows, 2 * half, _ptr(S),
                                                               _stream(stream)))
    return S
