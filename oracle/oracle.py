"""ctypes wrapper of the CPU oracle (liboracle.so) with numpy conveniences.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg. The GPU library and its Python binding never
import this module.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
_LIBS = {}
_THREADED = False


def use_threads(on: bool = True) -> None:
    """Route every call through liboracle_omp.so (the same source with the
    loops over independent matrix rows spread over OpenMP threads; bit for
    bit the results of the plain build) or back to liboracle.so."""
    global _THREADED
    _THREADED = bool(on)


def threads() -> int:
    """Threads the selected build's row loops use (1 for the plain build)."""
    return int(_lib().oracle_threads())


def _lib():
    name = "liboracle_omp.so" if _THREADED else "liboracle.so"
    if name not in _LIBS:
        # COLI_LIB_VARIANT=asan: the sanitizer build of the CPU test suite
        path = os.path.join(HERE, "_asan" if os.environ.get("COLI_LIB_VARIANT") == "asan" else "", name)
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i, f = ctypes.c_int, ctypes.c_float
        L.oracle_pack_int4_rows.argtypes = [P, i, i, P, P]
        L.oracle_nibble.argtypes = [ctypes.c_uint8, i]
        L.oracle_nibble.restype = i
        L.oracle_unpack_int4_rows.argtypes = [P, P, i, i, P]
        L.oracle_quant_q8.argtypes = [P, i, P, P]
        L.oracle_block_dots.argtypes = [P, P, i, i, P]
        L.oracle_rowdot.argtypes = [P, P, P, P, i, i, P]
        L.oracle_route.argtypes = [P, P, P, i, i, i, i, i, i, f, P, P, P]
        L.oracle_route.restype = i
        L.oracle_expert.argtypes = [P, P, P, P, P, P, i, i, P, P, P, P, P, P, P, P]
        L.oracle_combine.argtypes = [P, P, i, P, i, P]
        L.oracle_rmsnorm.argtypes = [P, P, i, i, f, P]
        L.oracle_expert_dense.argtypes = [P, P, P, P, P, P, i, i, P, P]
        L.oracle_moe_forward.argtypes = [P, P, i, P, P, P]
        L.oracle_moe_forward.restype = i
        L.oracle_pack_int8_rows.argtypes = [P, i, i, P, P]
        L.oracle_block_dots_i8.argtypes = [P, P, i, i, P]
        L.oracle_rowdot_i8.argtypes = [P, P, P, P, i, i, P]
        L.oracle_expert_w.argtypes = [i, P, P, P, P, P, P, i, i, P, P, P, P, P, P, P, P]
        L.oracle_expert_dense_i8.argtypes = [P, P, P, P, P, P, i, i, P, P]
        L.oracle_pack_int4_groups.argtypes = [P, i, i, i, P, P]
        L.oracle_pack_int2_rows.argtypes = [P, i, i, P, P]
        L.oracle_crumb.argtypes = [ctypes.c_uint8, i]
        L.oracle_crumb.restype = i
        L.oracle_unpack_int2_rows.argtypes = [P, P, i, i, P]
        L.oracle_block_dots_i2.argtypes = [P, P, i, i, P]
        L.oracle_rowdot_i2.argtypes = [P, P, P, P, i, i, P]
        L.oracle_unpack_int4_groups.argtypes = [P, P, i, i, i, P]
        L.oracle_rowdot_groups.argtypes = [P, P, i, P, P, i, i, P]
        L.oracle_expert_groups.argtypes = [i, P, P, P, P, P, P, i, i, P, P, P, P, P, P, P, P]
        L.oracle_threads.restype = i
        L.oracle_expert_tokens.argtypes = [i, i, P, P, P, P, P, P, i, i, i, P, P, P, P, P, P, P, P]
        _LIBS[name] = L
    return _LIBS[name]


def _p(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ------------------------------------------------------------------ O1 / O2
def pack_int4_rows(w: np.ndarray):
    w = _c(w, np.float32)
    rows, cols = w.shape
    q = np.empty((rows, cols // 2), dtype=np.uint8)
    s = np.empty(rows, dtype=np.float32)
    _lib().oracle_pack_int4_rows(_p(w), rows, cols, _p(q), _p(s))
    return q, s


def nibble(byte: int, hi: int) -> int:
    return int(_lib().oracle_nibble(byte, hi))


def unpack_int4_rows(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    q = _c(q, np.uint8)
    s = _c(s, np.float32)
    rows, half = q.shape
    out = np.empty((rows, 2 * half), dtype=np.float64)
    _lib().oracle_unpack_int4_rows(_p(q), _p(s), rows, 2 * half, _p(out))
    return out


# ----------------------------------------------------------------------- O3
def quant_q8(x: np.ndarray):
    x = _c(x, np.float32)
    n = x.size
    q = np.empty(x.shape, dtype=np.int8)
    d = np.empty(x.shape[:-1] + (x.shape[-1] // 32,), dtype=np.float32)
    _lib().oracle_quant_q8(_p(x), n, _p(q), _p(d))
    return q, d


# ------------------------------------------------------------------ O4 / O5
def block_dots(q4: np.ndarray, q8: np.ndarray) -> np.ndarray:
    q4 = _c(q4, np.uint8)
    q8 = _c(q8, np.int8)
    rows, half = q4.shape
    S = np.empty((rows, 2 * half // 32), dtype=np.int32)
    _lib().oracle_block_dots(_p(q4), _p(q8), rows, 2 * half, _p(S))
    return S


def rowdot(q4, s4, q8, d8) -> np.ndarray:
    q4 = _c(q4, np.uint8)
    rows, half = q4.shape
    out = np.empty(rows, dtype=np.float32)
    _lib().oracle_rowdot(_p(q4), _p(_c(s4, np.float32)), _p(_c(q8, np.int8)), _p(_c(d8, np.float32)),
                         rows, 2 * half, _p(out))
    return out


# ---------------------------------------------------------------- O16 / O17
def pack_int4_groups(w: np.ndarray, group: int):
    """int4 codes (O1's byte layout) and one f32 scale per group of `group` columns."""
    w = _c(w, np.float32)
    rows, cols = w.shape
    if group < 2 or group % 2 or cols % group:
        raise ValueError("group must be even and divide the row length")
    q = np.empty((rows, cols // 2), dtype=np.uint8)
    s = np.empty((rows, cols // group), dtype=np.float32)
    _lib().oracle_pack_int4_groups(_p(w), rows, cols, group, _p(q), _p(s))
    return q, s


def unpack_int4_groups(q: np.ndarray, s: np.ndarray, group: int) -> np.ndarray:
    q = _c(q, np.uint8)
    s = _c(s, np.float32)
    rows, half = q.shape
    out = np.empty((rows, 2 * half), dtype=np.float64)
    _lib().oracle_unpack_int4_groups(_p(q), _p(s), rows, 2 * half, group, _p(out))
    return out


def rowdot_groups(q4, s4, group: int, q8, d8) -> np.ndarray:
    q4 = _c(q4, np.uint8)
    rows, half = q4.shape
    if group % 32 or (2 * half) % group:
        raise ValueError("group must be a multiple of 32 that divides the row length")
    out = np.empty(rows, dtype=np.float32)
    _lib().oracle_rowdot_groups(_p(q4), _p(_c(s4, np.float32)), group, _p(_c(q8, np.int8)),
                                _p(_c(d8, np.float32)), rows, 2 * half, _p(out))
    return out


# ---------------------------------------------------------------- O18 / O19
def pack_int2_rows(w: np.ndarray):
    """int2 codes, four per byte (element 4j+i in bits 2i..2i+1 of byte j), and f32 row scales."""
    w = _c(w, np.float32)
    rows, cols = w.shape
    if cols % 4:
        raise ValueError("cols must be a multiple of 4")
    q = np.empty((rows, cols // 4), dtype=np.uint8)
    s = np.empty(rows, dtype=np.float32)
    _lib().oracle_pack_int2_rows(_p(w), rows, cols, _p(q), _p(s))
    return q, s


def crumb(byte: int, i: int) -> int:
    return int(_lib().oracle_crumb(byte, i))


def unpack_int2_rows(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    q = _c(q, np.uint8)
    rows, quarter = q.shape
    out = np.empty((rows, 4 * quarter), dtype=np.float64)
    _lib().oracle_unpack_int2_rows(_p(q), _p(_c(s, np.float32)), rows, 4 * quarter, _p(out))
    return out


def block_dots_i2(q2: np.ndarray, q8: np.ndarray) -> np.ndarray:
    q2 = _c(q2, np.uint8)
    rows, quarter = q2.shape
    S = np.empty((rows, 4 * quarter // 32), dtype=np.int32)
    _lib().oracle_block_dots_i2(_p(q2), _p(_c(q8, np.int8)), rows, 4 * quarter, _p(S))
    return S


def rowdot_i2(q2, s2, q8, d8) -> np.ndarray:
    q2 = _c(q2, np.uint8)
    rows, quarter = q2.shape
    out = np.empty(rows, dtype=np.float32)
    _lib().oracle_rowdot_i2(_p(q2), _p(_c(s2, np.float32)), _p(_c(q8, np.int8)), _p(_c(d8, np.float32)),
                            rows, 4 * quarter, _p(out))
    return out


# ---------------------------------------------------------------- O11 - O13
def pack_int8_rows(w: np.ndarray):
    """int8 weight rows (natural element order) and their f32 scales."""
    w = _c(w, np.float32)
    rows, cols = w.shape
    q = np.empty((rows, cols), dtype=np.int8)
    s = np.empty(rows, dtype=np.float32)
    _lib().oracle_pack_int8_rows(_p(w), rows, cols, _p(q), _p(s))
    return q, s


def block_dots_i8(qw: np.ndarray, q8: np.ndarray) -> np.ndarray:
    qw = _c(qw, np.int8)
    q8 = _c(q8, np.int8)
    rows, cols = qw.shape
    S = np.empty((rows, cols // 32), dtype=np.int32)
    _lib().oracle_block_dots_i8(_p(qw), _p(q8), rows, cols, _p(S))
    return S


def rowdot_i8(qw, sw, q8, d8) -> np.ndarray:
    qw = _c(qw, np.int8)
    rows, cols = qw.shape
    out = np.empty(rows, dtype=np.float32)
    _lib().oracle_rowdot_i8(_p(qw), _p(_c(sw, np.float32)), _p(_c(q8, np.int8)), _p(_c(d8, np.float32)),
                            rows, cols, _p(out))
    return out


# ----------------------------------------------------------------------- O6
def route(W, b, x, top_k: int, n_group: int = 1, topk_group: int = 1, route_scale: float = 1.0,
          want_keys: bool = False):
    W = _c(W, np.float32)
    b = _c(b, np.float32)
    x = _c(np.atleast_2d(x), np.float32)
    E, H = W.shape
    T = x.shape[0]
    idx = np.empty((T, top_k), dtype=np.int32)
    w = np.empty((T, top_k), dtype=np.float32)
    keys = np.empty((T, E), dtype=np.float64) if want_keys else None
    rc = _lib().oracle_route(_p(W), _p(b), _p(x), T, H, E, top_k, n_group, topk_group,
                             route_scale, _p(idx), _p(w), _p(keys))
    if rc != 0:
        raise ValueError("oracle_route rejected its arguments")
    return (idx, w, keys) if want_keys else (idx, w)


# ----------------------------------------------------------------------- O7
@dataclass
class ExpertOut:
    y: np.ndarray
    g: np.ndarray
    u: np.ndarray
    h: np.ndarray
    hq: np.ndarray
    hs: np.ndarray


def _wbits(q) -> int:
    """Weight format from the packed array's dtype: int8 rows, or uint8 bytes
    of int4 pairs (int2 bytes are uint8 too: callers name them, wbits=2)."""
    return 8 if np.asarray(q).dtype == np.int8 else 4


def expert(gate_q, gate_s, up_q, up_s, down_q, down_s, xq, xs, group: int = 0, wbits: int = 0) -> ExpertOut:
    """O7 (int4 rows, uint8 [I][H/2]), its int8 form (int8 rows [I][H]) or its
    int2 form (wbits=2, uint8 [I][H/4]); with group > 0,
    int4 rows with O16 group scales (gate/up [I][H/group], down [H][I/group])."""
    wb = wbits or _wbits(gate_q)
    dt = np.int8 if wb == 8 else np.uint8
    gate_q = _c(gate_q, dt)
    I, Hc = gate_q.shape
    H = Hc * 8 // wb
    o = ExpertOut(y=np.empty(H, np.float32), g=np.empty(I, np.float32), u=np.empty(I, np.float32),
                  h=np.empty(I, np.float32), hq=np.empty(I, np.int8), hs=np.empty(I // 32, np.float32))
    tail = (H, I, _p(_c(xq, np.int8)), _p(_c(xs, np.float32)), _p(o.y), _p(o.g), _p(o.u), _p(o.h), _p(o.hq),
            _p(o.hs))
    heads = (_p(gate_q), _p(_c(gate_s, np.float32)), _p(_c(up_q, dt)), _p(_c(up_s, np.float32)), _p(_c(down_q, dt)),
             _p(_c(down_s, np.float32)))
    if group:
        if wb != 4:
            raise ValueError("group scales are an int4 format")
        _lib().oracle_expert_groups(group, *heads, *tail)
    else:
        _lib().oracle_expert_w(wb, *heads, *tail)
    return o


def expert_tokens(gate_q, gate_s, up_q, up_s, down_q, down_s, xq, xs, group: int = 0,
                  wbits: int = 0) -> ExpertOut:
    """O7 of one expert for n tokens: row t of every output is expert() on
    row t of xq [n][H] / xs [n][H/32]. With the threaded build the tokens
    run in parallel when there are enough of them, else each token's row
    loops do; either way every token's arithmetic is expert()'s."""
    wb = wbits or _wbits(gate_q)
    if group and wb != 4:
        raise ValueError("group scales are an int4 format")
    dt = np.int8 if wb == 8 else np.uint8
    gate_q = _c(gate_q, dt)
    I, Hc = gate_q.shape
    H = Hc * 8 // wb
    xq = _c(np.atleast_2d(xq), np.int8)
    xs = _c(np.atleast_2d(xs), np.float32)
    n = xq.shape[0]
    if xq.shape[1] != H or xs.shape != (n, H // 32):
        raise ValueError("xq must be [n][H] and xs [n][H/32]")
    o = ExpertOut(y=np.empty((n, H), np.float32), g=np.empty((n, I), np.float32), u=np.empty((n, I), np.float32),
                  h=np.empty((n, I), np.float32), hq=np.empty((n, I), np.int8), hs=np.empty((n, I // 32), np.float32))
    heads = [_c(gate_q, dt), _c(gate_s, np.float32), _c(up_q, dt), _c(up_s, np.float32), _c(down_q, dt),
             _c(down_s, np.float32)]
    if _THREADED and n < threads():
        for t in range(n):
            r = expert(*heads, xq[t], xs[t], group=group, wbits=wb)
            o.y[t], o.g[t], o.u[t], o.h[t], o.hq[t], o.hs[t] = r.y, r.g, r.u, r.h, r.hq, r.hs
        return o
    _lib().oracle_expert_tokens(wb, group, *[_p(a) for a in heads], H, I, n, _p(xq), _p(xs), _p(o.y), _p(o.g),
                                _p(o.u), _p(o.h), _p(o.hq), _p(o.hs))
    return o


def expert_dense(gate_q, gate_s, up_q, up_s, down_q, down_s, x) -> np.ndarray:
    """O10 / O14: dequantised weights, unquantised x and h, in double."""
    wb = _wbits(gate_q)
    dt = np.int8 if wb == 8 else np.uint8
    gate_q = _c(gate_q, dt)
    I, Hc = gate_q.shape
    H = Hc if wb == 8 else 2 * Hc
    y = np.empty(H, np.float64)
    fn = _lib().oracle_expert_dense_i8 if wb == 8 else _lib().oracle_expert_dense
    fn(_p(gate_q), _p(_c(gate_s, np.float32)), _p(_c(up_q, dt)), _p(_c(up_s, np.float32)),
       _p(_c(down_q, dt)), _p(_c(down_s, np.float32)), H, I, _p(_c(x, np.float32)), _p(y))
    return y


# ---------------------------------------------------------------------- O15
def dense_forward(gate_q, gate_s, up_q, up_s, down_q, down_s, x, gamma=None, eps: float = 1e-6) -> np.ndarray:
    """O15 [P1 s4: dense_mlp, the first layers] the dense SwiGLU MLP with the
    experts' numerics, every token, no routing: y_t = O7(weights, O3(x_t)).y,
    with x first replaced by O9's RMSNorm(x) * gamma when gamma is given."""
    x = np.atleast_2d(np.asarray(x, np.float32))
    if gamma is not None:
        x = rmsnorm(x, gamma, eps)
    y = np.empty_like(x)
    for t in range(x.shape[0]):
        xq, xs = quant_q8(x[t])
        y[t] = expert(gate_q, gate_s, up_q, up_s, down_q, down_s, xq, xs).y
    return y


# ----------------------------------------------------------------------- O8
def combine(y_routed, w, y_shared=None) -> np.ndarray:
    y_routed = _c(np.atleast_2d(y_routed), np.float32)
    k, H = y_routed.shape
    y = np.empty(H, np.float32)
    _lib().oracle_combine(_p(y_routed), _p(_c(w, np.float32)), k,
                          None if y_shared is None else _p(_c(y_shared, np.float32)), H, _p(y))
    return y


# ----------------------------------------------------------------------- O9
def rmsnorm(x, gamma, eps: float = 1e-6) -> np.ndarray:
    x = _c(np.atleast_2d(x), np.float32)
    T, H = x.shape
    out = np.empty((T, H), np.float32)
    _lib().oracle_rmsnorm(_p(x), _p(_c(gamma, np.float32)), T, H, eps, _p(out))
    return out


# --------------------------------------------------------------- whole layer
class _CLayer(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("H", "I", "E", "top_k", "n_group", "topk_group", "has_shared")] + [
        ("route_scale", ctypes.c_float),
        ("router_w", ctypes.c_void_p), ("router_b", ctypes.c_void_p),
        ("gate_q", ctypes.c_void_p), ("up_q", ctypes.c_void_p), ("down_q", ctypes.c_void_p),
        ("gate_s", ctypes.c_void_p), ("up_s", ctypes.c_void_p), ("down_s", ctypes.c_void_p),
        ("weight_bits", ctypes.c_int), ("group_size", ctypes.c_int)]


def moe_forward(layer, x):
    # weight_bits 2: gate_q/up_q [E+s][I][H/4], down_q [E+s][H][I/4] uint8 (four codes per byte)
    """layer: object with H, I, E, top_k, n_group, topk_group, has_shared, route_scale,
    weight_bits (4 if absent) and numpy arrays router_w [E][H], router_b [E],
    gate_q/up_q [E+s][I][H/2] uint8, down_q [E+s][H][I/2] uint8 (int4) or
    gate_q/up_q [E+s][I][H], down_q [E+s][H][I] int8 (int8), gate_s/up_s [E+s][I],
    down_s [E+s][H]; with group_size G > 0 (int4 only) the scales are per group
    of G columns: gate_s/up_s [E+s][I][H/G], down_s [E+s][H][I/G].
    Returns y [T][H], idx [T][k], w [T][k]."""
    x = _c(np.atleast_2d(x), np.float32)
    T = x.shape[0]
    wb = getattr(layer, "weight_bits", 4) or 4
    qt = np.int8 if wb == 8 else np.uint8
    arrs = {n: _c(getattr(layer, n), dt) for n, dt in (
        ("router_w", np.float32), ("router_b", np.float32), ("gate_q", qt), ("up_q", qt),
        ("down_q", qt), ("gate_s", np.float32), ("up_s", np.float32), ("down_s", np.float32))}
    cl = _CLayer(layer.H, layer.I, layer.E, layer.top_k, layer.n_group, layer.topk_group,
                 layer.has_shared, layer.route_scale,
                 *[arrs[n].ctypes.data for n in ("router_w", "router_b", "gate_q", "up_q", "down_q",
                                                 "gate_s", "up_s", "down_s")], wb,
                 getattr(layer, "group_size", 0))
    y = np.empty((T, layer.H), np.float32)
    idx = np.empty((T, layer.top_k), np.int32)
    w = np.empty((T, layer.top_k), np.float32)
    rc = _lib().oracle_moe_forward(ctypes.byref(cl), _p(x), T, _p(y), _p(idx), _p(w))
    if rc != 0:
        raise ValueError("oracle_moe_forward rejected its arguments")
    return y, idx, w
