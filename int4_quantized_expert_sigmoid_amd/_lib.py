"""ctypes binding of libcoli_moe.so (the C ABI in include/coli_moe.h).

Argument marshalling only: every step of the layer runs in the HIP library.
There is no CPU fallback; if the library is not built, importing the
functions raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# COLI_LIB_VARIANT=asan selects the host-sanitizer build of the CPU test suite
# (host code only, no device code: see tests/run_sanitized.py)
LIB_PATH = os.path.join(HERE, "_asan" if os.environ.get("COLI_LIB_VARIANT") == "asan" else "", "libcoli_moe.so")

COLI_OK, COLI_EINVAL, COLI_EWORKSPACE, COLI_EDEVICE, COLI_EUNSUPPORTED = 0, -1, -2, -3, -4
COLI_ACCUMULATE, COLI_PATH_GEMV, COLI_PATH_GROUPED = 1, 2, 4
COLI_GEMV_MAX_T, COLI_MAX_T, COLI_MAX_TOPK, COLI_PROFILE_EVENTS = 8, 65536, 16, 6
COLI_NOALLOC_MAX_BYTES = 32 << 20

EXPORTS = ("coli_quant_act_q8", "coli_moe_workspace_bytes", "coli_moe_workspace_init",
           "coli_moe_route", "coli_moe_forward", "coli_moe_forward_noalloc", "coli_moe_forward_profiled", "coli_moe_forward_timed", "coli_moe_forward_rms",
           "coli_dense_workspace_bytes", "coli_dense_forward", "coli_timer_begin", "coli_timer_end", "coli_moe_experts", "coli_moe_workspace_layout",
           "coli_rmsnorm", "coli_pack_int4_rows", "coli_pack_int4_rows_dev", "coli_pack_int4_groups_dev", "coli_pack_int2_rows_dev", "coli_pack_int8_rows",
           "coli_pack_int8_rows_dev", "coli_debug_block_dots", "coli_version")


class ColiError(RuntimeError):
    def __init__(self, name: str, code: int):
        names = {COLI_EINVAL: "COLI_EINVAL", COLI_EWORKSPACE: "COLI_EWORKSPACE",
                 COLI_EDEVICE: "COLI_EDEVICE", COLI_EUNSUPPORTED: "COLI_EUNSUPPORTED"}
        super().__init__(f"{name} returned {names.get(code, code)}")
        self.code = code


class CLayer(ctypes.Structure):
    """Mirror of struct coli_moe_layer."""
    _fields_ = [("H", ctypes.c_int32), ("I", ctypes.c_int32), ("E", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("n_group", ctypes.c_int32), ("topk_group", ctypes.c_int32),
                ("has_shared", ctypes.c_int32), ("route_scale", ctypes.c_float),
                ("router_w", ctypes.c_void_p), ("router_b", ctypes.c_void_p),
                ("gate_q", ctypes.c_void_p), ("up_q", ctypes.c_void_p), ("down_q", ctypes.c_void_p),
                ("gate_s", ctypes.c_void_p), ("up_s", ctypes.c_void_p), ("down_s", ctypes.c_void_p),
                ("weight_bits", ctypes.c_int32), ("group_size", ctypes.c_int32)]


class CDense(ctypes.Structure):
    """Mirror of struct coli_dense_mlp."""
    _fields_ = [("H", ctypes.c_int32), ("I", ctypes.c_int32), ("weight_bits", ctypes.c_int32),
                ("gate_q", ctypes.c_void_p), ("up_q", ctypes.c_void_p), ("down_q", ctypes.c_void_p),
                ("gate_s", ctypes.c_void_p), ("up_s", ctypes.c_void_p), ("down_s", ctypes.c_void_p)]


class CWsLayout(ctypes.Structure):
    """Mirror of struct coli_moe_ws_layout."""
    _fields_ = [(n, ctypes.c_size_t) for n in ("xq", "xs", "idx", "w", "pair_of", "shared_pair", "h", "hq",
                                                "hs", "ye", "n_pairs_max")] + [("path", ctypes.c_int32)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() "
                               "(there is no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        P, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        LP = ctypes.POINTER(CLayer)
        sig = {
            "coli_quant_act_q8": ([P, i, i, P, P, P], i),
            "coli_moe_workspace_bytes": ([LP, i], sz),
            "coli_moe_workspace_init": ([P, sz, P], i),
            "coli_moe_route": ([LP, P, i, P, P, P, sz, P], i),
            "coli_moe_forward": ([LP, P, i, P, i, P, sz, P], i),
            "coli_moe_forward_noalloc": ([LP, P, i, P, i, P], i),
            "coli_moe_forward_profiled": ([LP, P, i, P, i, P, sz, P, ctypes.POINTER(P), i], i),
            "coli_moe_forward_rms": ([LP, P, P, f, i, P, i, P, sz, P], i),
            "coli_dense_workspace_bytes": ([ctypes.POINTER(CDense), i], sz),
            "coli_timer_begin": ([ctypes.POINTER(P), ctypes.POINTER(P), i, ctypes.POINTER(ctypes.c_char_p)], i),
            "coli_timer_end": ([ctypes.POINTER(i)], i),
            "coli_dense_forward": ([ctypes.POINTER(CDense), P, P, f, i, P, i, P, sz, P], i),
            "coli_moe_forward_timed": ([LP, P, P, f, i, P, i, P, sz, P, ctypes.POINTER(P), ctypes.POINTER(P), i,
                                        ctypes.POINTER(i), ctypes.POINTER(ctypes.c_char_p)], i),
            "coli_moe_experts": ([LP, P, P, P, P, i, P, i, P, sz, P], i),
            "coli_moe_workspace_layout": ([LP, i, i, ctypes.POINTER(CWsLayout)], i),
            "coli_rmsnorm": ([P, P, i, i, f, P, P], i),
            "coli_pack_int4_rows": ([P, i, i, P, P], i),
            "coli_pack_int4_rows_dev": ([P, i, i, P, P, P], i),
            "coli_pack_int4_groups_dev": ([P, i, i, i, P, P, P], i),
            "coli_pack_int2_rows_dev": ([P, i, i, P, P, P], i),
            "coli_pack_int8_rows": ([P, i, i, P, P], i),
            "coli_pack_int8_rows_dev": ([P, i, i, P, P, P], i),
            "coli_debug_block_dots": ([P, P, i, i, P, P], i),
            "coli_version": ([], ctypes.c_char_p),
        }
        for name, (args, res) in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def check(name: str, rc: int) -> None:
    if rc != COLI_OK:
        raise ColiError(name, rc)
