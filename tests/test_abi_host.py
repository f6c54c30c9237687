"""Host-side checks of the C ABI (no GPU): the library loads and exports every
function include/coli_moe.h declares, argument validation returns its status
codes before anything is launched, workspace sizing, and the host int4 packer
produces the oracle packer's bytes."""
import ctypes
import os
import re

import numpy as np
import pytest

from int4_quantized_expert_sigmoid_amd import _lib
from int4_quantized_expert_sigmoid_amd._lib import CLayer, CWsLayout, lib
from oracle import oracle as O
from synth import synth as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(coli_\w+)\s*\(", text, flags=re.M))
    return names


def test_library_exports_every_declared_function():
    names = header_functions()
    assert {"coli_moe_route", "coli_quant_act_q8", "coli_moe_forward"} <= names
    L = lib()
    for n in sorted(names):
        assert hasattr(L, n), n
    assert set(_lib.EXPORTS) == names
    assert b"gfx950" in L.coli_version()


def fake_layer(H=6144, I=2048, E=256, k=8, **kw):
    p = 1 << 20     # aligned dummy address: never dereferenced by the checks below
    args = dict(H=H, I=I, E=E, top_k=k, n_group=1, topk_group=1, has_shared=1, route_scale=1.0)
    args.update(kw)
    L = CLayer(args["H"], args["I"], args["E"], args["top_k"], args["n_group"], args["topk_group"],
               args["has_shared"], args["route_scale"], p, p, p, p, p, p, p, p)
    L.weight_bits = args.get("weight_bits", 4)
    L.group_size = args.get("group_size", 0)
    return L


def ws_bytes(layer, T):
    return lib().coli_moe_workspace_bytes(ctypes.byref(layer), T)


def test_workspace_sizes():
    L = fake_layer()
    b1 = ws_bytes(L, 1)
    assert 0 < b1 < 8 * 2 ** 20
    b512 = ws_bytes(L, 512)
    n_pairs = 512 * 8 + 512
    assert b512 >= n_pairs * (6144 + 2048) * 4       # per-pair h and y
    assert ws_bytes(fake_layer(H=100), 1) == 0        # H not a multiple of 32
    assert ws_bytes(L, 0) == 0


@pytest.mark.parametrize("bad", [
    dict(H=48), dict(I=40), dict(E=0), dict(E=600), dict(top_k=0), dict(top_k=17), dict(top_k=9, E=8),
    dict(n_group=3), dict(n_group=8, topk_group=9), dict(n_group=8, topk_group=1, top_k=33),
    dict(has_shared=2), dict(route_scale=float("nan")), dict(weight_bits=5), dict(weight_bits=16),
    dict(group_size=16), dict(group_size=48), dict(group_size=96), dict(group_size=-32),
    dict(group_size=4096), dict(group_size=32, weight_bits=8), dict(group_size=64, I=2080),
    dict(group_size=32, weight_bits=2), dict(weight_bits=1), dict(weight_bits=3),
])
def test_invalid_layers_rejected(bad):
    L = fake_layer(**bad)
    p = ctypes.c_void_p(1 << 20)
    assert ws_bytes(L, 1) == 0
    rc = lib().coli_moe_forward(ctypes.byref(L), p, 1, p, 0, p, 1 << 30, None)
    assert rc == _lib.COLI_EINVAL


def test_forward_argument_errors_before_launch():
    L = fake_layer()
    p = ctypes.c_void_p(1 << 20)
    F = lib().coli_moe_forward
    assert F(ctypes.byref(L), p, 0, p, 0, p, 1 << 30, None) == _lib.COLI_EINVAL          # T = 0
    assert F(ctypes.byref(L), p, 70000, p, 0, p, 1 << 40, None) == _lib.COLI_EINVAL      # T > max
    assert F(ctypes.byref(L), p, 1, p, 64, p, 1 << 30, None) == _lib.COLI_EINVAL         # unknown flag
    assert F(ctypes.byref(L), p, 1, p, 6, p, 1 << 30, None) == _lib.COLI_EINVAL          # two paths
    assert F(ctypes.byref(L), p, 9, p, 2, p, 1 << 30, None) == _lib.COLI_EINVAL          # GEMV needs T <= 8
    assert F(ctypes.byref(L), p, 1, p, 8, p, 1 << 30, None) == _lib.COLI_EINVAL          # unknown flag 8
    assert F(ctypes.byref(L), ctypes.c_void_p((1 << 20) + 4), 1, p, 0, p, 1 << 30, None) == _lib.COLI_EINVAL
    assert F(ctypes.byref(L), p, 1, p, 0, p, 100, None) == _lib.COLI_EWORKSPACE
    assert F(None, p, 1, p, 0, p, 1 << 30, None) == _lib.COLI_EINVAL
    R = lib().coli_moe_route
    assert R(ctypes.byref(L), p, 1, p, p, p, 10, None) == _lib.COLI_EWORKSPACE
    Q = lib().coli_quant_act_q8
    assert Q(p, 1, 100, p, p, None) == _lib.COLI_EINVAL
    assert Q(p, 0, 64, p, p, None) == _lib.COLI_EINVAL
    N = lib().coli_rmsnorm
    assert N(p, p, 1, 64, ctypes.c_float(-1.0), p, None) == _lib.COLI_EINVAL
    D = lib().coli_debug_block_dots
    assert D(p, p, 4, 48, p, None) == _lib.COLI_EINVAL


def test_rms_forward_argument_errors_before_launch():
    L = fake_layer()
    p = ctypes.c_void_p(1 << 20)
    R = lib().coli_moe_forward_rms
    f = ctypes.c_float
    assert R(ctypes.byref(L), p, None, f(1e-6), 1, p, 0, p, 1 << 30, None) == _lib.COLI_EINVAL      # no gamma
    assert R(ctypes.byref(L), p, ctypes.c_void_p((1 << 20) + 4), f(1e-6), 1, p, 0, p, 1 << 30, None) \
        == _lib.COLI_EINVAL                                                                      # misaligned gamma
    assert R(ctypes.byref(L), p, p, f(-1.0), 1, p, 0, p, 1 << 30, None) == _lib.COLI_EINVAL         # eps < 0
    assert R(ctypes.byref(L), p, p, f(float("nan")), 1, p, 0, p, 1 << 30, None) == _lib.COLI_EINVAL
    assert R(ctypes.byref(L), p, p, f(1e-6), 0, p, 0, p, 1 << 30, None) == _lib.COLI_EINVAL         # T = 0
    assert R(ctypes.byref(L), p, p, f(1e-6), 1, p, 0, p, 100, None) == _lib.COLI_EWORKSPACE


def test_timer_scope_errors():
    L = lib()
    ev = (ctypes.c_void_p * 2)(1 << 20, 1 << 20)     # stand-ins: nothing is launched in the scope
    nul = (ctypes.c_void_p * 2)(1 << 20, None)
    n = ctypes.c_int(-1)
    assert L.coli_timer_end(ctypes.byref(n)) == _lib.COLI_EINVAL             # no open scope
    assert L.coli_timer_begin(ev, ev, 0, None) == _lib.COLI_EINVAL
    assert L.coli_timer_begin(ev, nul, 2, None) == _lib.COLI_EINVAL
    assert L.coli_timer_begin(None, ev, 2, None) == _lib.COLI_EINVAL
    assert L.coli_timer_begin(ev, ev, 2, None) == _lib.COLI_OK
    assert L.coli_timer_begin(ev, ev, 2, None) == _lib.COLI_EINVAL           # one scope at a time
    assert L.coli_timer_end(None) == _lib.COLI_EINVAL
    assert L.coli_timer_end(ctypes.byref(n)) == _lib.COLI_OK
    assert n.value == 0
    assert L.coli_timer_end(ctypes.byref(n)) == _lib.COLI_EINVAL


def test_timed_forward_argument_errors_before_launch():
    L = fake_layer()
    p = ctypes.c_void_p(1 << 20)
    TM = lib().coli_moe_forward_timed
    ev = (ctypes.c_void_p * 4)(*([1 << 20] * 4))           # non-null stand-ins: nothing is launched
    nul = (ctypes.c_void_p * 4)(1 << 20, None, 1 << 20, 1 << 20)
    n = ctypes.c_int(-7)
    assert TM(ctypes.byref(L), p, None, ctypes.c_float(0.0), 1, p, 0, p, 1 << 30, None, ev, ev, 4, None, None) == _lib.COLI_EINVAL
    assert TM(ctypes.byref(L), p, None, ctypes.c_float(0.0), 1, p, 0, p, 1 << 30, None, ev, ev, -1, ctypes.byref(n), None) == _lib.COLI_EINVAL
    assert TM(ctypes.byref(L), p, None, ctypes.c_float(0.0), 1, p, 0, p, 1 << 30, None, ev, nul, 4, ctypes.byref(n), None) == _lib.COLI_EINVAL
    assert TM(ctypes.byref(L), p, None, ctypes.c_float(0.0), 1, p, 0, p, 1 << 30, None, None, None, 2, ctypes.byref(n), None) == _lib.COLI_EINVAL
    # a layer call rejected before launching: no launch counted
    assert TM(ctypes.byref(L), p, None, ctypes.c_float(0.0), 0, p, 0, p, 1 << 30, None, ev, ev, 4, ctypes.byref(n), None) == _lib.COLI_EINVAL
    assert n.value == 0
    assert TM(ctypes.byref(L), p, None, ctypes.c_float(0.0), 1, p, 0, p, 100, None, ev, ev, 4, ctypes.byref(n), None) == _lib.COLI_EWORKSPACE
    assert n.value == 0


def test_workspace_layout_paths():
    L = fake_layer()
    out = CWsLayout()
    assert lib().coli_moe_workspace_layout(ctypes.byref(L), 1, 0, ctypes.byref(out)) == 0
    assert out.path == 0 and out.n_pairs_max == (8 + 1) * 8
    assert lib().coli_moe_workspace_layout(ctypes.byref(L), 512, 0, ctypes.byref(out)) == 0
    assert out.path == 1 and out.n_pairs_max == 512 * 9
    assert lib().coli_moe_workspace_layout(ctypes.byref(L), 4, _lib.COLI_PATH_GROUPED, ctypes.byref(out)) == 0
    assert out.path == 1
    assert lib().coli_moe_workspace_layout(ctypes.byref(L), 8, 0, ctypes.byref(out)) == 0
    assert out.path == 0 and out.ye % 256 == 0
    for f in ("xq", "xs", "idx", "w", "h", "hq", "hs", "ye"):
        assert getattr(out, f) % 256 == 0


def host_pack(w):
    w = np.ascontiguousarray(w, np.float32)
    q = np.empty((w.shape[0], w.shape[1] // 2), np.uint8)
    s = np.empty(w.shape[0], np.float32)
    rc = lib().coli_pack_int4_rows(ctypes.c_void_p(w.ctypes.data), w.shape[0], w.shape[1],
                                   ctypes.c_void_p(q.ctypes.data), ctypes.c_void_p(s.ctypes.data))
    assert rc == 0
    return q, s


def test_host_packer_matches_oracle_packer():
    w = S.expert_matrix(S.GLM52, 0, 0, 7, S.DOWN)
    q, s = host_pack(w)
    qo, so = O.pack_int4_rows(w)
    assert np.array_equal(q, qo) and np.array_equal(s, so)
    edge = np.zeros((4, 64), np.float32)
    edge[1, :] = 1e-40                      # subnormal row: 1/d overflows
    edge[2, 5] = -3.5                       # single nonzero
    edge[3, :] = np.linspace(-7, 7, 64)     # ties at .5 after scaling
    q, s = host_pack(edge)
    qo, so = O.pack_int4_rows(edge)
    assert np.array_equal(q, qo) and np.array_equal(s, so)


def test_int8_experts_take_both_paths():
    """int8 experts have token-GEMV and grouped kernels: the layout of a
    large or forced-grouped batch is the grouped one, as for int4 (no launch
    here: the pointers are dummies)."""
    L = fake_layer(weight_bits=8)
    out = CWsLayout()
    assert ws_bytes(L, 4) > 0 and ws_bytes(L, 512) == ws_bytes(fake_layer(), 512)
    assert lib().coli_moe_workspace_layout(ctypes.byref(L), 512, 0, ctypes.byref(out)) == 0
    assert out.path == 1
    assert lib().coli_moe_workspace_layout(ctypes.byref(L), 4, _lib.COLI_PATH_GROUPED, ctypes.byref(out)) == 0
    assert out.path == 1
    assert lib().coli_moe_workspace_layout(ctypes.byref(L), 4, 0, ctypes.byref(out)) == 0
    assert out.path == 0


def test_group_scales_take_both_paths():
    """Group-scaled int4 experts: valid groups are accepted (workspace sized)
    and, like every format, have token-GEMV and grouped kernels: a large or
    forced-grouped batch gets the grouped layout (no launch here)."""
    for G in (32, 64, 128, 256, 2048):
        assert ws_bytes(fake_layer(group_size=G), 4) > 0, G
    L = fake_layer(group_size=32)
    out = CWsLayout()
    assert lib().coli_moe_workspace_layout(ctypes.byref(L), 512, 0, ctypes.byref(out)) == 0
    assert out.path == 1
    assert lib().coli_moe_workspace_layout(ctypes.byref(L), 4, _lib.COLI_PATH_GROUPED, ctypes.byref(out)) == 0
    assert out.path == 1

def test_int2_experts_take_both_paths():
    """int2 experts have token-GEMV and grouped kernels: the layout of a
    large or forced-grouped batch is the grouped one (no launch here)."""
    L = fake_layer(weight_bits=2)
    p = ctypes.c_void_p(1 << 20)
    out = CWsLayout()
    assert ws_bytes(L, 4) > 0
    assert lib().coli_moe_workspace_layout(ctypes.byref(L), 512, 0, ctypes.byref(out)) == 0
    assert out.path == 1
    assert lib().coli_moe_workspace_layout(ctypes.byref(L), 4, _lib.COLI_PATH_GROUPED, ctypes.byref(out)) == 0
    assert out.path == 1
    P = lib().coli_pack_int2_rows_dev
    for rows, cols in ((0, 64), (4, 48), (4, 16)):
        assert P(p, rows, cols, p, p, None) == _lib.COLI_EINVAL
    assert P(p, 4, 64, ctypes.c_void_p((1 << 20) + 8), p, None) == _lib.COLI_EINVAL      # q not 16-byte aligned


def test_group_packer_argument_errors():
    P = lib().coli_pack_int4_groups_dev
    p = ctypes.c_void_p(1 << 20)
    for rows, cols, G in ((0, 64, 32), (4, 64, 3), (4, 64, 0), (4, 96, 64), (4, 32, 64), (4, 8192, 8192)):
        assert P(p, rows, cols, G, p, p, None) == _lib.COLI_EINVAL, (rows, cols, G)
    assert P(None, 4, 64, 32, p, p, None) == _lib.COLI_EINVAL


def _perm8(j):
    return 4 + (j >> 1) if j & 1 else j >> 1


def int8_positions(cols):
    """Byte of column c in a library int8 row: the 8-group order 0,2,4,6,1,3,5,7
    inside its block, then the block halves split (all first halves, then all
    second halves)."""
    p = np.array([(c & 31 & ~7) + _perm8(c & 7) for c in range(cols)])
    b = np.arange(cols) >> 5
    return (p >> 4) * 16 * (cols // 32) + b * 16 + (p & 15)


def test_host_int8_packer_matches_oracle_in_library_layout():
    w = S.expert_matrix(S.LayerSpec(H=256, I=128, E=4, top_k=1), 0, 0, 1, S.GATE)
    edge = np.zeros((4, 96), np.float32)
    edge[1, :] = 1e-40                      # subnormal row: 1/d overflows
    edge[2, 5] = -3.5                       # single nonzero
    edge[3, :] = np.linspace(-127, 127, 96) # ties at .5 after scaling
    for m in (w, edge):
        rows, cols = m.shape
        q = np.empty((rows, cols), np.int8)
        s = np.empty(rows, np.float32)
        assert lib().coli_pack_int8_rows(ctypes.c_void_p(m.ctypes.data), rows, cols, ctypes.c_void_p(q.ctypes.data),
                                         ctypes.c_void_p(s.ctypes.data)) == 0
        qo, so = O.pack_int8_rows(m)
        pos = int8_positions(cols)
        assert sorted(pos.tolist()) == list(range(cols))
        assert np.array_equal(s, so)
        assert np.array_equal(q[:, pos], qo)       # column c of the oracle sits at byte pos[c]
    bad = np.zeros((2, 48), np.float32)
    for cols in (12, 48):
        assert lib().coli_pack_int8_rows(ctypes.c_void_p(bad.ctypes.data), 2, cols, ctypes.c_void_p(bad.ctypes.data),
                                         ctypes.c_void_p(bad.ctypes.data)) == _lib.COLI_EINVAL
