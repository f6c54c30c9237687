"""GPU parity of the int8, int2 and group-scale weight formats on the
grouped MFMA path (T > 8) through the C ABI: tiny and odd-shaped layers in
full (every token and pair; the odd shape runs part-filled stages and scales
loaded one by one), the compute-bound case of full tiles, path invariance
against the token-GEMV path, the cross-format identities on the grouped
kernels (int8 or int2 layers whose codes an int4 layer holds too give the
int4 layer's outputs bit for bit), and the whole GLM-5.2-shaped Zipf
prefill (T = 512) against the threaded oracle.

Group scales: the grouped kernels compute every block term as the oracle
does, s_g * (d_b * S_b) rounded once, and sum the terms in block order, so
their results match the oracle's bit for bit as the row formats' do; the
token-GEMV kernels sum in another order, so the two paths agree within the
bar there."""
from dataclasses import replace

import numpy as np
import pytest
import torch

from int4_quantized_expert_sigmoid_amd import api, COLI_PATH_GEMV, COLI_PATH_GROUPED
from int4_quantized_expert_sigmoid_amd.synthetic import device_layer
from oracle import layers as OL
from oracle import oracle as O
from synth import synth as S

from gpu_common import dev, rel_err, ws_views
from test_gpu_grouped import _full_layer_check, _tiny_batch_check
from test_gpu_int2 import as_int4, codes_of

pytestmark = pytest.mark.gpu
TOL = 1e-4
FORMATS = [dict(weight_bits=8), dict(weight_bits=2), dict(group_size=32), dict(group_size=64),
           dict(group_size=128)]


def fmt_id(f):
    return f"int{f['weight_bits']}" if "weight_bits" in f else f"g{f['group_size']}"


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.set_device(0)


@pytest.fixture(scope="module", params=FORMATS, ids=fmt_id)
def tiny_f(request):
    spec = replace(S.TINY, **request.param)
    return spec, device_layer(spec, 0, 0), OL.full_layer(spec, 0, 0)


def label(spec):
    return f"g{spec.group_size}" if spec.group_size else f"int{spec.weight_bits}"


@pytest.mark.parametrize("T", [9, 64, 200])
def test_grouped_tiny_full_outputs(tiny_f, T):
    spec, L, ref = tiny_f
    x = S.tokens(S.TokenSpec(T=T, token_set=900 + T), spec.H, 0)
    ws = api.workspace(L, T)
    say(f"grouped {label(spec)} tiny T={T}")
    y = api.moe_forward(L, dev(x), ws).cpu().numpy()
    st = _tiny_batch_check(spec, L, ref, x, ws, y, f"{label(spec)} tiny T={T}")
    if spec.group_size:                          # the oracle's terms in the oracle's order
        assert st["h_bit_identical"] == 1.0 and st["y_bit_identical"] == 1.0


@pytest.mark.parametrize("fmt", [dict(weight_bits=8), dict(weight_bits=2), dict(group_size=32)], ids=fmt_id)
@pytest.mark.parametrize("T", [9, 40, 77])
def test_grouped_odd_shape_full_outputs(fmt, T):
    """H = 320 (10 blocks: part-filled last stages), I = 96 (3 row tiles, 3
    down blocks); neither block count is a multiple of 4, so the scales load
    one by one."""
    spec = S.LayerSpec(H=320, I=96, E=16, top_k=4, **fmt)
    L, ref = device_layer(spec, 0, 0), OL.full_layer(spec, 0, 0)
    x = S.tokens(S.TokenSpec(T=T, token_set=950 + T), spec.H, 0)
    ws = api.workspace(L, T)
    say(f"grouped {label(spec)} odd shape T={T}")
    y = api.moe_forward(L, dev(x), ws).cpu().numpy()
    _tiny_batch_check(spec, L, ref, x, ws, y, f"{label(spec)} odd T={T}")


@pytest.mark.parametrize("fmt", [dict(weight_bits=8), dict(weight_bits=2), dict(group_size=64)], ids=fmt_id)
def test_grouped_hot_experts_full_tiles(fmt):
    spec = S.LayerSpec(H=256, I=128, E=16, top_k=2, hot_experts=2, **fmt)
    L, ref = device_layer(spec, 0, 0), OL.full_layer(spec, 0, 0)
    T = 100
    x = S.tokens(S.TokenSpec(T=T, token_set=17), spec.H, 0)
    ws = api.workspace(L, T)
    y = api.moe_forward(L, dev(x), ws).cpu().numpy()
    _, idx_o, _ = O.moe_forward(ref, x)
    assert len(np.unique(idx_o)) == 2
    _tiny_batch_check(spec, L, ref, x, ws, y, f"{label(spec)} hot experts T={T}")


@pytest.mark.parametrize("T", [1, 4, 8])
def test_path_invariance(tiny_f, T):
    """The same tokens on both paths: routing bit for bit; for the row
    formats h, Q8(h) and its scales bit for bit per pair, for group scales
    (whose token-GEMV kernels sum in another order) h within 2 f32 ulps;
    outputs within the bar."""
    spec, L, _ = tiny_f
    x = S.tokens(S.TokenSpec(T=T, token_set=960 + T), spec.H, 0)
    ws = api.workspace(L, T)
    yg = api.moe_forward(L, dev(x), ws, flags=COLI_PATH_GEMV).cpu().numpy()
    vg = ws_views(L, T, ws, COLI_PATH_GEMV)
    ym = api.moe_forward(L, dev(x), ws, flags=COLI_PATH_GROUPED).cpu().numpy()
    vm = ws_views(L, T, ws, COLI_PATH_GROUPED)
    assert vg["path"] == 0 and vm["path"] == 1
    assert np.array_equal(vg["idx"], vm["idx"])
    for t in range(T):
        for j in range(spec.top_k):
            pg, pm = vg["pair_of"][t, j], vm["pair_of"][t, j]
            if spec.group_size:
                hg, hm = vg["h"][pg], vm["h"][pm]
                assert np.all(np.abs(hg - hm) <= 2 * np.spacing(np.maximum(np.abs(hg), np.abs(hm))))
            else:
                assert np.array_equal(vg["h"][pg], vm["h"][pm])
                assert np.array_equal(vg["hq"][pg], vm["hq"][pm]) and np.array_equal(vg["hs"][pg], vm["hs"][pm])
    say(f"{label(spec)} path invariance T={T}: bit-identical outputs {np.mean(yg == ym):.4f}")
    assert rel_err(ym, yg).max() <= TOL


def _int8_copy_of_int4(L4, spec):
    """An int8 layer holding the int4 layer's codes and scales, in the int8
    layout (8-groups reordered, block halves split)."""
    L8 = api.MoELayer.empty(spec.H, spec.I, spec.E, spec.top_k, weight_bits=8)
    L8.router_w.copy_(L4.router_w)
    L8.router_b.copy_(L4.router_b)
    for name in ("gate_s", "up_s", "down_s"):
        getattr(L8, name).copy_(getattr(L4, name))
    for name in ("gate_q", "up_q", "down_q"):
        b = getattr(L4, name).cpu().numpy()
        lo = (b & 0xF).astype(np.int16)
        hi = (b >> 4).astype(np.int16)
        lo = np.where(lo >= 8, lo - 16, lo)
        hi = np.where(hi >= 8, hi - 16, hi)
        codes = np.empty(b.shape[:-1] + (2 * b.shape[-1],), np.int8)
        codes[..., 0::2] = lo
        codes[..., 1::2] = hi
        n = codes.shape[-1]
        stored = np.empty_like(codes)
        i = np.arange(n)
        p = (i & 31 & ~7) + np.where(i & 1, 4 + ((i & 7) >> 1), (i & 7) >> 1)     # byte in its block
        stored[..., (p >> 4) * 16 * (n // 32) + (i >> 5) * 16 + (p & 15)] = codes
        getattr(L8, name).copy_(torch.from_numpy(stored))
    return L8


@pytest.mark.parametrize("T", [9, 40, 100])
def test_grouped_int8_equals_int4_on_shared_codes(T):
    """Codes in [-8, 7] written both ways give the same block dots, and the
    grouped int8 kernels scale and sum them as the int4 ones do: outputs bit
    for bit (a wrong half order, row stride or a leftover x16 factor breaks
    it)."""
    sp4 = S.LayerSpec(H=256, I=128, E=16, top_k=2)
    L4 = device_layer(sp4, 0, 0)
    L8 = _int8_copy_of_int4(L4, sp4)
    x = S.tokens(S.TokenSpec(T=T, token_set=970 + T), sp4.H, 0)
    y4 = api.moe_forward(L4, dev(x), api.workspace(L4, T)).cpu().numpy()
    y8 = api.moe_forward(L8, dev(x), api.workspace(L8, T)).cpu().numpy()
    say(f"grouped int8 vs int4 codes T={T}: identical {np.mean(y4 == y8):.4f}")
    assert np.array_equal(y4, y8)


@pytest.fixture(scope="module")
def tiny2():
    spec = replace(S.TINY, weight_bits=2)
    return spec, device_layer(spec, 0, 0), OL.full_layer(spec, 0, 0)


@pytest.mark.parametrize("T", [9, 40, 100])
def test_grouped_int2_equals_int4_on_shared_codes(tiny2, T):
    """The int2 layer's codes written as int4 nibbles (same scales): the
    grouped int4 kernels give the grouped int2 kernels' outputs bit for bit
    (a wrong field order, a leftover x64 factor or a row stride of the wrong
    format breaks it)."""
    spec, L2, ref = tiny2
    L4 = api.MoELayer.empty(spec.H, spec.I, spec.E, spec.top_k)
    L4.router_w.copy_(L2.router_w)
    L4.router_b.copy_(L2.router_b)
    for name in ("gate_s", "up_s", "down_s"):
        getattr(L4, name).copy_(getattr(L2, name))
    for name in ("gate_q", "up_q", "down_q"):
        getattr(L4, name).copy_(torch.from_numpy(as_int4(codes_of(getattr(ref, name)))))
    x = S.tokens(S.TokenSpec(T=T, token_set=980 + T), spec.H, 0)
    y2 = api.moe_forward(L2, dev(x), api.workspace(L2, T)).cpu().numpy()
    y4 = api.moe_forward(L4, dev(x), api.workspace(L4, T)).cpu().numpy()
    say(f"grouped int2 vs int4 codes T={T}: identical {np.mean(y2 == y4):.4f}")
    assert np.array_equal(y2, y4)


@pytest.fixture(scope="module", params=["glm52_int8_prefill_T512", "glm52_int2_prefill_T512", "glm52_g32_prefill_T512"])
def glm_f_prefill(request):
    wl = S.WORKLOADS[request.param]
    say(f"building the GLM-5.2-shaped {label(wl.layer)} layer with Zipf-skewed bias on device")
    L = device_layer(wl.layer, 0, 0)
    W, b = S.router(wl.layer, 0, 0)
    yield wl, L, W, b
    del L
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_grouped_glm_prefill_T512(glm_f_prefill):
    """All 512 tokens and all 4,608 pairs of the Zipf-routed prefill batch."""
    wl, L, W, b = glm_f_prefill
    st, load = _full_layer_check(wl, L, W, b, f"{label(wl.layer)} prefill T=512")
    assert (load > 0).sum() > 100


@pytest.mark.parametrize("fmt", [dict(weight_bits=4), dict(weight_bits=8), dict(weight_bits=2)], ids=fmt_id)
@pytest.mark.parametrize("T", [9, 40, 77])
def test_grouped_whole_stages_small_grid(fmt, T):
    """H = I = 256: whole stages in gate/up and down for every row-scale
    format, in launches small enough for the quarter-tile kernels; every
    token and pair against the oracle, and the timed call's launches name
    those kernels."""
    spec = S.LayerSpec(H=256, I=256, E=16, top_k=2, **fmt)
    L, ref = device_layer(spec, 0, 0), OL.full_layer(spec, 0, 0)
    x = S.tokens(S.TokenSpec(T=T, token_set=990 + T), spec.H, 0)
    ws = api.workspace(L, T)
    say(f"grouped {label(spec)} whole stages, small grid, T={T}")
    y = api.moe_forward(L, dev(x), ws).cpu().numpy()
    ev = api.KernelEvents(16)
    y1 = api.moe_forward_timed(L, dev(x), api.workspace(L, T), ev).cpu().numpy()
    names = [n for n, _ in ev.durations_ms()]
    assert any("k_gateup_quad" in n for n in names) and any("k_down_quad" in n for n in names), names
    assert np.array_equal(y, y1)
    _tiny_batch_check(spec, L, ref, x, ws, y, f"{label(spec)} whole stages T={T}")


@pytest.mark.parametrize("fmt", [dict(group_size=32), dict(group_size=128)], ids=fmt_id)
@pytest.mark.parametrize("T", [40, 77])
def test_grouped_groups_whole_stages(fmt, T):
    """H = I = 256 with group scales: whole stages in gate/up and down (the
    stage loads addressed from a wave-wide base) on ragged tiles; every token
    and pair against the oracle, bit-identical, and the timed call's launches
    name the grouped kernels."""
    spec = S.LayerSpec(H=256, I=256, E=16, top_k=2, **fmt)
    L, ref = device_layer(spec, 0, 0), OL.full_layer(spec, 0, 0)
    x = S.tokens(S.TokenSpec(T=T, token_set=2990 + T), spec.H, 0)
    ws = api.workspace(L, T)
    say(f"grouped {label(spec)} whole stages with group scales, T={T}")
    y = api.moe_forward(L, dev(x), ws).cpu().numpy()
    ev = api.KernelEvents(16)
    y1 = api.moe_forward_timed(L, dev(x), api.workspace(L, T), ev).cpu().numpy()
    names = [n for n, _ in ev.durations_ms()]
    assert any("k_gateup_mfma" in n for n in names) and any("k_down_mfma" in n for n in names), names
    assert np.array_equal(y, y1)
    st = _tiny_batch_check(spec, L, ref, x, ws, y, f"{label(spec)} whole stages T={T}")
    assert st["h_bit_identical"] == 1.0 and st["y_bit_identical"] == 1.0


@pytest.mark.timeout(600)
@pytest.mark.parametrize("fmt", [dict(weight_bits=4), dict(weight_bits=8), dict(weight_bits=2)], ids=fmt_id)
def test_grouped_part_stages_large_grid(fmt):
    """H = 320, I = 96 (part-filled stages in gate/up and down) with 256
    experts and T = 6,000: grids past one resident round, so the larger-tile
    kernels run in their part-filled-stage forms rather than the quarter-tile
    ones; every token and pair against the oracle, and the timed call's
    launches name those kernels."""
    spec = S.LayerSpec(H=320, I=96, E=256, top_k=4, **fmt)
    L, ref = device_layer(spec, 0, 0), OL.full_layer(spec, 0, 0)
    T = 6000
    x = S.tokens(S.TokenSpec(T=T, token_set=1990), spec.H, 0)
    ws = api.workspace(L, T)
    say(f"grouped {label(spec)} part-filled stages, large grid, T={T}")
    y = api.moe_forward(L, dev(x), ws).cpu().numpy()
    ev = api.KernelEvents(16)
    y1 = api.moe_forward_timed(L, dev(x), api.workspace(L, T), ev).cpu().numpy()
    names = [n for n, _ in ev.durations_ms()]
    assert any("k_gateup_mfma" in n for n in names) and any("k_down_mfma" in n for n in names), names
    assert np.array_equal(y, y1)
    _tiny_batch_check(spec, L, ref, x, ws, y, f"{label(spec)} part-filled stages T={T}")
