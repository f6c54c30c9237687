"""GPU parity of the grouped int8-MFMA path (prefill, T > 8) and path
invariance against the token-GEMV path, through the C ABI."""
import numpy as np
import pytest
import torch

from int4_quantized_expert_sigmoid_amd import api, COLI_PATH_GEMV, COLI_PATH_GROUPED
from int4_quantized_expert_sigmoid_amd.synthetic import device_layer
from oracle import layers as OL
from oracle import oracle as O
from synth import synth as S

import parity as PR
from gpu_common import DeviceGenExperts, dev, rel_err, unreorder, ws_views

pytestmark = pytest.mark.gpu
TOL = 1e-4


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.set_device(0)


@pytest.fixture(scope="module")
def tiny():
    return device_layer(S.TINY, 0, 0), OL.full_layer(S.TINY, 0, 0)


def _tiny_batch_check(spec, L, ref, x, ws, y, label):
    """Every token and pair of a small batch against the oracle's whole batch."""
    v = ws_views(L, x.shape[0], ws)
    assert v["path"] == 1
    cache = OL.ExpertCache(spec, 0, 0)
    o = OL.forward_batch(spec, ref.router_w, ref.router_b, x, lambda e: cache[e])
    y_o, _, _ = O.moe_forward(ref, x)
    assert np.array_equal(o.y, y_o)              # the batch driver is the per-token oracle
    st = PR.check_free_running(spec, PR.gpu_pairs(v, spec.has_shared, y), PR.batch_pairs(o),
                               lambda e: cache[e], say)
    say(f"  {label}: max rel {st['worst_y']:.2e}, bit-identical {st['y_bit_identical']:.4f}")
    return st


@pytest.mark.parametrize("T", [9, 64, 200])
def test_grouped_tiny_full_outputs(tiny, T):
    L, ref = tiny
    x = S.tokens(S.TokenSpec(T=T, token_set=100 + T), S.TINY.H, 0)
    ws = api.workspace(L, T)
    say(f"grouped tiny T={T}")
    y = api.moe_forward(L, dev(x), ws).cpu().numpy()
    _tiny_batch_check(S.TINY, L, ref, x, ws, y, f"tiny T={T}")


def test_grouped_hot_experts_full_tiles():
    """Every token on the same experts: each expert's bucket holds all T
    tokens (several full 32-pair tiles of one expert), the compute-bound
    regime of the grouped GEMM."""
    spec = S.LayerSpec(H=256, I=128, E=16, top_k=2, hot_experts=2)
    L, ref = device_layer(spec, 0, 0), OL.full_layer(spec, 0, 0)
    T = 100
    x = S.tokens(S.TokenSpec(T=T, token_set=7), spec.H, 0)
    ws = api.workspace(L, T)
    say(f"grouped hot experts T={T}")
    y = api.moe_forward(L, dev(x), ws).cpu().numpy()
    y_o, idx_o, _ = O.moe_forward(ref, x)
    assert len(np.unique(idx_o)) == 2                 # the two hot experts, for every token
    v = ws_views(L, T, ws)
    assert v["path"] == 1
    assert np.array_equal(np.sort(v["idx"], axis=1), np.sort(idx_o, axis=1))
    _tiny_batch_check(spec, L, ref, x, ws, y, f"hot experts T={T}")


# H = 320: 10 blocks per gate/up row (a part-filled last stage of 8 blocks,
# scales loaded one by one); I = 96: 3 gate/up row tiles (a wave without
# rows in the workgroup) and 3 down blocks (an odd last block).
ODD = S.LayerSpec(H=320, I=96, E=16, top_k=4)


@pytest.fixture(scope="module")
def odd():
    return device_layer(ODD, 0, 0), OL.full_layer(ODD, 0, 0)


@pytest.mark.parametrize("T", [9, 40, 77])
def test_grouped_odd_shape_full_outputs(odd, T):
    L, ref = odd
    x = S.tokens(S.TokenSpec(T=T, token_set=700 + T), ODD.H, 0)
    ws = api.workspace(L, T)
    say(f"grouped odd shape H={ODD.H} I={ODD.I} T={T}")
    y = api.moe_forward(L, dev(x), ws).cpu().numpy()
    _tiny_batch_check(ODD, L, ref, x, ws, y, f"odd T={T}")


@pytest.mark.parametrize("T", [1, 4, 8])
def test_path_invariance_tiny(tiny, T):
    L, _ = tiny
    x = S.tokens(S.TokenSpec(T=T, token_set=300 + T), S.TINY.H, 0)
    ws = api.workspace(L, T)
    yg = api.moe_forward(L, dev(x), ws, flags=COLI_PATH_GEMV).cpu().numpy()
    vg = ws_views(L, T, ws, COLI_PATH_GEMV)
    ym = api.moe_forward(L, dev(x), ws, flags=COLI_PATH_GROUPED).cpu().numpy()
    vm = ws_views(L, T, ws, COLI_PATH_GROUPED)
    assert vg["path"] == 0 and vm["path"] == 1
    for t in range(T):
        for j in range(S.TINY.top_k):
            pg, pm = vg["pair_of"][t, j], vm["pair_of"][t, j]
            assert np.array_equal(vg["hq"][pg], vm["hq"][pm]) and np.array_equal(vg["hs"][pg], vm["hs"][pm])
            assert np.array_equal(vg["h"][pg], vm["h"][pm])
    say(f"path invariance T={T}: bit-identical outputs {np.mean(yg == ym):.4f}")
    assert rel_err(ym, yg).max() <= TOL


@pytest.fixture(scope="module")
def glm_prefill():
    wl = S.WORKLOADS["glm52_prefill_T512"]
    say("building GLM-5.2-shaped layer with Zipf-skewed bias on device")
    L = device_layer(wl.layer, 0, 0)
    W, b = S.router(wl.layer, 0, 0)
    return wl, L, W, b


def _full_layer_check(wl, L, W, b, label):
    """Every token and every (token, expert) pair of a GLM-shaped batch on
    the grouped path against the oracle's whole batch (the threaded build,
    bit for bit the plain one), free-running with flip accounting."""
    spec, T = wl.layer, wl.tokens.T
    x = S.tokens(wl.tokens, spec.H, 0)
    ws = api.workspace(L, T)
    say(f"{label}: GPU forward T={T}")
    y = api.moe_forward(L, dev(x), ws).cpu().numpy()
    v = ws_views(L, T, ws)
    assert v["path"] == 1
    experts = DeviceGenExperts(spec, 0, 0)
    O.use_threads(True)
    try:
        say(f"{label}: oracle batch on {O.threads()} threads")
        ref = OL.forward_batch(spec, W, b, x, experts, log=say)
    finally:
        O.use_threads(False)
    load = np.bincount(ref.idx.reshape(-1), minlength=spec.E)
    say(f"{label}: {int((load > 0).sum())} experts touched, top load {load.max()}, "
        f"median {np.median(load[load > 0])}, {T * (spec.top_k + spec.has_shared)} pairs compared")
    return PR.check_free_running(spec, PR.gpu_pairs(v, spec.has_shared, y), PR.batch_pairs(ref), experts, say), load


@pytest.mark.timeout(900)
def test_grouped_glm_prefill_T512(glm_prefill):
    """All 512 tokens and all 4,608 pairs of the Zipf-routed prefill batch."""
    wl, L, W, b = glm_prefill
    st, load = _full_layer_check(wl, L, W, b, "prefill T=512")
    assert (load > 0).sum() > 100                 # the skewed load spreads over most experts


@pytest.fixture(scope="module")
def glm_hot8():
    wl = S.WORKLOADS["glm52_hot8_T512"]
    say("building GLM-5.2-shaped layer with 8 hot experts on device")
    L = device_layer(wl.layer, 0, 0)
    W, b = S.router(wl.layer, 0, 0)
    return wl, L, W, b


@pytest.mark.timeout(900)
def test_grouped_glm_hot8_T512(glm_hot8):
    """Every token on the same 8 experts: 9 experts x 512 pairs in full
    32-pair tiles at H = 6144, I = 2048 (the XCD-aware tile order runs)."""
    wl, L, W, b = glm_hot8
    st, load = _full_layer_check(wl, L, W, b, "hot8 T=512")
    assert (load > 0).sum() == 8 and load.max() == 512


def test_grouped_glm_prefill_graph_replays(glm_prefill):
    """The timed prefill configuration: the T = 512 Zipf-routed layer call
    captured in a HIP graph and replayed, with eager calls on another input
    between replays, gives the eager output bit for bit every time."""
    wl, L, W, b = glm_prefill
    T = wl.tokens.T
    x = dev(S.tokens(wl.tokens, wl.layer.H, 0))
    x2 = dev(S.tokens(wl.tokens, wl.layer.H, 1))
    ws = api.workspace(L, T)
    eager = api.moe_forward(L, x, ws).clone()
    eager2 = api.moe_forward(L, x2, ws).clone()
    y = torch.empty_like(x)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        api.moe_forward(L, x, ws, y=y, stream=torch.cuda.current_stream())
    say("GLM prefill T=512 graph replays")
    for rep in range(3):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, eager), f"replay {rep}"
        assert torch.equal(api.moe_forward(L, x2, ws), eager2)   # eager work between replays
        torch.cuda.synchronize()
    assert not torch.equal(eager, eager2)


def test_path_invariance_glm_T4(glm_prefill):
    wl, L, W, b = glm_prefill
    x = S.tokens(S.TokenSpec(T=4, rho=0.8, outlier_channels=61), wl.layer.H, 0)
    ws = api.workspace(L, 4)
    yg = api.moe_forward(L, dev(x), ws, flags=COLI_PATH_GEMV).cpu().numpy()
    ym = api.moe_forward(L, dev(x), ws, flags=COLI_PATH_GROUPED).cpu().numpy()
    say(f"GLM path invariance T=4: bit-identical {np.mean(yg == ym):.4f}")
    assert rel_err(ym, yg).max() <= TOL
