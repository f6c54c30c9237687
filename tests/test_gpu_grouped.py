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

from gpu_common import dev, rel_err, unreorder, ws_views

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


@pytest.mark.parametrize("T", [9, 64, 200])
def test_grouped_tiny_full_outputs(tiny, T):
    L, ref = tiny
    x = S.tokens(S.TokenSpec(T=T, token_set=100 + T), S.TINY.H, 0)
    ws = api.workspace(L, T)
    say(f"grouped tiny T={T}")
    y = api.moe_forward(L, dev(x), ws).cpu().numpy()
    assert ws_views(L, T, ws)["path"] == 1
    y_o, idx_o, _ = O.moe_forward(ref, x)
    err = rel_err(y, y_o).max()
    say(f"  max rel {err:.2e}, bit-identical {np.mean(y == y_o):.4f}")
    assert err <= TOL
    # intermediates of every pair bit-exact
    v = ws_views(L, T, ws)
    cache = OL.ExpertCache(S.TINY, 0, 0)
    for t in range(0, T, max(1, T // 7)):
        r = OL.forward_token(S.TINY, cache, ref.router_w, ref.router_b, x[t])
        pairs = list(v["pair_of"][t]) + [v["shared_pair"][t]]
        for p, eo in zip(pairs, r.experts):
            assert np.array_equal(unreorder(v["hq"][p]), eo.hq)
            assert np.array_equal(v["hs"][p], eo.hs)


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
    err = rel_err(y, y_o).max()
    say(f"  max rel {err:.2e}, bit-identical {np.mean(y == y_o):.4f}")
    assert err <= TOL


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
    v = ws_views(L, T, ws)
    assert v["path"] == 1
    y_o, idx_o, _ = O.moe_forward(ref, x)
    assert np.array_equal(v["idx"], idx_o)
    err = rel_err(y, y_o).max()
    say(f"  max rel {err:.2e}, bit-identical {np.mean(y == y_o):.4f}")
    assert err <= TOL
    cache = OL.ExpertCache(ODD, 0, 0)
    for t in range(0, T, max(1, T // 5)):
        r = OL.forward_token(ODD, cache, ref.router_w, ref.router_b, x[t])
        pairs = list(v["pair_of"][t]) + [v["shared_pair"][t]]
        for p, eo in zip(pairs, r.experts):
            assert np.array_equal(unreorder(v["hq"][p]), eo.hq)
            assert np.array_equal(v["hs"][p], eo.hs)


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


def test_grouped_glm_prefill_T512(glm_prefill):
    wl, L, W, b = glm_prefill
    spec = wl.layer
    x = S.tokens(wl.tokens, spec.H, 0)
    ws = api.workspace(L, 512)
    xd = dev(x)
    y = api.moe_forward(L, xd, ws).cpu().numpy()
    v = ws_views(L, 512, ws)
    idx_o, w_o = O.route(W, b, x, spec.top_k)
    assert np.array_equal(v["idx"], idx_o)
    load = np.bincount(idx_o.reshape(-1), minlength=spec.E)
    say(f"prefill T=512: {int((load > 0).sum())} experts touched, top load {load.max()}, median {np.median(load[load > 0])}")
    cache = OL.ExpertCache(spec, 0, 0)
    hot = int(np.argmax(load))
    sample = [0, 511] + [int(np.nonzero((idx_o == hot).any(axis=1))[0][0])]
    for t in sample:
        r = OL.forward_token(spec, cache, W, b, x[t])
        err = rel_err(y[t][None], r.y[None]).max()
        pairs = list(v["pair_of"][t]) + [v["shared_pair"][t]]
        for p, eo in zip(pairs, r.experts):
            assert np.array_equal(unreorder(v["hq"][p]), eo.hq)
        say(f"  token {t}: max rel {err:.2e}, bit-identical {np.mean(y[t] == r.y):.4f}")
        assert err <= TOL


def test_path_invariance_glm_T4(glm_prefill):
    wl, L, W, b = glm_prefill
    x = S.tokens(S.TokenSpec(T=4, rho=0.8, outlier_channels=61), wl.layer.H, 0)
    ws = api.workspace(L, 4)
    yg = api.moe_forward(L, dev(x), ws, flags=COLI_PATH_GEMV).cpu().numpy()
    ym = api.moe_forward(L, dev(x), ws, flags=COLI_PATH_GROUPED).cpu().numpy()
    say(f"GLM path invariance T=4: bit-identical {np.mean(yg == ym):.4f}")
    assert rel_err(ym, yg).max() <= TOL
