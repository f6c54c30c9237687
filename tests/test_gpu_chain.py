"""GPU check of the decode chain, through the C ABI: one token through the 16
GLM-5.2-shaped layers of the chain workload, each
x <- x + MoE(RMSNorm(x) * gamma) (eps 1e-6, independent seeded weights and
gamma per layer), run free on the GPU and on the oracle from the same input. At every layer the routing must be
identical and x within the output bar; the oracle's layer l consumes its own
x_l, so the two runs are compared after every layer without being re-synced."""
import numpy as np
import pytest
import torch

from int4_quantized_expert_sigmoid_amd import api, COLI_ACCUMULATE
from int4_quantized_expert_sigmoid_amd.synthetic import device_layer
from oracle import layers as OL
from oracle import oracle as O
from synth import synth as S

from gpu_common import dev, rel_err, ws_views

pytestmark = pytest.mark.gpu
TOL = 1e-4
N_LAYERS = 16


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.set_device(0)


@pytest.mark.parametrize("one_call", [False, True], ids=["norm_then_forward", "forward_rms"])
def test_sixteen_layer_chain_free_running(one_call):
    spec = S.GLM52
    wl = S.WORKLOADS["glm52_chain16_T1"]
    x0 = S.tokens(wl.tokens, spec.H, wl.seed)                # [1, H]
    xd = dev(x0)
    x_o = x0[0].copy()
    divergences = 0
    for li in range(N_LAYERS):
        say(f"chain layer {li}: building the layer on the GPU and its router on the host")
        L = device_layer(spec, wl.seed, li)
        g = S.rms_gamma(spec.H, wl.seed, li)
        ws = api.workspace(L, 1)
        if one_call:                                      # the router launch takes the norm itself
            api.moe_forward_rms(L, xd, dev(g), wl.rms_eps, ws, y=xd, flags=COLI_ACCUMULATE)
        else:
            xn = api.rmsnorm(xd, dev(g), wl.rms_eps)
            api.moe_forward(L, xn, ws, y=xd, flags=COLI_ACCUMULATE)
        v = ws_views(L, 1, ws)
        x_gpu = xd.cpu().numpy()[0]

        W, b = S.router(spec, wl.seed, li)
        cache = OL.ExpertCache(spec, wl.seed, li)
        xn_o = O.rmsnorm(x_o[None, :], g, wl.rms_eps)[0]
        r = OL.forward_token(spec, cache, W, b, xn_o)
        x_o = (x_o + r.y).astype(np.float32)
        same_route = np.array_equal(v["idx"][0], r.idx)
        divergences += 0 if same_route else 1
        err = rel_err(x_gpu[None], x_o[None]).max()
        say(f"  layer {li}: experts {r.idx.tolist()}, routing {'identical' if same_route else 'DIFFERS'}, "
            f"max rel {err:.2e}, bit-identical {np.mean(x_gpu == x_o):.4f}")
        assert same_route, f"routing diverged at layer {li}: {v['idx'][0].tolist()} vs {r.idx.tolist()}"
        assert err <= TOL
        del L, ws, cache
        torch.cuda.empty_cache()
    assert divergences == 0
