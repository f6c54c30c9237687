"""GPU checks of coli_moe_forward_rms through the C ABI: one chain layer in
one call (the router launch takes the RMSNorm itself on the decode path)
gives coli_rmsnorm followed by coli_moe_forward bit for bit, on every path,
with the residual added in place."""
import numpy as np
import pytest
import torch

from int4_quantized_expert_sigmoid_amd import api, COLI_ACCUMULATE, COLI_PATH_GEMV, COLI_PATH_GROUPED
from int4_quantized_expert_sigmoid_amd.synthetic import device_layer
from synth import synth as S

from gpu_common import dev

pytestmark = pytest.mark.gpu
EPS = 1e-6


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.set_device(0)


@pytest.fixture(scope="module")
def tiny():
    return device_layer(S.TINY, 0, 0)


def _both(L, x, g, flags):
    """(fused, separate) outputs of x + MoE(RMSNorm(x) * g), residual in place."""
    T = x.shape[0]
    xa = dev(x)
    api.moe_forward_rms(L, xa, dev(g), EPS, api.workspace(L, T, ), y=xa, flags=flags | COLI_ACCUMULATE)
    xb = dev(x)
    xn = api.rmsnorm(xb, dev(g), EPS)
    api.moe_forward(L, xn, api.workspace(L, T), y=xb, flags=flags | COLI_ACCUMULATE)
    return xa.cpu().numpy(), xb.cpu().numpy()


@pytest.mark.parametrize("T,flags", [(1, 0), (2, 0), (4, 0), (8, 0), (3, COLI_PATH_GEMV), (40, 0),
                                     (5, COLI_PATH_GROUPED)])
def test_rms_forward_equals_norm_then_forward(tiny, T, flags):
    x = S.tokens(S.TokenSpec(T=T, token_set=90 + T, outlier_channels=3), S.TINY.H, 0)
    g = S.rms_gamma(S.TINY.H, 0, 5)
    say(f"rms forward tiny T={T} flags={flags}")
    a, b = _both(tiny, x, g, flags)
    assert np.array_equal(a, b)
    assert not np.array_equal(a, x)


def test_rms_forward_equals_norm_then_forward_glm():
    spec = S.GLM52
    L = device_layer(spec, 0, 3)
    for T in (1, 4):
        x = S.tokens(S.TokenSpec(T=T, outlier_channels=61, token_set=11), spec.H, 0)
        g = S.rms_gamma(spec.H, 0, 3)
        say(f"rms forward GLM T={T}")
        a, b = _both(L, x, g, 0)
        assert np.array_equal(a, b)
        # the chain layer as a decode step captures it: residual added in place
        x0, xr, gd = dev(x), dev(x), dev(g)
        ws = api.workspace(L, T)
        say(f"rms forward GLM T={T} graph replays")
        _replay(lambda st: api.moe_forward_rms(L, xr, gd, EPS, ws, y=xr, flags=COLI_ACCUMULATE, stream=st),
                [torch.from_numpy(a).cuda()], [xr], reset=lambda: xr.copy_(x0))
    del L
    torch.cuda.empty_cache()


def test_rms_forward_not_accumulating(tiny):
    x = S.tokens(S.TokenSpec(T=2, token_set=95), S.TINY.H, 0)
    g = S.rms_gamma(S.TINY.H, 0, 6)
    y1 = api.moe_forward_rms(tiny, dev(x), dev(g), EPS, api.workspace(tiny, 2)).cpu().numpy()
    xn = api.rmsnorm(dev(x), dev(g), EPS)
    y2 = api.moe_forward(tiny, xn, api.workspace(tiny, 2)).cpu().numpy()
    assert np.array_equal(y1, y2)


def _replay(capture, eager, outs, n=4, reset=None):
    """Capture `capture` in a HIP graph, replay it n times with eager work in
    between, and compare every replay with the eager results. `reset` restores
    the outputs' starting values before each replay (default: zeros)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        capture(torch.cuda.current_stream())
    for rep in range(n):
        if reset is None:
            for o in outs:
                o.zero_()
        else:
            reset()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o, e), f"replay {rep}"
        capture(torch.cuda.current_stream())       # the same work eagerly between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("T", [1, 4, 20])
def test_rms_forward_graph_replays(tiny, T):
    x = dev(S.tokens(S.TokenSpec(T=T, token_set=97 + T), S.TINY.H, 0))
    g = dev(S.rms_gamma(S.TINY.H, 0, 7))
    ws = api.workspace(tiny, T)
    eager = [api.moe_forward_rms(tiny, x, g, EPS, ws).clone()]
    y = torch.empty_like(x)
    _replay(lambda st: api.moe_forward_rms(tiny, x, g, EPS, ws, y=y, stream=st), eager, [y])


@pytest.mark.parametrize("T", [1, 3, 12])
def test_dense_forward_graph_replays(T):
    from int4_quantized_expert_sigmoid_amd.synthetic import device_dense
    spec = S.DenseSpec(H=256, I=512, weight_bits=4)
    M = device_dense(spec, 0, 0)
    x = dev(S.tokens(S.TokenSpec(T=T, token_set=98 + T), spec.H, 0))
    g = dev(S.rms_gamma(spec.H, 0, 8))
    ws = api.dense_workspace(M, T)
    eager = [api.dense_forward(M, x, ws, gamma=g).clone()]
    y = torch.empty_like(x)
    _replay(lambda st: api.dense_forward(M, x, ws, y=y, gamma=g, stream=st), eager, [y])
