"""GPU checks of coli_moe_forward_rms through the C ABI: one chain layer in
one call (the router launch takes the RMSNorm itself on the decode path)
gives coli_rmsnorm followed by coli_moe_forward bit for bit, on every path,
with the residual added in place."""
import numpy as np
import pytest
import torch

from int4_quantized_expert_sigmoid_amd import api, COLI_ACCUMULATE, COLI_PATH_FUSED, COLI_PATH_GROUPED
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


@pytest.mark.parametrize("T,flags", [(1, 0), (2, 0), (4, 0), (8, 0), (3, COLI_PATH_FUSED), (40, 0),
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
    del L
    torch.cuda.empty_cache()


def test_rms_forward_not_accumulating(tiny):
    x = S.tokens(S.TokenSpec(T=2, token_set=95), S.TINY.H, 0)
    g = S.rms_gamma(S.TINY.H, 0, 6)
    y1 = api.moe_forward_rms(tiny, dev(x), dev(g), EPS, api.workspace(tiny, 2)).cpu().numpy()
    xn = api.rmsnorm(dev(x), dev(g), EPS)
    y2 = api.moe_forward(tiny, xn, api.workspace(tiny, 2)).cpu().numpy()
    assert np.array_equal(y1, y2)
