"""coli_moe_forward_noalloc (the library's own device scratch in place of a
caller workspace, for callers that cannot allocate) against
coli_moe_forward with a caller workspace, through the C ABI: two calls in a
row, the second with a smaller batch, on the token-GEMV path, the grouped
path and the GLM-5.2-shaped decode layer; results bit for bit (the same
kernels on the same inputs), and a batch past the scratch limit refused."""
import numpy as np
import pytest
import torch

from int4_quantized_expert_sigmoid_amd import api, COLI_ACCUMULATE
from int4_quantized_expert_sigmoid_amd._lib import COLI_EWORKSPACE, COLI_NOALLOC_MAX_BYTES, ColiError
from int4_quantized_expert_sigmoid_amd.synthetic import device_layer
from synth import synth as S

from gpu_common import dev, rel_err

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.set_device(0)


def _pair(L, x, flags=0, y0=None):
    """(no-alloc result, workspace result) of one batch."""
    T = x.shape[0]
    xd = dev(x)
    ya = dev(y0) if y0 is not None else torch.empty_like(xd)
    yb = dev(y0) if y0 is not None else torch.empty_like(xd)
    api.moe_forward_noalloc(L, xd, ya, flags=flags)
    api.moe_forward(L, xd, api.workspace(L, T), y=yb, flags=flags)
    return ya.cpu().numpy(), yb.cpu().numpy()


@pytest.mark.parametrize("Ts", [(6, 2), (40, 9), (9, 1)])
def test_noalloc_equals_workspace_tiny(Ts):
    L = device_layer(S.TINY, 0, 0)
    for i, T in enumerate(Ts):
        x = S.tokens(S.TokenSpec(T=T, token_set=900 + T), S.TINY.H, 0)
        ya, yb = _pair(L, x)
        say(f"no-alloc tiny call {i} T={T}: identical {np.mean(ya == yb):.4f}")
        assert np.array_equal(ya, yb)
    # accumulate into a nonzero y
    x = S.tokens(S.TokenSpec(T=3, token_set=77), S.TINY.H, 0)
    ya, yb = _pair(L, x, COLI_ACCUMULATE, np.full((3, S.TINY.H), 0.5, np.float32))
    assert np.array_equal(ya, yb)


def test_noalloc_equals_workspace_glm_decode():
    say("building the GLM-5.2-shaped layer on the GPU")
    L = device_layer(S.GLM52, 0, 0)
    for i, wl in enumerate(("glm52_mtp_verify_T4", "glm52_decode_T1")):
        x = S.tokens(S.WORKLOADS[wl].tokens, S.GLM52.H, 0)
        ya, yb = _pair(L, x)
        say(f"no-alloc GLM call {i} T={x.shape[0]}: identical {np.mean(ya == yb):.4f}")
        assert np.array_equal(ya, yb)
        assert rel_err(ya, yb).max() <= 1e-4
    # past the scratch limit: refused before anything runs; the next call works
    T = 512
    assert api.workspace_bytes(L, T) > COLI_NOALLOC_MAX_BYTES
    x = dev(S.tokens(S.TokenSpec(T=T, token_set=5), S.GLM52.H, 0))
    with pytest.raises(ColiError) as e:
        api.moe_forward_noalloc(L, x, torch.empty_like(x))
    assert e.value.code == COLI_EWORKSPACE
    x1 = S.tokens(S.TokenSpec(T=1, token_set=6, outlier_channels=61), S.GLM52.H, 0)
    ya, yb = _pair(L, x1)
    assert np.array_equal(ya, yb)
    del L
    torch.cuda.empty_cache()
