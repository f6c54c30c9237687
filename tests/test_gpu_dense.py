"""GPU parity of the dense MLP (coli_dense_forward) through the C ABI against
the oracle's O15, on both paths (token-GEMV for T <= 8, grouped MFMA above,
for int4 and int8 weights),
both weight formats, intermediate sizes below and above 256 blocks (for one
token slot the down kernel then gives each thread a second block column, for
more slots it adds waves), with the RMSNorm input and the residual added in
place."""
import numpy as np
import pytest
import torch

from int4_quantized_expert_sigmoid_amd import api, COLI_ACCUMULATE, COLI_PATH_GEMV, COLI_PATH_GROUPED
from int4_quantized_expert_sigmoid_amd.synthetic import device_dense
from oracle import oracle as O
from synth import synth as S

from gpu_common import dev, rel_err

pytestmark = pytest.mark.gpu
TOL = 1e-4


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.set_device(0)


def oracle_weights(spec, seed=0, layer=0):
    pack = O.pack_int8_rows if spec.weight_bits == 8 else O.pack_int4_rows
    out = []
    for m in (S.GATE, S.UP, S.DOWN):
        out.extend(pack(S.dense_matrix(spec, seed, layer, m)))
    return out


def check(spec, T, flags=0, gamma=False, accumulate=False, token_set=0):
    M = device_dense(spec, 0, 0)
    w = oracle_weights(spec)
    x = S.tokens(S.TokenSpec(T=T, outlier_channels=2, token_set=token_set), spec.H, 0)
    g = S.rms_gamma(spec.H, 0, 1) if gamma else None
    xd = dev(x)
    ws = api.dense_workspace(M, T)
    say(f"dense H={spec.H} I={spec.I} int{spec.weight_bits} T={T} flags={flags} gamma={gamma} acc={accumulate}")
    if accumulate:
        y = api.dense_forward(M, xd, ws, y=xd, flags=flags | COLI_ACCUMULATE,
                              gamma=None if g is None else dev(g)).cpu().numpy()
    else:
        y = api.dense_forward(M, xd, ws, flags=flags, gamma=None if g is None else dev(g)).cpu().numpy()
    y_o = O.dense_forward(*w, x, gamma=g)
    if accumulate:
        y_o = (x + y_o).astype(np.float32)
    err = rel_err(y, y_o).max()
    say(f"  max rel {err:.2e}, bit-identical {np.mean(y == y_o):.4f}")
    assert err <= TOL
    return y


SMALL = S.DenseSpec(H=128, I=352, w_outlier_rate=0.01, weight_bits=4)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("T", [1, 2, 5, 8])
def test_dense_gemv_small(bits, T):
    from dataclasses import replace
    check(replace(SMALL, weight_bits=bits), T, token_set=T)


@pytest.mark.parametrize("T,flags", [(12, 0), (40, 0), (3, COLI_PATH_GROUPED)])
def test_dense_grouped_small(T, flags):
    check(SMALL, T, flags, token_set=20 + T)


@pytest.mark.parametrize("T,flags", [(9, 0), (16, 0), (21, 0), (40, 0), (3, COLI_PATH_GROUPED)])
def test_dense_int8_grouped(T, flags):
    """int8 weights on the grouped int8-MFMA kernels (one expert holding
    every token): past 8 tokens, and forced at T = 3."""
    from dataclasses import replace
    spec = replace(SMALL, weight_bits=8)
    check(spec, T, flags, token_set=70 + T, accumulate=(T == 21))


def test_dense_paths_agree():
    """The same tokens through both paths: identical outputs (same integer
    block dots, f64 sums)."""
    M = device_dense(SMALL, 0, 0)
    x = dev(S.tokens(S.TokenSpec(T=6, token_set=33), SMALL.H, 0))
    a = api.dense_forward(M, x, api.dense_workspace(M, 6), flags=COLI_PATH_GEMV).cpu().numpy()
    b = api.dense_forward(M, x, api.dense_workspace(M, 6), flags=COLI_PATH_GROUPED).cpu().numpy()
    assert np.max(rel_err(a, b)) <= TOL


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("T", [1, 3])
def test_dense_down_past_256_blocks(bits, T):
    """I = 8448: 264 blocks per down row. One token slot (T = 1) takes the
    four-wave form with a second block column per thread for the blocks past
    256; more slots (T = 3) take one column per thread with a fifth wave, 8
    of its lanes in use."""
    spec = S.DenseSpec(H=256, I=8448, w_outlier_rate=0.01, weight_bits=bits)
    check(spec, T, token_set=41 + T)


def test_dense_rmsnorm_and_residual_in_place():
    spec = S.DenseSpec(H=256, I=512, weight_bits=8)
    check(spec, 4, gamma=True, accumulate=True, token_set=51)
    check(spec, 1, gamma=True, accumulate=False, token_set=52)
    check(S.DenseSpec(H=256, I=512, weight_bits=4), 20, gamma=True, accumulate=True, token_set=53)


@pytest.mark.parametrize("bits,T", [(8, 1), (4, 2), (8, 12)])
def test_dense_glm_shape(bits, T):
    """H = 6144, I = 12288: the dense layers' shape read for GLM-5.2."""
    from dataclasses import replace
    check(replace(S.GLM52_DENSE, weight_bits=bits), T, token_set=60 + T)
    torch.cuda.empty_cache()
