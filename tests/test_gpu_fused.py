"""GPU checks of the decode paths that hand work between workgroups of one
launch through counters in the workspace: the single-launch persistent path
(COLI_PATH_FUSED) and the default path, whose first launch counts its router
workgroups. Through the C ABI: results bit-identical between the paths and
within the oracle bar, counters back at zero and the error word clear after
every call, repeated calls and HIP-graph replays stable."""
import numpy as np
import pytest
import torch

from int4_quantized_expert_sigmoid_amd import api, COLI_ACCUMULATE, COLI_PATH_FUSED
from int4_quantized_expert_sigmoid_amd.synthetic import device_layer
from oracle import layers as OL
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


@pytest.fixture(scope="module")
def tiny():
    return device_layer(S.TINY, 0, 0), OL.full_layer(S.TINY, 0, 0)


@pytest.fixture(scope="module")
def glm():
    say("building GLM-5.2-shaped layer on device")
    return device_layer(S.GLM52, 0, 0)


def sync_words(layer, T, ws):
    lay = api.workspace_layout(layer, T)
    return ws[lay.sync: lay.sync + 4 * (64 + 129 + 63 + 256)].view(torch.int32).cpu().numpy()


def check_clean(layer, T, ws):
    w = sync_words(layer, T, ws)
    assert w[5] == 0, "bounded wait timed out (error word set)"
    assert not w.any(), f"counters left nonzero: {np.nonzero(w)[0][:10]}"


@pytest.mark.parametrize("T", [1, 2, 3, 5, 8])
def test_fused_equals_staged_and_oracle_tiny(tiny, T):
    L, ref = tiny
    x = S.tokens(S.TokenSpec(T=T, token_set=500 + T), S.TINY.H, 0)
    ws = api.workspace(L, T)
    say(f"fused tiny T={T}")
    yf = api.moe_forward(L, dev(x), ws, flags=COLI_PATH_FUSED).cpu().numpy()
    check_clean(L, T, ws)
    ys = api.moe_forward(L, dev(x), ws).cpu().numpy()
    assert np.array_equal(yf, ys)
    y_o, _, _ = O.moe_forward(ref, x)
    err = rel_err(yf, y_o).max()
    say(f"  max rel vs oracle {err:.2e}, bit-identical {np.mean(yf == y_o):.4f}")
    assert err <= TOL


def test_fused_repeated_calls_and_accumulate(tiny):
    L, ref = tiny
    ws = api.workspace(L, 4)
    for rep in range(6):
        x = S.tokens(S.TokenSpec(T=4, token_set=600 + rep), S.TINY.H, 0)
        y0 = np.full((4, S.TINY.H), 0.5, np.float32)
        y = api.moe_forward(L, dev(x), ws, y=dev(y0), flags=COLI_ACCUMULATE | COLI_PATH_FUSED).cpu().numpy()
        check_clean(L, 4, ws)
        y_o, _, _ = O.moe_forward(ref, x)
        assert rel_err(y, (np.float32(0.5) + y_o).astype(np.float32)).max() <= TOL


def test_fused_glm_T1_T4(glm):
    L = glm
    for name in ("glm52_decode_T1", "glm52_mtp_verify_T4"):
        wl = S.WORKLOADS[name]
        x = S.tokens(wl.tokens, S.GLM52.H, 0)
        T = x.shape[0]
        ws = api.workspace(L, T)
        yf = api.moe_forward(L, dev(x), ws, flags=COLI_PATH_FUSED).cpu().numpy()
        check_clean(L, T, ws)
        ys = api.moe_forward(L, dev(x), ws).cpu().numpy()
        say(f"fused GLM {name}: bit-identical to default path {np.mean(yf == ys):.4f}")
        assert np.array_equal(yf, ys)


@pytest.mark.parametrize("T", [1, 2, 3, 8])
def test_default_path_leaves_counters_clean(tiny, T):
    L, ref = tiny
    ws = api.workspace(L, T)
    for rep in range(3):
        x = S.tokens(S.TokenSpec(T=T, token_set=900 + 10 * T + rep), S.TINY.H, 0)
        y = api.moe_forward(L, dev(x), ws).cpu().numpy()
        check_clean(L, T, ws)
        y_o, _, _ = O.moe_forward(ref, x)
        assert rel_err(y, y_o).max() <= TOL


@pytest.mark.parametrize("F", [COLI_PATH_FUSED, 0], ids=["fused", "default"])
def test_graph_replays(glm, F):
    L = glm
    x = S.tokens(S.TokenSpec(T=1, token_set=700, outlier_channels=61), S.GLM52.H, 0)
    x2 = S.tokens(S.TokenSpec(T=1, token_set=701, outlier_channels=61), S.GLM52.H, 0)
    xd, xd2 = dev(x), dev(x2)
    ws = api.workspace(L, 1)
    y_eager = api.moe_forward(L, xd, ws, flags=F).clone()
    y_eager2 = api.moe_forward(L, xd2, ws, flags=F).clone()
    ya = torch.empty_like(xd)
    yb = torch.empty_like(xd)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        api.moe_forward(L, xd, ws, y=ya, flags=F, stream=torch.cuda.current_stream())
        api.moe_forward(L, xd2, ws, y=yb, flags=F, stream=torch.cuda.current_stream())
    for rep in range(4):
        ya.zero_(); yb.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ya, y_eager), f"replay {rep}"
        assert torch.equal(yb, y_eager2), f"replay {rep}"
        api.moe_forward(L, xd2, ws, flags=F)          # eager work between replays
        torch.cuda.synchronize()
        check_clean(L, 1, ws)
