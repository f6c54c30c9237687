"""GPU checks of coli_moe_forward_timed through the C ABI: the same launches
and bit-identical results as coli_moe_forward on every path, one start/stop
event pair per launch in launch order, and the launch count and kernel names
the bench's roofline field relies on."""
import numpy as np
import pytest
import torch

from int4_quantized_expert_sigmoid_amd import api, COLI_PATH_GROUPED
from int4_quantized_expert_sigmoid_amd.synthetic import device_layer
from synth import synth as S

from gpu_common import dev

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.set_device(0)


@pytest.fixture(scope="module")
def tiny():
    return device_layer(S.TINY, 0, 0)


def _check(L, x, flags, expect):
    T = x.shape[0]
    xd = dev(x)
    ws = api.workspace(L, T)
    y0 = api.moe_forward(L, xd, ws, flags=flags).cpu().numpy()
    ev = api.KernelEvents(16)
    ws2 = api.workspace(L, T)
    y1 = api.moe_forward_timed(L, xd, ws2, ev, flags=flags).cpu().numpy()
    torch.cuda.synchronize()
    assert np.array_equal(y0, y1)
    d = ev.durations_ms()
    names = [n for n, _ in d]
    say(f"timed T={T} flags={flags}: " + ", ".join(f"{n} {ms * 1e3:.1f} us" for n, ms in d))
    assert len(d) == ev.count.value
    for k in expect:
        assert any(k in n for n in names), (k, names)
    assert all(ms > 0.0 for _, ms in d)
    return names


@pytest.mark.parametrize("T", [1, 2, 4, 8])
def test_timed_decode_launches(tiny, T):
    x = S.tokens(S.TokenSpec(T=T, token_set=70 + T), S.TINY.H, 0)
    names = _check(tiny, x, 0, ["k_router", "k_select_gateup"])
    # router, routed gate/up, then down + combine in one launch (T <= 2) or two
    assert len(names) == (3 if T <= 2 else 4), names
    assert "k_select_gateup" in names[1]


def test_timed_grouped_launches(tiny):
    # launches this small take the quarter-tile gate/up and down kernels
    # (no more workgroups than one resident round of the larger-tile ones)
    x = S.tokens(S.TokenSpec(T=40, token_set=79), S.TINY.H, 0)
    names = _check(tiny, x, COLI_PATH_GROUPED, ["k_gateup_quad", "k_down_quad", "k_combine"])
    assert names.index([n for n in names if "k_gateup_quad" in n][0]) < \
        names.index([n for n in names if "k_down_quad" in n][0])


def test_timed_fewer_pairs_than_launches(tiny):
    x = S.tokens(S.TokenSpec(T=1, token_set=81), S.TINY.H, 0)
    xd = dev(x)
    ws = api.workspace(tiny, 1)
    y0 = api.moe_forward(tiny, xd, ws).cpu().numpy()
    ev = api.KernelEvents(1)                      # only the first launch timed, the rest run untimed
    y1 = api.moe_forward_timed(tiny, xd, api.workspace(tiny, 1), ev).cpu().numpy()
    assert np.array_equal(y0, y1)
    assert ev.count.value == 3
    d = ev.durations_ms()
    assert len(d) == 1 and "k_router" in d[0][0]
