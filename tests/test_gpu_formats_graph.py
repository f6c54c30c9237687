"""HIP-graph replays of the layer for every weight format (int4 rows, int8,
int2, int4 with group scales), on the decode path (T = 1, 4) and the grouped
MFMA path (T = 40: routing buckets, tile lists and the grouped kernels): a
captured coli_moe_forward replayed several times, with the same work done
eagerly between replays, gives the eager result bit for bit each time (the
launches keep no state between calls that a replay could see stale)."""
from dataclasses import replace

import numpy as np
import pytest
import torch

from int4_quantized_expert_sigmoid_amd import api
from int4_quantized_expert_sigmoid_amd.synthetic import device_layer
from synth import synth as S

from gpu_common import dev

pytestmark = pytest.mark.gpu

FORMATS = {"int4": S.TINY, "int8": replace(S.TINY, weight_bits=8), "int2": replace(S.TINY, weight_bits=2),
           "g64": replace(S.TINY, group_size=64)}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.set_device(0)


@pytest.mark.parametrize("fmt", list(FORMATS))
@pytest.mark.parametrize("T", [1, 4, 40])
def test_format_graph_replays(fmt, T):
    spec = FORMATS[fmt]
    L = device_layer(spec, 0, 5)
    x = dev(S.tokens(S.TokenSpec(T=T, token_set=120 + T), spec.H, 0))
    x2 = dev(S.tokens(S.TokenSpec(T=T, token_set=130 + T), spec.H, 0))
    ws = api.workspace(L, T)
    eager = api.moe_forward(L, x, ws).clone()
    eager2 = api.moe_forward(L, x2, ws).clone()
    ya, yb = torch.empty_like(x), torch.empty_like(x)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        api.moe_forward(L, x, ws, y=ya, stream=torch.cuda.current_stream())
        api.moe_forward(L, x2, ws, y=yb, stream=torch.cuda.current_stream())
    print(f"graph replays {fmt} T={T}", flush=True)
    for rep in range(3):
        ya.zero_(); yb.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ya, eager), f"replay {rep}"
        assert torch.equal(yb, eager2), f"replay {rep}"
        api.moe_forward(L, x2, ws)                     # eager work between replays
        torch.cuda.synchronize()
    assert not np.array_equal(eager.cpu().numpy(), eager2.cpu().numpy())
