"""GPU checks of the routing the decode path (T <= 8) computes inside its
routed gate/up launch, through the C ABI: the top-k indices it publishes are
bit-identical to the oracle's, weights and outputs within the bar, with
group-limited routing, route_scale, exact key ties (equal keys go to the lower
expert index) and keys that agree in their upper 32 bits but not below."""
from dataclasses import replace

import numpy as np
import pytest
import torch

from int4_quantized_expert_sigmoid_amd import api
from int4_quantized_expert_sigmoid_amd.synthetic import device_layer
from oracle import layers as OL
from oracle import oracle as O
from synth import synth as S

from gpu_common import dev, rel_err, ws_views

pytestmark = pytest.mark.gpu
TOL = 1e-4
WIDE = S.LayerSpec(H=256, I=128, E=512, top_k=8)     # 8 keys per lane in the selection


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.set_device(0)


@pytest.fixture(scope="module")
def layers():
    return {name: (device_layer(spec, 0, 0), OL.full_layer(spec, 0, 0))
            for name, spec in (("tiny", S.TINY), ("wide", WIDE))}


def _run(L, ref, x):
    T = x.shape[0]
    ws = api.workspace(L, T)
    y = api.moe_forward(L, dev(x), ws).cpu().numpy()
    v = ws_views(L, T, ws)
    assert v["path"] == 0
    y_o, idx_o, w_o = O.moe_forward(ref, x)
    assert np.array_equal(v["idx"], idx_o)
    assert np.allclose(v["w"], w_o, rtol=1e-6, atol=0)
    err = rel_err(y, y_o).max()
    assert err <= TOL, err
    return v["idx"]


@pytest.mark.parametrize("name", ["tiny", "wide"])
@pytest.mark.parametrize("T", [1, 3, 8])
def test_decode_routing_group_limited_and_scale(layers, name, T):
    L, ref = layers[name]
    x = S.tokens(S.TokenSpec(T=T, token_set=40 + T), L.H, 0)
    variants = ((1, 1, 1.0), (4, 2, 2.5), (8, 8, 1.0), (16, 3, 1.0)) if name == "tiny" else \
        ((1, 1, 1.0), (8, 4, 2.5), (64, 2, 1.0))
    for ng, tg, rs in variants:
        say(f"decode routing {name} T={T} n_group={ng} topk_group={tg} route_scale={rs}")
        L.n_group, L.topk_group, L.route_scale = ng, tg, rs
        try:
            _run(L, replace(ref, n_group=ng, topk_group=tg, route_scale=rs), x)
        finally:
            L.n_group, L.topk_group, L.route_scale = 1, 1, 1.0


def _tie_bias(E, rng):
    """Biases with exact repeats and neighbours one f32 ulp apart: with a zero
    router every key is 0.5 + b, so equal biases give exactly equal keys and
    ulp neighbours give keys equal in their upper 32 bits."""
    base = rng.choice(np.array([0.011, 0.023, 0.037, 0.041], np.float32), size=E)
    nb = base.copy()
    up = rng.random(E) < 0.3
    nb[up] = np.nextafter(base[up], np.float32(1.0))
    return nb.astype(np.float32)


@pytest.mark.parametrize("name", ["tiny", "wide"])
@pytest.mark.parametrize("T", [1, 4])
def test_decode_routing_ties(layers, name, T):
    L, ref = layers[name]
    rng = np.random.default_rng(7 + T)
    w_save, b_save = L.router_w.clone(), L.router_b.clone()
    try:
        for rep in range(3):
            b = _tie_bias(L.E, rng)
            L.router_w.zero_()
            L.router_b.copy_(torch.from_numpy(b))
            ref_t = replace(ref, router_w=np.zeros_like(ref.router_w), router_b=b)
            x = S.tokens(S.TokenSpec(T=T, token_set=80 + rep), L.H, 0)
            say(f"decode routing ties {name} T={T} rep={rep}")
            idx = _run(L, ref_t, x)
            # every token sees the same keys: the same experts, lower index first among equals
            assert (idx == idx[0]).all()
    finally:
        L.router_w.copy_(w_save)
        L.router_b.copy_(b_save)


@pytest.mark.parametrize("name", ["tiny", "wide"])
def test_decode_routing_ties_inside_topk(layers, name):
    """Keys equal in their upper 32 bits, or exactly equal, inside the top-k
    but not across its last place: the selection is decided by the upper
    bits and the chosen keys must still be ranked by the exact (key desc,
    expert asc) order. Pairs of experts hold biases one f32 ulp apart or
    equal; every other bias is far lower."""
    L, ref = layers[name]
    rng = np.random.default_rng(11)
    k, E = L.top_k, L.E
    w_save, b_save = L.router_w.clone(), L.router_b.clone()
    try:
        for rep in range(3):
            b = np.full(E, -0.5, np.float32) + rng.random(E).astype(np.float32) * 0.01
            top = rng.choice(E, size=k, replace=False)
            levels = np.float32(0.1) * (1 + np.arange((k + 1) // 2, dtype=np.float32))
            for j in range(0, k, 2):
                b[top[j]] = levels[j // 2]
                if j + 1 < k:   # the partner: equal, or one ulp above
                    b[top[j + 1]] = levels[j // 2] if rep == 1 else np.nextafter(levels[j // 2], np.float32(1))
            L.router_w.zero_()
            L.router_b.copy_(torch.from_numpy(b))
            ref_t = replace(ref, router_w=np.zeros_like(ref.router_w), router_b=b)
            x = S.tokens(S.TokenSpec(T=2, token_set=90 + rep), L.H, 0)
            say(f"decode routing ties inside the top-k {name} rep={rep}")
            idx = _run(L, ref_t, x)
            assert set(idx[0].tolist()) == set(top.tolist())
    finally:
        L.router_w.copy_(w_save)
        L.router_b.copy_(b_save)
