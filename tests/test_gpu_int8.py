"""GPU parity of int8-weight experts (the pages' quantize_rows / dot_i8i8
path, one byte per weight, as the MTP head keeps) through the C ABI: the
device packer bit-exact against the host packer, and whole layers against
the oracle (routing bit-exact, per-pair Q8(h) and its scales bit-exact,
outputs within the bar) on the token-GEMV path, tiny and GLM-5.2-shaped, plus
the cross-format identity on the device (an int8 layer whose codes lie in
[-8, 7] gives the int4 layer's outputs bit for bit). The grouped path's int8
kernels are tested in test_gpu_grouped_int8.py."""
import ctypes

import numpy as np
import pytest
import torch

from int4_quantized_expert_sigmoid_amd import api, COLI_ACCUMULATE
from int4_quantized_expert_sigmoid_amd.synthetic import device_layer
from oracle import layers as OL
from oracle import oracle as O
from synth import synth as S

import parity as PR
from gpu_common import dev, rel_err, unreorder, ws_views

pytestmark = pytest.mark.gpu
TOL = 1e-4
TINY8 = S.LayerSpec(H=256, I=128, E=16, top_k=2, weight_bits=8)
GLM8 = S.LayerSpec(H=6144, I=2048, E=256, top_k=8, w_outlier_rate=0.001, weight_bits=8)


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.set_device(0)


@pytest.fixture(scope="module")
def tiny8():
    return device_layer(TINY8, 0, 0), OL.full_layer(TINY8, 0, 0)


def test_pack_int8_dev_matches_host():
    r = np.random.default_rng(3)
    for w in (S.expert_matrix(GLM8, 0, 0, 5, S.DOWN), (r.standard_normal((64, 256)) * 0.02).astype(np.float32)):
        w = np.ascontiguousarray(w, np.float32)
        w[0, :] = 0.0                                   # zero row
        w[1, 3] = 1e30                                  # one huge element
        q_h, s_h = api.pack_int8_rows(w)
        q_d = torch.empty(w.shape, dtype=torch.int8, device="cuda")
        s_d = torch.empty(w.shape[0], dtype=torch.float32, device="cuda")
        api.pack_int8_rows_dev(dev(w), q_d, s_d)
        torch.cuda.synchronize()
        assert np.array_equal(q_d.cpu().numpy(), q_h)
        assert np.array_equal(s_d.cpu().numpy(), s_h)


def _check(L, ref_tokens, T, ws, y, spec, cache):
    """Free-running against the oracle's tokens, with Q8(h) flips accounted."""
    assert ws_views(L, T, ws)["path"] == 0
    PR.check_tokens(spec, L, T, ws, y, ref_tokens, lambda e: cache[e], say)


@pytest.mark.parametrize("T", [1, 2, 3, 5, 8])
def test_forward_tiny_int8(tiny8, T):
    L, ref = tiny8
    x = S.tokens(S.TokenSpec(T=T, token_set=200 + T), TINY8.H, 0)
    ws = api.workspace(L, T)
    say(f"forward tiny int8 T={T}")
    y = api.moe_forward(L, dev(x), ws).cpu().numpy()
    cache = OL.ExpertCache(TINY8, 0, 0)
    toks = [OL.forward_token(TINY8, cache, ref.router_w, ref.router_b, x[t]) for t in range(T)]
    _check(L, toks, T, ws, y, TINY8, cache)
    y_o, _, _ = O.moe_forward(ref, x)
    assert rel_err(y, y_o).max() <= TOL
    # accumulate into a nonzero y
    y0 = np.full((T, TINY8.H), 0.5, np.float32)
    yd = dev(y0)
    api.moe_forward(L, dev(x), ws, y=yd, flags=COLI_ACCUMULATE)
    assert rel_err(yd.cpu().numpy(), (np.float32(0.5) + y_o).astype(np.float32)).max() <= TOL


def test_int8_device_layer_equals_int4_on_shared_codes():
    """Codes in [-8, 7] written both ways: the int8 kernels must reproduce the
    int4 kernels' outputs exactly (a wrong byte order, row stride or a
    leftover x16 factor breaks it)."""
    sp4 = S.LayerSpec(H=256, I=128, E=16, top_k=2)
    L4 = device_layer(sp4, 0, 0)
    L8 = api.MoELayer.empty(sp4.H, sp4.I, sp4.E, sp4.top_k, weight_bits=8)
    L8.router_w.copy_(L4.router_w); L8.router_b.copy_(L4.router_b)
    for name in ("gate_s", "up_s", "down_s"):
        getattr(L8, name).copy_(getattr(L4, name))
    for name in ("gate_q", "up_q", "down_q"):
        b = getattr(L4, name).cpu().numpy()
        lo = (b & 0xF).astype(np.int16); hi = (b >> 4).astype(np.int16)
        lo = np.where(lo >= 8, lo - 16, lo); hi = np.where(hi >= 8, hi - 16, hi)
        codes = np.empty(b.shape[:-1] + (2 * b.shape[-1],), np.int8)
        codes[..., 0::2] = lo; codes[..., 1::2] = hi                    # natural order
        n = codes.shape[-1]
        stored = np.empty_like(codes)
        i = np.arange(n)
        p = (i & 31 & ~7) + np.where(i & 1, 4 + ((i & 7) >> 1), (i & 7) >> 1)     # byte in its block
        stored[..., (p >> 4) * 16 * (n // 32) + (i >> 5) * 16 + (p & 15)] = codes
        getattr(L8, name).copy_(torch.from_numpy(stored))
    for T in (1, 4, 8):
        x = S.tokens(S.TokenSpec(T=T, token_set=300 + T), sp4.H, 0)
        y4 = api.moe_forward(L4, dev(x), api.workspace(L4, T)).cpu().numpy()
        y8 = api.moe_forward(L8, dev(x), api.workspace(L8, T)).cpu().numpy()
        say(f"int8 vs int4 codes T={T}: identical {np.mean(y4 == y8):.4f}")
        assert np.array_equal(y4, y8)


@pytest.fixture(scope="module")
def glm8():
    say("building the GLM-5.2-shaped int8 layer on the GPU")
    L = device_layer(GLM8, 0, 0)
    W, b = S.router(GLM8, 0, 0)
    return L, OL.ExpertCache(GLM8, 0, 0), W, b


@pytest.mark.parametrize("T", [1, 4])
def test_forward_glm_int8(glm8, T):
    L, cache, W, b = glm8
    x = S.tokens(S.TokenSpec(T=T, token_set=50 + T, outlier_channels=61), GLM8.H, 0)
    ws = api.workspace(L, T)
    say(f"forward GLM int8 T={T}")
    y = api.moe_forward(L, dev(x), ws).cpu().numpy()
    toks = [OL.forward_token(GLM8, cache, W, b, x[t]) for t in range(T)]
    _check(L, toks, T, ws, y, GLM8, cache)


@pytest.mark.parametrize("T", [1, 3, 8])
def test_experts_teacher_forced_tiny_int8(tiny8, T):
    """The expert stage alone (coli_moe_experts: the standalone GEMV gate/up
    and down kernels) fed the GPU's Q8(x) and the oracle's routing."""
    L, ref = tiny8
    x = S.tokens(S.TokenSpec(T=T, token_set=230 + T), TINY8.H, 0)
    xq, xs = api.quant_act_q8(dev(x))
    idx_o, w_o = O.route(ref.router_w, ref.router_b, x, TINY8.top_k)
    y = api.moe_experts(L, xq, xs, dev(idx_o), dev(w_o), api.workspace(L, T)).cpu().numpy()
    xq_h, xs_h = xq.cpu().numpy(), xs.cpu().numpy()
    cache = OL.ExpertCache(TINY8, 0, 0)
    for t in range(T):
        outs = [O.expert(*cache[int(e)].args(), xq_h[t], xs_h[t]) for e in idx_o[t]]
        sh = O.expert(*cache[TINY8.E].args(), xq_h[t], xs_h[t])
        y_o = O.combine(np.stack([o.y for o in outs]), w_o[t], sh.y)
        assert np.array_equal(y[t], y_o), f"token {t}"
