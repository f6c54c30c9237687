"""GPU parity of int2 experts (the pages' experimental int2 packing, four
2-bit codes per byte, and matmul_i2 on the IDOT path) through the C ABI: the
device packer against the oracle's packer (the same codes and scales, in the
library's column order), whole layers against the oracle on the token-GEMV
path (routing, Q8(h) codes and scales bit-exact, outputs within the bar),
tiny and GLM-5.2-shaped, the cross-format identity on the device (int2 codes
written as int4 nibbles give the int4 kernels' outputs bit for bit). The
grouped path's int2 kernels are tested in test_gpu_grouped_formats.py."""
import numpy as np
import pytest
import torch
from dataclasses import replace

from int4_quantized_expert_sigmoid_amd import api, COLI_ACCUMULATE
from int4_quantized_expert_sigmoid_amd.synthetic import device_layer
from oracle import layers as OL
from oracle import oracle as O
from synth import synth as S

import parity as PR
from gpu_common import dev, rel_err, unreorder, ws_views

pytestmark = pytest.mark.gpu
TOL = 1e-4
TINY2 = replace(S.TINY, weight_bits=2)
GLM2 = replace(S.GLM52, weight_bits=2)


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.set_device(0)


def codes_of(q_nat: np.ndarray) -> np.ndarray:
    """Signed codes of natural-order int2 bytes (element 4j+i in field i of byte j)."""
    q = np.asarray(q_nat, dtype=np.uint8)
    c = np.stack([(q >> (2 * i)) & 3 for i in range(4)], axis=-1).reshape(q.shape[:-1] + (-1,)).astype(np.int16)
    return np.where(c >= 2, c - 4, c)


def library_order(codes: np.ndarray) -> np.ndarray:
    """The library's int2 bytes: in each 16-column group, byte k holds columns
    2k, 2k+1, 2k+8, 2k+9 in fields 0..3."""
    n = codes.shape[-1]
    g = (codes & 3).astype(np.uint8).reshape(codes.shape[:-1] + (n // 16, 16))
    out = np.zeros(codes.shape[:-1] + (n // 16, 4), np.uint8)
    for k in range(4):
        for i, c in enumerate((2 * k, 2 * k + 1, 2 * k + 8, 2 * k + 9)):
            out[..., k] |= g[..., c] << (2 * i)
    return out.reshape(codes.shape[:-1] + (n // 4,))


def as_int4(codes: np.ndarray) -> np.ndarray:
    n = (codes & 0xF).astype(np.uint8)
    return (n[..., 0::2] | (n[..., 1::2] << 4)).astype(np.uint8)


def test_pack_int2_dev_matches_oracle():
    r = np.random.default_rng(4)
    for w in (S.expert_matrix(GLM2, 0, 0, 5, S.DOWN), (r.standard_normal((64, 256)) * 0.02).astype(np.float32)):
        w = np.ascontiguousarray(w, np.float32)
        w[0, :] = 0.0                                   # zero row
        w[1, 3] = 1e30                                  # one huge element
        w[2, :8] = np.array([0.5, -0.5, 1.5, -1.5, 1.0, -1.0, 0.25, -0.75], np.float32) * np.abs(w[2]).max()
        q_o, s_o = O.pack_int2_rows(w)
        q_d = torch.empty((w.shape[0], w.shape[1] // 4), dtype=torch.uint8, device="cuda")
        s_d = torch.empty(w.shape[0], dtype=torch.float32, device="cuda")
        api.pack_int2_rows_dev(dev(w), q_d, s_d)
        torch.cuda.synchronize()
        assert np.array_equal(s_d.cpu().numpy(), s_o)
        assert np.array_equal(q_d.cpu().numpy(), library_order(codes_of(q_o)))


def _check(L, ref_tokens, T, ws, y, spec, cache):
    """Free-running against the oracle's tokens, with Q8(h) flips accounted."""
    assert ws_views(L, T, ws)["path"] == 0
    PR.check_tokens(spec, L, T, ws, y, ref_tokens, lambda e: cache[e], say)


@pytest.fixture(scope="module")
def tiny2():
    return device_layer(TINY2, 0, 0), OL.full_layer(TINY2, 0, 0)


@pytest.mark.parametrize("T", [1, 2, 3, 5, 8])
def test_forward_tiny_int2(tiny2, T):
    L, ref = tiny2
    x = S.tokens(S.TokenSpec(T=T, token_set=600 + T, outlier_channels=2), TINY2.H, 0)
    ws = api.workspace(L, T)
    say(f"forward tiny int2 T={T}")
    y = api.moe_forward(L, dev(x), ws).cpu().numpy()
    cache = OL.ExpertCache(TINY2, 0, 0)
    toks = [OL.forward_token(TINY2, cache, ref.router_w, ref.router_b, x[t]) for t in range(T)]
    _check(L, toks, T, ws, y, TINY2, cache)
    y_o, _, _ = O.moe_forward(ref, x)
    assert rel_err(y, y_o).max() <= TOL
    y0 = np.full((T, TINY2.H), 0.5, np.float32)
    yd = dev(y0)
    api.moe_forward(L, dev(x), ws, y=yd, flags=COLI_ACCUMULATE)
    assert rel_err(yd.cpu().numpy(), (np.float32(0.5) + y_o).astype(np.float32)).max() <= TOL


def test_int2_device_layer_equals_int4_on_shared_codes(tiny2):
    """The int2 layer's codes written as int4 nibbles (same scales): the int4
    kernels must give the int2 kernels' outputs bit for bit (a wrong field
    order, a leftover x64 factor or a row stride of the wrong format breaks it)."""
    L2, ref = tiny2
    L4 = api.MoELayer.empty(TINY2.H, TINY2.I, TINY2.E, TINY2.top_k)
    L4.router_w.copy_(L2.router_w); L4.router_b.copy_(L2.router_b)
    for name in ("gate_s", "up_s", "down_s"):
        getattr(L4, name).copy_(getattr(L2, name))
    for name in ("gate_q", "up_q", "down_q"):
        getattr(L4, name).copy_(torch.from_numpy(as_int4(codes_of(getattr(ref, name)))))
    for T in (1, 4, 8):
        x = S.tokens(S.TokenSpec(T=T, token_set=700 + T), TINY2.H, 0)
        y2 = api.moe_forward(L2, dev(x), api.workspace(L2, T)).cpu().numpy()
        y4 = api.moe_forward(L4, dev(x), api.workspace(L4, T)).cpu().numpy()
        say(f"int2 vs int4 codes T={T}: identical {np.mean(y2 == y4):.4f}")
        assert np.array_equal(y2, y4)


@pytest.fixture(scope="module")
def glm2():
    say("building the GLM-5.2-shaped int2 layer on the GPU")
    L = device_layer(GLM2, 0, 0)
    W, b = S.router(GLM2, 0, 0)
    yield L, OL.ExpertCache(GLM2, 0, 0), W, b
    del L
    torch.cuda.empty_cache()


@pytest.mark.parametrize("T", [1, 4])
def test_forward_glm_int2(glm2, T):
    L, cache, W, b = glm2
    x = S.tokens(S.TokenSpec(T=T, token_set=70 + T, outlier_channels=61), GLM2.H, 0)
    ws = api.workspace(L, T)
    say(f"forward GLM int2 T={T}")
    y = api.moe_forward(L, dev(x), ws).cpu().numpy()
    toks = [OL.forward_token(GLM2, cache, W, b, x[t]) for t in range(T)]
    _check(L, toks, T, ws, y, GLM2, cache)


@pytest.mark.parametrize("T", [1, 3, 8])
def test_experts_teacher_forced_tiny_int2(tiny2, T):
    """The expert stage alone (coli_moe_experts: the standalone GEMV gate/up
    and down kernels) fed the GPU's Q8(x) and the oracle's routing."""
    L, ref = tiny2
    x = S.tokens(S.TokenSpec(T=T, token_set=630 + T), TINY2.H, 0)
    xq, xs = api.quant_act_q8(dev(x))
    idx_o, w_o = O.route(ref.router_w, ref.router_b, x, TINY2.top_k)
    y = api.moe_experts(L, xq, xs, dev(idx_o), dev(w_o), api.workspace(L, T)).cpu().numpy()
    xq_h, xs_h = xq.cpu().numpy(), xs.cpu().numpy()
    cache = OL.ExpertCache(TINY2, 0, 0)
    for t in range(T):
        outs = [O.expert(*cache[int(e)].args(), xq_h[t], xs_h[t], wbits=2) for e in idx_o[t]]
        sh = O.expert(*cache[TINY2.E].args(), xq_h[t], xs_h[t], wbits=2)
        y_o = O.combine(np.stack([o.y for o in outs]), w_o[t], sh.y)
        assert np.array_equal(y[t], y_o), f"token {t}"
