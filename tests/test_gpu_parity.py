"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bar: bit-exact for integer/byte/index results (Q8 codes of x, int4 bytes,
int32 block dots, expert indices); fp32 outputs within
max_i |y_i - o_i| / max(|o_i|, rms(o)) <= 1e-4. Whole layers run free: the
GPU and the oracle each quantise their own h, so a Q8(h) code may move by
one where h * (1/d) sits on a rounding boundary; every such move is logged
and accounted for (tests/parity.py). The teacher-forced stage test feeds the
oracle the GPU's own Q8(x) and Q8(h) and holds every code bit for bit. The
kernels sum block terms in f64 like the oracle, so most fp32 outputs come out
bit-identical; the tests report how many.
"""
import numpy as np
import pytest
import torch

from int4_quantized_expert_sigmoid_amd import api, COLI_ACCUMULATE, COLI_PATH_GEMV
from int4_quantized_expert_sigmoid_amd.synthetic import device_layer
from oracle import layers as OL
from oracle import oracle as O
from synth import synth as S

import parity as PR
from gpu_common import dev, rel_err, unreorder, ws_views

pytestmark = pytest.mark.gpu
TOL = 1e-4


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


@pytest.fixture(scope="module")
def glm_layer():
    say("building GLM-5.2-shaped layer on device (H=6144 I=2048 E=256+1, seed 0)")
    L = device_layer(S.GLM52, 0, 0)
    torch.cuda.synchronize()
    W, b = S.router(S.GLM52, 0, 0)
    return L, OL.ExpertCache(S.GLM52, 0, 0), W, b


@pytest.fixture(scope="module")
def tiny_layer():
    L = device_layer(S.TINY, 0, 0)
    return L, OL.full_layer(S.TINY, 0, 0)


# ------------------------------------------------------------- generator
def test_device_generator_matches_host():
    spec = S.GLM52
    n = spec.I * spec.H
    buf = torch.empty(n, dtype=torch.float32, device="cuda")
    for e, m in ((3, S.GATE), (256, S.DOWN)):
        say(f"synth device vs host: expert {e} matrix {m}")
        S.dev_expert_matrix(buf.data_ptr(), spec, 0, 0, e, m, hip_stream=torch.cuda.current_stream().cuda_stream)
        host = S.expert_matrix(spec, 0, 0, e, m)
        d = buf.view(host.shape).cpu().numpy()
        assert np.array_equal(d.view(np.uint32), host.view(np.uint32))


# ------------------------------------------------------------- quantisers
def _edge_rows():
    x = np.zeros((4, 128), np.float32)
    x[1, 0] = 127.0
    x[1, 1:9] = [2.5, 3.5, -2.5, -3.5, 0.5, -0.5, 1.5, 126.5]    # half-even ties
    x[2, 32] = np.float32(1e-39)                                 # subnormal scale, 1/d = inf
    x[2, 40] = np.float32(-3e-40)
    x[3] = np.linspace(-3, 3, 128, dtype=np.float32)
    return x


@pytest.mark.parametrize("name", ["tiny_T1", "glm52_mtp_verify_T4", "glm52_prefill_T512", "edge"])
def test_quant_act_q8_bitexact(name):
    if name == "edge":
        x = _edge_rows()
    else:
        wl = S.WORKLOADS[name]
        x = S.tokens(wl.tokens, wl.layer.H, 0)
    say(f"quant_act_q8 {name} shape {x.shape}")
    xq, xs = api.quant_act_q8(dev(x))
    qo, do = O.quant_q8(x)
    assert np.array_equal(xq.cpu().numpy(), qo)
    assert np.array_equal(xs.cpu().numpy().view(np.uint32), do.view(np.uint32))


def test_pack_int4_dev_bitexact():
    for rows, cols, e, m in ((2048, 6144, 11, S.UP), (6144, 2048, 256, S.DOWN)):
        w = S.expert_matrix(S.GLM52, 0, 0, e, m)
        say(f"pack_int4_rows_dev {w.shape}")
        q = torch.empty((rows, cols // 2), dtype=torch.uint8, device="cuda")
        s = torch.empty(rows, dtype=torch.float32, device="cuda")
        api.pack_int4_rows_dev(dev(w), q, s)
        qo, so = O.pack_int4_rows(w)
        assert np.array_equal(q.cpu().numpy(), qo)
        assert np.array_equal(s.cpu().numpy().view(np.uint32), so.view(np.uint32))
    edge = np.zeros((4, 64), np.float32)
    edge[1, :] = 1e-40
    edge[2, 5] = -3.5
    edge[3, :] = np.linspace(-7, 7, 64)
    q = torch.empty((4, 32), dtype=torch.uint8, device="cuda")
    s = torch.empty(4, dtype=torch.float32, device="cuda")
    api.pack_int4_rows_dev(dev(edge), q, s)
    qo, so = O.pack_int4_rows(edge)
    assert np.array_equal(q.cpu().numpy(), qo) and np.array_equal(s.cpu().numpy(), so)


@pytest.mark.parametrize("rows,cols", [(5, 32), (300, 6144), (97, 2048)])
def test_block_dots_bitexact(rows, cols):
    r = np.random.default_rng(rows)
    q4 = r.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    q8 = r.integers(-127, 128, size=cols).astype(np.int8)
    q8[:32] = np.int8(-127)                                       # extreme products
    q4[:, :16] = 0x88                                             # code -8 in both nibbles
    say(f"block dots {rows}x{cols}")
    S_ = api.debug_block_dots(dev(q4), dev(q8)).cpu().numpy()
    assert np.array_equal(S_, O.block_dots(q4, q8))


# ------------------------------------------------------------------ router
@pytest.mark.parametrize("name", ["glm52_decode_T1", "glm52_mtp_verify_T4"])
def test_route_glm(glm_layer, name):
    L, cache, W, b = glm_layer
    wl = S.WORKLOADS[name]
    x = S.tokens(wl.tokens, wl.layer.H, 0)
    ws = api.workspace(L, x.shape[0])
    idx, w = api.moe_route(L, dev(x), ws)
    idx_o, w_o, keys = O.route(W, b, x, 8, want_keys=True)
    say(f"route {name}: gpu {idx.cpu().numpy().tolist()}")
    assert np.array_equal(idx.cpu().numpy(), idx_o)
    wg = w.cpu().numpy()
    assert np.max(np.abs(wg - w_o) / np.abs(w_o)) <= 1e-6
    say(f"route weights bit-identical: {np.mean(wg == w_o):.3f}")


def test_route_group_limited_and_scale(tiny_layer):
    L, ref = tiny_layer
    x = S.tokens(S.TokenSpec(T=6), S.TINY.H, 3)
    for ng, tg, rs in ((4, 2, 2.5), (8, 8, 1.0), (16, 3, 1.0)):
        L.n_group, L.topk_group, L.route_scale = ng, tg, rs
        ws = api.workspace(L, 6)
        idx, w = api.moe_route(L, dev(x), ws)
        io, wo = O.route(ref.router_w, ref.router_b, x, S.TINY.top_k, ng, tg, rs)
        assert np.array_equal(idx.cpu().numpy(), io), (ng, tg)
        assert np.allclose(w.cpu().numpy(), wo, rtol=1e-6, atol=0)
    L.n_group, L.topk_group, L.route_scale = 1, 1, 1.0


# ------------------------------------------------------------ whole layer
def _check_pairs(spec, L, T, ws, y, tok_results, cache, flags=0):
    """Free-running against the oracle's tokens (tests/parity.py): routing
    bit for bit, every moved Q8(h) code shown to sit on a rounding boundary
    and to account for the outputs it moves, everything else within the bar.
    Returns the fraction of h values bit-identical to the oracle's."""
    st = PR.check_tokens(spec, L, T, ws, y, tok_results, lambda e: cache[e], say, flags=flags)
    return st["h_bit_identical"]


@pytest.mark.parametrize("T", [1, 3, 5, 8])
def test_forward_tiny(tiny_layer, T):
    L, ref = tiny_layer
    x = S.tokens(S.TokenSpec(T=T, token_set=T), S.TINY.H, 0)
    ws = api.workspace(L, T)
    say(f"forward tiny T={T}")
    y = api.moe_forward(L, dev(x), ws).cpu().numpy()
    y_o, idx_o, w_o = O.moe_forward(ref, x)
    cache = OL.ExpertCache(S.TINY, 0, 0)
    toks = [OL.forward_token(S.TINY, cache, ref.router_w, ref.router_b, x[t]) for t in range(T)]
    frac = _check_pairs(S.TINY, L, T, ws, y, toks, cache)
    err = rel_err(y, y_o).max()
    say(f"  max rel {err:.2e}, outputs bit-identical {np.mean(y == y_o):.4f}, h bit-identical {frac:.4f}")
    assert err <= TOL


def test_forward_zero_token_and_accumulate(tiny_layer):
    L, ref = tiny_layer
    x = S.tokens(S.TokenSpec(T=2), S.TINY.H, 5)
    x[1] = 0.0                                   # Q8 scale 0, every code 0
    ws = api.workspace(L, 2)
    y0 = dev(np.full((2, S.TINY.H), 0.25, np.float32))
    y = api.moe_forward(L, dev(x), ws, y=y0, flags=COLI_ACCUMULATE).cpu().numpy()
    y_o, _, _ = O.moe_forward(ref, x)
    acc = (np.float32(0.25) + y_o).astype(np.float32)
    assert np.all(y_o[1] == 0.0)
    assert rel_err(y, acc).max() <= TOL


def _glm_oracle_tokens(cache, W, b, x):
    return [OL.forward_token(S.GLM52, cache, W, b, x[t]) for t in range(x.shape[0])]


def test_forward_glm_decode_T1(glm_layer):
    L, cache, W, b = glm_layer
    wl = S.WORKLOADS["glm52_decode_T1"]
    x = S.tokens(wl.tokens, S.GLM52.H, 0)
    ws = api.workspace(L, 1)
    say("forward GLM decode T=1")
    y = api.moe_forward(L, dev(x), ws).cpu().numpy()
    toks = _glm_oracle_tokens(cache, W, b, x)
    frac = _check_pairs(S.GLM52, L, 1, ws, y, toks, cache)
    y_o = np.stack([t.y for t in toks])
    err = rel_err(y, y_o).max()
    say(f"  experts {toks[0].idx.tolist()} max rel {err:.2e} bit-identical {np.mean(y == y_o):.4f} h {frac:.4f}")
    assert err <= TOL


def test_forward_glm_mtp_verify_T4_and_batch_invariance(glm_layer):
    L, cache, W, b = glm_layer
    wl = S.WORKLOADS["glm52_mtp_verify_T4"]
    x = S.tokens(wl.tokens, S.GLM52.H, 0)
    ws = api.workspace(L, 4)
    say("forward GLM MTP-verify T=4")
    y = api.moe_forward(L, dev(x), ws).cpu().numpy()
    toks = _glm_oracle_tokens(cache, W, b, x)
    union = len({int(e) for t in toks for e in t.idx})
    frac = _check_pairs(S.GLM52, L, 4, ws, y, toks, cache)
    y_o = np.stack([t.y for t in toks])
    err = rel_err(y, y_o).max()
    say(f"  union {union} of 32 picks, max rel {err:.2e}, bit-identical {np.mean(y == y_o):.4f}, h {frac:.4f}")
    assert err <= TOL
    ws1 = api.workspace(L, 1)
    for t in range(4):
        y1 = api.moe_forward(L, dev(x[t: t + 1]), ws1).cpu().numpy()
        assert np.array_equal(y1[0], y[t]), f"token {t} differs between T=4 and T=1"


def test_forward_glm_T8_many_units(glm_layer):
    """Eight independent tokens at GLM shape: a union of about 60 items, so
    the gate/up launch's routed workgroups (no more than fit on the device)
    each take several units of the union. Every pair and token against the
    oracle, and each token equal to its own T=1 call."""
    L, cache, W, b = glm_layer
    x = S.tokens(S.TokenSpec(T=8, token_set=21, outlier_channels=61), S.GLM52.H, 0)
    ws = api.workspace(L, 8)
    say("forward GLM T=8 independent tokens")
    y = api.moe_forward(L, dev(x), ws).cpu().numpy()
    toks = _glm_oracle_tokens(cache, W, b, x)
    union = len({int(e) for t in toks for e in t.idx})
    frac = _check_pairs(S.GLM52, L, 8, ws, y, toks, cache)
    y_o = np.stack([t.y for t in toks])
    err = rel_err(y, y_o).max()
    say(f"  union {union} of 64 picks, max rel {err:.2e}, bit-identical {np.mean(y == y_o):.4f}, h {frac:.4f}")
    assert union > 40 and err <= TOL
    ws1 = api.workspace(L, 1)
    for t in range(8):
        y1 = api.moe_forward(L, dev(x[t: t + 1]), ws1).cpu().numpy()
        assert np.array_equal(y1[0], y[t]), f"token {t} differs between T=8 and T=1"


def test_experts_teacher_forced_glm(glm_layer):
    """Stage-isolated: the expert stage fed the GPU's own Q8(x) and the
    oracle's routing; every integer boundary bit-exact."""
    L, cache, W, b = glm_layer
    x = S.tokens(S.TokenSpec(T=2, token_set=7, outlier_channels=61), S.GLM52.H, 0)
    xq, xs = api.quant_act_q8(dev(x))
    idx_o, w_o = O.route(W, b, x, 8)
    ws = api.workspace(L, 2)
    y = api.moe_experts(L, xq, xs, dev(idx_o), dev(w_o), ws).cpu().numpy()
    v = ws_views(L, 2, ws)
    xq_h, xs_h = xq.cpu().numpy(), xs.cpu().numpy()
    for t in range(2):
        outs = [O.expert(*cache[int(e)].args(), xq_h[t], xs_h[t]) for e in idx_o[t]]
        sh = O.expert(*cache[S.GLM52.E].args(), xq_h[t], xs_h[t])
        y_o = O.combine(np.stack([o.y for o in outs]), w_o[t], sh.y)
        assert rel_err(y[t][None], y_o[None]).max() <= TOL
        # the gate/up stage from the same Q8(x): h and its Q8 codes bit for
        # bit; the down stage fed the GPU's own Q8(h): outputs bit for bit
        pairs = list(v["pair_of"][t]) + [v["shared_pair"][t]]
        experts = list(idx_o[t]) + [S.GLM52.E]
        for p, e, eo in zip(pairs, experts, outs + [sh]):
            assert np.array_equal(v["h"][p], eo.h) and np.array_equal(unreorder(v["hq"][p]), eo.hq)
            assert np.array_equal(v["hs"][p], eo.hs)
            ye_o = PR.down_rowdot(S.GLM52, cache[int(e)], unreorder(v["hq"][p]), v["hs"][p])
            assert np.array_equal(v["ye"][p], ye_o), f"token {t} expert {e}: down stage differs"


def test_rmsnorm_and_two_layer_chain(glm_layer):
    """x <- x + MoE(RMSNorm(x)) for two layers, each checked against the oracle
    fed the GPU's own x_l (teacher-forced per layer)."""
    L0, cache0, W0, b0 = glm_layer
    say("building second GLM layer (layer index 1)")
    L1 = device_layer(S.GLM52, 0, 1)
    W1, b1 = S.router(S.GLM52, 0, 1)
    cache1 = OL.ExpertCache(S.GLM52, 0, 1)
    x = S.tokens(S.TokenSpec(T=1, token_set=11, outlier_channels=61), S.GLM52.H, 0)
    xd = dev(x)
    ws = api.workspace(L0, 1)
    for li, (L, cache, W, b) in enumerate(((L0, cache0, W0, b0), (L1, cache1, W1, b1))):
        g = S.rms_gamma(S.GLM52.H, 0, li)
        x_in = xd.cpu().numpy()
        xn = api.rmsnorm(xd, dev(g), 1e-6)
        xn_o = O.rmsnorm(x_in, g, 1e-6)
        xn_h = xn.cpu().numpy()
        assert rel_err(xn_h, xn_o).max() <= 1e-6
        api.moe_forward(L, xn, ws, y=xd, flags=COLI_ACCUMULATE)
        r = OL.forward_token(S.GLM52, cache, W, b, xn_h[0])
        x_o = (x_in[0] + r.y).astype(np.float32)
        err = rel_err(xd.cpu().numpy(), x_o[None]).max()
        say(f"  chain layer {li}: max rel {err:.2e}")
        assert err <= TOL
    del L1
    torch.cuda.empty_cache()
