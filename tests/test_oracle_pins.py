"""Pins of the CPU oracle against things other than itself.

Each test ties one oracle step to an exact round trip, an exactly
representable special case that reduces to an integer matmul (numpy), a brute
force over all candidates, a closed form, or the statistical law of rounding
error. A plausible slip in the oracle (wrong nibble order, a dropped block
scale, a transposed operand, round-half-away instead of half-even, the bias
leaking into the weights, a wrong combine order) fails at least one of them.
"""
import itertools
import math

import numpy as np
import pytest

from oracle import oracle as O
from oracle import layers as OL
from synth import synth as S


def rng(seed=0):
    return np.random.default_rng(seed)


# ------------------------------------------------------------------ P1 pack
def test_nibble_decoding_all_bytes_matches_int8_shifts():
    b = np.arange(256, dtype=np.uint8)
    lo_ref = (b.astype(np.int8) << 4).astype(np.int8) >> 4     # arithmetic shift, numpy
    hi_ref = b.astype(np.int8) >> 4
    assert [O.nibble(int(v), 0) for v in b] == lo_ref.tolist()
    assert [O.nibble(int(v), 1) for v in b] == hi_ref.tolist()


def test_pack_exact_codes_even_index_in_low_nibble():
    # amax = 7 gives d = 1 exactly, so w == code and packing is lossless
    codes = np.array([[c_even, c_odd] for c_even in range(-7, 8) for c_odd in range(-7, 8)],
                     dtype=np.float32).reshape(1, -1)
    codes = np.concatenate([codes, np.array([[7.0, -7.0]], np.float32)], axis=1)
    q, s = O.pack_int4_rows(codes)
    assert s[0] == 1.0
    expect = ((codes[0, 0::2].astype(np.int64) & 0xF) | ((codes[0, 1::2].astype(np.int64) & 0xF) << 4))
    assert np.array_equal(q[0].astype(np.int64), expect)
    assert np.array_equal(O.unpack_int4_rows(q, s), codes.astype(np.float64))


def test_pack_int4_rounds_half_to_even():
    # amax = 7 gives d = 1 exactly, so w * (1/d) == w: every k.5 is a tie,
    # and round-half-to-even gives the even neighbour (half away from zero
    # would give 1, 2, 3, 4, 5, 6, 7)
    ties = np.array([0.5, 1.5, 2.5, 3.5, 4.5, 5.5, 6.5], np.float32)
    w = np.concatenate([ties, -ties, [7.0, 0.0]]).astype(np.float32).reshape(1, -1)
    q, s = O.pack_int4_rows(w)
    assert s[0] == 1.0
    codes = O.unpack_int4_rows(q, s)[0]
    assert codes.tolist() == [0, 2, 2, 4, 4, 6, 6, 0, -2, -2, -4, -4, -6, -6, 7, 0]


# ------------------------------------------------------------- P2 invariants
@pytest.mark.parametrize("cols", [32, 256, 6144])
def test_int4_invariants(cols):
    w = (rng(cols).standard_normal((64, cols)) * 0.02).astype(np.float32)
    w[3] = 0.0
    q, s = O.pack_int4_rows(w)
    dq = O.unpack_int4_rows(q, s)
    codes = dq / np.where(s == 0, 1, s)[:, None]
    amax = np.abs(w).max(axis=1)
    assert np.array_equal(s, (amax / np.float32(7)).astype(np.float32))
    assert s[3] == 0 and np.all(q[3] == 0)
    assert codes.min() >= -7 and codes.max() <= 7                   # -8 never produced
    nz = np.arange(64) != 3
    arg = np.abs(w).argmax(axis=1)
    assert np.all(np.abs(codes[nz, arg[nz]]) == 7)
    err = np.abs(w.astype(np.float64) - dq)
    assert np.all(err <= s[:, None].astype(np.float64) * 0.5 * (1 + 1e-6))


def test_q8_invariants_and_zero_block():
    x = rng(1).standard_normal(32 * 50).astype(np.float32)
    x[64:96] = 0.0
    q, d = O.quant_q8(x)
    blocks = x.reshape(-1, 32)
    amax = np.abs(blocks).max(axis=1)
    assert np.array_equal(d, (amax / np.float32(127)).astype(np.float32))
    assert d[2] == 0 and np.all(q[64:96] == 0)
    qb = q.reshape(-1, 32).astype(np.int64)
    assert qb.min() >= -127 and qb.max() <= 127
    nz = amax > 0
    assert np.all(np.abs(qb[nz, np.abs(blocks).argmax(axis=1)[nz]]) == 127)
    err = np.abs(blocks.astype(np.float64) - qb * d[:, None].astype(np.float64))
    assert np.all(err <= d[:, None] * 0.5 * (1 + 1e-6))


def test_q8_rounds_half_to_even():
    # amax 127 gives d = 1 and id = 1, so x*id = x exactly; .5 cases tie
    x = np.zeros(32, np.float32)
    x[0] = 127.0
    x[1:9] = [2.5, 3.5, -2.5, -3.5, 0.5, -0.5, 1.5, 126.5]
    q, d = O.quant_q8(x)
    assert d[0] == 1.0
    assert q[1:9].tolist() == [2, 4, -2, -4, 0, 0, 2, 126]


def test_q8_subnormal_block_is_finite():
    x = np.zeros(32, np.float32)
    x[0] = np.float32(1e-39)           # d = amax/127 is subnormal, 1/d overflows to inf
    x[5] = np.float32(-3e-40)
    q, d = O.quant_q8(x)
    assert np.isfinite(d[0]) and d[0] > 0
    assert q[0] == 127 and q[5] == -127 and np.all(q[[1, 2, 3, 4]] == 0)


# ---------------------------------------------- P3 exactly representable case
def _exact_case(rows, cols, seed):
    r = rng(seed)
    codes = r.integers(-7, 8, size=(rows, cols))
    codes[:, 0] = 7 * np.where(r.random(rows) < 0.5, 1, -1)        # amax = 7 * 2^-6 in every row
    w = (codes * 2.0 ** -6).astype(np.float32)
    xi = r.integers(-127, 128, size=cols)
    xi.reshape(-1, 32)[:, 5] = 127                                   # d_b = 1 in every block
    return codes, w, xi, xi.astype(np.float32)


def test_block_dots_equal_integer_matmul():
    codes, w, xi, x = _exact_case(40, 256, 2)
    q4, s4 = O.pack_int4_rows(w)
    q8, d8 = O.quant_q8(x)
    assert np.all(s4 == 2.0 ** -6) and np.all(d8 == 1.0) and np.array_equal(q8, xi.astype(np.int8))
    S_ = O.block_dots(q4, q8)
    ref = np.einsum("rbk,bk->rb", codes.reshape(40, -1, 32).astype(np.int64), xi.reshape(-1, 32))
    assert np.array_equal(S_, ref)


def test_rowdot_equals_exact_dot_times_scale():
    codes, w, xi, x = _exact_case(64, 6144, 3)
    q4, s4 = O.pack_int4_rows(w)
    q8, d8 = O.quant_q8(x)
    out = O.rowdot(q4, s4, q8, d8)
    exact = (codes.astype(np.int64) @ xi.astype(np.int64)).astype(np.float64) * 2.0 ** -6
    assert np.array_equal(out, exact.astype(np.float32))


def test_rowdot_uses_each_block_scale():
    # blocks with different power-of-two scales: still exact
    codes, w, xi, x = _exact_case(8, 128, 4)
    scale = np.repeat(2.0 ** np.array([0, -3, 4, 1]), 32)
    x2 = (x * scale).astype(np.float32)
    q4, s4 = O.pack_int4_rows(w)
    q8, d8 = O.quant_q8(x2)
    assert np.array_equal(d8, (2.0 ** np.array([0, -3, 4, 1])).astype(np.float32))
    out = O.rowdot(q4, s4, q8, d8)
    exact = (codes.astype(np.float64) * 2.0 ** -6) @ (xi * scale)
    assert np.array_equal(out, exact.astype(np.float32))


# ------------------------------------------------------------ P4/P6 routing
def _keys_np(W, b, x):
    z = W.astype(np.float64) @ x.astype(np.float64)
    s = 1.0 / (1.0 + np.exp(-z))
    return s, s + b.astype(np.float64)


@pytest.mark.parametrize("seed", range(5))
def test_route_top_k_is_best_subset(seed):
    r = rng(10 + seed)
    E, H, k = 8, 64, 3
    W = (r.standard_normal((E, H)) / 8).astype(np.float32)
    b = (r.standard_normal(E) * 0.3).astype(np.float32)
    x = r.standard_normal((2, H)).astype(np.float32)
    idx, w = O.route(W, b, x, k, route_scale=2.5)
    for t in range(2):
        s, key = _keys_np(W, b, x[t])
        best = max(itertools.combinations(range(E), k), key=lambda c: sum(key[list(c)]))
        assert sorted(idx[t].tolist()) == sorted(best)
        assert np.all(np.diff(key[idx[t]]) <= 0)                   # largest key first
        ws = s[idx[t]] / s[idx[t]].sum() * 2.5                      # weights from unbiased s
        assert np.allclose(w[t], ws, rtol=1e-6)
        assert abs(w[t].sum() - 2.5) < 1e-5


def test_route_without_bias_is_top_k_of_logits():
    r = rng(20)
    E, H, k = 256, 512, 8
    W = (r.standard_normal((E, H)) / math.sqrt(H)).astype(np.float32)
    x = r.standard_normal((6, H)).astype(np.float32)
    idx, _ = O.route(W, np.zeros(E, np.float32), x, k)
    z = x.astype(np.float64) @ W.astype(np.float64).T
    assert np.array_equal(idx, np.argsort(-z, axis=1, kind="stable")[:, :k])


def test_route_all_experts_and_ties():
    E, H = 6, 32
    W = np.zeros((E, H), np.float32)                                # all logits 0: all keys tie
    idx, w = O.route(W, np.zeros(E, np.float32), np.ones((1, H), np.float32), E, route_scale=1.0)
    assert idx[0].tolist() == list(range(E))                         # ties to the lower index
    assert np.allclose(w, 1.0 / E) and abs(w.sum() - 1.0) < 1e-6


def test_route_group_limited():
    # keys built so the group choice is forced: groups {0..3},{4..7},{8..11},{12..15}
    E, H, k = 16, 16, 4
    W = np.zeros((E, H), np.float32)
    b = np.array([0.30, 0.29, 0.0, 0.0, 0.50, 0.0, 0.0, 0.0,
                  0.20, 0.20, 0.20, 0.0, 0.25, 0.24, 0.0, 0.0], np.float32)
    x = np.zeros((1, H), np.float32)
    # group scores (top-2 sums): g0 .59, g1 .50, g2 .40, g3 .49 -> keep g0, g1
    idx, _ = O.route(W, b, x, k, n_group=4, topk_group=2)
    assert idx[0].tolist() == [4, 0, 1, 2]
    idx_all, _ = O.route(W, b, x, k, n_group=4, topk_group=4)
    idx_plain, _ = O.route(W, b, x, k)
    assert np.array_equal(idx_all, idx_plain) and idx_plain[0].tolist() == [4, 0, 1, 12]


# ------------------------------------------------------- P5 rounding-error law
def test_idot_error_matches_uniform_rounding_law():
    # gate projection with and without Q8 of x: E[err^2] = sum_b d_b^2/12 * sum_k w~_k^2
    spec = S.LayerSpec(H=1024, I=4096, E=1, top_k=1)
    w = S.expert_matrix(spec, 0, 0, 0, S.GATE)
    q4, s4 = O.pack_int4_rows(w)
    wd = O.unpack_int4_rows(q4, s4)
    x = rng(5).standard_normal(spec.H).astype(np.float32)
    q8, d8 = O.quant_q8(x)
    idot = O.rowdot(q4, s4, q8, d8).astype(np.float64)
    dense = wd @ x.astype(np.float64)
    err2 = ((idot - dense) ** 2).mean()
    pred = ((wd.reshape(spec.I, -1, 32) ** 2).sum(axis=2) @ (d8.astype(np.float64) ** 2 / 12)).mean()
    assert abs(err2 / pred - 1) < 0.05
    rel = math.sqrt(err2 / (dense ** 2).mean())
    assert 0.003 < rel < 0.008                 # ~0.5% for N(0,1) activations


def test_expert_idot_close_to_dense_reference():
    wl = S.WORKLOADS["tiny_T1"]
    ex = OL.packed_expert(wl.layer, 0, 0, 5)
    x = S.tokens(wl.tokens, wl.layer.H, 0)[0]
    xq, xs = O.quant_q8(x)
    o = O.expert(*ex.args(), xq, xs)
    ref = O.expert_dense(*ex.args(), x)
    rel = np.sqrt(((o.y - ref) ** 2).mean() / (ref ** 2).mean())
    assert rel < 0.02                           # two activation quantisations, ~0.5% each
    # intermediates are mutually consistent
    hq, hs = O.quant_q8(o.h)
    assert np.array_equal(hq, o.hq) and np.array_equal(hs, o.hs)
    assert np.array_equal(o.y, O.rowdot(ex.down_q, ex.down_s, o.hq, o.hs))


def test_expert_dense_exact_case_is_f64_matmul():
    """O10 with exactly representable weights (codes * 2^-6) and integer
    activations: g and u are exact, so they equal the integer matmul; h and
    y then follow the f64 formula, which a numpy matmul reproduces to
    rounding (a transposed operand, a dropped term or a wrong sign would be
    off by far more)."""
    codes_g, wg, xi, x = _exact_case(32, 64, 16)
    codes_u, wu, _, _ = _exact_case(32, 64, 17)
    codes_d, wd, _, _ = _exact_case(64, 32, 18)
    gq, gs = O.pack_int4_rows(wg)
    uq, us = O.pack_int4_rows(wu)
    dq, ds = O.pack_int4_rows(wd)
    y = O.expert_dense(gq, gs, uq, us, dq, ds, x)
    g = (codes_g.astype(np.int64) @ xi.astype(np.int64)) * 2.0 ** -6       # exact
    u = (codes_u.astype(np.int64) @ xi.astype(np.int64)) * 2.0 ** -6
    h = g / (1.0 + np.exp(-g)) * u
    y_ref = (codes_d.astype(np.float64) * 2.0 ** -6) @ h
    assert np.allclose(y, y_ref, rtol=1e-12, atol=1e-12 * np.abs(y_ref).max())
    # the same weights with x quantised losslessly (d_b = 1): O7's g and u are O10's
    xq, xs = O.quant_q8(x)
    o = O.expert(gq, gs, uq, us, dq, ds, xq, xs)
    assert np.array_equal(o.g.astype(np.float64), g) and np.array_equal(o.u.astype(np.float64), u)


def test_expert_swiglu_exact_case():
    # exactly representable gate/up/x: g and u are exact, h = silu(g)*u in double
    codes_g, wg, xi, x = _exact_case(32, 64, 6)
    codes_u, wu, _, _ = _exact_case(32, 64, 7)
    wdown = (_exact_case(64, 32, 8)[1])
    gq, gs = O.pack_int4_rows(wg)
    uq, us = O.pack_int4_rows(wu)
    dq, ds = O.pack_int4_rows(wdown)
    xq, xs = O.quant_q8(x)
    o = O.expert(gq, gs, uq, us, dq, ds, xq, xs)
    g = codes_g.astype(np.float64) @ xi * 2.0 ** -6
    u = codes_u.astype(np.float64) @ xi * 2.0 ** -6
    assert np.array_equal(o.g, g.astype(np.float32)) and np.array_equal(o.u, u.astype(np.float32))
    h = (g / (1 + np.exp(-g)) * u).astype(np.float32)
    assert np.allclose(o.h, h, rtol=2e-7, atol=0)


# ------------------------------------------------------------ P7 combine
def test_combine_order_and_shared():
    y = np.array([[1.0, 2.0], [3.0, -4.0]], np.float32)
    out = O.combine(y, np.array([0.25, 0.5], np.float32), np.array([10.0, 20.0], np.float32))
    assert out.tolist() == [11.75, 18.5]
    assert O.combine(y, np.array([0.25, 0.5], np.float32)).tolist() == [1.75, -1.5]


def test_dense_mixture_when_all_experts_chosen():
    spec = S.LayerSpec(H=64, I=32, E=4, top_k=4)
    L = OL.full_layer(spec, 1, 0)
    L.router_b = np.zeros_like(L.router_b)
    x = S.tokens(S.TokenSpec(T=2), spec.H, 1)
    y, idx, w = O.moe_forward(L, x)
    for t in range(2):
        s, _ = _keys_np(L.router_w, L.router_b, x[t])
        xq, xs = O.quant_q8(x[t])
        ys = [O.expert(L.gate_q[e], L.gate_s[e], L.up_q[e], L.up_s[e], L.down_q[e], L.down_s[e],
                       xq, xs).y.astype(np.float64) for e in range(5)]
        mix = sum(s[e] / s.sum() * ys[e] for e in range(4)) + ys[4]
        assert np.allclose(y[t], mix, rtol=1e-5, atol=1e-7)


def test_single_expert_layer_is_expert_plus_shared():
    spec = S.LayerSpec(H=64, I=32, E=1, top_k=1)
    L = OL.full_layer(spec, 2, 0)
    x = S.tokens(S.TokenSpec(T=1), spec.H, 2)
    y, idx, w = O.moe_forward(L, x)
    xq, xs = O.quant_q8(x[0])
    e0 = O.expert(L.gate_q[0], L.gate_s[0], L.up_q[0], L.up_s[0], L.down_q[0], L.down_s[0], xq, xs).y
    sh = O.expert(L.gate_q[1], L.gate_s[1], L.up_q[1], L.up_s[1], L.down_q[1], L.down_s[1], xq, xs).y
    assert idx[0, 0] == 0 and w[0, 0] == 1.0
    assert np.array_equal(y[0], (e0.astype(np.float64) + sh).astype(np.float32))


def test_layer_equals_per_token_composition():
    wl = S.WORKLOADS["tiny_T1"]
    L = OL.full_layer(wl.layer, 0, 0)
    x = S.tokens(S.TokenSpec(T=3), wl.layer.H, 0)
    y, idx, w = O.moe_forward(L, x)
    cache = OL.ExpertCache(wl.layer, 0, 0)
    for t in range(3):
        r = OL.forward_token(wl.layer, cache, L.router_w, L.router_b, x[t])
        assert np.array_equal(r.idx, idx[t]) and np.array_equal(r.y, y[t])


# ------------------------------------------------------------ P8 rmsnorm
@pytest.mark.parametrize("c", [1.0, -3.5, 1e-4])
def test_rmsnorm_constant_input(c):
    H = 6144
    gamma = S.rms_gamma(H, 0, 0)
    out = O.rmsnorm(np.full((1, H), c, np.float32), gamma, 1e-6)
    ref = (gamma.astype(np.float64) * c / math.sqrt(c * c + 1e-6)).astype(np.float32)
    assert np.allclose(out[0], ref, rtol=1e-7, atol=0)


def test_rmsnorm_scale_invariance():
    x = rng(9).standard_normal((3, 512)).astype(np.float32)
    g = np.ones(512, np.float32)
    a = O.rmsnorm(x, g, 0.0)
    b = O.rmsnorm(x * np.float32(8.0), g, 0.0)
    assert np.array_equal(a, b)                                # power-of-two scale is exact
    assert np.allclose((a.astype(np.float64) ** 2).mean(axis=1), 1.0, rtol=1e-6)
