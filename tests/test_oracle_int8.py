"""Pins of the oracle's int8-weight experts (the pages' quantize_rows and
dot_i8i8: one byte per weight) against things other than themselves: exact
round trips, half-to-even cases, integer matmuls (numpy), exactly
representable row products, and a cross-format identity. An int8 layer whose
codes all lie in [-8, 7] is the int4 layer with the same codes and scales, so
the int8 path must give the int4 path's results bit for bit. A wrong row
stride, a dropped block scale, a leftover x16 factor or a nibble decode on
int8 bytes fails one of them."""
import numpy as np
import pytest

from oracle import oracle as O
from oracle import layers as OL
from synth import synth as S


def rng(seed=0):
    return np.random.default_rng(seed)


def test_pack_int8_exact_round_trip():
    r = rng(1)
    codes = r.integers(-127, 128, size=(16, 96)).astype(np.int64)
    codes[:, 5] = np.where(r.random(16) < 0.5, 127, -127)            # absmax code in every row
    scale = np.float32(2.0) ** r.integers(-12, -2, size=16).astype(np.float32)
    w = (codes * scale[:, None]).astype(np.float32)                  # exact: power-of-two scales
    q, s = O.pack_int8_rows(w)
    assert q.dtype == np.int8
    assert np.array_equal(s, scale)
    assert np.array_equal(q.astype(np.int64), codes)


def test_pack_int8_half_to_even_zero_row_and_range():
    d = np.float32(2.0 ** -7)
    row = np.array([127, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5], np.float32) * d
    q, s = O.pack_int8_rows(np.stack([row, np.zeros(8, np.float32)]))
    assert s[0] == d and s[1] == 0.0
    assert q[0].tolist() == [127, 0, 2, 2, 0, -2, -2, 126]
    assert q[1].tolist() == [0] * 8
    w = (rng(2).standard_normal((32, 256)) * 0.02).astype(np.float32)
    q, s = O.pack_int8_rows(w)
    assert q.min() >= -127 and q.max() <= 127
    assert np.all(np.abs(q).max(axis=1) == 127)                      # the absmax element maps to +-127
    err = np.abs(w - q.astype(np.float64) * s[:, None])
    assert np.all(err <= 0.5 * s[:, None] * (1 + 1e-6))              # half a step at most


def test_block_dots_i8_equal_integer_matmul():
    r = rng(3)
    qw = r.integers(-127, 128, size=(24, 256)).astype(np.int8)
    qw[0] = -127
    x = r.integers(-127, 128, size=256).astype(np.int8)
    x[:32] = -127                                                    # the extreme block: 32*127*127
    S = O.block_dots_i8(qw, x)
    ref = (qw.astype(np.int64).reshape(24, 8, 32) * x.astype(np.int64).reshape(8, 32)).sum(-1)
    assert np.array_equal(S.astype(np.int64), ref)
    assert S[0, 0] == 32 * 127 * 127


def test_rowdot_i8_exact_when_representable():
    r = rng(4)
    qw = r.integers(-20, 21, size=(8, 128)).astype(np.int8)
    q8 = r.integers(-20, 21, size=128).astype(np.int8)
    d8 = (np.float32(2.0) ** r.integers(-6, 0, size=4)).astype(np.float32)
    sw = (np.float32(2.0) ** r.integers(-8, -3, size=8)).astype(np.float32)
    out = O.rowdot_i8(qw, sw, q8, d8)
    S = (qw.astype(np.int64).reshape(8, 4, 32) * q8.astype(np.int64).reshape(4, 32)).sum(-1)
    exact = (S * d8.astype(np.float64)).sum(-1) * sw.astype(np.float64)   # exact in double here
    assert np.array_equal(out.astype(np.float64), exact)


def _int4_from_codes(codes):
    """Pack int codes in [-8, 7] as int4 bytes, even element in the low nibble."""
    c = codes.astype(np.int64) & 0xF
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def test_expert_int8_equals_int4_on_shared_codes():
    r = rng(5)
    H, I = 256, 96
    mats = [r.integers(-8, 8, size=shape).astype(np.int8) for shape in ((I, H), (I, H), (H, I))]
    scales = [(r.random(n) * 0.01 + 0.001).astype(np.float32) for n in (I, I, H)]
    x = r.standard_normal(H).astype(np.float32)
    x[7] *= 20.0
    xq, xs = O.quant_q8(x)
    e8 = O.expert(mats[0], scales[0], mats[1], scales[1], mats[2], scales[2], xq, xs)
    e4 = O.expert(_int4_from_codes(mats[0]), scales[0], _int4_from_codes(mats[1]), scales[1],
                  _int4_from_codes(mats[2]), scales[2], xq, xs)
    for name in ("g", "u", "h", "hq", "hs", "y"):
        assert np.array_equal(getattr(e8, name), getattr(e4, name)), name
    d8 = O.expert_dense(mats[0], scales[0], mats[1], scales[1], mats[2], scales[2], x)
    d4 = O.expert_dense(_int4_from_codes(mats[0]), scales[0], _int4_from_codes(mats[1]), scales[1],
                        _int4_from_codes(mats[2]), scales[2], x)
    assert np.array_equal(d8, d4)


def test_layer_int8_equals_int4_on_shared_codes():
    sp = S.LayerSpec(H=256, I=128, E=16, top_k=2, weight_bits=8)
    L8 = OL.full_layer(sp, 0, 0)
    r = rng(6)
    for name in ("gate_q", "up_q", "down_q"):
        setattr(L8, name, r.integers(-8, 8, size=getattr(L8, name).shape).astype(np.int8))
    L4 = OL.FullLayer(**{**L8.__dict__, "weight_bits": 4,
                         "gate_q": _int4_from_codes(L8.gate_q), "up_q": _int4_from_codes(L8.up_q),
                         "down_q": _int4_from_codes(L8.down_q)})
    x = S.tokens(S.TokenSpec(T=6, token_set=3), sp.H, 0)
    y8, i8, w8 = O.moe_forward(L8, x)
    y4, i4, w4 = O.moe_forward(L4, x)
    assert np.array_equal(i8, i4) and np.array_equal(w8, w4)
    assert np.array_equal(y8, y4)


def test_int8_expert_idot_close_to_dense_reference():
    sp = S.LayerSpec(H=512, I=256, E=4, top_k=1, weight_bits=8)
    cache = OL.ExpertCache(sp, 0, 0)
    errs = []
    for t in range(4):
        x = S.tokens(S.TokenSpec(T=1, token_set=20 + t), sp.H, 0)[0]
        xq, xs = O.quant_q8(x)
        pe = cache[t % 4]
        y = O.expert(*pe.args(), xq, xs).y.astype(np.float64)
        yd = O.expert_dense(*pe.args(), x)
        errs.append(np.sqrt(np.mean((y - yd) ** 2) / np.mean(yd ** 2)))
    # activation rounding dominates: a few tenths of a percent to ~1% at these shapes
    assert max(errs) < 0.03


def test_int8_layer_matches_per_token_composition():
    sp = S.LayerSpec(H=256, I=128, E=16, top_k=2, weight_bits=8)
    L8 = OL.full_layer(sp, 0, 0)
    cache = OL.ExpertCache(sp, 0, 0)
    x = S.tokens(S.TokenSpec(T=4, token_set=9), sp.H, 0)
    y, idx, _ = O.moe_forward(L8, x)
    for t in range(4):
        r = OL.forward_token(sp, cache, L8.router_w, L8.router_b, x[t])
        assert np.array_equal(r.idx, idx[t])
        assert np.array_equal(r.y, y[t])
