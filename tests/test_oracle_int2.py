"""Pins of the oracle's int2 experts (the pages' experimental int2 packing,
four 2-bit codes per byte, and its matmul_i2) against things other than
themselves: every 2-bit field of every byte value, exact round trips with
power-of-two scales, half-to-even and zero rows, block dots equal to an
integer matmul, exactly representable row products, the dequantised
brute-force product, and a cross-format identity: int2 codes written as int4
nibbles with the same scales give the int4 expert's and layer's results bit
for bit (so a wrong field order, a leftover factor, or a row stride of the
wrong format fails)."""
from dataclasses import replace

import numpy as np
import pytest

from oracle import layers as OL
from oracle import oracle as O
from synth import synth as S


def rng(seed=0):
    return np.random.default_rng(seed)


def test_crumb_every_byte():
    for byte in range(256):
        for i in range(4):
            v = (byte >> (2 * i)) & 3
            assert O.crumb(byte, i) == (v - 4 if v >= 2 else v)


def test_pack_int2_exact_round_trip():
    r = rng(1)
    rows, cols = 12, 128
    codes = r.integers(-1, 2, size=(rows, cols)).astype(np.int64)
    codes[:, 7] = np.where(r.random(rows) < 0.5, 1, -1)               # the absmax element
    scale = (np.float32(2.0) ** r.integers(-10, -2, size=rows)).astype(np.float32)
    w = (codes * scale[:, None]).astype(np.float32)
    q, s = O.pack_int2_rows(w)
    assert q.shape == (rows, cols // 4)
    assert np.array_equal(s, scale)
    assert np.array_equal(O.unpack_int2_rows(q, s), w.astype(np.float64))
    # field i of byte j is element 4j + i
    for i in range(4):
        got = np.vectorize(lambda b: O.crumb(int(b), i))(np.asarray(q))
        assert np.array_equal(got, codes[:, i::4])


def test_pack_int2_rounding_range_and_zero_row():
    d = np.float32(0.25)
    row = np.array([1.0, 0.5, -0.5, 0.49, -0.51, -1.0, 0.0, 0.75], np.float32) * d
    q, s = O.pack_int2_rows(np.stack([row, np.zeros(8, np.float32)]))
    assert s[0] == d and s[1] == 0.0
    deq = O.unpack_int2_rows(q, s)
    assert (deq[0] / d).tolist() == [1, 0, 0, 0, -1, -1, 0, 1]       # half to even at +-0.5
    assert not deq[1].any()
    w = (rng(2).standard_normal((32, 256)) * 0.02).astype(np.float32)
    q, s = O.pack_int2_rows(w)
    codes = np.round(O.unpack_int2_rows(q, s) / s[:, None].astype(np.float64)).astype(int)
    assert codes.min() >= -1 and codes.max() <= 1                    # -2 is never produced
    assert np.all(np.abs(codes).max(axis=1) == 1)
    assert np.all(np.abs(w - codes * s[:, None]) <= 0.5 * s[:, None] * (1 + 1e-6))


def test_block_dots_i2_equal_integer_matmul():
    r = rng(3)
    rows, cols = 16, 256
    codes = r.integers(-2, 2, size=(rows, cols))                     # the full 2-bit range, -2 included
    codes[0] = -2
    f = (codes & 3).astype(np.uint8)
    q = (f[:, 0::4] | (f[:, 1::4] << 2) | (f[:, 2::4] << 4) | (f[:, 3::4] << 6)).astype(np.uint8)
    x = r.integers(-127, 128, size=cols).astype(np.int8)
    x[:32] = -127
    S = O.block_dots_i2(q, x)
    ref = (codes.astype(np.int64).reshape(rows, cols // 32, 32) * x.astype(np.int64).reshape(cols // 32, 32)).sum(-1)
    assert np.array_equal(S.astype(np.int64), ref)
    assert S[0, 0] == 2 * 127 * 32
    # the exactly representable row product: power-of-two scales, sum exact in f32
    s2 = (np.float32(2.0) ** r.integers(-3, 1, size=rows)).astype(np.float32)
    d8 = (np.float32(2.0) ** r.integers(-7, -3, size=cols // 32)).astype(np.float32)
    out = O.rowdot_i2(q, s2, x, d8)
    exact = (codes * s2[:, None].astype(np.float64)) @ (x.astype(np.float64) * np.repeat(d8, 32))
    assert np.array_equal(out, exact.astype(np.float32))


def test_rowdot_i2_against_dequantised_brute_force():
    r = rng(4)
    w = (r.standard_normal((24, 512)) * 0.02).astype(np.float32)
    q, s = O.pack_int2_rows(w)
    x = (r.standard_normal(512) * 2).astype(np.float32)
    xq, xs = O.quant_q8(x)
    out = O.rowdot_i2(q, s, xq, xs).astype(np.float64)
    wd = O.unpack_int2_rows(q, s)
    xd = xq.astype(np.float64) * np.repeat(xs.astype(np.float64), 32)
    ref = wd @ xd
    assert np.all(np.abs(out - ref) <= 2.0 ** -24 * np.abs(ref) + 1e-12 * (np.abs(wd) @ np.abs(xd)))


def _as_int4(q2: np.ndarray) -> np.ndarray:
    """The same codes as int4 bytes (two per byte, even element in bits 0-3)."""
    q2 = np.asarray(q2, dtype=np.uint8)
    codes = np.stack([(q2 >> (2 * i)) & 3 for i in range(4)], axis=-1).reshape(q2.shape[:-1] + (-1,))
    codes = np.where(codes >= 2, codes.astype(np.int16) - 4, codes.astype(np.int16))
    n = (codes & 0xF).astype(np.uint8)
    return (n[..., 0::2] | (n[..., 1::2] << 4)).astype(np.uint8)


def test_expert_int2_equals_int4_on_the_same_codes():
    spec = replace(S.TINY, weight_bits=2)
    p2 = OL.packed_expert(spec, 0, 0, 3)
    x = S.tokens(S.TokenSpec(T=1, outlier_channels=2), spec.H, 0)[0]
    xq, xs = O.quant_q8(x)
    a = O.expert(*p2.args(), xq, xs, wbits=2)
    b = O.expert(_as_int4(p2.gate_q), p2.gate_s, _as_int4(p2.up_q), p2.up_s, _as_int4(p2.down_q), p2.down_s, xq, xs)
    for f in ("y", "g", "u", "h", "hq", "hs"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    assert np.any(a.y != 0)


def test_layer_int2_equals_int4_on_the_same_codes():
    spec = replace(S.TINY, weight_bits=2)
    L2 = OL.full_layer(spec, 0, 2)
    assert L2.gate_q.shape == (spec.E + 1, spec.I, spec.H // 4)
    assert L2.down_q.shape == (spec.E + 1, spec.H, spec.I // 4)
    L4 = OL.FullLayer(**{**L2.__dict__, "gate_q": _as_int4(L2.gate_q), "up_q": _as_int4(L2.up_q),
                         "down_q": _as_int4(L2.down_q), "weight_bits": 4})
    x = S.tokens(S.TokenSpec(T=3, token_set=6, outlier_channels=2), spec.H, 0)
    y2, i2, w2 = O.moe_forward(L2, x)
    y4, i4, w4 = O.moe_forward(L4, x)
    assert np.array_equal(i2, i4) and np.array_equal(w2, w4)
    assert np.array_equal(y2, y4)
    # and the per-token composition of separately packed experts
    cache = OL.ExpertCache(spec, 0, 2)
    for t in range(3):
        tr = OL.forward_token(spec, cache, L2.router_w, L2.router_b, x[t])
        assert np.array_equal(tr.y, y2[t])
