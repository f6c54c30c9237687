"""The free-running comparison with Q8(h) flip accounting (tests/parity.py),
checked on the CPU with the oracle on both sides: identical results pass
with no flip; a code moved where the oracle's h * (1/d) sits on a rounding
boundary, with the outputs that code gives, is logged and accepted; a code
moved away from a boundary, or an output moved without a flip, fails.
Every planted change is made to oracle results, on the CPU."""
import copy

import numpy as np
import pytest

from oracle import layers as OL
from oracle import oracle as O
from synth import synth as S

import parity as PR

SPEC = S.TINY


@pytest.fixture(scope="module")
def batch():
    x = S.tokens(S.TokenSpec(T=6, token_set=91), SPEC.H, 0)
    W, b = S.router(SPEC, 0, 0)
    cache = OL.ExpertCache(SPEC, 0, 0)
    return PR.batch_pairs(OL.forward_batch(SPEC, W, b, x, lambda e: cache[e])), cache


def _pick(o, t, s):
    """A row of pair (t, s) that is not its block's largest |h|."""
    blk = np.abs(o.h[t, s, :32])
    return int(np.argsort(blk)[len(blk) // 2])


def test_identical_results_pass(batch):
    o, cache = batch
    st = PR.check_free_running(SPEC, copy.deepcopy(o), o, lambda e: cache[e])
    assert st["flips"] == 0 and st["worst_y"] == 0.0


def test_boundary_flip_is_attributed(batch):
    o0, cache = batch
    o, g = copy.deepcopy(o0), copy.deepcopy(o0)
    t, s = 2, 0
    i = _pick(o, t, s)
    c = int(o.hq[t, s, i])
    d = np.float32(o.hs[t, s, i // 32])
    inv = np.float32(1.0) / d
    # the oracle's h of that row moved to sit just above the boundary below c
    # (its code stays c); the GPU side takes the code one step down
    target = np.float32(c - 0.5 + 3e-5)
    h = np.float32(target / inv)
    while np.float32(h * inv) < target:
        h = np.nextafter(h, np.float32(np.inf), dtype=np.float32)
    o.h[t, s, i] = g.h[t, s, i] = h
    assert int(np.rint(np.float32(h * inv))) == c
    g.hq[t, s, i] = c - 1
    e = int(o.idx[t, s])
    g.ye[t, s] = PR.down_rowdot(SPEC, cache[e], g.hq[t, s], g.hs[t, s])
    g.y[t] = O.combine(g.ye[t, :SPEC.top_k], g.w[t], g.ye[t, SPEC.top_k])
    st = PR.check_free_running(SPEC, g, o, lambda e: cache[e])
    assert st["flips"] == 1 and st["tokens_with_flips"] == 1


def test_flip_away_from_a_boundary_fails(batch):
    o, cache = batch
    g = copy.deepcopy(o)
    t, s = 1, 1
    v = PR.q8_value(o.h[t, s], o.hs[t, s])
    i = int(np.argmax(np.abs(np.abs(v - np.floor(v)) - 0.5)))    # the row farthest from a boundary
    g.hq[t, s, i] = g.hq[t, s, i] - 1 if g.hq[t, s, i] > -127 else g.hq[t, s, i] + 1
    with pytest.raises(AssertionError, match="rounding boundary"):
        PR.check_free_running(SPEC, g, o, lambda e: cache[e])


def test_output_moved_without_a_flip_fails(batch):
    o, cache = batch
    g = copy.deepcopy(o)
    g.y[3, 7] = g.y[3, 7] * np.float32(1.001) + np.float32(1e-3)
    with pytest.raises(AssertionError, match="without a flip"):
        PR.check_free_running(SPEC, g, o, lambda e: cache[e])


def test_routing_difference_fails(batch):
    o, cache = batch
    g = copy.deepcopy(o)
    g.idx[0, [0, 1]] = g.idx[0, [1, 0]]
    with pytest.raises(AssertionError, match="routing"):
        PR.check_free_running(SPEC, g, o, lambda e: cache[e])
