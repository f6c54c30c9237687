"""Free-running parity with Q8(h) flip accounting.

In a free-running comparison the GPU and the oracle each compute the whole
layer from the same inputs. Both quantise h = silu(g) * u to Q8 in 32-row
blocks. Where the two h differ in their last bits (their f64 block sums run
in different orders), h * (1/d) can fall on the other side of a .5 rounding
boundary, and that one code moves by one. Such a flip is legitimate only if
the oracle's own h * (1/d) sits within FLIP_BAND of the boundary. Every flip
is logged, and it must account for every output beyond the bar: the outputs
of a token with a flip are compared with the oracle's down projection and
combine recomputed from the GPU's own Q8(h) of the flipped pair (the
teacher-forced stage), which must then meet the bar.

Everything else is compared as it is: routing bit for bit, h within a few
f32 ulps, block scales within two ulps, per-pair outputs and layer outputs
within the relative bar rel_i = |y_i - o_i| / max(|o_i|, rms(o)).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Callable, List, Sequence

import numpy as np

from oracle import oracle as O

from gpu_common import rel_err, unreorder

FLIP_BAND = 1e-4


@dataclass
class Flip:
    token: int
    slot: int
    row: int
    oracle_value: float      # the oracle's h * (1/d) in f32
    code_oracle: int
    code_gpu: int


@dataclass
class PairSet:
    """Per (token, slot) arrays: slots 0..k-1 routed in routing order, slot k
    the shared expert."""
    idx: np.ndarray
    w: np.ndarray
    h: np.ndarray
    hq: np.ndarray           # natural order
    hs: np.ndarray
    ye: np.ndarray
    y: np.ndarray


def gpu_pairs(v: dict, has_shared: int, y: np.ndarray) -> PairSet:
    """The intermediates a GPU call left in its workspace (ws_views), per
    (token, slot)."""
    pidx = v["pair_of"]
    if has_shared:
        pidx = np.concatenate([pidx, v["shared_pair"][:, None]], axis=1)
    return PairSet(v["idx"], v["w"], v["h"][pidx], unreorder(v["hq"][pidx]), v["hs"][pidx], v["ye"][pidx], y)


def oracle_pairs(tok_results: Sequence) -> PairSet:
    """The same arrays from oracle.layers.forward_token results."""
    st = lambda name: np.stack([np.stack([getattr(e, name) for e in r.experts]) for r in tok_results])
    return PairSet(np.stack([r.idx for r in tok_results]), np.stack([r.w for r in tok_results]), st("h"),
                   st("hq"), st("hs"), st("y"), np.stack([r.y for r in tok_results]))


def batch_pairs(b) -> PairSet:
    """The same arrays from an oracle.layers.forward_batch result."""
    return PairSet(b.idx, b.w, b.h, b.hq, b.hs, b.ye, b.y)


def ulps(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    a = np.asarray(a, np.float32).astype(np.float64)
    b = np.asarray(b, np.float32).astype(np.float64)
    sp = np.spacing(np.maximum(np.abs(a), np.abs(b)).astype(np.float32)).astype(np.float64)
    return np.abs(a - b) / sp


def q8_value(h: np.ndarray, hs: np.ndarray) -> np.ndarray:
    """h * (1/d) as the quantiser forms it: the f32 reciprocal of the block
    scale (0 for a zero scale), one f32 product. h [..., I], hs [..., I/32]."""
    hs = np.asarray(hs, np.float32)
    with np.errstate(divide="ignore"):
        inv = np.where(hs != 0, np.float32(1.0) / hs, np.float32(0.0)).astype(np.float32)
    return (np.asarray(h, np.float32) * np.repeat(inv, 32, axis=-1)).astype(np.float32)


def down_rowdot(spec, P, hq: np.ndarray, hs: np.ndarray) -> np.ndarray:
    """The oracle's down projection of one packed expert from given Q8(h)."""
    if spec.group_size:
        return O.rowdot_groups(P.down_q, P.down_s, spec.group_size, hq, hs)
    if spec.weight_bits == 8:
        return O.rowdot_i8(P.down_q, P.down_s, hq, hs)
    if spec.weight_bits == 2:
        return O.rowdot_i2(P.down_q, P.down_s, hq, hs)
    return O.rowdot(P.down_q, P.down_s, hq, hs)


def check_free_running(spec, g: PairSet, o: PairSet, expert_of: Callable[[int], object],
                       say: Callable[..., None] = print, tol: float = 1e-4, h_ulps: float = 4.0,
                       w_rel: float = 1e-6) -> dict:
    """Compare a free-running GPU result with the oracle's (see the module
    docstring). expert_of(e) gives the oracle's packed expert e (only used
    for tokens with a flip). Returns counts and worst errors."""
    k = spec.top_k
    assert np.array_equal(g.idx, o.idx), "routing differs"
    wr = np.abs(g.w.astype(np.float64) - o.w) / np.maximum(np.abs(o.w), 1e-30)
    assert wr.max() <= w_rel, f"routing weights differ by {wr.max():.2e}"
    hu = ulps(g.h, o.h)
    assert hu.max() <= h_ulps, f"h differs by {hu.max():.0f} ulp"
    su = ulps(g.hs, o.hs)
    assert su.max() <= 2, f"Q8(h) scales differ by {su.max():.0f} ulp"

    dq = g.hq.astype(np.int32) - o.hq.astype(np.int32)
    assert np.abs(dq).max(initial=0) <= 1, "a Q8(h) code moved by more than one step"
    flips: List[Flip] = []
    for t, s, i in zip(*np.nonzero(dq)):
        v = float(q8_value(o.h[t, s], o.hs[t, s])[i])
        dist = abs(abs(v - np.floor(v)) - 0.5)
        assert dist < FLIP_BAND, (f"token {t} slot {s} row {i}: code {o.hq[t, s, i]} -> {g.hq[t, s, i]} "
                                  f"but h*(1/d) = {v!r} is {dist:.2e} from a rounding boundary")
        flips.append(Flip(int(t), int(s), int(i), v, int(o.hq[t, s, i]), int(g.hq[t, s, i])))
    for f in flips:
        say(f"  Q8(h) flip: token {f.token} slot {f.slot} row {f.row}: oracle h*(1/d) = {f.oracle_value!r}, "
            f"code {f.code_oracle} -> {f.code_gpu}")

    flipped = {}                                  # (token, slot) -> True where hq or hs moved
    for t, s in zip(*np.nonzero((dq != 0).any(axis=-1) | (g.hs != o.hs).any(axis=-1))):
        flipped[(int(t), int(s))] = True

    # per-pair expert outputs of unmoved pairs, and layer outputs of tokens
    # without a moved pair, as they are
    ye_err = rel_err(g.ye, o.ye)
    worst_ye = 0.0
    for (t, s) in flipped:
        ye_err[t, s] = 0.0
    worst_ye = float(ye_err.max(initial=0.0))
    assert worst_ye <= tol, f"per-pair expert output differs by {worst_ye:.2e}"
    y_err = rel_err(g.y, o.y)
    tok_flipped = sorted({t for t, _ in flipped})
    clean = np.ones(g.y.shape[0], bool)
    clean[tok_flipped] = False
    worst_clean = float(y_err[clean].max(initial=0.0))
    assert worst_clean <= tol, f"layer output differs by {worst_clean:.2e} in a token without a flip"

    # tokens with a moved code: the oracle's down projection from the GPU's
    # Q8(h) for the moved pairs, then the oracle's combine
    worst_forced = 0.0
    for t in tok_flipped:
        ye = o.ye[t].copy()
        for s in range(ye.shape[0]):
            if (t, s) in flipped:
                e = int(o.idx[t, s]) if s < k else spec.E
                ye[s] = down_rowdot(spec, expert_of(e), g.hq[t, s], g.hs[t, s])
        yt = O.combine(ye[:k], o.w[t], ye[k] if spec.has_shared else None)
        err = float(rel_err(g.y[t][None], yt[None]).max())
        say(f"  token {t}: max rel {y_err[t].max():.2e} free-running, {err:.2e} with the GPU's Q8(h)")
        assert err <= tol, f"token {t}: {err:.2e} even with the GPU's Q8(h)"
        worst_forced = max(worst_forced, err)
    stats = dict(flips=len(flips), moved_pairs=len(flipped), tokens_with_flips=len(tok_flipped),
                 worst_y=float(y_err.max(initial=0.0)), worst_y_unflipped=worst_clean, worst_ye=worst_ye,
                 worst_forced=worst_forced, h_max_ulps=float(hu.max(initial=0.0)),
                 h_bit_identical=float(np.mean(g.h == o.h)), y_bit_identical=float(np.mean(g.y == o.y)))
    say("  free-running: " + ", ".join(f"{a} {b:.3g}" if isinstance(b, float) else f"{a} {b}"
                                        for a, b in stats.items()))
    return stats


def check_tokens(spec, L, T: int, ws, y: np.ndarray, tok_results: Sequence, expert_of, say=print, flags: int = 0,
                 **kw) -> dict:
    """check_free_running for a GPU call whose workspace ws still holds its
    intermediates, against oracle.layers.forward_token results."""
    from gpu_common import ws_views
    v = ws_views(L, T, ws, flags)
    return check_free_running(spec, gpu_pairs(v, spec.has_shared, y), oracle_pairs(tok_results),
                              expert_of, say, **kw)
