"""Oracle-side layer assembly: synthetic f32 weights from synth, packed with the
oracle's own packer. TEST INFRASTRUCTURE ONLY (tests, smoke, CPU baseline).

For the GLM-5.2-shaped layers the oracle never holds all 257 experts: it
regenerates only the experts a token selects (ExpertCache), or, for a whole
batch (forward_batch), takes the experts one at a time from a source the
caller gives (the f32 weights may come from the generator's device twin,
which writes the same values; the packing is always the oracle's own)."""
from __future__ import annotations

from dataclasses import dataclass
from typing import Callable, Dict, Tuple

import numpy as np

from synth import synth as S
from oracle import oracle as O


@dataclass
class PackedExpert:
    gate_q: np.ndarray
    gate_s: np.ndarray
    up_q: np.ndarray
    up_s: np.ndarray
    down_q: np.ndarray
    down_s: np.ndarray

    def args(self):
        return (self.gate_q, self.gate_s, self.up_q, self.up_s, self.down_q, self.down_s)


def pack_matrices(spec: S.LayerSpec, gate_w: np.ndarray, up_w: np.ndarray, down_w: np.ndarray) -> PackedExpert:
    """One expert's f32 matrices packed in the spec's format by the oracle."""
    if spec.group_size:
        pack = lambda w: O.pack_int4_groups(w, spec.group_size)
    elif spec.weight_bits == 2:
        pack = O.pack_int2_rows
    else:
        pack = O.pack_int8_rows if spec.weight_bits == 8 else O.pack_int4_rows
    mats = []
    for w in (gate_w, up_w, down_w):
        mats.extend(pack(w))
    return PackedExpert(*mats)


def packed_expert(spec: S.LayerSpec, seed: int, layer: int, e: int) -> PackedExpert:
    return pack_matrices(spec, *[S.expert_matrix(spec, seed, layer, e, m) for m in (S.GATE, S.UP, S.DOWN)])


class ExpertCache:
    """Regenerates and packs experts on demand (oracle packer)."""

    def __init__(self, spec: S.LayerSpec, seed: int, layer: int):
        self.spec, self.seed, self.layer = spec, seed, layer
        self._c: Dict[int, PackedExpert] = {}

    def __getitem__(self, e: int) -> PackedExpert:
        if e not in self._c:
            self._c[e] = packed_expert(self.spec, self.seed, self.layer, e)
        return self._c[e]


@dataclass
class FullLayer:
    """Every expert in host memory, in the stacked layout oracle.moe_forward takes."""
    H: int
    I: int
    E: int
    top_k: int
    n_group: int
    topk_group: int
    has_shared: int
    route_scale: float
    router_w: np.ndarray
    router_b: np.ndarray
    gate_q: np.ndarray
    gate_s: np.ndarray
    up_q: np.ndarray
    up_s: np.ndarray
    down_q: np.ndarray
    down_s: np.ndarray
    weight_bits: int = 4
    group_size: int = 0


def full_layer(spec: S.LayerSpec, seed: int = 0, layer: int = 0) -> FullLayer:
    W, b = S.router(spec, seed, layer)
    ex = [packed_expert(spec, seed, layer, e) for e in range(spec.n_experts_stored)]
    st = lambda name: np.stack([getattr(p, name) for p in ex])
    return FullLayer(spec.H, spec.I, spec.E, spec.top_k, spec.n_group, spec.topk_group,
                     spec.has_shared, spec.route_scale, W, b, st("gate_q"), st("gate_s"),
                     st("up_q"), st("up_s"), st("down_q"), st("down_s"), spec.weight_bits, spec.group_size)


@dataclass
class TokenResult:
    idx: np.ndarray      # [k]
    w: np.ndarray        # [k]
    xq: np.ndarray       # [H]
    xs: np.ndarray       # [H/32]
    experts: Tuple       # ExpertOut per routed slot, then shared (if any)
    y: np.ndarray        # [H]


def forward_token(spec: S.LayerSpec, cache: ExpertCache, W: np.ndarray, b: np.ndarray,
                  x: np.ndarray) -> TokenResult:
    """One token through the layer (O6 -> O3 -> O7 -> O8), regenerating experts."""
    idx, w = O.route(W, b, x[None, :], spec.top_k, spec.n_group, spec.topk_group, spec.route_scale)
    xq, xs = O.quant_q8(x)
    kw = dict(group=spec.group_size, wbits=spec.weight_bits)
    outs = [O.expert(*cache[int(e)].args(), xq, xs, **kw) for e in idx[0]]
    sh = O.expert(*cache[spec.E].args(), xq, xs, **kw) if spec.has_shared else None
    y = O.combine(np.stack([o.y for o in outs]), w[0], None if sh is None else sh.y)
    return TokenResult(idx[0], w[0], xq, xs, tuple(outs) + ((sh,) if sh else ()), y)


@dataclass
class BatchResult:
    """A batch through the layer. Per (token, slot): slots 0..k-1 are the
    routed experts in routing order, slot k the shared expert."""
    idx: np.ndarray      # [T][k]
    w: np.ndarray        # [T][k]
    xq: np.ndarray       # [T][H]
    xs: np.ndarray       # [T][H/32]
    h: np.ndarray        # [T][k+s][I]
    hq: np.ndarray       # [T][k+s][I]
    hs: np.ndarray       # [T][k+s][I/32]
    ye: np.ndarray       # [T][k+s][H]
    y: np.ndarray        # [T][H]


def forward_batch(spec: S.LayerSpec, W: np.ndarray, b: np.ndarray, x: np.ndarray,
                  expert_of: Callable[[int], PackedExpert], log: Callable[[str], None] = None) -> BatchResult:
    """O6 (routing of every token) -> O3 (Q8 of every token) -> O7 for every
    (token, expert) pair -> O8 for every token: the same arithmetic as
    forward_token, token by token, with each expert taken once (from
    expert_of) for all of its tokens."""
    x = np.ascontiguousarray(np.atleast_2d(x), np.float32)
    T, H = x.shape
    k, I, E = spec.top_k, spec.I, spec.E
    idx, w = O.route(W, b, x, k, spec.n_group, spec.topk_group, spec.route_scale)
    xq, xs = O.quant_q8(x)
    ns = k + spec.has_shared
    r = BatchResult(idx, w, xq, xs, np.zeros((T, ns, I), np.float32), np.zeros((T, ns, I), np.int8),
                    np.zeros((T, ns, I // 32), np.float32), np.zeros((T, ns, H), np.float32),
                    np.empty((T, H), np.float32))
    experts = sorted(set(int(e) for e in idx.reshape(-1)))
    if spec.has_shared:
        experts.append(E)
    kw = dict(group=spec.group_size, wbits=spec.weight_bits)
    for n, e in enumerate(experts):
        if e == E and spec.has_shared:
            toks, slots = np.arange(T), np.full(T, k)
        else:
            toks, slots = np.nonzero(idx == e)
        P = expert_of(e)
        o = O.expert_tokens(*P.args(), xq[toks], xs[toks], **kw)
        r.ye[toks, slots], r.h[toks, slots], r.hq[toks, slots], r.hs[toks, slots] = o.y, o.h, o.hq, o.hs
        if log and (n + 1) % 32 == 0:
            log(f"oracle: {n + 1} of {len(experts)} experts")
    for t in range(T):
        r.y[t] = O.combine(r.ye[t, :k], w[t], r.ye[t, k] if spec.has_shared else None)
    return r
