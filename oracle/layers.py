"""Oracle-side layer assembly: synthetic f32 weights from synth, packed with the
oracle's own packer. TEST INFRASTRUCTURE ONLY (tests, smoke, CPU baseline).

For the GLM-5.2-shaped layers the oracle never holds all 257 experts: it
regenerates only the experts a token selects (ExpertCache)."""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Tuple

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


def packed_expert(spec: S.LayerSpec, seed: int, layer: int, e: int) -> PackedExpert:
    if spec.group_size:
        pack = lambda w: O.pack_int4_groups(w, spec.group_size)
    elif spec.weight_bits == 2:
        pack = O.pack_int2_rows
    else:
        pack = O.pack_int8_rows if spec.weight_bits == 8 else O.pack_int4_rows
    mats = []
    for m in (S.GATE, S.UP, S.DOWN):
        mats.extend(pack(S.expert_matrix(spec, seed, layer, e, m)))
    return PackedExpert(*mats)


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
