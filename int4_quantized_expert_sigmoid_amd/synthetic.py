"""Synthetic MoE layers resident in HBM.

Weights come from the seeded generator (synth/, counter-addressed, its device
twin writes f32 rows straight into HBM) and are packed to int4 on the GPU by
the library's own packer (coli_pack_int4_rows_dev, or coli_pack_int8_rows_dev
for int8 experts, coli_pack_int4_groups_dev for group scales). Router weights, bias,
tokens and RMSNorm gains are small and generated on the host.
"""
from __future__ import annotations

import numpy as np
import torch

from synth import synth as S

from .api import (DenseMLP, MoELayer, pack_int2_rows_dev, pack_int4_groups_dev, pack_int4_rows_dev,
                  pack_int8_rows_dev)


def device_layer(spec: S.LayerSpec, seed: int = 0, layer: int = 0, device: str = "cuda",
                 scratch: torch.Tensor = None) -> MoELayer:
    L = MoELayer.empty(spec.H, spec.I, spec.E, spec.top_k, spec.has_shared, spec.n_group, spec.topk_group,
                       spec.route_scale, device=device, weight_bits=spec.weight_bits, group_size=spec.group_size)
    if spec.group_size:
        pack = lambda w, q, s: pack_int4_groups_dev(w, spec.group_size, q, s)
    elif spec.weight_bits == 2:
        pack = pack_int2_rows_dev
    else:
        pack = pack_int8_rows_dev if spec.weight_bits == 8 else pack_int4_rows_dev
    W, b = S.router(spec, seed, layer)
    L.router_w.copy_(torch.from_numpy(W))
    L.router_b.copy_(torch.from_numpy(b))
    n = spec.H * spec.I
    if scratch is None or scratch.numel() < n:
        scratch = torch.empty(n, dtype=torch.float32, device=device)
    stream = torch.cuda.current_stream().cuda_stream
    for e in range(spec.n_experts_stored):
        for m, q, s, shape in ((S.GATE, L.gate_q, L.gate_s, (spec.I, spec.H)),
                               (S.UP, L.up_q, L.up_s, (spec.I, spec.H)),
                               (S.DOWN, L.down_q, L.down_s, (spec.H, spec.I))):
            buf = scratch[:n].view(shape)
            S.dev_expert_matrix(buf.data_ptr(), spec, seed, layer, e, m, hip_stream=stream)
            pack(buf, q[e], s[e])
    return L


def host_tokens(tspec: S.TokenSpec, H: int, seed: int = 0) -> np.ndarray:
    return S.tokens(tspec, H, seed)


def device_dense(spec: S.DenseSpec, seed: int = 0, layer: int = 0, device: str = "cuda",
                 scratch: torch.Tensor = None) -> DenseMLP:
    """A dense MLP's weights from the seeded generator, packed on the GPU."""
    M = DenseMLP.empty(spec.H, spec.I, device=device, weight_bits=spec.weight_bits)
    pack = pack_int8_rows_dev if spec.weight_bits == 8 else pack_int4_rows_dev
    n = spec.H * spec.I
    if scratch is None or scratch.numel() < n:
        scratch = torch.empty(n, dtype=torch.float32, device=device)
    stream = torch.cuda.current_stream().cuda_stream
    for m, q, s, shape in ((S.GATE, M.gate_q, M.gate_s, (spec.I, spec.H)), (S.UP, M.up_q, M.up_s, (spec.I, spec.H)),
                           (S.DOWN, M.down_q, M.down_s, (spec.H, spec.I))):
        buf = scratch[:n].view(shape)
        S.dev_dense_matrix(buf.data_ptr(), spec, seed, layer, m, hip_stream=stream)
        pack(buf, q, s)
    return M
