"""Seeded synthetic inputs for the MoE expert-FFN layer (Python side).

Thin ctypes wrapper over libsynth.so (host) and libsynth_dev.so (device), plus
the workload recipes: layer shapes, weight/router/bias/token distributions.
Everything here is input generation; none of the method's arithmetic lives
here. Both the oracle harness and the GPU harness take their inputs from this
module, addressed by (seed, stream, element index), so that any expert of any
layer can be regenerated on its own.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
_host = None
_dev = None

GATE, UP, DOWN = 0, 1, 2


def _lib():
    global _host
    if _host is None:
        # COLI_LIB_VARIANT=asan: the sanitizer build of the CPU test suite
        path = os.path.join(HERE, "_asan" if os.environ.get("COLI_LIB_VARIANT") == "asan" else "", "libsynth.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(path)
        u32, i64, f64, f32 = ctypes.c_uint32, ctypes.c_int64, ctypes.c_double, ctypes.c_float
        L.synth_philox4x32_10.argtypes = [ctypes.POINTER(u32), ctypes.POINTER(u32), ctypes.POINTER(u32)]
        L.synth_normal_scale.argtypes = [f64]
        L.synth_normal_scale.restype = f32
        L.synth_stream_expert.argtypes = [ctypes.c_int] * 3
        L.synth_stream_expert.restype = u32
        L.synth_stream_layer.argtypes = [ctypes.c_int] * 2
        L.synth_stream_layer.restype = u32
        L.synth_stream_tokens.argtypes = [ctypes.c_int] * 2
        L.synth_stream_tokens.restype = u32
        L.synth_normal_int.argtypes = [u32, u32, ctypes.c_uint64]
        L.synth_normal_int.restype = ctypes.c_int32
        L.synth_fill_matrix.argtypes = [u32, u32, i64, i64, i64, f64, f64, f32, ctypes.c_void_p]
        L.synth_outlier_threshold.argtypes = [f64]
        L.synth_outlier_threshold.restype = u32
        L.synth_outlier_col.argtypes = [u32, u32, i64, i64, f64]
        L.synth_outlier_col.restype = i64
        L.synth_uniform.argtypes = [u32, u32, ctypes.c_uint64]
        L.synth_uniform.restype = f64
        L.synth_permutation.argtypes = [u32, u32, ctypes.c_int, ctypes.c_void_p]
        _host = L
    return _host


def _devlib():
    global _dev
    if _dev is None:
        path = os.path.join(HERE, "libsynth_dev.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(path)
        L.synth_dev_fill_matrix.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int64, ctypes.c_int64,
                                            ctypes.c_int64, ctypes.c_float, ctypes.c_uint32, ctypes.c_float,
                                            ctypes.c_void_p, ctypes.c_void_p]
        L.synth_dev_fill_matrix.restype = ctypes.c_int
        _dev = L
    return _dev


# ---------------------------------------------------------------- primitives
def philox(ctr, key):
    L = _lib()
    c = (ctypes.c_uint32 * 4)(*ctr)
    k = (ctypes.c_uint32 * 2)(*key)
    o = (ctypes.c_uint32 * 4)()
    L.synth_philox4x32_10(c, k, o)
    return list(o)


def normal_scale(sigma: float) -> float:
    return float(_lib().synth_normal_scale(sigma))


def stream_expert(layer: int, expert: int, matrix: int) -> int:
    return int(_lib().synth_stream_expert(layer, expert, matrix))


def stream_layer(layer: int, what: int) -> int:
    return int(_lib().synth_stream_layer(layer, what))


def stream_tokens(set_id: int, what: int) -> int:
    return int(_lib().synth_stream_tokens(set_id, what))


def fill_matrix(seed: int, stream: int, rows: int, cols: int, sigma: float,
                outlier_rate: float = 0.0, outlier_mult: float = 1.0, row0: int = 0) -> np.ndarray:
    out = np.empty((rows, cols), dtype=np.float32)
    _lib().synth_fill_matrix(seed, stream, row0, rows, cols, sigma, outlier_rate, outlier_mult,
                             out.ctypes.data)
    return out


def outlier_col(seed: int, stream: int, row: int, cols: int, rate: float) -> int:
    return int(_lib().synth_outlier_col(seed, stream, row, cols, rate))


def uniform(seed: int, stream: int, n: int) -> float:
    return float(_lib().synth_uniform(seed, stream, n))


def permutation(seed: int, stream: int, n: int) -> np.ndarray:
    p = np.empty(n, dtype=np.int32)
    _lib().synth_permutation(seed, stream, n, p.ctypes.data)
    return p


def dev_fill_matrix(ptr: int, seed: int, stream: int, rows: int, cols: int, sigma: float,
                    outlier_rate: float = 0.0, outlier_mult: float = 1.0, row0: int = 0,
                    hip_stream: int = 0) -> None:
    """Same values as fill_matrix(), written to device memory at ptr."""
    c = normal_scale(sigma)
    thr = int(_lib().synth_outlier_threshold(outlier_rate))
    rc = _devlib().synth_dev_fill_matrix(seed, stream, row0, rows, cols, c, thr, outlier_mult,
                                         ctypes.c_void_p(ptr), ctypes.c_void_p(hip_stream))
    if rc != 0:
        raise RuntimeError(f"synth_dev_fill_matrix failed with HIP error {rc}")


# ---------------------------------------------------------------- recipes
@dataclass(frozen=True)
class LayerSpec:
    """Shape and weight distribution of one MoE layer (one routed-expert FFN)."""
    H: int
    I: int
    E: int
    top_k: int
    has_shared: int = 1
    n_group: int = 1
    topk_group: int = 1
    route_scale: float = 1.0
    w_sigma: float = 0.02            # expert weights ~ N(0, w_sigma)
    w_outlier_rate: float = 0.0      # fraction of rows with one element scaled
    w_outlier_mult: float = 10.0
    bias_sigma: float = 0.01         # router bias ~ N(0, bias_sigma)
    zipf_s: float = 0.0              # > 0: bias -= zipf_alpha * zipf_s * ln(rank)
    zipf_alpha: float = 0.02
    hot_experts: int = 0             # > 0: that many seeded experts get hot_bias added (chosen by every token)
    hot_bias: float = 2.0
    weight_bits: int = 4             # packed expert format: 4 (two codes per byte) or 8
    group_size: int = 0              # int4 only: > 0 gives one scale per group of that many columns

    @property
    def router_sigma(self) -> float:
        return 1.0 / math.sqrt(self.H)

    @property
    def n_experts_stored(self) -> int:
        return self.E + self.has_shared

    @property
    def expert_bytes(self) -> int:
        """Packed bytes (int4: two codes per byte; int8: one) + f32 scales of one
        expert (gate, up, down): one per row, or one per group of columns."""
        codes = 3 * self.H * self.I * self.weight_bits // 8
        if self.group_size:
            return codes + 4 * 3 * self.H * self.I // self.group_size
        return codes + 4 * (2 * self.I + self.H)


@dataclass(frozen=True)
class TokenSpec:
    """Distribution of the T input rows."""
    T: int
    rho: float = 0.0                 # equicorrelation between tokens
    outlier_channels: int = 0        # number of channels scaled in every token
    outlier_mult: float = 20.0
    token_set: int = 0               # selects an independent draw of tokens


@dataclass(frozen=True)
class Workload:
    name: str
    layer: LayerSpec
    tokens: TokenSpec
    n_layers: int = 1
    seed: int = 0
    rms_eps: float = 1e-6


TINY = LayerSpec(H=256, I=128, E=16, top_k=2)
GLM52 = LayerSpec(H=6144, I=2048, E=256, top_k=8, w_outlier_rate=0.001)

WORKLOADS = {
    "tiny_T1": Workload("tiny_T1", TINY, TokenSpec(T=1)),
    "glm52_decode_T1": Workload("glm52_decode_T1", GLM52, TokenSpec(T=1, outlier_channels=61)),
    "glm52_mtp_verify_T4": Workload("glm52_mtp_verify_T4", GLM52,
                                    TokenSpec(T=4, rho=0.8, outlier_channels=61)),
    "glm52_prefill_T512": Workload("glm52_prefill_T512", replace(GLM52, zipf_s=1.1),
                                   TokenSpec(T=512, outlier_channels=61)),
    "glm52_chain16_T1": Workload("glm52_chain16_T1", GLM52, TokenSpec(T=1, outlier_channels=61),
                                 n_layers=16),
    # every token on the same 8 experts (router bias +2 on a seeded set): 9
    # experts x 512 pairs, a compute-bound grouped GEMM (about 2,000 int8
    # ops per weight byte), where the matrix-core rate is the measure
    "glm52_hot8_T512": Workload("glm52_hot8_T512", replace(GLM52, hot_experts=8),
                                TokenSpec(T=512, outlier_channels=61)),
    # the same layer with int8 experts (one byte per weight), the format the
    # pages keep for the MTP head: its draft step (T=1) and a verify-sized batch
    "glm52_int8_mtp_T1": Workload("glm52_int8_mtp_T1", replace(GLM52, weight_bits=8),
                                  TokenSpec(T=1, outlier_channels=61)),
    "glm52_int8_T4": Workload("glm52_int8_T4", replace(GLM52, weight_bits=8),
                              TokenSpec(T=4, rho=0.8, outlier_channels=61)),
    # the Zipf prefill batch on int8 experts (the grouped int8-MFMA kernels)
    "glm52_int8_prefill_T512": Workload("glm52_int8_prefill_T512", replace(GLM52, zipf_s=1.1, weight_bits=8),
                                        TokenSpec(T=512, outlier_channels=61)),
    # the scale-granularity variant: int4 codes with one f32 scale per group of
    # 32 (or 128) columns instead of one per row (scale bytes +25% / +6%)
    "glm52_g32_decode_T1": Workload("glm52_g32_decode_T1", replace(GLM52, group_size=32),
                                    TokenSpec(T=1, outlier_channels=61)),
    "glm52_g128_decode_T1": Workload("glm52_g128_decode_T1", replace(GLM52, group_size=128),
                                     TokenSpec(T=1, outlier_channels=61)),
    "glm52_g32_verify_T4": Workload("glm52_g32_verify_T4", replace(GLM52, group_size=32),
                                    TokenSpec(T=4, rho=0.8, outlier_channels=61)),
    "glm52_g32_prefill_T512": Workload("glm52_g32_prefill_T512", replace(GLM52, zipf_s=1.1, group_size=32),
                                       TokenSpec(T=512, outlier_channels=61)),
    # the experimental int2 experts (four codes per byte): half the int4 bytes
    "glm52_int2_decode_T1": Workload("glm52_int2_decode_T1", replace(GLM52, weight_bits=2),
                                     TokenSpec(T=1, outlier_channels=61)),
    "glm52_int2_verify_T4": Workload("glm52_int2_verify_T4", replace(GLM52, weight_bits=2),
                                     TokenSpec(T=4, rho=0.8, outlier_channels=61)),
    "glm52_int2_prefill_T512": Workload("glm52_int2_prefill_T512", replace(GLM52, zipf_s=1.1, weight_bits=2),
                                        TokenSpec(T=512, outlier_channels=61)),
}


# ------------------------------------------------ dense MLP (the first layers)
DENSE_EXPERT = 4095   # stream id of a layer's dense MLP weights, past every routed and shared expert


@dataclass(frozen=True)
class DenseSpec:
    """Shape and weight distribution of one dense SwiGLU MLP."""
    H: int
    I: int
    w_sigma: float = 0.02
    w_outlier_rate: float = 0.0
    w_outlier_mult: float = 10.0
    weight_bits: int = 8             # the dense layers' format on the pages

    @property
    def nbytes(self) -> int:
        return 3 * self.H * self.I * self.weight_bits // 8 + 4 * (2 * self.I + self.H)


@dataclass(frozen=True)
class DenseWorkload:
    name: str
    dense: DenseSpec
    tokens: TokenSpec
    seed: int = 0
    rms_eps: float = 1e-6


# intermediate size 12288 = 2H: the pages do not give it (a stated reading)
GLM52_DENSE = DenseSpec(H=6144, I=12288, w_outlier_rate=0.001)
DENSE_WORKLOADS = {
    "glm52_dense_T1": DenseWorkload("glm52_dense_T1", GLM52_DENSE, TokenSpec(T=1, outlier_channels=61)),
    "glm52_dense_T4": DenseWorkload("glm52_dense_T4", GLM52_DENSE, TokenSpec(T=4, rho=0.8, outlier_channels=61)),
    # a 64-token prefill chunk through an int8 dense layer (the grouped int8-MFMA kernels)
    "glm52_dense_T64": DenseWorkload("glm52_dense_T64", GLM52_DENSE, TokenSpec(T=64, outlier_channels=61)),
}


def dense_matrix(spec: DenseSpec, seed: int, layer: int, matrix: int) -> np.ndarray:
    """f32 weights of one dense MLP matrix: gate/up are [I][H], down is [H][I]."""
    rows, cols = (spec.I, spec.H) if matrix in (GATE, UP) else (spec.H, spec.I)
    return fill_matrix(seed, stream_expert(layer, DENSE_EXPERT, matrix), rows, cols, spec.w_sigma,
                       spec.w_outlier_rate, spec.w_outlier_mult)


def dev_dense_matrix(ptr: int, spec: DenseSpec, seed: int, layer: int, matrix: int, hip_stream: int = 0) -> None:
    rows, cols = (spec.I, spec.H) if matrix in (GATE, UP) else (spec.H, spec.I)
    dev_fill_matrix(ptr, seed, stream_expert(layer, DENSE_EXPERT, matrix), rows, cols, spec.w_sigma,
                    spec.w_outlier_rate, spec.w_outlier_mult, hip_stream=hip_stream)


def expert_matrix(spec: LayerSpec, seed: int, layer: int, expert: int, matrix: int) -> np.ndarray:
    """f32 weights of one expert matrix: gate/up are [I][H], down is [H][I]."""
    rows, cols = (spec.I, spec.H) if matrix in (GATE, UP) else (spec.H, spec.I)
    return fill_matrix(seed, stream_expert(layer, expert, matrix), rows, cols, spec.w_sigma,
                       spec.w_outlier_rate, spec.w_outlier_mult)


def dev_expert_matrix(ptr: int, spec: LayerSpec, seed: int, layer: int, expert: int, matrix: int,
                      hip_stream: int = 0) -> None:
    rows, cols = (spec.I, spec.H) if matrix in (GATE, UP) else (spec.H, spec.I)
    dev_fill_matrix(ptr, seed, stream_expert(layer, expert, matrix), rows, cols, spec.w_sigma,
                    spec.w_outlier_rate, spec.w_outlier_mult, hip_stream=hip_stream)


def router(spec: LayerSpec, seed: int, layer: int):
    """Router weights W_r [E][H] ~ N(0, 1/sqrt(H)) and selection bias b [E]."""
    W = fill_matrix(seed, stream_layer(layer, 0), spec.E, spec.H, spec.router_sigma)
    b = fill_matrix(seed, stream_layer(layer, 1), 1, spec.E, spec.bias_sigma)[0]
    if spec.zipf_s > 0:
        rank = permutation(seed, stream_layer(layer, 3), spec.E).astype(np.float64) + 1.0
        b = (b.astype(np.float64) - spec.zipf_alpha * spec.zipf_s * np.log(rank)).astype(np.float32)
    if spec.hot_experts > 0:
        hot = permutation(seed, stream_layer(layer, 4), spec.E)[:spec.hot_experts]
        b = b.copy()
        b[hot] += np.float32(spec.hot_bias)
    return W, b


def rms_gamma(H: int, seed: int, layer: int) -> np.ndarray:
    g = fill_matrix(seed, stream_layer(layer, 2), 1, H, 0.02)[0]
    return (np.float32(1.0) + g).astype(np.float32)


def outlier_channels(H: int, seed: int, count: int) -> np.ndarray:
    if count <= 0:
        return np.zeros(0, dtype=np.int64)
    return np.sort(permutation(seed, stream_tokens(0, 2), H)[:count].astype(np.int64))


def tokens(tspec: TokenSpec, H: int, seed: int) -> np.ndarray:
    """x [T][H] f32: N(0,1) rows, optionally equicorrelated, with outlier channels."""
    z = fill_matrix(seed, stream_tokens(tspec.token_set, 0), tspec.T, H, 1.0)
    if tspec.rho > 0:
        c = fill_matrix(seed, stream_tokens(tspec.token_set, 1), 1, H, 1.0)
        x = (math.sqrt(tspec.rho) * c.astype(np.float64)
             + math.sqrt(1.0 - tspec.rho) * z.astype(np.float64)).astype(np.float32)
    else:
        x = z
    ch = outlier_channels(H, seed, tspec.outlier_channels)
    if len(ch):
        x[:, ch] = x[:, ch] * np.float32(tspec.outlier_mult)
    return np.ascontiguousarray(x, dtype=np.float32)
