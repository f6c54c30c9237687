"""Helpers shared by the GPU parity tests."""
import numpy as np
import torch

from int4_quantized_expert_sigmoid_amd import api
from synth import synth as S

PERM8 = np.array([0, 2, 4, 6, 1, 3, 5, 7])   # stored position of element i of an 8-group is perm8(i)
INV8 = np.array([0, 4, 1, 5, 2, 6, 3, 7])    # element at stored position p


def perm_positions(n):
    """Stored position of each natural index for a reordered [n] int8 vector."""
    i = np.arange(n)
    return (i & ~7) + np.where(i & 1, 4 + ((i & 7) >> 1), (i & 7) >> 1)


def unreorder(stored: np.ndarray) -> np.ndarray:
    n = stored.shape[-1]
    return stored[..., perm_positions(n)]


def rel_err(y: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """|y - ref| / max(|ref|, rms(ref)) per element (rms over each token's row)."""
    ref64 = ref.astype(np.float64)
    rms = np.sqrt((ref64 ** 2).mean(axis=-1, keepdims=True))
    return np.abs(y.astype(np.float64) - ref64) / np.maximum(np.abs(ref64), rms)


def ws_views(layer, T, ws: torch.Tensor, flags=0):
    """numpy copies of the intermediates the last call left in the workspace."""
    lay = api.workspace_layout(layer, T, flags)
    b = ws.cpu().numpy()
    k, H, I = layer.top_k, layer.H, layer.I
    n = lay.n_pairs_max

    def arr(off, count, dt):
        return np.frombuffer(b[off: off + count * np.dtype(dt).itemsize].tobytes(), dtype=dt)

    return dict(path=lay.path,
                pair_of=arr(lay.pair_of, T * k, np.int32).reshape(T, k),
                shared_pair=arr(lay.shared_pair, T, np.int32),
                h=arr(lay.h, n * I, np.float32).reshape(n, I),
                hq=arr(lay.hq, n * I, np.int8).reshape(n, I),
                hs=arr(lay.hs, n * (I // 32), np.float32).reshape(n, I // 32),
                ye=arr(lay.ye, n * H, np.float32).reshape(n, H),
                idx=arr(lay.idx, T * k, np.int32).reshape(T, k),
                w=arr(lay.w, T * k, np.float32).reshape(T, k))


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


class DeviceGenExperts:
    """The oracle's packed experts of one layer, from f32 weights the
    generator's device twin writes (the same values as the host generator,
    checked bit for bit by test_device_generator_matches_host), copied to
    the host and packed by the oracle's own packer. expert_of(e) for
    oracle.layers.forward_batch; the f32 generation on the GPU is what makes
    a whole GLM-shaped layer affordable on the host."""

    def __init__(self, spec, seed: int = 0, layer: int = 0):
        self.spec, self.seed, self.layer = spec, seed, layer
        self.buf = torch.empty(spec.H * spec.I, dtype=torch.float32, device="cuda")

    def __call__(self, e: int):
        from oracle import layers as OL
        sp = self.spec
        n = sp.H * sp.I
        stream = torch.cuda.current_stream().cuda_stream
        mats = []
        for m, shape in ((S.GATE, (sp.I, sp.H)), (S.UP, (sp.I, sp.H)), (S.DOWN, (sp.H, sp.I))):
            S.dev_expert_matrix(self.buf.data_ptr(), sp, self.seed, self.layer, e, m, hip_stream=stream)
            mats.append(self.buf[:n].view(shape).cpu().numpy())
        return OL.pack_matrices(sp, *mats)
