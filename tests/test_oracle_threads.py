"""The threaded oracle build (liboracle_omp.so: the same source with the
loops over independent matrix rows, and the tokens of one expert, spread over
OpenMP threads) against the plain build, bit for bit, for every weight format:
its results are the checker of the full-size GPU batches."""
from dataclasses import replace

import numpy as np
import pytest

from oracle import layers as OL
from oracle import oracle as O
from synth import synth as S

MID = S.LayerSpec(H=512, I=256, E=8, top_k=2, w_outlier_rate=0.01)
FORMATS = {"int4": MID, "int8": replace(MID, weight_bits=8), "int2": replace(MID, weight_bits=2),
           "groups64": replace(MID, group_size=64)}


@pytest.fixture(autouse=True)
def plain_after():
    yield
    O.use_threads(False)


def test_threaded_build_reports_threads():
    O.use_threads(False)
    assert O.threads() == 1
    O.use_threads(True)
    assert O.threads() >= 1


@pytest.mark.parametrize("fmt", sorted(FORMATS))
def test_threaded_layer_equals_plain(fmt):
    spec = FORMATS[fmt]
    x = S.tokens(S.TokenSpec(T=20, token_set=31, outlier_channels=5), spec.H, 0)
    W, b = S.router(spec, 0, 0)
    runs = []
    for thr in (False, True):
        O.use_threads(thr)
        ref = OL.full_layer(spec, 0, 0)                         # packers, threaded or not
        y, idx, w = O.moe_forward(ref, x)                       # row products, threaded or not
        cache = OL.ExpertCache(spec, 0, 0)
        bt = OL.forward_batch(spec, W, b, x, lambda e: cache[e])  # tokens of an expert in parallel
        runs.append((ref, y, idx, w, bt))
    (r0, y0, i0, w0, b0), (r1, y1, i1, w1, b1) = runs
    for name in ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s"):
        assert np.array_equal(getattr(r0, name), getattr(r1, name)), name
    assert np.array_equal(y0, y1) and np.array_equal(i0, i1) and np.array_equal(w0, w1)
    for name in ("h", "hq", "hs", "ye", "y"):
        assert np.array_equal(getattr(b0, name), getattr(b1, name)), name
    assert np.array_equal(b1.y, y0)                             # the batch driver is the layer
