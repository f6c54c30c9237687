"""Pins of the seeded input generator (not the method): Philox4x32-10 against the
known-answer vectors published with the generator's definition (Salmon et al.,
SC'11, Random123 distribution), determinism, counter addressing and moments."""
import math

import numpy as np
import pytest

from synth import synth as S


@pytest.mark.parametrize("ctr,key,expect", [
    ([0, 0, 0, 0], [0, 0], [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]),
    ([0xFFFFFFFF] * 4, [0xFFFFFFFF] * 2, [0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD]),
    ([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344], [0xA4093822, 0x299F31D0],
     [0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]),
])
def test_philox_known_answers(ctr, key, expect):
    assert S.philox(ctr, key) == expect


def test_row_range_addressing_is_counter_based():
    full = S.fill_matrix(0, S.stream_expert(0, 3, 1), 64, 96, 0.02, 0.05, 10.0)
    part = S.fill_matrix(0, S.stream_expert(0, 3, 1), 16, 96, 0.02, 0.05, 10.0, row0=40)
    assert np.array_equal(full[40:56], part)
    again = S.fill_matrix(0, S.stream_expert(0, 3, 1), 64, 96, 0.02, 0.05, 10.0)
    assert np.array_equal(full, again)
    other = S.fill_matrix(0, S.stream_expert(0, 4, 1), 64, 96, 0.02, 0.05, 10.0)
    assert not np.array_equal(full, other)


def test_irwin_hall_integer_and_scale():
    # the float value is exactly (float)z * c for the integer Irwin-Hall sum z
    c = S.normal_scale(0.02)
    m = S.fill_matrix(7, 123, 4, 8, 0.02)
    lib = S._lib()
    for r in range(4):
        for col in range(8):
            z = lib.synth_normal_int(7, 123, r * 8 + col)
            assert z % 2 == 0 and abs(z) <= 524280
            assert m[r, col] == np.float32(np.float32(z) * np.float32(c))


def test_moments_and_outlier_rate():
    m = S.fill_matrix(0, S.stream_expert(0, 0, 0), 2048, 1024, 0.02)
    assert abs(m.mean()) < 2e-5
    assert abs(m.std() / 0.02 - 1) < 2e-3
    kurt = ((m.astype(np.float64) / m.std()) ** 4).mean()
    assert abs(kurt - (3 - 1.2 / 8)) < 0.02          # Irwin-Hall n=8 excess kurtosis -1.2/n
    rows = 200000
    hits = sum(S.outlier_col(0, 99, r, 6144, 0.001) >= 0 for r in range(rows))
    assert abs(hits / rows - 0.001) < 4 * math.sqrt(0.001 / rows)


def test_token_recipes():
    wl = S.WORKLOADS["glm52_mtp_verify_T4"]
    x = S.tokens(wl.tokens, wl.layer.H, 0)
    assert x.shape == (4, 6144) and x.dtype == np.float32
    ch = S.outlier_channels(6144, 0, 61)
    assert len(set(ch.tolist())) == 61
    mask = np.ones(6144, bool)
    mask[ch] = False
    base = x[:, mask].astype(np.float64)
    corr = np.corrcoef(base)
    off = corr[~np.eye(4, dtype=bool)]
    assert abs(off.mean() - 0.8) < 0.03
    assert abs(np.abs(x[:, ch]).mean() / np.abs(base).mean() - 20) < 2


def test_zipf_bias_skews_toward_low_ranks():
    spec = S.WORKLOADS["glm52_prefill_T512"].layer
    _, b = S.router(spec, 0, 0)
    rank = S.permutation(0, S.stream_layer(0, 3), spec.E) + 1
    # the bias falls with ln(rank) at slope alpha*s
    slope = np.polyfit(np.log(rank), b.astype(np.float64), 1)[0]
    assert abs(slope + spec.zipf_alpha * spec.zipf_s) < 0.004
