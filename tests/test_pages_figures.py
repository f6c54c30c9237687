"""The layer shape and format against the figures the pages print
(tests/golden/pages_figures.json, each entry cited there)."""
import json
import os

from synth import synth as S

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_figures.json")))


def test_expert_size_matches_pages():
    spec = S.GLM52
    # gate and up are [I][H] nibbles, down is [H][I], one f32 scale per row
    assert spec.expert_bytes == 18_915_328
    assert round(spec.expert_bytes / 1e6) == GOLD["expert_int4_megabytes_approx"]["value"]


def test_layer_counts_match_pages():
    assert S.GLM52.top_k == GOLD["routed_experts_per_token"]["value"]
    assert S.GLM52.E == GOLD["experts_per_moe_layer"]["value"]
    per_token = 75 * S.GLM52.top_k * S.GLM52.expert_bytes
    assert round(per_token / 1e9) == GOLD["cold_bytes_per_token_gb_approx"]["value"]


def test_tiny_layer_oracle_regression():
    """The oracle still reproduces the stored tiny-layer result (written by
    tests/golden/make_golden.py, which calls only the oracle)."""
    import numpy as np
    from oracle import oracle as O, layers as OL
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "tiny_layer_oracle.json")))
    L = OL.full_layer(S.TINY, 0, 0)
    for T in (1, 3):
        case = gold["cases"][f"T{T}"]
        y, idx, w = O.moe_forward(L, S.tokens(S.TokenSpec(T=T), S.TINY.H, 0))
        assert idx.tolist() == case["idx"]
        assert [[float(v).hex() for v in r] for r in w] == case["w_hex"]
        assert [[float(v).hex() for v in r] for r in y] == case["y_hex"]
