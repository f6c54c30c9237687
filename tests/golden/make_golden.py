"""Writes tiny_layer_oracle.json: the oracle's routing and outputs on the tiny
layer (H=256, I=128, 16 experts, top-2, shared expert, seed 0) for T=1 and
T=3. Calls only oracle/ and synth/. Rerun only when a change to the oracle's
arithmetic is justified by a reading of the pages."""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
from oracle import oracle as O, layers as OL  # noqa: E402
from synth import synth as S  # noqa: E402


def main():
    spec = S.TINY
    L = OL.full_layer(spec, 0, 0)
    out = {"_about": __doc__.strip(), "cases": {}}
    for T in (1, 3):
        x = S.tokens(S.TokenSpec(T=T), spec.H, 0)
        y, idx, w = O.moe_forward(L, x)
        out["cases"][f"T{T}"] = {"idx": idx.tolist(), "w_hex": [[float(v).hex() for v in r] for r in w],
                                 "y_hex": [[float(v).hex() for v in r] for r in y]}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_layer_oracle.json")
    with open(path, "w") as f:
        json.dump(out, f)
    print("wrote", path)


if __name__ == "__main__":
    main()
