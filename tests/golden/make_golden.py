"""Write tests/golden/tiny_rows.json from the oracle's 50-digit brute force.

Run from the repository root:  python tests/golden/make_golden.py

The cases are small rows that exercise the case list of "[RL] Avoid full-vocab
gather for TP policy statistics" (torchtitan PR #4685), section "Correctness
and compatibility": FP32 and BF16 logits, even and uneven (odd) vocabulary
sizes, ignored labels (-100), partially masked (-inf) logits and non-uniform
per-token weights.  The expected values come only from ``oracle.brute_force``
(mpmath, 50 digits, textbook softmax without a shift).
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle.bi_oracle import brute_force, decode  # noqa: E402
from workloads import f32_to_bf16_bits  # noqa: E402


def cases():
    g = np.random.default_rng(4685)
    out = []
    specs = [(1, "f32"), (2, "f32"), (3, "bf16"), (7, "f32"), (8, "bf16"), (9, "bf16"),
             (16, "f32"), (17, "bf16"), (31, "f32"), (33, "bf16"), (64, "f32"), (65, "bf16")]
    for k, (V, dtype) in enumerate(specs):
        x = (g.standard_normal(V) * 2.5).astype(np.float32)
        y = int(g.integers(0, V))
        if k % 3 == 1 and V > 2:
            cols = g.choice([j for j in range(V) if j != y], size=V // 4, replace=False)
            x[cols] = -np.inf
        if k % 4 == 2:
            y = -100
        w = float(np.float32(g.uniform(0.0, 2.0)))
        if dtype == "bf16":
            bits = f32_to_bf16_bits(x)
            z = decode(bits, "bf16")
            enc = [int(b) for b in bits]
        else:
            z = decode(x, "f32")
            enc = [float(v) for v in x]
        lp, h, lse, grad = brute_force(z, y, w)
        out.append({"vocab": V, "dtype": dtype, "logits": enc, "label": y, "weight": w,
                    "logprob": lp, "entropy": h, "lse": lse, "grad": grad})
    return out


if __name__ == "__main__":
    doc = {
        "source": ("oracle.brute_force (mpmath, 50 digits); case list of torchtitan PR "
                   "#4685 'Avoid full-vocab gather for TP policy statistics', section "
                   "'Correctness and compatibility'"),
        "encoding": "f32 logits as JSON numbers (-Infinity for masked); bf16 as uint16 bits",
        "cases": cases(),
    }
    with open(os.path.join(HERE, "tiny_rows.json"), "w") as f:
        json.dump(doc, f, indent=1, allow_nan=True)
    print("wrote", len(doc["cases"]), "cases")
