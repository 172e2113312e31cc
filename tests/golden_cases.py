"""Loader of tests/golden/tiny_rows.json (written by tests/golden/make_golden.py)."""
import json
import os

import numpy as np

PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "tiny_rows.json")


def load():
    with open(PATH) as f:
        doc = json.load(f)
    out = []
    for c in doc["cases"]:
        if c["dtype"] == "bf16":
            logits = np.array(c["logits"], dtype=np.uint16)
        else:
            logits = np.array(c["logits"], dtype=np.float32)
        out.append(dict(c, logits=logits))
    return out
