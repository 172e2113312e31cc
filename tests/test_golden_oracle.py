"""The oracle's fast mode against the stored 50-digit brute-force fixture."""
import numpy as np
import pytest

import oracle.bi_oracle as orc
from golden_cases import load

CASES = load()


@pytest.mark.parametrize("k", range(len(CASES)))
def test_fast_mode_matches_golden(k):
    c = CASES[k]
    z = orc.decode(c["logits"], c["dtype"])[None, :]
    lp, h, lse = orc.forward(z, np.array([c["label"]]))
    assert lp[0] == pytest.approx(c["logprob"], abs=1e-13)
    assert h[0] == pytest.approx(c["entropy"], abs=1e-13)
    assert lse[0] == pytest.approx(c["lse"], abs=1e-13)
    g = orc.backward(z, np.array([c["label"]]), lse, np.array([c["weight"]]))[0]
    np.testing.assert_allclose(g, c["grad"], rtol=1e-12, atol=1e-15)
