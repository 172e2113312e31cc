"""The seeded input generators: determinism, exact counts, bf16 rounding."""
import numpy as np
import pytest

import workloads as wl


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    g = np.random.default_rng(0)
    x = np.concatenate([g.standard_normal(100_000).astype(np.float32) * 7,
                        np.array([-np.inf, 0.0, -0.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8,
                                  3.0e38], dtype=np.float32)])
    ours = wl.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_rows_regenerate_identically():
    full = wl.draw(1, rows=np.arange(20), threads=4)
    part = wl.draw(1, rows=[3, 17], threads=1)
    np.testing.assert_array_equal(part.logits, full.logits[[3, 17]])
    np.testing.assert_array_equal(part.labels, full.labels[[3, 17]])


def test_exact_counts():
    w1 = wl.WORKLOADS[1]
    b = wl.draw(1, threads=8)
    assert b.logits.shape == (256, 151_936) and b.logits.dtype == np.float32
    assert (b.labels == wl.IGNORE_INDEX).sum() == 13 == w1.n_ignored
    assert b.weights is None
    plan = wl._plan(wl.DEFAULT_SEED, wl.WORKLOADS[2])
    assert len(plan.boosted) == 2048 and len(plan.ignored) == 123
    plan5 = wl._plan(wl.DEFAULT_SEED, wl.WORKLOADS[5])
    assert len(plan5.boosted) == 2621 and len(plan5.ignored) == 0


def test_masked_workload_rows():
    b = wl.draw(3, rows=[0, 5, 2047], threads=1)
    assert b.logits.shape == (3, 151_937)
    for i in range(3):
        masked = np.isneginf(b.logits[i])
        assert masked.sum() == 15_193
        assert not masked[b.labels[i]]


def test_bf16_workload_and_boost():
    rows = sorted(wl._plan(wl.DEFAULT_SEED, wl.WORKLOADS[2]).boosted)[:3]
    b = wl.draw(2, rows=rows, threads=1)
    assert b.logits.dtype == np.uint16 and b.weights is not None
    assert np.all((b.weights >= 0) & (b.weights < 2))
    for i in range(3):
        if b.labels[i] >= 0:
            z = (b.logits[i].astype(np.uint32) << 16).view(np.float32)
            assert z[b.labels[i]] > 3.0   # +8 on the label logit


def test_invariance_batches_place_the_same_rows():
    core = wl.draw(4, threads=2)
    for n, cases in wl.invariance_batches(sizes=(1, 16, 512), threads=4):
        for case in cases:
            b = case.batch
            assert b.rows == n
            if n == 1:
                continue
            np.testing.assert_array_equal(b.logits[case.positions], core.logits)
            np.testing.assert_array_equal(b.labels[case.positions], core.labels)
            np.testing.assert_array_equal(b.weights[case.positions], core.weights)


def test_chunk_bounds():
    assert wl.chunk_bounds(151_936, 4) == [(0, 37_984), (37_984, 75_968),
                                           (75_968, 113_952), (113_952, 151_936)]
    b = wl.chunk_bounds(151_937, 4)
    assert b[-1] == (113_955, 151_937) and sum(e - a for a, e in b) == 151_937
