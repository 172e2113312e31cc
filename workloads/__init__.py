"""Seeded synthetic inputs for per-token logprob / entropy / gradient workloads.

This module only draws inputs: logits, labels, per-token weights, masks and the
positions of rows inside a batch.  It holds none of the arithmetic of the
method itself, so both the fp64 oracle and the GPU path may use it.

Every row is drawn from its own PCG64 stream, ``default_rng([seed, cfg, 1, row])``,
so any row of any workload can be regenerated on the host without drawing the
others.  Choices that concern a whole workload (which rows are ignored or get a
peaked label logit) come from ``default_rng([seed, cfg, 0, k])``.

Logits are drawn in fp32 (``standard_normal`` times sigma, one fp32 rounding),
label boosts are added in fp32, and bf16 workloads then round to bf16 with
round-to-nearest-even.  A bf16 row is returned as its uint16 bit patterns.

The workload shapes follow the vocabulary size of the Qwen3 component benchmark
in "[RL] Avoid full-vocab gather for TP policy statistics" (torchtitan PR #4685,
"Performance evidence": V = 151,936) and the case list of that PR's
"Correctness and compatibility" section (FP32/BF16, even/uneven vocabulary,
ignored labels, partially masked logits, non-uniform weights).  The real RL
rollouts behind those numbers are not available; these draws stand in for them.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

IGNORE_INDEX = -100
QWEN3_VOCAB = 151_936
DEFAULT_SEED = 20260916


@dataclasses.dataclass(frozen=True)
class Workload:
    """Recipe of one synthetic workload."""

    cfg: int                 # workload id, part of every seed
    name: str
    rows: int
    vocab: int
    dtype: str               # "f32" or "bf16"
    sigma: float             # logits ~ sigma * N(0, 1)
    boost: float = 0.0       # added to the label logit of the boosted rows
    n_boosted: int = 0       # rows whose label logit gets +boost
    n_ignored: int = 0       # rows whose label is IGNORE_INDEX
    n_masked_cols: int = 0   # -inf columns per row, never the label
    weighted: bool = False   # per-row weights ~ U(0, 2) (else None, meaning 1)
    backward: bool = True


WORKLOADS = {
    1: Workload(1, "fwd_256x151936_f32", 256, QWEN3_VOCAB, "f32", 2.0,
                n_ignored=round(0.05 * 256), backward=False),
    2: Workload(2, "fwdbwd_4096x151936_bf16", 4096, QWEN3_VOCAB, "bf16", 3.0,
                boost=8.0, n_boosted=2048, n_ignored=round(0.03 * 4096),
                weighted=True),
    3: Workload(3, "masked_2048x151937_f32", 2048, QWEN3_VOCAB + 1, "f32", 1.5,
                n_masked_cols=int(0.1 * (QWEN3_VOCAB + 1))),
    4: Workload(4, "invariance_bf16", 16, QWEN3_VOCAB, "bf16", 2.0,
                weighted=True),
    5: Workload(5, "large_32768x151936_bf16", 32_768, QWEN3_VOCAB, "bf16", 2.0,
                boost=10.0, n_boosted=round(0.08 * 32_768), weighted=True),
}

# Batch sizes of the invariance sweep and the chunking of the large workload.
INVARIANCE_BATCHES = (1, 16, 512, 8192)
LARGE_CHUNKS = 4


@dataclasses.dataclass
class Batch:
    """A drawn batch.  ``logits`` is float32 [n, V] or uint16 bf16 bits [n, V]."""

    logits: np.ndarray
    labels: np.ndarray                 # int64 [n]
    weights: Optional[np.ndarray]      # float32 [n] or None
    dtype: str
    vocab: int

    @property
    def rows(self) -> int:
        return int(self.labels.shape[0])


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); return bits.

    Only finite values and -inf occur in these workloads.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def _workload_choice(seed: int, w: Workload, k: int, size: int) -> np.ndarray:
    """Rows chosen for workload-level property ``k`` (exact count, no Bernoulli)."""
    if size == 0:
        return np.zeros(0, dtype=np.int64)
    g = np.random.default_rng([seed, w.cfg, 0, k])
    return np.sort(g.choice(w.rows, size=size, replace=False)).astype(np.int64)


@dataclasses.dataclass(frozen=True)
class _RowPlan:
    boosted: frozenset
    ignored: frozenset


def _plan(seed: int, w: Workload) -> _RowPlan:
    return _RowPlan(
        boosted=frozenset(_workload_choice(seed, w, 1, w.n_boosted).tolist()),
        ignored=frozenset(_workload_choice(seed, w, 2, w.n_ignored).tolist()),
    )


def _draw_row(seed: int, w: Workload, plan: _RowPlan, r: int, stream: int = 1):
    """Draw row ``r``: (fp32 logits, label, weight)."""
    g = np.random.default_rng([seed, w.cfg, stream, r])
    x = g.standard_normal(w.vocab, dtype=np.float32)
    x *= np.float32(w.sigma)
    label = int(g.integers(0, w.vocab))
    weight = np.float32(g.random(dtype=np.float32) * np.float32(2.0))
    if w.n_masked_cols:
        # masked columns drawn among the other V-1 columns, so never the label
        m = g.choice(w.vocab - 1, size=w.n_masked_cols, replace=False)
        m = np.where(m >= label, m + 1, m)
        x[m] = -np.inf
    if r in plan.boosted:
        x[label] += np.float32(w.boost)
    if r in plan.ignored:
        label = IGNORE_INDEX
    return x, label, weight


def _fill(seed, w, plan, rows, logits, labels, weights, stream, threads):
    def one(i):
        x, lab, wt = _draw_row(seed, w, plan, int(rows[i]), stream)
        logits[i] = f32_to_bf16_bits(x) if w.dtype == "bf16" else x
        labels[i] = lab
        weights[i] = wt

    if threads <= 1 or len(rows) < 8:
        for i in range(len(rows)):
            one(i)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(one, range(len(rows))))


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def draw(cfg: int, rows=None, seed: int = DEFAULT_SEED, threads: Optional[int] = None,
         stream: int = 1) -> Batch:
    """Draw workload ``cfg`` (all rows, or the given row indices)."""
    w = WORKLOADS[cfg]
    rows = np.arange(w.rows) if rows is None else np.asarray(rows, dtype=np.int64)
    plan = _plan(seed, w)
    dt = np.uint16 if w.dtype == "bf16" else np.float32
    logits = np.empty((len(rows), w.vocab), dtype=dt)
    labels = np.empty(len(rows), dtype=np.int64)
    weights = np.empty(len(rows), dtype=np.float32)
    _fill(seed, w, plan, rows, logits, labels, weights, stream,
          default_threads() if threads is None else threads)
    return Batch(logits, labels, weights if w.weighted else None, w.dtype, w.vocab)


# ---------------------------------------------------------------------------
# Batch-invariance sweep: 16 fixed rows placed inside batches of other rows.
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class InvarianceCase:
    batch: Batch
    positions: np.ndarray      # where the 16 fixed rows sit, in fixed-row order


def invariance_batches(seed: int = DEFAULT_SEED, sizes=INVARIANCE_BATCHES,
                       threads: Optional[int] = None):
    """Yield (n, [InvarianceCase]) for the invariance sweep.

    n == 1 yields 16 single-row batches; n == 16 is the 16 rows in a seeded
    order; larger n puts them at seeded positions among fresh filler rows
    (filler drawn from stream n, so every batch size gets its own filler).
    """
    w = WORKLOADS[4]
    core = draw(4, seed=seed, threads=threads)
    for n in sizes:
        if n == 1:
            yield n, [InvarianceCase(
                Batch(core.logits[i:i + 1].copy(), core.labels[i:i + 1].copy(),
                      core.weights[i:i + 1].copy(), w.dtype, w.vocab),
                np.array([0]))
                for i in range(w.rows)]
            continue
        g = np.random.default_rng([seed, w.cfg, 0, 100 + n])
        if n == w.rows:
            pos = g.permutation(n)
            logits = np.empty_like(core.logits)
            labels = np.empty_like(core.labels)
            weights = np.empty_like(core.weights)
        else:
            pos = g.choice(n, size=w.rows, replace=False)
            filler_rows = np.arange(n)
            filler = _filler(seed, w, filler_rows, n, threads)
            logits, labels, weights = filler.logits, filler.labels, filler.weights
        logits[pos] = core.logits
        labels[pos] = core.labels
        weights[pos] = core.weights
        yield n, [InvarianceCase(Batch(logits, labels, weights, w.dtype, w.vocab),
                                 np.asarray(pos))]


def _filler(seed, w, rows, n, threads):
    plan = _RowPlan(frozenset(), frozenset())
    logits = np.empty((len(rows), w.vocab), dtype=np.uint16)
    labels = np.empty(len(rows), dtype=np.int64)
    weights = np.empty(len(rows), dtype=np.float32)
    _fill(seed, w, plan, rows, logits, labels, weights, 1000 + n,
          default_threads() if threads is None else threads)
    return Batch(logits, labels, weights, w.dtype, w.vocab)


def chunk_bounds(vocab: int, n_chunks: int):
    """Column bounds of ``n_chunks`` contiguous vocabulary chunks (last one ragged)."""
    width = -(-vocab // n_chunks)
    return [(c * width, min(vocab, (c + 1) * width)) for c in range(n_chunks)
            if c * width < vocab]


def random_batch(rows: int, vocab: int, dtype: str, seed: int, sigma: float = 2.0,
                 ignore_frac: float = 0.0, mask_frac: float = 0.0,
                 weighted: bool = True, stream: int = 7) -> Batch:
    """A small free-form batch for tests (shapes outside the named workloads)."""
    g = np.random.default_rng([seed, 999, stream, rows, vocab])
    x = (g.standard_normal((rows, vocab), dtype=np.float32) * np.float32(sigma))
    labels = g.integers(0, vocab, size=rows).astype(np.int64)
    if mask_frac > 0.0 and vocab > 1:
        k = int(mask_frac * vocab)
        for r in range(rows):
            cols = g.choice(vocab - 1, size=min(k, vocab - 1), replace=False)
            cols = np.where(cols >= labels[r], cols + 1, cols)
            x[r, cols] = -np.inf
    n_ign = int(round(ignore_frac * rows))
    if n_ign:
        labels[g.choice(rows, size=n_ign, replace=False)] = IGNORE_INDEX
    weights = (g.random(rows, dtype=np.float32) * np.float32(2.0)) if weighted else None
    logits = f32_to_bf16_bits(x) if dtype == "bf16" else x
    return Batch(logits, labels, weights, dtype, vocab)


# ---------------------------------------------------------------------------
# Hidden states and lm_head rows (bf16) whose products are N(0, sigma^2)-sized
# logits: hidden ~ N(0, 1), weight ~ N(0, (sigma / sqrt(d))^2).  Qwen3-4B's
# hidden size is 2,560 and its vocabulary 151,936.
# ---------------------------------------------------------------------------

LMHEAD_HIDDEN = 2560


@dataclasses.dataclass
class LmheadBatch:
    hidden: np.ndarray      # uint16 bf16 bits [n, d]
    weight: np.ndarray      # uint16 bf16 bits [V, d]
    labels: np.ndarray      # int64 [n]


def lmhead_batch(n: int, vocab: int, d: int, seed: int = DEFAULT_SEED, sigma: float = 2.0,
                 ignore_frac: float = 0.0, threads: Optional[int] = None) -> LmheadBatch:
    threads = default_threads() if threads is None else threads
    hidden = np.empty((n, d), dtype=np.uint16)
    weight = np.empty((vocab, d), dtype=np.uint16)
    scale = np.float32(sigma / np.sqrt(d))

    def rows(arr, kind, a, b, sc):
        g = np.random.default_rng([seed, 600 + kind, a])
        x = g.standard_normal((b - a, d), dtype=np.float32)
        if sc is not None:
            x *= sc
        arr[a:b] = f32_to_bf16_bits(x)

    blocks = [(hidden, 0, a, min(a + 1024, n), None) for a in range(0, n, 1024)] + \
             [(weight, 1, a, min(a + 1024, vocab), scale) for a in range(0, vocab, 1024)]
    with ThreadPoolExecutor(max(1, threads)) as ex:
        list(ex.map(lambda t: rows(*t), blocks))
    g = np.random.default_rng([seed, 700, n, vocab])
    labels = g.integers(0, vocab, size=n).astype(np.int64)
    k = int(round(ignore_frac * n))
    if k:
        labels[g.choice(n, size=k, replace=False)] = IGNORE_INDEX
    return LmheadBatch(hidden, weight, labels)


def sparse_lmhead_batch(n: int, vocab: int, d: int, seed: int = DEFAULT_SEED, nnz: int = 64,
                        pool: int = 1024) -> LmheadBatch:
    """Hidden and lm_head rows (bf16 bits) that are zero except for ``nnz``
    entries of +1 or -1 per row, at columns drawn from one seeded pool of
    ``pool`` columns spread over [0, d) that always holds column d - 1.  Every
    logit is then a small integer, which fp32 accumulates exactly at any d:
    inputs for the largest hidden sizes, where dense random rows would make the
    logits' own rounding the subject of the test."""
    g = np.random.default_rng([seed, 800, n, vocab, d])
    cols = np.unique(np.concatenate([g.choice(d, size=pool - 1, replace=False), [d - 1]]))
    one, minus_one = f32_to_bf16_bits(np.array([1.0, -1.0], dtype=np.float32))

    def fill(rows):
        out = np.zeros((rows, d), dtype=np.uint16)
        for r in range(rows):
            c = g.choice(cols, size=min(nnz, cols.size), replace=False)
            out[r, c] = np.where(g.random(c.size) < 0.5, one, minus_one)
        return out

    hidden, weight = fill(n), fill(vocab)
    labels = g.integers(0, vocab, size=n).astype(np.int64)
    return LmheadBatch(hidden, weight, labels)
