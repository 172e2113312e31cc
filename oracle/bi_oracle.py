"""fp64 CPU oracle for per-token logprob, entropy, gradient and vocabulary-chunk
statistics.

TEST INFRASTRUCTURE ONLY.  This module is the plain, slow, obviously correct
definition that the GPU library is checked against.  Only the tests, the smoke
check and the benchmark's CPU-baseline leg may import it; the library itself
never does, and it shares no code with the GPU path (kernels, host code,
binding).  Inputs come from ``workloads`` (which holds no arithmetic of the
method), and everything here runs in float64 on the exact input values
(bf16 and fp32 upcast exactly).

Sources (page titles and sections; no code is copied from them):

* "[RL] Avoid full-vocab gather for TP policy statistics" (torchtitan PR #4685):
  - Summary: token logprobs and entropy per token; per-token gradients from the
    cross-entropy backward; exact entropy from sufficient statistics.
  - Why: the per-token statistics are the global maximum, the softmax
    denominator, the target contribution and the entropy-weighted sum; entropy
    is a metric without a gradient.
  - Correctness and compatibility: FP32/BF16 logits, even and uneven vocabulary,
    ignored labels, partially masked logits, non-uniformly weighted gradients.
  - review reply "Input sharding contract of compute_logprobs": on full logits
    the logprob is plain per-token cross-entropy (reduction "none"), negated.
  - review reply "Batch invariance under the patched logprob path", Q1 and Q2:
    entropy is logsumexp plus softmax on the full row; the maximum combines
    exactly across shards while the sums do not.
  - review comments: the backward yields only the logits gradient.

Definitions (row i, logits z in R^V with -inf allowed, label y, weight w;
F = set of columns with z_j > -inf, m = max_j z_j):

    S       = sum_{j in F} exp(z_j - m)
    U       = sum_{j in F} exp(z_j - m) * (z_j - m)        (0 for masked columns)
    lse     = m + ln S
    logprob = z_y - lse                     (+0.0 when y == ignore_index)
    entropy = -sum_{j in F} p_j ln p_j = ln S - U / S      (for every row)
    grad_j  = w * (p_j - [j == y]),  p_j = exp(z_j - lse)  (+0.0 rows when ignored)

Readings taken where the pages are silent (the plainest reading that the rest of
the pages supports, each pinned by a test):
  * masked columns contribute 0 * ln 0 = 0 to the entropy (limit value);
  * ignored rows still get an entropy; their logprob and gradient are +0.0;
  * a label outside [0, V) that is not ignore_index yields NaN logprob and a
    NaN gradient row (the GPU library also raises a status flag);
  * chunk statistics store U about the chunk's own max, and a chunk's target
    contribution is 0.0 unless it holds the label (sums to the label logit);
  * fully masked chunks (S == 0) contribute nothing to the combine.

A slow brute-force mode (``brute_force``) evaluates the textbook form
-sum p ln p with p = exp(z) / sum exp(z) (no shift) in 50-digit mpmath; it is a
different formula from the fast mode, so their agreement checks the identity.
"""
from __future__ import annotations

import numpy as np

IGNORE_INDEX = -100


# ---------------------------------------------------------------------------
# input decoding (exact)
# ---------------------------------------------------------------------------

def decode(logits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of fp32 logits or of bf16 bit patterns (uint16)."""
    if dtype == "bf16":
        bits = np.asarray(logits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(logits, dtype=np.float32).astype(np.float64)
    if dtype == "f64":
        return np.asarray(logits, dtype=np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def _as2d(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    return z[None, :] if z.ndim == 1 else z


# ---------------------------------------------------------------------------
# per-row sufficient statistics ("Why": max, denominator, entropy-weighted sum)
# ---------------------------------------------------------------------------

def row_max(z: np.ndarray) -> np.ndarray:
    """m = max_j z_j (exact); -inf for a row with no finite entry."""
    return z.max(axis=1)


def finite_mask(z: np.ndarray) -> np.ndarray:
    """Columns that take part in the softmax: every column that is not -inf."""
    return ~np.isneginf(z)


def shifted(z: np.ndarray, m: np.ndarray) -> np.ndarray:
    """z_j - m, with the shift taken as 0 when the row has no finite entry."""
    ref = np.where(np.isfinite(m), m, 0.0)
    return z - ref[:, None]


def denominator(d: np.ndarray, keep: np.ndarray) -> np.ndarray:
    """S = sum over finite columns of exp(z_j - m)."""
    return np.where(keep, np.exp(np.where(keep, d, 0.0)), 0.0).sum(axis=1)


def weighted_sum(d: np.ndarray, keep: np.ndarray) -> np.ndarray:
    """U = sum over finite columns of exp(z_j - m) * (z_j - m); 0 for -inf columns."""
    dd = np.where(keep, d, 0.0)
    return np.where(keep, np.exp(dd) * dd, 0.0).sum(axis=1)


def row_statistics(z: np.ndarray):
    """(m, S, U) of every row of z, about the row's own max."""
    z = _as2d(z)
    m = row_max(z)
    keep = finite_mask(z)
    d = shifted(z, m)
    return m, denominator(d, keep), weighted_sum(d, keep)


# ---------------------------------------------------------------------------
# target contribution ("Why": the target logit; labels may be ignored)
# ---------------------------------------------------------------------------

def label_kind(labels: np.ndarray, vocab: int, ignore_index: int = IGNORE_INDEX):
    """0 = valid label, 1 = ignored, 2 = out of range (bad)."""
    labels = np.asarray(labels, dtype=np.int64)
    kind = np.where(labels == ignore_index, 1,
                    np.where((labels >= 0) & (labels < vocab), 0, 2))
    return kind


def target_logit(z: np.ndarray, labels: np.ndarray, ignore_index=IGNORE_INDEX):
    """z_y for valid labels; 0.0 for ignored rows; NaN for bad labels."""
    z = _as2d(z)
    n, v = z.shape
    kind = label_kind(labels, v, ignore_index)
    idx = np.where(kind == 0, labels, 0)
    t = z[np.arange(n), idx]
    return np.where(kind == 0, t, np.where(kind == 1, 0.0, np.nan))


# ---------------------------------------------------------------------------
# forward: logprob, entropy, lse
# ---------------------------------------------------------------------------

def finalize(m, S, U, t, kind):
    """lse = m + ln S, logprob = t - lse (+0.0 if ignored), entropy = ln S - U/S."""
    with np.errstate(divide="ignore", invalid="ignore"):
        ln_s = np.log(S)
        lse = m + ln_s
        entropy = ln_s - U / S
        logprob = np.where(kind == 1, 0.0, t - lse)
    logprob = np.where(kind == 2, np.nan, logprob)
    return logprob, entropy, lse


def forward(z: np.ndarray, labels: np.ndarray, ignore_index: int = IGNORE_INDEX):
    """Per-row (logprob, entropy, lse) in float64 for logits z [n, V] (float64)."""
    z = _as2d(z)
    m, S, U = row_statistics(z)
    kind = label_kind(labels, z.shape[1], ignore_index)
    t = target_logit(z, labels, ignore_index)
    return finalize(m, S, U, t, kind)


# ---------------------------------------------------------------------------
# backward: grad = w * (softmax - onehot)
# ---------------------------------------------------------------------------

def softmax_from_lse(z: np.ndarray, lse: np.ndarray) -> np.ndarray:
    """p_j = exp(z_j - lse) on finite columns, 0 on -inf columns."""
    keep = finite_mask(z)
    with np.errstate(invalid="ignore"):
        d = np.where(keep, z - lse[:, None], 0.0)
    return np.where(keep, np.exp(d), 0.0)


def backward(z: np.ndarray, labels: np.ndarray, lse: np.ndarray, weights=None,
             ignore_index: int = IGNORE_INDEX) -> np.ndarray:
    """grad [n, V] float64: w * (p - onehot(y)); +0.0 rows if ignored, NaN rows if bad."""
    z = _as2d(z)
    n, v = z.shape
    lse = np.asarray(lse, dtype=np.float64)
    w = np.ones(n) if weights is None else np.asarray(weights, dtype=np.float64)
    kind = label_kind(labels, v, ignore_index)
    p = softmax_from_lse(z, lse)
    grad = w[:, None] * p
    rows = np.nonzero(kind == 0)[0]
    cols = np.asarray(labels, dtype=np.int64)[rows]
    grad[rows, cols] = w[rows] * (p[rows, cols] - 1.0)
    grad[kind == 1] = 0.0
    grad[kind == 2] = np.nan
    return grad


# ---------------------------------------------------------------------------
# vocabulary-chunk statistics and their exact combine
# ("Why" + "Batch invariance under the patched logprob path", Q2)
# ---------------------------------------------------------------------------

STAT_FIELDS = ("max", "sumexp", "target", "sumexp_logit")


def chunk_stats(z_chunk: np.ndarray, labels: np.ndarray, vocab_offset: int, vocab: int,
                ignore_index: int = IGNORE_INDEX) -> np.ndarray:
    """Per-row statistics of the columns [vocab_offset, vocab_offset + W) -> [n, 4].

    Fields: max m_c, sumexp S_c and sumexp_logit U_c about m_c, and target t_c,
    which is z_y when the label falls in this chunk, else 0.0 (NaN for a bad
    label, so the combine propagates it).
    """
    z = _as2d(z_chunk)
    n, width = z.shape
    if vocab_offset < 0 or vocab_offset + width > vocab:
        raise ValueError("chunk outside the vocabulary")
    m, S, U = row_statistics(z)
    labels = np.asarray(labels, dtype=np.int64)
    kind = label_kind(labels, vocab, ignore_index)
    local = labels - vocab_offset
    inside = (kind == 0) & (local >= 0) & (local < width)
    t = np.where(inside, z[np.arange(n), np.where(inside, local, 0)], 0.0)
    t = np.where(kind == 2, np.nan, t)
    return np.stack([m, S, t, U], axis=1)


def combine(stats: np.ndarray, labels: np.ndarray, vocab: int,
            ignore_index: int = IGNORE_INDEX):
    """Combine stats [C, n, 4] over chunks in ascending order -> (logprob, entropy, lse).

    M = max_c m_c; then for c = 0, 1, ...: a_c = exp(m_c - M),
    S += a_c S_c, U += a_c (U_c + (m_c - M) S_c), t += t_c.  A chunk with
    S_c == 0 (fully masked) contributes nothing.
    """
    stats = np.asarray(stats, dtype=np.float64)
    C, n, _ = stats.shape
    M = stats[:, :, 0].max(axis=0)
    S = np.zeros(n)
    U = np.zeros(n)
    t = np.zeros(n)
    for c in range(C):
        m_c, S_c, t_c, U_c = (stats[c, :, k] for k in range(4))
        live = S_c > 0
        with np.errstate(invalid="ignore"):
            gap = np.where(live, m_c - M, 0.0)
        a = np.where(live, np.exp(gap), 0.0)
        S = S + np.where(live, a * S_c, 0.0)
        U = U + np.where(live, a * (U_c + gap * S_c), 0.0)
        t = t + t_c
    kind = label_kind(labels, vocab, ignore_index)
    return finalize(M, S, U, t, kind)


# ---------------------------------------------------------------------------
# lm_head projection fused with the statistics ("ZeroSyncGRPOTrainer" PR:
# chunked lm_head over a replicated vocabulary projection; "[RL] Avoid
# full-vocab gather ...", Why: shard-local statistics)
# ---------------------------------------------------------------------------

def lmhead_logits(hidden: np.ndarray, weight: np.ndarray) -> np.ndarray:
    """logits [n, V] = hidden [n, d] @ weight[V, d]^T, exactly (float64 matmul)."""
    return np.asarray(hidden, dtype=np.float64) @ np.asarray(weight, dtype=np.float64).T


def lmhead_tile_stats(hidden, weight, labels, vocab_offset: int, vocab: int, tile: int,
                      ignore_index: int = IGNORE_INDEX) -> np.ndarray:
    """chunk_stats of each `tile`-row block of the lm_head rows -> [ceil(V_c / tile), n, 4]."""
    z = lmhead_logits(hidden, weight)
    vc = z.shape[1]
    return np.stack([chunk_stats(z[:, a:min(a + tile, vc)], labels, vocab_offset + a, vocab,
                                 ignore_index) for a in range(0, vc, tile)])


def lmhead_backward(hidden, weight, labels, lse, token_weights=None,
                    ignore_index: int = IGNORE_INDEX):
    """(G [n, V], grad_hidden [n, d], grad_weight [V, d]) in float64.

    G = w * (softmax - onehot) of the logits hidden @ weight^T from the given
    lse (the cross-entropy backward, as `backward`); the chain rule through the
    projection gives grad_hidden = G @ weight and grad_weight = G^T @ hidden
    (the chunked lm_head backward of "ZeroSyncGRPOTrainer", exact here).
    """
    h = np.asarray(hidden, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    g = backward(lmhead_logits(h, w), labels, lse, token_weights, ignore_index)
    return g, g @ w, g.T @ h


# ---------------------------------------------------------------------------
# several label columns per row, and trainer-vs-generator difference metrics
# ("[RL] Avoid full-vocab gather ...", Correctness and compatibility: the
#  generator's compute_logprobs(logits, labels) with multi-column token ids;
#  "torchtitan-batch-invarient-GDN", Code map and Result: the bit_wise
#  logprob_diff mean / abs_mean / max and ratio_tokens_different metrics)
# ---------------------------------------------------------------------------

def forward_multi(z: np.ndarray, labels: np.ndarray, ignore_index: int = IGNORE_INDEX):
    """logprob [n, K] = z[i, y_ik] - lse_i for every label column; plus entropy, lse."""
    z = _as2d(z)
    labels = np.asarray(labels, dtype=np.int64)
    n, v = z.shape
    m, S, U = row_statistics(z)
    kind = label_kind(labels, v, ignore_index)
    idx = np.where(kind == 0, labels, 0)
    t = np.take_along_axis(z, idx, axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        lse = m + np.log(S)
        entropy = np.log(S) - U / S
        lp = np.where(kind == 1, 0.0, t - lse[:, None])
    lp = np.where(kind == 2, np.nan, lp)
    return lp, entropy, lse


def diff_stats(a, b, labels=None, ignore_index: int = IGNORE_INDEX, a_bits=None, b_bits=None):
    """(mean, abs_mean, max_abs, ratio_different) of d = a - b over valid tokens.

    A token is valid unless its label is ignore_index.  ratio_different counts
    tokens whose values differ bit for bit (bit patterns passed as uint32, or
    compared as float32 values when not given).  No valid token gives zeros.
    """
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    valid = np.ones(a.shape, dtype=bool) if labels is None else \
        (np.asarray(labels, dtype=np.int64) != ignore_index)
    if not valid.any():
        return 0.0, 0.0, 0.0, 0.0
    d = (a - b)[valid]
    if a_bits is None:
        a_bits = np.asarray(a, dtype=np.float32).view(np.uint32)
        b_bits = np.asarray(b, dtype=np.float32).view(np.uint32)
    differ = (np.asarray(a_bits) != np.asarray(b_bits))[valid]
    return (float(d.sum() / d.size), float(np.abs(d).sum() / d.size),
            float(np.abs(d).max()), float(differ.sum() / d.size))


# ---------------------------------------------------------------------------
# clipped-ratio policy loss per token (the weight of the fused backward)
# ("torchtitan-batch-invarient-GDN", MATH recipe: DAPO with clip (0.2, 0.28);
#  "[RL] Avoid full-vocab gather ...", Summary: per-token gradients for
#  DAPO/GRPO losses)
# ---------------------------------------------------------------------------

def policy_terms(logprob, old_logprob, advantages, clip_low, clip_high, loss_scale=None,
                 ignored=None):
    """Per-token (loss, weight, clipped) of the clipped-ratio surrogate.

    r = exp(logprob - old_logprob); the surrogate is min(r A, clip(r, 1 - lo,
    1 + hi) A) and the token's loss is -c times it.  The weight is
    w = -d loss / d logprob = c A r where the unclipped term is the minimum
    (ties count as unclipped) and 0 where the clipped term is strictly
    smaller.  Ignored tokens have loss 0 and weight 0.
    """
    lp = np.asarray(logprob, dtype=np.float64)
    r = np.exp(lp - np.asarray(old_logprob, dtype=np.float64))
    A = np.asarray(advantages, dtype=np.float64)
    c = np.ones_like(lp) if loss_scale is None else np.asarray(loss_scale, dtype=np.float64)
    rc = np.minimum(np.maximum(r, 1.0 - clip_low), 1.0 + clip_high)
    unclipped = r * A <= rc * A
    loss = -c * np.where(unclipped, r * A, rc * A)
    w = np.where(unclipped, c * A * r, 0.0)
    if ignored is not None:
        ign = np.asarray(ignored, dtype=bool)
        loss = np.where(ign, 0.0, loss)
        w = np.where(ign, 0.0, w)
    return loss, w, ~unclipped


# ---------------------------------------------------------------------------
# brute force: 50-digit textbook softmax, different formula, tiny V only
# ---------------------------------------------------------------------------

def brute_force(z_row, label: int, weight: float = 1.0, ignore_index: int = IGNORE_INDEX,
                dps: int = 50):
    """(logprob, entropy, lse, grad list) of one row from p = e^z / sum e^z, mpmath.

    Entropy uses -sum p ln p over p > 0; no max shift is taken.  Meant for
    rows of at most a few dozen columns.
    """
    import mpmath as mp

    vals = [float(x) for x in z_row]
    with mp.workdps(dps):
        ex = [mp.e ** mp.mpf(x) if x != float("-inf") else mp.mpf(0) for x in vals]
        Z = mp.fsum(ex)
        p = [e / Z for e in ex]
        lse = mp.log(Z)
        ent = -mp.fsum(q * mp.log(q) for q in p if q > 0)
        v = len(vals)
        if label == ignore_index:
            logprob = mp.mpf(0)
            grad = [mp.mpf(0)] * v
        else:
            logprob = mp.log(p[label])
            w = mp.mpf(weight)
            grad = [w * (p[j] - (1 if j == label else 0)) for j in range(v)]
        return (float(logprob), float(ent), float(lse), [float(g) for g in grad])


# ---------------------------------------------------------------------------
# convenience wrappers over workload batches (row blocks bound the memory)
# ---------------------------------------------------------------------------

def forward_batch(logits, labels, dtype: str, ignore_index: int = IGNORE_INDEX,
                  block: int = 64):
    n = len(labels)
    out = np.empty((3, n))
    for a in range(0, n, block):
        z = decode(logits[a:a + block], dtype)
        out[:, a:a + block] = forward(z, labels[a:a + block], ignore_index)
    return out[0], out[1], out[2]


def backward_rows(logits, labels, lse, weights, dtype: str,
                  ignore_index: int = IGNORE_INDEX) -> np.ndarray:
    z = decode(logits, dtype)
    return backward(z, labels, lse, weights, ignore_index)
