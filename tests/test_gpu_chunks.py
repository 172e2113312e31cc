"""GPU parity of the vocabulary-chunk path (bi_vocab_chunk_stats +
bi_stats_combine) on the cases of the vocabulary-parallel parity matrix in
"[RL] Avoid full-vocab gather for TP policy statistics" (torchtitan PR #4685),
Correctness and compatibility: FP32 and BF16 logits, uneven vocabulary and
chunks, ignored labels and partially masked logits; plus a chunk whose columns
are all masked and labels outside the vocabulary.

Every per-chunk statistic is compared with the oracle's ``chunk_stats`` row by
row (the max and the target bit for bit: both are plain fp32 values of the
input; the two sums within a relative 2e-5), and the combined logprob, entropy
and lse with the oracle's ``combine`` and with its full-row ``forward``, at the
tolerances of the full-row path (fp32 logits 2e-4, bf16 5e-3).  The combine
takes chunks in ascending order (review reply "Batch invariance under the
patched logprob path", Q2), so a fully masked chunk must leave every combined
bit unchanged wherever it sits.
"""
import numpy as np
import pytest
import torch

import entropy_bi_logprob_amd as bi
import oracle.bi_oracle as orc
import workloads as wl
from gpu_util import TOL, assert_close, dev, dev_logits, host
from workloads import f32_to_bf16_bits, random_batch

pytestmark = pytest.mark.gpu
STATS = bi.STATS_FIELDS


def gpu_chunks(logits, labels, bounds, vocab, flag=None, ignore_index=-100):
    """[C, N, 4] statistics and the combined (logprob, entropy, lse), on the device."""
    st = torch.empty((len(bounds), logits.shape[0], 4), dtype=torch.float32, device="cuda")
    for c, (a, e) in enumerate(bounds):
        bi.vocab_chunk_stats(logits[:, a:e], labels, a, vocab, ignore_index, out=st[c],
                             status=flag)
    return st, bi.stats_combine(st, labels, ignore_index)


def check_stats(st, z, labels, bounds, vocab, rows=None):
    """Per-chunk statistics of the given rows against the oracle."""
    rows = np.arange(z.shape[0]) if rows is None else rows
    ost = np.stack([orc.chunk_stats(z[:, a:e], labels, a, vocab) for a, e in bounds])
    got = st[:, rows]
    np.testing.assert_array_equal(got[:, :, 0], ost[:, :, 0])           # max: exact
    np.testing.assert_array_equal(got[:, :, 2], ost[:, :, 2])           # target: exact (or NaN)
    np.testing.assert_allclose(got[:, :, 1], ost[:, :, 1], rtol=2e-5, atol=0)
    np.testing.assert_allclose(got[:, :, 3], ost[:, :, 3], rtol=2e-5, atol=1e-3)
    return ost


def check_combined(outs, ost, z, labels, vocab, dtype):
    tl, te, _ = TOL[dtype]
    lp, ent, lse = outs
    clp, cent, clse = orc.combine(ost, labels, vocab)
    flp, fent, flse = orc.forward(z, labels)
    for what, want in (("combine", (clp, cent, clse)), ("full row", (flp, fent, flse))):
        assert_close(lp, want[0], tl, f"logprob vs oracle {what}")
        assert_close(ent, want[1], te, f"entropy vs oracle {what}")
        assert_close(lse, want[2], tl, f"lse vs oracle {what}")
    ign = labels == -100
    assert np.all(lp[ign] == 0) and not np.any(np.signbit(lp[ign])), "ignored logprob not +0.0"


def test_masked_fp32_uneven_chunks_at_full_size():
    # the masked 2,048 x 151,937 fp32 workload: 15,193 -inf columns per row, an
    # odd width (rows 4 mod 16 bytes apart) and four uneven chunks starting at
    # columns 1 mod 4, so chunk starts fall on every 4-byte phase of 16 across
    # rows; all rows on the device, sampled rows against the oracle
    w = wl.WORKLOADS[3]
    b = wl.draw(3)
    labels = b.labels.copy()
    labels[[3, 17, 1500]] = -100                     # a few ignored rows as well
    V = w.vocab
    bounds = [(0, 37_001), (37_001, 75_001), (75_001, 113_997), (113_997, V)]
    assert all((a * 4) % 16 == 4 for a, _ in bounds[1:])
    logits, dlab = dev_logits(b.logits, "f32"), dev(labels)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    st, outs = gpu_chunks(logits, dlab, bounds, V, flag)
    flp, fent, flse = bi.fwd(logits, dlab)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    st = host(st)
    outs = tuple(host(t) for t in outs)
    # every row: the chunked path against the full-row path
    for k, full in enumerate((flp, fent, flse)):
        assert_close(outs[k], host(full), 1e-4, "chunked vs full row")
    rows = np.array(sorted({0, 3, 17, 1500, 2047} | set(
        np.random.default_rng(31).choice(2048, 40, replace=False).tolist())))
    z = orc.decode(b.logits[rows], "f32")
    ost = check_stats(st, z, labels[rows], bounds, V, rows)
    check_combined(tuple(o[rows] for o in outs), ost, z, labels[rows], V, "f32")


def test_masked_bf16_odd_chunk_starts():
    # bf16 rows of an odd width (every other row starts on a 2-byte boundary),
    # 10% masked columns, chunks starting at odd columns, one of them a single
    # column that holds row 0's label
    V, n = 50_001, 24
    b = random_batch(n, V, "bf16", seed=505, ignore_frac=0.1, mask_frac=0.1)
    labels = b.labels.copy()
    labels[0] = 9_999
    b.logits[0, 9_999] = f32_to_bf16_bits(np.array([1.5], dtype=np.float32))[0]
    bounds = [(0, 9_999), (9_999, 10_000), (10_000, 31_113), (31_113, V)]
    logits, dlab = dev_logits(b.logits, "bf16"), dev(labels)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    st, outs = gpu_chunks(logits, dlab, bounds, V, flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    st = host(st)
    z = orc.decode(b.logits, "bf16")
    ost = check_stats(st, z, labels, bounds, V)
    assert st[1, 0, 2] == np.float32(1.5)            # the one-column chunk holds the label
    check_combined(tuple(host(t) for t in outs), ost, z, labels, V, "bf16")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fully_masked_chunk_is_a_no_op(dtype):
    # columns [5,000, 9,000) are -inf in every row.  That chunk's statistics are
    # (-inf, 0, 0, 0) (its target is 0: no label lies in it, and ignored rows
    # have none); combined with live chunks before, between or after it, every
    # output equals the combine without it, bit for bit, and the oracle
    V, n = 20_000, 16
    b = random_batch(n, V, dtype, seed=606, ignore_frac=0.2, mask_frac=0.05)
    x = orc.decode(b.logits, dtype).astype(np.float32)
    labels = b.labels.copy()
    live = labels != -100
    labels[live] = labels[live] % 5_000               # never inside the masked chunk
    x[np.nonzero(live)[0], labels[live]] = np.float32(0.25)   # and never on a masked column
    x[:, 5_000:9_000] = -np.inf
    b.logits = f32_to_bf16_bits(x) if dtype == "bf16" else x
    logits, dlab = dev_logits(b.logits, dtype), dev(labels)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    bounds = [(0, 5_000), (5_000, 9_000), (9_000, V)]
    st, outs = gpu_chunks(logits, dlab, bounds, V, flag)
    alone = bi.vocab_chunk_stats(logits[:, 5_000:9_000], dlab, 5_000, V)
    live_only = st[[0, 2]].contiguous()
    ref = bi.stats_combine(live_only, dlab)
    orders = {
        "first": torch.stack([st[1], st[0], st[2]]),
        "middle": st,
        "last": torch.stack([st[0], st[2], st[1]]),
        "twice": torch.stack([st[1], st[0], st[1], st[2], st[1]]),
    }
    combos = {k: bi.stats_combine(v.contiguous(), dlab) for k, v in orders.items()}
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    for s in (host(st)[1], host(alone)):
        assert np.all(np.isneginf(s[:, 0])), "max of a fully masked chunk"
        for k in (1, 2, 3):
            assert np.all(s[:, k] == 0) and not np.any(np.signbit(s[:, k])), STATS[k]
    i32 = torch.int32
    for k, outs_k in combos.items():
        for a, c in zip(outs_k, ref):
            assert torch.equal(a.view(i32), c.view(i32)), f"masked chunk {k} changed a bit"
    z = orc.decode(b.logits, dtype)
    ost = check_stats(host(st), z, labels, bounds, V)
    check_combined(tuple(host(t) for t in outs), ost, z, labels, V, dtype)



@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bad_labels_through_chunks(dtype):
    # labels outside [0, V) that are not ignore_index: NaN target in every chunk,
    # NaN combined logprob, the status flag raised by the chunk call; entropy and
    # lse of those rows, and every other row, unaffected
    V, n = 30_011, 20
    b = random_batch(n, V, dtype, seed=707, ignore_frac=0.1, mask_frac=0.05)
    labels = b.labels.copy()
    bad = [2, 5, 9]
    labels[bad] = [V + 7, -3, V]
    bounds = [(0, 7_777), (7_777, 21_000), (21_000, V)]
    logits, dlab = dev_logits(b.logits, dtype), dev(labels)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    st, outs = gpu_chunks(logits, dlab, bounds, V, flag)
    good = torch.tensor(np.delete(np.arange(n), bad), device="cuda")
    flag2 = torch.zeros(1, dtype=torch.int32, device="cuda")
    gpu_chunks(logits[good].contiguous(), dlab[good].contiguous(), bounds, V, flag2)
    torch.cuda.synchronize()
    assert int(flag.item()) == bi.BI_FLAG_BAD_LABEL
    assert int(flag2.item()) == 0
    st = host(st)
    assert np.all(np.isnan(st[:, bad, 2])), "bad label: target NaN in every chunk"
    z = orc.decode(b.logits, dtype)
    ost = check_stats(st, z, labels, bounds, V)
    lp, ent, lse = (host(t) for t in outs)
    assert np.all(np.isnan(lp[bad]))
    tl, te, _ = TOL[dtype]
    clp, cent, clse = orc.combine(ost, labels, V)
    assert_close(lp, clp, tl, "logprob")            # NaN pattern included
    assert_close(ent, cent, te, "entropy")
    assert_close(lse, clse, tl, "lse")
    assert np.all(np.isfinite(ent[bad])) and np.all(np.isfinite(lse[bad]))
