"""GPU parity and batch invariance on the full-size synthetic workloads.

 * fwd_256x151936_f32: forward only; every row against the oracle.
 * fwdbwd_4096x151936_bf16: forward on every row against the oracle; fp32 and
   bf16 gradients on sampled rows; bf16 == RNE(fp32) on every element.
 * masked_2048x151937_f32: odd width (rows 4 mod 16 bytes apart), 10% -inf
   columns per row; forward on every row, gradients on sampled rows.
 * invariance_bf16: 16 fixed rows inside batches of 1, 16, 512 and 8,192 rows;
   logprob, entropy, lse and gradient rows must be bit-identical across all of
   them, across repeated runs, and when a batch is split into two calls.
 * large_32768x151936_bf16: the headline shape, in the launch configuration the
   benchmark times; sampled rows against the oracle, and the 4-chunk path
   (bi_vocab_chunk_stats x 4 + bi_stats_combine) against the full-row path:
   the chunk maxima bit-exact, everything else within tolerance.

Tolerances (|delta| against fp64): fp32 logits 2e-4 / 2e-4 / 1e-5 (logprob /
entropy / grad), bf16 logits 5e-3 / 5e-3 / 1e-3.
"""
import gc

import numpy as np
import pytest
import torch

import entropy_bi_logprob_amd as bi
import oracle.bi_oracle as orc
import workloads as wl
from gpu_util import TOL, assert_close, dev, dev_logits, host, oracle_forward, ulp_bf16

pytestmark = pytest.mark.gpu


def sample_rows(n, k, seed=7):
    g = np.random.default_rng([seed, n])
    rows = set(g.choice(n, size=min(k, n), replace=False).tolist()) | {0, n - 1}
    return np.array(sorted(rows))


def check_grads(b, rows, g32_rows, gb16_rows=None):
    # the oracle's gradient from its own lse, against the GPU's end to end
    tg = TOL[b.dtype][2]
    z = orc.decode(b.logits[rows], b.dtype)
    _, _, olse = orc.forward(z, b.labels[rows])
    w = None if b.weights is None else b.weights[rows]
    og = orc.backward(z, b.labels[rows], olse, w)
    assert_close(g32_rows, og, tg, "grad")
    if gb16_rows is not None:
        gbv = orc.decode(gb16_rows, "bf16")
        assert np.all(np.abs(gbv - og) <= tg + 0.5 * ulp_bf16(og)), "bf16 grad bound"


def test_fwd_256_f32_all_rows():
    b = wl.draw(1)
    lp, ent, lse = (host(t) for t in bi.fwd(dev_logits(b.logits, "f32"), dev(b.labels)))
    olp, oent, olse = oracle_forward(b.logits, b.labels, "f32")
    tl, te, _ = TOL["f32"]
    print("max |d| logprob %.3g entropy %.3g lse %.3g" % (
        assert_close(lp, olp, tl, "logprob"), assert_close(ent, oent, te, "entropy"),
        assert_close(lse, olse, tl, "lse")))
    ign = b.labels == -100
    assert ign.sum() == 13 and np.all(lp[ign] == 0) and not np.any(np.signbit(lp[ign]))


def test_fwdbwd_4096_bf16():
    b = wl.draw(2)
    logits, labels, w = dev_logits(b.logits, "bf16"), dev(b.labels), dev(b.weights)
    lp, ent, lse = bi.fwd(logits, labels)
    g16 = bi.bwd(logits, labels, lse, w, torch.bfloat16)
    g32 = bi.bwd(logits, labels, lse, w, torch.float32)
    torch.cuda.synchronize()
    # bf16 gradient == fp32 gradient rounded to nearest even, every element
    assert torch.equal(g16.view(torch.int16), g32.to(torch.bfloat16).view(torch.int16))
    ign = torch.from_numpy(b.labels == -100).cuda()
    assert int((g32[ign] != 0).sum()) == 0 and int(torch.signbit(g32[ign]).sum()) == 0
    olp, oent, olse = oracle_forward(b.logits, b.labels, "bf16")
    tl, te, _ = TOL["bf16"]
    assert_close(host(lp), olp, tl, "logprob")
    assert_close(host(ent), oent, te, "entropy")
    rows = sample_rows(4096, 48)
    ridx = torch.from_numpy(rows).cuda()
    check_grads(b, rows, host(g32[ridx]), host(g16[ridx]))


def test_masked_2048_f32_odd_width():
    b = wl.draw(3)
    logits, labels = dev_logits(b.logits, "f32"), dev(b.labels)
    lp, ent, lse = bi.fwd(logits, labels)
    olp, oent, olse = oracle_forward(b.logits, b.labels, "f32")
    tl, te, _ = TOL["f32"]
    assert_close(host(lp), olp, tl, "logprob")
    assert_close(host(ent), oent, te, "entropy")
    assert_close(host(lse), olse, tl, "lse")
    g = bi.bwd(logits, labels, lse, None, torch.float32)
    torch.cuda.synchronize()
    masked = torch.isneginf(logits)
    assert int((g[masked] != 0).sum()) == 0
    rows = sample_rows(2048, 32)
    check_grads(b, rows, host(g[torch.from_numpy(rows).cuda()]))


# ------------------------------------------------------------ batch invariance

def _run_rows(batch, fused=False):
    logits, labels, w = dev_logits(batch.logits, "bf16"), dev(batch.labels), dev(batch.weights)
    if fused:
        lp, ent, lse, g = bi.fwd_bwd(logits, labels, w, torch.bfloat16)
    else:
        lp, ent, lse = bi.fwd(logits, labels)
        g = bi.bwd(logits, labels, lse, w, torch.bfloat16)
    gf = bi.bwd(logits, labels, lse, w, torch.float32)
    return logits, labels, w, lp, ent, lse, g, gf


@pytest.mark.parametrize("fused", [False, True], ids=["two_calls", "fused"])
def test_batch_invariance_sweep(fused):
    per_n = {}
    for n, cases in wl.invariance_batches():
        outs = []
        for case in cases:
            _, _, _, lp, ent, lse, g, gf = _run_rows(case.batch, fused)
            pos = torch.from_numpy(case.positions).cuda()
            outs.append((lp[pos], ent[pos], lse[pos], g[pos], gf[pos]))
        torch.cuda.synchronize()
        per_n[n] = [torch.cat([o[k] for o in outs]) for k in range(5)]
        del outs
    ref = per_n[1]
    for n, got in per_n.items():
        for k, name in enumerate(("logprob", "entropy", "lse", "grad_bf16", "grad_f32")):
            a = ref[k].view(torch.int32 if ref[k].dtype == torch.float32 else torch.int16)
            c = got[k].view(a.dtype)
            assert torch.equal(a, c), f"{name} differs between N=1 and N={n}"
    # and the 16 rows agree with the oracle
    core = wl.draw(4)
    olp, oent, olse = orc.forward(orc.decode(core.logits, "bf16"), core.labels)
    tl, te, _ = TOL["bf16"]
    assert_close(host(ref[0]), olp, tl, "logprob")
    assert_close(host(ref[1]), oent, te, "entropy")
    check_grads(core, np.arange(16), host(ref[4]), host(ref[3]))


def test_chunk_and_multi_paths_are_batch_invariant():
    # the 16 fixed rows: chunk statistics, combined outputs and multi-column
    # logprobs must not depend on the batch either
    V = wl.WORKLOADS[4].vocab
    bounds = wl.chunk_bounds(V, wl.LARGE_CHUNKS)
    per_n = {}
    for n, cases in wl.invariance_batches():
        outs = []
        for case in cases:
            logits = dev_logits(case.batch.logits, "bf16")
            labels = dev(case.batch.labels)
            st = torch.empty((len(bounds), case.batch.rows, 4), device="cuda")
            for c, (a, e) in enumerate(bounds):
                bi.vocab_chunk_stats(logits[:, a:e], labels, a, V, out=st[c])
            clp, cent, clse = bi.stats_combine(st, labels)
            ids = torch.stack([labels, torch.zeros_like(labels), labels.flip(0)], dim=1)
            mlp, _, _ = bi.fwd_multi(logits, ids.contiguous())
            pos = torch.from_numpy(case.positions).cuda()
            # statistics row-major ([row, chunk, 4]) so that cases concatenate in row order
            outs.append((st[:, pos].transpose(0, 1).reshape(-1), clp[pos], cent[pos], clse[pos],
                         mlp[pos, :2].reshape(-1)))
        torch.cuda.synchronize()
        per_n[n] = [torch.cat([o[k] for o in outs]) for k in range(5)]
    ref = per_n[1]
    for n, got in per_n.items():
        for k in range(5):
            assert torch.equal(ref[k].view(torch.int32), got[k].view(torch.int32)), (n, k)


def test_repeat_and_split_invariance():
    b = wl.draw(2, rows=np.arange(1024))
    logits, labels, w, lp, ent, lse, g, _ = _run_rows(b)
    # the same call again
    lp2, ent2, lse2 = bi.fwd(logits, labels)
    g2 = bi.bwd(logits, labels, lse2, w, torch.bfloat16)
    # the rows in two calls (token-chunked), split at an odd point
    k = 397
    lpa, enta, lsea = bi.fwd(logits[:k], labels[:k])
    lpb, entb, lseb = bi.fwd(logits[k:], labels[k:])
    ga = bi.bwd(logits[:k], labels[:k], lsea, w[:k], torch.bfloat16)
    gb = bi.bwd(logits[k:], labels[k:], lseb, w[k:], torch.bfloat16)
    # reversed row order
    rev = torch.arange(1023, -1, -1, device="cuda")
    lpr, entr, lser = bi.fwd(logits[rev].contiguous(), labels[rev].contiguous())
    torch.cuda.synchronize()
    i32 = torch.int32
    for a, c in ((lp, lp2), (ent, ent2), (lse, lse2), (lp, torch.cat([lpa, lpb])),
                 (ent, torch.cat([enta, entb])), (lse, torch.cat([lsea, lseb])),
                 (lp, lpr[rev]), (ent, entr[rev]), (lse, lser[rev])):
        assert torch.equal(a.view(i32), c.view(i32))
    assert torch.equal(g.view(torch.int16), g2.view(torch.int16))
    assert torch.equal(g.view(torch.int16), torch.cat([ga, gb]).view(torch.int16))


# ------------------------------------------------------- large (headline shape)

@pytest.fixture(scope="module")
def large():
    b = wl.draw(5)
    t = dict(b=b, logits=dev_logits(b.logits, "bf16"), labels=dev(b.labels), w=dev(b.weights))
    yield t
    t.clear()
    gc.collect()
    torch.cuda.empty_cache()


def test_large_fwd_bwd_sampled_rows(large):
    b = large["b"]
    logits, labels, w = large["logits"], large["labels"], large["w"]
    lp, ent, lse = bi.fwd(logits, labels)
    g16 = bi.bwd(logits, labels, lse, w, torch.bfloat16)
    rows = sample_rows(b.rows, 192)
    ridx = torch.from_numpy(rows).cuda()
    # fp32 gradients of the sampled rows from a call over just those rows
    # (bit-identical to the full call, by batch invariance)
    sub = logits[ridx].contiguous()
    g32 = bi.bwd(sub, labels[ridx].contiguous(), lse[ridx].contiguous(), w[ridx].contiguous(),
                 torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(g16[ridx].view(torch.int16), g32.to(torch.bfloat16).view(torch.int16))
    z = orc.decode(b.logits[rows], "bf16")
    olp, oent, olse = orc.forward(z, b.labels[rows])
    tl, te, _ = TOL["bf16"]
    assert_close(host(lp)[rows], olp, tl, "logprob")
    assert_close(host(ent)[rows], oent, te, "entropy")
    assert_close(host(lse)[rows], olse, tl, "lse")
    check_grads(b, rows, host(g32), host(g16[ridx]))
    assert np.all(np.isfinite(host(lp))) and np.all(np.isfinite(host(ent)))


def test_large_fused_equals_two_calls(large):
    logits, labels, w = large["logits"], large["labels"], large["w"]
    lp, ent, lse = bi.fwd(logits, labels)
    g = bi.bwd(logits, labels, lse, w, torch.bfloat16)
    flp, fent, flse, fg = bi.fwd_bwd(logits, labels, w, torch.bfloat16)
    torch.cuda.synchronize()
    for a, c in ((lp, flp), (ent, fent), (lse, flse)):
        assert torch.equal(a.view(torch.int32), c.view(torch.int32))
    assert torch.equal(g.view(torch.int16), fg.view(torch.int16))
    del g, fg


def test_large_policy_loss_matches_two_calls(large):
    b = large["b"]
    logits, labels = large["logits"], large["labels"]
    g = np.random.default_rng([b.rows, 17])
    old = torch.from_numpy(g.normal(-11.0, 1.5, b.rows).astype(np.float32)).cuda()
    adv = torch.from_numpy(g.standard_normal(b.rows).astype(np.float32)).cuda()
    lp, ent, lse, loss, w, grad = bi.policy_loss_fwd_bwd(logits, labels, old, adv, 0.2, 0.28)
    lp2, ent2, lse2 = bi.fwd(logits, labels)
    g2 = bi.bwd(logits, labels, lse2, w, torch.bfloat16)
    torch.cuda.synchronize()
    for a, c in ((lp, lp2), (ent, ent2), (lse, lse2)):
        assert torch.equal(a.view(torch.int32), c.view(torch.int32))
    assert torch.equal(grad.view(torch.int16), g2.view(torch.int16))
    # sampled rows: weight and loss against the oracle
    rows = sample_rows(b.rows, 64, seed=9)
    olp, _, _ = orc.forward(orc.decode(b.logits[rows], "bf16"), b.labels[rows])
    oldh, advh = host(old)[rows], host(adv)[rows]
    oloss, ow, _ = orc.policy_terms(olp, oldh, advh, 0.2, 0.28)
    r = np.exp(olp - oldh)
    sure = (np.abs(r - 0.8) > 1e-4 * r) & (np.abs(r - 1.28) > 1e-4 * r)
    wr, lr = host(w)[rows], host(loss)[rows]
    assert np.all(np.abs(wr - ow)[sure] <= 1e-5 * np.maximum(1.0, np.abs(ow[sure])))
    assert np.all(np.abs(lr - oloss)[sure] <= 1e-5 * np.maximum(1.0, np.abs(oloss[sure])))
    del grad, g2


def test_large_chunked_path_equals_full_rows(large):
    b = large["b"]
    logits, labels = large["logits"], large["labels"]
    V = b.vocab
    bounds = wl.chunk_bounds(V, wl.LARGE_CHUNKS)
    assert [e - a for a, e in bounds] == [37_984] * 4
    stats = torch.empty((len(bounds), b.rows, 4), dtype=torch.float32, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    for c, (a, e) in enumerate(bounds):
        bi.vocab_chunk_stats(logits[:, a:e], labels, a, V, out=stats[c], status=flag)
    clp, cent, clse = bi.stats_combine(stats, labels)
    lp, ent, lse = bi.fwd(logits, labels)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    tl, te, _ = TOL["bf16"]
    d_lp = assert_close(host(clp), host(lp), 1e-4, "chunked logprob vs full")
    d_ent = assert_close(host(cent), host(ent), 1e-4, "chunked entropy vs full")
    d_lse = assert_close(host(clse), host(lse), 1e-4, "chunked lse vs full")
    print("chunked vs full max |d|: logprob %.3g entropy %.3g lse %.3g" % (d_lp, d_ent, d_lse))
    # per-chunk statistics against the oracle on sampled rows; the max is exact
    rows = sample_rows(b.rows, 64, seed=3)
    st = host(stats)[:, rows]
    z = orc.decode(b.logits[rows], "bf16")
    ost = np.stack([orc.chunk_stats(z[:, a:e], b.labels[rows], a, V) for a, e in bounds])
    np.testing.assert_array_equal(st[:, :, 0], ost[:, :, 0])
    np.testing.assert_allclose(st[:, :, 1], ost[:, :, 1], rtol=2e-5)
    np.testing.assert_array_equal(st[:, :, 2], ost[:, :, 2])
    np.testing.assert_allclose(st[:, :, 3], ost[:, :, 3], rtol=2e-5, atol=1e-3)
    olp, oent, olse = orc.combine(ost, b.labels[rows], V)
    assert_close(host(clp)[rows], olp, tl, "combined logprob")
    assert_close(host(cent)[rows], oent, te, "combined entropy")
