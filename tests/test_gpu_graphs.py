"""The kernels under HIP-graph capture.

Each path is captured once into a torch CUDAGraph (HIP graph) with its outputs
preallocated, then replayed several times with other eager work and
synchronisations between the replays; every replay must reproduce the eager
call bit for bit.  The library allocates nothing and issues no memset, so
every one of its launches is a plain kernel node.  Inputs are the seeded
synthetic batches of the other tests.
"""
import numpy as np
import pytest
import torch

import entropy_bi_logprob_amd as bi
import workloads as wl
from gpu_util import dev, dev_logits

pytestmark = pytest.mark.gpu
REPLAYS = 3


def same(a: torch.Tensor, b: torch.Tensor) -> bool:
    view = torch.int16 if a.element_size() == 2 else torch.int32
    return bool(torch.equal(a.contiguous().view(view), b.contiguous().view(view)))


def capture(fn):
    """Warm up on a side stream, then capture fn() into a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def replay_and_check(g, outs, refs, other_work):
    for r in range(REPLAYS):
        for o in outs:
            o.fill_(float("nan") if o.is_floating_point() else 0)
        other_work(r)                 # eager kernels of our own between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, ref in zip(outs, refs):
            assert same(o, ref), f"replay {r} differs from the eager call"


def test_fused_fwd_bwd_replays():
    b = wl.random_batch(700, 50_000, "bf16", seed=41, ignore_frac=0.05)
    z, y, w = dev_logits(b.logits, "bf16"), dev(b.labels), dev(b.weights)
    lp, ent, lse = (torch.empty(700, device="cuda") for _ in range(3))
    grad = torch.empty_like(z)
    ref = [t.clone() for t in bi.fwd_bwd(z, y, w)]
    o = wl.random_batch(300, 50_000, "bf16", seed=42)
    oz, oy = dev_logits(o.logits, "bf16"), dev(o.labels)

    g = capture(lambda: bi.fwd_bwd(z, y, w, out=(lp, ent, lse), grad=grad))
    replay_and_check(g, (lp, ent, lse, grad), ref, lambda r: bi.fwd(oz, oy))


def test_fused_row_on_chip_and_policy_replay():
    # the Qwen3 width in bf16: the kernel that keeps each row on chip, plain
    # and with the clipped-ratio weights derived in it; 300 rows, so some
    # workgroups walk a second row
    n, v = 300, 151_936
    b = wl.random_batch(n, v, "bf16", seed=45, ignore_frac=0.05, mask_frac=0.01)
    z, y, w = dev_logits(b.logits, "bf16"), dev(b.labels), dev(b.weights)
    gen = np.random.default_rng(46)
    old = dev(gen.normal(-12.0, 1.0, n).astype(np.float32))
    adv = dev(gen.standard_normal(n).astype(np.float32))
    lp, ent, lse = (torch.empty(n, device="cuda") for _ in range(3))
    grad = torch.empty_like(z)
    plp, pent, plse, ploss, pw = (torch.empty(n, device="cuda") for _ in range(5))
    pgrad = torch.empty((n, v), dtype=torch.float32, device="cuda")

    def step():
        bi.fwd_bwd(z, y, w, out=(lp, ent, lse), grad=grad)
        bi.policy_loss_fwd_bwd(z, y, old, adv, 0.2, 0.28, grad=pgrad)

    ref_fused = [t.clone() for t in bi.fwd_bwd(z, y, w)]
    ref_policy = [t.clone() for t in bi.policy_loss_fwd_bwd(z, y, old, adv, 0.2, 0.28,
                                                             grad_dtype=torch.float32)]
    torch.cuda.synchronize()
    g = capture(step)
    o = wl.random_batch(64, v, "bf16", seed=47)
    oz, oy = dev_logits(o.logits, "bf16"), dev(o.labels)
    replay_and_check(g, (lp, ent, lse, grad, pgrad), ref_fused + [ref_policy[5]],
                     lambda r: bi.fwd_bwd(oz, oy))


def test_two_calls_and_chunked_path_replay():
    n, v = 513, 40_001
    b = wl.random_batch(n, v, "f32", seed=43, ignore_frac=0.05, mask_frac=0.05)
    z, y, w = dev_logits(b.logits, "f32"), dev(b.labels), dev(b.weights)
    bounds = wl.chunk_bounds(v, 3)
    stats = torch.empty((len(bounds), n, 4), device="cuda")
    lp, ent, lse = (torch.empty(n, device="cuda") for _ in range(3))
    lp2, ent2, lse2 = (torch.empty(n, device="cuda") for _ in range(3))
    grad = torch.empty((n, v), dtype=torch.float32, device="cuda")

    def step():
        bi.fwd(z, y, out=(lp, ent, lse))
        bi.bwd(z, y, lse, w, out=grad)
        for c, (lo, hi) in enumerate(bounds):
            bi.vocab_chunk_stats(z[:, lo:hi], y, lo, v, out=stats[c])
        bi.stats_combine(stats, y, out=(lp2, ent2, lse2))

    step()
    torch.cuda.synchronize()
    outs = (lp, ent, lse, grad, stats, lp2, ent2, lse2)
    ref = [t.clone() for t in outs]
    g = capture(step)
    replay_and_check(g, outs, ref, lambda r: bi.fwd_bwd(z[:64].contiguous(), y[:64], w[:64]))


def test_lmhead_statistics_replay():
    n, vc, d = 600, 3000, 256
    b = wl.lmhead_batch(n, vc, d, seed=44, ignore_frac=0.05)
    to_bf16 = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda() \
        .view(torch.bfloat16)
    H, W, y = to_bf16(b.hidden), to_bf16(b.weight), dev(b.labels)
    st = torch.empty((bi.lib().bi_lmhead_tiles(vc), n, 4), device="cuda")
    lp, ent, lse = (torch.empty(n, device="cuda") for _ in range(3))

    def step():
        bi.lmhead_tile_stats(H, W, y, out=st)
        bi.stats_combine(st, y, out=(lp, ent, lse))

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (st, lp, ent, lse)]
    g = capture(step)
    replay_and_check(g, (st, lp, ent, lse), ref,
                     lambda r: bi.lmhead_logprob(H[:100], W, y[:100]))


def test_lmhead_backward_replays():
    # grad-logits kernel plus two matrix-core products per vocabulary chunk;
    # the workspace and the outputs are the caller's, so the graph owns nothing
    n, vc, d, chunk = 300, 1000, 128, 256   # 300 tokens: G padded to 320 columns
    b = wl.lmhead_batch(n, vc, d, seed=45, ignore_frac=0.05)
    to_bf16 = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda() \
        .view(torch.bfloat16)
    H, W, y = to_bf16(b.hidden), to_bf16(b.weight), dev(b.labels)
    _, _, lse = bi.lmhead_logprob(H, W, y)
    tw = torch.linspace(-1.0, 1.0, n, device="cuda")
    ws = torch.empty(int(bi.lib().bi_lmhead_backward_workspace(n, d, chunk)), dtype=torch.uint8,
                     device="cuda")
    gh = torch.zeros((n, d), device="cuda")
    gw = torch.empty((vc, d), dtype=torch.bfloat16, device="cuda")

    def step():
        gh.zero_()   # a fill kernel (grad_hidden is accumulated into)
        bi.lmhead_backward(H, W, y, lse, tw, grad_hidden=gh, grad_weight=gw, chunk_rows=chunk,
                           workspace=ws)

    step()
    torch.cuda.synchronize()
    ref = [gh.clone(), gw.clone()]
    g = capture(step)
    replay_and_check(g, (gh, gw), ref, lambda r: bi.lmhead_logprob(H, W, y))
