"""Concurrent use: two host threads, each on its own stream, call the library
at the same time (the row kernels, among them the fused kernel that keeps each
row on chip, the lm_head statistics and the lm_head backward) on different
inputs; every result must equal the one computed alone on the default stream,
bit for bit."""
import threading

import numpy as np
import pytest
import torch

import entropy_bi_logprob_amd as bi
import workloads as wl
from gpu_util import dev, dev_logits

pytestmark = pytest.mark.gpu
REPEATS = 4


def to_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def make_case(seed):
    b = wl.random_batch(400, 30_000, "bf16", seed=seed, ignore_frac=0.05)
    h = wl.lmhead_batch(300, 1500, 128, seed=seed + 1, ignore_frac=0.05)
    q = wl.random_batch(300, 151_936, "bf16", seed=seed + 2, ignore_frac=0.05)   # rows on chip
    return {"z": dev_logits(b.logits, "bf16"), "y": dev(b.labels), "w": dev(b.weights),
            "zq": dev_logits(q.logits, "bf16"), "yq": dev(q.labels), "wq": dev(q.weights),
            "H": to_bf16(h.hidden), "W": to_bf16(h.weight), "hy": dev(h.labels),
            "tw": torch.linspace(-1.0, 1.0, 300, device="cuda")}


def run(case):
    lp, ent, lse, grad = bi.fwd_bwd(case["z"], case["y"], case["w"])
    hlp, hent, hlse = bi.lmhead_logprob(case["H"], case["W"], case["hy"])
    gh, gw = bi.lmhead_backward(case["H"], case["W"], case["hy"], hlse, case["tw"], chunk_rows=512)
    qlp, qent, qlse, qgrad = bi.fwd_bwd(case["zq"], case["yq"], case["wq"])
    return [lp, ent, lse, grad, hlp, hent, hlse, gh, gw, qlp, qent, qlse, qgrad]


def same(a, b):
    view = torch.int16 if a.element_size() == 2 else torch.int32
    return bool(torch.equal(a.view(view), b.view(view)))


def test_two_threads_two_streams():
    cases = [make_case(61), make_case(71)]
    refs = [run(c) for c in cases]
    torch.cuda.synchronize()
    errors = []
    barrier = threading.Barrier(len(cases))

    def worker(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                barrier.wait(timeout=60)
                for r in range(REPEATS):
                    outs = run(cases[i])
                    s.synchronize()
                    for k, (o, ref) in enumerate(zip(outs, refs[i])):
                        if not same(o, ref):
                            errors.append(f"thread {i}, repeat {r}, output {k} differs")
        except Exception as e:  # reported below, with the thread that raised it
            errors.append(f"thread {i}: {e!r}")

    threads = [threading.Thread(target=worker, args=(i,), daemon=True)
               for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors


@pytest.mark.parametrize("handle", [False, True], ids=["torch_stream", "raw_handle"])
def test_explicit_side_stream(handle):
    # every wrapper given stream= a side stream (not torch's current one): the
    # outputs, the zero-filled grad_hidden, the lm_head backward's workspace and
    # the lm_head statistics it allocates belong to that stream, so churning the
    # allocator on the current stream meanwhile changes nothing
    case = make_case(81)
    ref = run(case)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    arg = s.cuda_stream if handle else s
    lp, ent, lse, grad = bi.fwd_bwd(case["z"], case["y"], case["w"], stream=arg)
    hlp, hent, hlse = bi.lmhead_logprob(case["H"], case["W"], case["hy"], stream=arg)
    gh, gw = bi.lmhead_backward(case["H"], case["W"], case["hy"], hlse, case["tw"],
                                chunk_rows=512, stream=arg)
    qlp, qent, qlse, qgrad = bi.fwd_bwd(case["zq"], case["yq"], case["wq"], stream=arg)
    junk = [torch.full((1 << 22,), float(i), device="cuda") for i in range(16)]
    del junk
    s.synchronize()
    outs = [lp, ent, lse, grad, hlp, hent, hlse, gh, gw, qlp, qent, qlse, qgrad]
    for k, (o, r) in enumerate(zip(outs, ref)):
        assert same(o, r), f"output {k} differs on a side stream"
