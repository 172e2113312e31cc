"""Benchmark: batch-invariant per-token logprob / entropy / gradient on one MI355X.

One step is one pass of the hot path over a batch of 32,768 x 151,936 bf16
logits (64 rollouts x 512 tokens, Qwen3 vocabulary) with per-token weights:
the full-row forward (logprob, entropy, lse) and the backward (bf16 grad =
w * (softmax - onehot)), as one bi_logprob_fwd_bwd call.  The same step as two
calls (bi_logprob_fwd + bi_logprob_bwd, "two_call") and the vocabulary-chunked
variant (4 x bi_vocab_chunk_stats of 37,984 columns + bi_stats_combine + the
backward, "chunked") are timed in the same run.  Inputs are seeded synthetic
logits, resident in HBM before the timed region.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline]

Prints one JSON line.  Kernel times come from HIP events recorded on the
stream the kernels run on (torch's current stream).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "logits GB/s & rows/s fwd+bwd at 32768×151936 bf16; % of HBM peak"
HBM_PEAK_GBPS = 8000.0     # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-rows", type=int, default=32768)
    ap.add_argument("--profile-steps", type=int, default=None,
                    help="run only this many steps, after one warm-up step (for profilers); "
                         "still prints the line")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workload shapes (256 x 151,936 fp32 forward, "
                         "4,096 x 151,936 bf16 and 2,048 x 151,937 masked fp32 fwd + bwd)")
    ap.add_argument("--no-lmhead", action="store_true",
                    help="skip the lm_head-projection leg (GEMM + statistics on matrix cores)")
    ap.add_argument("--calibrate-copy-gib", type=float, default=0.0,
                    help="first run one plain elementwise copy of this many GiB (bf16 in, "
                         "bf16 out), a known-size reference for memory counters")
    return ap.parse_args()


def algorithmic_bytes(vocab, e_in, e_grad, chunks):
    """Bytes per row the method must move (read logits, labels; write outputs)."""
    fwd = vocab * e_in + 8 + 12                # logits + label + (logprob, entropy, lse)
    bwd = vocab * (e_in + e_grad) + 8 + 4 + 4  # logits + grad + label + lse + weight
    chunk = vocab * e_in + chunks * (8 + 16)   # all chunks: logits + label + bi_stats each
    combine = chunks * 16 + 8 + 12             # stats + label + outputs
    return fwd, bwd, chunk, combine


TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "large_32768x151936_bf16_hbm_traffic.md")
# the sources of the row kernels (the counters below are only valid for them)
KERNEL_SOURCES = [os.path.join(ROOT, "entropy_bi_logprob_amd", "csrc", f)
                  for f in ("bi_common.h", "bi_logprob.hip")]


LMHEAD_SUMMARY = os.path.join(ROOT, "profiles", "lmhead_32768x2560x151936_bf16_counters.md")
LMHEAD_SOURCES = [os.path.join(ROOT, "entropy_bi_logprob_amd", "csrc", f)
                  for f in ("bi_common.h", "bi_lmhead.hip")]


def measured_traffic(kernel, summary=TRAFFIC_SUMMARY, sources=KERNEL_SOURCES):
    """HBM bytes per launch from a committed counter summary, or None when the
    kernel source has changed since the counters were taken."""
    import hashlib
    import re

    try:
        text = open(summary).read()
        block = json.loads(re.search(r"```json\n(.*?)\n```", text, re.S).group(1))
        h = hashlib.sha256()
        for f in sources:
            h.update(open(f, "rb").read())
        sha = h.hexdigest()
    except (OSError, AttributeError, ValueError):
        return None
    if block.get("source_sha256") != sha or kernel not in block.get("per_launch", {}):
        return None
    return block["per_launch"][kernel]["traffic_bytes"]


MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16


def host_cpu():
    """(cores this process may run on, oracle worker threads).  The threads are
    capped at 16, the host share of one GPU on the boxes this runs on."""
    import workloads as wl

    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cores = os.cpu_count() or 1
    return cores, wl.default_threads()


def ceilings_lib():
    """libbi_ceilings.so: a plain read-only stream and a plain copy (bench only)."""
    import ctypes

    path = os.path.join(ROOT, "entropy_bi_logprob_amd", "libbi_ceilings.so")
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build with `python -m entropy_bi_logprob_amd.build`")
    L = ctypes.CDLL(path)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    L.bi_ceiling_read.argtypes = [vp, i64, vp, vp]
    L.bi_ceiling_copy.argtypes = [vp, vp, i64, vp]
    L.bi_ceiling_read.restype = L.bi_ceiling_copy.restype = ctypes.c_int
    return L


def lmhead_leg(bi, torch, np, wl, N, V, seed, steps, warm, stream, with_cpu=True):
    """Logprob/entropy straight from hidden states: hidden [N, 2560] x lm_head [V, 2560]^T
    on the matrix cores, reduced to statistics without materialising the logits; timed
    beside the unfused pipeline (library GEMM to bf16 logits, then bi_logprob_fwd)."""
    d = wl.LMHEAD_HIDDEN
    b = wl.lmhead_batch(N, V, d, seed=seed)
    dev = torch.device("cuda:0")
    H = torch.from_numpy(b.hidden.view(np.int16)).to(dev).view(torch.bfloat16)
    W = torch.from_numpy(b.weight.view(np.int16)).to(dev).view(torch.bfloat16)
    labels = torch.from_numpy(b.labels).to(dev)
    tiles = int(bi.lib().bi_lmhead_tiles(V))
    st = torch.empty((tiles, N, 4), dtype=torch.float32, device=dev)
    outs = tuple(torch.empty(N, dtype=torch.float32, device=dev) for _ in range(3))
    ks = max(1, min(steps, 10))

    def timed(fns):
        for _ in range(max(1, min(warm, 2))):
            for f in fns:
                f()
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)]
              for _ in range(ks)]
        for k in range(ks):
            ev[k][0].record(stream)
            for i, f in enumerate(fns):
                f()
                ev[k][i + 1].record(stream)
        torch.cuda.synchronize()
        return [float(np.mean([e[i].elapsed_time(e[i + 1]) for e in ev])) for i in range(len(fns))]

    t_stats, t_comb = timed([lambda: bi.lmhead_tile_stats(H, W, labels, out=st, stream=stream),
                             lambda: bi.stats_combine(st, labels, out=outs, stream=stream)])
    # backward from the saved lse (token weights: a mean over tokens)
    lse = outs[2]
    tw = torch.full((N,), -1.0 / N, dtype=torch.float32, device=dev)
    gh = torch.zeros((N, d), dtype=torch.float32, device=dev)
    gw = torch.empty((V, d), dtype=torch.bfloat16, device=dev)
    chunk = 32768
    ws = torch.empty(int(bi.lib().bi_lmhead_backward_workspace(N, d, chunk)), dtype=torch.uint8,
                     device=dev)
    (t_bwd,) = timed([lambda: bi.lmhead_backward(H, W, labels, lse, tw, grad_hidden=gh,
                                                 grad_weight=gw, workspace=ws, stream=stream)])
    del ws
    logits = torch.empty((N, V), dtype=torch.bfloat16, device=dev)
    t_gemm, t_fwd = timed([lambda: torch.matmul(H, W.t(), out=logits),
                           lambda: bi.fwd(logits, labels, out=outs, stream=stream)])
    # unfused backward: logits, their gradient (10 GB each), then two library GEMMs
    glog = torch.empty((N, V), dtype=torch.bfloat16, device=dev)
    ghu = torch.empty((N, d), dtype=torch.bfloat16, device=dev)
    t_ub = timed([lambda: torch.matmul(H, W.t(), out=logits),
                  lambda: bi.bwd(logits, labels, lse, tw, torch.bfloat16, out=glog,
                                 stream=stream),
                  lambda: torch.matmul(glog, W, out=ghu),
                  lambda: torch.matmul(glog.t(), H, out=gw)])
    del logits, glog, st, ghu, gh, gw
    # the pages' chunked-backward shape: 16 x 330 tokens, one tp = 4 vocabulary shard
    ns, vs = 16 * 330, V // 4
    Hs, Ws, ls = H[:ns].contiguous(), W[:vs].contiguous(), labels[:ns] % vs
    _, _, lses = bi.lmhead_logprob(Hs, Ws, ls)
    ghs = torch.zeros((ns, d), dtype=torch.float32, device=dev)
    gws = torch.empty((vs, d), dtype=torch.bfloat16, device=dev)
    (t_small,) = timed([lambda: bi.lmhead_backward(Hs, Ws, ls, lses, tw[:ns], grad_hidden=ghs,
                                                   grad_weight=gws, stream=stream)])
    flops = 2.0 * N * V * d
    tf = flops / (t_stats * 1e-3) / 1e12
    tfb = 3 * flops / (t_bwd * 1e-3) / 1e12
    cpu = lmhead_cpu_baseline(b, np, wl) if with_cpu else None
    return {"workload": f"hidden {N}x{d} bf16, lm_head {V}x{d} bf16",
            "fused_ms": t_stats + t_comb, "tile_stats_ms": t_stats, "combine_ms": t_comb,
            "rows_per_s": N / ((t_stats + t_comb) * 1e-3),
            "roofline": {"bound": "mfma", "achieved": tf, "peak": MFMA_BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": tf / MFMA_BF16_PEAK_TFLOPS,
                         "traffic": (measured_traffic("lmhead", LMHEAD_SUMMARY, LMHEAD_SOURCES)
                                     if (N, V, d) == (32768, 151936, 2560) else None)},
            "unfused_ms": t_gemm + t_fwd, "unfused_gemm_ms": t_gemm, "unfused_fwd_ms": t_fwd,
            "unfused_gemm_TFLOPs": flops / (t_gemm * 1e-3) / 1e12,
            "speedup_vs_unfused": (t_gemm + t_fwd) / (t_stats + t_comb),
            "backward": {
                "what": "bi_lmhead_backward: grad_hidden (fp32) and grad_weight (bf16) from the "
                        "saved lse, 32768-row vocabulary chunks",
                "ms": t_bwd, "TFLOPs_3gemm": tfb,
                "roofline": {"bound": "mfma", "achieved": tfb, "peak": MFMA_BF16_PEAK_TFLOPS,
                             "unit": "TFLOP/s", "frac": tfb / MFMA_BF16_PEAK_TFLOPS,
                             "traffic": (measured_traffic("lmhead_backward", LMHEAD_SUMMARY,
                                                          LMHEAD_SOURCES)
                                         if (N, V, d) == (32768, 151936, 2560) else None)},
                "unfused_ms": sum(t_ub), "unfused_parts_ms": t_ub,
                "unfused_what": "torch.matmul logits, bi_logprob_bwd to bf16, two torch.matmul "
                                "(20 GB of logits and gradient)",
                "speedup_vs_unfused": sum(t_ub) / t_bwd,
                "pages_shape_ms": t_small,
                "pages_shape": "16 x 330 tokens, 37984 vocabulary rows (one tp = 4 shard), "
                               "d 2560"},
            "cpu_baseline": cpu}


def blas_threads():
    """Threads numpy's BLAS runs its matrix products on (threadpoolctl, else
    OMP_NUM_THREADS), or None if neither says."""
    try:
        import numpy  # noqa: F401  (loads its BLAS, so that threadpoolctl finds it)
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads") for i in threadpool_info() if i.get("user_api") == "blas"]
        if n and all(isinstance(k, int) for k in n):
            return max(n)
    except Exception:
        pass
    v = os.environ.get("OMP_NUM_THREADS", "")
    return int(v) if v.isdigit() else None


def lmhead_cpu_baseline(b, np, wl, sample=2048):
    """The fp64 oracle on the first `sample` tokens of the lm_head workload: forward
    (logits, logprob, entropy) and backward (the gradient of the logits, grad_hidden
    and those tokens' grad_weight terms), full vocabulary and hidden size."""
    import oracle.bi_oracle as orc

    h = orc.decode(b.hidden[:sample], "bf16")
    w = orc.decode(b.weight, "bf16")
    labels = b.labels[:sample]
    t0 = time.perf_counter()
    lp, ent, lse = orc.forward(orc.lmhead_logits(h, w), labels)
    t1 = time.perf_counter()
    orc.lmhead_backward(h, w, labels, lse, np.full(sample, -1.0 / sample))
    t2 = time.perf_counter()
    cores, _ = host_cpu()
    return {"fwd_tokens_per_s": sample / (t1 - t0), "fwd_bwd_tokens_per_s": sample / (t2 - t0),
            "unit": "tokens/s", "cores": cores, "threads": blas_threads(),
            "threads_what": "BLAS threads of numpy's matrix products", "kind": "oracle",
            "sample": f"{sample} tokens x 151936 lm_head rows x d 2560, fp64 numpy "
                      f"(BLAS threads as configured), {t2 - t0:.1f} s wall"}


def cpu_baseline(rows_total, sample_rows, seed):
    """The fp64 oracle (as it stands) on a bounded sample of the same workload."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle.bi_oracle as orc
    import workloads as wl

    g = np.random.default_rng([seed, 77])
    rows = np.sort(g.choice(rows_total, size=sample_rows, replace=False))
    b = wl.draw(5, rows=rows, seed=seed)
    cores, threads = host_cpu()
    block = 16

    def run(a):
        z = orc.decode(b.logits[a:a + block], "bf16")
        lp, ent, lse = orc.forward(z, b.labels[a:a + block])
        orc.backward(z, b.labels[a:a + block], lse, b.weights[a:a + block])

    t0 = time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(run, range(0, sample_rows, block)))
    dt = time.perf_counter() - t0
    return {"value": sample_rows / dt, "unit": "rows/s", "cores": cores, "threads": threads,
            "kind": "oracle",
            "sample": f"{sample_rows} seeded rows of the 32768x151936 bf16 workload, "
                      f"fp64 numpy forward+backward, {threads} worker threads (capped at the "
                      f"16-core host share of one GPU) over 16-row blocks on a host with "
                      f"{cores} cores available, {dt:.2f} s wall"}


def generator_leg(bi, torch, np, logits, labels, trainer_logprob, seed, steps, warm, stream,
                  k=8):
    """The generator side on the large workload: K token ids per row sharing one lse
    (the sampled label and K - 1 seeded candidates), then the trainer-vs-generator
    difference metrics between its label column and the fused call's logprob."""
    n, v = logits.shape
    g = np.random.default_rng([seed, 31])
    cand = torch.from_numpy(g.integers(0, v, size=(n, k), dtype=np.int64)).to(logits.device)
    cand[:, 0] = labels

    def timed(fn):
        for _ in range(max(warm, 1)):
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        outs = []
        for e0, e1 in ev:
            e0.record(stream)
            outs.append(fn())
            e1.record(stream)
        torch.cuda.synchronize()
        return float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev])), outs[-1]

    ms_multi, (lp, _, _) = timed(lambda: bi.fwd_multi(logits, cand, stream=stream))
    gen = lp[:, 0].contiguous()
    ms_diff, d = timed(lambda: bi.diff_stats(trainer_logprob, gen, labels, stream=stream))
    d = d.cpu().tolist()
    nbytes = n * (v * 2 + k * 8 + k * 4 + 8)
    gbps = nbytes / (ms_multi * 1e-3) / 1e9
    return {"what": f"bi_logprob_fwd_multi: {k} token ids per row sharing one lse; "
                    "bi_logprob_diff_stats between its label column and the fused call's "
                    "logprob", "k": k, "ms": ms_multi, "rows_per_s": n / (ms_multi * 1e-3),
            "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": gbps / HBM_PEAK_GBPS, "traffic": None},
            "diff_stats_ms": ms_diff,
            "trainer_vs_generator": {"mean": d[0], "abs_mean": d[1], "max": d[2],
                                     "frac_tokens_different": d[3]}}


def configs_leg(bi, torch, np, wl, seed, steps, warm, stream, with_cpu=True):
    """The pages' other workload shapes (256 x 151,936 fp32 forward; 4,096 x 151,936
    bf16 and 2,048 x 151,937 masked fp32 forward + backward), all rows drawn as the
    tests draw them, each timed on the GPU path, with the fp64 oracle timed on the
    same rows beside it."""
    from concurrent.futures import ThreadPoolExecutor

    dev = torch.device("cuda:0")
    out = {}
    for cfg in (1, 2, 3):
        w = wl.WORKLOADS[cfg]
        b = wl.draw(cfg, seed=seed)
        bf16 = w.dtype == "bf16"
        e_in = 2 if bf16 else 4
        gdt = torch.bfloat16 if bf16 else torch.float32
        e_g = 2 if bf16 else 4
        host = b.logits.view(np.int16) if bf16 else b.logits
        # a workload smaller than the 256 MB Infinity Cache is rotated over copies
        # (1 GiB in all at least) so that every call reads its logits from HBM
        size = w.rows * w.vocab * e_in
        copies = max(1, -(-(1 << 30) // size))
        logits = [torch.from_numpy(host).to(dev) for _ in range(copies)]
        if bf16:
            logits = [t.view(torch.bfloat16) for t in logits]
        labels = torch.from_numpy(b.labels).to(dev)
        weights = None if b.weights is None else torch.from_numpy(b.weights).to(dev)
        outs = tuple(torch.empty(w.rows, dtype=torch.float32, device=dev) for _ in range(3))
        grad = torch.empty((w.rows, w.vocab), dtype=gdt, device=dev) if w.backward else None
        f_b, b_b, _, _ = algorithmic_bytes(w.vocab, e_in, e_g, 1)

        def timed(fn):
            for i in range(max(warm, 1)):
                fn(logits[i % copies])
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(steps)]
            for i, (e0, e1) in enumerate(ev):
                e0.record(stream)
                fn(logits[i % copies])
                e1.record(stream)
            torch.cuda.synchronize()
            return float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev]))

        def two_calls(z):
            bi.fwd(z, labels, out=outs, stream=stream)
            if grad is not None:
                bi.bwd(z, labels, outs[2], weights, out=grad, stream=stream)

        ms = timed(two_calls)
        nbytes = w.rows * (f_b + (b_b if w.backward else 0))
        res = {"rows": w.rows, "vocab": w.vocab, "logits_dtype": w.dtype,
               "path": "bi_logprob_fwd + bi_logprob_bwd" if w.backward else "bi_logprob_fwd",
               "ms": ms, "rows_per_s": w.rows / (ms * 1e-3),
               "hbm_GBps": nbytes / (ms * 1e-3) / 1e9,
               "pct_hbm_peak": 100 * nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
               "logits_copies": copies}
        if w.backward:
            res["grad_dtype"] = "bf16" if bf16 else "f32"
            fms = timed(lambda z: bi.fwd_bwd(z, labels, weights, out=outs, grad=grad,
                                             stream=stream))
            fb = w.rows * (w.vocab * (e_in + e_g) + 24)
            res["fused"] = {"ms": fms, "rows_per_s": w.rows / (fms * 1e-3),
                            "hbm_GBps": fb / (fms * 1e-3) / 1e9,
                            "pct_hbm_peak": 100 * fb / (fms * 1e-3) / 1e9 / HBM_PEAK_GBPS}
        if with_cpu:
            import oracle.bi_oracle as orc

            cores, threads = host_cpu()
            block = 16

            def run(a):
                z = orc.decode(b.logits[a:a + block], w.dtype)
                lp, ent, lse = orc.forward(z, b.labels[a:a + block])
                if w.backward:
                    orc.backward(z, b.labels[a:a + block], lse,
                                 None if b.weights is None else b.weights[a:a + block])

            t0 = time.perf_counter()
            with ThreadPoolExecutor(threads) as ex:
                list(ex.map(run, range(0, w.rows, block)))
            dt = time.perf_counter() - t0
            res["cpu_oracle"] = {"rows_per_s": w.rows / dt, "cores": cores, "threads": threads,
                                 "s": dt, "sample": "all rows, fp64 numpy, 16-row blocks"}
        out[w.name] = res
        del logits, grad
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(rows shard across GPUs with no exchange: each GPU would run this path on its "
              "own rows)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import entropy_bi_logprob_amd as bi
    import workloads as wl

    seed = wl.DEFAULT_SEED if args.seed is None else args.seed
    w5 = wl.WORKLOADS[5]
    N, V = w5.rows, w5.vocab

    # inputs: drawn on the host (seeded, per row), then resident in HBM
    t0 = time.perf_counter()
    b = wl.draw(5, seed=seed)
    gen_s = time.perf_counter() - t0
    dev = torch.device("cuda:0")
    logits = torch.from_numpy(b.logits.view(np.int16)).to(dev).view(torch.bfloat16)
    labels = torch.from_numpy(b.labels).to(dev)
    weights = torch.from_numpy(b.weights).to(dev)
    del b
    lp = torch.empty(N, dtype=torch.float32, device=dev)
    ent = torch.empty_like(lp)
    lse = torch.empty_like(lp)
    grad = torch.empty((N, V), dtype=torch.bfloat16, device=dev)
    bounds = wl.chunk_bounds(V, wl.LARGE_CHUNKS)
    stats = torch.empty((len(bounds), N, 4), dtype=torch.float32, device=dev)
    clp, cent, clse = torch.empty_like(lp), torch.empty_like(lp), torch.empty_like(lp)
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    def step_fused(ev=None):
        if ev: ev[0].record(stream)
        bi.fwd_bwd(logits, labels, weights, out=(lp, ent, lse), grad=grad, status=flag,
                   stream=stream)
        if ev: ev[1].record(stream)

    g = np.random.default_rng([seed, 17])
    old_lp = torch.from_numpy(g.normal(-11.0, 1.5, N).astype(np.float32)).to(dev)
    adv = torch.from_numpy(g.standard_normal(N).astype(np.float32)).to(dev)
    scale = torch.full((N,), 1.0 / N, dtype=torch.float32, device=dev)
    ploss, pw = torch.empty_like(lp), torch.empty_like(lp)

    def step_policy(ev=None):
        if ev: ev[0].record(stream)
        L = bi.lib()
        rc = L.bi_policy_loss_fwd_bwd(
            logits.data_ptr(), bi.BI_BF16, N, V, V, labels.data_ptr(), -100, old_lp.data_ptr(),
            adv.data_ptr(), scale.data_ptr(), 0.2, 0.28, lp.data_ptr(), ent.data_ptr(),
            lse.data_ptr(), ploss.data_ptr(), pw.data_ptr(), grad.data_ptr(), bi.BI_BF16, V,
            flag.data_ptr(), stream.cuda_stream)
        assert rc == 0, rc
        if ev: ev[1].record(stream)

    def step_two_calls(ev=None):
        if ev: ev[0].record(stream)
        bi.fwd(logits, labels, out=(lp, ent, lse), status=flag, stream=stream)
        if ev: ev[1].record(stream)
        bi.bwd(logits, labels, lse, weights, out=grad, status=flag, stream=stream)
        if ev: ev[2].record(stream)

    def step_chunked(ev=None):
        if ev: ev[0].record(stream)
        for c, (a, e) in enumerate(bounds):
            bi.vocab_chunk_stats(logits[:, a:e], labels, a, V, out=stats[c], status=flag,
                                 stream=stream)
        if ev: ev[1].record(stream)
        bi.stats_combine(stats, labels, out=(clp, cent, clse), stream=stream)
        if ev: ev[2].record(stream)
        bi.bwd(logits, labels, clse, weights, out=grad, status=flag, stream=stream)
        if ev: ev[3].record(stream)

    if args.calibrate_copy_gib > 0:
        n_el = int(args.calibrate_copy_gib * (1 << 30)) // 2
        src = torch.ones(n_el, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)            # reads n_el*2 bytes, writes n_el*2 bytes
        torch.cuda.synchronize()
        del src, dst

    steps = args.profile_steps or args.steps
    # a profiled run still takes one warm-up step, so the traced averages are
    # not skewed by a first call on cold caches and clocks
    warm = min(args.warmup, 1) if args.profile_steps else args.warmup
    for _ in range(warm):
        step_fused()
        step_two_calls()
        step_chunked()
        step_policy()
    torch.cuda.synchronize()

    def timed(step, n_events):
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_events)]
               for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(steps):
            step(evs[k])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        seg = [[e[i].elapsed_time(e[i + 1]) for e in evs] for i in range(n_events - 1)]
        return wall * 1e3 / steps, seg

    # timed region: K steps of the whole path (one fused pass per row)
    ms_step, (t_fused,) = timed(step_fused, 2)
    # the same work as two calls, and the vocabulary-chunked variant, same run
    ms_two, (t_fwd, t_bwd) = timed(step_two_calls, 3)
    ms_chunked, (t_chunk, t_comb, t_cbwd) = timed(step_chunked, 4)
    ms_policy, (t_policy,) = timed(step_policy, 2)
    assert int(flag.item()) == 0

    # same-run reference for the fused kernel's HBM traffic: a library copy of
    # the logits into the gradient buffer reads and writes exactly the bytes the
    # fused kernel must move (its re-read comes from the caches)
    def step_copy(ev=None):
        if ev: ev[0].record(stream)
        torch.neg(logits, out=grad)
        if ev: ev[1].record(stream)

    step_copy()
    _, (t_copy,) = timed(step_copy, 2)

    # same-run ceilings: a plain read-only stream over the logits and a plain
    # copy of the logits into the gradient buffer (libbi_ceilings.so)
    CL = ceilings_lib()
    nbytes_logits = N * V * 2
    sink = torch.zeros(4, dtype=torch.int32, device=dev)

    def step_read(ev=None):
        if ev: ev[0].record(stream)
        rc = CL.bi_ceiling_read(logits.data_ptr(), nbytes_logits, sink.data_ptr(),
                                stream.cuda_stream)
        assert rc == 0, rc
        if ev: ev[1].record(stream)

    def step_plain_copy(ev=None):
        if ev: ev[0].record(stream)
        rc = CL.bi_ceiling_copy(logits.data_ptr(), grad.data_ptr(), nbytes_logits,
                                stream.cuda_stream)
        assert rc == 0, rc
        if ev: ev[1].record(stream)

    step_read()
    step_plain_copy()
    _, (t_read,) = timed(step_read, 2)
    _, (t_pcopy,) = timed(step_plain_copy, 2)

    f_b, b_b, c_b, m_b = algorithmic_bytes(V, 2, 2, len(bounds))
    fused_b = V * (2 + 2) + 8 + 4 + 12       # one read of the logits, one write of the grad
    med = lambda xs: float(np.median(xs))
    mean = lambda xs: float(np.mean(xs))
    gbps = lambda nbytes, ms: nbytes / (ms * 1e-3) / 1e9
    hbm = gbps(N * fused_b, ms_step)
    rows_s = N / (ms_step * 1e-3)
    kernels = {
        "fused": {"ms": mean(t_fused), "ms_median": med(t_fused),
                  "GBps": gbps(N * fused_b, mean(t_fused)), "bytes": N * fused_b},
        "fwd": {"ms": mean(t_fwd), "ms_median": med(t_fwd), "GBps": gbps(N * f_b, mean(t_fwd)),
                "bytes": N * f_b},
        "bwd": {"ms": mean(t_bwd), "ms_median": med(t_bwd), "GBps": gbps(N * b_b, mean(t_bwd)),
                "bytes": N * b_b},
        "chunk_stats_x4": {"ms": mean(t_chunk), "GBps": gbps(N * c_b, mean(t_chunk)),
                           "bytes": N * c_b},
        "combine": {"ms": mean(t_comb), "GBps": gbps(N * m_b, mean(t_comb)), "bytes": N * m_b},
    }
    read_ceiling = gbps(nbytes_logits, mean(t_read))
    copy_ceiling = gbps(2 * nbytes_logits, mean(t_pcopy))
    ceilings = {"what": "same run, same tensors: a plain read-only stream of the logits and "
                        "a plain copy of the logits into the gradient buffer (256-lane "
                        "workgroups, 16-byte non-temporal loads and stores)",
                "read_GBps": read_ceiling, "copy_GBps": copy_ceiling,
                "read_ms": mean(t_read), "copy_ms": mean(t_pcopy),
                "read_frac_of_peak": read_ceiling / HBM_PEAK_GBPS,
                "copy_frac_of_peak": copy_ceiling / HBM_PEAK_GBPS}
    # the ceiling each kernel is held to: reads only (forward, chunk statistics)
    # or a read and a write per element (backward, fused)
    ceiling_of = {"fused": copy_ceiling, "fwd": read_ceiling, "bwd": copy_ceiling,
                  "chunk_stats_x4": read_ceiling, "combine": read_ceiling}
    for name, k in kernels.items():
        k["frac_of_peak"] = k["GBps"] / HBM_PEAK_GBPS
        k["frac_of_ceiling"] = k["GBps"] / ceiling_of[name]
    dom = "fused"
    two_call = {"ms_per_step": ms_two, "rows_per_s": N / (ms_two * 1e-3),
                "hbm_GBps": gbps(N * (f_b + b_b), ms_two),
                "pct_hbm_peak": 100 * gbps(N * (f_b + b_b), ms_two) / HBM_PEAK_GBPS}
    policy = {"ms_per_step": ms_policy, "rows_per_s": N / (ms_policy * 1e-3),
              "kernel_ms": mean(t_policy), "clip": [0.2, 0.28],
              "what": "bi_policy_loss_fwd_bwd: logprob, entropy, clipped-ratio loss and its "
                      "gradient in one pass (weights derived in the kernel)"}
    chunked = {"ms_per_step": ms_chunked, "rows_per_s": N / (ms_chunked * 1e-3),
               "hbm_GBps": gbps(N * (c_b + m_b + b_b), ms_chunked),
               "bwd_ms": mean(t_cbwd)}
    line = {
        "metric": METRIC,
        "value": rows_s,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "large_32768x151936_bf16", "rows": N, "vocab": V,
                   "logits_dtype": "bf16", "grad_dtype": "bf16", "accum_dtype": "f32",
                   "path": "bi_logprob_fwd_bwd (full-row fwd + bwd, one call)", "seed": seed},
        "logits_GBps": N * V * 2 / (ms_step * 1e-3) / 1e9,
        "hbm_GBps": hbm,
        "pct_hbm_peak": 100.0 * hbm / HBM_PEAK_GBPS,
        "roofline": {"bound": "hbm", "achieved": kernels[dom]["GBps"], "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": kernels[dom]["GBps"] / HBM_PEAK_GBPS,
                     "traffic": measured_traffic(dom),
                     "kernel": "fused fwd+bwd (bf16 logits, bf16 grad)",
                     "bytes_per_launch": kernels[dom]["bytes"]},
        "kernels": kernels,
        "vs_target": {
            "what": "the target is 70% of 8 TB/s.  On its own bytes (one read of the logits, "
                    "one write of the gradient) the fused kernel reaches "
                    "fused_kernel_frac_of_peak; the two-call path reaches "
                    "two_call_pct_hbm_peak on its two-pass bytes.  Context only: "
                    "target_ms is 70% of peak over the two-pass bytes, which the fused "
                    "kernel does not move",
            "fused_kernel_frac_of_peak": kernels[dom]["GBps"] / HBM_PEAK_GBPS,
            "fused_kernel_frac_of_copy_ceiling": kernels[dom]["frac_of_ceiling"],
            "two_call_pct_hbm_peak": 100 * gbps(N * (f_b + b_b), ms_two) / HBM_PEAK_GBPS,
            "target_ms": N * (f_b + b_b) / (0.7 * HBM_PEAK_GBPS * 1e9) * 1e3,
            "fused_step_vs_two_pass_target": N * (f_b + b_b) / (0.7 * HBM_PEAK_GBPS * 1e9) * 1e3
            / ms_step},
        "ceilings": ceilings,
        "reference_copy": {
            "what": "torch.neg(logits, out=grad): a library copy of the same tensor, one read "
                    "and one write per element (the fused kernel's HBM bytes), same run",
            "ms": mean(t_copy), "GBps": gbps(2 * N * V * 2, mean(t_copy)),
            "fused_kernel_vs_copy": mean(t_copy) / mean(t_fused)},
        "two_call": two_call,
        "chunked": chunked,
        "policy_loss": policy,
        "input_gen_s": gen_s,
    }
    if not args.no_lmhead:
        line["lmhead"] = lmhead_leg(bi, torch, np, wl, N, V, seed, steps, warm, stream,
                                    with_cpu=not args.no_cpu_baseline and not args.profile_steps)
    if not args.profile_steps:
        step_fused()     # lp: the trainer's logprob, from the fused call
        line["generator"] = generator_leg(bi, torch, np, logits, labels, lp, seed, steps, warm,
                                          stream)
    if not args.no_configs and not args.profile_steps:
        line["configs"] = configs_leg(bi, torch, np, wl, seed, steps, warm, stream,
                                      with_cpu=not args.no_cpu_baseline)
    if not args.no_cpu_baseline and not args.profile_steps:
        line["cpu_baseline"] = cpu_baseline(N, args.cpu_sample_rows, seed)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
