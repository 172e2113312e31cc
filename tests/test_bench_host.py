"""Host logic of bench.py (no GPU): the one-GPU contract, the algorithmic byte
counts of the large workload, and the rule that HBM traffic from a committed
counter summary is reported only while the kernel sources are the ones it was
taken from."""
import json
import os
import re
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_large_workload_algorithmic_bytes():
    # 32,768 x 151,936 bf16 logits, bf16 gradient: 9.957 GB for the forward and
    # 19.91 GB for the backward, 29.87 GB for the two passes
    n, v = 32768, 151936
    f, b, c, m = bench.algorithmic_bytes(v, 2, 2, 4)
    assert round(n * f / 1e9, 3) == 9.958
    assert round(n * b / 1e9, 2) == 19.92
    assert round(n * (f + b) / 1e9, 2) == 29.87
    # the chunked path reads the logits once more than the combine's few bytes
    assert c > v * 2 and m < 100


def _block(path):
    text = open(path).read()
    return json.loads(re.search(r"```json\n(.*?)\n```", text, re.S).group(1))


def test_committed_summaries_hold_the_bench_bytes():
    blk = _block(bench.TRAFFIC_SUMMARY)
    n, v = 32768, 151936
    f, b, _, _ = bench.algorithmic_bytes(v, 2, 2, 4)
    per = blk["per_launch"]
    assert per["fwd"]["algorithmic_bytes"] == n * f
    assert per["bwd"]["algorithmic_bytes"] == n * b
    assert per["fused"]["algorithmic_bytes"] == n * (v * 4 + 8 + 4 + 12)
    for k in per.values():
        assert abs(k["traffic_bytes"] - k["read_bytes"] - k["write_bytes"]) < 1.0
    lm = _block(bench.LMHEAD_SUMMARY)["per_launch"]
    assert {"lmhead", "lmhead_backward"} <= set(lm)


def test_traffic_is_reported_only_for_the_sources_it_was_taken_from(tmp_path):
    got = bench.measured_traffic("fused")
    blk = _block(bench.TRAFFIC_SUMMARY)
    import hashlib
    h = hashlib.sha256()
    for f in bench.KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    if h.hexdigest() == blk["source_sha256"]:
        assert got == blk["per_launch"]["fused"]["traffic_bytes"]
    else:
        assert got is None
    # a changed source (here: another file in its place) voids the figure
    other = tmp_path / "changed.hip"
    other.write_text("// not the kernel the counters were taken from\n")
    assert bench.measured_traffic("fused", sources=[str(other)]) is None
    # an unknown kernel or a missing summary gives no figure either
    assert bench.measured_traffic("no_such_kernel") is None
    assert bench.measured_traffic("fused", summary=str(tmp_path / "missing.md")) is None


def test_cpu_baseline_reports_host_cores_and_threads_separately():
    cores, threads = bench.host_cpu()
    assert cores == len(os.sched_getaffinity(0))
    assert 1 <= threads <= min(cores, 16)


def test_ceilings_library_exports_and_validates():
    # the same-run read and copy ceilings come from libbi_ceilings.so; its host
    # checks reject bad arguments before anything is launched (no GPU here)
    import ctypes
    import pytest
    path = os.path.join(ROOT, "entropy_bi_logprob_amd", "libbi_ceilings.so")
    if not os.path.exists(path):
        pytest.skip("libbi_ceilings.so not built")
    L = bench.ceilings_lib()
    P = ctypes.c_void_p(0x10000)
    assert L.bi_ceiling_read(P, 100, P, None) == -1          # not a multiple of 16
    assert L.bi_ceiling_read(None, 160, P, None) == -1       # no source
    assert L.bi_ceiling_read(ctypes.c_void_p(0x10004), 160, P, None) == -1   # misaligned
    assert L.bi_ceiling_copy(P, None, 160, None) == -1
    assert L.bi_ceiling_copy(P, P, -16, None) == -1
    assert L.bi_ceiling_read(P, 0, P, None) == 0             # nothing to do


def test_blas_threads_is_a_count():
    n = bench.blas_threads()
    assert n is None or (isinstance(n, int) and n >= 1)
