"""Helpers shared by the GPU parity tests: moving seeded batches to the device
and running the fp64 oracle on row blocks in parallel threads."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle.bi_oracle as orc
from workloads import default_threads

# |delta| bounds per logits dtype: (logprob, entropy, grad)
TOL = {"f32": (2e-4, 2e-4, 1e-5), "bf16": (5e-3, 5e-3, 1e-3)}


def dev_logits(logits: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(logits).view(np.int16))
        return t.to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(logits)).to(device)


def dev(x, device="cuda"):
    return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to(device)


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return orc.decode(bits, "bf16")


def oracle_forward(logits, labels, dtype, block=32, threads=None):
    """Oracle (logprob, entropy, lse) over all rows, row blocks in threads."""
    n = len(labels)
    out = np.empty((3, n))

    def run(a):
        z = orc.decode(logits[a:a + block], dtype)
        out[:, a:a + block] = orc.forward(z, labels[a:a + block])

    with ThreadPoolExecutor(threads or default_threads()) as ex:
        list(ex.map(run, range(0, n, block)))
    return out[0], out[1], out[2]


def ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |x| (normal range)."""
    a = np.abs(x)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, 2.0 ** (e - 7), 2.0 ** -133)


def assert_close(got, want, tol, what):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, what
    same_nan = np.isnan(got) == np.isnan(want)
    assert same_nan.all(), f"{what}: NaN pattern differs"
    inf_ok = np.where(np.isinf(want), got == want, True)
    assert inf_ok.all(), f"{what}: infinities differ"
    fin = np.isfinite(want)
    err = np.abs(got[fin] - want[fin])
    worst = float(err.max()) if err.size else 0.0
    assert worst <= tol, f"{what}: max |delta| {worst:.3g} > {tol:.3g}"
    return worst
