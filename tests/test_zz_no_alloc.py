"""bi_lmhead_backward_noalloc (the lm_head backward for callers that cannot
allocate) against bi_lmhead_backward, called through the C ABI: on the same
inputs and a workspace of the static scratch's size (the same chunking) every
output bit must agree, on two calls in a row, the second with a smaller input
(the static scratch keeps the first call's contents), and on a shape that
takes many chunks of the scratch.  The small cases are also held to the
oracle's error bound."""
import ctypes

import numpy as np
import pytest
import torch

import entropy_bi_logprob_amd as bi
import oracle.bi_oracle as orc
import workloads as wl
from gpu_util import dev, host, ulp_bf16

pytestmark = pytest.mark.gpu

SCRATCH = 64 << 20        # BI_LMHEAD_NOALLOC_SCRATCH_BYTES
MAX_TOKENS = 131072       # BI_LMHEAD_NOALLOC_MAX_TOKENS


def to_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def noalloc(H, W, labels, lse, tw, gh, gw):
    """The entry point itself through ctypes: outputs are the caller's."""
    n, d = H.shape
    vc = W.shape[0]
    s = torch.cuda.current_stream().cuda_stream
    rc = bi.lib().bi_lmhead_backward_noalloc(
        H.data_ptr(), W.data_ptr(), n, vc, d, H.stride(0), W.stride(0), 0, vc,
        labels.data_ptr(), -100, lse.data_ptr(), tw.data_ptr(), gh.data_ptr(), gh.stride(0),
        gw.data_ptr(), bi.BI_BF16 if gw.dtype == torch.bfloat16 else bi.BI_F32, gw.stride(0),
        None, ctypes.c_void_p(s))
    assert rc == bi.BI_OK, bi.lib().bi_last_error()


def with_workspace(H, W, labels, lse, tw, gdt):
    ws = torch.empty(SCRATCH, dtype=torch.uint8, device="cuda")
    return bi.lmhead_backward(H, W, labels, lse, tw, grad_weight_dtype=gdt, workspace=ws)


def case(n, vc, d, seed):
    b = wl.lmhead_batch(n, vc, d, seed=seed, ignore_frac=0.05)
    H, W, labels = to_bf16(b.hidden), to_bf16(b.weight), dev(b.labels)
    _, _, lse = bi.lmhead_logprob(H, W, labels)
    tw = torch.linspace(-1.0, 1.0, n, device="cuda")
    return b, H, W, labels, lse, tw


def same(a, b):
    view = torch.int16 if a.element_size() == 2 else torch.int32
    return bool(torch.equal(a.view(view), b.view(view)))


def oracle_bound(b, lse, tw, gh, gw, gw_bf16):
    h, w = orc.decode(b.hidden, "bf16"), orc.decode(b.weight, "bf16")
    G, oh, ow = orc.lmhead_backward(h, w, b.labels, host(lse).astype(np.float64),
                                    host(tw).astype(np.float64))
    bh = (2.0 ** -8 + G.shape[1] * 2.0 ** -24) * (np.abs(G) @ np.abs(w)) + 1e-7
    bw = (2.0 ** -8 + G.shape[0] * 2.0 ** -24) * (np.abs(G).T @ np.abs(h)) + 1e-7
    if gw_bf16:
        bw = bw + 0.5 * ulp_bf16(ow)
    assert np.all(np.abs(host(gh) - oh) <= bh)
    assert np.all(np.abs(host(gw.float()) - ow) <= bw)


@pytest.mark.parametrize("gdt", [torch.bfloat16, torch.float32], ids=["gw_bf16", "gw_f32"])
def test_noalloc_equals_workspace_call_twice_then_smaller(gdt):
    for n, vc, d, seed in ((300, 1000, 128, 5), (77, 333, 64, 6)):   # the second is smaller
        b, H, W, labels, lse, tw = case(n, vc, d, seed)
        gh = torch.zeros((n, d), dtype=torch.float32, device="cuda")
        gw = torch.full((vc, d), float("nan"), dtype=gdt, device="cuda")
        noalloc(H, W, labels, lse, tw, gh, gw)
        rh, rw = with_workspace(H, W, labels, lse, tw, gdt)
        torch.cuda.synchronize()
        assert same(gh, rh) and same(gw, rw), (n, vc, d)
        oracle_bound(b, lse, tw, gh, gw, gdt == torch.bfloat16)


def test_noalloc_many_chunks_of_the_scratch():
    # 32,768 tokens: 1,024 lm_head rows per chunk of the 64 MiB scratch, so a
    # 20,000-row shard takes 20 chunks (the last ragged); grad_hidden adds them
    # in order, exactly as the workspace call does
    n, vc, d = 32768, 20_000, 128
    b, H, W, labels, lse, tw = case(n, vc, d, 7)
    gh = torch.zeros((n, d), dtype=torch.float32, device="cuda")
    gw = torch.empty((vc, d), dtype=torch.bfloat16, device="cuda")
    noalloc(H, W, labels, lse, tw, gh, gw)
    rh, rw = with_workspace(H, W, labels, lse, tw, torch.bfloat16)
    torch.cuda.synchronize()
    assert same(gh, rh) and same(gw, rw)
    assert torch.isfinite(gh).all() and torch.isfinite(gw.float()).all()


def test_noalloc_rejects_too_many_tokens():
    n, d = MAX_TOKENS + 1, 64
    H = torch.zeros((n, d), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((256, d), dtype=torch.bfloat16, device="cuda")
    labels = torch.zeros(n, dtype=torch.int64, device="cuda")
    lse = torch.zeros(n, dtype=torch.float32, device="cuda")
    gh = torch.zeros((n, d), dtype=torch.float32, device="cuda")
    gw = torch.zeros((256, d), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="static scratch"):
        bi.lmhead_backward_noalloc(H, W, labels, lse, None, gh, gw)
