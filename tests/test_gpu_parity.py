"""GPU parity on small and medium shapes: the HIP path (through the C ABI)
against the fp64 oracle, element by element.

Shapes span one and many workgroup tiles, ragged last vectors and steps, odd
widths, row strides that leave rows 2- or 4-byte aligned, ignored labels,
masked (-inf) logits, non-uniform weights, and the degenerate V = 1 and N = 0.

Tolerances (|delta| against fp64): fp32 logits 2e-4 logprob, 2e-4 entropy,
1e-5 grad; bf16 logits 5e-3, 5e-3, 1e-3 (fp32 gradient).  A bf16 gradient must
equal the fp32 gradient rounded to nearest even, bit for bit, and lie within
1e-3 + half a bf16 ulp of the oracle.
"""
import numpy as np
import pytest
import torch

import entropy_bi_logprob_amd as bi
import oracle.bi_oracle as orc
from golden_cases import load as load_golden
from gpu_util import TOL, assert_close, dev, dev_logits, host, ulp_bf16
from workloads import f32_to_bf16_bits, random_batch

pytestmark = pytest.mark.gpu

WIDTHS = [1, 2, 3, 7, 8, 9, 15, 16, 17, 63, 64, 65, 127, 513, 1000, 4097, 8192, 16_389,
          65_539, 151_936, 151_937]


def run_all(b, grad_dtypes=("f32",)):
    logits = dev_logits(b.logits, b.dtype)
    labels = dev(b.labels)
    w = dev(b.weights)
    lp, ent, lse = bi.fwd(logits, labels)
    grads = {}
    for gd in grad_dtypes:
        tdt = torch.float32 if gd == "f32" else torch.bfloat16
        grads[gd] = bi.bwd(logits, labels, lse, w, tdt)
    torch.cuda.synchronize()
    return (host(lp), host(ent), host(lse)), {k: host(v) for k, v in grads.items()}


def check_against_oracle(b, outs, grads):
    tl, te, tg = TOL[b.dtype]
    z = orc.decode(b.logits, b.dtype)
    olp, oent, olse = orc.forward(z, b.labels)
    lp, ent, lse = outs
    assert_close(lp, olp, tl, "logprob")
    assert_close(ent, oent, te, "entropy")
    assert_close(lse, olse, tl, "lse")
    ign = b.labels == -100
    assert np.all(lp[ign] == 0) and not np.any(np.signbit(lp[ign])), "ignored logprob not +0.0"
    og = orc.backward(z, b.labels, olse, b.weights)
    if "f32" in grads:
        g = grads["f32"]
        assert_close(g, og, tg, "grad")
        assert np.all(g[ign] == 0) and not np.any(np.signbit(g[ign])), "ignored grad not +0.0"
        if "bf16" in grads:
            gb = grads["bf16"]
            np.testing.assert_array_equal(gb, f32_to_bf16_bits(g))     # RNE of the fp32 path
            gbv = orc.decode(gb, "bf16")
            bound = tg + 0.5 * ulp_bf16(og)
            assert np.all(np.abs(gbv - og) <= bound), "bf16 grad outside 1e-3 + ulp/2"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", WIDTHS)
def test_widths(dtype, V):
    rows = 6 if V > 60_000 else 19
    b = random_batch(rows, V, dtype, seed=V, ignore_frac=0.2,
                     mask_frac=0.1 if V > 4 else 0.0)
    gds = ("f32", "bf16") if dtype == "bf16" else ("f32",)
    outs, grads = run_all(b, gds)
    check_against_oracle(b, outs, grads)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_peaked_and_shifted_rows(dtype):
    # large offsets and one dominant logit per row
    b = random_batch(12, 50_001, dtype, seed=3, sigma=3.0)
    x = orc.decode(b.logits, dtype).astype(np.float32)
    x += np.float32(200.0)
    for i, y in enumerate(b.labels):
        x[i, y] += np.float32(25.0 if i % 2 else 9.0)
    b.logits = f32_to_bf16_bits(x) if dtype == "bf16" else x
    outs, grads = run_all(b)
    check_against_oracle(b, outs, grads)


def test_uniform_rows_closed_form():
    V = 151_936
    x = np.full((4, V), 1.5, dtype=np.float32)
    labels = np.array([0, 7, V - 1, -100])
    lp, ent, lse = (host(t) for t in bi.fwd(dev_logits(x, "f32"), dev(labels)))
    assert np.abs(lp[:3] + np.log(V)).max() < 2e-6
    assert np.abs(ent - np.log(V)).max() < 2e-6
    assert np.abs(lse - (1.5 + np.log(V))).max() < 2e-6


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("pad,offset", [(0, 1), (1, 0), (3, 1), (8, 3)])
def test_strided_and_unaligned_rows(dtype, pad, offset):
    V, n = 20_011, 7
    b = random_batch(n, V, dtype, seed=11 + pad, ignore_frac=0.2, mask_frac=0.05)
    stride = V + pad
    store = np.zeros(offset + n * stride, dtype=b.logits.dtype)
    for i in range(n):
        store[offset + i * stride: offset + i * stride + V] = b.logits[i]
    base = dev_logits(store, dtype)
    view = base[offset:offset + (n - 1) * stride + V].as_strided((n, V), (stride, 1))
    labels, w = dev(b.labels), dev(b.weights)
    lp, ent, lse = bi.fwd(view, labels)
    gstore = torch.zeros(offset + n * stride, dtype=torch.float32, device="cuda")
    gview = gstore[offset:offset + (n - 1) * stride + V].as_strided((n, V), (stride, 1))
    bi.bwd(view, labels, lse, w, out=gview)
    # contiguous copy: must be bit-identical (row alignment changes nothing)
    lp2, ent2, lse2 = bi.fwd(dev_logits(b.logits, dtype), labels)
    g2 = bi.bwd(dev_logits(b.logits, dtype), labels, lse2, w, torch.float32)
    torch.cuda.synchronize()
    for a, c in ((lp, lp2), (ent, ent2), (lse, lse2), (gview, g2)):
        np.testing.assert_array_equal(host(a.contiguous()), host(c))
    check_against_oracle(b, (host(lp), host(ent), host(lse)), {"f32": host(gview.contiguous())})


def test_bf16_gradient_on_odd_rows_with_2_byte_alignment():
    V, n = 3001, 5
    b = random_batch(n, V, "bf16", seed=5, ignore_frac=0.2)
    stride = V + 1
    store = np.zeros(1 + n * stride, dtype=np.uint16)
    for i in range(n):
        store[1 + i * stride: 1 + i * stride + V] = b.logits[i]
    base = dev_logits(store, "bf16")
    view = base[1:1 + (n - 1) * stride + V].as_strided((n, V), (stride, 1))
    labels, w = dev(b.labels), dev(b.weights)
    lp, ent, lse = bi.fwd(view, labels)
    gstore = torch.zeros(1 + n * stride, dtype=torch.bfloat16, device="cuda")
    gview = gstore[1:1 + (n - 1) * stride + V].as_strided((n, V), (stride, 1))
    bi.bwd(view, labels, lse, w, out=gview)
    g32 = bi.bwd(view, labels, lse, w, torch.float32)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(gview.contiguous()), f32_to_bf16_bits(host(g32)))
    check_against_oracle(b, (host(lp), host(ent), host(lse)), {"f32": host(g32)})


def test_golden_tiny_rows():
    for c in load_golden():
        logits = dev_logits(c["logits"][None, :], c["dtype"])
        labels = dev(np.array([c["label"]]))
        lp, ent, lse = bi.fwd(logits, labels)
        g = bi.bwd(logits, labels, lse, dev(np.array([c["weight"]], np.float32)), torch.float32)
        torch.cuda.synchronize()
        tl, te, tg = TOL[c["dtype"]]
        assert abs(host(lp)[0] - c["logprob"]) <= tl
        assert abs(host(ent)[0] - c["entropy"]) <= te
        assert abs(host(lse)[0] - c["lse"]) <= tl
        assert np.abs(host(g)[0] - np.array(c["grad"])).max() <= tg


def test_bad_labels_raise_the_flag_and_give_nan():
    V = 1000
    b = random_batch(5, V, "bf16", seed=2)
    labels = np.array([3, V, -1, -100, 10 ** 12])
    logits, lab = dev_logits(b.logits, "bf16"), dev(labels)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    lp, ent, lse = bi.fwd(logits, lab, status=flag)
    g = bi.bwd(logits, lab, lse, None, torch.float32, status=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == bi.BI_FLAG_BAD_LABEL
    lp, g = host(lp), host(g)
    assert np.isfinite(lp[0]) and np.isnan(lp[1]) and np.isnan(lp[2]) and lp[3] == 0
    assert np.isnan(lp[4]) and np.all(np.isfinite(host(ent)))
    assert np.isnan(g[1]).all() and np.isnan(g[2]).all() and np.isnan(g[4]).all()
    assert np.isfinite(g[0]).all() and np.all(g[3] == 0)
    flag.zero_()
    bi.fwd(logits[:1], lab[:1], status=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0


def test_empty_batch_and_fully_masked_rows():
    lp, ent, lse = bi.fwd(torch.empty((0, 10), dtype=torch.bfloat16, device="cuda"),
                          torch.empty(0, dtype=torch.int64, device="cuda"))
    assert lp.numel() == 0
    x = np.full((2, 300), -np.inf, dtype=np.float32)
    x[1, 5] = 2.0
    lp, ent, lse = (host(t) for t in bi.fwd(dev_logits(x, "f32"), dev(np.array([1, 5]))))
    assert lse[0] == -np.inf and np.isnan(lp[0]) and np.isnan(ent[0])
    assert lse[1] == 2.0 and lp[1] == 0.0 and ent[1] == 0.0


def test_nan_logits_propagate():
    x = np.zeros((1, 5000), dtype=np.float32)
    x[0, 1234] = np.nan
    lp, ent, lse = (host(t) for t in bi.fwd(dev_logits(x, "f32"), dev(np.array([0]))))
    assert np.isnan(lse[0]) and np.isnan(lp[0])


def test_autograd_wrapper_matches_bwd():
    b = random_batch(8, 7001, "bf16", seed=9, ignore_frac=0.25)
    logits = dev_logits(b.logits, "bf16").requires_grad_(True)
    labels = dev(b.labels)
    lp, ent = bi.logprob_entropy(logits, labels)
    adv = torch.linspace(-1.0, 2.0, 8, device="cuda")
    (-(adv * lp).sum()).backward()
    assert not ent.requires_grad
    _, _, lse = bi.fwd(logits.detach(), labels)
    g = bi.bwd(logits.detach(), labels, lse, adv.contiguous(), torch.bfloat16)
    torch.cuda.synchronize()
    assert logits.grad.dtype == torch.bfloat16
    np.testing.assert_array_equal(host(logits.grad), host(g))


@pytest.mark.parametrize("V", [4097, 65_539, 147_456, 151_936, 151_937])
@pytest.mark.parametrize("dt,gdt", [("bf16", torch.bfloat16), ("bf16", torch.float32),
                                    ("f32", torch.float32)])
def test_bwd_writes_every_element_deterministically(V, dt, gdt):
    # regression: gradient stores must neither be dropped nor corrupted; the
    # output starts as NaN (or zeros) and two runs must agree bit for bit
    b = random_batch(6, V, dt, seed=V + 1, ignore_frac=0.2, mask_frac=0.1)
    logits, labels, w = dev_logits(b.logits, dt), dev(b.labels), dev(b.weights)
    lp, ent, lse = bi.fwd(logits, labels)
    g1 = torch.full((6, V), float("nan"), dtype=gdt, device="cuda")
    g2 = torch.zeros((6, V), dtype=gdt, device="cuda")
    bi.bwd(logits, labels, lse, w, out=g1)
    bi.bwd(logits, labels, lse, w, out=g2)
    torch.cuda.synchronize()
    assert not bool(torch.isnan(g1).any())
    ity = torch.int16 if gdt == torch.bfloat16 else torch.int32
    assert torch.equal(g1.view(ity), g2.view(ity))


@pytest.mark.parametrize("dt,gdt,V", [("bf16", torch.bfloat16, 151_936),
                                      ("bf16", torch.float32, 131_072),
                                      ("bf16", torch.bfloat16, 151_938),
                                      ("f32", torch.float32, 65_539),
                                      ("f32", torch.float32, 30_000),
                                      ("bf16", torch.bfloat16, 30_728)])
def test_bwd_sweep_equals_row_kernel(dt, gdt, V):
    # wide rows on 4-byte boundaries take the backward as a sweep of 256-vector
    # pieces; the fused kernel's second pass and (for bf16) rows on 2-byte
    # boundaries walk whole rows.  The gradients must agree bit for bit, with
    # labels on both sides of every piece seam, in the first and last columns
    # and in a ragged tail, ignored rows, one bad label, and a padded row pitch.
    n, vec = 37, (8 if dt == "bf16" else 4)
    seam = 256 * vec                         # elements per piece
    b = random_batch(n, V, dt, seed=V + 11, ignore_frac=0.15, mask_frac=0.05)
    labels = b.labels.copy()
    for r in range(n):
        if labels[r] != -100 and r % 3 != 2:
            k = 1 + (r * 7) % (V // seam - 1)    # a seam inside the row
            labels[r] = k * seam if r % 3 == 0 else k * seam - 1
    labels[1], labels[2], labels[4], labels[5] = 0, V - 1, V - 1 - (V % vec) // 2, V + 3
    logits, lab, w = dev_logits(b.logits, dt), dev(labels), dev(b.weights)
    f1 = torch.zeros(1, dtype=torch.int32, device="cuda")
    lp, ent, lse = bi.fwd(logits, lab)
    sweep = bi.bwd(logits, lab, lse, w, gdt, status=f1)
    _, _, flse, fused = bi.fwd_bwd(logits, lab, w, gdt)
    wide = torch.zeros((n, V + 64), dtype=logits.dtype, device="cuda")
    wide[:, :V] = logits
    gwide = torch.full((n, V + 8), float("nan"), dtype=gdt, device="cuda")
    padded = bi.bwd(wide[:, :V], lab, lse, w, out=gwide[:, :V])
    torch.cuda.synchronize()
    assert int(f1.item()) != 0
    ity = torch.int16 if gdt == torch.bfloat16 else torch.int32
    assert torch.equal(lse.view(torch.int32), flse.view(torch.int32))
    assert torch.equal(sweep.view(ity), fused.view(ity))
    assert torch.equal(sweep.view(ity), padded.view(ity))
    if dt == "bf16":
        odd = torch.zeros(n * (V + 1) + 1, dtype=logits.dtype, device="cuda")
        view = odd[1:].view(n, V + 1)[:, :V]          # rows on 2-byte boundaries
        view.copy_(logits)
        rowk = bi.bwd(view, lab, lse, w, gdt)
        torch.cuda.synchronize()
        assert torch.equal(sweep.view(ity), rowk.view(ity))
    assert bool(torch.isnan(sweep[5].float()).all())
    ign = torch.from_numpy(labels == -100).cuda()
    assert int((sweep[ign].view(ity) != 0).sum().item()) == 0   # ignored rows: +0.0 everywhere


def _fused_vs_two_calls(logits, labels, w, gdt):
    lp, ent, lse = bi.fwd(logits, labels)
    g = bi.bwd(logits, labels, lse, w, gdt)
    flp, fent, flse, fg = bi.fwd_bwd(logits, labels, w, gdt)
    torch.cuda.synchronize()
    for a, c in ((lp, flp), (ent, fent), (lse, flse)):
        assert torch.equal(a.view(torch.int32), c.view(torch.int32))
    ity = torch.int16 if gdt == torch.bfloat16 else torch.int32
    assert torch.equal(g.view(ity), fg.view(ity))
    return flp, fent, flse, fg


@pytest.mark.parametrize("V", [1, 7, 16, 65, 1000, 4097, 16_389, 65_539, 151_936, 151_937])
@pytest.mark.parametrize("dt,gdt", [("bf16", torch.bfloat16), ("bf16", torch.float32),
                                    ("f32", torch.float32)])
def test_fused_equals_fwd_then_bwd_bitwise(V, dt, gdt):
    b = random_batch(7, V, dt, seed=V + 3, ignore_frac=0.2, mask_frac=0.1 if V > 4 else 0.0)
    logits, labels, w = dev_logits(b.logits, dt), dev(b.labels), dev(b.weights)
    flp, fent, flse, fg = _fused_vs_two_calls(logits, labels, w, gdt)
    # and against the oracle
    grads = {"f32": host(fg)} if gdt == torch.float32 else {}
    check_against_oracle(b, (host(flp), host(fent), host(flse)), grads)


@pytest.mark.parametrize("V", [131_080, 151_938, 155_640, 155_648])
@pytest.mark.parametrize("gdt", [torch.bfloat16, torch.float32], ids=["g_bf16", "g_f32"])
def test_fused_wide_rows_tail_cases_equal_two_calls(V, gdt):
    # widths around the headline vocabulary (bf16 rows of 1024 lanes, 17 to 19
    # vectors per lane): a ragged last step with a whole or a partial vector,
    # or none; labels in the first column, the last column, the last whole
    # vector, ignored and out of range
    n = 8
    b = random_batch(n, V, "bf16", seed=V, ignore_frac=0.0)
    labels = b.labels.copy()
    labels[:6] = [0, V - 1, V - 2, (V // 8) * 8 - 1, -100, V + 5]
    logits, lab = dev_logits(b.logits, "bf16"), dev(labels)
    for w in (dev(b.weights), None):
        _fused_vs_two_calls(logits, lab, w, gdt)
    ok = labels[:] != V + 5
    lp, ent, lse, g = bi.fwd_bwd(logits, lab, dev(b.weights), gdt)
    torch.cuda.synchronize()
    rows = np.flatnonzero(ok)
    z = orc.decode(b.logits[rows], "bf16")
    olp, oent, olse = orc.forward(z, labels[rows])
    tl, te, tg = TOL["bf16"]
    assert_close(host(lp)[rows], olp, tl, "logprob")
    assert_close(host(ent)[rows], oent, te, "entropy")
    og = orc.backward(z, labels[rows], olse, b.weights[rows])
    gh = host(g.float())[rows]
    assert np.all(np.abs(gh - og) <= tg + (0.5 * ulp_bf16(og) if gdt == torch.bfloat16 else 0))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("pad,offset", [(1, 0), (3, 1)])
def test_fused_on_strided_unaligned_rows(dt, pad, offset):
    V, n = 20_011, 6
    b = random_batch(n, V, dt, seed=21 + pad, ignore_frac=0.2, mask_frac=0.05)
    stride = V + pad
    store = np.zeros(offset + n * stride, dtype=b.logits.dtype)
    for i in range(n):
        store[offset + i * stride: offset + i * stride + V] = b.logits[i]
    base = dev_logits(store, dt)
    view = base[offset:offset + (n - 1) * stride + V].as_strided((n, V), (stride, 1))
    labels, w = dev(b.labels), dev(b.weights)
    gdt = torch.bfloat16 if dt == "bf16" else torch.float32
    gstore = torch.zeros(offset + n * stride, dtype=gdt, device="cuda")
    gview = gstore[offset:offset + (n - 1) * stride + V].as_strided((n, V), (stride, 1))
    flp, fent, flse, _ = bi.fwd_bwd(view, labels, w, grad=gview)
    lp, ent, lse = bi.fwd(dev_logits(b.logits, dt), labels)
    g = bi.bwd(dev_logits(b.logits, dt), labels, lse, w, gdt)
    torch.cuda.synchronize()
    for a, c in ((lp, flp), (ent, fent), (lse, flse)):
        assert torch.equal(a.view(torch.int32), c.view(torch.int32))
    ity = torch.int16 if gdt == torch.bfloat16 else torch.int32
    assert torch.equal(g.view(ity), gview.contiguous().view(ity))


def test_fused_bad_labels_and_null_outputs():
    V = 3000
    b = random_batch(4, V, "bf16", seed=8)
    logits = dev_logits(b.logits, "bf16")
    labels = dev(np.array([5, V + 2, -100, 17]))
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    grad = torch.full((4, V), float("nan"), dtype=torch.float32, device="cuda")
    lib = bi.lib()
    import ctypes
    rc = lib.bi_logprob_fwd_bwd(ctypes.c_void_p(logits.data_ptr()), bi.BI_BF16, 4, V, V,
                                ctypes.c_void_p(labels.data_ptr()), -100, None, None, None, None,
                                ctypes.c_void_p(grad.data_ptr()), bi.BI_F32, V,
                                ctypes.c_void_p(flag.data_ptr()), None)
    torch.cuda.synchronize()
    assert rc == 0 and int(flag.item()) == bi.BI_FLAG_BAD_LABEL
    g = host(grad)
    assert np.isfinite(g[0]).all() and np.isnan(g[1]).all() and np.all(g[2] == 0)
    assert np.isfinite(g[3]).all()


@pytest.mark.parametrize("dt,V", [("bf16", 151_936), ("f32", 65_539), ("bf16", 1000)])
def test_policy_loss_against_oracle_and_two_calls(dt, V):
    n, lo, hi = 48, 0.2, 0.28
    b = random_batch(n, V, dt, seed=V + 11, ignore_frac=0.15, mask_frac=0.05)
    z = orc.decode(b.logits, dt)
    olp, _, olse = orc.forward(z, b.labels)
    g = np.random.default_rng([V, 5])
    # behaviour logprobs around the current ones, so ratios span both clip sides
    old = (olp - g.uniform(-0.5, 0.5, n)).astype(np.float32)
    adv = g.standard_normal(n).astype(np.float32)
    scale = np.full(n, 1.0 / n, dtype=np.float32)
    logits, labels = dev_logits(b.logits, dt), dev(b.labels)
    gdt = torch.bfloat16 if dt == "bf16" else torch.float32
    lp, ent, lse, loss, w, grad = bi.policy_loss_fwd_bwd(
        logits, labels, dev(old), dev(adv), lo, hi, dev(scale), gdt)
    lp2, ent2, lse2 = bi.fwd(logits, labels)
    g2 = bi.bwd(logits, labels, lse2, w, gdt)
    torch.cuda.synchronize()
    for a, c in ((lp, lp2), (ent, ent2), (lse, lse2)):
        assert torch.equal(a.view(torch.int32), c.view(torch.int32))
    ity = torch.int16 if gdt == torch.bfloat16 else torch.int32
    assert torch.equal(grad.view(ity), g2.view(ity))
    # weights and losses against the fp64 oracle
    ign = b.labels == -100
    oloss, ow, ocl = orc.policy_terms(olp, old, adv, lo, hi, scale, ign)
    w, loss = host(w), host(loss)
    r = np.exp(olp - old)
    edge = (np.abs(r - (1 - lo)) < 1e-4) | (np.abs(r - (1 + hi)) < 1e-4)
    sure = ~edge
    assert np.abs(w[sure] - ow[sure]).max() <= 1e-5 * max(1.0, np.abs(ow).max())
    assert np.abs(loss[sure] - oloss[sure]).max() <= 1e-5 * max(1.0, np.abs(oloss).max())
    # near a clip boundary either branch is correct: zero, or c A r
    for i in np.nonzero(edge & ~ign)[0]:
        assert w[i] == 0.0 or abs(w[i] - scale[i] * adv[i] * r[i]) <= 1e-5
    assert np.all(w[ign] == 0) and np.all(loss[ign] == 0)
    assert 0 < ocl[~ign].sum() < (~ign).sum()        # both branches are exercised


@pytest.mark.parametrize("dt,V,K", [("bf16", 151_936, 5), ("f32", 20_011, 1), ("bf16", 4097, 1300)])
def test_fwd_multi_columns(dt, V, K):
    n = 9
    b = random_batch(n, V, dt, seed=V + K, ignore_frac=0.0, mask_frac=0.05)
    g = np.random.default_rng([V, K])
    ids = g.integers(0, V, size=(n, K)).astype(np.int64)
    ids[:, 0] = b.labels                      # column 0 holds the row's label
    if K > 1:
        ids[1, -1] = -100
    if K > 2:
        ids[2, 1] = V + 3                     # one bad id
    logits = dev_logits(b.logits, dt)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    lp, ent, lse = bi.fwd_multi(logits, dev(ids), status=flag)
    lp1, ent1, lse1 = bi.fwd(logits, dev(b.labels))
    torch.cuda.synchronize()
    assert torch.equal(lse.view(torch.int32), lse1.view(torch.int32))
    assert torch.equal(ent.view(torch.int32), ent1.view(torch.int32))
    assert torch.equal(lp[:, 0].contiguous().view(torch.int32), lp1.view(torch.int32))
    assert int(flag.item()) == (bi.BI_FLAG_BAD_LABEL if K > 2 else 0)
    olp, oent, olse = orc.forward_multi(orc.decode(b.logits, dt), ids)
    assert_close(host(lp), olp, TOL[dt][0], "multi logprob")
    h = host(lp)
    if K > 1:
        assert h[1, -1] == 0.0 and not np.signbit(h[1, -1])


def test_diff_stats_against_oracle():
    g = np.random.default_rng(4)
    n = 50_001
    a = g.standard_normal(n).astype(np.float32)
    b = a.copy()
    idx = g.choice(n, 7_000, replace=False)
    b[idx] += g.standard_normal(7_000).astype(np.float32) * 1e-3
    labels = g.integers(0, 100, n).astype(np.int64)
    labels[g.choice(n, 500, replace=False)] = -100
    out = host(bi.diff_stats(dev(a), dev(b), dev(labels)))
    want = orc.diff_stats(a, b, labels)
    np.testing.assert_allclose(out[:2], want[:2], rtol=1e-6, atol=1e-12)
    assert out[2] == np.float32(want[2]) and out[3] == np.float32(want[3])
    zero = host(bi.diff_stats(dev(a), dev(a)))
    assert np.all(zero == 0)


def test_trainer_and_generator_logprobs_are_bitwise_equal():
    # trainer: one call over a batch of 512 rows; generator: the same rows one at
    # a time through the multi-column path with the label in column 3
    b = random_batch(512, 151_936, "bf16", seed=77, ignore_frac=0.05)
    logits, labels = dev_logits(b.logits, "bf16"), dev(b.labels)
    pi, _, _ = bi.fwd(logits, labels)
    g = np.random.default_rng(5)
    mu = torch.empty_like(pi)
    for i in range(0, 512, 37):
        ids = g.integers(0, 151_936, size=(1, 6)).astype(np.int64)
        ids[0, 3] = b.labels[i]
        lp, _, _ = bi.fwd_multi(logits[i:i + 1], dev(ids))
        mu[i] = lp[0, 3]
    rows = torch.arange(0, 512, 37, device="cuda")
    stats = host(bi.diff_stats(pi[rows].contiguous(), mu[rows].contiguous(), labels[rows].contiguous()))
    assert np.all(stats == 0), stats


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_ignore_index_that_is_a_column(dt):
    # ignore_index 3 is also a valid column: rows labelled 3 are ignored (+0
    # logprob and gradient, entropy kept) on every path that takes a label, and
    # column 3 still gets the softmax term of every other row
    ii, n, v = 3, 37, 5_003
    b = random_batch(n, v, dt, seed=91, ignore_frac=0.0)
    lab = np.where(b.labels == ii, ii + 1, b.labels)
    lab[np.random.default_rng(5).choice(n, 9, replace=False)] = ii
    ign = lab == ii
    tl, te, tg = TOL[dt]
    z = orc.decode(b.logits, dt)
    olp, oent, olse = orc.forward(z, lab, ignore_index=ii)
    og = orc.backward(z, lab, olse, b.weights, ignore_index=ii)
    logits, labels, w = dev_logits(b.logits, dt), dev(lab), dev(b.weights)
    lp, ent, lse = bi.fwd(logits, labels, ii)
    g = bi.bwd(logits, labels, lse, w, torch.float32, ii)
    flp, fent, flse, fg = bi.fwd_bwd(logits, labels, w, torch.float32, ii)
    bounds = [(0, 2000), (2000, 2001), (2001, v)]
    st = torch.stack([bi.vocab_chunk_stats(logits[:, a:c], labels, a, v, ii) for a, c in bounds])
    clp, cent, clse = bi.stats_combine(st, labels, ii)
    mlab = torch.stack([labels, torch.full_like(labels, ii), (labels + 1) % v], dim=1)
    mlp, ment, mlse = bi.fwd_multi(logits, mlab, ii)
    torch.cuda.synchronize()
    for what, (a, e, s) in {"fwd": (lp, ent, lse), "fwd_bwd": (flp, fent, flse),
                            "chunked": (clp, cent, clse)}.items():
        assert_close(host(a), olp, tl, f"{what} logprob")
        assert_close(host(e), oent, te, f"{what} entropy")
        assert_close(host(s), olse, tl, f"{what} lse")
        assert np.all(host(a)[ign] == 0) and not np.any(np.signbit(host(a)[ign])), what
    for what, x in {"bwd": g, "fwd_bwd": fg}.items():
        gx = host(x)
        assert_close(gx, og, tg, f"{what} grad")
        assert np.all(gx[ign] == 0) and not np.any(np.signbit(gx[ign])), what
    omlp, _, _ = orc.forward_multi(z, host(mlab), ignore_index=ii)
    assert_close(host(mlp), omlp, tl, "multi logprob")
    assert np.all(host(mlp)[:, 1] == 0) and not np.any(np.signbit(host(mlp)[:, 1]))


# bf16 widths whose 1,024-lane rows fit the registers (17 to 19 vectors per
# lane): every (full steps, ragged step) class the row-on-chip fused kernel
# has, 300 rows so that each workgroup walks more than one row (the next row's
# vectors requested during this one), ignored rows and a bad label
# every on-chip shape (17..19 vectors per lane, with and without a ragged
# step), and just outside the band, where the re-reading kernel takes over:
# 131,072 (512-lane geometry), 155,650 (not a multiple of 8), 155,656 (20
# vectors per lane)
ONCHIP_WIDTHS = [131_080, 139_264, 139_272, 147_456, 147_464, 151_936, 155_648,
                 131_072, 155_650, 155_656]


@pytest.mark.parametrize("V", ONCHIP_WIDTHS)
@pytest.mark.parametrize("gdt", [torch.bfloat16, torch.float32], ids=["g_bf16", "g_f32"])
def test_fused_row_on_chip_equals_two_calls(V, gdt):
    n = 300
    b = random_batch(n, V, "bf16", seed=V % 1000, ignore_frac=0.1, mask_frac=0.01)
    labels = b.labels.copy()
    labels[7] = V + 3                              # a bad label: NaN row, flag raised
    logits, dlab, w = dev_logits(b.logits, "bf16"), dev(labels), dev(b.weights)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    flp, fent, flse, fg = bi.fwd_bwd(logits, dlab, w, gdt, status=flag)
    lp, ent, lse = bi.fwd(logits, dlab)
    g = bi.bwd(logits, dlab, lse, w, gdt)
    torch.cuda.synchronize()
    assert int(flag.item()) == bi.BI_FLAG_BAD_LABEL
    i32 = torch.int32
    for a, c in ((flp, lp), (fent, ent), (flse, lse)):
        assert torch.equal(a.view(i32), c.view(i32))
    gv = torch.int16 if gdt == torch.bfloat16 else torch.int32
    assert torch.equal(fg.view(gv), g.view(gv))
    assert torch.isnan(fg[7].float()).all() and torch.isnan(flp[7])
    rows = np.array([0, 1, 255, 256, 257, 299])    # rows of a second walk included
    z = orc.decode(b.logits[rows], "bf16")
    olp, oent, olse = orc.forward(z, labels[rows])
    tl, te, tg = TOL["bf16"]
    assert_close(host(flp)[rows], olp, tl, "logprob")
    assert_close(host(fent)[rows], oent, te, "entropy")
    if gdt == torch.float32:
        og = orc.backward(z, labels[rows], olse, b.weights[rows])
        assert_close(host(fg)[rows], og, tg, "grad")


def _padded(rows, stride, dtype):
    """[n, V] rows copied into a zero buffer of row pitch `stride`; the [n, V] view."""
    n, V = rows.shape
    buf = torch.zeros((n, stride), dtype=dtype, device="cuda")
    buf[:, :V] = rows
    return buf[:, :V]


@pytest.mark.parametrize("V", [139_272, 151_936, 155_648])   # 17 + ragged, 18 + ragged, 19 steps
@pytest.mark.parametrize("n", [1, 257, 600])                  # one row; a second walk for a few
def test_fused_row_on_chip_strided_rows_and_step_seams(V, n):   # workgroups; three walks
    # padded logits and gradient pitches, labels on the first and last column
    # and on each side of every step seam (a step is 1,024 vectors of 8), a
    # bad label, the policy kernel with its in-kernel weights: each against
    # the two calls on contiguous rows, bit for bit
    b = random_batch(n, V, "bf16", seed=n + V % 977, ignore_frac=0.1, mask_frac=0.01)
    labels = b.labels.copy()
    seams = [0, V - 1] + [s * 8192 + d for s in range(1, V // 8192 + 1) for d in (-1, 0)
                          if 0 <= s * 8192 + d < V]
    for i in range(n):
        if labels[i] != -100:
            labels[i] = seams[i % len(seams)]
    if n > 1:
        labels[1] = V + 5                                     # a bad label: NaN row, flag raised
    dense = dev_logits(b.logits, "bf16")
    logits = _padded(dense, V + 24, torch.bfloat16)          # 48 more bytes per row
    dlab, w = dev(labels), dev(b.weights)
    i32 = torch.int32
    for gdt, gpad in ((torch.bfloat16, 6), (torch.float32, 3)):
        grad = _padded(torch.full((n, V), float("nan"), dtype=gdt, device="cuda"), V + gpad, gdt)
        flag = torch.zeros(1, dtype=torch.int32, device="cuda")
        flp, fent, flse, _ = bi.fwd_bwd(logits, dlab, w, grad=grad, status=flag)
        lp, ent, lse = bi.fwd(dense, dlab)
        g = bi.bwd(dense, dlab, lse, w, gdt)
        torch.cuda.synchronize()
        assert int(flag.item()) == (bi.BI_FLAG_BAD_LABEL if n > 1 else 0)
        for a, c in ((flp, lp), (fent, ent), (flse, lse)):
            assert torch.equal(a.view(i32), c.view(i32))
        gv = torch.int16 if gdt == torch.bfloat16 else torch.int32
        assert torch.equal(grad.contiguous().view(gv), g.view(gv))
    # the policy kernel (its weights derived in the kernel) against fwd + bwd
    z = orc.decode(b.logits, "bf16")
    olp, _, _ = orc.forward(z, labels)
    gen = np.random.default_rng([V, n])
    old = (olp - gen.uniform(-0.5, 0.5, n)).astype(np.float32)
    adv = gen.standard_normal(n).astype(np.float32)
    pflag = torch.zeros(1, dtype=torch.int32, device="cuda")
    plp, pent, plse, loss, pw, pg = bi.policy_loss_fwd_bwd(
        logits, dlab, dev(old), dev(adv), 0.2, 0.28, None, torch.bfloat16, status=pflag)
    lp, ent, lse = bi.fwd(dense, dlab)
    g = bi.bwd(dense, dlab, lse, pw, torch.bfloat16)
    torch.cuda.synchronize()
    assert int(pflag.item()) == (bi.BI_FLAG_BAD_LABEL if n > 1 else 0)
    if n > 1:
        assert torch.isnan(plp[1]) and torch.isnan(pw[1]) and torch.isnan(loss[1])
        assert torch.isnan(pg[1].float()).all()
    for a, c in ((plp, lp), (pent, ent), (plse, lse)):
        assert torch.equal(a.view(i32), c.view(i32))
    assert torch.equal(pg.view(torch.int16), g.view(torch.int16))
    rows = np.unique(np.array([0, n // 2, n - 1]))
    tl, te, _ = TOL["bf16"]
    assert_close(host(plp)[rows], olp[rows], tl, "policy logprob")
