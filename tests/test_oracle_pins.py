"""Pins of the fp64 oracle against things other than itself.

Each check below fixes the oracle to a closed form, a 50-digit brute force of a
different formula, a library routine (torch fp64 on the CPU), an invariant of
the mathematics, or finite differences.  ``test_planted_mistakes`` plants
plausible mistakes in the oracle (on the CPU) and checks that the core pins
catch every one of them.

Sources: "[RL] Avoid full-vocab gather for TP policy statistics" (torchtitan
PR #4685), sections Summary, Why, and Correctness and compatibility; its review
reply "Batch invariance under the patched logprob path" (Q1: plain
cross-entropy and logsumexp + softmax on full logits; Q2: MAX combines exactly,
SUM does not).
"""
import math

import mpmath as mp
import numpy as np
import pytest

import oracle.bi_oracle as orc
from workloads import random_batch

IGN = -100


def fwd1(z, y):
    lp, h, lse = orc.forward(np.asarray(z, dtype=np.float64)[None, :], np.array([y]))
    return lp[0], h[0], lse[0]


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("V", [1, 2, 7, 1000, 151_936, 151_937])
@pytest.mark.parametrize("c", [0.0, 3.5, -20.0, 250.0])
def test_uniform_row(V, c):
    z = np.full(V, c)
    y = V // 3
    lp, h, lse = fwd1(z, y)
    assert lp == pytest.approx(-math.log(V), abs=1e-12)
    assert h == pytest.approx(math.log(V), abs=1e-12)
    assert lse == pytest.approx(c + math.log(V), rel=1e-15, abs=1e-12)
    g = orc.backward(z[None, :], np.array([y]), np.array([lse]), np.array([0.75]))[0]
    expect = np.full(V, 0.75 / V)
    expect[y] = 0.75 * (1.0 / V - 1.0)
    np.testing.assert_allclose(g, expect, rtol=1e-12, atol=1e-15)


def test_qwen3_vocab_uniform_value():
    # -ln 151936, the uniform-row logprob at the Qwen3 vocabulary size
    lp, h, _ = fwd1(np.zeros(151_936), 5)
    assert lp == pytest.approx(-11.931214658529285, abs=1e-12)
    assert h == pytest.approx(11.931214658529285, abs=1e-12)


@pytest.mark.parametrize("V,k,a,b", [(10, 3, 2.0, -1.0), (151_936, 17, 6.0, 0.5),
                                     (5000, 4999, -3.0, 4.0)])
def test_two_level_row(V, k, a, b):
    z = np.full(V, b)
    z[:k] = a
    with mp.workdps(40):
        Z = k * mp.e ** a + (V - k) * mp.e ** b
        pa, pb = mp.e ** a / Z, mp.e ** b / Z
        lse = mp.log(Z)
        H = -(k * pa * mp.log(pa) + (V - k) * pb * mp.log(pb))
    lp, h, l2 = fwd1(z, 0)
    assert l2 == pytest.approx(float(lse), rel=1e-14)
    assert lp == pytest.approx(float(a - lse), abs=1e-12)
    assert h == pytest.approx(float(H), rel=1e-12)
    lp_b, _, _ = fwd1(z, V - 1)
    assert lp_b == pytest.approx(float(b - lse), abs=1e-12)


@pytest.mark.parametrize("delta", [0.0, 1.0, 8.0, 30.0, 60.0])
def test_dominant_logit(delta):
    V, c, y = 151_936, -1.25, 4242
    z = np.full(V, c)
    z[y] = c + delta
    lp, h, _ = fwd1(z, y)
    with mp.workdps(50):
        q = (V - 1) * mp.e ** (-delta)
        exact_lp = -mp.log1p(q)
        py = 1 / (1 + q)
        po = mp.e ** (-delta) * py
        exact_h = -(py * mp.log(py) + (V - 1) * po * mp.log(po))
    assert lp == pytest.approx(float(exact_lp), abs=1e-12)
    assert h == pytest.approx(float(exact_h), abs=1e-12, rel=1e-11)
    if delta >= 60:
        assert h < 1e-19   # entropy -> 0 for one dominant logit


def test_v1_and_v2():
    lp, h, lse = fwd1([3.0], 0)
    assert (lp, h, lse) == (0.0, 0.0, 3.0)
    g = orc.backward(np.array([[3.0]]), np.array([0]), np.array([lse]), np.array([2.0]))
    assert g[0, 0] == 0.0
    for zy, zo in [(0.3, -1.1), (-4.0, 7.5), (20.0, 20.0)]:
        lp, h, _ = fwd1([zo, zy], 1)
        x = zy - zo
        assert lp == pytest.approx(-math.log1p(math.exp(-x)), abs=1e-14)
        p = 1.0 / (1.0 + math.exp(-x))
        hb = -(p * math.log(p) + (1 - p) * math.log(1 - p))
        assert h == pytest.approx(hb, abs=1e-14)


# ------------------------------------------------- brute force (mpmath, 50 digits)

def _tiny_cases():
    g = np.random.default_rng(7)
    cases = []
    for V in (1, 2, 3, 5, 8, 16):
        for trial in range(4):
            z = g.standard_normal(V) * 3.0
            y = int(g.integers(0, V))
            if V > 2 and trial == 1:
                cols = [j for j in range(V) if j != y][: V // 3]
                z[cols] = -np.inf
            if trial == 2:
                y = IGN
            w = float(g.uniform(-1.0, 2.0))
            cases.append((z, y, w))
    return cases


@pytest.mark.parametrize("case", range(24))
def test_brute_force(case):
    z, y, w = _tiny_cases()[case]
    blp, bh, blse, bg = orc.brute_force(z, y, w)
    lp, h, lse = fwd1(z, y)
    assert lse == pytest.approx(blse, rel=1e-14, abs=1e-14)
    assert lp == pytest.approx(blp, abs=1e-13)
    assert h == pytest.approx(bh, abs=1e-13)
    g = orc.backward(z[None, :], np.array([y]), np.array([lse]), np.array([w]))[0]
    np.testing.assert_allclose(g, bg, rtol=1e-12, atol=1e-14)


# --------------------------------------------- library routine: torch fp64 (CPU)

def test_torch_fp64_cross_entropy_entropy_and_grad():
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    b = random_batch(48, 3001, "f32", seed=11, sigma=2.5, ignore_frac=0.1, mask_frac=0.1)
    z = orc.decode(b.logits, "f32")
    lp, h, lse = orc.forward(z, b.labels)
    zt = torch.tensor(z, dtype=torch.float64, requires_grad=True)
    yt = torch.tensor(b.labels)
    ce = F.cross_entropy(zt, yt, reduction="none", ignore_index=IGN)
    np.testing.assert_allclose(lp, -ce.detach().numpy(), rtol=0, atol=1e-12)
    ent = torch.special.entr(torch.softmax(zt.detach(), dim=1)).sum(1).numpy()
    np.testing.assert_allclose(h, ent, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, torch.logsumexp(zt.detach(), 1).numpy(), rtol=1e-14)
    w = torch.tensor(b.weights, dtype=torch.float64)
    (w * ce).sum().backward()
    g = orc.backward(z, b.labels, lse, b.weights)
    np.testing.assert_allclose(g, zt.grad.numpy(), rtol=1e-10, atol=1e-15)


# ----------------------------------------------------------------- invariants

def test_shift_invariance_and_bounds():
    b = random_batch(16, 777, "f32", seed=3, sigma=4.0, mask_frac=0.2)
    z = orc.decode(b.logits, "f32")
    lp, h, lse = orc.forward(z, b.labels)
    lp2, h2, lse2 = orc.forward(z + 123.5, b.labels)
    np.testing.assert_allclose(lp2, lp, atol=1e-10)
    np.testing.assert_allclose(h2, h, atol=1e-10)
    np.testing.assert_allclose(lse2 - 123.5, lse, atol=1e-10)
    nfin = np.isfinite(z).sum(1)
    assert np.all(h >= -1e-15) and np.all(h <= np.log(nfin) + 1e-12)


def test_gradient_invariants():
    b = random_batch(32, 501, "f32", seed=5, ignore_frac=0.25, mask_frac=0.1)
    z = orc.decode(b.logits, "f32")
    lp, h, lse = orc.forward(z, b.labels)
    g = orc.backward(z, b.labels, lse, b.weights)
    for i, y in enumerate(b.labels):
        if y == IGN:
            assert np.all(g[i] == 0.0) and not np.any(np.signbit(g[i]))
            continue
        w = float(b.weights[i])
        assert abs(g[i].sum()) < 1e-14 * max(1.0, w)
        py = math.exp(lp[i])
        assert g[i, y] == pytest.approx(w * (py - 1.0), rel=1e-12, abs=1e-16)
        others = np.delete(g[i], y)
        assert np.all(others >= 0.0)
        assert np.all(g[i][np.isneginf(z[i])] == 0.0)


def test_masked_row_equals_compacted_row():
    b = random_batch(8, 400, "f32", seed=9, mask_frac=0.3, ignore_frac=0.0)
    z = orc.decode(b.logits, "f32")
    lp, h, lse = orc.forward(z, b.labels)
    for i in range(8):
        keep = np.isfinite(z[i])
        zc = z[i][keep]
        yc = int(np.count_nonzero(keep[: b.labels[i]]))
        lpc, hc, lsec = fwd1(zc, yc)
        assert lp[i] == pytest.approx(lpc, abs=1e-13)
        assert h[i] == pytest.approx(hc, abs=1e-13)
        assert lse[i] == pytest.approx(lsec, abs=1e-13)


def test_ignored_rows_are_plus_zero_and_keep_entropy():
    b = random_batch(6, 300, "f32", seed=1, ignore_frac=0.0)
    z = orc.decode(b.logits, "f32")
    ign = np.full(6, IGN)
    lp, h, lse = orc.forward(z, ign)
    lp_v, h_v, lse_v = orc.forward(z, b.labels)
    assert np.all(lp == 0.0) and not np.any(np.signbit(lp))
    np.testing.assert_array_equal(h, h_v)
    np.testing.assert_array_equal(lse, lse_v)
    g = orc.backward(z, ign, lse, b.weights)
    assert np.all(g == 0.0) and not np.any(np.signbit(g))


def test_bad_label_is_nan():
    z = np.zeros((3, 10))
    lp, h, lse = orc.forward(z, np.array([10, -1, 3]))
    assert np.isnan(lp[0]) and np.isnan(lp[1]) and lp[2] == pytest.approx(-math.log(10))
    assert np.isfinite(h).all()
    g = orc.backward(z, np.array([10, -1, 3]), lse)
    assert np.isnan(g[0]).all() and np.isnan(g[1]).all() and np.isfinite(g[2]).all()


def test_fully_masked_row_natural_results():
    lp, h, lse = fwd1([-np.inf] * 4, 1)
    assert lse == -np.inf and np.isnan(lp) and np.isnan(h)


# ------------------------------------------------- finite differences (V <= 16)

@pytest.mark.parametrize("V", [2, 5, 16])
def test_finite_differences(V):
    g = np.random.default_rng(V)
    z = g.standard_normal(V) * 2.0
    y, w, hstep = int(g.integers(0, V)), 1.7, 1e-6
    lp, _, lse = fwd1(z, y)
    grad = orc.backward(z[None, :], np.array([y]), np.array([lse]), np.array([w]))[0]
    for j in range(V):
        zp, zm = z.copy(), z.copy()
        zp[j] += hstep
        zm[j] -= hstep
        fd = (-w * fwd1(zp, y)[0] + w * fwd1(zm, y)[0]) / (2 * hstep)
        assert grad[j] == pytest.approx(fd, abs=1e-8)


# ------------------------------------------------------------ chunks + combine

@pytest.mark.parametrize("bounds", [
    [(0, 1000)],
    [(0, 250), (250, 500), (500, 750), (750, 1000)],
    [(0, 1), (1, 333), (333, 334), (334, 1000)],
    [(j, j + 1) for j in range(1000)],
])
def test_chunk_combine_equals_full(bounds):
    b = random_batch(12, 1000, "f32", seed=21, ignore_frac=0.2, mask_frac=0.05)
    z = orc.decode(b.logits, "f32")
    lp, h, lse = orc.forward(z, b.labels)
    st = np.stack([orc.chunk_stats(z[:, a:e], b.labels, a, 1000) for a, e in bounds])
    lp2, h2, lse2 = orc.combine(st, b.labels, 1000)
    np.testing.assert_array_equal(st[:, :, 0].max(0), z.max(1))   # max is exact
    np.testing.assert_allclose(lse2, lse, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lp2, lp, rtol=0, atol=1e-12)
    np.testing.assert_allclose(h2, h, rtol=0, atol=1e-12)
    assert not np.any(np.signbit(lp2[b.labels == IGN]))


def test_fully_masked_chunk_is_a_no_op():
    b = random_batch(5, 600, "f32", seed=2, ignore_frac=0.0)
    z = orc.decode(b.logits, "f32")
    z[:, 200:400] = -np.inf
    labels = np.where((b.labels >= 200) & (b.labels < 400), 0, b.labels)
    lp, h, lse = orc.forward(z, labels)
    bounds = [(0, 200), (200, 400), (400, 600)]
    st = np.stack([orc.chunk_stats(z[:, a:e], labels, a, 600) for a, e in bounds])
    assert np.all(st[1, :, 0] == -np.inf) and np.all(st[1, :, 1] == 0) and np.all(st[1, :, 3] == 0)
    lp2, h2, lse2 = orc.combine(st, labels, 600)
    np.testing.assert_allclose(np.stack([lp2, h2, lse2]), np.stack([lp, h, lse]), atol=1e-12)


def test_chunk_uneven_qwen3_width():
    # V = 151,937 split into 4 contiguous chunks (the last one ragged)
    b = random_batch(3, 151_937, "f32", seed=4, mask_frac=0.1)
    z = orc.decode(b.logits, "f32")
    lp, h, lse = orc.forward(z, b.labels)
    w = -(-151_937 // 4)
    bounds = [(a, min(a + w, 151_937)) for a in range(0, 151_937, w)]
    st = np.stack([orc.chunk_stats(z[:, a:e], b.labels, a, 151_937) for a, e in bounds])
    lp2, h2, lse2 = orc.combine(st, b.labels, 151_937)
    np.testing.assert_allclose(np.stack([lp2, h2, lse2]), np.stack([lp, h, lse]), atol=1e-12)


def test_raw_weighted_sum_identity():
    # sum exp(z - m) * z == U + m * S (the unshifted form of the 4th statistic)
    b = random_batch(4, 257, "f32", seed=6)
    z = orc.decode(b.logits, "f32")
    m, S, U = orc.row_statistics(z)
    raw = (np.exp(z - m[:, None]) * z).sum(1)
    np.testing.assert_allclose(U + m * S, raw, rtol=1e-13, atol=1e-12)


# ------------------------------------------------------------- input decoding

def test_bf16_decode_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0xFF80, 0x7F80, 0x0001, 0x4049, 0x8000], dtype=np.uint16)
    v = orc.decode(bits, "bf16")
    assert v[0] == 1.0 and v[1] == -2.0 and v[2] == -np.inf and v[3] == np.inf
    assert v[4] == 2.0 ** -133 and v[5] == 3.140625
    assert v[6] == 0.0 and np.signbit(v[6])


# ------------------------------------------------------------ planted mistakes

def _pin_blocks():
    """Compact versions of the pins, as (name, callable returning bool)."""

    def uniform():
        lp, h, lse = fwd1(np.full(1000, 2.0), 3)
        return (abs(lp + math.log(1000)) < 1e-12 and abs(h - math.log(1000)) < 1e-12
                and abs(lse - 2.0 - math.log(1000)) < 1e-12)

    def dominant():
        z = np.full(50, -1.0)
        z[7] = 4.0
        lp, _, _ = fwd1(z, 7)
        return abs(lp + math.log1p(49 * math.exp(-5.0))) < 1e-12

    def brute():
        ok = True
        for zz, y, w in _tiny_cases()[::3]:
            blp, bh, blse, bg = orc.brute_force(zz, y, w)
            lp, h, lse = fwd1(zz, y)
            g = orc.backward(np.asarray(zz)[None, :], np.array([y]), np.array([lse]),
                             np.array([w]))[0]
            ok &= bool(abs(lp - blp) < 1e-12 and abs(h - bh) < 1e-12
                       and abs(lse - blse) < 1e-12 and np.allclose(g, bg, atol=1e-12))
        return ok

    bb = random_batch(64, 64, "f32", seed=31, ignore_frac=0.1, mask_frac=0.1)

    def square_batch():
        # a square batch, so that a transposed operand shows
        zb = orc.decode(bb.logits, "f32")
        lp, h, lse = orc.forward(zb, bb.labels)
        ok = True
        for i in range(0, 64, 9):
            blp, bh, _, _ = orc.brute_force(zb[i], int(bb.labels[i]), float(bb.weights[i]))
            ok &= bool(abs(lp[i] - blp) < 1e-12 and abs(h[i] - bh) < 1e-12)
        return ok

    def combine():
        zb = orc.decode(bb.logits, "f32")
        lp, h, lse = orc.forward(zb, bb.labels)
        st = np.stack([orc.chunk_stats(zb[:, a:e], bb.labels, a, 64)
                       for a, e in [(0, 10), (10, 40), (40, 64)]])
        lp2, h2, lse2 = orc.combine(st, bb.labels, 64)
        return bool(np.allclose(lp2, lp, atol=1e-12) and np.allclose(h2, h, atol=1e-12)
                    and np.allclose(lse2, lse, atol=1e-12))

    def bf16():
        return orc.decode(np.array([0x3F80, 0xC040], np.uint16), "bf16").tolist() == [1.0, -3.0]

    def policy():
        lo, hi = 0.2, 0.28
        lp = np.log(np.array([0.5, 0.9, 1.5, 0.5, 1.5]))
        A = np.array([2.0, 1.0, 2.0, -1.0, -1.0])
        loss, w, cl = orc.policy_terms(lp, np.zeros(5), A, lo, hi)
        want_w = np.array([1.0, 0.9, 0.0, 0.0, -1.5])
        want_loss = np.array([-1.0, -0.9, -2.56, 0.8, 1.5])
        return bool(np.allclose(w, want_w, atol=1e-12) and np.allclose(loss, want_loss, atol=1e-12))

    return [("uniform", uniform), ("dominant", dominant), ("brute", brute),
            ("square_batch", square_batch), ("combine", combine), ("bf16", bf16),
            ("policy", policy)]


def _core_pin_failures():
    """Run the compact pins; return the names of the failing ones."""
    fails = []
    for name, block in _pin_blocks():
        try:
            with np.errstate(all="ignore"):
                ok = block()
        except Exception:  # a crash is a failed pin too
            ok = False
        if not ok:
            fails.append(name)
    return fails


def test_core_pins_pass_on_the_oracle():
    assert _core_pin_failures() == []


def _mutations():
    o = orc
    real = {n: getattr(o, n) for n in ("weighted_sum", "finalize", "denominator",
                                       "target_logit", "backward", "combine", "decode",
                                       "row_max", "softmax_from_lse", "policy_terms")}

    def drop_u(d, keep):
        return np.zeros(d.shape[0])

    def entropy_sign(m, S, U, t, kind):
        lp, h, lse = real["finalize"](m, S, U, t, kind)
        return lp, np.log(S) + U / S, lse

    def no_shift(d, keep):
        return np.where(keep, np.exp(np.where(keep, d + 1.0, 0.0)), 0.0).sum(axis=1)

    def label_off_by_one(z, labels, ignore_index=IGN):
        lab = np.where(labels == ignore_index, labels, (labels + 1) % z.shape[1])
        return real["target_logit"](z, lab, ignore_index)

    def grad_sign(z, labels, lse, weights=None, ignore_index=IGN):
        return -real["backward"](z, labels, lse, weights, ignore_index)

    def grad_no_weight(z, labels, lse, weights=None, ignore_index=IGN):
        return real["backward"](z, labels, lse, None, ignore_index)

    def combine_no_rescale(stats, labels, vocab, ignore_index=IGN):
        st = np.array(stats, dtype=np.float64)
        M = st[:, :, 0].max(0)
        S = st[:, :, 1].sum(0)
        U = st[:, :, 3].sum(0)
        t = st[:, :, 2].sum(0)
        return real["finalize"](M, S, U, t, o.label_kind(labels, vocab, ignore_index))

    def combine_no_cross_term(stats, labels, vocab, ignore_index=IGN):
        st = np.array(stats, dtype=np.float64)
        M = st[:, :, 0].max(0)
        a = np.exp(st[:, :, 0] - M)
        S = (a * st[:, :, 1]).sum(0)
        U = (a * st[:, :, 3]).sum(0)
        t = st[:, :, 2].sum(0)
        return real["finalize"](M, S, U, t, o.label_kind(labels, vocab, ignore_index))

    def decode_shift15(logits, dtype):
        if dtype == "bf16":
            bits = np.asarray(logits, np.uint16).astype(np.uint32) << np.uint32(15)
            return bits.view(np.float32).astype(np.float64)
        return real["decode"](logits, dtype)

    def transposed_max(z):
        return z.max(axis=0)

    def softmax_wrong_ref(z, lse):
        return real["softmax_from_lse"](z, lse - 0.5)

    def policy_clip_swapped(logprob, old_logprob, advantages, clip_low, clip_high,
                            loss_scale=None, ignored=None):
        return real["policy_terms"](logprob, old_logprob, advantages, clip_high, clip_low,
                                    loss_scale, ignored)

    def policy_weight_without_ratio(logprob, old_logprob, advantages, clip_low, clip_high,
                                    loss_scale=None, ignored=None):
        loss, w, cl = real["policy_terms"](logprob, old_logprob, advantages, clip_low, clip_high,
                                           loss_scale, ignored)
        r = np.exp(np.asarray(logprob, float) - np.asarray(old_logprob, float))
        return loss, np.where(cl, 0.0, w / r), cl

    return {
        "policy_clip_swapped": ("policy_terms", policy_clip_swapped),
        "policy_weight_without_ratio": ("policy_terms", policy_weight_without_ratio),
        "drop_weighted_sum": ("weighted_sum", drop_u),
        "entropy_sign": ("finalize", entropy_sign),
        "denominator_shift": ("denominator", no_shift),
        "label_off_by_one": ("target_logit", label_off_by_one),
        "grad_sign": ("backward", grad_sign),
        "grad_no_weight": ("backward", grad_no_weight),
        "combine_no_rescale": ("combine", combine_no_rescale),
        "combine_no_cross_term": ("combine", combine_no_cross_term),
        "bf16_decode_shift": ("decode", decode_shift15),
        "transposed_max": ("row_max", transposed_max),
        "softmax_wrong_reference": ("softmax_from_lse", softmax_wrong_ref),
    }


@pytest.mark.parametrize("name", sorted(_mutations().keys()))
def test_planted_mistakes(name, monkeypatch):
    attr, fn = _mutations()[name]
    monkeypatch.setattr(orc, attr, fn)
    assert _core_pin_failures(), f"planted mistake {name!r} went unnoticed"


# ------------------------------------------------- clipped-ratio policy terms

def test_policy_terms_closed_cases():
    lo, hi = 0.2, 0.28
    # r = 1 exactly: unclipped, w = c A
    loss, w, cl = orc.policy_terms([-2.0], [-2.0], [1.5], lo, hi, [0.5])
    assert w[0] == 0.75 and loss[0] == -0.75 and not cl[0]
    # A > 0, r above 1 + hi: clipped, no gradient, loss = -c A (1 + hi)
    lp, old = np.log(1.5), 0.0
    loss, w, cl = orc.policy_terms([lp], [old], [2.0], lo, hi)
    assert w[0] == 0.0 and cl[0] and loss[0] == pytest.approx(-2.0 * 1.28)
    # A > 0, r below 1 - lo: unclipped (min picks r A), gradient A r
    loss, w, cl = orc.policy_terms([np.log(0.5)], [0.0], [2.0], lo, hi)
    assert not cl[0] and w[0] == pytest.approx(1.0) and loss[0] == pytest.approx(-1.0)
    # A < 0, r below 1 - lo: clipped; r above 1 + hi: unclipped
    loss, w, cl = orc.policy_terms([np.log(0.5), np.log(1.5)], [0.0, 0.0], [-1.0, -1.0], lo, hi)
    assert cl[0] and w[0] == 0.0 and loss[0] == pytest.approx(0.8)
    assert not cl[1] and w[1] == pytest.approx(-1.5) and loss[1] == pytest.approx(1.5)
    # ignored tokens contribute nothing
    loss, w, _ = orc.policy_terms([0.1], [0.0], [3.0], lo, hi, ignored=[True])
    assert loss[0] == 0.0 and w[0] == 0.0


def test_policy_weight_is_minus_dloss_dlogprob():
    g = np.random.default_rng(3)
    lp = g.normal(-3.0, 1.0, 200)
    old = lp + g.uniform(-0.5, 0.5, 200)
    A = g.normal(0.0, 1.0, 200)
    c = g.uniform(0.1, 1.0, 200)
    h = 1e-7
    lp_p, _, _ = orc.policy_terms(lp + h, old, A, 0.2, 0.28, c)
    lp_m, _, _ = orc.policy_terms(lp - h, old, A, 0.2, 0.28, c)
    _, w, cl = orc.policy_terms(lp, old, A, 0.2, 0.28, c)
    r = np.exp(lp - old)
    far = (np.abs(r - 0.8) > 1e-4) & (np.abs(r - 1.28) > 1e-4)
    fd = -(lp_p - lp_m) / (2 * h)
    np.testing.assert_allclose(w[far], fd[far], rtol=1e-6, atol=1e-9)


def test_policy_gradient_through_the_softmax():
    # d loss / d z = w (p - onehot) with w from policy_terms: finite differences
    g = np.random.default_rng(5)
    V, y = 9, 4
    z = g.standard_normal(V) * 2
    old, A, c = -1.7, 0.8, 0.3

    def loss_of(zz):
        lp, _, _ = fwd1(zz, y)
        return orc.policy_terms([lp], [old], [A], 0.2, 0.28, [c])[0][0]

    lp, _, lse = fwd1(z, y)
    _, w, _ = orc.policy_terms([lp], [old], [A], 0.2, 0.28, [c])
    grad = orc.backward(z[None, :], np.array([y]), np.array([lse]), w)[0]
    for j in range(V):
        zp, zm = z.copy(), z.copy()
        zp[j] += 1e-6
        zm[j] -= 1e-6
        assert grad[j] == pytest.approx((loss_of(zp) - loss_of(zm)) / 2e-6, abs=1e-8)


# ------------------------------------------- label columns and diff metrics

def test_forward_multi_against_brute_force():
    g = np.random.default_rng(12)
    V = 11
    z = g.standard_normal((3, V)) * 2
    z[1, 3] = -np.inf
    labels = np.array([[0, 5, 10, -100], [2, 2, 7, 1], [9, -100, 4, 0]])
    lp, ent, lse = orc.forward_multi(z, labels)
    for i in range(3):
        for k in range(4):
            blp, bh, blse, _ = orc.brute_force(z[i], int(labels[i, k]))
            assert lp[i, k] == pytest.approx(blp, abs=1e-13)
            assert ent[i] == pytest.approx(bh, abs=1e-13) and lse[i] == pytest.approx(blse, abs=1e-13)
    assert lp[0, 3] == 0.0 and not np.signbit(lp[0, 3])
    lp_bad, _, _ = orc.forward_multi(z, np.array([[V, -1, 0, 0]] * 3))
    assert np.isnan(lp_bad[:, :2]).all() and np.isfinite(lp_bad[:, 2:]).all()


def test_diff_stats_closed_cases():
    a = np.array([1.0, 2.0, 3.0, 4.0], dtype=np.float32)
    assert orc.diff_stats(a, a) == (0.0, 0.0, 0.0, 0.0)
    b = np.array([1.0, 2.5, 3.0, 3.0], dtype=np.float32)
    mean, amean, mx, ratio = orc.diff_stats(a, b)
    assert mean == pytest.approx((0 - 0.5 + 0 + 1.0) / 4) and amean == pytest.approx(1.5 / 4)
    assert mx == 1.0 and ratio == 0.5
    # ignored tokens do not count; -0.0 and +0.0 differ bit for bit
    mean, amean, mx, ratio = orc.diff_stats(np.array([0.0, 5.0], np.float32),
                                            np.array([-0.0, 1.0], np.float32), [3, -100])
    assert (mean, amean, mx, ratio) == (0.0, 0.0, 0.0, 1.0)
    assert orc.diff_stats(a, b, [-100] * 4) == (0.0, 0.0, 0.0, 0.0)


# ------------------------------------------------- lm_head projection + stats

def test_lmhead_logits_brute_force_and_one_hot():
    g = np.random.default_rng(21)
    H = g.standard_normal((5, 7))
    W = g.standard_normal((3, 7))
    z = orc.lmhead_logits(H, W)
    for n in range(5):
        for v in range(3):
            assert z[n, v] == pytest.approx(sum(H[n, k] * W[v, k] for k in range(7)), abs=1e-13)
    # one-hot projection rows pick hidden coordinates (a transposed operand fails this)
    W1 = np.zeros((7, 7))
    W1[np.arange(7), (np.arange(7) * 3) % 7] = 1.0
    np.testing.assert_array_equal(orc.lmhead_logits(H, W1), H[:, (np.arange(7) * 3) % 7])


def test_lmhead_tile_stats_combine_to_the_full_row():
    g = np.random.default_rng(22)
    H = g.standard_normal((6, 16))
    W = g.standard_normal((300, 16)) * 0.5
    labels = np.array([0, 299, 128, 127, -100, 200])
    st = orc.lmhead_tile_stats(H, W, labels, 0, 300, 128)
    assert st.shape == (3, 6, 4)
    lp, ent, lse = orc.combine(st, labels, 300)
    flp, fent, flse = orc.forward(orc.lmhead_logits(H, W), labels)
    np.testing.assert_allclose(np.stack([lp, ent, lse]), np.stack([flp, fent, flse]), atol=1e-12)


# ---- lm_head backward: chain rule through the projection

def _lm_loss(H, W, labels, w):
    """sum_n w_n * (-logprob_n) of the lm_head logits (ignored tokens: 0)."""
    lp, _, _ = orc.forward(orc.lmhead_logits(H, W), labels)
    return float(np.sum(w * -lp))


def _lmhead_backward_fd_check(fn):
    g = np.random.default_rng(31)
    n, V, d = 4, 9, 5
    H = g.standard_normal((n, d))
    W = g.standard_normal((V, d)) * 0.7
    labels = np.array([3, 0, -100, 8])
    w = np.array([0.5, -1.25, 2.0, 1.0])
    _, _, lse = orc.forward(orc.lmhead_logits(H, W), labels)
    _, gh, gw = fn(H, W, labels, lse, w)
    eps = 1e-6
    for X, G in ((H, gh), (W, gw)):
        num = np.zeros_like(X)
        for idx in np.ndindex(*X.shape):
            keep = X[idx]
            X[idx] = keep + eps
            up = _lm_loss(H, W, labels, w)
            X[idx] = keep - eps
            dn = _lm_loss(H, W, labels, w)
            X[idx] = keep
            num[idx] = (up - dn) / (2 * eps)
        np.testing.assert_allclose(G, num, rtol=1e-6, atol=1e-7)


def test_lmhead_backward_is_the_finite_difference_gradient():
    _lmhead_backward_fd_check(orc.lmhead_backward)


def test_lmhead_backward_zero_projection_closed_form():
    # W = 0: every logit is 0, softmax is uniform, so grad_hidden = 0 and
    # grad_weight[v] = sum_n w_n (1/V - [v == y_n]) H[n]
    g = np.random.default_rng(32)
    n, V, d = 5, 6, 3
    H = g.standard_normal((n, d))
    W = np.zeros((V, d))
    labels = np.array([1, 5, -100, 0, 1])
    w = g.uniform(0.5, 2.0, n)
    _, _, lse = orc.forward(orc.lmhead_logits(H, W), labels)
    np.testing.assert_allclose(lse, np.log(V), rtol=0, atol=1e-15)
    G, gh, gw = orc.lmhead_backward(H, W, labels, lse, w)
    assert np.all(gh == 0)
    want = np.zeros((V, d))
    for i in range(n):
        if labels[i] == -100:
            continue
        for v in range(V):
            want[v] += w[i] * (1.0 / V - (v == labels[i])) * H[i]
    np.testing.assert_allclose(gw, want, rtol=1e-13, atol=1e-14)


def test_lmhead_backward_ignored_tokens_contribute_nothing():
    g = np.random.default_rng(33)
    H = g.standard_normal((5, 4))
    W = g.standard_normal((7, 4))
    labels = np.array([2, -100, 6, 0, -100])
    _, _, lse = orc.forward(orc.lmhead_logits(H, W), labels)
    _, gh, gw = orc.lmhead_backward(H, W, labels, lse)
    keep = labels != -100
    _, gh2, gw2 = orc.lmhead_backward(H[keep], W, labels[keep], lse[keep])
    assert np.all(gh[~keep] == 0)
    np.testing.assert_allclose(gh[keep], gh2, rtol=0, atol=1e-15)
    np.testing.assert_allclose(gw, gw2, rtol=0, atol=1e-14)


@pytest.mark.parametrize("mistake", ["transposed_weight_grad", "no_onehot", "weight_dropped",
                                     "sign"])
def test_lmhead_backward_planted_mistakes_are_caught(mistake):
    def wrong(H, W, labels, lse, w):
        G, gh, gw = orc.lmhead_backward(H, W, labels, lse, w)
        if mistake == "transposed_weight_grad":
            gw = (G.T @ H)[::-1]
        elif mistake == "no_onehot":
            p = orc.softmax_from_lse(orc.lmhead_logits(H, W), lse)
            G2 = np.where(np.asarray(labels)[:, None] == -100, 0.0, w[:, None] * p)
            gh, gw = G2 @ W, G2.T @ H
        elif mistake == "weight_dropped":
            _, gh, gw = orc.lmhead_backward(H, W, labels, lse, None)
        elif mistake == "sign":
            gh = -gh
        return G, gh, gw
    with pytest.raises(AssertionError):
        _lmhead_backward_fd_check(wrong)

