"""GPU parity of the lm_head projection fused with the statistics.

bi_lmhead_tile_stats computes the logits hidden @ weight^T on the matrix cores
and reduces them to per-token statistics of 256-row tiles; bi_stats_combine
finishes.  Checked against the fp64 oracle (exact float64 products of the bf16
inputs): per-tile statistics, and the combined logprob / entropy / lse within
2e-4 (the logits are fp32 accumulations of exact bf16 products, so the
fp32-logits tolerance applies).  Also: ragged token and vocabulary tiles, tiles
of a token that do not depend on the batch (bit for bit), and vocabulary
shards that reproduce the unsharded tiles.
"""
import numpy as np
import pytest
import torch

import entropy_bi_logprob_amd as bi
import oracle.bi_oracle as orc
import workloads as wl
from gpu_util import assert_close, dev, host, ulp_bf16

pytestmark = pytest.mark.gpu
TOL = 2e-4


def to_dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def check_tiles(st, ost):
    st = np.asarray(st, dtype=np.float64)
    np.testing.assert_allclose(st[..., 0], ost[..., 0], rtol=0, atol=2e-5)          # max
    np.testing.assert_allclose(st[..., 1], ost[..., 1], rtol=2e-5)                  # sumexp
    np.testing.assert_allclose(st[..., 2], ost[..., 2], rtol=0, atol=2e-5)          # target
    np.testing.assert_allclose(st[..., 3], ost[..., 3], rtol=2e-5, atol=2e-4)       # sumexp_logit


@pytest.mark.parametrize("n,vc,d", [(300, 1000, 128), (128, 128, 64), (77, 333, 256),
                                    (64, 1, 64), (513, 257, 192),
                                    (1000, 4099, 512), (5, 130, 64)])
def test_tiles_and_combine_against_oracle(n, vc, d):
    b = wl.lmhead_batch(n, vc, d, seed=n + vc + d, ignore_frac=0.1)
    H, W, labels = to_dev_bf16(b.hidden), to_dev_bf16(b.weight), dev(b.labels)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    st = bi.lmhead_tile_stats(H, W, labels, status=flag)
    lp, ent, lse = bi.stats_combine(st, labels)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    h = orc.decode(b.hidden, "bf16")
    w = orc.decode(b.weight, "bf16")
    check_tiles(host(st), orc.lmhead_tile_stats(h, w, b.labels, 0, vc, bi.lmhead_tile_rows()))
    olp, oent, olse = orc.forward(orc.lmhead_logits(h, w), b.labels)
    assert_close(host(lp), olp, TOL, "logprob")
    assert_close(host(ent), oent, TOL, "entropy")
    assert_close(host(lse), olse, TOL, "lse")
    ign = b.labels == -100
    assert np.all(host(lp)[ign] == 0) and not np.any(np.signbit(host(lp)[ign]))


@pytest.mark.parametrize("n,vc,d", [(1100, 20000, 128), (700, 30000, 64), (300, 60000, 192)])
def test_many_tiles_per_workgroup(n, vc, d):
    # more tiles than compute units: workgroups run several tiles in turn
    # (K = 64 takes the one-tile-per-workgroup kernel); every tile is checked,
    # and a token's tiles are bit-identical when it is computed alone
    b = wl.lmhead_batch(n, vc, d, seed=n + d, ignore_frac=0.05)
    H, W, labels = to_dev_bf16(b.hidden), to_dev_bf16(b.weight), dev(b.labels)
    st = bi.lmhead_tile_stats(H, W, labels)
    lp, ent, lse = bi.stats_combine(st, labels)
    idx = torch.tensor([n - 1, 0, n // 2], device="cuda")
    sub = bi.lmhead_tile_stats(H[idx].contiguous(), W, labels[idx].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(st[:, idx].contiguous().view(torch.int32), sub.view(torch.int32))
    h = orc.decode(b.hidden, "bf16")
    w = orc.decode(b.weight, "bf16")
    check_tiles(host(st), orc.lmhead_tile_stats(h, w, b.labels, 0, vc, bi.lmhead_tile_rows()))
    olp, oent, olse = orc.forward(orc.lmhead_logits(h, w), b.labels)
    assert_close(host(lp), olp, TOL, "logprob")
    assert_close(host(ent), oent, TOL, "entropy")
    assert_close(host(lse), olse, TOL, "lse")


def test_largest_hidden_size():
    # d = 2^22, the largest the lm_head entry points accept: a load's 32-bit
    # offset from its tile's base reaches 255 rows x 2^23 bytes, and the K loop
    # runs 65,536 stages; 300 lm_head rows make one full and one ragged tile.
    # Sparse +-1 rows keep every logit an exact small integer, so the usual
    # tolerances apply; the oracle sees only the columns that are nonzero
    # somewhere (the others add exact zeros).
    n, vc, d = 8, 300, 1 << 22
    b = wl.sparse_lmhead_batch(n, vc, d, seed=23)
    H, W, labels = to_dev_bf16(b.hidden), to_dev_bf16(b.weight), dev(b.labels)
    cols = np.nonzero((b.hidden != 0).any(axis=0) | (b.weight != 0).any(axis=0))[0]
    assert cols[-1] == d - 1
    h, w = orc.decode(b.hidden[:, cols], "bf16"), orc.decode(b.weight[:, cols], "bf16")
    z = orc.lmhead_logits(h, w)
    olp, oent, olse = orc.forward(z, b.labels)
    lse_in, lse_o = _saved_lse(olse)
    tw = np.full(n, 0.5, dtype=np.float32)
    st = bi.lmhead_tile_stats(H, W, labels)
    lp, ent, lse = bi.stats_combine(st, labels)
    g = bi.lmhead_grad_logits(H, W, labels, lse_in, dev(tw))
    torch.cuda.synchronize()
    check_tiles(host(st), orc.lmhead_tile_stats(h, w, b.labels, 0, vc, bi.lmhead_tile_rows()))
    assert_close(host(lp), olp, TOL, "logprob")
    assert_close(host(ent), oent, TOL, "entropy")
    assert_close(host(lse), olse, TOL, "lse")
    G = orc.backward(z, b.labels, lse_o, tw)
    got = orc.decode(host(g.view(torch.int16)).view(np.uint16), "bf16").T
    assert np.all(np.abs(got - G) <= 1e-5 * 0.5 + ulp_bf16(G))


def test_tiles_do_not_depend_on_the_batch():
    n, vc, d = 640, 1500, 256
    b = wl.lmhead_batch(n, vc, d, seed=3)
    H, W, labels = to_dev_bf16(b.hidden), to_dev_bf16(b.weight), dev(b.labels)
    full = bi.lmhead_tile_stats(H, W, labels)
    idx = torch.tensor([5, 600, 129, 0, 333, 639, 64], device="cuda")
    sub = bi.lmhead_tile_stats(H[idx].contiguous(), W, labels[idx].contiguous())
    one = bi.lmhead_tile_stats(H[idx[1:2]].contiguous(), W, labels[idx[1:2]].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(full[:, idx].contiguous().view(torch.int32), sub.view(torch.int32))
    assert torch.equal(full[:, idx[1:2]].contiguous().view(torch.int32), one.view(torch.int32))


def test_vocabulary_shards_reproduce_the_unsharded_tiles():
    n, vc, d = 200, 1000, 128
    b = wl.lmhead_batch(n, vc, d, seed=5)
    H, W, labels = to_dev_bf16(b.hidden), to_dev_bf16(b.weight), dev(b.labels)
    full = bi.lmhead_tile_stats(H, W, labels)
    # two shards split at a tile boundary: the same tiles, bit for bit
    a = bi.lmhead_tile_stats(H, W[:512].contiguous(), labels, 0, vc)
    c = bi.lmhead_tile_stats(H, W[512:].contiguous(), labels, 512, vc)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([a, c]).view(torch.int32), full.view(torch.int32))
    # a split inside a tile: same combined result within tolerance
    a = bi.lmhead_tile_stats(H, W[:300].contiguous(), labels, 0, vc)
    c = bi.lmhead_tile_stats(H, W[300:].contiguous(), labels, 300, vc)
    lp1, ent1, lse1 = bi.stats_combine(full, labels)
    lp2, ent2, lse2 = bi.stats_combine(torch.cat([a, c]).contiguous(), labels)
    torch.cuda.synchronize()
    for x, y in ((lp1, lp2), (ent1, ent2), (lse1, lse2)):
        assert_close(host(x), host(y), 1e-5, "sharded vs unsharded")


def test_qwen3_vocab_sampled_tokens():
    # the full Qwen3 vocabulary with a Qwen3-4B hidden size, sampled tokens
    n, vc, d = 2048, wl.QWEN3_VOCAB, wl.LMHEAD_HIDDEN
    b = wl.lmhead_batch(n, vc, d, seed=11, ignore_frac=0.02)
    H, W, labels = to_dev_bf16(b.hidden), to_dev_bf16(b.weight), dev(b.labels)
    lp, ent, lse = bi.lmhead_logprob(H, W, labels)
    torch.cuda.synchronize()
    rows = np.array(sorted({0, n - 1, *np.random.default_rng(1).choice(n, 24, replace=False)}))
    z = orc.lmhead_logits(orc.decode(b.hidden[rows], "bf16"), orc.decode(b.weight, "bf16"))
    olp, oent, olse = orc.forward(z, b.labels[rows])
    assert_close(host(lp)[rows], olp, TOL, "logprob")
    assert_close(host(ent)[rows], oent, TOL, "entropy")
    assert_close(host(lse)[rows], olse, TOL, "lse")


# ---- backward: the gradient of the logits, and the two GEMMs

def _setup(n, vc, d, seed, ignore_frac=0.1):
    b = wl.lmhead_batch(n, vc, d, seed=seed, ignore_frac=ignore_frac)
    H, W, labels = to_dev_bf16(b.hidden), to_dev_bf16(b.weight), dev(b.labels)
    h = orc.decode(b.hidden, "bf16")
    w = orc.decode(b.weight, "bf16")
    _, _, olse = orc.forward(orc.lmhead_logits(h, w), b.labels)
    tw = np.random.default_rng([seed, 9]).uniform(-1.5, 1.5, n).astype(np.float32)
    return b, H, W, labels, h, w, olse, tw


def _saved_lse(olse):
    # the lse a forward pass saves, in fp32: the oracle's, so that the GPU
    # backward and the oracle's take the same input
    lse32 = olse.astype(np.float32)
    return dev(lse32), lse32.astype(np.float64)


@pytest.mark.parametrize("n,vc,d", [(300, 1000, 128), (77, 333, 256), (513, 257, 192),
                                    (5, 130, 64)])
def test_grad_logits_against_oracle(n, vc, d):
    b, H, W, labels, h, w, olse, tw = _setup(n, vc, d, seed=n + vc)
    lse, lse_o = _saved_lse(olse)
    g = bi.lmhead_grad_logits(H, W, labels, lse, dev(tw))
    torch.cuda.synchronize()
    G, _, _ = orc.lmhead_backward(h, w, b.labels, lse_o, tw)
    got = orc.decode(host(g.view(torch.int16)).view(np.uint16), "bf16").T   # [n, vc]
    # fp32 logits: |dp| <~ 1e-5 p; then one bf16 rounding (at most one ulp of
    # the exact value, whichever binade the computed value falls in)
    bound = 1e-5 * np.abs(tw)[:, None] + ulp_bf16(G)
    assert np.all(np.abs(got - G) <= bound), float(np.max(np.abs(got - G) - bound))
    ign = b.labels == -100
    assert np.all(got[ign] == 0) and not np.any(np.signbit(got[ign]))


def test_grad_logits_bad_label_is_nan_and_flagged():
    b, H, W, labels, h, w, olse, tw = _setup(8, 300, 64, seed=4, ignore_frac=0.0)
    lab = b.labels.copy()
    lab[3] = 300 + 7
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    g = bi.lmhead_grad_logits(H, W, dev(lab), dev(olse.astype(np.float32)), status=flag)
    torch.cuda.synchronize()
    gf = host(g.float())
    assert int(flag.item()) == bi.BI_FLAG_BAD_LABEL
    assert np.isnan(gf[:, 3]).all() and np.isfinite(np.delete(gf, 3, axis=1)).all()


def test_ignore_index_that_is_a_vocabulary_row():
    # ignore_index 7 is also a row of the lm_head: tokens labelled 7 are
    # ignored (logprob and gradient +0, no onehot term at row 7), and row 7
    # still gets every other token's softmax term
    n, vc, d, ii = 300, 700, 128, 7
    b, H, W, _, h, w, olse, tw = _setup(n, vc, d, seed=31, ignore_frac=0.0)
    lab = np.where(b.labels == ii, ii + 1, b.labels)
    lab[np.random.default_rng(3).choice(n, 40, replace=False)] = ii
    ign = lab == ii
    lp, ent, lse = bi.lmhead_logprob(H, W, dev(lab), ignore_index=ii)
    torch.cuda.synchronize()
    olp, oent, olse2 = orc.forward(orc.lmhead_logits(h, w), lab, ignore_index=ii)
    assert_close(host(lp), olp, TOL, "logprob")
    assert_close(host(ent), oent, TOL, "entropy")
    assert_close(host(lse), olse2, TOL, "lse")
    assert np.all(host(lp)[ign] == 0) and not np.any(np.signbit(host(lp)[ign]))
    lse_d, lse_o = _saved_lse(olse)
    g = bi.lmhead_grad_logits(H, W, dev(lab), lse_d, dev(tw), ignore_index=ii)
    gh, gw = bi.lmhead_backward(H, W, dev(lab), lse_d, dev(tw), ignore_index=ii,
                                grad_weight_dtype=torch.float32)
    torch.cuda.synchronize()
    G = orc.lmhead_backward(h, w, lab, lse_o, tw, ignore_index=ii)
    got = orc.decode(host(g.view(torch.int16)).view(np.uint16), "bf16").T   # [n, vc]
    bound = 1e-5 * np.abs(tw)[:, None] + ulp_bf16(G[0])
    assert np.all(np.abs(got - G[0]) <= bound), float(np.max(np.abs(got - G[0]) - bound))
    assert np.all(got[ign] == 0) and not np.any(np.signbit(got[ign]))
    _check_grads(host(gh), host(gw), G, h, w, False)


def _check_grads(gh, gw, G, h, w, gw_bf16):
    """|error| within bf16 rounding of G (2^-9 relative) plus fp32 accumulation,
    bounded through the absolute products: (2^-8 + K 2^-24) |G| @ |operand|."""
    _, oh, ow = G
    Gm = G[0]
    kv, kn = Gm.shape[1], Gm.shape[0]
    bh = (2.0 ** -8 + kv * 2.0 ** -24) * (np.abs(Gm) @ np.abs(w)) + 1e-7
    bw = (2.0 ** -8 + kn * 2.0 ** -24) * (np.abs(Gm).T @ np.abs(h)) + 1e-7
    if gw_bf16:
        bw = bw + 0.5 * ulp_bf16(ow)
    eh, ew = np.abs(gh - oh), np.abs(gw - ow)
    assert np.all(eh <= bh), float(np.max(eh - bh))
    assert np.all(ew <= bw), float(np.max(ew - bw))


@pytest.mark.parametrize("n,vc,d,chunk", [(300, 1000, 128, 256), (77, 333, 256, 16384),
                                          (513, 1030, 192, 512), (5, 130, 64, 256)])
@pytest.mark.parametrize("gdt", [torch.float32, torch.bfloat16], ids=["gw_f32", "gw_bf16"])
def test_backward_against_oracle(n, vc, d, chunk, gdt):
    b, H, W, labels, h, w, olse, tw = _setup(n, vc, d, seed=n + d)
    lse, lse_o = _saved_lse(olse)
    gh, gw = bi.lmhead_backward(H, W, labels, lse, dev(tw), grad_weight_dtype=gdt,
                                chunk_rows=chunk)
    torch.cuda.synchronize()
    G = orc.lmhead_backward(h, w, b.labels, lse_o, tw)
    _check_grads(host(gh), host(gw.float()), G, h, w, gdt == torch.bfloat16)


@pytest.mark.parametrize("n,vc,d,pad", [(256, 1000, 128, 0), (300, 1030, 192, 0),
                                        (77, 700, 128, 64)])
@pytest.mark.parametrize("gdt", [torch.float32, torch.bfloat16], ids=["gw_f32", "gw_bf16"])
def test_backward_workspace_sizes(n, vc, d, pad, gdt):
    # every token count runs on the matrix-core pipeline: G is padded with zero
    # columns to a whole 64-deep K stage (the workspace starts as NaN bytes, so
    # a padding column left unwritten would show).  Workspaces of one 256-row
    # chunk, of a chunk that does not divide the shard, one byte short of a
    # chunk, and of the whole shard: grad_weight is the same bits for every
    # chunking (each row is one product), grad_hidden (summed over chunks in
    # their order) meets the bound each time
    b, H, W, labels, h, w, olse, tw = _setup(n, vc, d, seed=n + d + pad)
    if pad:
        H = _padded(H, pad)
    lse, lse_o = _saved_lse(olse)
    G = orc.lmhead_backward(h, w, b.labels, lse_o, tw)
    one = int(bi.lib().bi_lmhead_backward_workspace(n, d, 256))
    assert one == 256 * (-(-n // 64) * 64) * 2
    gws = []
    for wsb in (one, 3 * one - 1, int(bi.lib().bi_lmhead_backward_workspace(n, d, vc))):
        ws = torch.full((wsb,), 255, dtype=torch.uint8, device="cuda")
        gh, gw = bi.lmhead_backward(H, W, labels, lse, dev(tw), grad_weight_dtype=gdt,
                                    workspace=ws)
        torch.cuda.synchronize()
        _check_grads(host(gh), host(gw.float()), G, h, w, gdt == torch.bfloat16)
        gws.append(gw)
    for other in gws[1:]:
        assert torch.equal(gws[0].view(torch.int16 if gdt == torch.bfloat16 else torch.int32),
                           other.view(torch.int16 if gdt == torch.bfloat16 else torch.int32))
    ws = torch.empty(one - 1, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        bi.lmhead_backward(H, W, labels, lse, dev(tw), workspace=ws)


def _padded(t, extra):
    # the same values in rows `extra` elements longer (a column slice of a wider buffer)
    wide = torch.zeros((t.shape[0], t.shape[1] + extra), dtype=t.dtype, device=t.device)
    wide[:, :t.shape[1]] = t
    return wide[:, :t.shape[1]]


def test_padded_row_strides_give_the_same_bits():
    n, vc, d = 300, 1000, 192
    b, H, W, labels, h, w, olse, tw = _setup(n, vc, d, seed=17)
    Hp, Wp = _padded(H, 64), _padded(W, 136)
    assert Hp.stride(0) == d + 64 and Wp.stride(0) == d + 136
    st = bi.lmhead_tile_stats(H, W, labels)
    stp = bi.lmhead_tile_stats(Hp, Wp, labels)
    lse, lse_o = _saved_lse(olse)
    twd = dev(tw)
    g = bi.lmhead_grad_logits(H, W, labels, lse, twd)
    gp = bi.lmhead_grad_logits(Hp, Wp, labels, lse, twd)
    # gradient rows padded too: a stride that is a multiple of 8 (16-byte
    # vector stores) and an odd one (the element path, as for n = 300 itself)
    g8 = _padded(torch.empty_like(g), 44)
    g3 = _padded(torch.empty_like(g), 3)
    assert g8.stride(0) % 8 == 0 and g3.stride(0) % 2 == 1
    bi.lmhead_grad_logits(H, W, labels, lse, twd, out=g8)
    bi.lmhead_grad_logits(H, W, labels, lse, twd, out=g3)
    torch.cuda.synchronize()
    assert torch.equal(st.view(torch.int32), stp.view(torch.int32))
    for other in (gp, g8, g3):
        assert torch.equal(g.contiguous().view(torch.int16), other.contiguous().view(torch.int16))
    # the backward with padded operands
    gh, gw = bi.lmhead_backward(Hp, Wp, labels, lse, twd, chunk_rows=512)
    torch.cuda.synchronize()
    G = orc.lmhead_backward(h, w, b.labels, lse_o, tw)
    _check_grads(host(gh), host(gw.float()), G, h, w, True)


def test_backward_accumulates_over_vocabulary_shards():
    n, vc, d = 200, 1000, 128
    b, H, W, labels, h, w, olse, tw = _setup(n, vc, d, seed=17)
    lse, lse_o = _saved_lse(olse)
    twd = dev(tw)
    gh_full, gw_full = bi.lmhead_backward(H, W, labels, lse, twd, grad_weight_dtype=torch.float32)
    # two shards (one split inside a 256-row tile) adding into one grad_hidden
    gh = torch.zeros((n, d), dtype=torch.float32, device="cuda")
    _, gwa = bi.lmhead_backward(H, W[:300].contiguous(), labels, lse, twd, 0, vc, grad_hidden=gh,
                                grad_weight_dtype=torch.float32)
    _, gwb = bi.lmhead_backward(H, W[300:].contiguous(), labels, lse, twd, 300, vc,
                                grad_hidden=gh, grad_weight_dtype=torch.float32)
    torch.cuda.synchronize()
    G = orc.lmhead_backward(h, w, b.labels, lse_o, tw)
    _check_grads(host(gh), host(torch.cat([gwa, gwb])), G, h, w, False)
    _check_grads(host(gh_full), host(gw_full), G, h, w, False)


def test_autograd_through_the_lm_head():
    n, vc, d = 130, 700, 128
    b, H, W, labels, h, w, olse, tw = _setup(n, vc, d, seed=23)
    Hp = H.clone().requires_grad_(True)
    Wp = W.clone().requires_grad_(True)
    lp, ent = bi.lmhead_logprob_entropy(Hp, Wp, labels)
    coef = torch.from_numpy(tw).cuda()
    (lp * coef).sum().backward()
    torch.cuda.synchronize()
    # d(sum c lp)/dz = c (onehot - p): the backward with token weights -c
    G = orc.lmhead_backward(h, w, b.labels, olse, -tw)
    # the hidden gradient comes back in bf16 (the hidden dtype)
    gh = host(Hp.grad.float())
    gw = host(Wp.grad.float())
    _, oh, ow = G
    bh = (2.0 ** -8 + vc * 2.0 ** -24) * (np.abs(G[0]) @ np.abs(w)) + 0.5 * ulp_bf16(oh) + 1e-6
    bw = (2.0 ** -8 + n * 2.0 ** -24) * (np.abs(G[0]).T @ np.abs(h)) + 0.5 * ulp_bf16(ow) + 1e-6
    assert np.all(np.abs(gh - oh) <= bh) and np.all(np.abs(gw - ow) <= bw)
    olp, oent, _ = orc.forward(orc.lmhead_logits(h, w), b.labels)
    assert_close(host(lp.detach()), olp, TOL, "logprob")
    assert_close(host(ent), oent, TOL, "entropy")



# ---- the full-size lm_head step, sampled

def _vocab_columns_backward(h, w, labels, lse, tw, cols):
    """Columns `cols` of G = w (softmax - onehot) and the grad_weight rows
    G[:, cols]^T @ hidden, from the oracle's logits and backward.  The
    softmax of a column needs only its logit and the row's saved lse; one
    extra column at -inf takes the onehot of every label outside `cols`
    (its probability is exactly 0), so the kept columns are the full
    matrix's."""
    z = np.concatenate([orc.lmhead_logits(h, w[cols]), np.full((h.shape[0], 1), -np.inf)], axis=1)
    pos = {int(c): i for i, c in enumerate(cols)}
    lab = np.array([pos.get(int(y), len(cols)) if y != -100 else -100 for y in labels])
    G = orc.backward(z, lab, lse, tw)[:, :len(cols)]
    return G, G.T @ h


@pytest.mark.timeout(900)
def test_bench_shape_sampled():
    # 32768 tokens, the Qwen3 vocabulary, hidden size 2560: the statistics and
    # the backward launched as the throughput benchmark launches them (one
    # 32768-row chunk, a mean over tokens, grad_weight in bf16, the product on
    # the lm_head kernel).  A grad_hidden row needs the token's whole logit
    # row, a grad_weight row one logit column over every token: the oracle
    # checks sampled tokens and sampled vocabulary rows (both tile edges, the
    # ragged last tile, and the labels of sampled tokens for the onehot term).
    n, vc, d = 32768, wl.QWEN3_VOCAB, wl.LMHEAD_HIDDEN
    b = wl.lmhead_batch(n, vc, d, seed=19)
    H, W, labels = to_dev_bf16(b.hidden), to_dev_bf16(b.weight), dev(b.labels)
    lp, ent, lse = bi.lmhead_logprob(H, W, labels)
    h, w = orc.decode(b.hidden, "bf16"), orc.decode(b.weight, "bf16")
    # the saved lse, a seeded stand-in near each row's normaliser: the logits
    # of these inputs are Gaussian with variance 4 |h|^2 / d, so sum exp(z)
    # is about vc exp(2 |h|^2 / d)
    lse32 = (np.log(vc) + 2.0 * np.mean(h * h, axis=1)).astype(np.float32)
    lse_o = lse32.astype(np.float64)
    tw = np.full(n, -1.0 / n, dtype=np.float32)
    ws = torch.empty(int(bi.lib().bi_lmhead_backward_workspace(n, d, n)), dtype=torch.uint8,
                     device="cuda")
    gh = torch.zeros((n, d), dtype=torch.float32, device="cuda")
    gw = torch.empty((vc, d), dtype=torch.bfloat16, device="cuda")
    bi.lmhead_backward(H, W, labels, dev(lse32), dev(tw), grad_hidden=gh, grad_weight=gw,
                       chunk_rows=n, workspace=ws)
    torch.cuda.synchronize()
    del ws

    rng = np.random.default_rng(20)
    rows = np.array(sorted({0, 1, n - 1, *rng.choice(n, 13, replace=False)}))
    olp, oent, olse = orc.forward(orc.lmhead_logits(h[rows], w), b.labels[rows])
    assert_close(host(lp)[rows], olp, TOL, "logprob")
    assert_close(host(ent)[rows], oent, TOL, "entropy")
    assert_close(host(lse)[rows], olse, TOL, "lse")

    G, oh, _ = orc.lmhead_backward(h[rows], w, b.labels[rows], lse_o[rows], tw[rows])
    bh = (2.0 ** -8 + vc * 2.0 ** -24) * (np.abs(G) @ np.abs(w)) + 1e-7
    eh = np.abs(host(gh)[rows] - oh)
    assert np.all(eh <= bh), float(np.max(eh - bh))

    last = vc - vc % 256 if vc % 256 else vc - 256
    cols = np.array(sorted({0, 255, 256, last - 1, last, vc - 1,
                            *b.labels[rows[:6]], *rng.choice(vc, 6, replace=False)}))
    G, ow = _vocab_columns_backward(h, w, b.labels, lse_o, tw, cols)
    assert np.count_nonzero(np.isin(b.labels, cols)) >= 6
    bw = (2.0 ** -8 + n * 2.0 ** -24) * (np.abs(G).T @ np.abs(h)) + 1e-7 + 0.5 * ulp_bf16(ow)
    ew = np.abs(host(gw[torch.from_numpy(cols).cuda()].float()) - ow)
    assert np.all(ew <= bw), float(np.max(ew - bw))
