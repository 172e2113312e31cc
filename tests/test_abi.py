"""The C ABI on the host: the library loads, exports every declared symbol, and
rejects bad arguments with the documented status before touching the device.

These run without a GPU: every call here fails validation on the host, so no
HIP work is ever queued.
"""
import ctypes
import os
import re
import shutil
import subprocess

import pytest

import entropy_bi_logprob_amd as bi

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "bi_logprob.h")

P = ctypes.c_void_p(0x10000)      # a well-aligned stand-in pointer, never dereferenced
P2 = ctypes.c_void_p(0x10002)     # 2-byte aligned
NUL = None


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(bi.library_path()):
        pytest.skip("library not built")
    return bi.lib()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"BI_API\s+[\w\s\*]+?\b(bi_\w+)\s*\(", text)))


def test_header_declares_the_four_entry_points():
    names = declared_functions()
    for fn in ("bi_logprob_fwd", "bi_logprob_bwd", "bi_vocab_chunk_stats", "bi_stats_combine",
               "bi_logprob_fwd_bwd", "bi_policy_loss_fwd_bwd", "bi_logprob_fwd_multi",
               "bi_logprob_diff_stats", "bi_lmhead_tile_stats", "bi_lmhead_tiles",
               "bi_lmhead_tile_rows", "bi_lmhead_grad_logits", "bi_lmhead_backward",
               "bi_lmhead_backward_workspace", "bi_lmhead_backward_noalloc"):
        assert fn in names


def test_every_declared_symbol_is_exported(L):
    for fn in declared_functions():
        assert hasattr(L, fn), fn


def test_status_strings(L):
    for code in range(6):
        assert L.bi_status_string(code)
    assert b"unknown" in L.bi_status_string(99)


def fwd(L, logits=P, dtype=bi.BI_BF16, n=4, v=100, rs=100, labels=P, ign=-100,
        lp=P, ent=P, lse=P, flag=NUL):
    return L.bi_logprob_fwd(logits, dtype, n, v, rs, labels, ign, lp, ent, lse, flag, NUL)


def test_fwd_argument_errors(L):
    assert fwd(L, dtype=7) == bi.BI_ERR_DTYPE
    assert fwd(L, n=-1) == bi.BI_ERR_SHAPE
    assert fwd(L, v=0) == bi.BI_ERR_SHAPE
    assert fwd(L, v=1 << 29, rs=1 << 29) == bi.BI_ERR_SHAPE
    assert fwd(L, rs=99) == bi.BI_ERR_SHAPE
    assert fwd(L, logits=NUL) == bi.BI_ERR_NULL
    assert fwd(L, labels=NUL) == bi.BI_ERR_NULL
    assert fwd(L, lp=NUL, ent=NUL, lse=NUL) == bi.BI_ERR_NULL
    assert fwd(L, logits=P2, dtype=bi.BI_F32) == bi.BI_ERR_ALIGN
    assert fwd(L, labels=ctypes.c_void_p(0x10004)) == bi.BI_ERR_ALIGN
    assert fwd(L, lp=ctypes.c_void_p(0x10001)) == bi.BI_ERR_ALIGN
    assert fwd(L, rs=99) == bi.BI_ERR_SHAPE
    assert b"row_stride" in L.bi_last_error()


def test_fwd_empty_batch_is_a_no_op(L):
    # n_rows == 0 succeeds even with NULL buffers and queues nothing
    assert fwd(L, n=0, logits=NUL, labels=NUL, lp=NUL, ent=NUL, lse=NUL) == bi.BI_OK
    assert L.bi_last_error() == b""


def bwd(L, logits=P, dtype=bi.BI_BF16, n=4, v=100, rs=100, labels=P, ign=-100, lse=P,
        w=NUL, grad=P, gdt=bi.BI_BF16, grs=100, flag=NUL):
    return L.bi_logprob_bwd(logits, dtype, n, v, rs, labels, ign, lse, w, grad, gdt, grs, flag, NUL)


def test_bwd_argument_errors(L):
    assert bwd(L, dtype=bi.BI_F32, gdt=bi.BI_BF16) == bi.BI_ERR_DTYPE
    assert bwd(L, gdt=5) == bi.BI_ERR_DTYPE
    assert bwd(L, grs=50) == bi.BI_ERR_SHAPE
    assert bwd(L, lse=NUL) == bi.BI_ERR_NULL
    assert bwd(L, grad=NUL) == bi.BI_ERR_NULL
    assert bwd(L, grad=P2, gdt=bi.BI_F32) == bi.BI_ERR_ALIGN
    assert bwd(L, w=ctypes.c_void_p(0x10002)) == bi.BI_ERR_ALIGN
    assert bwd(L, n=0, logits=NUL, labels=NUL, lse=NUL, grad=NUL) == bi.BI_OK


def fused(L, logits=P, dtype=bi.BI_BF16, n=4, v=100, rs=100, labels=P, w=NUL, lp=NUL,
          grad=P, gdt=bi.BI_BF16, grs=100, flag=NUL):
    return L.bi_logprob_fwd_bwd(logits, dtype, n, v, rs, labels, -100, w, lp, NUL, NUL, grad, gdt,
                                grs, flag, NUL)


def test_fused_argument_errors(L):
    assert fused(L, dtype=bi.BI_F32, gdt=bi.BI_BF16) == bi.BI_ERR_DTYPE
    assert fused(L, dtype=3) == bi.BI_ERR_DTYPE
    assert fused(L, grs=99) == bi.BI_ERR_SHAPE
    assert fused(L, v=0) == bi.BI_ERR_SHAPE
    assert fused(L, grad=NUL) == bi.BI_ERR_NULL
    assert fused(L, labels=NUL) == bi.BI_ERR_NULL
    assert fused(L, w=ctypes.c_void_p(0x10002)) == bi.BI_ERR_ALIGN
    assert fused(L, lp=ctypes.c_void_p(0x10001)) == bi.BI_ERR_ALIGN
    assert fused(L, n=0, logits=NUL, labels=NUL, grad=NUL) == bi.BI_OK


def test_fused_gradient_must_not_overlap_the_logits(L):
    # 4 rows of 100 bf16 logits at P (bytes [P, P + 800)): the same buffer,
    # the last row's last element, a buffer ending in the first element
    for g in (0x10000, 0x10000 + 3 * 200 + 198, 0x10000 - 3 * 200 - 198):
        assert fused(L, grad=ctypes.c_void_p(g)) == bi.BI_ERR_SHAPE, hex(g)
        assert b"overlaps" in L.bi_last_error()
    assert policy(L, grad=P) == bi.BI_ERR_SHAPE
    assert b"overlaps" in L.bi_last_error()


def policy(L, old=P, adv=P, lo=0.2, hi=0.28, n=4, loss=NUL, grad=P):
    return L.bi_policy_loss_fwd_bwd(P, bi.BI_BF16, n, 100, 100, P, -100, old, adv, NUL, lo, hi,
                                    NUL, NUL, NUL, loss, NUL, grad, bi.BI_BF16, 100, NUL, NUL)


def test_policy_argument_errors(L):
    assert policy(L, lo=1.0) == bi.BI_ERR_SHAPE
    assert policy(L, lo=-0.1) == bi.BI_ERR_SHAPE
    assert policy(L, hi=float("nan")) == bi.BI_ERR_SHAPE
    assert policy(L, old=NUL) == bi.BI_ERR_NULL
    assert policy(L, adv=NUL) == bi.BI_ERR_NULL
    assert policy(L, loss=ctypes.c_void_p(0x10002)) == bi.BI_ERR_ALIGN
    assert policy(L, n=0, old=NUL, adv=NUL) == bi.BI_OK


def test_multi_and_diff_argument_errors(L):
    m = L.bi_logprob_fwd_multi
    assert m(P, bi.BI_BF16, 4, 100, 100, P, 3, 4, -100, P, NUL, NUL, NUL, NUL) == bi.BI_ERR_SHAPE
    assert m(P, bi.BI_BF16, 4, 100, 100, P, 4, 0, -100, P, NUL, NUL, NUL, NUL) == bi.BI_ERR_SHAPE
    assert m(P, bi.BI_BF16, 4, 100, 100, P, 4, 4, -100, NUL, NUL, NUL, NUL, NUL) == bi.BI_ERR_NULL
    assert m(P, 9, 4, 100, 100, P, 4, 4, -100, P, NUL, NUL, NUL, NUL) == bi.BI_ERR_DTYPE
    d = L.bi_logprob_diff_stats
    assert d(P, P, NUL, -100, -1, P, NUL) == bi.BI_ERR_SHAPE
    assert d(P, P, NUL, -100, 10, NUL, NUL) == bi.BI_ERR_NULL
    assert d(NUL, P, NUL, -100, 10, P, NUL) == bi.BI_ERR_NULL
    assert d(P, P, ctypes.c_void_p(0x10004), -100, 10, P, NUL) == bi.BI_ERR_ALIGN


def test_lmhead_argument_errors(L):
    f = L.bi_lmhead_tile_stats
    args = dict(h=P, w=P, n=8, vc=300, d=128, ldh=128, ldw=128, off=0, v=300, lab=P, st=P)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["h"], a["w"], a["n"], a["vc"], a["d"], a["ldh"], a["ldw"], a["off"], a["v"],
                 a["lab"], -100, a["st"], NUL, NUL)

    assert call(d=100) == bi.BI_ERR_SHAPE        # not a multiple of 64
    assert call(d=96) == bi.BI_ERR_SHAPE
    assert call(d=0) == bi.BI_ERR_SHAPE
    assert call(ldh=130) == bi.BI_ERR_SHAPE      # stride not a multiple of 8
    assert call(ldw=(1 << 22) + 8) == bi.BI_ERR_SHAPE   # row pitch past 2^22 elements
    assert call(d=1 << 22, ldh=1 << 22, ldw=(1 << 22) + 8) == bi.BI_ERR_SHAPE
    assert call(d=(1 << 22) + 64, ldh=(1 << 22) + 64, ldw=(1 << 22) + 64) == bi.BI_ERR_SHAPE
    assert call(off=10) == bi.BI_ERR_SHAPE       # rows past the vocabulary
    assert call(h=NUL) == bi.BI_ERR_NULL
    assert call(w=ctypes.c_void_p(0x10008)) == bi.BI_ERR_ALIGN
    assert call(n=0, h=NUL, w=NUL, lab=NUL, st=NUL) == bi.BI_OK
    t = L.bi_lmhead_tile_rows()
    assert t == 256
    assert L.bi_lmhead_tiles(300) == 2 and L.bi_lmhead_tiles(t) == 1 and L.bi_lmhead_tiles(0) == 0
    assert L.bi_lmhead_tiles(t + 1) == 2


def test_lmhead_grad_logits_argument_errors(L):
    f = L.bi_lmhead_grad_logits
    args = dict(h=P, w=P, n=8, vc=300, d=128, ldh=128, ldw=128, off=0, v=300, lab=P, lse=P,
                g=P, ldg=8)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["h"], a["w"], a["n"], a["vc"], a["d"], a["ldh"], a["ldw"], a["off"], a["v"],
                 a["lab"], -100, a["lse"], NUL, a["g"], a["ldg"], NUL, NUL)

    assert call(d=100) == bi.BI_ERR_SHAPE
    assert call(ldg=7) == bi.BI_ERR_SHAPE          # grad stride below n_tokens
    assert call(lse=NUL) == bi.BI_ERR_NULL
    assert call(g=NUL) == bi.BI_ERR_NULL
    assert call(g=ctypes.c_void_p(0x10001)) == bi.BI_ERR_ALIGN
    assert call(n=0, h=NUL, w=NUL, lab=NUL, lse=NUL, g=NUL, ldg=0) == bi.BI_OK


def test_lmhead_backward_argument_errors(L):
    f = L.bi_lmhead_backward
    ws = L.bi_lmhead_backward_workspace
    need = ws(8, 128, 256)
    # one chunk of G: its rows (a multiple of 256) by the tokens padded to 64
    assert need == 256 * 64 * 2 and ws(9, 128, 1) == 256 * 64 * 2
    assert ws(64, 128, 257) == 512 * 64 * 2 and ws(65, 128, 256) == 256 * 128 * 2
    assert ws(1 << 22, 128, 256) == 256 * (1 << 22) * 2
    assert ws(-1, 128, 256) == -1 and ws(8, 128, 0) == -1 and ws(8, -1, 256) == -1
    assert ws((1 << 22) + 1, 128, 256) == -1
    args = dict(h=P, w=P, n=8, vc=300, d=128, ldh=128, ldw=128, off=0, v=300, lab=P, lse=P,
                gh=P, ldgh=128, gw=P, gdt=bi.BI_BF16, ldgw=128, ws=ctypes.c_void_p(0x100000),
                wsb=need)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["h"], a["w"], a["n"], a["vc"], a["d"], a["ldh"], a["ldw"], a["off"], a["v"],
                 a["lab"], -100, a["lse"], NUL, a["gh"], a["ldgh"], a["gw"], a["gdt"], a["ldgw"],
                 a["ws"], a["wsb"], NUL, NUL)

    assert call(gdt=7) == bi.BI_ERR_DTYPE
    assert call(ldgh=100) == bi.BI_ERR_SHAPE       # gradient stride below d
    assert call(n=1 << 31) == bi.BI_ERR_SHAPE
    assert call(n=(1 << 22) + 1) == bi.BI_ERR_SHAPE   # beyond the pipeline's 2^22-element rows
    assert call(ws=NUL) == bi.BI_ERR_NULL
    assert call(gh=NUL) == bi.BI_ERR_NULL
    assert call(ws=ctypes.c_void_p(0x100010)) == bi.BI_ERR_ALIGN
    assert call(wsb=need - 1) == bi.BI_ERR_SHAPE   # not even one 256-row chunk fits
    assert call(n=0) == bi.BI_OK


def chunk(L, logits=P, dtype=bi.BI_BF16, n=4, w=25, rs=100, off=25, v=100, labels=P,
          stats=P, flag=NUL):
    return L.bi_vocab_chunk_stats(logits, dtype, n, w, rs, off, v, labels, -100, stats, flag, NUL)


def test_chunk_requires_the_global_vocabulary(L):
    # the vocabulary-parallel path needs the global vocabulary size
    assert chunk(L, v=0) == bi.BI_ERR_SHAPE
    assert b"global vocabulary size is required" in L.bi_last_error()
    assert chunk(L, off=-1) == bi.BI_ERR_SHAPE
    assert chunk(L, off=80) == bi.BI_ERR_SHAPE        # 80 + 25 > 100
    assert chunk(L, w=0) == bi.BI_ERR_SHAPE
    assert chunk(L, rs=20) == bi.BI_ERR_SHAPE
    assert chunk(L, stats=NUL) == bi.BI_ERR_NULL
    assert chunk(L, stats=ctypes.c_void_p(0x10002)) == bi.BI_ERR_ALIGN


def test_combine_argument_errors(L):
    f = L.bi_stats_combine
    assert f(P, 0, 4, P, -100, P, P, P, NUL) == bi.BI_ERR_SHAPE
    assert f(P, 2, -1, P, -100, P, P, P, NUL) == bi.BI_ERR_SHAPE
    assert f(NUL, 2, 4, P, -100, P, P, P, NUL) == bi.BI_ERR_NULL
    assert f(P, 2, 4, P, -100, NUL, NUL, NUL, NUL) == bi.BI_ERR_NULL
    assert f(P, 2, 0, NUL, -100, NUL, NUL, NUL, NUL) == bi.BI_OK


def test_geometry_depends_on_dtype_and_width_only(L):
    def geo(dt, w):
        a, b, c = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
        assert L.bi_row_geometry(dt, w, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)) == 0
        return a.value, b.value, c.value

    assert geo(bi.BI_BF16, 151_936) == (1024, 8, 2)
    assert geo(bi.BI_F32, 151_936) == (1024, 4, 4)
    assert geo(bi.BI_F32, 151_937) == (1024, 4, 4)
    assert geo(bi.BI_BF16, 37_984)[1:] == (8, 2)
    assert geo(bi.BI_BF16, 16)[0] == 64
    for w in (1, 7, 100, 5000, 151_936):
        t, vec, grp = geo(bi.BI_BF16, w)
        assert t % 64 == 0 and 64 <= t <= 1024 and vec * grp == 16
    assert L.bi_row_geometry(bi.BI_BF16, 0, None, None, None) == bi.BI_ERR_SHAPE


def test_python_binding_rejects_host_tensors():
    import torch
    x = torch.zeros(2, 10, dtype=torch.bfloat16)
    y = torch.zeros(2, dtype=torch.int64)
    with pytest.raises(ValueError):
        bi.fwd(x, y)
    with pytest.raises(ValueError):
        bi.vocab_chunk_stats(x, y, 0, None)


def test_a_c_program_links_and_calls_the_abi(tmp_path):
    # the header as C99 (-pedantic, warnings are errors) and the library linked
    # into a C executable; the program calls host-side entry points only
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    libdir = os.path.dirname(bi.library_path())
    exe = str(tmp_path / "abi_consumer")
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
           "-I", os.path.join(root, "include"), os.path.join(root, "tests", "c", "abi_consumer.c"),
           "-L", libdir, "-lbi_logprob", "-Wl,-rpath," + libdir,
           "-Wl,-rpath-link,/opt/rocm/lib", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ)
    env["LD_LIBRARY_PATH"] = "/opt/rocm/lib:" + env.get("LD_LIBRARY_PATH", "")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=60)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    assert "1024 threads" in r.stdout and "bi_logprob_fwd(n_rows = -1)" in r.stdout


def test_lmhead_backward_noalloc_argument_errors(L):
    # host checks only: every error below returns before the device is touched
    f = L.bi_lmhead_backward_noalloc
    args = dict(n=8, vc=300, d=128, lse=P, gh=P, gw=P, gdt=bi.BI_BF16, ldgh=128)

    def call(**kw):
        a = dict(args, **kw)
        return f(P, P, a["n"], a["vc"], a["d"], 128, 128, 0, a["vc"], P, -100, a["lse"], NUL,
                 a["gh"], a["ldgh"], a["gw"], a["gdt"], 128, NUL, NUL)

    assert call(n=131072 + 1) == bi.BI_ERR_SHAPE          # beyond the static scratch
    assert b"static scratch" in L.bi_last_error()
    assert call(gdt=5) == bi.BI_ERR_DTYPE
    assert call(ldgh=64) == bi.BI_ERR_SHAPE
    assert call(gh=NUL) == bi.BI_ERR_NULL
    assert call(lse=NUL) == bi.BI_ERR_NULL
    assert call(gh=ctypes.c_void_p(0x10002)) == bi.BI_ERR_ALIGN
    assert call(n=0) == bi.BI_OK and call(vc=0) == bi.BI_OK
