"""Batch-invariant per-token logprob, entropy and gradient for MI355X (gfx950).

A thin Python binding over the C ABI of ``libbi_logprob.so``
(include/bi_logprob.h).  Every step of the computation runs in that library's
HIP kernels; PyTorch only provides device memory and the current stream.  There
is no fallback: if the library is missing, importing the binding's entry points
raises.

What is computed follows "[RL] Avoid full-vocab gather for TP policy
statistics" (torchtitan PR #4685): per-token logprob (negated per-token
cross-entropy) and exact entropy from full rows, the gradient
``w * (softmax - onehot)``, and vocabulary-chunk statistics that combine
exactly (sections Summary, Why, Correctness and compatibility).
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Optional, Tuple

import torch  # first: the library then binds to the HIP runtime torch has loaded

__all__ = [
    "IGNORE_INDEX", "BiError", "fwd", "bwd", "fwd_bwd", "policy_loss_fwd_bwd", "vocab_chunk_stats", "stats_combine",
    "row_geometry", "fwd_multi", "diff_stats", "lmhead_tile_stats", "lmhead_logprob",
    "lmhead_tile_rows", "lmhead_grad_logits", "lmhead_backward", "lmhead_backward_noalloc",
    "lmhead_logprob_entropy",
    "LogprobEntropy", "logprob_entropy", "lib",
    "library_path",
]

IGNORE_INDEX = -100
BI_F32, BI_BF16 = 0, 1
BI_OK, BI_ERR_NULL, BI_ERR_SHAPE, BI_ERR_DTYPE, BI_ERR_ALIGN, BI_ERR_LAUNCH = range(6)
BI_FLAG_BAD_LABEL = 1
STATS_FIELDS = ("max", "sumexp", "target", "sumexp_logit")

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libbi_logprob.so"
_lib = None


class BiError(RuntimeError):
    """A call into libbi_logprob failed."""

    def __init__(self, fn: str, status: int, detail: str):
        self.status = status
        super().__init__(f"{fn}: status {status} ({detail})")


def library_path() -> str:
    return os.path.join(_HERE, _LIB_NAME)


def _hip_runtimes_mapped():
    paths = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    paths.add(os.path.realpath(line.split()[-1]))
    except OSError:  # pragma: no cover
        pass
    return paths


def lib() -> ctypes.CDLL:
    """Load the HIP library once (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python -m entropy_bi_logprob_amd.build` "
            "(or __graft_entry__.build()); there is no fallback implementation")
    L = ctypes.CDLL(path)
    runtimes = _hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise ImportError(f"two HIP runtimes are mapped into this process: {sorted(runtimes)}")
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.bi_logprob_fwd.argtypes = [vp, i32, i64, i64, i64, vp, i64, vp, vp, vp, vp, vp]
    L.bi_logprob_bwd.argtypes = [vp, i32, i64, i64, i64, vp, i64, vp, vp, vp, i32, i64, vp, vp]
    L.bi_logprob_fwd_bwd.argtypes = [vp, i32, i64, i64, i64, vp, i64, vp, vp, vp, vp, vp, i32,
                                     i64, vp, vp]
    f32 = ctypes.c_float
    L.bi_policy_loss_fwd_bwd.argtypes = [vp, i32, i64, i64, i64, vp, i64, vp, vp, vp, f32, f32,
                                         vp, vp, vp, vp, vp, vp, i32, i64, vp, vp]
    L.bi_vocab_chunk_stats.argtypes = [vp, i32, i64, i64, i64, i64, i64, vp, i64, vp, vp, vp]
    L.bi_logprob_fwd_multi.argtypes = [vp, i32, i64, i64, i64, vp, i64, i64, i64, vp, vp, vp,
                                       vp, vp]
    L.bi_logprob_diff_stats.argtypes = [vp, vp, vp, i64, i64, vp, vp]
    L.bi_lmhead_tile_stats.argtypes = [vp, vp, i64, i64, i64, i64, i64, i64, i64, vp, i64, vp,
                                       vp, vp]
    L.bi_lmhead_tile_stats.restype = i32
    L.bi_lmhead_tiles.argtypes = [i64]
    L.bi_lmhead_tiles.restype = i64
    L.bi_lmhead_tile_rows.argtypes = []
    L.bi_lmhead_tile_rows.restype = i64
    L.bi_lmhead_grad_logits.argtypes = [vp, vp, i64, i64, i64, i64, i64, i64, i64, vp, i64, vp,
                                        vp, vp, i64, vp, vp]
    L.bi_lmhead_grad_logits.restype = i32
    L.bi_lmhead_backward.argtypes = [vp, vp, i64, i64, i64, i64, i64, i64, i64, vp, i64, vp, vp,
                                     vp, i64, vp, i32, i64, vp, i64, vp, vp]
    L.bi_lmhead_backward.restype = i32
    L.bi_lmhead_backward_noalloc.argtypes = [vp, vp, i64, i64, i64, i64, i64, i64, i64, vp,
                                             i64, vp, vp, vp, i64, vp, i32, i64, vp, vp]
    L.bi_lmhead_backward_noalloc.restype = i32
    L.bi_lmhead_backward_workspace.argtypes = [i64, i64, i64]
    L.bi_lmhead_backward_workspace.restype = i64
    L.bi_stats_combine.argtypes = [vp, i64, i64, vp, i64, vp, vp, vp, vp]
    L.bi_row_geometry.argtypes = [i32, i64, ctypes.POINTER(i32), ctypes.POINTER(i32),
                                  ctypes.POINTER(i32)]
    for fn in ("bi_logprob_fwd", "bi_logprob_bwd", "bi_logprob_fwd_bwd",
               "bi_policy_loss_fwd_bwd", "bi_vocab_chunk_stats", "bi_logprob_fwd_multi",
               "bi_logprob_diff_stats",
               "bi_stats_combine", "bi_row_geometry"):
        getattr(L, fn).restype = i32
    L.bi_status_string.argtypes = [i32]
    L.bi_status_string.restype = ctypes.c_char_p
    L.bi_last_error.argtypes = []
    L.bi_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(fn: str, status: int) -> None:
    if status == BI_OK:
        return
    L = lib()
    detail = (L.bi_last_error() or b"").decode() or L.bi_status_string(status).decode()
    if status == BI_ERR_LAUNCH:
        raise BiError(fn, status, detail)
    raise ValueError(f"{fn}: {detail}")


# ----------------------------------------------------------------- marshalling

def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return BI_F32
    if dt == torch.bfloat16:
        return BI_BF16
    raise ValueError(f"logits must be float32 or bfloat16, got {dt}")


def _rows(t: torch.Tensor, name: str) -> Tuple[int, int, int]:
    """(n_rows, width, row_stride) of a 2-D device tensor with a contiguous last dim."""
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D [rows, width], got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    n, w = t.shape
    if w > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have a contiguous last dimension")
    return n, w, (t.stride(0) if n > 1 else w)


def _vec(t: Optional[torch.Tensor], n: int, dtype: torch.dtype, name: str):
    if t is None:
        return None
    if t.dtype != dtype or t.dim() != 1 or t.shape[0] != n or not t.is_cuda:
        raise ValueError(f"{name} must be a device {dtype} vector of length {n}")
    if n > 1 and t.stride(0) != 1:
        raise ValueError(f"{name} must be contiguous")
    return t


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


@contextlib.contextmanager
def _on_stream(stream):
    """Make ``stream`` (torch's current stream when None; a torch stream or a raw
    hipStream_t) current while a wrapper allocates, fills and launches, and yield
    its handle.  Tensors the wrapper allocates (outputs, a zero-filled
    grad_hidden, workspaces and intermediate statistics) then belong to that
    stream: their fills are ordered before the library's kernels, and the
    caching allocator hands their memory to other work only after everything
    queued on that stream before the release."""
    if stream is None:
        s = torch.cuda.current_stream()
    elif isinstance(stream, torch.cuda.Stream):
        s = stream
    else:
        s = torch.cuda.ExternalStream(int(getattr(stream, "cuda_stream", stream)))
    with torch.cuda.stream(s):
        yield ctypes.c_void_p(s.cuda_stream)


# ------------------------------------------------------------------ entry points

def fwd(logits: torch.Tensor, labels: torch.Tensor, ignore_index: int = IGNORE_INDEX, *,
        out: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None,
        status: Optional[torch.Tensor] = None, stream=None):
    """(logprob, entropy, lse) fp32 [N] for full rows of ``logits`` [N, V]."""
    n, v, rs = _rows(logits, "logits")
    _vec(labels, n, torch.int64, "labels")
    _vec(status, 1, torch.int32, "status")
    with _on_stream(stream) as hs:
        if out is None:
            out = tuple(torch.empty(n, dtype=torch.float32, device=logits.device)
                        for _ in range(3))
        lp, ent, lse = (_vec(o, n, torch.float32, "out") for o in out)
        _check("bi_logprob_fwd", lib().bi_logprob_fwd(
            _ptr(logits), _dtype_code(logits.dtype), n, v, rs, _ptr(labels), ignore_index,
            _ptr(lp), _ptr(ent), _ptr(lse), _ptr(status), hs))
    return lp, ent, lse


def bwd(logits: torch.Tensor, labels: torch.Tensor, lse: torch.Tensor,
        weights: Optional[torch.Tensor] = None, grad_dtype: Optional[torch.dtype] = None,
        ignore_index: int = IGNORE_INDEX, *, out: Optional[torch.Tensor] = None,
        status: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """grad [N, V] = w * (softmax - onehot(label)) from the saved lse."""
    n, v, rs = _rows(logits, "logits")
    _vec(labels, n, torch.int64, "labels")
    _vec(lse, n, torch.float32, "lse")
    _vec(weights, n, torch.float32, "weights")
    _vec(status, 1, torch.int32, "status")
    with _on_stream(stream) as hs:
        if out is None:
            out = torch.empty((n, v), dtype=grad_dtype or logits.dtype, device=logits.device)
        gn, gv, grs = _rows(out, "grad")
        if (gn, gv) != (n, v):
            raise ValueError("grad must have the logits' shape")
        _check("bi_logprob_bwd", lib().bi_logprob_bwd(
            _ptr(logits), _dtype_code(logits.dtype), n, v, rs, _ptr(labels), ignore_index,
            _ptr(lse), _ptr(weights), _ptr(out), _dtype_code(out.dtype), grs, _ptr(status), hs))
    return out


def fwd_bwd(logits: torch.Tensor, labels: torch.Tensor, weights: Optional[torch.Tensor] = None,
            grad_dtype: Optional[torch.dtype] = None, ignore_index: int = IGNORE_INDEX, *,
            out=None, grad: Optional[torch.Tensor] = None, status: Optional[torch.Tensor] = None,
            stream=None):
    """(logprob, entropy, lse, grad) in one pass over each row (weights known up front).

    Bit-identical to ``fwd`` followed by ``bwd`` with the same weights.
    """
    n, v, rs = _rows(logits, "logits")
    _vec(labels, n, torch.int64, "labels")
    _vec(weights, n, torch.float32, "weights")
    _vec(status, 1, torch.int32, "status")
    with _on_stream(stream) as hs:
        if out is None:
            out = tuple(torch.empty(n, dtype=torch.float32, device=logits.device)
                        for _ in range(3))
        lp, ent, lse = (_vec(o, n, torch.float32, "out") for o in out)
        if grad is None:
            grad = torch.empty((n, v), dtype=grad_dtype or logits.dtype, device=logits.device)
        gn, gv, grs = _rows(grad, "grad")
        if (gn, gv) != (n, v):
            raise ValueError("grad must have the logits' shape")
        _check("bi_logprob_fwd_bwd", lib().bi_logprob_fwd_bwd(
            _ptr(logits), _dtype_code(logits.dtype), n, v, rs, _ptr(labels), ignore_index,
            _ptr(weights), _ptr(lp), _ptr(ent), _ptr(lse), _ptr(grad), _dtype_code(grad.dtype),
            grs, _ptr(status), hs))
    return lp, ent, lse, grad


def policy_loss_fwd_bwd(logits: torch.Tensor, labels: torch.Tensor, old_logprob: torch.Tensor,
                        advantages: torch.Tensor, clip_low: float = 0.2, clip_high: float = 0.28,
                        loss_scale: Optional[torch.Tensor] = None,
                        grad_dtype: Optional[torch.dtype] = None,
                        ignore_index: int = IGNORE_INDEX, *, grad: Optional[torch.Tensor] = None,
                        status: Optional[torch.Tensor] = None, stream=None):
    """Clipped-ratio policy loss in one pass over each row.

    Returns (logprob, entropy, lse, loss, weight, grad): per-token fp32 vectors
    and the gradient of the loss with respect to the logits.
    """
    n, v, rs = _rows(logits, "logits")
    _vec(labels, n, torch.int64, "labels")
    _vec(old_logprob, n, torch.float32, "old_logprob")
    _vec(advantages, n, torch.float32, "advantages")
    _vec(loss_scale, n, torch.float32, "loss_scale")
    _vec(status, 1, torch.int32, "status")
    with _on_stream(stream) as hs:
        outs = tuple(torch.empty(n, dtype=torch.float32, device=logits.device)
                     for _ in range(5))
        if grad is None:
            grad = torch.empty((n, v), dtype=grad_dtype or logits.dtype, device=logits.device)
        gn, gv, grs = _rows(grad, "grad")
        if (gn, gv) != (n, v):
            raise ValueError("grad must have the logits' shape")
        lp, ent, lse, loss, w = outs
        _check("bi_policy_loss_fwd_bwd", lib().bi_policy_loss_fwd_bwd(
            _ptr(logits), _dtype_code(logits.dtype), n, v, rs, _ptr(labels), ignore_index,
            _ptr(old_logprob), _ptr(advantages), _ptr(loss_scale), float(clip_low),
            float(clip_high), _ptr(lp), _ptr(ent), _ptr(lse), _ptr(loss), _ptr(w), _ptr(grad),
            _dtype_code(grad.dtype), grs, _ptr(status), hs))
    return lp, ent, lse, loss, w, grad


def vocab_chunk_stats(logits_chunk: torch.Tensor, labels: torch.Tensor, vocab_offset: int,
                      vocab: Optional[int], ignore_index: int = IGNORE_INDEX, *,
                      out: Optional[torch.Tensor] = None, status: Optional[torch.Tensor] = None,
                      stream=None) -> torch.Tensor:
    """[N, 4] fp32 statistics (max, sumexp, target, sumexp_logit) of one chunk.

    ``logits_chunk`` is the [N, W] view of global columns
    [vocab_offset, vocab_offset + W); ``vocab`` is the global vocabulary size
    and is required.
    """
    if vocab is None:
        raise ValueError("the global vocabulary size is required for vocabulary-chunk statistics")
    n, w, rs = _rows(logits_chunk, "logits_chunk")
    _vec(labels, n, torch.int64, "labels")
    _vec(status, 1, torch.int32, "status")
    with _on_stream(stream) as hs:
        if out is None:
            out = torch.empty((n, 4), dtype=torch.float32, device=logits_chunk.device)
        if out.shape != (n, 4) or out.dtype != torch.float32 or not out.is_contiguous():
            raise ValueError("out must be a contiguous float32 [N, 4] tensor")
        _check("bi_vocab_chunk_stats", lib().bi_vocab_chunk_stats(
            _ptr(logits_chunk), _dtype_code(logits_chunk.dtype), n, w, rs, vocab_offset, vocab,
            _ptr(labels), ignore_index, _ptr(out), _ptr(status), hs))
    return out


def stats_combine(stats: torch.Tensor, labels: torch.Tensor, ignore_index: int = IGNORE_INDEX, *,
                  out=None, stream=None):
    """Combine [C, N, 4] chunk statistics in chunk order -> (logprob, entropy, lse)."""
    if stats.dim() != 3 or stats.shape[2] != 4 or stats.dtype != torch.float32 \
            or not stats.is_contiguous() or not stats.is_cuda:
        raise ValueError("stats must be a contiguous device float32 [C, N, 4] tensor")
    c, n, _ = stats.shape
    _vec(labels, n, torch.int64, "labels")
    with _on_stream(stream) as hs:
        if out is None:
            out = tuple(torch.empty(n, dtype=torch.float32, device=stats.device)
                        for _ in range(3))
        lp, ent, lse = (_vec(o, n, torch.float32, "out") for o in out)
        _check("bi_stats_combine", lib().bi_stats_combine(
            _ptr(stats), c, n, _ptr(labels), ignore_index, _ptr(lp), _ptr(ent), _ptr(lse), hs))
    return lp, ent, lse


def fwd_multi(logits: torch.Tensor, labels: torch.Tensor, ignore_index: int = IGNORE_INDEX, *,
              status: Optional[torch.Tensor] = None, stream=None):
    """(logprob [N, K], entropy [N], lse [N]) for K token ids per row (labels [N, K])."""
    n, v, rs = _rows(logits, "logits")
    if labels.dim() != 2 or labels.shape[0] != n or labels.dtype != torch.int64 \
            or not labels.is_cuda or (labels.shape[1] > 1 and labels.stride(1) != 1):
        raise ValueError("labels must be a device int64 [N, K] tensor, last dim contiguous")
    k = labels.shape[1]
    _vec(status, 1, torch.int32, "status")
    ls = labels.stride(0) if n > 1 else k
    with _on_stream(stream) as hs:
        lp = torch.empty((n, k), dtype=torch.float32, device=logits.device)
        ent = torch.empty(n, dtype=torch.float32, device=logits.device)
        lse = torch.empty(n, dtype=torch.float32, device=logits.device)
        _check("bi_logprob_fwd_multi", lib().bi_logprob_fwd_multi(
            _ptr(logits), _dtype_code(logits.dtype), n, v, rs, _ptr(labels), ls, k, ignore_index,
            _ptr(lp), _ptr(ent), _ptr(lse), _ptr(status), hs))
    return lp, ent, lse


def diff_stats(a: torch.Tensor, b: torch.Tensor, labels: Optional[torch.Tensor] = None,
               ignore_index: int = IGNORE_INDEX, stream=None) -> torch.Tensor:
    """[4] fp32: mean (a-b), mean |a-b|, max |a-b|, fraction of tokens whose bits differ."""
    n = a.shape[0] if a.dim() == 1 else -1
    _vec(a, n, torch.float32, "a")
    _vec(b, n, torch.float32, "b")
    _vec(labels, n, torch.int64, "labels")
    with _on_stream(stream) as hs:
        out = torch.empty(4, dtype=torch.float32, device=a.device)
        _check("bi_logprob_diff_stats", lib().bi_logprob_diff_stats(
            _ptr(a), _ptr(b), _ptr(labels), ignore_index, n, _ptr(out), hs))
    return out


def lmhead_tile_stats(hidden: torch.Tensor, weight: torch.Tensor, labels: torch.Tensor,
                      vocab_offset: int = 0, vocab: Optional[int] = None,
                      ignore_index: int = IGNORE_INDEX, *, out: Optional[torch.Tensor] = None,
                      status: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """[tiles, N, 4] statistics of hidden [N, d] @ weight[Vc, d]^T, by tiles of
    lmhead_tile_rows() lm_head rows.

    ``weight`` holds the lm_head rows of global vocabulary ids
    vocab_offset .. vocab_offset + Vc - 1; ``vocab`` is the global size
    (defaults to vocab_offset + Vc).
    """
    n, d, ldh = _rows(hidden, "hidden")
    vc, dw, ldw = _rows(weight, "weight")
    if hidden.dtype != torch.bfloat16 or weight.dtype != torch.bfloat16 or d != dw:
        raise ValueError("hidden [N, d] and weight [Vc, d] must be bfloat16 with the same d")
    _vec(labels, n, torch.int64, "labels")
    _vec(status, 1, torch.int32, "status")
    vocab = vocab_offset + vc if vocab is None else vocab
    tiles = int(lib().bi_lmhead_tiles(vc))
    with _on_stream(stream) as hs:
        if out is None:
            out = torch.empty((tiles, n, 4), dtype=torch.float32, device=hidden.device)
        if out.shape != (tiles, n, 4) or out.dtype != torch.float32 or not out.is_contiguous():
            raise ValueError(f"out must be a contiguous float32 [{tiles}, {n}, 4] tensor")
        _check("bi_lmhead_tile_stats", lib().bi_lmhead_tile_stats(
            _ptr(hidden), _ptr(weight), n, vc, d, ldh, ldw, vocab_offset, vocab, _ptr(labels),
            ignore_index, _ptr(out), _ptr(status), hs))
    return out


def lmhead_tile_rows() -> int:
    """lm_head rows per statistics tile of lmhead_tile_stats."""
    return int(lib().bi_lmhead_tile_rows())


def lmhead_logprob(hidden: torch.Tensor, weight: torch.Tensor, labels: torch.Tensor,
                   ignore_index: int = IGNORE_INDEX, status=None, stream=None):
    """(logprob, entropy, lse) of the logits hidden @ weight^T without materialising them."""
    with _on_stream(stream):
        # the intermediate statistics belong to the launch stream: their memory
        # is reused only after the combine that reads them
        st = lmhead_tile_stats(hidden, weight, labels, 0, weight.shape[0], ignore_index,
                               status=status, stream=stream)
        return stats_combine(st, labels, ignore_index, stream=stream)


def _lmhead_operands(hidden, weight, labels):
    n, d, ldh = _rows(hidden, "hidden")
    vc, dw, ldw = _rows(weight, "weight")
    if hidden.dtype != torch.bfloat16 or weight.dtype != torch.bfloat16 or d != dw:
        raise ValueError("hidden [N, d] and weight [Vc, d] must be bfloat16 with the same d")
    _vec(labels, n, torch.int64, "labels")
    return n, d, ldh, vc, ldw


def lmhead_grad_logits(hidden: torch.Tensor, weight: torch.Tensor, labels: torch.Tensor,
                       lse: torch.Tensor, token_weights: Optional[torch.Tensor] = None,
                       vocab_offset: int = 0, vocab: Optional[int] = None,
                       ignore_index: int = IGNORE_INDEX, *, out: Optional[torch.Tensor] = None,
                       status: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """[Vc, N] bf16 gradient of the lm_head logits, vocabulary-major:
    w_n * (softmax(z_n)[v] - [v == y_n]) with the logits recomputed."""
    n, d, ldh, vc, ldw = _lmhead_operands(hidden, weight, labels)
    _vec(lse, n, torch.float32, "lse")
    _vec(token_weights, n, torch.float32, "token_weights")
    _vec(status, 1, torch.int32, "status")
    vocab = vocab_offset + vc if vocab is None else vocab
    with _on_stream(stream) as hs:
        if out is None:
            out = torch.empty((vc, n), dtype=torch.bfloat16, device=hidden.device)
        _, ncols, ldg = _rows(out, "out")
        if out.dtype != torch.bfloat16 or out.shape[0] != vc or ncols != n:
            raise ValueError(f"out must be a bfloat16 [{vc}, {n}] tensor")
        _check("bi_lmhead_grad_logits", lib().bi_lmhead_grad_logits(
            _ptr(hidden), _ptr(weight), n, vc, d, ldh, ldw, vocab_offset, vocab, _ptr(labels),
            ignore_index, _ptr(lse), _ptr(token_weights), _ptr(out), ldg, _ptr(status), hs))
    return out


def lmhead_backward(hidden: torch.Tensor, weight: torch.Tensor, labels: torch.Tensor,
                    lse: torch.Tensor, token_weights: Optional[torch.Tensor] = None,
                    vocab_offset: int = 0, vocab: Optional[int] = None,
                    ignore_index: int = IGNORE_INDEX, *, grad_hidden: Optional[torch.Tensor] = None,
                    grad_weight: Optional[torch.Tensor] = None,
                    grad_weight_dtype: torch.dtype = torch.bfloat16, chunk_rows: int = 32768,
                    workspace: Optional[torch.Tensor] = None,
                    status: Optional[torch.Tensor] = None, stream=None):
    """(grad_hidden fp32 [N, d], grad_weight [Vc, d]) of sum_n w_n * CE_n through the
    lm_head, from the saved lse.  grad_hidden is accumulated into when given."""
    n, d, ldh, vc, ldw = _lmhead_operands(hidden, weight, labels)
    _vec(lse, n, torch.float32, "lse")
    _vec(token_weights, n, torch.float32, "token_weights")
    _vec(status, 1, torch.int32, "status")
    vocab = vocab_offset + vc if vocab is None else vocab
    dev = hidden.device
    L = lib()
    with _on_stream(stream) as hs:
        # a fresh grad_hidden is zero-filled on the launch stream, ahead of the
        # kernels that accumulate into it; the workspace belongs to that stream
        if grad_hidden is None:
            grad_hidden = torch.zeros((n, d), dtype=torch.float32, device=dev)
        _, dh, ldgh = _rows(grad_hidden, "grad_hidden")
        if grad_hidden.dtype != torch.float32 or grad_hidden.shape[0] != n or dh != d:
            raise ValueError(f"grad_hidden must be a float32 [{n}, {d}] tensor")
        if grad_weight is None:
            grad_weight = torch.empty((vc, d), dtype=grad_weight_dtype, device=dev)
        _, dgw, ldgw = _rows(grad_weight, "grad_weight")
        if grad_weight.shape[0] != vc or dgw != d:
            raise ValueError(f"grad_weight must be a [{vc}, {d}] tensor")
        if workspace is None:
            nbytes = int(L.bi_lmhead_backward_workspace(n, d, min(chunk_rows, max(vc, 1))))
            if nbytes < 0:
                raise ValueError(f"no workspace size for {n} tokens, d {d}, "
                                 f"chunk_rows {chunk_rows} (at most 2^22 tokens)")
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        _check("bi_lmhead_backward", L.bi_lmhead_backward(
            _ptr(hidden), _ptr(weight), n, vc, d, ldh, ldw, vocab_offset, vocab, _ptr(labels),
            ignore_index, _ptr(lse), _ptr(token_weights), _ptr(grad_hidden), ldgh,
            _ptr(grad_weight), _dtype_code(grad_weight.dtype), ldgw, _ptr(workspace),
            workspace.numel() * workspace.element_size(), _ptr(status), hs))
    return grad_hidden, grad_weight


def lmhead_backward_noalloc(hidden: torch.Tensor, weight: torch.Tensor, labels: torch.Tensor,
                            lse: torch.Tensor, token_weights: Optional[torch.Tensor],
                            grad_hidden: torch.Tensor, grad_weight: torch.Tensor,
                            vocab_offset: int = 0, vocab: Optional[int] = None,
                            ignore_index: int = IGNORE_INDEX, *,
                            status: Optional[torch.Tensor] = None, stream=None):
    """lmhead_backward into the caller's grad_hidden (accumulated) and grad_weight,
    with no workspace: the library's static device scratch holds the logits
    gradient (at most 131,072 tokens).  Nothing is allocated, here or in the
    library; calls that may overlap on one GPU race on that scratch."""
    n, d, ldh, vc, ldw = _lmhead_operands(hidden, weight, labels)
    _vec(lse, n, torch.float32, "lse")
    _vec(token_weights, n, torch.float32, "token_weights")
    _vec(status, 1, torch.int32, "status")
    vocab = vocab_offset + vc if vocab is None else vocab
    _, dh, ldgh = _rows(grad_hidden, "grad_hidden")
    if grad_hidden.dtype != torch.float32 or grad_hidden.shape[0] != n or dh != d:
        raise ValueError(f"grad_hidden must be a float32 [{n}, {d}] tensor")
    _, dgw, ldgw = _rows(grad_weight, "grad_weight")
    if grad_weight.shape[0] != vc or dgw != d:
        raise ValueError(f"grad_weight must be a [{vc}, {d}] tensor")
    with _on_stream(stream) as hs:
        _check("bi_lmhead_backward_noalloc", lib().bi_lmhead_backward_noalloc(
            _ptr(hidden), _ptr(weight), n, vc, d, ldh, ldw, vocab_offset, vocab, _ptr(labels),
            ignore_index, _ptr(lse), _ptr(token_weights), _ptr(grad_hidden), ldgh,
            _ptr(grad_weight), _dtype_code(grad_weight.dtype), ldgw, _ptr(status), hs))
    return grad_hidden, grad_weight


def row_geometry(dtype: torch.dtype, width: int) -> Tuple[int, int, int]:
    """(threads per workgroup, elements per 16-byte load, loads per rescale group)."""
    a, b, c = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _check("bi_row_geometry", lib().bi_row_geometry(_dtype_code(dtype), width,
                                                    ctypes.byref(a), ctypes.byref(b),
                                                    ctypes.byref(c)))
    return a.value, b.value, c.value


# ----------------------------------------------------------------- autograd

class LogprobEntropy(torch.autograd.Function):
    """logprob (differentiable) and entropy (a metric, no gradient) of full rows."""

    @staticmethod
    def forward(ctx, logits, labels, ignore_index=IGNORE_INDEX, grad_dtype=None):
        lp, ent, lse = fwd(logits, labels, ignore_index)
        ctx.save_for_backward(logits, labels, lse)
        ctx.ignore_index = ignore_index
        ctx.grad_dtype = grad_dtype
        ctx.mark_non_differentiable(ent)
        return lp, ent

    @staticmethod
    def backward(ctx, grad_lp, grad_ent):
        logits, labels, lse = ctx.saved_tensors
        # d logprob / d z = onehot - softmax, so grad = (-g) * (softmax - onehot)
        w = (-grad_lp).to(torch.float32).contiguous()
        g = bwd(logits, labels, lse, w, ctx.grad_dtype or logits.dtype, ctx.ignore_index)
        return g, None, None, None


def logprob_entropy(logits, labels, ignore_index=IGNORE_INDEX, grad_dtype=None):
    """Autograd-aware (logprob, entropy) of full rows."""
    return LogprobEntropy.apply(logits, labels, ignore_index, grad_dtype)


class LmHeadLogprobEntropy(torch.autograd.Function):
    """logprob (differentiable in hidden and weight) and entropy (a metric) of the
    lm_head logits hidden @ weight^T, which are never materialised."""

    @staticmethod
    def forward(ctx, hidden, weight, labels, ignore_index=IGNORE_INDEX, chunk_rows=32768):
        lp, ent, lse = lmhead_logprob(hidden, weight, labels, ignore_index)
        ctx.save_for_backward(hidden, weight, labels, lse)
        ctx.ignore_index = ignore_index
        ctx.chunk_rows = chunk_rows
        ctx.mark_non_differentiable(ent)
        return lp, ent

    @staticmethod
    def backward(ctx, grad_lp, grad_ent):
        hidden, weight, labels, lse = ctx.saved_tensors
        w = (-grad_lp).to(torch.float32).contiguous()   # d logprob / d z = onehot - softmax
        gh, gw = lmhead_backward(hidden, weight, labels, lse, w, 0, None, ctx.ignore_index,
                                 grad_weight_dtype=weight.dtype, chunk_rows=ctx.chunk_rows)
        return gh.to(hidden.dtype), gw, None, None, None


def lmhead_logprob_entropy(hidden, weight, labels, ignore_index=IGNORE_INDEX, chunk_rows=32768):
    """Autograd-aware (logprob, entropy) straight from hidden states and lm_head rows."""
    return LmHeadLogprobEntropy.apply(hidden, weight, labels, ignore_index, chunk_rows)
