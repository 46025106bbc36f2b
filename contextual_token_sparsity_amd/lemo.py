"""Thin ctypes binding of liblemo.so (include/lemo.h), same names as the C ABI.

Argument marshalling only: tensors are turned into device pointers, leading
dimensions and the current HIP stream; every step of the hot path runs in the
library's kernels.  There is no fallback: if the library is missing the first
call raises.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
# LEMO_LIB_PATH selects another build of the same library (the CPU tests
# point it at the sanitizer build of the host-side layer)
LIB_PATH = os.environ.get("LEMO_LIB_PATH") or os.path.join(PKG, "liblemo.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "lemo.h")

LEMO_OK = 0
REDUCE_PAPER, REDUCE_HEADMAX = 0, 1
SELECT_THRESHOLD, SELECT_TOPK, SELECT_MEAN = 0, 1, 2
DEV_CAP_OVERFLOW, DEV_NONFINITE, DEV_BAD_KEPT = 1, 2, 4
LEMO_SCORES_CAUSAL = 1

_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_SIGS = {
    "lemo_block_scores_workspace": (_sz, [_i, _i]),
    "lemo_block_scores": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _sz, _vp]),
    "lemo_block_scores_batched_workspace": (_sz, [_i, _i, _i]),
    "lemo_block_scores_batched": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _i, ctypes.c_int64, ctypes.c_int64, _i, _i, _i,
                                       _vp, _vp, _vp, _sz, _vp]),
    "lemo_predict_scores_workspace": (_sz, [_i, _i, _i, _i]),
    "lemo_predict_scores": (_i, [_vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _i, _vp, _vp, _vp, _sz, _vp]),
    "lemo_predict_scores_noalloc": (_i, [_vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _i, _vp, _vp, _vp]),
    "lemo_token_embeddings_workspace": (_sz, [_i, _i, _i]),
    "lemo_token_embeddings": (_i, [_vp, _i, _i, _i, _vp, _vp, _vp, _vp, _i, _vp, _vp, _i, _vp, _sz, _vp]),
    "lemo_select_mask": (_i, [_vp, _i, _i, _f, _i, _vp, _vp, _vp, _vp, _vp, _vp]),
    "lemo_gather_pad": (_i, [_vp, _i, _i, _i, _i, _vp, _vp, _vp, _i, _i, _i, _vp, _vp]),
    "lemo_scatter_residual": (_i, [_vp, _i, _i, _i, _i, _vp, _vp, _vp, _i, _vp, _vp]),
    "lemo_residual_recompute": (_i, [_vp, _i, _i, _i, _i, _vp, _vp, _vp, _i, _vp, _vp]),
    "lemo_gather_pad_multi": (_i, [_i, _vp, _vp, _vp, _vp, _vp, _i, _i, _vp, _vp, _i, _i, _vp, _vp]),
    "lemo_scatter_residual_capped": (_i, [_vp, _i, _i, _i, _i, _vp, _vp, _vp, _i, _i, _vp, _vp]),
    "lemo_residual_recompute_capped": (_i, [_vp, _i, _i, _i, _i, _vp, _vp, _vp, _i, _i, _vp, _vp]),
    "lemo_mlp_block_scores_workspace": (_sz, [_i, _i, _i]),
    "lemo_mlp_block_scores": (_i, [_vp, _i, _i, _i, _i, _vp, _vp, _sz, _vp]),
    "lemo_mlp_block_scores_gated": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _sz, _vp]),
    "lemo_gather_linear": (_i, [_vp, _i, _i, _i, _i, _vp, _vp, _vp, _i, _i, _vp, _i, _i, _i, _vp, _vp]),
    "lemo_linear_scatter": (_i, [_vp, _i, _i, _i, _vp, _i, _i, _vp, _i, _i, _i, _vp, _vp, _vp, _vp]),
    "lemo_status_string": (ctypes.c_char_p, [_i]),
    "lemo_last_error": (ctypes.c_char_p, []),
    "lemo_version": (_i, []),
}

_lib = None


class LemoError(RuntimeError):
    def __init__(self, status: int, fn: str, detail: str):
        super().__init__(f"{fn}: status {status}: {detail}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load liblemo.so (built in-tree by build.py); raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m contextual_token_sparsity_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def declared_symbols() -> list:
    """Function names declared in include/lemo.h."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w ]*\**\s+\**(lemo_\w+)\s*\(", text, re.M)))


def _check(status: int, fn: str):
    if status != LEMO_OK:
        raise LemoError(status, fn, lib().lemo_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _ld(t) -> int:
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("expected a row-major 2-D tensor with unit column stride")
    return t.stride(0)


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _bf16(t):
    if t.dtype not in (torch.int16, torch.uint16, torch.bfloat16):
        raise TypeError("bf16 operands are passed as bfloat16 or 16-bit integer tensors")
    if not t.is_cuda:
        raise ValueError("operands must be device tensors")
    return t


def _buf(t, dtype, numel: int, name: str, dev):
    """A caller-provided buffer the library writes or reads as a flat array:
    a contiguous tensor of `dtype` on the operands' device with at least
    `numel` elements (the C side sees only its address).  None passes."""
    if t is None:
        return None
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, {numel} needed")
    if not t.is_cuda or t.device != dev:
        raise ValueError(f"{name} must be a tensor on {dev}")
    return t


def _ws_bytes(t, dev) -> int:
    """Size in bytes of a caller's workspace tensor (any dtype, contiguous,
    on the operands' device); 0 for None."""
    if t is None:
        return 0
    if not t.is_contiguous():
        raise ValueError("workspace must be contiguous")
    if not t.is_cuda or t.device != dev:
        raise ValueError(f"workspace must be a tensor on {dev}")
    return t.numel() * t.element_size()


def _kept_bufs(kept_blocks, n_kept, dev_status, dev):
    """The kept-block list (int32, read up to the device-side count), the
    count (int32[1]) and the optional status word (int32[1])."""
    if kept_blocks is None or n_kept is None:
        raise ValueError("kept_blocks and n_kept are required")
    _buf(kept_blocks, torch.int32, 0, "kept_blocks", dev)
    _buf(n_kept, torch.int32, 1, "n_kept", dev)
    _buf(dev_status, torch.int32, 1, "dev_status", dev)


def _rows_within(t, n_rows: int, width: int, name: str):
    """n_rows x width must lie inside the 2-D tensor t."""
    if n_rows > t.shape[0] or width > t.shape[1]:
        raise ValueError(f"{name} is {tuple(t.shape)}, {n_rows} x {width} needed")


# ---------------------------------------------------------------- calls
def lemo_block_scores_workspace(n_tokens: int, block: int) -> int:
    return lib().lemo_block_scores_workspace(n_tokens, block)


def lemo_block_scores(q, k, n_heads: int, head_dim: int, block: int, head_reduce: int = REDUCE_PAPER,
                      block_scores=None, scores=None, workspace=None):
    """Exact block scores.  Returns (scores [nb] fp32, block_scores [nb][nb] or None)."""
    _bf16(q), _bf16(k)
    n = q.shape[0]
    if block <= 0:
        raise ValueError(f"block must be positive (got {block})")
    nb = n // block
    # the C side sees only the row stride: the columns the heads span must lie
    # inside each operand (a narrow view of a wider matrix has ld >= width)
    _rows_within(q, n, n_heads * head_dim, "q")
    _rows_within(k, n, n_heads * head_dim, "k")
    if scores is None:
        scores = torch.empty(nb, dtype=torch.float32, device=q.device)
    _buf(scores, torch.float32, nb, "scores", q.device)
    _buf(block_scores, torch.float32, nb * nb, "block_scores", q.device)
    if block_scores is None and workspace is None:
        workspace = torch.empty(max(lemo_block_scores_workspace(n, block), 1), dtype=torch.uint8, device=q.device)
    st = lib().lemo_block_scores(_ptr(q), _ptr(k), n, n_heads, head_dim, _ld(q), _ld(k), block, head_reduce,
                                 _ptr(block_scores), _ptr(scores), _ptr(workspace),
                                 _ws_bytes(workspace, q.device), _stream(q.device))
    _check(st, "lemo_block_scores")
    return scores, block_scores


def lemo_block_scores_batched_workspace(n_batch: int, n_tokens: int, block: int) -> int:
    return lib().lemo_block_scores_batched_workspace(n_batch, n_tokens, block)


def lemo_block_scores_batched(q, k, n_heads: int, head_dim: int, block: int, head_reduce: int = REDUCE_PAPER,
                              causal: bool = False, block_scores=None, scores=None, workspace=None):
    """Exact block scores of a batch.  q, k: [B][N][width] with unit column
    stride (row stride and batch stride taken from the tensors) or [N][width]
    for one sequence.  N need not be a multiple of block.  Returns (scores
    [B][nb] fp32, block_scores [B][nb][nb] or None)."""
    _bf16(q), _bf16(k)
    if q.dim() == 2:
        q, k = q.unsqueeze(0), k.unsqueeze(0)
    if q.dim() != 3 or k.dim() != 3 or q.shape[:2] != k.shape[:2] or q.stride(2) != 1 or k.stride(2) != 1:
        raise ValueError("q and k must be [B][N][width] with unit column stride and the same B, N")
    B, n = q.shape[0], q.shape[1]
    if block <= 0:
        raise ValueError(f"block must be positive (got {block})")
    for name, t in (("q", q), ("k", k)):
        if t.shape[2] < n_heads * head_dim:
            raise ValueError(f"{name} is {tuple(t.shape)}, {n_heads * head_dim} columns needed")
    nb = (n + block - 1) // block
    if scores is None:
        scores = torch.empty(B, nb, dtype=torch.float32, device=q.device)
    _buf(scores, torch.float32, B * nb, "scores", q.device)
    _buf(block_scores, torch.float32, B * nb * nb, "block_scores", q.device)
    if block_scores is None and workspace is None:
        workspace = torch.empty(max(lemo_block_scores_batched_workspace(B, n, block), 1), dtype=torch.uint8,
                                device=q.device)
    st = lib().lemo_block_scores_batched(_ptr(q), _ptr(k), B, n, n_heads, head_dim, q.stride(1), k.stride(1),
                                         q.stride(0), k.stride(0), block, head_reduce, LEMO_SCORES_CAUSAL if causal else 0,
                                         _ptr(block_scores), _ptr(scores), _ptr(workspace),
                                         _ws_bytes(workspace, q.device), _stream(q.device))
    _check(st, "lemo_block_scores_batched")
    return scores, block_scores


def lemo_predict_scores_workspace(n_tokens: int, d_model: int, block: int, rank: int) -> int:
    return lib().lemo_predict_scores_workspace(n_tokens, d_model, block, rank)


def lemo_predict_scores(x, u_q, v_q, u_k, v_k, block: int, d_model: int = None, block_scores=None,
                        scores=None, workspace=None):
    """Predicted block scores.  Returns (scores [nb] fp32, block_scores or None)."""
    for t in (x, u_q, v_q, u_k, v_k):
        _bf16(t)
    n = x.shape[0]
    d = x.shape[1] if d_model is None else d_model
    rank = u_q.shape[1]
    if block <= 0:
        raise ValueError(f"block must be positive (got {block})")
    nb = -(-n // block)                 # a ragged last block counts
    _rows_within(x, n, d, "x")
    for name, t, r, c in (("u_q", u_q, d, rank), ("u_k", u_k, d, rank), ("v_q", v_q, rank, rank),
                          ("v_k", v_k, rank, rank)):
        _buf(t, t.dtype, r * c, name, x.device)
    if scores is None:
        scores = torch.empty(nb, dtype=torch.float32, device=x.device)
    _buf(scores, torch.float32, nb, "scores", x.device)
    _buf(block_scores, torch.float32, nb * nb, "block_scores", x.device)
    if workspace is None:
        workspace = torch.empty(max(lemo_predict_scores_workspace(n, d, block, rank), 1), dtype=torch.uint8,
                                device=x.device)
    st = lib().lemo_predict_scores(_ptr(x), n, d, _ld(x), block, _ptr(u_q), _ptr(v_q), _ptr(u_k), _ptr(v_k), rank,
                                   _ptr(block_scores), _ptr(scores), _ptr(workspace), _ws_bytes(workspace, x.device),
                                   _stream(x.device))
    _check(st, "lemo_predict_scores")
    return scores, block_scores


def lemo_predict_scores_noalloc(x, u_q, v_q, u_k, v_k, block: int, d_model: int = None, block_scores=None,
                                scores=None):
    """lemo_predict_scores with the library's fixed per-device scratch instead
    of a workspace (the library allocates nothing; shapes needing more than
    its 16 MiB are refused).  Calls that overlap on one device race.
    Returns (scores [nb] fp32, block_scores or None)."""
    for t in (x, u_q, v_q, u_k, v_k):
        _bf16(t)
    n = x.shape[0]
    d = x.shape[1] if d_model is None else d_model
    rank = u_q.shape[1]
    if block <= 0:
        raise ValueError(f"block must be positive (got {block})")
    nb = -(-n // block)
    _rows_within(x, n, d, "x")
    for name, t, r, c in (("u_q", u_q, d, rank), ("u_k", u_k, d, rank), ("v_q", v_q, rank, rank),
                          ("v_k", v_k, rank, rank)):
        _buf(t, t.dtype, r * c, name, x.device)
    if scores is None:
        scores = torch.empty(nb, dtype=torch.float32, device=x.device)
    _buf(scores, torch.float32, nb, "scores", x.device)
    _buf(block_scores, torch.float32, nb * nb, "block_scores", x.device)
    st = lib().lemo_predict_scores_noalloc(_ptr(x), n, d, _ld(x), block, _ptr(u_q), _ptr(v_q), _ptr(u_k),
                                           _ptr(v_k), rank, _ptr(block_scores), _ptr(scores), _stream(x.device))
    _check(st, "lemo_predict_scores_noalloc")
    return scores, block_scores


def lemo_token_embeddings_workspace(n_tokens: int, d_model: int, rank: int) -> int:
    return lib().lemo_token_embeddings_workspace(n_tokens, d_model, rank)


def lemo_token_embeddings(x, u_q, v_q, u_k, v_k, d_model: int = None, q_hat=None, k_hat=None, workspace=None):
    """Per-token predictor embeddings.  Returns (q_hat, k_hat), bf16 bits [N][rank]
    as int16 tensors (the query and key of one head of width rank)."""
    for t in (x, u_q, v_q, u_k, v_k):
        _bf16(t)
    n = x.shape[0]
    d = x.shape[1] if d_model is None else d_model
    rank = u_q.shape[1]
    if q_hat is None:
        q_hat = torch.empty((n, rank), dtype=torch.int16, device=x.device)
    if k_hat is None:
        k_hat = torch.empty((n, rank), dtype=torch.int16, device=x.device)
    _bf16(q_hat), _bf16(k_hat)
    if _ld(q_hat) != _ld(k_hat):
        raise ValueError("q_hat and k_hat must share a row stride")
    _rows_within(x, n, d, "x")
    _rows_within(q_hat, n, rank, "q_hat")
    _rows_within(k_hat, n, rank, "k_hat")
    for name, t, r, c in (("u_q", u_q, d, rank), ("u_k", u_k, d, rank), ("v_q", v_q, rank, rank),
                          ("v_k", v_k, rank, rank)):
        _buf(t, t.dtype, r * c, name, x.device)
    if workspace is None:
        workspace = torch.empty(max(lemo_token_embeddings_workspace(n, d, rank), 1), dtype=torch.uint8,
                                device=x.device)
    st = lib().lemo_token_embeddings(_ptr(x), n, d, _ld(x), _ptr(u_q), _ptr(v_q), _ptr(u_k), _ptr(v_k), rank,
                                     _ptr(q_hat), _ptr(k_hat), _ld(q_hat), _ptr(workspace),
                                     _ws_bytes(workspace, x.device), _stream(x.device))
    _check(st, "lemo_token_embeddings")
    return q_hat, k_hat


def lemo_select_mask(scores, mode: int, threshold: float = 0.0, keep_blocks: int = 0, mask=None, kept_blocks=None,
                     n_kept=None, threshold_used=None, dev_status=None):
    """Threshold + compaction.  Returns (mask u8, kept_blocks i32, n_kept i32[1], threshold_used f32[1])."""
    nb = scores.shape[0]
    dev = scores.device
    _buf(scores, torch.float32, nb, "scores", dev)
    mask = torch.empty(nb, dtype=torch.uint8, device=dev) if mask is None else mask
    kept_blocks = torch.empty(nb, dtype=torch.int32, device=dev) if kept_blocks is None else kept_blocks
    n_kept = torch.empty(1, dtype=torch.int32, device=dev) if n_kept is None else n_kept
    threshold_used = torch.empty(1, dtype=torch.float32, device=dev) if threshold_used is None else threshold_used
    _buf(mask, torch.uint8, nb, "mask", dev)
    _buf(kept_blocks, torch.int32, nb, "kept_blocks", dev)
    _buf(n_kept, torch.int32, 1, "n_kept", dev)
    _buf(threshold_used, torch.float32, 1, "threshold_used", dev)
    _buf(dev_status, torch.int32, 1, "dev_status", dev)
    st = lib().lemo_select_mask(_ptr(scores), nb, mode, float(threshold), int(keep_blocks), _ptr(mask),
                                _ptr(kept_blocks), _ptr(n_kept), _ptr(threshold_used), _ptr(dev_status),
                                _stream(dev))
    _check(st, "lemo_select_mask")
    return mask, kept_blocks, n_kept, threshold_used


def lemo_gather_pad(src, block: int, kept_blocks, n_kept, dst, pad_multiple: int = 1, width: int = None,
                    n_tokens: int = None, dev_status=None):
    """Selective load of the kept rows of src into dst (rows padded with zeros)."""
    _bf16(src), _bf16(dst)
    w = src.shape[1] if width is None else width
    n = src.shape[0] if n_tokens is None else n_tokens
    _rows_within(src, n, w, "src")
    _rows_within(dst, 0, w, "dst")
    _kept_bufs(kept_blocks, n_kept, dev_status, src.device)
    st = lib().lemo_gather_pad(_ptr(src), n, w, _ld(src), block, _ptr(kept_blocks), _ptr(n_kept), _ptr(dst),
                               _ld(dst), dst.shape[0], pad_multiple, _ptr(dev_status), _stream(src.device))
    _check(st, "lemo_gather_pad")
    return dst


def lemo_gather_pad_multi(srcs, dsts, block: int, kept_blocks, n_kept, pad_multiple: int = 1, widths=None,
                          n_tokens: int = None, dev_status=None):
    """Selective load of up to 4 matrices on one kept list in one launch:
    dsts[i] receives what lemo_gather_pad(srcs[i], ...) would write.  The
    capacity is the smallest destination's row count."""
    if not 1 <= len(srcs) == len(dsts) <= 4:
        raise ValueError("1 to 4 sources, one destination each")
    for t in list(srcs) + list(dsts):
        _bf16(t)
    ws = [t.shape[1] for t in srcs] if widths is None else list(widths)
    n = srcs[0].shape[0] if n_tokens is None else n_tokens
    for i, (a, b_) in enumerate(zip(srcs, dsts)):
        _rows_within(a, n, ws[i], f"srcs[{i}]")
        _rows_within(b_, 0, ws[i], f"dsts[{i}]")
        if a.device != srcs[0].device or b_.device != srcs[0].device:
            raise ValueError("all matrices must be on one device")
    _kept_bufs(kept_blocks, n_kept, dev_status, srcs[0].device)
    k = len(srcs)
    arr_p = (ctypes.c_void_p * k)(*[t.data_ptr() for t in srcs])
    arr_d = (ctypes.c_void_p * k)(*[t.data_ptr() for t in dsts])
    arr_w = (ctypes.c_int * k)(*ws)
    arr_ls = (ctypes.c_int * k)(*[_ld(t) for t in srcs])
    arr_ld = (ctypes.c_int * k)(*[_ld(t) for t in dsts])
    cap = min(t.shape[0] for t in dsts)
    st = lib().lemo_gather_pad_multi(k, arr_p, arr_w, arr_ls, arr_d, arr_ld, n, block, _ptr(kept_blocks),
                                     _ptr(n_kept), cap, pad_multiple, _ptr(dev_status), _stream(srcs[0].device))
    _check(st, "lemo_gather_pad_multi")
    return dsts


def _scatter(fn, residual, block, kept_blocks, n_kept, y, width, n_tokens, dev_status, y_rows):
    _bf16(residual), _bf16(y)
    w = residual.shape[1] if width is None else width
    n = residual.shape[0] if n_tokens is None else n_tokens
    rows = y.shape[0] if y_rows is None else y_rows
    _rows_within(residual, n, w, "residual")
    _rows_within(y, rows, w, "y")
    _kept_bufs(kept_blocks, n_kept, dev_status, residual.device)
    st = getattr(lib(), fn)(_ptr(residual), n, w, _ld(residual), block, _ptr(kept_blocks), _ptr(n_kept), _ptr(y),
                            _ld(y), rows, _ptr(dev_status), _stream(residual.device))
    _check(st, fn)
    return residual


def lemo_scatter_residual(residual, block: int, kept_blocks, n_kept, y, width: int = None, n_tokens: int = None,
                          dev_status=None):
    """In-place addition of y's rows into the kept rows of residual.  Calls
    the capped entry point with y's row count, so a layer output shorter than
    the kept rows is never read past its end (the rows it lacks are left out
    and flag DEV_CAP_OVERFLOW)."""
    return _scatter("lemo_scatter_residual_capped", residual, block, kept_blocks, n_kept, y, width, n_tokens,
                    dev_status, None)


def lemo_scatter_residual_capped(residual, block: int, kept_blocks, n_kept, y, y_rows: int = None,
                                 width: int = None, n_tokens: int = None, dev_status=None):
    """lemo_scatter_residual with an explicit count of y's rows (default: all of them)."""
    return _scatter("lemo_scatter_residual_capped", residual, block, kept_blocks, n_kept, y, width, n_tokens,
                    dev_status, y_rows)


def lemo_residual_recompute(residual, block: int, kept_blocks, n_kept, y, width: int = None, n_tokens: int = None,
                            dev_status=None):
    """Backward recompute: subtracts y's rows from the kept rows of residual,
    in place (capped at y's row count as lemo_scatter_residual is)."""
    return _scatter("lemo_residual_recompute_capped", residual, block, kept_blocks, n_kept, y, width, n_tokens,
                    dev_status, None)


def lemo_residual_recompute_capped(residual, block: int, kept_blocks, n_kept, y, y_rows: int = None,
                                   width: int = None, n_tokens: int = None, dev_status=None):
    """lemo_residual_recompute with an explicit count of y's rows (default: all of them)."""
    return _scatter("lemo_residual_recompute_capped", residual, block, kept_blocks, n_kept, y, width, n_tokens,
                    dev_status, y_rows)


def lemo_mlp_block_scores_workspace(n_tokens: int, width: int, block: int) -> int:
    return lib().lemo_mlp_block_scores_workspace(n_tokens, width, block)


def _mlp_out(a, block, width, scores, workspace):
    n = a.shape[0]
    w = a.shape[1] if width is None else width
    if block <= 0:
        raise ValueError(f"block must be positive (got {block})")
    _rows_within(a, n, w, "act")
    if scores is None:
        scores = torch.empty(-(-n // block), dtype=torch.float32, device=a.device)
    _buf(scores, torch.float32, -(-n // block), "scores", a.device)
    if workspace is None:
        workspace = torch.empty(max(lemo_mlp_block_scores_workspace(n, w, block), 1), dtype=torch.uint8,
                                device=a.device)
    return n, w, scores, workspace


def lemo_mlp_block_scores(act, block: int, width: int = None, scores=None, workspace=None):
    """MLP-block token scores from an activation [N][w]; returns scores [ceil(N / block)] fp32."""
    _bf16(act)
    n, w, scores, workspace = _mlp_out(act, block, width, scores, workspace)
    st = lib().lemo_mlp_block_scores(_ptr(act), n, w, _ld(act), block, _ptr(scores), _ptr(workspace),
                                     _ws_bytes(workspace, act.device), _stream(act.device))
    _check(st, "lemo_mlp_block_scores")
    return scores


def lemo_mlp_block_scores_gated(gate, up, block: int, width: int = None, scores=None, workspace=None):
    """MLP-block token scores of SiLU(gate) * up; returns scores [ceil(N / block)] fp32."""
    _bf16(gate), _bf16(up)
    n, w, scores, workspace = _mlp_out(gate, block, width, scores, workspace)
    _rows_within(up, n, w, "up")
    st = lib().lemo_mlp_block_scores_gated(_ptr(gate), _ptr(up), n, w, _ld(gate), _ld(up), block, _ptr(scores),
                                           _ptr(workspace), _ws_bytes(workspace, gate.device), _stream(gate.device))
    _check(st, "lemo_mlp_block_scores_gated")
    return scores


def lemo_gather_linear(x, block: int, kept_blocks, n_kept, weight, y, pad_multiple: int = 1, d_in: int = None,
                       n_tokens: int = None, dev_status=None):
    """Selective load fused into a product: y[p] = bf16(x[token(p)] weightᵀ), zero-padded."""
    _bf16(x), _bf16(weight), _bf16(y)
    din = x.shape[1] if d_in is None else d_in
    n = x.shape[0] if n_tokens is None else n_tokens
    _rows_within(x, n, din, "x")
    _rows_within(weight, 0, din, "weight")
    _rows_within(y, 0, weight.shape[0], "y")
    _kept_bufs(kept_blocks, n_kept, dev_status, x.device)
    st = lib().lemo_gather_linear(_ptr(x), n, din, _ld(x), block, _ptr(kept_blocks), _ptr(n_kept), _ptr(weight),
                                  weight.shape[0], _ld(weight), _ptr(y), _ld(y), y.shape[0], pad_multiple,
                                  _ptr(dev_status), _stream(x.device))
    _check(st, "lemo_gather_linear")
    return y


def lemo_linear_scatter(a, weight, residual, block: int, kept_blocks, n_kept, d_in: int = None, dev_status=None):
    """In-place addition fused into a product: residual[token(p)] += bf16(a[p] weightᵀ)."""
    _bf16(a), _bf16(weight), _bf16(residual)
    din = a.shape[1] if d_in is None else d_in
    _rows_within(a, 0, din, "a")
    _rows_within(weight, 0, din, "weight")
    _rows_within(residual, 0, weight.shape[0], "residual")
    _kept_bufs(kept_blocks, n_kept, dev_status, a.device)
    st = lib().lemo_linear_scatter(_ptr(a), din, _ld(a), a.shape[0], _ptr(weight), weight.shape[0], _ld(weight),
                                   _ptr(residual), residual.shape[0], _ld(residual), block, _ptr(kept_blocks),
                                   _ptr(n_kept), _ptr(dev_status), _stream(a.device))
    _check(st, "lemo_linear_scatter")
    return residual


def lemo_status_string(s: int) -> str:
    return lib().lemo_status_string(s).decode()


def lemo_last_error() -> str:
    return lib().lemo_last_error().decode()


def lemo_version() -> int:
    return lib().lemo_version()
