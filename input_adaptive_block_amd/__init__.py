"""Input-adaptive block-sparse attention over 3D-blocked video tokens on MI355X.

The compute lives in libspade.so (hand-written HIP kernels for gfx950 behind a
C ABI, include/spade.h).  This package is its Python binding: `_lib` mirrors the
C entry points one to one; the helpers below only allocate outputs and
workspace with torch (device memory and streams) and forward to them.
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

from ._lib import (  # noqa: F401
    EXPORTED, LIB_PATH, MODES, SUMMARIZERS, Budget, Problem, SpadeError, SPADE_BF16, SPADE_F32,
    SPADE_SUM_MAX, SPADE_SUM_MEAN, SPADE_SUM_MIN,
    SPADE_KEEP_COUNT, SPADE_KEEP_MASS, SPADE_KEEP_RATIO, SPADE_OK, SPADE_ERR_CAPACITY,
    SPADE_ERR_DEVICE, SPADE_ERR_INVALID_ARG, SPADE_ERR_UNSUPPORTED, lib, spade_attn,
    spade_block_sparse_attn, spade_check, spade_debug_scores, spade_estimate_select,
    spade_estimate_select_static, SPADE_STATIC_SCRATCH_BYTES, spade_debug_dense_walk,
    spade_attn_schemes, spade_max_nnz, spade_num_blocks, spade_profile_events, spade_scheme_select,
    spade_schemes_workspace_bytes, spade_summarize, spade_summarize_sics,
    spade_workspace_bytes,
    status_string,
)

__all__ = [
    "Problem", "Budget", "SpadeError", "problem_for", "summarize", "summarize_sics", "estimate_select",
    "estimate_select_static", "spade_estimate_select_static", "SPADE_STATIC_SCRATCH_BYTES",
    "block_sparse_attn", "attn", "debug_scores", "alloc_workspace", "scheme_select", "attn_schemes",
    "spade_num_blocks", "spade_max_nnz", "spade_workspace_bytes", "spade_check",
    "spade_summarize", "spade_summarize_sics", "spade_estimate_select", "spade_block_sparse_attn", "spade_attn",
    "spade_debug_scores", "spade_schemes_workspace_bytes", "spade_scheme_select", "spade_attn_schemes",
]


def _torch():
    import torch
    return torch


def problem_for(q, grid: Sequence[int], block: Sequence[int], scale: Optional[float] = None,
                summarizer: str = "mean") -> Problem:
    """Problem of a [B, H, N, d] tensor on grid (T, Hh, W) with block (bt, bh, bw);
    summarizer is "mean", "max" or "min"."""
    torch = _torch()
    B, H, N, d = q.shape
    if q.dtype == torch.bfloat16:
        dt = SPADE_BF16
    elif q.dtype == torch.float32:
        dt = SPADE_F32
    else:
        raise SpadeError(SPADE_ERR_UNSUPPORTED, f"dtype {q.dtype}")
    T, Hh, W = grid
    bt, bh, bw = block
    if summarizer not in SUMMARIZERS:
        raise SpadeError(SPADE_ERR_INVALID_ARG, f"summarizer {summarizer!r}")
    return Problem(B, H, N, d, T, Hh, W, bt, bh, bw, dt, 0.0 if scale is None else float(scale),
                   SUMMARIZERS[summarizer])


def _check_tensor(t, name, shape=None, dtype=None, device=None):
    _check_tensors([(t, name, shape, dtype)], device)


def _check_tensors(specs, device=None):
    """Raise SpadeError unless every (tensor, name, shape, dtype) of specs is
    a contiguous tensor of that shape and dtype (None: any) and all of them are
    device tensors on `device` (None: the first one's).  Forms are checked for
    every tensor before any device, so each check can be exercised without a
    GPU."""
    torch = _torch()
    for t, name, shape, dtype in specs:
        if not isinstance(t, torch.Tensor):
            raise SpadeError(SPADE_ERR_INVALID_ARG, f"{name} must be a tensor")
        if shape is not None and tuple(t.shape) != tuple(shape):
            raise SpadeError(SPADE_ERR_INVALID_ARG, f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if dtype is not None and t.dtype != dtype:
            raise SpadeError(SPADE_ERR_INVALID_ARG, f"{name} has dtype {t.dtype}, expected {dtype}")
        if not t.is_contiguous():
            raise SpadeError(SPADE_ERR_INVALID_ARG, f"{name} must be contiguous")
    for t, name, _, _ in specs:
        if not t.is_cuda:
            raise SpadeError(SPADE_ERR_INVALID_ARG, f"{name} must be a device tensor")
        if device is None:
            device = t.device
        if t.device != device:
            raise SpadeError(SPADE_ERR_INVALID_ARG, f"{name} is on {t.device}, expected {device}")


def _workspace_specs(ws, problem: Problem):
    """[] for no caller workspace, else the workspace's spec for
    _check_tensors (a one-dimensional uint8 tensor); a uint8 workspace below
    spade_workspace_bytes raises SPADE_ERR_CAPACITY."""
    torch = _torch()
    if ws is None:
        return []
    if isinstance(ws, torch.Tensor) and ws.dtype == torch.uint8:
        need = spade_workspace_bytes(problem)
        if ws.numel() < need:
            raise SpadeError(SPADE_ERR_CAPACITY, f"workspace has {ws.numel()} bytes, needs {need}")
        return [(ws, "workspace", (ws.numel(),), torch.uint8)]
    return [(ws, "workspace", None, torch.uint8)]


def _summary_shape(problem: Problem):
    nblk = spade_num_blocks(problem)
    if nblk < 0:
        raise SpadeError(spade_check(problem), "problem")
    return (problem.B, problem.H, nblk, problem.d)


def alloc_workspace(problem: Problem, device=None):
    torch = _torch()
    n = spade_workspace_bytes(problem)
    if n == 0:
        raise SpadeError(spade_check(problem), "spade_workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def summarize(q, k, grid, block, summarizer: str = "mean") -> Tuple["object", "object"]:
    torch = _torch()
    p = problem_for(q, grid, block, summarizer=summarizer)
    nblk = spade_num_blocks(p)
    if nblk < 0:
        raise SpadeError(spade_check(p), "summarize")
    _check_tensors([(q, "q", None, None), (k, "k", q.shape, q.dtype)])
    qm = torch.empty(p.B, p.H, nblk, p.d, dtype=torch.float32, device=q.device)
    km = torch.empty_like(qm)
    spade_summarize(p, q, k, qm, km)
    return qm, km


def summarize_sics(q, k, grid, block, summarizer: str = "mean"):
    """Block summaries and the per-block intra-block cosine similarity (SICS,
    in [0, 1]) of q and k: returns (q_sum, k_sum, q_sics, k_sics)."""
    torch = _torch()
    p = problem_for(q, grid, block, summarizer=summarizer)
    nblk = spade_num_blocks(p)
    if nblk < 0:
        raise SpadeError(spade_check(p), "summarize_sics")
    _check_tensors([(q, "q", None, None), (k, "k", q.shape, q.dtype)])
    qm = torch.empty(p.B, p.H, nblk, p.d, dtype=torch.float32, device=q.device)
    km = torch.empty_like(qm)
    qs = torch.empty(p.B, p.H, nblk, dtype=torch.float32, device=q.device)
    ks = torch.empty_like(qs)
    spade_summarize_sics(p, q, k, qm, km, qs, ks)
    return qm, km, qs, ks


def estimate_select(q_mean, k_mean, problem: Problem, mode, per_head: Sequence[float], workspace=None,
                    window=None):
    torch = _torch()
    shape = _summary_shape(problem)
    _check_tensors([(q_mean, "q_mean", shape, torch.float32), (k_mean, "k_mean", shape, torch.float32)]
                   + _workspace_specs(workspace, problem))
    bud = Budget(mode, per_head, window)
    cap = spade_max_nnz(problem, bud)
    if cap < 0:
        raise SpadeError(spade_check(problem, bud), "estimate_select")
    nblk = spade_num_blocks(problem)
    R = problem.B * problem.H * nblk
    ws = alloc_workspace(problem, q_mean.device) if workspace is None else workspace
    row_ptr = torch.empty(R + 1, dtype=torch.int32, device=q_mean.device)
    col_idx = torch.empty(max(1, cap), dtype=torch.int32, device=q_mean.device)
    spade_estimate_select(problem, q_mean, k_mean, bud, row_ptr, col_idx, cap, ws, ws.numel())
    return row_ptr, col_idx


def estimate_select_static(q_mean, k_mean, problem: Problem, mode, per_head: Sequence[float], window=None,
                           out=None):
    """estimate_select with the library's static scratch instead of a
    workspace: the C call allocates nothing.  out=(row_ptr, col_idx) reuses
    caller buffers (row_ptr int32 [R+1], col_idx int32 with at least
    spade_max_nnz entries); otherwise they are allocated here."""
    torch = _torch()
    shape = _summary_shape(problem)
    specs = [(q_mean, "q_mean", shape, torch.float32), (k_mean, "k_mean", shape, torch.float32)]
    bud = Budget(mode, per_head, window)
    cap = spade_max_nnz(problem, bud)
    if cap < 0:
        raise SpadeError(spade_check(problem, bud), "estimate_select_static")
    R = problem.B * problem.H * shape[2]
    if out is None:
        row_ptr = torch.empty(R + 1, dtype=torch.int32, device=q_mean.device)
        col_idx = torch.empty(max(1, cap), dtype=torch.int32, device=q_mean.device)
    else:
        row_ptr, col_idx = out
        specs += [(row_ptr, "row_ptr", (R + 1,), torch.int32), (col_idx, "col_idx", None, torch.int32)]
    _check_tensors(specs)
    if col_idx.dim() != 1:
        raise SpadeError(SPADE_ERR_INVALID_ARG, "col_idx must be 1-D")
    spade_estimate_select_static(problem, q_mean, k_mean, bud, row_ptr, col_idx, col_idx.numel())
    return row_ptr, col_idx


def block_sparse_attn(q, k, v, grid, block, row_ptr, col_idx, scale=None, workspace=None, out=None):
    torch = _torch()
    p = problem_for(q, grid, block, scale)
    nblk = _summary_shape(p)[2]
    o = torch.empty_like(q) if out is None else out
    # the kernels read row_ptr[0 .. R]; col_idx is read only below the
    # capacity passed with it (its length)
    if not isinstance(col_idx, torch.Tensor) or col_idx.dim() != 1:
        raise SpadeError(SPADE_ERR_INVALID_ARG, "col_idx must be a one-dimensional tensor")
    _check_tensors([(q, "q", q.shape, q.dtype), (k, "k", q.shape, q.dtype), (v, "v", q.shape, q.dtype),
                    (row_ptr, "row_ptr", (p.B * p.H * nblk + 1,), torch.int32),
                    (col_idx, "col_idx", None, torch.int32), (o, "out", q.shape, q.dtype)]
                   + _workspace_specs(workspace, p))
    ws = alloc_workspace(p, q.device) if workspace is None else workspace
    spade_block_sparse_attn(p, q, k, v, row_ptr, col_idx, col_idx.numel(), o, ws, ws.numel())
    return o


def attn(q, k, v, grid, block, mode, per_head: Sequence[float], scale=None, workspace=None,
         summarizer: str = "mean", window=None):
    """Whole path; returns (o, row_ptr, col_idx).  window: None or the static
    window's radii (rt, rh, rw) in blocks, united with the scored blocks."""
    torch = _torch()
    p = problem_for(q, grid, block, scale, summarizer)
    _check_tensors([(q, "q", q.shape, q.dtype), (k, "k", q.shape, q.dtype), (v, "v", q.shape, q.dtype)]
                   + _workspace_specs(workspace, p))
    bud = Budget(mode, per_head, window)
    cap = spade_max_nnz(p, bud)
    if cap < 0:
        raise SpadeError(spade_check(p, bud), "attn")
    nblk = spade_num_blocks(p)
    R = p.B * p.H * nblk
    ws = alloc_workspace(p, q.device) if workspace is None else workspace
    row_ptr = torch.empty(R + 1, dtype=torch.int32, device=q.device)
    col_idx = torch.empty(max(1, cap), dtype=torch.int32, device=q.device)
    o = torch.empty_like(q)
    spade_attn(p, q, k, v, bud, o, row_ptr, col_idx, cap, ws, ws.numel())
    return o, row_ptr, col_idx


def debug_scores(q_mean, k_mean, problem: Problem):
    torch = _torch()
    shape = _summary_shape(problem)
    _check_tensors([(q_mean, "q_mean", shape, torch.float32), (k_mean, "k_mean", shape, torch.float32)])
    nblk = shape[2]
    S = torch.empty(problem.B, problem.H, nblk, nblk, dtype=torch.float64, device=q_mean.device)
    spade_debug_scores(problem, q_mean, k_mean, S)
    return S


def scheme_select(q, k, grid, candidates, summarizer: str = "mean"):
    """Aggregate SICS of every blocking candidate per (b, h) and the head-wise
    choice: returns (agg [C, B, H] fp32, scheme [B, H] int32)."""
    torch = _torch()
    p = problem_for(q, grid, candidates[0], summarizer=summarizer)
    _check_tensors([(q, "q", None, None), (k, "k", q.shape, q.dtype)])
    n = spade_schemes_workspace_bytes(p, candidates)
    if n == 0:
        raise SpadeError(SPADE_ERR_INVALID_ARG, "scheme_select")
    ws = torch.empty(n, dtype=torch.uint8, device=q.device)
    agg = torch.empty(len(candidates), p.B, p.H, dtype=torch.float32, device=q.device)
    scheme = torch.empty(p.B, p.H, dtype=torch.int32, device=q.device)
    spade_scheme_select(p, q, k, candidates, agg, scheme, ws, ws.numel())
    return agg, scheme


def attn_schemes(q, k, v, grid, candidates, mode, per_head: Sequence[float], scale=None,
                 summarizer: str = "mean", window=None):
    """Head-wise schemes end to end: returns (o, scheme [B, H], agg [C, B, H])."""
    torch = _torch()
    p = problem_for(q, grid, candidates[0], scale, summarizer)
    _check_tensors([(q, "q", q.shape, q.dtype), (k, "k", q.shape, q.dtype), (v, "v", q.shape, q.dtype)])
    bud = Budget(mode, per_head, window)
    n = spade_schemes_workspace_bytes(p, candidates, bud)
    if n == 0:
        raise SpadeError(SPADE_ERR_INVALID_ARG, "attn_schemes")
    ws = torch.empty(n, dtype=torch.uint8, device=q.device)
    o = torch.empty_like(q)
    agg = torch.empty(len(candidates), p.B, p.H, dtype=torch.float32, device=q.device)
    scheme = torch.empty(p.B, p.H, dtype=torch.int32, device=q.device)
    spade_attn_schemes(p, q, k, v, candidates, bud, o, agg, scheme, ws, ws.numel())
    return o, scheme, agg

