"""CPU oracle for SPADE's executor hot path (test infrastructure only).

This module is the plain, slow, obviously-correct statement of what the
block-sparse attention path computes.  Only the tests, __graft_entry__.smoke()
and the bench's CPU-baseline leg may import it; the product library never
does, and the two share no code.

Source: "SPADE: An Input-Adaptive Sparse Attention Engine for Fast Video
Diffusion Models Inference", the gist.science technical summary of the paper
(page https://gist.science/paper/2608.03335), sections "Problem Statement",
"Methodology 1. vDiT-SSR" (Blocking Scheme Candidates; Summarizer & Estimator
Expressions) and "Methodology 3. Head-wise Sparse Attention Execution" (Flash
Block-Sparse Attention), plus the abstract on the catalyzex author pages
(executor with index search and flash block-sparse attention).

Arithmetic is fp64 unless a step states otherwise.  Readings taken where the
pages are silent:

* tokens are flattened in raster order n = (t*Hh + h)*W + w;
* blocks tile the grid from the origin with stride (bt, bh, bw); the last
  block along an axis that the block size does not divide is partial; block
  j = (it*nH + ih)*nW + iw; Q and KV use the same tiling;
* the Summarizer is the mean over the block's real tokens, computed exactly
  and stored as fp32 (the summary tensor's storage type); the max and min
  Summarizers take the channel-wise extreme over the same tokens;
* the intra-block estimate (SICS) of a block is the mean cosine similarity
  over all ordered pairs of its real tokens, diagonal included (zero tokens:
  cosine 0), so it lies in [0, 1];
* the inter-block Estimator is S_ij = scale * <qbar_i, kbar_j>, scale = 1/sqrt(d);
* selection orders blocks by (S descending, j ascending); a count or ratio
  budget keeps the first k (k = ceil(r*nK - 1e-6) clamped to [1, nK] for a
  ratio); a mass budget keeps the shortest prefix whose softmax(S) mass over
  all nK blocks reaches tau (at least one block);
* an optional static window (radii in blocks along t, h, w) is united with
  the blocks the budget keeps by score; with a window the budget may be 0;
* attention is exact softmax attention of each query over all tokens of its
  kept KV blocks, renormalised over those keys only; every Q block is
  computed; output keeps the input raster layout.

Parity pins: blocking, summaries, estimate, selection and attention are each
pinned against closed forms, brute force and library routines in
tests/test_oracle_pins.py.  Parity against the authors' implementation itself
is unpinned (the pages print no code, equation or worked example).
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np

MODE_COUNT = "count"
MODE_RATIO = "ratio"
MODE_MASS = "mass"


# ---------------------------------------------------------------------------
# 3D blocking of the latent token grid (vDiT-SSR, Blocking Scheme Candidates)
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class Geometry:
    T: int
    Hh: int
    W: int
    bt: int
    bh: int
    bw: int

    @property
    def N(self) -> int:
        return self.T * self.Hh * self.W

    @property
    def counts(self) -> Tuple[int, int, int]:
        return (-(-self.T // self.bt), -(-self.Hh // self.bh), -(-self.W // self.bw))

    @property
    def nblk(self) -> int:
        a, b, c = self.counts
        return a * b * c


def block_extents(g: Geometry) -> List[Tuple[int, int, int, int, int, int]]:
    """Per block j: (t0, t1, h0, h1, w0, w1), half-open, in block order."""
    nT, nH, nW = g.counts
    out = []
    for it in range(nT):
        for ih in range(nH):
            for iw in range(nW):
                out.append((it * g.bt, min(g.T, (it + 1) * g.bt),
                            ih * g.bh, min(g.Hh, (ih + 1) * g.bh),
                            iw * g.bw, min(g.W, (iw + 1) * g.bw)))
    return out


def block_tokens(g: Geometry) -> List[np.ndarray]:
    """Raster token ids of each block, listed t-major, then h, then w."""
    toks = []
    for (t0, t1, h0, h1, w0, w1) in block_extents(g):
        t = np.arange(t0, t1)[:, None, None]
        h = np.arange(h0, h1)[None, :, None]
        w = np.arange(w0, w1)[None, None, :]
        toks.append(((t * g.Hh + h) * g.W + w).reshape(-1))
    return toks


def token_block_ids(g: Geometry) -> np.ndarray:
    """[N] block id of every token (brute force over the block list)."""
    ids = np.full(g.N, -1, dtype=np.int64)
    for j, tk in enumerate(block_tokens(g)):
        ids[tk] = j
    return ids


# ---------------------------------------------------------------------------
# Summarizer (vDiT-SSR, Summarizer & Estimator Expressions): block mean
# ---------------------------------------------------------------------------

SUMMARIZERS = ("mean", "max", "min")


def summarize(x: np.ndarray, g: Geometry, store_f32: bool = True, op: str = "mean") -> np.ndarray:
    """Block summaries of x [B, H, N, d] -> [B, H, nblk, d].

    The Summarizer reduces each block over its real tokens, channel by channel
    (technical summary, "Methodology 1. vDiT-SSR", Summarizer & Estimator
    Expressions: max, min or mean).  Mean: the sum is taken in fp64 and
    divided once by the token count.  Max / min: the largest / smallest value
    of each channel.  With store_f32 the summary is rounded to fp32 (returned
    as fp64 holding fp32 values); max and min of bf16 or fp32 inputs are
    exact.
    """
    x = np.asarray(x, dtype=np.float64)
    B, H, N, d = x.shape
    assert N == g.N
    if op not in SUMMARIZERS:
        raise ValueError(op)
    toks = block_tokens(g)
    out = np.empty((B, H, len(toks), d), dtype=np.float64)
    for j, tk in enumerate(toks):
        xb = x[:, :, tk, :]
        if op == "mean":
            out[:, :, j, :] = xb.sum(axis=2) / float(len(tk))
        elif op == "max":
            out[:, :, j, :] = xb.max(axis=2)
        else:
            out[:, :, j, :] = xb.min(axis=2)
    if store_f32:
        out = out.astype(np.float32).astype(np.float64)
    return out


# ---------------------------------------------------------------------------
# Intra-block estimator: Sum of Intra-block Cosine Similarities (SICS)
# ---------------------------------------------------------------------------

def sics(x: np.ndarray, g: Geometry, store_f32: bool = True) -> np.ndarray:
    """Normalised SICS of every block of x [B, H, N, d] -> [B, H, nblk].

    Technical summary, "Methodology 2. Scheme Generation", Aggregation
    Evaluation: SICS sums the cosine similarities of the embeddings inside a
    block; a high value means the block's tokens are tightly clustered.  Here
    the sum runs over all ordered pairs (i, j) of the block's real tokens, the
    pairs i = j included, and is divided by n_b^2, so it lies in [0, 1].  A
    zero token has no direction: its cosine with anything is taken as 0 (it
    still counts in n_b).

    This is the plain O(n_b^2 d) definition, written as the sum of all
    entries of U U^T where the rows of U are the block's unit token vectors;
    the online form of the same page (Online Optimization, O(n_b d)) must
    reach this value up to rounding.  fp64; with store_f32 the result is
    rounded once to fp32.
    """
    x = np.asarray(x, dtype=np.float64)
    B, H, N, d = x.shape
    assert N == g.N
    toks = block_tokens(g)
    out = np.empty((B, H, len(toks)), dtype=np.float64)
    for j, tk in enumerate(toks):
        xb = x[:, :, tk, :]                                   # [B, H, n, d]
        norm = np.sqrt((xb * xb).sum(axis=-1, keepdims=True))
        u = np.divide(xb, norm, out=np.zeros_like(xb), where=norm > 0)
        cos = u @ np.swapaxes(u, -1, -2)                      # [B, H, n, n]
        out[:, :, j] = cos.sum(axis=(-1, -2)) / float(len(tk)) ** 2
    if store_f32:
        out = out.astype(np.float32).astype(np.float64)
    return out


# ---------------------------------------------------------------------------
# Estimator (inter-block importance scores)
# ---------------------------------------------------------------------------

def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


def estimate(qm: np.ndarray, km: np.ndarray, scale: float) -> np.ndarray:
    """S[b, h, i, j] = scale * <qbar_i, kbar_j> in fp64."""
    return scale * np.matmul(qm, np.swapaxes(km, -1, -2))


# ---------------------------------------------------------------------------
# Index search: which KV blocks each Q block keeps
# ---------------------------------------------------------------------------

def keep_count(mode: str, value: float, nK: int, allow_zero: bool = False) -> int:
    """Blocks kept per row for a count or ratio budget.  With allow_zero (a
    static window supplies the rest of the mask) a budget of 0 keeps no
    block by score."""
    lo = 0 if allow_zero else 1
    if mode == MODE_COUNT:
        k = int(value)
        if k != value or k < lo or k > nK:
            raise ValueError(f"count budget must be an integer in [{lo}, nK]")
        return k
    if mode == MODE_RATIO:
        r = float(np.float32(value))
        if not ((0.0 < r or (allow_zero and r == 0.0)) and r <= 1.0):
            raise ValueError("ratio budget must be in (0, 1]")
        return min(nK, max(lo, math.ceil(r * nK - 1e-6)))
    raise ValueError(mode)


def window_blocks(g: Geometry, i: int, radius: Sequence[int]) -> np.ndarray:
    """Static window of Q block i: the KV blocks whose block coordinates differ
    from i's by at most (rt, rh, rw) along (t, h, w), ascending ids
    (technical summary, "Methodology 2. Scheme Generation", Policy Application:
    the budget balances static windows and dynamic selection)."""
    nT, nH, nW = g.counts
    it, rem = divmod(i, nH * nW)
    ih, iw = divmod(rem, nW)
    rt, rh, rw = (int(r) for r in radius)
    out = []
    for jt in range(max(0, it - rt), min(nT, it + rt + 1)):
        for jh in range(max(0, ih - rh), min(nH, ih + rh + 1)):
            for jw in range(max(0, iw - rw), min(nW, iw + rw + 1)):
                out.append((jt * nH + jh) * nW + jw)
    return np.array(out, dtype=np.int64)


@dataclass
class Selection:
    row_ptr: np.ndarray  # [R + 1] int64
    col_idx: np.ndarray  # [nnz] int64, ascending within each row
    counts: np.ndarray  # [R]
    margins: np.ndarray  # [R] decision margin of each row (inf if forced)
    order: np.ndarray  # [R, nK] the (S desc, j asc) order of each row

    def row(self, r: int) -> np.ndarray:
        return self.col_idx[self.row_ptr[r]:self.row_ptr[r + 1]]


def select(S: np.ndarray, mode: str, per_head: Sequence[float],
           window: Optional[Sequence[int]] = None, g: Optional[Geometry] = None) -> Selection:
    """Select KV blocks per row of S [B, H, nQ, nK]; rows r = (b*H + h)*nQ + i.

    With a static window (radii (rt, rh, rw) in blocks; needs the geometry g)
    the kept set of row i is the window of block i united with the blocks the
    budget keeps by score; a budget of 0 then keeps the window alone."""
    B, H, nQ, nK = S.shape
    per_head = [float(np.float32(v)) for v in per_head]
    assert len(per_head) == H
    S2 = S.reshape(B * H * nQ, nK)
    R = S2.shape[0]
    head_of_row = (np.arange(R) // nQ) % H
    # descending S with ties broken by ascending j (stable sort of -S)
    order = np.argsort(-S2, axis=1, kind="stable")
    s_sorted = np.take_along_axis(S2, order, axis=1)
    counts = np.empty(R, dtype=np.int64)
    margins = np.empty(R, dtype=np.float64)
    allow_zero = window is not None
    if mode in (MODE_COUNT, MODE_RATIO):
        for r in range(R):
            k = keep_count(mode, per_head[head_of_row[r]], nK, allow_zero)
            counts[r] = k
            margins[r] = (s_sorted[r, k - 1] - s_sorted[r, k]) if 0 < k < nK else math.inf
    elif mode == MODE_MASS:
        for r in range(R):
            tau = per_head[head_of_row[r]]
            if allow_zero and tau == 0.0:
                counts[r] = 0
                margins[r] = math.inf
                continue
            if not (0.0 < tau <= 1.0):
                raise ValueError("mass budget must be in (0, 1]")
            # softmax of the row over all nK blocks, taken in descending order
            p = np.exp(s_sorted[r] - s_sorted[r, 0])
            Z = p.sum()
            csum = np.cumsum(p)
            hit = np.nonzero(csum >= tau * Z)[0]
            k = int(hit[0]) + 1 if hit.size else nK
            counts[r] = k
            c_k = csum[k - 1] / Z
            c_prev = csum[k - 2] / Z if k >= 2 else 0.0
            m = tau - c_prev
            if k < nK:
                m = min(m, s_sorted[r, k - 1] - s_sorted[r, k], c_k - tau)
            margins[r] = m
    else:
        raise ValueError(mode)
    rows = [np.sort(order[r, :counts[r]]) for r in range(R)]
    if window is not None:
        assert g is not None and g.nblk == nQ == nK
        for r in range(R):
            rows[r] = np.union1d(rows[r], window_blocks(g, r % nQ, window))
        counts = np.array([len(x) for x in rows], dtype=np.int64)
    row_ptr = np.zeros(R + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum(counts)
    col_idx = np.concatenate(rows).astype(np.int64) if R else np.empty(0, dtype=np.int64)
    return Selection(row_ptr, col_idx, counts, margins, order)


# ---------------------------------------------------------------------------
# Attention over the kept blocks (exact softmax; online softmax reaches the
# same values, only faster)
# ---------------------------------------------------------------------------

def attention_block_row(q: np.ndarray, k: np.ndarray, v: np.ndarray, toks: List[np.ndarray],
                        i: int, kept: Iterable[int], scale: float,
                        return_weights: bool = False):
    """Output rows of Q block i for one (b, h).

    q, k, v are [N, d] fp64 of that head; kept lists KV blocks.
    Returns o [n_i, d] (and the [n_i, n_keys] weights and key ids if asked).
    """
    kept = sorted(set(int(j) for j in kept))  # reading: a row's kept blocks form a set
    qi = q[toks[i]]
    if not kept:  # reading: a row that keeps no block attends to nothing -> zeros
        z = np.zeros((len(toks[i]), v.shape[1]))
        return (z, np.zeros((len(toks[i]), 0)), np.zeros(0, np.int64)) if return_weights else z
    key_ids = np.concatenate([toks[j] for j in kept])
    logits = scale * (qi @ k[key_ids].T)
    logits = logits - logits.max(axis=1, keepdims=True)
    w = np.exp(logits)
    w = w / w.sum(axis=1, keepdims=True)
    o = w @ v[key_ids]
    if return_weights:
        return o, w, key_ids
    return o


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, g: Geometry,
              row_ptr: np.ndarray, col_idx: np.ndarray, scale: float,
              rows: Optional[Iterable[int]] = None) -> Dict[int, np.ndarray]:
    """Block-sparse attention of the given rows (default all) for any CSR.

    q, k, v: [B, H, N, d] (converted to fp64).  Returns {row: o [n_i, d]}.
    """
    B, H, N, d = q.shape
    nblk = g.nblk
    toks = block_tokens(g)
    R = B * H * nblk
    rows = range(R) if rows is None else rows
    out = {}
    cache = {}
    for r in rows:
        bh, i = divmod(int(r), nblk)
        b, h = divmod(bh, H)
        if bh not in cache:
            cache.clear()
            cache[bh] = tuple(np.asarray(t[b, h], dtype=np.float64) for t in (q, k, v))
        qh, kh, vh = cache[bh]
        kept = [int(j) for j in col_idx[row_ptr[r]:row_ptr[r + 1]]]
        out[int(r)] = attention_block_row(qh, kh, vh, toks, i, kept, scale)
    return out


def attention_full(q, k, v, g: Geometry, row_ptr, col_idx, scale) -> np.ndarray:
    """Whole output [B, H, N, d] in the input raster layout."""
    B, H, N, d = q.shape
    toks = block_tokens(g)
    O = np.zeros((B, H, N, d), dtype=np.float64)
    for r, o in attention(q, k, v, g, row_ptr, col_idx, scale).items():
        bh, i = divmod(r, g.nblk)
        b, h = divmod(bh, H)
        O[b, h, toks[i]] = o
    return O


def dense_attention(q, k, v, scale: float) -> np.ndarray:
    """Full softmax attention softmax(scale*Q K^T) V per (b, h), fp64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    logits = scale * np.matmul(q, np.swapaxes(k, -1, -2))
    logits -= logits.max(axis=-1, keepdims=True)
    w = np.exp(logits)
    w /= w.sum(axis=-1, keepdims=True)
    return np.matmul(w, v)


# ---------------------------------------------------------------------------
# whole path
# ---------------------------------------------------------------------------

def spade_attn(q, k, v, g: Geometry, mode: str, per_head: Sequence[float],
               scale: Optional[float] = None, summarizer: str = "mean",
               window: Optional[Sequence[int]] = None):
    """Summaries -> scores -> selection -> attention.  Returns (O, Selection, S)."""
    d = q.shape[-1]
    scale = default_scale(d) if scale is None else float(scale)
    qm = summarize(q, g, op=summarizer)
    km = summarize(k, g, op=summarizer)
    S = estimate(qm, km, scale)
    sel = select(S, mode, per_head, window, g)
    O = attention_full(q, k, v, g, sel.row_ptr, sel.col_idx, scale)
    return O, sel, S


# ---------------------------------------------------------------------------
# Scheme generation: blocking candidates, head-wise choice, head grouping
# ---------------------------------------------------------------------------

def scheme_aggregate(q: np.ndarray, k: np.ndarray, T: int, Hh: int, W: int,
                     candidates: Sequence[Tuple[int, int, int]]) -> np.ndarray:
    """Aggregate SICS of every blocking candidate for every (b, h) -> [C, B, H].

    Technical summary, "Methodology 2. Scheme Generation", Aggregation
    Evaluation: every blocking candidate (Methodology 1, Blocking Scheme
    Candidates) is scored by its SICS.  Here a candidate's score for one head
    is the token-weighted mean of its per-block normalised SICS over Q and K,
        A_c = sum_j n_j (sics_q[j] + sics_k[j]) / (2 N),
    taken in fp64 over the fp32-stored per-block values (the type of the
    per-block output).  A_c lies in [0, 1]; 1 means every block of the
    candidate holds tokens that all point the same way.
    """
    out = []
    for (bt, bh, bw) in candidates:
        g = Geometry(T, Hh, W, bt, bh, bw)
        n = np.array([len(t) for t in block_tokens(g)], dtype=np.float64)
        sq = sics(q, g, store_f32=True)
        sk = sics(k, g, store_f32=True)
        out.append(((sq + sk) * n).sum(axis=-1) / (2.0 * g.N))
    return np.stack(out)


def choose_scheme(agg: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Policy Application: each head takes the candidate with the highest
    aggregate score (ties to the earlier candidate).  Returns the choice
    [B, H] and its margin over the runner-up (inf with one candidate)."""
    choice = np.argmax(agg, axis=0)
    if agg.shape[0] == 1:
        return choice, np.full(choice.shape, math.inf)
    srt = np.sort(agg, axis=0)
    return choice, srt[-1] - srt[-2]


def spade_attn_schemes(q, k, v, T: int, Hh: int, W: int, candidates: Sequence[Tuple[int, int, int]],
                       mode: str, per_head: Sequence[float], scale: Optional[float] = None,
                       summarizer: str = "mean", window: Optional[Sequence[int]] = None):
    """Head-wise schemes: choose a blocking per (b, h), then run the path of
    each head with its own blocking ("Head Grouping": heads that share a
    scheme run together; the grouping changes no value).  Returns
    (O, choice [B, H], aggregates [C, B, H])."""
    agg = scheme_aggregate(q, k, T, Hh, W, candidates)
    choice, _ = choose_scheme(agg)
    B, H = q.shape[:2]
    O = np.zeros(q.shape, dtype=np.float64)
    for b in range(B):
        for h in range(H):
            g = Geometry(T, Hh, W, *candidates[choice[b, h]])
            sl = (slice(b, b + 1), slice(h, h + 1))
            O[sl], _, _ = spade_attn(q[sl], k[sl], v[sl], g, mode, [per_head[h]], scale, summarizer, window)
    return O, choice, agg

