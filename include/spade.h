/*
 * spade.h -- C ABI of the MI355X (gfx950) block-sparse video attention library.
 *
 * The library runs the hot path of SPADE's executor ("SPADE: An Input-Adaptive
 * Sparse Attention Engine for Fast Video Diffusion Models Inference"; the
 * gist.science technical summary, "Methodology 1. vDiT-SSR" and
 * "3. Head-wise Sparse Attention Execution"): per attention head it
 *   1. summarizes every 3D (t, h, w) block of Q and K by its mean,
 *   2. estimates block-to-block scores S = scale * qbar kbar^T,
 *   3. selects, for each Q block, the KV blocks to keep (index search) and
 *      emits them as a block-sparse row list (CSR), and
 *   4. runs flash-style block-sparse attention over only the kept blocks.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensors Q, K, V, O are contiguous [B, H, N, d] with d innermost and the
 *   N = T*Hh*W tokens in raster order n = (t*Hh + h)*W + w.
 * - Blocks tile the grid from the origin with stride (bt, bh, bw); the last
 *   block along an axis that the block size does not divide is partial.
 *   nT = ceil(T/bt), nH = ceil(Hh/bh), nW = ceil(W/bw), nblk = nT*nH*nW and
 *   block j = (it*nH + ih)*nW + iw.  Q and KV blocks use the same tiling.
 * - Selection rows: r = (b*H + h)*nblk + i, R = B*H*nblk rows.
 *   row_ptr[R+1] (int32) and col_idx[nnz] (int32) form a CSR whose row r lists
 *   the kept KV block ids of Q block i of head (b, h) in ascending order.
 * - Pointers named q, k, v, o, q_mean, k_mean, row_ptr, col_idx, scores and
 *   workspace are DEVICE pointers owned by the caller.  spade_problem and
 *   spade_budget (and budget->per_head) are HOST memory read during the call.
 *   The library never allocates or frees device memory.  Its only state is
 *   a per-device cache of the compute-unit count, the per-thread events of
 *   spade_profile_events and, on each device it runs on, one static device
 *   buffer of SPADE_STATIC_SCRATCH_BYTES (part of the loaded code object,
 *   held until the process ends) that spade_estimate_select_static uses.
 * - The workspace holds per-call scratch (summaries, scores, packed operand
 *   tiles, the attention kernel's unit counter): calls that may run at the same time,
 *   on one stream or several, each need a workspace of their own.  It must
 *   start on a 256-byte boundary (as hipMalloc returns); a misaligned
 *   workspace is rejected with SPADE_ERR_INVALID_ARG.
 * - Every compute call validates its arguments on the host first; on any
 *   error it returns a status and launches nothing.  Launches are
 *   asynchronous on `stream` (a hipStream_t; NULL = the default stream); the
 *   library never synchronizes the device.  A failed launch returns
 *   SPADE_ERR_DEVICE.
 * - NaN or Inf inputs give unspecified (but memory-safe) results.
 * - Results are deterministic: the same inputs give the same bits.
 */
#ifndef SPADE_H
#define SPADE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum spade_status {
  SPADE_OK = 0,
  SPADE_ERR_INVALID_ARG = 1, /* null pointer, inconsistent shape, bad budget */
  SPADE_ERR_UNSUPPORTED = 2, /* valid but outside the supported set */
  SPADE_ERR_CAPACITY = 3,    /* col_idx or workspace too small */
  SPADE_ERR_DEVICE = 4       /* a HIP runtime call or launch failed */
} spade_status;

typedef enum spade_dtype {
  SPADE_BF16 = 0, /* Q/K/V/O bf16; attention on bf16 MFMA, fp32 softmax */
  SPADE_F32 = 1   /* Q/K/V/O fp32; attention in fp32 FMA (debug mode) */
} spade_dtype;

typedef enum spade_keep_mode {
  SPADE_KEEP_COUNT = 0, /* keep k_h blocks per row, k_h integral in [1, nblk] */
  SPADE_KEEP_RATIO = 1, /* keep k_h = clamp(ceil(r_h*nblk - 1e-6), 1, nblk), r_h in (0, 1] */
  SPADE_KEEP_MASS = 2   /* keep the shortest score-ordered prefix whose softmax(S)
                           mass over all nblk blocks reaches tau_h, tau_h in (0, 1] */
} spade_keep_mode;

/* Summarizer of a block ("Methodology 1. vDiT-SSR", Summarizer & Estimator
 * Expressions: the Summarizer reduces Q/K blocks, e.g. via max/min/mean). */
typedef enum spade_summarizer {
  SPADE_SUM_MEAN = 0, /* mean over the block's real tokens (exact sum, one division) */
  SPADE_SUM_MAX = 1,  /* channel-wise maximum over the block's real tokens */
  SPADE_SUM_MIN = 2   /* channel-wise minimum over the block's real tokens */
} spade_summarizer;

/* Shape of one attention layer.
 * Supported: d in {64, 128}; B*H >= 0; 1 <= nblk <= 4096; N == T*Hh*W;
 * bt*bh*bw <= 1024; B*H*nblk < 2^31 rows.  scale == 0 selects 1/sqrt(d).
 * summarizer picks the block summary that every entry point computes and the
 * Estimator uses (an unknown value is SPADE_ERR_INVALID_ARG). */
typedef struct spade_problem {
  int32_t B, H, N, d;
  int32_t T, Hh, W;
  int32_t bt, bh, bw;
  int32_t dtype; /* spade_dtype */
  float scale;
  int32_t summarizer; /* spade_summarizer; 0 (mean) for the default path */
} spade_problem;

/* Per-head keep budget: per_head is a HOST array of H values interpreted by
 * mode.  The same budget applies to every batch entry.
 *
 * Static window ("Methodology 2. Scheme Generation", Policy Application: the
 * budget balances static windows and dynamic selection).  With
 * window_enable != 0, Q block i at block coordinates (it, ih, iw) also keeps
 * every KV block j with |jt-it| <= window_t, |jh-ih| <= window_h and
 * |jw-iw| <= window_w (radii in blocks, >= 0, clipped to the grid): the kept
 * set is that window united with the blocks the budget keeps by score.  With
 * a window the budget values may also be 0 (count 0, ratio 0, mass 0: the
 * window alone).  A zero-initialised budget has no window. */
typedef struct spade_budget {
  int32_t mode; /* spade_keep_mode */
  const float* per_head;
  int32_t window_enable;
  int32_t window_t, window_h, window_w;
} spade_budget;

/* ---- host-only helpers (no device access) ------------------------------ */

/* nblk of the problem, or -1 if the shape is invalid. */
int32_t spade_num_blocks(const spade_problem* p);

/* Entries col_idx must hold: exact for COUNT/RATIO without a window; with
 * a window sum over rows of min(nblk, k + window size of the row's block)
 * (exact when no scored block falls inside the window); the worst case
 * R*nblk for MASS.  -1 if the problem or budget is invalid. */
int64_t spade_max_nnz(const spade_problem* p, const spade_budget* budget);

/* Bytes of device workspace that every compute entry point of this problem
 * needs (the maximum over them); 0 if the problem is invalid. */
size_t spade_workspace_bytes(const spade_problem* p);

/* Full host-side validation of a problem, a budget (may be NULL) and a
 * col_idx capacity in entries (pass -1 to skip the capacity check). */
spade_status spade_check(const spade_problem* p, const spade_budget* budget, int64_t col_capacity);

/* Static string naming a status. */
const char* spade_status_string(spade_status s);

/* ---- compute entry points ----------------------------------------------- */

/* Summarizer ("Summarizer & Estimator Expressions"; fused blocking and
 * summarization of "Kernel Fusion"): q_mean[b,h,j,:] = mean of q over the real
 * tokens of block j (likewise k).  Sums are exact (fp64) and the mean is
 * rounded once to fp32.  q_mean, k_mean: fp32 [B, H, nblk, d]. */
spade_status spade_summarize(const spade_problem* p, const void* q, const void* k,
                             float* q_mean, float* k_mean, void* stream);

/* Summarizer plus the intra-block estimate of the same pass ("Methodology 2.
 * Scheme Generation": Aggregation Evaluation and Online Optimization; fused
 * with blocking and summarization as in "Kernel Fusion").  Writes the block
 * means exactly as spade_summarize, and for each block the normalised Sum of
 * Intra-block Cosine Similarities
 *     q_sics[b,h,j] = sum over ordered token pairs (i, i') of block j of
 *                     cos(q_i, q_i'), diagonal included, divided by n_j^2,
 * a value in [0, 1] (a zero token has cosine 0 with everything and counts in
 * n_j); likewise k_sics.  Computed in one read of the block with the online
 * identity sum cos = |sum_i q_i/|q_i| |^2 in fp64, rounded once to fp32.
 * q_sics, k_sics: fp32 [B, H, nblk]; either may be NULL (not computed).
 * q, k, q_mean, k_mean must not be NULL (SPADE_ERR_INVALID_ARG, nothing is
 * launched). */
spade_status spade_summarize_sics(const spade_problem* p, const void* q, const void* k,
                                  float* q_mean, float* k_mean, float* q_sics, float* k_sics,
                                  void* stream);

/* Estimator + index search (the author-page abstracts on catalyzex.com: the
 * executor's low-overhead index search; gist.science technical summary,
 * "Methodology 1. vDiT-SSR", Summarizer & Estimator Expressions: the
 * inter-block importance score decides which blocks each Q block retains):
 * S_ij = scale * <q_mean_i, k_mean_j> in fp64, then per row the blocks in
 * (S descending, j ascending) order are kept by the budget.  Writes row_ptr
 * [R+1] and col_idx (ascending ids per row).  col_capacity (entries) must be
 * >= spade_max_nnz.  Workspace as given by spade_workspace_bytes. */
spade_status spade_estimate_select(const spade_problem* p, const float* q_mean, const float* k_mean,
                                   const spade_budget* budget, int32_t* row_ptr, int32_t* col_idx,
                                   int64_t col_capacity, void* workspace, size_t ws_bytes, void* stream);

/* Size of the library's static selection buffer, per device. */
#define SPADE_STATIC_SCRATCH_BYTES ((size_t)8 << 20)

/* spade_estimate_select for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and the same results, with the selection
 * scratch (per-row counts, row bitmasks, scan chunk sums) in the library's
 * static device buffer instead of a workspace.  That scratch is
 *   align256(4 R) + align256(4 R ceil(nblk/32)) + align256(4 (ceil(R/4096) + 1))
 * bytes for nblk <= 1024 (wider rows would add 8 R nblk bytes of fp64 scores,
 * more than the buffer holds).  A problem whose scratch exceeds
 * SPADE_STATIC_SCRATCH_BYTES is rejected with SPADE_ERR_CAPACITY before
 * anything is launched (about 99k rows of 630 blocks fit; a 40-head layer of
 * 630 blocks needs 2.02 MiB).  The call makes no
 * device allocation of any kind.  On first use on a device it looks up that
 * device's buffer address (so call it with the stream's device current).
 * Every call on one device shares its buffer, which keeps the last call's
 * contents (no call relies on them).  Calls that may run at the same time on
 * one device (on several streams, or graphs replayed concurrently) race on
 * it: serialize them, for example on one stream.
 * Other arguments and errors as spade_estimate_select. */
spade_status spade_estimate_select_static(const spade_problem* p, const float* q_mean,
                                          const float* k_mean, const spade_budget* budget,
                                          int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                                          void* stream);

/* Flash block-sparse attention ("Flash Block-Sparse Attention"): for every
 * query token of Q block i, softmax(scale * q K_sel^T) V_sel over all tokens of
 * the KV blocks listed in CSR row i, written to o [B, H, N, d] in Q's dtype.
 * A CSR row is a SET of blocks: ids may come in any order and a repeated id
 * counts once.  Any CSR is accepted: ids outside [0, nblk), row extents
 * outside [0, col_capacity] or decreasing row_ptr are skipped (never read out
 * of bounds); a row with no valid block writes zeros. */
spade_status spade_block_sparse_attn(const spade_problem* p, const void* q, const void* k, const void* v,
                                     const int32_t* row_ptr, const int32_t* col_idx, int64_t col_capacity,
                                     void* o, void* workspace, size_t ws_bytes, void* stream);

/* The whole path of the executor (the catalyzex.com abstracts: index search,
 * flash block-sparse attention and kernel grouping; gist.science technical
 * summary, "Methodology 3. Head-wise Sparse Attention Execution"): the fused
 * blocking + summaries (Kernel Fusion) -> estimate/select -> block-sparse
 * attention, all heads in one launch per step (Head Grouping), on one stream
 * with no host synchronisation.  Also returns the CSR it used in row_ptr /
 * col_idx (capacity as above). */
spade_status spade_attn(const spade_problem* p, const void* q, const void* k, const void* v,
                        const spade_budget* budget, void* o, int32_t* row_ptr, int32_t* col_idx,
                        int64_t col_capacity, void* workspace, size_t ws_bytes, void* stream);

/* ---- head-wise schemes ("Methodology 2. Scheme Generation"; "Head Grouping")
 *
 * A blocking candidate is a 3D block shape (Blocking Scheme Candidates).  The
 * problem's own bt/bh/bw are ignored by these calls; every candidate must make
 * a valid problem (else its status is returned).  At most 16 candidates. */
typedef struct spade_block_shape {
  int32_t bt, bh, bw;
} spade_block_shape;

/* Device workspace bytes of spade_scheme_select (budget NULL) or of
 * spade_attn_schemes (its budget); 0 if anything is invalid. */
size_t spade_schemes_workspace_bytes(const spade_problem* p, const spade_block_shape* candidates,
                                     int32_t num_candidates, const spade_budget* budget);

/* Aggregation Evaluation + Policy Application: for every (b, h) and every
 * candidate c, agg[c, b*H+h] = sum_j n_j (q_sics_j + k_sics_j) / (2 N), the
 * token-weighted mean of the per-block SICS of Q and K under that blocking
 * (each per-block SICS as spade_summarize_sics stores it, fp32; the sum in
 * fp64; agg stored as fp32, may be NULL); scheme[b*H+h] = the candidate with
 * the largest aggregate in fp64, ties to the lower index.  candidates: HOST
 * array; agg: device fp32 [C, B*H]; scheme: device int32 [B*H]. */
spade_status spade_scheme_select(const spade_problem* p, const void* q, const void* k,
                                 const spade_block_shape* candidates, int32_t num_candidates, float* agg,
                                 int32_t* scheme, void* workspace, size_t ws_bytes, void* stream);

/* Head-wise schemes end to end: spade_scheme_select, then for each candidate
 * one launch segment of the whole path (summarize, estimate/select, block-
 * sparse attention) over the heads that chose it (Head Grouping), each with
 * its own blocking; every output element is written by exactly one segment.
 * budget as for spade_attn, valid for every candidate's block count.  The
 * CSR of each segment stays in the workspace.  No host synchronisation.
 * For bf16, candidate 0's per-block SICS come from one fused pass over every
 * head that also summarizes and packs Q, K, V into its operand tiles (gist.
 * science technical summary, "Methodology 3", Kernel Fusion: blocking,
 * summarization and intra-block estimation in one kernel); candidate 0's
 * segment reuses those tiles.  agg and scheme equal spade_scheme_select's
 * bit for bit. */
spade_status spade_attn_schemes(const spade_problem* p, const void* q, const void* k, const void* v,
                                const spade_block_shape* candidates, int32_t num_candidates,
                                const spade_budget* budget, void* o, float* agg, int32_t* scheme,
                                void* workspace, size_t ws_bytes, void* stream);

/* Measurement hook for benchmarks: while both events (hipEvent_t) are
 * non-NULL, every later spade_block_sparse_attn / spade_attn call on this host
 * thread records `start` just before and `stop` just after its flash
 * attention kernel, on the call's stream (the caller owns the events and reads
 * them with hipEventElapsedTime).  Pass NULLs to turn recording off. */
void spade_profile_events(void* start, void* stop);

/* Test hook (host only): which walk the bf16 attention kernel takes for this
 * problem -- 1: the kept blocks' keys streamed back to back (every block a
 * multiple of 8 tokens and at least 32, and a full block at least 16 keys
 * short of whole 32-key subtiles), 0: each block padded to whole subtiles,
 * -1: invalid problem. */
int32_t spade_debug_dense_walk(const spade_problem* p);

/* Test hook: the fp64 scores S [B, H, nblk, nblk] that estimate/select uses. */
spade_status spade_debug_scores(const spade_problem* p, const float* q_mean, const float* k_mean,
                                double* scores, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPADE_H */
