// Internal declarations shared by the HIP kernels and the host API.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/spade.h"

namespace spade {

constexpr int kMaxHeads = 256;     // per-head budgets travel as kernel arguments
constexpr int kMaxBlocks = 4096;   // nblk limit (selection keeps a row in registers)
constexpr int kMaxBlockTokens = 1024;

// Geometry of one problem, valid on host and device.
struct Geom {
  int B, H, N, d;
  int T, Hh, W;
  int bt, bh, bw;
  int nT, nH, nW, nblk;
  int ntok;   // bt*bh*bw, tokens of a full block
  int P;      // ntok rounded up to a multiple of 32 (padded tile rows)
  int BH;     // B*H
  int R;      // B*H*nblk selection rows
  int bf16;   // 1: bf16 tensors (packed MFMA tiles), 0: fp32 debug path
  int op;     // block summarizer: 0 mean, 1 max, 2 min
  // 1 when every block (partial edge blocks included) holds a multiple of 8
  // tokens and at least 32, and padding a full block to whole 32-key subtiles
  // would add 16 keys or more (bf16 only): attention streams the kept blocks'
  // keys back to back instead, and V tiles are packed with eight consecutive
  // keys per 16-byte vector
  int dense;
  // head filter of a scheme's launch segment: when hsel is set, only the
  // (b, h) pairs with hsel[b*H + h] == hval are computed (device array)
  const int* hsel;
  int hval;
};

__host__ __device__ inline bool head_active(const Geom& g, int bh) {
  return g.hsel == nullptr || g.hsel[bh] == g.hval;
}

struct BlockBox {
  int t0, h0, w0;  // origin
  int et, eh, ew;  // extents (partial at the far edges)
  int n;           // et*eh*ew
};

__host__ __device__ inline BlockBox block_box(const Geom& g, int j) {
  BlockBox b;
  int it = j / (g.nH * g.nW);
  int rem = j - it * g.nH * g.nW;
  int ih = rem / g.nW;
  int iw = rem - ih * g.nW;
  b.t0 = it * g.bt;
  b.h0 = ih * g.bh;
  b.w0 = iw * g.bw;
  b.et = min(g.bt, g.T - b.t0);
  b.eh = min(g.bh, g.Hh - b.h0);
  b.ew = min(g.bw, g.W - b.w0);
  b.n = b.et * b.eh * b.ew;
  return b;
}

// Raster token of local index l (t-major, then h, then w) inside block b.
__host__ __device__ inline int block_token(const Geom& g, const BlockBox& b, int l) {
  int ehw = b.eh * b.ew;
  int lt = l / ehw;
  int r = l - lt * ehw;
  int lh = r / b.ew;
  int lw = r - lh * b.ew;
  return ((b.t0 + lt) * g.Hh + (b.h0 + lh)) * g.W + (b.w0 + lw);
}

// Budget as passed to the selection kernel (by value).
struct SelectArgs {
  int mode;              // spade_keep_mode
  int k[kMaxHeads];      // COUNT / RATIO: blocks per row of head h (0: none by score)
  double tau[kMaxHeads]; // MASS: threshold of head h (0: none by score)
  int window;            // 1: unite the static window below with the scored set
  int wt, wh, ww;        // window radii in blocks along t, h, w
};

// Workspace carve-up (byte offsets, 256-aligned).
struct Workspace {
  size_t counts;    // int32 [R]
  size_t mask;      // uint32 [R * mask_words]
  size_t scores;    // double [R * nblk] (only when the fused select does not fit)
  size_t scan;      // int32 [scan_chunks(R) + 1]: chunk sums of the CSR scan
  size_t select_total;  // bytes of the four regions above: all that selection touches
  size_t qmean;     // float [BH * nblk * d]
  size_t kmean;     // float [BH * nblk * d]
  size_t qpack;     // bf16 [BH * nblk * P * d]
  size_t kpack;
  size_t vpack;
  size_t counter;   // int32: the attention kernel's unit counter
  size_t total;
  int mask_words;
};

Workspace workspace_layout(const Geom& g);

// ---- launchers (each returns hipSuccess or the launch error) -------------
hipError_t launch_summarize(const Geom& g, bool bf16, const void* q, const void* k, const void* v,
                            float* q_mean, float* k_mean, void* qpack, void* kpack, void* vpack,
                            hipStream_t s);
// block means plus the normalised intra-block cosine similarity (either sics
// pointer may be null)
hipError_t launch_summarize_sics(const Geom& g, bool bf16, const void* q, const void* k, float* q_mean,
                                 float* k_mean, float* q_sics, float* k_sics, hipStream_t s);
// bf16 only: the pack pass of launch_summarize (means + Q/K/V operand tiles)
// that also writes the SICS of every Q and K block, in one read of Q, K, V
hipError_t launch_summarize_pack_sics(const Geom& g, const void* q, const void* k, const void* v,
                                     float* q_mean, float* k_mean, void* qpack, void* kpack, void* vpack,
                                     float* q_sics, float* k_sics, hipStream_t s);
// scheme generation: aggregate SICS of candidate c for every (b, h) from the
// per-block SICS of Q and K, and the head-wise argmax over the candidates
hipError_t launch_scheme_aggregate(const Geom& g, const float* q_sics, const float* k_sics, int c,
                                   double* agg64, float* agg, hipStream_t s);
hipError_t launch_scheme_choose(int BH, int C, const double* agg64, int* scheme, hipStream_t s);
hipError_t launch_scores(const Geom& g, const float* q_mean, const float* k_mean, double scale,
                         double* scores, hipStream_t s);
hipError_t launch_select(const Geom& g, const double* scores, const SelectArgs& a, int* counts,
                         uint32_t* mask, int mask_words, hipStream_t s);
// Estimator and index search in one kernel, the scores of a 16-row tile kept
// in LDS (never written to HBM); for nblk <= kFusedMaxBlocks.
constexpr int kFusedMaxBlocks = 1024;
bool fused_select_fits(const Geom& g);
hipError_t launch_estimate_select(const Geom& g, const float* q_mean, const float* k_mean, double scale,
                                  const SelectArgs& a, int* counts, uint32_t* mask, int mask_words,
                                  hipStream_t s);
// row_ptr from the counts; chunk_sums holds scan_chunks(R) ints (unused when R == 0)
constexpr int kScanChunk = 4096;
inline int scan_chunks(long long R) { return (int)((R + kScanChunk - 1) / kScanChunk); }
hipError_t launch_scan(const Geom& g, const int* counts, int* row_ptr, int* chunk_sums, hipStream_t s);
// row_ptr and col_idx from the counts and row bitmasks; chunk_sums as for
// launch_scan.  attn_counter (may be null) is the attention kernel's unit
// counter, cleared here for an attention launch that follows on the stream.
hipError_t launch_csr(const Geom& g, const int* counts, const uint32_t* mask, int mask_words, int* row_ptr,
                      int* col_idx, int* chunk_sums, int* attn_counter, hipStream_t s);
// counter_cleared: a kernel earlier on the stream has set *counter to 0
// (else the launch clears it first)
hipError_t launch_bsattn_bf16(const Geom& g, const void* qpack, const void* kpack, const void* vpack,
                              const int* row_ptr, const int* col_idx, long long col_capacity,
                              float scale, void* o, int* counter, bool counter_cleared, int num_cus,
                              hipStream_t s);
hipError_t launch_bsattn_f32(const Geom& g, const float* q, const float* k, const float* v,
                             const int* row_ptr, const int* col_idx, long long col_capacity,
                             float scale, float* o, hipStream_t s);

// ---- entry-point bodies shared between source files ----------------------

// Returns the device address of a library-owned scratch buffer for the
// current device.
typedef hipError_t (*ScratchLookup)(void** ptr);

// Checks and launches of the estimate + select entry point.  Without lookup,
// ws is the caller's workspace and ws_bytes must cover the whole documented
// workspace; with lookup, ws_bytes is the library buffer's size, checked
// against the selection part only, and lookup supplies ws after every
// argument check has passed (so rejected calls touch no device).
spade_status estimate_select_entry(const spade_problem* p, const float* q_mean, const float* k_mean,
                                   const spade_budget* budget, int32_t* row_ptr, int32_t* col_idx,
                                   int64_t col_capacity, void* ws, size_t ws_bytes, ScratchLookup lookup,
                                   hipStream_t s);

}  // namespace spade
