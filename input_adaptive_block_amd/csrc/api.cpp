// Host side of the C ABI: validation, workspace carve-up and the launch
// sequence of each entry point (all kernels on the caller's stream).
#include <math.h>
#include <string.h>

#include <atomic>

#include "../../include/spade.h"
#include "spade_internal.h"

namespace spade {
namespace {

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Fill g from p; returns SPADE_OK or the reason the shape is rejected.
spade_status make_geom(const spade_problem* p, Geom* g) {
  if (p == nullptr) return SPADE_ERR_INVALID_ARG;
  if (p->B < 0 || p->H < 0 || p->d <= 0) return SPADE_ERR_INVALID_ARG;
  if (p->T <= 0 || p->Hh <= 0 || p->W <= 0) return SPADE_ERR_INVALID_ARG;
  if (p->bt <= 0 || p->bh <= 0 || p->bw <= 0) return SPADE_ERR_INVALID_ARG;
  if (p->dtype != SPADE_BF16 && p->dtype != SPADE_F32) return SPADE_ERR_INVALID_ARG;
  if (!(p->scale >= 0.0f) || isinf(p->scale)) return SPADE_ERR_INVALID_ARG;  // NaN, <0, inf
  if (p->summarizer != SPADE_SUM_MEAN && p->summarizer != SPADE_SUM_MAX && p->summarizer != SPADE_SUM_MIN)
    return SPADE_ERR_INVALID_ARG;
  const long long N = (long long)p->T * p->Hh * p->W;
  if (N != (long long)p->N) return SPADE_ERR_INVALID_ARG;
  if (p->d != 64 && p->d != 128) return SPADE_ERR_UNSUPPORTED;
  if (p->H > kMaxHeads) return SPADE_ERR_UNSUPPORTED;
  const int bt = p->bt < p->T ? p->bt : p->T;
  const int bh = p->bh < p->Hh ? p->bh : p->Hh;
  const int bw = p->bw < p->W ? p->bw : p->W;
  const long long ntok = (long long)bt * bh * bw;
  if (ntok > kMaxBlockTokens) return SPADE_ERR_UNSUPPORTED;
  const long long nT = (p->T + p->bt - 1) / p->bt, nH = (p->Hh + p->bh - 1) / p->bh,
                  nW = (p->W + p->bw - 1) / p->bw;
  const long long nblk = nT * nH * nW;
  if (nblk > kMaxBlocks) return SPADE_ERR_UNSUPPORTED;
  const long long BH = (long long)p->B * p->H;
  const long long R = BH * nblk;
  const int P = (int)((ntok + 31) / 32 * 32);
  if (R * ((P + 127) / 128) >= (1LL << 31)) return SPADE_ERR_UNSUPPORTED;
  if (BH * N * p->d >= (1LL << 50)) return SPADE_ERR_UNSUPPORTED;
  g->B = p->B; g->H = p->H; g->N = p->N; g->d = p->d;
  g->T = p->T; g->Hh = p->Hh; g->W = p->W;
  g->bt = p->bt; g->bh = p->bh; g->bw = p->bw;
  g->nT = (int)nT; g->nH = (int)nH; g->nW = (int)nW; g->nblk = (int)nblk;
  g->ntok = (int)ntok;
  g->P = P;
  g->BH = (int)BH;
  g->R = (int)R;
  g->bf16 = p->dtype == SPADE_BF16 ? 1 : 0;
  g->op = p->summarizer;
  // dense key streaming: when padding a full block to whole 32-key subtiles
  // would add at least 16 keys (72 -> 96, 40 -> 64; not 120 -> 128, where the
  // padded walk is faster), and every block extent (full or edge) along each
  // axis gives a multiple of 8 tokens, at least 32
  {
    const int ext[3][2] = {{bt, (int)(p->T % p->bt)}, {bh, (int)(p->Hh % p->bh)}, {bw, (int)(p->W % p->bw)}};
    bool dense = p->dtype == SPADE_BF16 && P - ntok >= 16;
    for (int a = 0; a < 2; ++a)
      for (int b = 0; b < 2; ++b)
        for (int c = 0; c < 2; ++c) {
          const int et = ext[0][a], eh = ext[1][b], ew = ext[2][c];
          if (et == 0 || eh == 0 || ew == 0) continue;  // no edge along that axis
          const int n = et * eh * ew;
          if (n % 8 != 0 || n < 32) dense = false;
        }
    g->dense = dense ? 1 : 0;
  }
  g->hsel = nullptr;
  g->hval = 0;
  return SPADE_OK;
}

// Blocks per row for COUNT / RATIO (host arithmetic in double); with a window
// a budget of 0 keeps no block by score.
int keep_k(int mode, float v, int nblk, bool window) {
  if (mode == SPADE_KEEP_COUNT) return (int)v;
  long long k = (long long)ceil((double)v * nblk - 1e-6);
  const long long lo = window ? 0 : 1;
  if (k < lo) k = lo;
  if (k > nblk) k = nblk;
  return (int)k;
}

// Number of blocks in the static window of block i (clipped to the grid).
long long window_size(const Geom& g, int i, int wt, int wh, int ww) {
  const int it = i / (g.nH * g.nW), rem = i - it * g.nH * g.nW;
  const int ih = rem / g.nW, iw = rem - ih * g.nW;
  auto span = [](int c, int r, int n) -> long long {
    const long long lo = c - (long long)r < 0 ? 0 : c - (long long)r;
    const long long hi = c + (long long)r > n - 1 ? n - 1 : c + (long long)r;
    return hi - lo + 1;
  };
  return span(it, wt, g.nT) * span(ih, wh, g.nH) * span(iw, ww, g.nW);
}

spade_status check_budget(const spade_budget* bgt, const Geom& g) {
  if (bgt == nullptr) return SPADE_ERR_INVALID_ARG;
  if (bgt->mode != SPADE_KEEP_COUNT && bgt->mode != SPADE_KEEP_RATIO && bgt->mode != SPADE_KEEP_MASS)
    return SPADE_ERR_INVALID_ARG;
  if (g.H > 0 && bgt->per_head == nullptr) return SPADE_ERR_INVALID_ARG;
  const bool win = bgt->window_enable != 0;
  if (win && (bgt->window_t < 0 || bgt->window_h < 0 || bgt->window_w < 0)) return SPADE_ERR_INVALID_ARG;
  const float lo = win ? 0.0f : 1.0f;
  for (int h = 0; h < g.H; ++h) {
    const float v = bgt->per_head[h];
    if (!(v == v) || isinf(v)) return SPADE_ERR_INVALID_ARG;
    if (bgt->mode == SPADE_KEEP_COUNT) {
      if (v != floorf(v) || v < lo || v > (float)g.nblk) return SPADE_ERR_INVALID_ARG;
    } else if (!((v > 0.0f || (win && v == 0.0f)) && v <= 1.0f)) {
      return SPADE_ERR_INVALID_ARG;
    }
  }
  return SPADE_OK;
}

long long max_nnz(const Geom& g, const spade_budget* bgt) {
  if (bgt->mode == SPADE_KEEP_MASS) return (long long)g.R * g.nblk;
  const bool win = bgt->window_enable != 0;
  long long per_batch = 0;
  for (int h = 0; h < g.H; ++h) {
    const long long k = keep_k(bgt->mode, bgt->per_head[h], g.nblk, win);
    if (!win) {
      per_batch += k * g.nblk;
      continue;
    }
    for (int i = 0; i < g.nblk; ++i) {
      const long long u = k + window_size(g, i, bgt->window_t, bgt->window_h, bgt->window_w);
      per_batch += u < g.nblk ? u : g.nblk;
    }
  }
  return per_batch * g.B;
}

int num_cus() {
  static std::atomic<int> cache[64];  // per device; host threads may race to fill it with the same value
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

inline float attn_scale(const spade_problem* p) {
  return p->scale > 0.0f ? p->scale : (float)(1.0 / sqrt((double)p->d));
}

inline double est_scale(const spade_problem* p) {
  return p->scale > 0.0f ? (double)p->scale : 1.0 / sqrt((double)p->d);
}

inline spade_status dev(hipError_t e) { return e == hipSuccess ? SPADE_OK : SPADE_ERR_DEVICE; }

thread_local hipEvent_t g_prof_start = nullptr, g_prof_stop = nullptr;

// The attention launch, bracketed by the measurement events when they are set.
template <class F>
spade_status timed_attention(hipStream_t s, F launch) {
  if (g_prof_start && g_prof_stop && hipEventRecord(g_prof_start, s) != hipSuccess) return SPADE_ERR_DEVICE;
  const hipError_t e = launch();
  if (e != hipSuccess) return SPADE_ERR_DEVICE;
  if (g_prof_start && g_prof_stop && hipEventRecord(g_prof_stop, s) != hipSuccess) return SPADE_ERR_DEVICE;
  return SPADE_OK;
}

#define SPADE_TRY(expr)                       \
  do {                                        \
    const spade_status st_ = (expr);          \
    if (st_ != SPADE_OK) return st_;          \
  } while (0)

SelectArgs make_select_args(const spade_budget* bgt, const Geom& g) {
  SelectArgs a;
  memset(&a, 0, sizeof(a));
  a.mode = bgt->mode;
  const bool win = bgt->window_enable != 0;
  for (int h = 0; h < g.H; ++h) {
    if (bgt->mode == SPADE_KEEP_MASS)
      a.tau[h] = (double)bgt->per_head[h];
    else
      a.k[h] = keep_k(bgt->mode, bgt->per_head[h], g.nblk, win);
  }
  a.window = win ? 1 : 0;
  a.wt = bgt->window_t;
  a.wh = bgt->window_h;
  a.ww = bgt->window_w;
  return a;
}

char* ws_ptr(void* ws, size_t off) { return reinterpret_cast<char*>(ws) + off; }

// every workspace region starts on a 256-byte boundary of the workspace, and
// the kernels read and write them with 16-byte accesses
bool misaligned(const void* ws) { return (reinterpret_cast<uintptr_t>(ws) & 255u) != 0; }

// attn_counter: the attention kernel's unit counter, cleared by the last
// kernel of the selection when an attention launch follows (else null)
spade_status run_select(const spade_problem* p, const Geom& g, const Workspace& L, const float* qm,
                        const float* km, const spade_budget* bgt, int* row_ptr, int* col_idx, void* ws,
                        int* attn_counter, hipStream_t s) {
  int* counts = reinterpret_cast<int*>(ws_ptr(ws, L.counts));
  uint32_t* mask = reinterpret_cast<uint32_t*>(ws_ptr(ws, L.mask));
  const SelectArgs a = make_select_args(bgt, g);
  if (fused_select_fits(g)) {
    // scores of a row tile stay in LDS
    SPADE_TRY(dev(launch_estimate_select(g, qm, km, est_scale(p), a, counts, mask, L.mask_words, s)));
  } else {
    double* scores = reinterpret_cast<double*>(ws_ptr(ws, L.scores));
    SPADE_TRY(dev(launch_scores(g, qm, km, est_scale(p), scores, s)));
    SPADE_TRY(dev(launch_select(g, scores, a, counts, mask, L.mask_words, s)));
  }
  return dev(launch_csr(g, counts, mask, L.mask_words, row_ptr, col_idx,
                        reinterpret_cast<int*>(ws_ptr(ws, L.scan)), attn_counter, s));
}

}  // namespace

Workspace workspace_layout(const Geom& g) {
  Workspace L;
  size_t off = 0;
  L.mask_words = (g.nblk + 31) / 32;
  L.counts = off; off = align256(off + (size_t)g.R * 4);
  L.mask = off; off = align256(off + (size_t)g.R * L.mask_words * 4);
  // fp64 scores in HBM only for rows wider than the fused kernel's LDS tile
  L.scores = off; off = align256(off + (fused_select_fits(g) ? 0 : (size_t)g.R * g.nblk * 8));
  L.scan = off; off = align256(off + ((size_t)scan_chunks(g.R) + 1) * 4);
  L.select_total = off;  // everything above is all that selection touches
  L.qmean = off; off = align256(off + (size_t)g.BH * g.nblk * g.d * 4);
  L.kmean = off; off = align256(off + (size_t)g.BH * g.nblk * g.d * 4);
  // packed tiles plus two spare 32-row subtiles: the attention kernel copies
  // whole two-subtile stages, which may run one subtile past a block's tile
  const size_t pack = g.bf16 ? ((size_t)g.BH * g.nblk * g.P + 64) * g.d * 2 : 0;
  L.qpack = off; off = align256(off + pack);
  L.kpack = off; off = align256(off + pack);
  L.vpack = off; off = align256(off + pack);
  L.counter = off; off = align256(off + 4);
  L.total = off;
  return L;
}

spade_status estimate_select_entry(const spade_problem* p, const float* q_mean, const float* k_mean,
                                   const spade_budget* budget, int32_t* row_ptr, int32_t* col_idx,
                                   int64_t col_capacity, void* ws, size_t ws_bytes, ScratchLookup lookup,
                                   hipStream_t s) {
  Geom g;
  SPADE_TRY(make_geom(p, &g));
  SPADE_TRY(check_budget(budget, g));
  const long long need = max_nnz(g, budget);
  if (need >= (1LL << 31)) return SPADE_ERR_UNSUPPORTED;
  if (col_capacity < need) return SPADE_ERR_CAPACITY;
  if (!row_ptr) return SPADE_ERR_INVALID_ARG;
  const Workspace L = workspace_layout(g);
  // a caller's workspace is checked against the documented whole size; the
  // library's own buffer only has to hold the selection part
  if (ws_bytes < (lookup ? L.select_total : L.total)) return SPADE_ERR_CAPACITY;
  if (g.R == 0) return dev(launch_scan(g, nullptr, row_ptr, nullptr, s));
  if (!q_mean || !k_mean || !col_idx) return SPADE_ERR_INVALID_ARG;
  if (lookup) SPADE_TRY(dev(lookup(&ws)));
  if (!ws || misaligned(ws)) return SPADE_ERR_INVALID_ARG;
  return run_select(p, g, L, q_mean, k_mean, budget, row_ptr, col_idx, ws, nullptr, s);
}

}  // namespace spade

using namespace spade;

extern "C" {

int32_t spade_num_blocks(const spade_problem* p) {
  Geom g;
  if (make_geom(p, &g) != SPADE_OK) return -1;
  return g.nblk;
}

int64_t spade_max_nnz(const spade_problem* p, const spade_budget* budget) {
  Geom g;
  if (make_geom(p, &g) != SPADE_OK) return -1;
  if (check_budget(budget, g) != SPADE_OK) return -1;
  return max_nnz(g, budget);
}

size_t spade_workspace_bytes(const spade_problem* p) {
  Geom g;
  if (make_geom(p, &g) != SPADE_OK) return 0;
  return workspace_layout(g).total;
}

spade_status spade_check(const spade_problem* p, const spade_budget* budget, int64_t col_capacity) {
  Geom g;
  SPADE_TRY(make_geom(p, &g));
  if (budget != nullptr) {
    SPADE_TRY(check_budget(budget, g));
    const long long need = max_nnz(g, budget);
    if (need >= (1LL << 31)) return SPADE_ERR_UNSUPPORTED;
    if (col_capacity >= 0 && col_capacity < need) return SPADE_ERR_CAPACITY;
  }
  return SPADE_OK;
}

const char* spade_status_string(spade_status s) {
  switch (s) {
    case SPADE_OK: return "SPADE_OK";
    case SPADE_ERR_INVALID_ARG: return "SPADE_ERR_INVALID_ARG";
    case SPADE_ERR_UNSUPPORTED: return "SPADE_ERR_UNSUPPORTED";
    case SPADE_ERR_CAPACITY: return "SPADE_ERR_CAPACITY";
    case SPADE_ERR_DEVICE: return "SPADE_ERR_DEVICE";
  }
  return "SPADE_ERR_UNKNOWN";
}

spade_status spade_summarize(const spade_problem* p, const void* q, const void* k, float* q_mean,
                             float* k_mean, void* stream) {
  Geom g;
  SPADE_TRY(make_geom(p, &g));
  if (g.BH == 0) return SPADE_OK;
  if (!q || !k || !q_mean || !k_mean) return SPADE_ERR_INVALID_ARG;
  return dev(launch_summarize(g, p->dtype == SPADE_BF16, q, k, nullptr, q_mean, k_mean, nullptr, nullptr,
                              nullptr, (hipStream_t)stream));
}

spade_status spade_summarize_sics(const spade_problem* p, const void* q, const void* k, float* q_mean,
                                  float* k_mean, float* q_sics, float* k_sics, void* stream) {
  Geom g;
  SPADE_TRY(make_geom(p, &g));
  if (g.BH == 0) return SPADE_OK;
  if (!q || !k || !q_mean || !k_mean) return SPADE_ERR_INVALID_ARG;
  return dev(launch_summarize_sics(g, p->dtype == SPADE_BF16, q, k, q_mean, k_mean, q_sics, k_sics,
                                   (hipStream_t)stream));
}

spade_status spade_estimate_select(const spade_problem* p, const float* q_mean, const float* k_mean,
                                   const spade_budget* budget, int32_t* row_ptr, int32_t* col_idx,
                                   int64_t col_capacity, void* workspace, size_t ws_bytes, void* stream) {
  return estimate_select_entry(p, q_mean, k_mean, budget, row_ptr, col_idx, col_capacity, workspace, ws_bytes,
                               nullptr, (hipStream_t)stream);
}

spade_status spade_block_sparse_attn(const spade_problem* p, const void* q, const void* k, const void* v,
                                     const int32_t* row_ptr, const int32_t* col_idx, int64_t col_capacity,
                                     void* o, void* workspace, size_t ws_bytes, void* stream) {
  Geom g;
  SPADE_TRY(make_geom(p, &g));
  if (col_capacity < 0) return SPADE_ERR_INVALID_ARG;
  const Workspace L = workspace_layout(g);
  if (ws_bytes < L.total) return SPADE_ERR_CAPACITY;
  if (g.R == 0) return SPADE_OK;
  if (!q || !k || !v || !row_ptr || !o || !workspace || misaligned(workspace)) return SPADE_ERR_INVALID_ARG;
  if (col_capacity > 0 && !col_idx) return SPADE_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  const float scale = attn_scale(p);
  if (p->dtype == SPADE_BF16) {
    void* qp = ws_ptr(workspace, L.qpack);
    void* kp = ws_ptr(workspace, L.kpack);
    void* vp = ws_ptr(workspace, L.vpack);
    SPADE_TRY(dev(launch_summarize(g, true, q, k, v, nullptr, nullptr, qp, kp, vp, s)));
    return timed_attention(s, [&] {
      return launch_bsattn_bf16(g, qp, kp, vp, row_ptr, col_idx, col_capacity, scale, o,
                                reinterpret_cast<int*>(ws_ptr(workspace, L.counter)), false, num_cus(), s);
    });
  }
  return timed_attention(s, [&] {
    return launch_bsattn_f32(g, (const float*)q, (const float*)k, (const float*)v, row_ptr, col_idx,
                             col_capacity, scale, (float*)o, s);
  });
}

spade_status spade_attn(const spade_problem* p, const void* q, const void* k, const void* v,
                        const spade_budget* budget, void* o, int32_t* row_ptr, int32_t* col_idx,
                        int64_t col_capacity, void* workspace, size_t ws_bytes, void* stream) {
  Geom g;
  SPADE_TRY(make_geom(p, &g));
  SPADE_TRY(check_budget(budget, g));
  const long long need = max_nnz(g, budget);
  if (need >= (1LL << 31)) return SPADE_ERR_UNSUPPORTED;
  if (col_capacity < need) return SPADE_ERR_CAPACITY;
  const Workspace L = workspace_layout(g);
  if (ws_bytes < L.total) return SPADE_ERR_CAPACITY;
  if (!row_ptr) return SPADE_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  if (g.R == 0) return dev(launch_scan(g, nullptr, row_ptr, nullptr, s));
  if (!q || !k || !v || !o || !col_idx || !workspace || misaligned(workspace)) return SPADE_ERR_INVALID_ARG;
  float* qm = reinterpret_cast<float*>(ws_ptr(workspace, L.qmean));
  float* km = reinterpret_cast<float*>(ws_ptr(workspace, L.kmean));
  const float scale = attn_scale(p);
  if (p->dtype == SPADE_BF16) {
    void* qp = ws_ptr(workspace, L.qpack);
    void* kp = ws_ptr(workspace, L.kpack);
    void* vp = ws_ptr(workspace, L.vpack);
    SPADE_TRY(dev(launch_summarize(g, true, q, k, v, qm, km, qp, kp, vp, s)));
    int* counter = reinterpret_cast<int*>(ws_ptr(workspace, L.counter));
    SPADE_TRY(run_select(p, g, L, qm, km, budget, row_ptr, col_idx, workspace, counter, s));
    return timed_attention(s, [&] {
      return launch_bsattn_bf16(g, qp, kp, vp, row_ptr, col_idx, col_capacity, scale, o, counter, true,
                                num_cus(), s);
    });
  }
  SPADE_TRY(dev(launch_summarize(g, false, q, k, nullptr, qm, km, nullptr, nullptr, nullptr, s)));
  SPADE_TRY(run_select(p, g, L, qm, km, budget, row_ptr, col_idx, workspace, nullptr, s));
  return timed_attention(s, [&] {
    return launch_bsattn_f32(g, (const float*)q, (const float*)k, (const float*)v, row_ptr, col_idx,
                             col_capacity, scale, (float*)o, s);
  });
}

void spade_profile_events(void* start, void* stop) {
  g_prof_start = (hipEvent_t)start;
  g_prof_stop = (hipEvent_t)stop;
}

int32_t spade_debug_dense_walk(const spade_problem* p) {
  Geom g;
  if (make_geom(p, &g) != SPADE_OK) return -1;
  return g.dense;
}

spade_status spade_debug_scores(const spade_problem* p, const float* q_mean, const float* k_mean,
                                double* scores, void* stream) {
  Geom g;
  SPADE_TRY(make_geom(p, &g));
  if (g.BH == 0) return SPADE_OK;
  if (!q_mean || !k_mean || !scores) return SPADE_ERR_INVALID_ARG;
  return dev(launch_scores(g, q_mean, k_mean, est_scale(p), scores, (hipStream_t)stream));
}

}  // extern "C"

// ---------------------------------------------------------------------------
// scheme generation and head-wise schemes
// ---------------------------------------------------------------------------
namespace {

constexpr int kMaxCandidates = 16;

struct SchemeLayout {
  size_t agg64;    // double [C * BH]
  size_t qsics;    // float [BH * max nblk]
  size_t ksics;    // float [BH * max nblk]
  size_t row_ptr;  // int32 [BH * max nblk + 1]      (head-wise attention only)
  size_t col_idx;  // int32 [max over candidates of the CSR capacity]
  size_t pipe;     // the single-scheme workspace of the largest candidate
  size_t total_select;
  size_t total_attn;
  long long cap;   // col_idx entries
};

spade_status scheme_geoms(const spade_problem* p, const spade_block_shape* cand, int C, Geom* gs) {
  if (p == nullptr || cand == nullptr || C < 1) return SPADE_ERR_INVALID_ARG;
  if (C > kMaxCandidates) return SPADE_ERR_UNSUPPORTED;
  for (int c = 0; c < C; ++c) {
    spade_problem pc = *p;
    pc.bt = cand[c].bt;
    pc.bh = cand[c].bh;
    pc.bw = cand[c].bw;
    SPADE_TRY(make_geom(&pc, &gs[c]));
  }
  return SPADE_OK;
}

// budget may be null (scheme selection only)
spade_status scheme_layout(const Geom* gs, int C, const spade_budget* budget, SchemeLayout* L) {
  int max_nblk = 0;
  size_t pipe = 0;
  long long cap = 0;
  for (int c = 0; c < C; ++c) {
    max_nblk = gs[c].nblk > max_nblk ? gs[c].nblk : max_nblk;
    const size_t w = workspace_layout(gs[c]).total;
    pipe = w > pipe ? w : pipe;
    if (budget) {
      SPADE_TRY(check_budget(budget, gs[c]));
      const long long n = max_nnz(gs[c], budget);
      if (n >= (1LL << 31)) return SPADE_ERR_UNSUPPORTED;
      cap = n > cap ? n : cap;
    }
  }
  const Geom& g = gs[0];
  size_t off = 0;
  L->agg64 = off; off = align256(off + (size_t)C * g.BH * 8);
  L->qsics = off; off = align256(off + (size_t)g.BH * max_nblk * 4);
  L->ksics = off; off = align256(off + (size_t)g.BH * max_nblk * 4);
  L->total_select = off;
  L->row_ptr = off; off = align256(off + ((size_t)g.BH * max_nblk + 1) * 4);
  L->col_idx = off; off = align256(off + (size_t)(cap > 0 ? cap : 1) * 4);
  L->pipe = off; off = align256(off + pipe);
  L->total_attn = off;
  L->cap = cap;
  return SPADE_OK;
}

// Aggregate SICS of every candidate and the head-wise choice.  With pipe set
// (bf16 head-wise attention), candidate 0's SICS come from its pack pass over
// every head -- layout transformation, summarization and intra-block
// estimation in one read of Q, K, V -- whose tiles its launch segment reuses.
spade_status run_scheme_select(const spade_problem* p, const Geom* gs, int C, const SchemeLayout& L,
                               const void* q, const void* k, const void* v, void* pipe, float* agg,
                               int32_t* scheme, void* ws, hipStream_t s) {
  double* agg64 = reinterpret_cast<double*>(ws_ptr(ws, L.agg64));
  float* qs = reinterpret_cast<float*>(ws_ptr(ws, L.qsics));
  float* ks = reinterpret_cast<float*>(ws_ptr(ws, L.ksics));
  const bool bf16 = p->dtype == SPADE_BF16;
  for (int c = 0; c < C; ++c) {
    if (c == 0 && pipe != nullptr && bf16) {
      const Workspace W = workspace_layout(gs[0]);
      SPADE_TRY(dev(launch_summarize_pack_sics(
          gs[0], q, k, v, reinterpret_cast<float*>(ws_ptr(pipe, W.qmean)),
          reinterpret_cast<float*>(ws_ptr(pipe, W.kmean)), ws_ptr(pipe, W.qpack), ws_ptr(pipe, W.kpack),
          ws_ptr(pipe, W.vpack), qs, ks, s)));
    } else {
      SPADE_TRY(dev(launch_summarize_sics(gs[c], bf16, q, k, nullptr, nullptr, qs, ks, s)));
    }
    SPADE_TRY(dev(launch_scheme_aggregate(gs[c], qs, ks, c, agg64, agg, s)));
  }
  return dev(launch_scheme_choose(gs[0].BH, C, agg64, scheme, s));
}

}  // namespace

extern "C" {

size_t spade_schemes_workspace_bytes(const spade_problem* p, const spade_block_shape* candidates,
                                     int32_t num_candidates, const spade_budget* budget) {
  Geom gs[kMaxCandidates];
  if (scheme_geoms(p, candidates, num_candidates, gs) != SPADE_OK) return 0;
  SchemeLayout L;
  if (scheme_layout(gs, num_candidates, budget, &L) != SPADE_OK) return 0;
  return budget ? L.total_attn : L.total_select;
}

spade_status spade_scheme_select(const spade_problem* p, const void* q, const void* k,
                                 const spade_block_shape* candidates, int32_t num_candidates, float* agg,
                                 int32_t* scheme, void* workspace, size_t ws_bytes, void* stream) {
  Geom gs[kMaxCandidates];
  SPADE_TRY(scheme_geoms(p, candidates, num_candidates, gs));
  SchemeLayout L;
  SPADE_TRY(scheme_layout(gs, num_candidates, nullptr, &L));
  if (ws_bytes < L.total_select) return SPADE_ERR_CAPACITY;
  if (gs[0].BH == 0) return SPADE_OK;
  if (!q || !k || !scheme || !workspace || misaligned(workspace)) return SPADE_ERR_INVALID_ARG;
  return run_scheme_select(p, gs, num_candidates, L, q, k, nullptr, nullptr, agg, scheme, workspace,
                           (hipStream_t)stream);
}

spade_status spade_attn_schemes(const spade_problem* p, const void* q, const void* k, const void* v,
                                const spade_block_shape* candidates, int32_t num_candidates,
                                const spade_budget* budget, void* o, float* agg, int32_t* scheme,
                                void* workspace, size_t ws_bytes, void* stream) {
  Geom gs[kMaxCandidates];
  SPADE_TRY(scheme_geoms(p, candidates, num_candidates, gs));
  if (budget == nullptr) return SPADE_ERR_INVALID_ARG;
  SchemeLayout L;
  SPADE_TRY(scheme_layout(gs, num_candidates, budget, &L));
  if (ws_bytes < L.total_attn) return SPADE_ERR_CAPACITY;
  if (gs[0].BH == 0) return SPADE_OK;
  if (!q || !k || !v || !o || !scheme || !workspace || misaligned(workspace)) return SPADE_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  void* pw = ws_ptr(workspace, L.pipe);
  SPADE_TRY(run_scheme_select(p, gs, num_candidates, L, q, k, v, pw, agg, scheme, workspace, s));
  // one launch segment per candidate over the heads that chose it
  int32_t* row_ptr = reinterpret_cast<int32_t*>(ws_ptr(workspace, L.row_ptr));
  int32_t* col_idx = reinterpret_cast<int32_t*>(ws_ptr(workspace, L.col_idx));
  const float scale = attn_scale(p);
  for (int c = 0; c < num_candidates; ++c) {
    Geom g = gs[c];
    g.hsel = scheme;
    g.hval = c;
    const Workspace W = workspace_layout(g);
    float* qm = reinterpret_cast<float*>(ws_ptr(pw, W.qmean));
    float* km = reinterpret_cast<float*>(ws_ptr(pw, W.kmean));
    if (p->dtype == SPADE_BF16) {
      void* qp = ws_ptr(pw, W.qpack);
      void* kp = ws_ptr(pw, W.kpack);
      void* vp = ws_ptr(pw, W.vpack);
      // candidate 0's tiles and means are already in place for every head
      if (c > 0) SPADE_TRY(dev(launch_summarize(g, true, q, k, v, qm, km, qp, kp, vp, s)));
      int* counter = reinterpret_cast<int*>(ws_ptr(pw, W.counter));
      SPADE_TRY(run_select(p, g, W, qm, km, budget, row_ptr, col_idx, pw, counter, s));
      SPADE_TRY(dev(launch_bsattn_bf16(g, qp, kp, vp, row_ptr, col_idx, L.cap, scale, o, counter, true,
                                       num_cus(), s)));
    } else {
      SPADE_TRY(dev(launch_summarize(g, false, q, k, nullptr, qm, km, nullptr, nullptr, nullptr, s)));
      SPADE_TRY(run_select(p, g, W, qm, km, budget, row_ptr, col_idx, pw, nullptr, s));
      SPADE_TRY(dev(launch_bsattn_f32(g, (const float*)q, (const float*)k, (const float*)v, row_ptr, col_idx,
                                      L.cap, scale, (float*)o, s)));
    }
  }
  return SPADE_OK;
}

}  // extern "C"
