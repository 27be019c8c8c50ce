// Estimator and index search.
//
// SPADE technical summary (gist.science), "Methodology 1. vDiT-SSR",
// Summarizer & Estimator Expressions: an inter-block importance score decides
// which blocks each Q block retains; the abstract's executor does this with a
// low-overhead index search, and "3. Head-wise Sparse Attention Execution"
// feeds the result to the attention kernel as a block-sparse row format.
//
// Stages (all on the caller's stream, no host synchronization):
//   scores_kernel   S = scale * qbar kbar^T per head in fp64 on
//                   v_mfma_f64_16x16x4_f64 (summaries are fp32, exact in fp64).
//   select_kernel   one wavefront per row.  The row lives in registers as
//                   64-bit order keys; a bitwise threshold search (64 rounds of
//                   ballots or masked fp64 sums) finds the k-th key (count /
//                   ratio) or the mass cut (mass), ties go to the lower block
//                   id.  Emits the kept set as a bitmask and a count.
//   scan_kernel     row_ptr = exclusive prefix sum of the counts.
//   compact_kernel  one wavefront per row writes the kept ids ascending.
#include "spade_internal.h"

namespace spade {
namespace {

typedef double f64x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// scores
// ---------------------------------------------------------------------------
constexpr int kSRows = 32, kSCols = 64;

template <int D>
__global__ __launch_bounds__(256) void scores_kernel(Geom g, const float* __restrict__ qm,
                                                     const float* __restrict__ km, double scale,
                                                     double* __restrict__ S) {
  constexpr int LD = D + 4;
  __shared__ __attribute__((aligned(16))) float qs[kSRows * LD];
  __shared__ __attribute__((aligned(16))) float ks[kSCols * LD];
  const int bh = blockIdx.z;
  if (!head_active(g, bh)) return;  // another scheme's head (whole workgroup)
  const int row0 = blockIdx.x * kSRows, col0 = blockIdx.y * kSCols;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nb = g.nblk;
  const float* qh = qm + (size_t)bh * nb * D;
  const float* kh = km + (size_t)bh * nb * D;
  // 16-byte loads and stores (rows of D floats; the LDS row stride D + 4
  // keeps every row 16-byte aligned)
  constexpr int V = D / 4;
  for (int t = tid; t < kSRows * V; t += 256) {
    const int r = t / V, c = 4 * (t - r * V);
    const float4 x = (row0 + r < nb) ? *reinterpret_cast<const float4*>(qh + (size_t)(row0 + r) * D + c)
                                     : make_float4(0.f, 0.f, 0.f, 0.f);
    *reinterpret_cast<float4*>(&qs[r * LD + c]) = x;
  }
  for (int t = tid; t < kSCols * V; t += 256) {
    const int r = t / V, c = 4 * (t - r * V);
    const float4 x = (col0 + r < nb) ? *reinterpret_cast<const float4*>(kh + (size_t)(col0 + r) * D + c)
                                     : make_float4(0.f, 0.f, 0.f, 0.f);
    *reinterpret_cast<float4*>(&ks[r * LD + c]) = x;
  }
  __syncthreads();
  const int wr = wave >> 1, wc = wave & 1;
  f64x4 acc0 = {0.0, 0.0, 0.0, 0.0}, acc1 = {0.0, 0.0, 0.0, 0.0};
  const int li = lane & 15, lk = lane >> 4;
#pragma unroll 4
  for (int s = 0; s < D / 4; ++s) {
    const double a = (double)qs[(16 * wr + li) * LD + 4 * s + lk];
    const double b0 = (double)ks[(32 * wc + li) * LD + 4 * s + lk];
    const double b1 = (double)ks[(32 * wc + 16 + li) * LD + 4 * s + lk];
    acc0 = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b0, acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b1, acc1, 0, 0, 0);
  }
  double* Sh = S + (size_t)bh * nb * nb;
  // v_mfma_f64_16x16x4_f64 leaves D[lk + 4 v][li] in lane (lk, li), register v
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int i = row0 + 16 * wr + lk + 4 * v;
    const int j0 = col0 + 32 * wc + li, j1 = j0 + 16;
    if (i < nb) {
      if (j0 < nb) Sh[(size_t)i * nb + j0] = scale * acc0[v];
      if (j1 < nb) Sh[(size_t)i * nb + j1] = scale * acc1[v];
    }
  }
}

// ---------------------------------------------------------------------------
// selection
// ---------------------------------------------------------------------------

// exp(x) for x <= 0 in fp64: Cody-Waite reduction x = k ln2 + r, |r| <= ln2/2,
// with ln2 split into a 32-bit-exact high part and a low remainder, then the
// Taylor series of exp(r) to degree 14 (truncation < 1e-18 relative) by Horner,
// and a scale by 2^k.
__device__ inline double exp_nonpos(double x) {
  if (x < -745.2) return 0.0;
  const double kLog2e = 1.4426950408889634074;
  const double kLn2Hi = 6.93147180369123816490e-01;
  const double kLn2Lo = 1.90821492927058770002e-10;
  const double kd = __builtin_rint(x * kLog2e);
  const double r = (x - kd * kLn2Hi) - kd * kLn2Lo;
  double p = 1.0 / 87178291200.0;          // 1/14!
  p = p * r + 1.0 / 6227020800.0;          // 1/13!
  p = p * r + 1.0 / 479001600.0;           // 1/12!
  p = p * r + 1.0 / 39916800.0;            // 1/11!
  p = p * r + 1.0 / 3628800.0;             // 1/10!
  p = p * r + 1.0 / 362880.0;              // 1/9!
  p = p * r + 1.0 / 40320.0;               // 1/8!
  p = p * r + 1.0 / 5040.0;                // 1/7!
  p = p * r + 1.0 / 720.0;                 // 1/6!
  p = p * r + 1.0 / 120.0;                 // 1/5!
  p = p * r + 1.0 / 24.0;                  // 1/4!
  p = p * r + 1.0 / 6.0;                   // 1/3!
  p = p * r + 0.5;                         // 1/2!
  p = p * r + 1.0;
  p = p * r + 1.0;
  const int k = (int)kd;
  // 2^k may be subnormal for k < -1022: split the scaling in two steps
  if (k < -1000) return __builtin_ldexp(__builtin_ldexp(p, k + 600), -600);
  return __builtin_ldexp(p, k);
}

__device__ inline uint64_t order_key(double s) {
  const double x = s + 0.0;  // -0 -> +0 so equal scores compare equal
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

__device__ inline double wave_sum(double x) {
  // butterfly: every lane ends with the same bits (each step adds the same
  // pair of operands, only in swapped order)
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) x += __shfl_xor(x, off);
  return x;
}

__device__ inline double wave_max(double x) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) x = fmax(x, __shfl_xor(x, off));
  return x;
}

// The bitwise threshold searches below fix the threshold's bits from the
// top.  The threshold they converge to is itself one of the keys (the
// smallest key kept), so once exactly one key shares the bits fixed so far,
// that key is the threshold and the remaining rounds can be skipped (checked
// every fourth round).  Returns true and sets T when that is the case.
template <int E>
__device__ inline bool isolated_threshold(const uint64_t (&key)[E], int bit, uint64_t& T) {
  const uint64_t hi = ~((1ull << bit) - 1ull);
  int c = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) c += __popcll(__ballot((key[e] & hi) == T));
  if (c != 1) return false;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint64_t b = __ballot((key[e] & hi) == T);
    if (b != 0ull) {
      const int l = __builtin_ctzll(b);
      const uint32_t lo32 = __shfl((uint32_t)key[e], l), hi32 = __shfl((uint32_t)(key[e] >> 32), l);
      T = ((uint64_t)hi32 << 32) | lo32;
    }
  }
  return true;
}

template <int E>
__global__ __launch_bounds__(256) void select_kernel(Geom g, const double* __restrict__ S, SelectArgs a,
                                                     int* __restrict__ counts, uint32_t* __restrict__ mask,
                                                     int mask_words) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= g.R) return;  // whole wave exits together
  const int nK = g.nblk;
  const int h = (row / nK) % g.H;
  if (!head_active(g, row / nK)) {
    // another scheme's head: an empty row (its scores were never computed)
    uint32_t* mrow = mask + (size_t)row * mask_words;
    for (int w = lane; w < mask_words; w += 64) mrow[w] = 0u;
    if (lane == 0) counts[row] = 0;
    return;
  }
  const double* Sr = S + (size_t)row * nK;

  uint64_t key[E];
  double sv[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = 64 * e + lane;
    if (j < nK) {
      sv[e] = Sr[j];
      key[e] = order_key(sv[e]);
    } else {
      sv[e] = -__builtin_huge_val();
      key[e] = 0ull;  // below every real score
    }
  }

  bool kept[E];
  if (a.mode != 2) {
    // ---- count / ratio: the k-th largest key, ties to the lower id ----
    const int kk = a.k[h];
    uint64_t T = 0ull;
    for (int bit = 63; bit >= 0; --bit) {
      const uint64_t cand = T | (1ull << bit);
      int cnt = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) cnt += __popcll(__ballot(key[e] >= cand));
      if (cnt >= kk) T = cand;
      if ((bit & 3) == 0 && bit > 0 && isolated_threshold(key, bit, T)) break;
    }
    int gt = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) gt += __popcll(__ballot(key[e] > T));
    int need = kk - gt;  // ties at T to keep, lowest ids first
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint64_t tie = __ballot(key[e] == T);
      const int rank = __popcll(tie & lt_mask);
      kept[e] = key[e] > T || (key[e] == T && rank < need);
      need -= __popcll(tie);
    }
  } else {
    // ---- mass: shortest (S desc, id asc) prefix with softmax mass >= tau ----
    double mx = sv[0];
#pragma unroll
    for (int e = 1; e < E; ++e) mx = fmax(mx, sv[e]);
    mx = wave_max(mx);
    double p[E];
    double loc = 0.0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      p[e] = (64 * e + lane < nK) ? exp_nonpos(sv[e] - mx) : 0.0;
      loc += p[e];
    }
    const double Z = wave_sum(loc);
    const double target = a.tau[h] * Z;
    // largest T with mass(key >= T) >= target; mass(key >= T) is monotone
    // non-increasing in T because every partial sum only drops non-negative
    // terms when T grows
    uint64_t T = 0ull;
    for (int bit = 63; bit >= 0; --bit) {
      const uint64_t cand = T | (1ull << bit);
      double f = 0.0;
#pragma unroll
      for (int e = 0; e < E; ++e) f += (key[e] >= cand) ? p[e] : 0.0;
      if (wave_sum(f) >= target) T = cand;
      if ((bit & 3) == 0 && bit > 0 && isolated_threshold(key, bit, T)) break;
    }
    double f = 0.0;
#pragma unroll
    for (int e = 0; e < E; ++e) f += (key[e] > T) ? p[e] : 0.0;
    double cum = wave_sum(f);  // mass strictly above the cut
    // ties at T join one at a time in ascending id until the target is met
#pragma unroll
    for (int e = 0; e < E; ++e) {
      kept[e] = key[e] > T;
      uint64_t tie = __ballot(key[e] == T);
      while (tie != 0ull) {
        const int l = __builtin_ctzll(tie);
        tie &= tie - 1;
        if (cum < target || (cum == 0.0 && target == 0.0)) {
          if (lane == l) kept[e] = true;
          cum += __shfl(p[e], l);
        }
      }
    }
  }

  if (a.window) {
    // static window of this row's Q block, united with the scored set
    const int i = row % nK;
    const int it = i / (g.nH * g.nW), rem = i - it * g.nH * g.nW;
    const int ih = rem / g.nW, iw = rem - ih * g.nW;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int j = 64 * e + lane;
      if (j < nK) {
        const int jt = j / (g.nH * g.nW), jr = j - jt * g.nH * g.nW;
        const int jh = jr / g.nW, jw = jr - jh * g.nW;
        if (abs(jt - it) <= a.wt && abs(jh - ih) <= a.wh && abs(jw - iw) <= a.ww) kept[e] = true;
      }
    }
  }

  int cnt = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint64_t bits = __ballot(kept[e]);
    cnt += __popcll(bits);
    if (lane == 0) {
      uint32_t* mrow = mask + (size_t)row * mask_words;
      if (2 * e < mask_words) mrow[2 * e] = (uint32_t)bits;
      if (2 * e + 1 < mask_words) mrow[2 * e + 1] = (uint32_t)(bits >> 32);
    }
  }
  if (lane == 0) counts[row] = cnt;
}

// ---------------------------------------------------------------------------
// scheme generation: aggregate SICS per candidate and head, head-wise argmax
// ---------------------------------------------------------------------------
constexpr int kAggThreads = 256;

// A_c[bh] = sum_j n_j (q_sics[bh][j] + k_sics[bh][j]) / (2 N), fp64
__global__ __launch_bounds__(kAggThreads) void scheme_aggregate_kernel(Geom g, const float* __restrict__ qs,
                                                                      const float* __restrict__ ks, int c,
                                                                      double* __restrict__ agg64,
                                                                      float* __restrict__ agg) {
  __shared__ double part[kAggThreads / 64];
  const int bh = blockIdx.x;
  const int tid = threadIdx.x;
  double s = 0.0;
  for (int j = tid; j < g.nblk; j += kAggThreads) {
    const size_t at = (size_t)bh * g.nblk + j;
    s += (double)block_box(g, j).n * ((double)qs[at] + (double)ks[at]);
  }
  s = wave_sum(s);
  if ((tid & 63) == 0) part[tid >> 6] = s;
  __syncthreads();
  if (tid == 0) {
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < kAggThreads / 64; ++w) t += part[w];
    const double a = t / (2.0 * (double)g.N);
    agg64[(size_t)c * g.BH + bh] = a;
    if (agg) agg[(size_t)c * g.BH + bh] = (float)a;
  }
}

// scheme[bh] = argmax_c A_c[bh], ties to the lower c
__global__ __launch_bounds__(256) void scheme_choose_kernel(int BH, int C, const double* __restrict__ agg64,
                                                            int* __restrict__ scheme) {
  const int bh = blockIdx.x * 256 + threadIdx.x;
  if (bh >= BH) return;
  int best = 0;
  double bv = agg64[bh];
  for (int c = 1; c < C; ++c) {
    const double v = agg64[(size_t)c * BH + bh];
    if (v > bv) {
      bv = v;
      best = c;
    }
  }
  scheme[bh] = best;
}

// ---------------------------------------------------------------------------
// CSR
// ---------------------------------------------------------------------------
constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(kScanThreads) void scan_kernel(int R, const int* __restrict__ counts,
                                                            int* __restrict__ row_ptr) {
  __shared__ int part[kScanThreads];
  const int tid = threadIdx.x;
  const int per = (R + kScanThreads - 1) / kScanThreads;
  const int lo = min(R, tid * per), hi = min(R, lo + per);
  int s = 0;
  for (int r = lo; r < hi; ++r) s += counts[r];
  part[tid] = s;
  __syncthreads();
  // Hillis-Steele inclusive scan over the per-thread sums
  for (int off = 1; off < kScanThreads; off <<= 1) {
    const int add = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += add;
    __syncthreads();
  }
  int run = part[tid] - s;
  if (tid == 0) row_ptr[0] = 0;
  for (int r = lo; r < hi; ++r) {
    run += counts[r];
    row_ptr[r + 1] = run;
  }
}

__global__ __launch_bounds__(256) void compact_kernel(Geom g, const int* __restrict__ row_ptr,
                                                      const uint32_t* __restrict__ mask, int mask_words,
                                                      int* __restrict__ col_idx) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= g.R) return;
  const uint32_t* mrow = mask + (size_t)row * mask_words;
  int out = row_ptr[row];
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int base = 0; base < g.nblk; base += 64) {
    const int j = base + lane;
    bool bit = false;
    if (j < g.nblk) bit = (mrow[j >> 5] >> (j & 31)) & 1u;
    const uint64_t b = __ballot(bit);
    if (bit) col_idx[out + __popcll(b & lt_mask)] = j;
    out += __popcll(b);
  }
}

}  // namespace

hipError_t launch_scheme_aggregate(const Geom& g, const float* q_sics, const float* k_sics, int c,
                                   double* agg64, float* agg, hipStream_t s) {
  if (g.BH == 0) return hipSuccess;
  scheme_aggregate_kernel<<<g.BH, kAggThreads, 0, s>>>(g, q_sics, k_sics, c, agg64, agg);
  return hipGetLastError();
}

hipError_t launch_scheme_choose(int BH, int C, const double* agg64, int* scheme, hipStream_t s) {
  if (BH == 0) return hipSuccess;
  scheme_choose_kernel<<<(BH + 255) / 256, 256, 0, s>>>(BH, C, agg64, scheme);
  return hipGetLastError();
}

hipError_t launch_scores(const Geom& g, const float* q_mean, const float* k_mean, double scale,
                         double* scores, hipStream_t s) {
  if (g.BH == 0) return hipSuccess;
  dim3 grid((g.nblk + kSRows - 1) / kSRows, (g.nblk + kSCols - 1) / kSCols, g.BH);
  if (g.d == 128)
    scores_kernel<128><<<grid, 256, 0, s>>>(g, q_mean, k_mean, scale, scores);
  else
    scores_kernel<64><<<grid, 256, 0, s>>>(g, q_mean, k_mean, scale, scores);
  return hipGetLastError();
}

hipError_t launch_select(const Geom& g, const double* scores, const SelectArgs& a, int* counts,
                         uint32_t* mask, int mask_words, hipStream_t s) {
  if (g.R == 0) return hipSuccess;
  const int grid = (g.R + 3) / 4;
  if (g.nblk <= 64 * 4)
    select_kernel<4><<<grid, 256, 0, s>>>(g, scores, a, counts, mask, mask_words);
  else if (g.nblk <= 64 * 16)
    select_kernel<16><<<grid, 256, 0, s>>>(g, scores, a, counts, mask, mask_words);
  else if (g.nblk <= 64 * 32)
    select_kernel<32><<<grid, 256, 0, s>>>(g, scores, a, counts, mask, mask_words);
  else
    select_kernel<64><<<grid, 256, 0, s>>>(g, scores, a, counts, mask, mask_words);
  return hipGetLastError();
}

hipError_t launch_scan(const Geom& g, const int* counts, int* row_ptr, hipStream_t s) {
  scan_kernel<<<1, kScanThreads, 0, s>>>(g.R, counts, row_ptr);
  return hipGetLastError();
}

hipError_t launch_compact(const Geom& g, const int* row_ptr, const uint32_t* mask, int mask_words,
                          int* col_idx, hipStream_t s) {
  if (g.R == 0) return hipSuccess;
  compact_kernel<<<(g.R + 3) / 4, 256, 0, s>>>(g, row_ptr, mask, mask_words, col_idx);
  return hipGetLastError();
}

}  // namespace spade
