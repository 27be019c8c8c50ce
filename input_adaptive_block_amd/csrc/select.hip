// Estimator and index search.
//
// SPADE technical summary (gist.science), "Methodology 1. vDiT-SSR",
// Summarizer & Estimator Expressions: an inter-block importance score decides
// which blocks each Q block retains; the abstract's executor does this with a
// low-overhead index search, and "3. Head-wise Sparse Attention Execution"
// feeds the result to the attention kernel as a block-sparse row format.
//
// Stages (all on the caller's stream, no host synchronization):
//   estimate_select_kernel
//                   one workgroup per tile of 16 rows of a head: their fp64
//                   scores S = scale * qbar kbar^T on v_mfma_f64_16x16x4_f64
//                   (summaries are fp32, their products exact in fp64) go into
//                   LDS, never to HBM; then one wavefront per row holds the row
//                   in registers as 64-bit order keys and a bitwise threshold
//                   search (ballots or masked fp64 sums, per bit from the top)
//                   finds the k-th key (count / ratio) or the mass cut (mass),
//                   ties to the lower block id.  Emits the kept set as a
//                   bitmask and a count.  Rows wider than the LDS tile take
//                   scores_kernel (S in HBM) + select_kernel, same arithmetic.
//   csr_build_kernel
//                   (up to 32768 rows) row_ptr = exclusive prefix sum of the
//                   counts and the kept ids ascending, in one kernel.
//   chunk_sum / chunk_offsets / scan_apply, compact_kernel
//                   the same for more rows: the prefix sum over chunks, then
//                   one wavefront per row writes the kept ids ascending.
#include "spade_internal.h"

namespace spade {
namespace {

typedef double f64x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// scores
// ---------------------------------------------------------------------------

// 16 x 16 tiles of S / scale: rows row0 .. row0 + 15 and columns
// 16 ct .. 16 ct + 15 of one head, on v_mfma_f64_16x16x4_f64.  At k-step s
// lane (li, lk) feeds channel lk D/4 + s of row li (A) and of column li (B):
// a permutation of the channels that lets each lane read its D/4 channels of
// a summary as contiguous 16-byte loads.  The fp32 summaries' products are
// exact in fp64; rows or columns past nK repeat the last one (never stored).
// A wave keeps its rows' operands in registers for all of its tiles.
// f(ct, acc) receives each tile's result: D[lk + 4 v][li] in lane (lk, li),
// register v.
template <int D, class F>
__device__ inline void score_tiles(const float* __restrict__ qh, const float* __restrict__ kh, int nK, int row0,
                                   int ct0, int step, int lane, F f) {
  constexpr int NS = D / 4;  // k-steps
  constexpr int NV = NS / 4; // float4 loads per operand
  const int li = lane & 15, lk = lane >> 4;
  const int ntiles = (nK + 15) / 16;
  if (ct0 >= ntiles) return;
  float4 qa[NV], kb[NV];
  const float4* qrow = reinterpret_cast<const float4*>(qh + (size_t)min(row0 + li, nK - 1) * D + lk * NS);
#pragma unroll
  for (int v = 0; v < NV; ++v) qa[v] = qrow[v];
  // the next tile's operands are loaded while this tile's MFMAs run (the row
  // index is clamped, so the load past the last tile reads a valid row)
  auto load_k = [&](float4 (&dst)[NV], int ct) __attribute__((always_inline)) {
    const float4* krow = reinterpret_cast<const float4*>(kh + (size_t)min(16 * ct + li, nK - 1) * D + lk * NS);
#pragma unroll
    for (int v = 0; v < NV; ++v) dst[v] = krow[v];
  };
  load_k(kb, ct0);
  for (int ct = ct0; ct < ntiles; ct += step) {
    float4 kn[NV];
    load_k(kn, ct + step);
    f64x4 acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)qa[v].x, (double)kb[v].x, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)qa[v].y, (double)kb[v].y, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)qa[v].z, (double)kb[v].z, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)qa[v].w, (double)kb[v].w, acc, 0, 0, 0);
    }
    f(ct, acc);
#pragma unroll
    for (int v = 0; v < NV; ++v) kb[v] = kn[v];
  }
}

constexpr int kFRows = 16;   // selection rows per workgroup (one row tile)
constexpr int kFWaves = 8;   // waves per workgroup

// S = scale * qbar kbar^T written to HBM, one row tile per workgroup (rows
// wider than the fused kernel's LDS tile, and the scores test hook).  The
// same arithmetic as the fused kernel, bit for bit.
template <int D>
__global__ __launch_bounds__(64 * kFWaves) void scores_kernel(Geom g, const float* __restrict__ qm,
                                                              const float* __restrict__ km, double scale,
                                                              double* __restrict__ S) {
  const int bh = blockIdx.y;
  if (!head_active(g, bh)) return;  // another scheme's head (whole workgroup)
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nK = g.nblk;
  const int row0 = blockIdx.x * kFRows;
  const float* qh = qm + (size_t)bh * nK * D;
  const float* kh = km + (size_t)bh * nK * D;
  double* Sh = S + (size_t)bh * nK * nK;
  const int li = lane & 15, lk = lane >> 4;
  score_tiles<D>(qh, kh, nK, row0, wave, kFWaves, lane, [&](int ct, const f64x4& acc) {
    const int j = 16 * ct + li;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = row0 + lk + 4 * v;
      if (i < nK && j < nK) Sh[(size_t)i * nK + j] = scale * acc[v];
    }
  });
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

// One lane-exchange step of a butterfly over the wavefront for a double:
// DPP within a 16-lane row (CTRL: quad_perm [1,0,3,2] = xor 1, quad_perm
// [2,3,0,1] = xor 2, row_half_mirror, row_mirror), then v_permlane16_swap and
// v_permlane32_swap across rows.  After xor 1 and xor 2 every lane of a quad
// holds the same bits, so the mirrors meet the same partner values as xor 4
// and xor 8 would, and the swaps those of xor 16 and xor 32: the steps add
// the same operand pairs as a shuffle-xor butterfly, every lane ending with
// the same bits, at VALU latency instead of LDS-permute latency.
// (Every lane has a source in these patterns, so the moves need no old value.)
template <int CTRL>
__device__ inline uint64_t dpp_u64(uint64_t b) {
  const int lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)b, CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(b >> 32), CTRL, 0xF, 0xF, false);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

template <int CTRL>
__device__ inline double dpp_f64(double x) {
  return __builtin_bit_cast(double, dpp_u64<CTRL>(__builtin_bit_cast(uint64_t, x)));
}

// The two values a permlane swap leaves a lane: its own and its partner's
// (xor 16 for SWAP16, xor 32 otherwise), in either order.
template <bool SWAP16>
__device__ inline void swap_f64(double x, double& a, double& b) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = (uint32_t)u, hi = (uint32_t)(u >> 32);
  const auto sl = SWAP16 ? __builtin_amdgcn_permlane16_swap(lo, lo, false, false)
                         : __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
  const auto sh = SWAP16 ? __builtin_amdgcn_permlane16_swap(hi, hi, false, false)
                         : __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
  a = __builtin_bit_cast(double, ((uint64_t)sh[0] << 32) | sl[0]);
  b = __builtin_bit_cast(double, ((uint64_t)sh[1] << 32) | sl[1]);
}

__device__ inline double wave_sum(double x) {
  x += dpp_f64<0xB1>(x);   // quad_perm [1, 0, 3, 2]
  x += dpp_f64<0x4E>(x);   // quad_perm [2, 3, 0, 1]
  x += dpp_f64<0x141>(x);  // row_half_mirror
  x += dpp_f64<0x140>(x);  // row_mirror
  double a, b;
  swap_f64<true>(x, a, b);
  x = a + b;
  swap_f64<false>(x, a, b);
  return a + b;
}

__device__ inline double wave_max(double x) {
  x = fmax(x, dpp_f64<0xB1>(x));
  x = fmax(x, dpp_f64<0x4E>(x));
  x = fmax(x, dpp_f64<0x141>(x));
  x = fmax(x, dpp_f64<0x140>(x));
  double a, b;
  swap_f64<true>(x, a, b);
  x = fmax(a, b);
  swap_f64<false>(x, a, b);
  return fmax(a, b);
}

// The same butterfly for the bitwise OR and AND of 64-bit words.
__device__ inline void wave_or_and(uint64_t& o, uint64_t& a) {
  o |= dpp_u64<0xB1>(o);
  a &= dpp_u64<0xB1>(a);
  o |= dpp_u64<0x4E>(o);
  a &= dpp_u64<0x4E>(a);
  o |= dpp_u64<0x141>(o);
  a &= dpp_u64<0x141>(a);
  o |= dpp_u64<0x140>(o);
  a &= dpp_u64<0x140>(a);
  double x0, x1, y0, y1;
  swap_f64<true>(__builtin_bit_cast(double, o), x0, x1);
  swap_f64<true>(__builtin_bit_cast(double, a), y0, y1);
  o = __builtin_bit_cast(uint64_t, x0) | __builtin_bit_cast(uint64_t, x1);
  a = __builtin_bit_cast(uint64_t, y0) & __builtin_bit_cast(uint64_t, y1);
  swap_f64<false>(__builtin_bit_cast(double, o), x0, x1);
  swap_f64<false>(__builtin_bit_cast(double, a), y0, y1);
  o = __builtin_bit_cast(uint64_t, x0) | __builtin_bit_cast(uint64_t, x1);
  a = __builtin_bit_cast(uint64_t, y0) & __builtin_bit_cast(uint64_t, y1);
}

// lane l's double (l uniform)
__device__ inline double read_lane_f64(double x, int l) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
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
      const uint32_t lo32 = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)key[e], l);
      const uint32_t hi32 = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(key[e] >> 32), l);
      T = ((uint64_t)hi32 << 32) | lo32;
    }
  }
  return true;
}

// In the mass search below, the candidates at bit b are the real keys that
// share the bits above b fixed in T.  Wherever they all agree, the
// threshold's bit follows without a mass test: a common 1 keeps every
// candidate at or above the tested value (the same set of keys as T itself,
// whose mass reaches the target), a common 0 puts every candidate below it
// (the same set as the last test that failed).  So T takes the candidates'
// common bits b .. d+1, d the highest bit where they differ, and the search
// resumes at d; -1 when they agree on every bit (T is then their key).
template <int E>
__device__ inline int skip_common_bits(const uint64_t (&key)[E], int nK, int lane, uint64_t& T, int b) {
  const uint64_t low = b >= 63 ? ~0ull : ((2ull << b) - 1ull);  // bits b .. 0
  uint64_t o = 0ull, a = ~0ull;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool cand = 64 * e + lane < nK && ((key[e] ^ T) & ~low) == 0ull;
    o |= cand ? key[e] : 0ull;
    a &= cand ? key[e] : ~0ull;
  }
  wave_or_and(o, a);
  // every lane holds the same words: read them into scalar registers, so the
  // bit the search resumes at is wave-uniform and the search loop stays a
  // scalar loop
  o = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(o >> 32)) << 32) |
      (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)o);
  a = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32)) << 32) |
      (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint64_t diff = (o ^ a) & low;
  if (diff == 0ull) {
    T = (T & ~low) | (o & low);
    return -1;
  }
  const int d = 63 - __builtin_clzll(diff);
  const uint64_t common = low & ~((2ull << d) - 1ull);  // bits b .. d+1
  T = (T & ~common) | (o & common);
  return d;
}

// The score an order key encodes (order_key is a bijection on doubles).
__device__ inline double key_score(uint64_t k) {
  const uint64_t u = (k >> 63) ? (k & 0x7FFFFFFFFFFFFFFFull) : ~k;
  return __longlong_as_double((long long)u);
}

// Selection of one row whose scores S are held by the wave as E order keys
// per lane (block 64 e + lane in key[e], 0 past nK): the kept set as a
// bitmask row and its count.
template <int E>
__device__ inline void select_row(const Geom& g, const SelectArgs& a, int row, int lane, uint64_t (&key)[E],
                                  int* __restrict__ counts, uint32_t* __restrict__ mask, int mask_words) {
  const int nK = g.nblk;
  const int h = (row / nK) % g.H;
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
    uint64_t kmax = key[0];
#pragma unroll
    for (int e = 1; e < E; ++e) kmax = key[e] > kmax ? key[e] : kmax;
    const double mx = wave_max(key_score(kmax));  // lane 0 always holds a real key
    double p[E];
    double loc = 0.0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      p[e] = (64 * e + lane < nK) ? exp_nonpos(key_score(key[e]) - mx) : 0.0;
      loc += p[e];
    }
    // (every lane holds the same sum: read into scalar registers, so the
    // target and the search's control flow below are wave-uniform)
    const double Z = read_lane_f64(wave_sum(loc), 0);
    const double target = a.tau[h] * Z;
    // largest T with mass(key >= T) >= target; mass(key >= T) is monotone
    // non-increasing in T because every partial sum only drops non-negative
    // terms when T grows
    uint64_t T = 0ull;
    // common bits are skipped before the first test (all real keys are
    // candidates) and after it (the candidates then share the sign bit, and
    // mostly the exponent's high bits too); with a target of 0 every test
    // passes and no key is kept by score
    const bool skip = target > 0.0;
    int bit = skip ? skip_common_bits(key, nK, lane, T, 63) : 63;
    bool tested = false;
    for (; bit >= 0; --bit) {
      const uint64_t cand = T | (1ull << bit);
      double f0 = 0.0, f1 = 0.0;  // two chains of adds instead of one
#pragma unroll
      for (int e = 0; e < E; e += 2) {
        f0 += (key[e] >= cand) ? p[e] : 0.0;
        if (e + 1 < E) f1 += (key[e + 1] >= cand) ? p[e + 1] : 0.0;
      }
      // every lane holds the same sum: the ballot makes the test wave-uniform
      if (__builtin_amdgcn_ballot_w64(wave_sum(f0 + f1) >= target) != 0ull) T = cand;
      if (skip && !tested && bit > 0) {
        tested = true;
        bit = skip_common_bits(key, nK, lane, T, bit - 1) + 1;  // the loop steps to the returned bit
        continue;
      }
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
          cum += read_lane_f64(p[e], l);
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
  uint32_t* mrow = mask + (size_t)row * mask_words;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint64_t bits = __ballot(kept[e]);
    cnt += __popcll(bits);
    if (lane == 0) {
      if (2 * e < mask_words) mrow[2 * e] = (uint32_t)bits;
      if (2 * e + 1 < mask_words) mrow[2 * e + 1] = (uint32_t)(bits >> 32);
    }
  }
  if (lane == 0) counts[row] = cnt;
}

// An empty row (another scheme's head: its scores were never computed).
__device__ inline void empty_row(int row, int lane, int* __restrict__ counts, uint32_t* __restrict__ mask,
                                 int mask_words) {
  uint32_t* mrow = mask + (size_t)row * mask_words;
  for (int w = lane; w < mask_words; w += 64) mrow[w] = 0u;
  if (lane == 0) counts[row] = 0;
}

// One wavefront per row, the row's fp64 scores read from HBM (rows wider than
// the fused kernel's LDS tile).
template <int E>
__global__ __launch_bounds__(256) void select_kernel(Geom g, const double* __restrict__ S, SelectArgs a,
                                                     int* __restrict__ counts, uint32_t* __restrict__ mask,
                                                     int mask_words) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= g.R) return;  // whole wave exits together
  const int nK = g.nblk;
  if (!head_active(g, row / nK)) {
    empty_row(row, lane, counts, mask, mask_words);
    return;
  }
  const double* Sr = S + (size_t)row * nK;
  uint64_t key[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = 64 * e + lane;
    key[e] = j < nK ? order_key(Sr[j]) : 0ull;  // below every real score
  }
  select_row<E>(g, a, row, lane, key, counts, mask, mask_words);
}

// ---------------------------------------------------------------------------
// fused estimate + select: one row tile's fp64 scores in LDS
// ---------------------------------------------------------------------------

// The workgroup's 16 rows of S (score_tile over every column tile, wave w
// taking tiles w, w + 8, ...) go into LDS, then each wave selects its rows
// straight from there: S is never written to HBM.
template <int D, int E>
__global__ __launch_bounds__(64 * kFWaves) __attribute__((amdgpu_waves_per_eu(4, 4))) void estimate_select_kernel(Geom g, const float* __restrict__ qm,
                                                                        const float* __restrict__ km, double scale,
                                                                        SelectArgs a, int* __restrict__ counts,
                                                                        uint32_t* __restrict__ mask,
                                                                        int mask_words) {
  constexpr int NB = 64 * E;  // widest row the tile holds
  __shared__ double St[kFRows * NB];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nK = g.nblk;
  const int bh = blockIdx.y;
  const int row0 = blockIdx.x * kFRows;  // first Q block of the tile
  if (!head_active(g, bh)) {
    for (int r = wave; r < kFRows && row0 + r < nK; r += kFWaves)
      empty_row(bh * nK + row0 + r, lane, counts, mask, mask_words);
    return;
  }
  const float* qh = qm + (size_t)bh * nK * D;
  const float* kh = km + (size_t)bh * nK * D;
  const int li = lane & 15, lk = lane >> 4;
  score_tiles<D>(qh, kh, nK, row0, wave, kFWaves, lane, [&](int ct, const f64x4& acc) {
    const int j = 16 * ct + li;
    if (j < nK) {
#pragma unroll
      for (int v = 0; v < 4; ++v) St[(lk + 4 * v) * NB + j] = scale * acc[v];
    }
  });
  __syncthreads();
  for (int r = wave; r < kFRows && row0 + r < nK; r += kFWaves) {
    uint64_t key[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int j = 64 * e + lane;
      key[e] = j < nK ? order_key(St[r * NB + j]) : 0ull;  // below every real score
    }
    select_row<E>(g, a, bh * nK + row0 + r, lane, key, counts, mask, mask_words);
  }
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
// row_ptr in three passes over chunks of kScanChunk rows: each chunk's sum,
// an exclusive scan of the chunk sums (one workgroup), then each chunk's
// exclusive scan plus its offset.
constexpr int kScanThreads = 256;
constexpr int kScanPer = kScanChunk / kScanThreads;  // rows per thread

__device__ inline int block_exclusive_scan(int x, int* part) {
  // exclusive prefix of x over the workgroup (kScanThreads threads)
  const int tid = threadIdx.x;
  part[tid] = x;
  __syncthreads();
  for (int off = 1; off < kScanThreads; off <<= 1) {
    const int add = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += add;
    __syncthreads();
  }
  return part[tid] - x;
}

__global__ __launch_bounds__(kScanThreads) void chunk_sum_kernel(int R, const int* __restrict__ counts,
                                                                 int* __restrict__ sums) {
  __shared__ int part[kScanThreads];
  const int base = blockIdx.x * kScanChunk + threadIdx.x * kScanPer;
  int s = 0;
  for (int i = 0; i < kScanPer; ++i)
    if (base + i < R) s += counts[base + i];
  const int ex = block_exclusive_scan(s, part);
  if (threadIdx.x == kScanThreads - 1) sums[blockIdx.x] = ex + s;
}

__global__ __launch_bounds__(1024) void chunk_offsets_kernel(int nc, int* __restrict__ sums) {
  // exclusive scan of the nc chunk sums in place
  __shared__ int part[1024];
  const int tid = threadIdx.x;
  const int per = (nc + 1023) / 1024;
  const int lo = min(nc, tid * per), hi = min(nc, lo + per);
  int s = 0;
  for (int c = lo; c < hi; ++c) s += sums[c];
  part[tid] = s;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int add = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += add;
    __syncthreads();
  }
  int run = part[tid] - s;
  for (int c = lo; c < hi; ++c) {
    const int v = sums[c];
    sums[c] = run;
    run += v;
  }
}

__global__ __launch_bounds__(kScanThreads) void scan_apply_kernel(int R, const int* __restrict__ counts,
                                                                  const int* __restrict__ offsets,
                                                                  int* __restrict__ row_ptr) {
  __shared__ int part[kScanThreads];
  const int base = blockIdx.x * kScanChunk + threadIdx.x * kScanPer;
  int c[kScanPer];
  int s = 0;
#pragma unroll
  for (int i = 0; i < kScanPer; ++i) {
    c[i] = base + i < R ? counts[base + i] : 0;
    s += c[i];
  }
  int run = offsets[blockIdx.x] + block_exclusive_scan(s, part);
  if (blockIdx.x == 0 && threadIdx.x == 0) row_ptr[0] = 0;
#pragma unroll
  for (int i = 0; i < kScanPer; ++i) {
    run += c[i];
    if (base + i < R) row_ptr[base + i + 1] = run;
  }
}

__global__ void zero_row_ptr_kernel(int* __restrict__ row_ptr) { row_ptr[0] = 0; }

// Kept ids id0 + 32 w + b for the set bits b of bitmask words w < nwords,
// held one per lane (word w in lane w, nwords <= 64), written ascending from
// col_idx[out]; returns the position after the last.  For each 64 ids the two
// words, made uniform with readlane, are the chunk's ballot.
__device__ inline int compact_row_from_lanes(uint32_t word, int nwords, int lane, int out, int id0,
                                             int* __restrict__ col_idx) {
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int w = 0; w < nwords; w += 2) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)word, w);
    const uint32_t hi = w + 1 < nwords ? (uint32_t)__builtin_amdgcn_readlane((int)word, w + 1) : 0u;
    const uint64_t m = ((uint64_t)hi << 32) | lo;
    if ((m >> lane) & 1ull) col_idx[out + __popcll(m & lt_mask)] = id0 + 32 * w + lane;
    out += __popcll(m);
  }
  return out;
}

// row_ptr and col_idx in one kernel when R <= kCsrMaxRows: a workgroup of
// sixteen waves takes kCsrRows rows.  The counts of every row before them are
// summed by the workgroup (at most kCsrMaxRows values, 16-byte loads), its
// own rows' counts scanned by one wave; then each wave writes the kept ids
// of four rows, their bitmask words loaded up front and the four rows walked
// together (rows of at most 2048 blocks), or one row and one 64-word chunk
// at a time.  Also clears the attention kernel's unit counter when it is
// given one (the next kernel on the stream).
constexpr int kCsrRows = 64;
constexpr int kCsrThreads = 1024;
constexpr int kCsrMaxRows = 32768;

__global__ __launch_bounds__(kCsrThreads) void csr_build_kernel(Geom g, const int* __restrict__ counts,
                                                                const uint32_t* __restrict__ mask, int mask_words,
                                                                int* __restrict__ row_ptr, int* __restrict__ col_idx,
                                                                int* __restrict__ counter) {
  constexpr int NW = kCsrThreads / 64;   // waves
  constexpr int RPW = kCsrRows / NW;     // rows per wave
  __shared__ int red[NW];
  __shared__ int start[kCsrRows];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row0 = blockIdx.x * kCsrRows;
  const int r0 = row0 + RPW * wave;
  // this wave's rows' bitmask words (rows of at most 2048 blocks), loaded
  // first, every load in bounds (row and word clamped), and all retired with
  // the loads of the counts, before any store: a wait issued after a store
  // would also wait for the store
  uint32_t words[RPW];
  if (mask_words <= 64) {
    const int lw = min(lane, mask_words - 1);
#pragma unroll
    for (int k = 0; k < RPW; ++k) words[k] = mask[(size_t)min(r0 + k, g.R - 1) * mask_words + lw];
  }
  // rows [0, row0): row0 is a multiple of 4, counts is 16-byte aligned
  // (two 16-byte loads in flight per thread: at most kCsrMaxRows / 8192
  // rounds of them)
  const int4* c4 = reinterpret_cast<const int4*>(counts);
  const int n4 = row0 / 4;
  int sum = 0;
  for (int i0 = 0; i0 < n4; i0 += 2 * kCsrThreads) {
    int4 v[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = i0 + kCsrThreads * u + tid;
      v[u] = i < n4 ? c4[i] : make_int4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) sum += v[u].x + v[u].y + v[u].z + v[u].w;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
  if (lane == 0) red[wave] = sum;
  const int c = (tid < kCsrRows && row0 + tid < g.R) ? counts[row0 + tid] : 0;
  __builtin_amdgcn_s_waitcnt(0);
  if (mask_words <= 64) {
#pragma unroll
    for (int k = 0; k < RPW; ++k) words[k] = (lane < mask_words && r0 + k < g.R) ? words[k] : 0u;
  }
  __syncthreads();
  int end = 0;  // wave 0: row_ptr[row0 + lane + 1]
  if (wave == 0) {
    int base = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) base += red[w];
    int inc = c;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(inc, off);
      if (lane >= off) inc += t;
    }
    end = base + inc;
    start[lane] = end - c;
  }
  __syncthreads();
  // stored after the barrier, which would otherwise wait for these stores
  if (counter != nullptr && blockIdx.x == 0 && tid == 0) *counter = 0;
  if (wave == 0) {
    if (row0 + lane < g.R) row_ptr[row0 + lane + 1] = end;
    if (blockIdx.x == 0 && lane == 0) row_ptr[0] = 0;
  }
  if (mask_words <= 64) {
    // for each 64 ids, the two words (made uniform with readlane) are the
    // chunk's ballot; the rows' chains are independent
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int out[RPW];
#pragma unroll
    for (int k = 0; k < RPW; ++k) out[k] = start[RPW * wave + k];
    for (int w = 0; w < mask_words; w += 2) {
#pragma unroll
      for (int k = 0; k < RPW; ++k) {
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)words[k], w);
        const uint32_t hi = w + 1 < mask_words ? (uint32_t)__builtin_amdgcn_readlane((int)words[k], w + 1) : 0u;
        const uint64_t m = ((uint64_t)hi << 32) | lo;
        if ((m >> lane) & 1ull) col_idx[out[k] + __popcll(m & lt_mask)] = 32 * w + lane;
        out[k] += __popcll(m);
      }
    }
  } else {
    for (int k = 0; k < RPW && r0 + k < g.R; ++k) {
      const uint32_t* mrow = mask + (size_t)(r0 + k) * mask_words;
      int out = start[RPW * wave + k];
      for (int w0 = 0; w0 < mask_words; w0 += 64) {
        const int nw = min(64, mask_words - w0);
        const uint32_t word = lane < nw ? mrow[w0 + lane] : 0u;
        out = compact_row_from_lanes(word, nw, lane, out, 32 * w0, col_idx);
      }
    }
  }
}

__global__ __launch_bounds__(256) void compact_kernel(Geom g, const int* __restrict__ row_ptr,
                                                      const uint32_t* __restrict__ mask, int mask_words,
                                                      int* __restrict__ col_idx, int* __restrict__ counter) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (counter != nullptr && blockIdx.x == 0 && threadIdx.x == 0) *counter = 0;
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
  dim3 grid((g.nblk + kFRows - 1) / kFRows, g.BH);
  if (g.d == 128)
    scores_kernel<128><<<grid, 64 * kFWaves, 0, s>>>(g, q_mean, k_mean, scale, scores);
  else
    scores_kernel<64><<<grid, 64 * kFWaves, 0, s>>>(g, q_mean, k_mean, scale, scores);
  return hipGetLastError();
}

hipError_t launch_select(const Geom& g, const double* scores, const SelectArgs& a, int* counts,
                         uint32_t* mask, int mask_words, hipStream_t s) {
  if (g.R == 0) return hipSuccess;
  const int grid = (g.R + 3) / 4;
  const int e = (g.nblk + 63) / 64;  // scores per lane
#define SPADE_SELECT(EE) select_kernel<EE><<<grid, 256, 0, s>>>(g, scores, a, counts, mask, mask_words)
  if (e <= 4) SPADE_SELECT(4);
  else if (e <= 16) SPADE_SELECT(16);
  else if (e <= 24) SPADE_SELECT(24);
  else if (e <= 32) SPADE_SELECT(32);
  else if (e <= 48) SPADE_SELECT(48);
  else SPADE_SELECT(64);
#undef SPADE_SELECT
  return hipGetLastError();
}

bool fused_select_fits(const Geom& g) { return g.nblk <= kFusedMaxBlocks; }

hipError_t launch_estimate_select(const Geom& g, const float* q_mean, const float* k_mean, double scale,
                                  const SelectArgs& a, int* counts, uint32_t* mask, int mask_words,
                                  hipStream_t s) {
  if (g.R == 0) return hipSuccess;
  dim3 grid((g.nblk + kFRows - 1) / kFRows, g.BH);
  const int e = (g.nblk + 63) / 64;  // scores per lane: the tile's width in units of 64
#define SPADE_FUSED(EE)                                                                                         \
  do {                                                                                                          \
    if (g.d == 128)                                                                                             \
      estimate_select_kernel<128, EE><<<grid, 64 * kFWaves, 0, s>>>(g, q_mean, k_mean, scale, a, counts, mask,  \
                                                                    mask_words);                               \
    else                                                                                                        \
      estimate_select_kernel<64, EE><<<grid, 64 * kFWaves, 0, s>>>(g, q_mean, k_mean, scale, a, counts, mask,   \
                                                                   mask_words);                                \
  } while (0)
  if (e <= 2) SPADE_FUSED(2);
  else if (e <= 4) SPADE_FUSED(4);
  else if (e <= 6) SPADE_FUSED(6);
  else if (e <= 8) SPADE_FUSED(8);
  else if (e <= 10) SPADE_FUSED(10);
  else if (e <= 12) SPADE_FUSED(12);
  else SPADE_FUSED(16);
#undef SPADE_FUSED
  return hipGetLastError();
}

hipError_t launch_scan(const Geom& g, const int* counts, int* row_ptr, int* chunk_sums, hipStream_t s) {
  if (g.R == 0) {
    zero_row_ptr_kernel<<<1, 1, 0, s>>>(row_ptr);
    return hipGetLastError();
  }
  const int nc = scan_chunks(g.R);
  chunk_sum_kernel<<<nc, kScanThreads, 0, s>>>(g.R, counts, chunk_sums);
  chunk_offsets_kernel<<<1, 1024, 0, s>>>(nc, chunk_sums);
  scan_apply_kernel<<<nc, kScanThreads, 0, s>>>(g.R, counts, chunk_sums, row_ptr);
  return hipGetLastError();
}

hipError_t launch_csr(const Geom& g, const int* counts, const uint32_t* mask, int mask_words, int* row_ptr,
                      int* col_idx, int* chunk_sums, int* attn_counter, hipStream_t s) {
  if (g.R == 0) return launch_scan(g, nullptr, row_ptr, nullptr, s);
  if (g.R <= kCsrMaxRows) {
    csr_build_kernel<<<(g.R + kCsrRows - 1) / kCsrRows, kCsrThreads, 0, s>>>(g, counts, mask, mask_words,
                                                                              row_ptr, col_idx, attn_counter);
    return hipGetLastError();
  }
  const hipError_t e = launch_scan(g, counts, row_ptr, chunk_sums, s);
  if (e != hipSuccess) return e;
  compact_kernel<<<(g.R + 3) / 4, 256, 0, s>>>(g, row_ptr, mask, mask_words, col_idx, attn_counter);
  return hipGetLastError();
}

}  // namespace spade
