// Fused blocking + Summarizer kernel.
//
// SPADE technical summary (gist.science), "Methodology 3. Head-wise Sparse
// Attention Execution", Kernel Fusion: the layout transformation into blocks
// and the block summaries come out of one pass over Q/K/V.  Summarizer
// ("Methodology 1. vDiT-SSR", Summarizer & Estimator Expressions): the mean of
// a block's real tokens.
//
// Intra-block estimate (optional side output): SICS, the sum of intra-block
// cosine similarities ("Methodology 2. Scheme Generation", Aggregation
// Evaluation), normalised by n_b^2.  The online form (Online Optimization)
// follows from bilinearity: with u_i = x_i / |x_i| (0 for a zero token),
// sum_{i,j in b} cos(x_i, x_j) = |sum_i u_i|^2, so it rides on the same single
// read of the block as the mean: each token's 16 threads reduce its squared
// norm with shuffles, scale their 8 channels by 1/|x| and add them to a
// second fp64 accumulator.
//
// One workgroup of 256 threads per (block j, head bh, role) with role
// 0 = Q, 1 = K, 2 = V.  Each thread moves 16-byte vectors of one token: the
// load of token l is a contiguous 16 B of its d-row, so a wave reads whole
// 256 B rows (bf16, d = 128) of bw consecutive tokens.  Sums are taken in fp64
// (exact for bf16 inputs) and reduced with wavefront shuffles, then across the
// four waves through LDS; the mean is rounded once to fp32.
//
// With packing on (bf16 path), the kernel also writes the block as the
// attention kernel's MFMA operand tiles (padded to P rows with zeros):
//   Q, K: per 32-row subtile s, chunk c of 16 channels and lane L,
//         8 contiguous bf16 = X[row 32 s + L%32][16 c + 8 (L/32) + 0..7];
//   V:    per 32-key subtile s, channel tile m (32 channels), key chunk kc and
//         lane L, 8 contiguous bf16 e = 0..7 holding
//         V[key 32 s + 16 kc + 8 (e/4) + 4 (L/32) + e%4][32 m + L%32],
//         which is the A operand of O^T += V^T P^T for the key order in which
//         the S^T accumulator of v_mfma_f32_32x32x16_bf16 leaves P.
#include <type_traits>

#include "spade_internal.h"

namespace spade {
namespace {

constexpr int kThreads = 256;

struct alignas(16) Vec16 {
  uint32_t w[4];
};

// One DPP move of both halves of a double (CTRL is a DPP control code).
template <int CTRL>
__device__ inline double dpp_f64(double x) {
  const uint64_t b = __builtin_bit_cast(uint64_t, x);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, 0xF, 0xF, false);
  return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// Sum of x over aligned groups of G consecutive lanes (G = 8, 16 or 32),
// every lane of a group receiving the total.  Within a 16-lane row the
// partners come from DPP (swap neighbours, swap pairs, mirror each half-row,
// mirror the row), which pair disjoint partial sums at every step; across the
// two rows of a 32-lane group one cross-lane shuffle finishes.
template <int G>
__device__ inline double group_sum(double x) {
  constexpr int kSwap1 = 0xB1;       // quad_perm [1, 0, 3, 2]
  constexpr int kSwap2 = 0x4E;       // quad_perm [2, 3, 0, 1]
  constexpr int kHalfMirror = 0x141;  // row_half_mirror
  constexpr int kMirror = 0x140;      // row_mirror
  x += dpp_f64<kSwap1>(x);
  x += dpp_f64<kSwap2>(x);
  x += dpp_f64<kHalfMirror>(x);
  if (G >= 16) x += dpp_f64<kMirror>(x);
  if (G >= 32) x += __shfl_xor(x, 16);
  return x;
}

// The Summarizer's reduction: sum (mean), maximum or minimum.
__device__ inline double sum_op(int op, double a, double b) {
  return op == 0 ? a + b : (op == 1 ? fmax(a, b) : fmin(a, b));
}
template <int OP>
__device__ inline double sum_op_t(double a, double b) {
  return OP == 0 ? a + b : (OP == 1 ? fmax(a, b) : fmin(a, b));
}
__device__ inline double sum_identity(int op) {
  return op == 0 ? 0.0 : (op == 1 ? -__builtin_huge_val() : __builtin_huge_val());
}

__device__ inline float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ inline float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

// MEAN false: the caller wants no summaries (a SICS-only pass), so the token
// loop keeps no per-channel reduction at all.
template <bool BF16, int D, bool PACK, bool SICS, bool MEAN = true>
__global__ __launch_bounds__(kThreads) void summarize_kernel(
    Geom g, const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    float* __restrict__ q_mean, float* __restrict__ k_mean, uint16_t* __restrict__ qpack,
    uint16_t* __restrict__ kpack, uint16_t* __restrict__ vpack, float* __restrict__ q_sics,
    float* __restrict__ k_sics) {
  constexpr int EPV = BF16 ? 8 : 4;     // elements per 16-byte vector
  constexpr int TPT = D / EPV;          // threads per token row
  constexpr int TPP = kThreads / TPT;   // tokens per pass
  constexpr int VROW = D + 8;           // LDS row stride (bf16) of the V transpose
  static_assert(kThreads % TPT == 0, "layout");
  static_assert(TPT == 8 || TPT == 16 || TPT == 32, "token lane groups");

  const int j = blockIdx.x;
  const int bh = blockIdx.y;
  const int role = blockIdx.z;
  if (!head_active(g, bh)) return;  // another scheme's head (whole workgroup)
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const BlockBox box = block_box(g, j);

  const char* src = reinterpret_cast<const char*>(role == 0 ? q : (role == 1 ? k : v));
  const size_t elem = BF16 ? 2 : 4;
  const size_t head_base = (size_t)bh * g.N * D;

  const int cv = tid % TPT;      // which 16-byte vector of the row
  const int c0 = cv * EPV;       // first channel of that vector
  const int lrow = tid / TPT;    // token slot within a pass

  float* mean_out = role == 0 ? q_mean : (role == 1 ? k_mean : nullptr);
  const bool want_mean = MEAN && mean_out != nullptr;
  float* sics_out = SICS ? (role == 0 ? q_sics : (role == 1 ? k_sics : nullptr)) : nullptr;
  const bool want_sics = SICS && sics_out != nullptr;

  __shared__ double red[kThreads / 64][D];
  __shared__ double ured[SICS ? kThreads / 64 : 1][SICS ? D : 1];
  __shared__ uint16_t vt[PACK ? 128 * VROW : 1];

  const int op = g.op;  // the block summary: sum (mean), max or min over the real tokens
  double acc[EPV];
  double uacc[EPV];  // sum of the unit token vectors (SICS)
#pragma unroll
  for (int e = 0; e < EPV; ++e) {
    acc[e] = sum_identity(op);
    uacc[e] = 0.0;
  }

  if (role < 2 || !PACK) {
    // the token loop, compiled once per reduction so each keeps only its own
    // fp64 arithmetic
    auto token_loop = [&](auto op_c) __attribute__((always_inline)) {
      constexpr int OP = decltype(op_c)::value;
      uint16_t* pk = nullptr;
      if (PACK) pk = (role == 0 ? qpack : kpack) + ((size_t)bh * g.nblk + j) * (size_t)g.P * D;
      const int rows = PACK ? g.P : box.n;
      // the token rows of NB passes are loaded before any of them is used
      constexpr int NB = 4;
      for (int l0 = lrow; l0 < rows; l0 += NB * TPP) {
        Vec16 xs[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const int l = l0 + b * TPP;
          xs[b] = Vec16{{0u, 0u, 0u, 0u}};
          if (l < box.n) {
            const int tok = block_token(g, box, l);
            xs[b] = *reinterpret_cast<const Vec16*>(src + (head_base + (size_t)tok * D + c0) * elem);
          }
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const int l = l0 + b * TPP;
          if (l >= rows) break;
          const Vec16 x = xs[b];
          if (want_mean || want_sics) {
            double xe[EPV];
            if (BF16) {
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                xe[2 * e] = (double)bf16_lo(x.w[e]);
                xe[2 * e + 1] = (double)bf16_hi(x.w[e]);
              }
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e) xe[e] = (double)__uint_as_float(x.w[e]);
            }
            if (MEAN && l < box.n) {  // padded rows (zeros) take no part in a max or min
#pragma unroll
              for (int e = 0; e < EPV; ++e) acc[e] = sum_op_t<OP>(acc[e], xe[e]);
            }
            if (want_sics) {
              // squared norm of the token over its TPT threads (consecutive lanes;
              // every thread of the group runs the same iterations)
              double ss = 0.0;
#pragma unroll
              for (int e = 0; e < EPV; ++e) ss += xe[e] * xe[e];
              ss = group_sum<TPT>(ss);
              // 1/|x|: fp32 reciprocal square root refined by one Newton step in
              // fp64 (relative error ~1e-14, far below the fp32 result's ulp)
              double inv = 0.0;
              if (ss > 0.0) {
                const double r = (double)__builtin_amdgcn_rsqf((float)ss);
                inv = r * (1.5 - 0.5 * ss * r * r);
              }
#pragma unroll
              for (int e = 0; e < EPV; ++e) uacc[e] += xe[e] * inv;
            }
          }
          if (PACK) {
            const int sub = l >> 5, kl = l & 31;
            const int c = c0 >> 4, half = (c0 >> 3) & 1;
            const size_t dst = ((size_t)(sub * (D / 16) + c) * 64 + kl + 32 * half) * 8;
            *reinterpret_cast<Vec16*>(pk + dst) = x;
          }
        }
      }
    };
    if (op == 0) token_loop(std::integral_constant<int, 0>{});
    else if (op == 1) token_loop(std::integral_constant<int, 1>{});
    else token_loop(std::integral_constant<int, 2>{});
  } else {
    // V: transpose through LDS, 128 tokens (four 32-key subtiles) at a time.
    uint16_t* pk = vpack + ((size_t)bh * g.nblk + j) * (size_t)g.P * D;
    for (int base = 0; base < g.P; base += 128) {
      const int nrows = min(128, g.P - base);
      constexpr int NB = 4;
      for (int l0 = lrow; l0 < nrows; l0 += NB * TPP) {
        Vec16 xs[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const int lt = base + l0 + b * TPP;
          xs[b] = Vec16{{0u, 0u, 0u, 0u}};
          if (l0 + b * TPP < nrows && lt < box.n) {
            const int tok = block_token(g, box, lt);
            xs[b] = *reinterpret_cast<const Vec16*>(src + (head_base + (size_t)tok * D + c0) * elem);
          }
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const int l = l0 + b * TPP;
          if (l >= nrows) break;
          uint32_t* row = reinterpret_cast<uint32_t*>(&vt[l * VROW + c0]);
#pragma unroll
          for (int e = 0; e < 4; ++e) row[e] = xs[b].w[e];
        }
      }
      __syncthreads();
      // output vectors of this chunk: (sub, m, kc, lane) -> 8 keys at one channel
      const int nsub = nrows >> 5;
      const int nvec = nsub * (D / 32) * 2 * 64;
      for (int t = tid; t < nvec; t += kThreads) {
        const int L = t & 63;
        const int kc = (t >> 6) & 1;
        const int m = (t >> 7) % (D / 32);
        const int s = (t >> 7) / (D / 32);
        const int ch = 32 * m + (L & 31);
        uint32_t w[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const int e0 = 2 * e2, e1 = 2 * e2 + 1;
          // keys of the lane's eight values: the order of the attention
          // kernel's P operand (eight consecutive keys when streaming densely)
          const int k0 = g.dense ? 32 * s + 16 * kc + 8 * (L >> 5) + e0
                                 : 32 * s + 16 * kc + 8 * (e0 >> 2) + 4 * (L >> 5) + (e0 & 3);
          const int k1 = g.dense ? k0 + 1 : 32 * s + 16 * kc + 8 * (e1 >> 2) + 4 * (L >> 5) + (e1 & 3);
          w[e2] = (uint32_t)vt[k0 * VROW + ch] | ((uint32_t)vt[k1 * VROW + ch] << 16);
        }
        const size_t sub_base = (size_t)((base >> 5) + s) * 32 * D;
        const size_t dst = sub_base + ((size_t)(m * 2 + kc) * 64 + L) * 8;
        *reinterpret_cast<Vec16*>(pk + dst) = Vec16{{w[0], w[1], w[2], w[3]}};
      }
      __syncthreads();
    }
  }

  // the spare subtiles after the last packed tile are read (and masked to
  // zero weight) by the attention kernel's two-subtile stages: keep them zero
  if (PACK && role > 0 && j == g.nblk - 1 && bh == g.BH - 1) {
    uint16_t* tail = (role == 1 ? kpack : vpack) + (size_t)g.BH * g.nblk * g.P * D;
    for (int t = tid; t < 64 * D / 8; t += kThreads) *reinterpret_cast<Vec16*>(tail + (size_t)t * 8) = Vec16{{0u, 0u, 0u, 0u}};
  }

  if (!want_mean && !want_sics) return;
  // reduce over token slots: lanes with equal tid % TPT inside the wave ...
#pragma unroll
  for (int off = TPT; off < 64; off <<= 1) {
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
      if (MEAN) acc[e] = sum_op(op, acc[e], __shfl_xor(acc[e], off));
      if (want_sics) uacc[e] += __shfl_xor(uacc[e], off);
    }
  }
  // ... then across the waves
  if (lane < TPT) {
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
      red[wave][c0 + e] = acc[e];
      if (want_sics) ured[wave][c0 + e] = uacc[e];
    }
  }
  __syncthreads();
  if (tid < D && want_mean) {
    double s = red[0][tid];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) s = sum_op(op, s, red[w][tid]);
    mean_out[((size_t)bh * g.nblk + j) * D + tid] = (float)(op == 0 ? s / (double)box.n : s);
  }
  if (want_sics) {
    // |sum_i u_i|^2 over the D channels (threads tid < D), then / n^2
    double u2 = 0.0;
    if (tid < D) {
      double u = 0.0;
#pragma unroll
      for (int w = 0; w < kThreads / 64; ++w) u += ured[w][tid];
      u2 = u * u;
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) u2 += __shfl_xor(u2, off);
    __syncthreads();  // ured is reused below
    if (lane == 0) ured[wave][0] = u2;
    __syncthreads();
    if (tid == 0) {
      double t = 0.0;
#pragma unroll
      for (int w = 0; w < kThreads / 64; ++w) t += ured[w][0];
      const double n = (double)box.n;
      sics_out[(size_t)bh * g.nblk + j] = (float)(t / (n * n));
    }
  }
}

template <bool BF16, int D, bool PACK, bool SICS = false, bool MEAN = true>
hipError_t launch_t(const Geom& g, const void* q, const void* k, const void* v, float* qm, float* km,
                    void* qp, void* kp, void* vp, int roles, hipStream_t s, float* qs = nullptr,
                    float* ks = nullptr) {
  dim3 grid(g.nblk, g.BH, roles);
  summarize_kernel<BF16, D, PACK, SICS, MEAN><<<grid, kThreads, 0, s>>>(
      g, q, k, v, qm, km, (uint16_t*)qp, (uint16_t*)kp, (uint16_t*)vp, qs, ks);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_summarize_sics(const Geom& g, bool bf16, const void* q, const void* k, float* q_mean,
                                 float* k_mean, float* q_sics, float* k_sics, hipStream_t s) {
  if (g.BH == 0) return hipSuccess;
  const bool mean = q_mean != nullptr || k_mean != nullptr;
#define SPADE_SICS_LAUNCH(B, DD)                                                                          \
  return mean ? launch_t<B, DD, false, true, true>(g, q, k, nullptr, q_mean, k_mean, nullptr, nullptr,      \
                                                   nullptr, 2, s, q_sics, k_sics)                          \
              : launch_t<B, DD, false, true, false>(g, q, k, nullptr, q_mean, k_mean, nullptr, nullptr,     \
                                                    nullptr, 2, s, q_sics, k_sics)
  if (bf16) {
    if (g.d == 128) SPADE_SICS_LAUNCH(true, 128);
    SPADE_SICS_LAUNCH(true, 64);
  }
  if (g.d == 128) SPADE_SICS_LAUNCH(false, 128);
  SPADE_SICS_LAUNCH(false, 64);
#undef SPADE_SICS_LAUNCH
}

hipError_t launch_summarize_pack_sics(const Geom& g, const void* q, const void* k, const void* v,
                                     float* q_mean, float* k_mean, void* qpack, void* kpack, void* vpack,
                                     float* q_sics, float* k_sics, hipStream_t s) {
  if (g.BH == 0) return hipSuccess;
  if (g.d == 128)
    return launch_t<true, 128, true, true>(g, q, k, v, q_mean, k_mean, qpack, kpack, vpack, 3, s, q_sics, k_sics);
  return launch_t<true, 64, true, true>(g, q, k, v, q_mean, k_mean, qpack, kpack, vpack, 3, s, q_sics, k_sics);
}

hipError_t launch_summarize(const Geom& g, bool bf16, const void* q, const void* k, const void* v,
                            float* q_mean, float* k_mean, void* qpack, void* kpack, void* vpack,
                            hipStream_t s) {
  if (g.BH == 0) return hipSuccess;
  const bool pack = qpack != nullptr;
  const int roles = pack ? 3 : 2;
  if (bf16) {
    if (g.d == 128)
      return pack ? launch_t<true, 128, true>(g, q, k, v, q_mean, k_mean, qpack, kpack, vpack, roles, s)
                  : launch_t<true, 128, false>(g, q, k, v, q_mean, k_mean, qpack, kpack, vpack, roles, s);
    return pack ? launch_t<true, 64, true>(g, q, k, v, q_mean, k_mean, qpack, kpack, vpack, roles, s)
                : launch_t<true, 64, false>(g, q, k, v, q_mean, k_mean, qpack, kpack, vpack, roles, s);
  }
  if (g.d == 128) return launch_t<false, 128, false>(g, q, k, v, q_mean, k_mean, nullptr, nullptr, nullptr, 2, s);
  return launch_t<false, 64, false>(g, q, k, v, q_mean, k_mean, nullptr, nullptr, nullptr, 2, s);
}

}  // namespace spade
