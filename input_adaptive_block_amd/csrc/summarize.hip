// Fused blocking + Summarizer kernel.
//
// SPADE technical summary (gist.science), "Methodology 3. Head-wise Sparse
// Attention Execution", Kernel Fusion: the layout transformation into blocks
// and the block summaries come out of one pass over Q/K/V.  Summarizer
// ("Methodology 1. vDiT-SSR", Summarizer & Estimator Expressions): the mean of
// a block's real tokens.
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
#include "spade_internal.h"

namespace spade {
namespace {

constexpr int kThreads = 256;

struct alignas(16) Vec16 {
  uint32_t w[4];
};

__device__ inline float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ inline float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

template <bool BF16, int D, bool PACK>
__global__ __launch_bounds__(kThreads) void summarize_kernel(
    Geom g, const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    float* __restrict__ q_mean, float* __restrict__ k_mean, uint16_t* __restrict__ qpack,
    uint16_t* __restrict__ kpack, uint16_t* __restrict__ vpack) {
  constexpr int EPV = BF16 ? 8 : 4;     // elements per 16-byte vector
  constexpr int TPT = D / EPV;          // threads per token row
  constexpr int TPP = kThreads / TPT;   // tokens per pass
  constexpr int VROW = D + 8;           // LDS row stride (bf16) of the V transpose
  static_assert(kThreads % TPT == 0, "layout");

  const int j = blockIdx.x;
  const int bh = blockIdx.y;
  const int role = blockIdx.z;
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
  const bool want_mean = mean_out != nullptr;

  __shared__ double red[kThreads / 64][D];
  __shared__ uint16_t vt[PACK ? 128 * VROW : 1];

  double acc[EPV];
#pragma unroll
  for (int e = 0; e < EPV; ++e) acc[e] = 0.0;

  if (role < 2 || !PACK) {
    uint16_t* pk = nullptr;
    if (PACK) pk = (role == 0 ? qpack : kpack) + ((size_t)bh * g.nblk + j) * (size_t)g.P * D;
    const int rows = PACK ? g.P : box.n;
    for (int l = lrow; l < rows; l += TPP) {
      Vec16 x = {{0u, 0u, 0u, 0u}};
      if (l < box.n) {
        const int tok = block_token(g, box, l);
        x = *reinterpret_cast<const Vec16*>(src + (head_base + (size_t)tok * D + c0) * elem);
        if (want_mean) {
          if (BF16) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              acc[2 * e] += (double)bf16_lo(x.w[e]);
              acc[2 * e + 1] += (double)bf16_hi(x.w[e]);
            }
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] += (double)__uint_as_float(x.w[e]);
          }
        }
      }
      if (PACK) {
        const int sub = l >> 5, kl = l & 31;
        const int c = c0 >> 4, half = (c0 >> 3) & 1;
        const size_t dst = ((size_t)(sub * (D / 16) + c) * 64 + kl + 32 * half) * 8;
        *reinterpret_cast<Vec16*>(pk + dst) = x;
      }
    }
  } else {
    // V: transpose through LDS, 128 tokens (four 32-key subtiles) at a time.
    uint16_t* pk = vpack + ((size_t)bh * g.nblk + j) * (size_t)g.P * D;
    for (int base = 0; base < g.P; base += 128) {
      const int nrows = min(128, g.P - base);
      for (int l = lrow; l < nrows; l += TPP) {
        Vec16 x = {{0u, 0u, 0u, 0u}};
        const int lt = base + l;
        if (lt < box.n) {
          const int tok = block_token(g, box, lt);
          x = *reinterpret_cast<const Vec16*>(src + (head_base + (size_t)tok * D + c0) * elem);
        }
        uint32_t* row = reinterpret_cast<uint32_t*>(&vt[l * VROW + c0]);
#pragma unroll
        for (int e = 0; e < 4; ++e) row[e] = x.w[e];
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
          const int k0 = 32 * s + 16 * kc + 8 * (e0 >> 2) + 4 * (L >> 5) + (e0 & 3);
          const int k1 = 32 * s + 16 * kc + 8 * (e1 >> 2) + 4 * (L >> 5) + (e1 & 3);
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

  if (!want_mean) return;
  // reduce over token slots: lanes with equal tid % TPT inside the wave ...
#pragma unroll
  for (int off = TPT; off < 64; off <<= 1) {
#pragma unroll
    for (int e = 0; e < EPV; ++e) acc[e] += __shfl_xor(acc[e], off);
  }
  // ... then across the waves
  if (lane < TPT) {
#pragma unroll
    for (int e = 0; e < EPV; ++e) red[wave][c0 + e] = acc[e];
  }
  __syncthreads();
  if (tid < D) {
    double s = 0.0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) s += red[w][tid];
    mean_out[((size_t)bh * g.nblk + j) * D + tid] = (float)(s / (double)box.n);
  }
}

template <bool BF16, int D, bool PACK>
hipError_t launch_t(const Geom& g, const void* q, const void* k, const void* v, float* qm, float* km,
                    void* qp, void* kp, void* vp, int roles, hipStream_t s) {
  dim3 grid(g.nblk, g.BH, roles);
  summarize_kernel<BF16, D, PACK><<<grid, kThreads, 0, s>>>(
      g, q, k, v, qm, km, (uint16_t*)qp, (uint16_t*)kp, (uint16_t*)vp);
  return hipGetLastError();
}

}  // namespace

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
