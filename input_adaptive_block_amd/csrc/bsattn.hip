// Flash block-sparse attention over the kept KV blocks.
//
// SPADE technical summary (gist.science), "Methodology 3. Head-wise Sparse
// Attention Execution": masks become a ranked block-sparse row format that the
// kernel walks sequentially, softmax is computed online so no dense attention
// matrix exists, and heads that share a blocking scheme are grouped into one
// launch to raise occupancy ("Head Grouping").  The pages' kernel targets
// Hopper (TMA, warp-group MMA); this one is written for CDNA4:
//
// * Work item = (selection row, 128-query tile).  One persistent grid pulls
//   items from eight contiguous queues, one per XCD, whose row ranges hold
//   equal shares of kept blocks; a workgroup starts on queue blockIdx % 8 (the
//   XCD the dispatcher places it on) and steals from the next queues when its
//   own is empty.  Neighbouring Q blocks of one head therefore run together on
//   one XCD and share that XCD's L2 for the K/V blocks they both keep.
// * 4 wavefronts x 32 queries.  Scores are computed transposed,
//   S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: each lane then owns one query
//   and 16 keys, so the row max and row sum are in-lane (one cross-half
//   exchange), and the S^T accumulator converted to bf16 is directly the B
//   operand of O^T += V^T P^T.  Q operands stay in registers for the item.
// * K and V come pre-packed (by the summarize kernel) in MFMA operand order,
//   so each 32-key subtile is one contiguous 8 KB copy HBM -> LDS and every
//   LDS operand read is a contiguous 1 KB ds_read_b128 per wavefront.  Stages
//   of two subtiles are double-buffered in LDS (64 KB per workgroup, two
//   workgroups per CU).
// * fp32 online softmax in the exp2 domain with the log2(e) factor folded into
//   the scale; the running max is only moved when a new score exceeds it by
//   more than 2^8, which bounds every p by 256 (exact in value, fewer
//   rescales of the 64-register O accumulator).
#include "spade_internal.h"

namespace spade {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kQTile = 32 * kWaves;  // queries per work item
constexpr float kLazy = 8.0f;        // log2 headroom before a rescale
constexpr bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};

struct alignas(16) Vec16 {
  uint32_t w[4];
};

// ---------------------------------------------------------------------------
// work queues: eight contiguous row ranges of equal cost (kept blocks + 1)
// ---------------------------------------------------------------------------
constexpr int kQThreads = 1024;

__global__ __launch_bounds__(kQThreads) void queue_kernel(int R, const int* __restrict__ row_ptr,
                                                          long long cap, int* __restrict__ queue) {
  __shared__ long long part[kQThreads];
  __shared__ int start[kQueues + 1];
  const int tid = threadIdx.x;
  if (tid <= kQueues) start[tid] = (tid == 0) ? 0 : R;
  const int per = (R + kQThreads - 1) / kQThreads;
  const int lo = min(R, tid * per), hi = min(R, lo + per);
  auto cost = [&](int r) -> long long {
    long long a = row_ptr[r], b = row_ptr[r + 1];
    a = a < 0 ? 0 : (a > cap ? cap : a);
    b = b < a ? a : (b > cap ? cap : b);
    return b - a + 1;
  };
  long long s = 0;
  for (int r = lo; r < hi; ++r) s += cost(r);
  part[tid] = s;
  __syncthreads();
  for (int off = 1; off < kQThreads; off <<= 1) {
    const long long add = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += add;
    __syncthreads();
  }
  const long long total = part[kQThreads - 1];
  long long run = part[tid] - s;  // exclusive prefix before row lo
  for (int r = lo; r < hi; ++r) {
    const long long c = cost(r);
    // start[x] = first row whose exclusive prefix reaches ceil(x * total / 8)
    for (int x = 1; x < kQueues; ++x) {
      const long long t = (x * total + kQueues - 1) / kQueues;
      if (run >= t && run - (r > 0 ? cost(r - 1) : 0) < t) start[x] = r;
    }
    run += c;
  }
  __syncthreads();
  if (tid <= kQueues) queue[tid] = start[tid];
  if (tid < kQueues) queue[kQueues + 1 + tid] = 0;  // cursors
}

// ---------------------------------------------------------------------------
// bf16 attention
// ---------------------------------------------------------------------------

typedef __attribute__((address_space(3))) void lds_void;

constexpr int kListChunk = 4096;  // kept-block ids staged in LDS per pass

// Position in a row's kept-block list: block j (entry pos of the staged list),
// subtiles [s0, s0 + ns) of it, nk valid keys from subtile s0 on.
struct Stage {
  int pos;  // -1: no more stages
  int j;
  int n;    // tokens of block j
  int s0;
  int ns;
  int nk;
};

__device__ inline Stage stage_at(const Geom& g, const uint16_t* list, int cn, int pos, int s0, int j, int n) {
  Stage st;
  for (;;) {
    if (s0 > 0 && s0 < ((n + 31) >> 5)) break;  // more subtiles of the same block
    s0 = 0;
    pos = pos + (j >= 0 ? 1 : 0);
    j = -1;
    while (pos < cn) {
      const int jj = __builtin_amdgcn_readfirstlane((int)list[pos]);
      if (jj < g.nblk) {
        j = jj;
        break;
      }
      ++pos;
    }
    if (j < 0) {
      st.pos = -1;
      st.j = 0; st.n = 0; st.s0 = 0; st.ns = 0; st.nk = 0;
      return st;
    }
    n = block_box(g, j).n;
    break;
  }
  st.pos = pos;
  st.j = j;
  st.n = n;
  st.s0 = s0;
  st.ns = min(2, ((n + 31) >> 5) - s0);
  st.nk = n - 32 * s0;
  return st;
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void bsattn_bf16_kernel(
    Geom g, const uint16_t* __restrict__ qpack, const uint16_t* __restrict__ kpack,
    const uint16_t* __restrict__ vpack, const int* __restrict__ row_ptr, const int* __restrict__ col_idx,
    long long cap, float scale_log2, uint16_t* __restrict__ out, int* __restrict__ queue) {
  constexpr int SUB = 32 * D;          // bf16 elements of one 32-key subtile
  constexpr int SUB_CPY = SUB * 2 / 1024;  // 1 KB wave copies per subtile
  constexpr int NC = D / 16;           // K-chunks of S^T
  constexpr int NM = D / 32;           // channel tiles of O^T
  // two stage buffers as distinct objects, so the compiler can tell the
  // in-flight copy into one from the operand reads of the other
  __shared__ __attribute__((aligned(1024))) uint16_t kvA[2][2 * SUB];  // [K,V][2 subtiles]
  __shared__ __attribute__((aligned(1024))) uint16_t kvB[2][2 * SUB];
  __shared__ uint16_t list[kListChunk];
  __shared__ int s_item;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int nqt = (g.P + kQTile - 1) / kQTile;
  const int* qstart = queue;
  int* qcursor = queue + kQueues + 1;
  int qx = blockIdx.x % kQueues;
  int visited = 0;

  // asynchronous HBM -> LDS copy of a stage (K and V subtiles) into buffer b:
  // each wave moves 1 KB per instruction, lane L's 16 bytes to offset 16 L
  auto issue = [&](const Stage& st, uint16_t (&buf)[2][2 * SUB], size_t head_off) {
    const size_t src = head_off + (size_t)st.j * g.P * D + (size_t)st.s0 * SUB;
    const char* ks = reinterpret_cast<const char*>(kpack + src) + lane * 16;
    const char* vs = reinterpret_cast<const char*>(vpack + src) + lane * 16;
    const int ncpy = st.ns * SUB_CPY;
    for (int t = wave; t < ncpy; t += kWaves) {
      __builtin_amdgcn_global_load_lds(ks + t * 1024, (lds_void*)(&buf[0][t * 512]), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(vs + t * 1024, (lds_void*)(&buf[1][t * 512]), 16, 0, 0);
    }
  };

  for (;;) {
    if (tid == 0) {
      int item = -1;
      while (visited < kQueues) {
        const int n = (qstart[qx + 1] - qstart[qx]) * nqt;
        const int it = n > 0 ? atomicAdd(&qcursor[qx], 1) : 0;
        if (it < n) {
          item = qstart[qx] * nqt + it;
          break;
        }
        ++visited;
        qx = (qx + 1) % kQueues;
      }
      s_item = item;
    }
    __syncthreads();
    const int item = s_item;
    if (item < 0) break;

    const int row = item / nqt;
    const int qt = item - row * nqt;
    const int bh = row / g.nblk;
    const int i = row - bh * g.nblk;
    const BlockBox qbox = block_box(g, i);
    const int qsub = qt * kWaves + wave;
    const bool active = 32 * qsub < qbox.n;

    // Q^T operands for this wave's 32 queries
    bf16x8 qop[NC];
    if (active) {
      const uint16_t* qp = qpack + ((size_t)bh * g.nblk + i) * (size_t)g.P * D + (size_t)qsub * SUB;
#pragma unroll
      for (int c = 0; c < NC; ++c) qop[c] = *reinterpret_cast<const bf16x8*>(qp + ((size_t)c * 64 + lane) * 8);
    }

    long long lo = row_ptr[row], hi = row_ptr[row + 1];
    lo = lo < 0 ? 0 : (lo > cap ? cap : lo);
    hi = hi < lo ? lo : (hi > cap ? cap : hi);

    f32x16 acc[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[m][v] = 0.f;
    float mref = -__builtin_huge_valf();
    float lsum = 0.f;
    const size_t head_off = (size_t)bh * g.nblk * (size_t)g.P * D;

    // one stage: S^T, online softmax and O^T update for each of its subtiles
    auto compute = [&](const Stage& st_, uint16_t (&buf)[2][2 * SUB]) {
        if (active) {
          for (int st = 0; st < st_.ns; ++st) {
            const bf16x8* kl = reinterpret_cast<const bf16x8*>(&buf[0][st * SUB]);
            const bf16x8* vl = reinterpret_cast<const bf16x8*>(&buf[1][st * SUB]);
            f32x16 s;
#pragma unroll
            for (int v = 0; v < 16; ++v) s[v] = 0.f;
#pragma unroll
            for (int c = 0; c < NC; ++c)
              s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kl[c * 64 + lane], qop[c], s, 0, 0, 0);
            const int kvalid = st_.nk - 32 * st;
            if (kvalid < 32) {
#pragma unroll
              for (int v = 0; v < 16; ++v) {
                const int key = 8 * (v >> 2) + 4 * half + (v & 3);
                if (key >= kvalid) s[v] = -__builtin_huge_valf();
              }
            }
            float mx = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
            for (int v = 3; v < 15; v += 2) mx = fmaxf(fmaxf(mx, s[v]), s[v + 1]);
            mx = fmaxf(mx, s[15]);
            {
              const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
              mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
            }
            const float mnew = mx * scale_log2;
            if (mnew > mref + kLazy) {
              const float alpha = __builtin_amdgcn_exp2f(mref - mnew);
              lsum *= alpha;
#pragma unroll
              for (int m = 0; m < NM; ++m)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[m][v] *= alpha;
              mref = mnew;
            }
            // p in bf16 (RNE); the row sum adds exactly those rounded values
            // (v_dot2_f32_bf16 against ones), so the normalisation matches
            // the weights the PV product uses
            bf16x2 pr[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * e], scale_log2, -mref));
              const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * e + 1], scale_log2, -mref));
              pr[e][0] = (__bf16)p0;
              pr[e][1] = (__bf16)p1;
              lsum = __builtin_amdgcn_fdot2_f32_bf16(pr[e], kOnes2, lsum, false);
            }
            const bf16x8 pk0 = __builtin_shufflevector(__builtin_shufflevector(pr[0], pr[1], 0, 1, 2, 3),
                                                       __builtin_shufflevector(pr[2], pr[3], 0, 1, 2, 3),
                                                       0, 1, 2, 3, 4, 5, 6, 7);
            const bf16x8 pk1 = __builtin_shufflevector(__builtin_shufflevector(pr[4], pr[5], 0, 1, 2, 3),
                                                       __builtin_shufflevector(pr[6], pr[7], 0, 1, 2, 3),
                                                       0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
            for (int m = 0; m < NM; ++m) {
              acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vl[(m * 2 + 0) * 64 + lane], pk0, acc[m], 0, 0, 0);
              acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vl[(m * 2 + 1) * 64 + lane], pk1, acc[m], 0, 0, 0);
            }
          }
        }
    };

    for (long long c0 = lo; c0 < hi; c0 += kListChunk) {
      const int cn = (int)min((long long)kListChunk, hi - c0);
      __syncthreads();  // earlier readers of list / kv are done
      for (int t = tid; t < cn; t += kThreads) {
        const int j = col_idx[c0 + t];
        list[t] = (j >= 0 && j < g.nblk) ? (uint16_t)j : (uint16_t)0xFFFF;
      }
      __syncthreads();
      Stage cur = stage_at(g, list, cn, 0, 0, -1, 0);
      if (cur.pos < 0) continue;
      issue(cur, kvA, head_off);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      // stages alternate between kvA and kvB; the copy of the next stage is
      // in flight while this one is computed
      for (;;) {
        const Stage nxt = stage_at(g, list, cn, cur.pos, cur.s0 + cur.ns, cur.j, cur.n);
        if (nxt.pos >= 0) issue(nxt, kvB, head_off);
        compute(cur, kvA);
        // the next stage's copy has landed for this wave; the barrier makes
        // it (and the end of every read of the other buffer) visible to all
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (nxt.pos < 0) break;
        cur = stage_at(g, list, cn, nxt.pos, nxt.s0 + nxt.ns, nxt.j, nxt.n);
        if (cur.pos >= 0) issue(cur, kvA, head_off);
        compute(nxt, kvB);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (cur.pos < 0) break;
      }
    }

    if (active) {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lsum), __float_as_uint(lsum), false, false);
      const float ltot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      const float inv = ltot > 0.f ? 1.0f / ltot : 0.f;
      const int qi = 32 * qsub + (lane & 31);
      if (qi < qbox.n) {
        const int tok = block_token(g, qbox, qi);
        uint16_t* orow = out + ((size_t)bh * g.N + tok) * D;
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int v4 = 0; v4 < 4; ++v4) {
            const int d0 = 32 * m + 8 * v4 + 4 * half;
            uint32_t w0 = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(acc[m][4 * v4 + 0] * inv)) |
                          ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(acc[m][4 * v4 + 1] * inv)) << 16);
            uint32_t w1 = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(acc[m][4 * v4 + 2] * inv)) |
                          ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(acc[m][4 * v4 + 3] * inv)) << 16);
            *reinterpret_cast<uint2*>(orow + d0) = make_uint2(w0, w1);
          }
      }
    }
    __syncthreads();  // s_item and list are reused by the next item
  }
}

// ---------------------------------------------------------------------------
// fp32 debug attention: plain FMA, exact expf, one thread per query
// ---------------------------------------------------------------------------
constexpr int kF32Threads = 128;
constexpr int kF32Keys = 32;

template <int D>
__global__ __launch_bounds__(kF32Threads) void bsattn_f32_kernel(
    Geom g, const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const int* __restrict__ row_ptr, const int* __restrict__ col_idx, long long cap, float scale,
    float* __restrict__ out) {
  __shared__ float ks[kF32Keys][D];
  __shared__ float vs[kF32Keys][D];
  const int row = blockIdx.x;
  const int bh = row / g.nblk;
  const int i = row - bh * g.nblk;
  const BlockBox qbox = block_box(g, i);
  const int qi = blockIdx.y * kF32Threads + threadIdx.x;
  const bool active = qi < qbox.n;
  const size_t head = (size_t)bh * g.N * D;
  float qr[D], o[D];
  if (active) {
    const int tok = block_token(g, qbox, qi);
#pragma unroll
    for (int c = 0; c < D; ++c) qr[c] = q[head + (size_t)tok * D + c];
  }
#pragma unroll
  for (int c = 0; c < D; ++c) o[c] = 0.f;
  float m = -__builtin_huge_valf(), l = 0.f;
  long long lo = row_ptr[row], hi = row_ptr[row + 1];
  lo = lo < 0 ? 0 : (lo > cap ? cap : lo);
  hi = hi < lo ? lo : (hi > cap ? cap : hi);
  for (long long kb = lo; kb < hi; ++kb) {
    const int j = col_idx[kb];
    if (j < 0 || j >= g.nblk) continue;
    const BlockBox kbox = block_box(g, j);
    for (int base = 0; base < kbox.n; base += kF32Keys) {
      const int nk = min(kF32Keys, kbox.n - base);
      __syncthreads();
      for (int t = threadIdx.x; t < nk * D; t += kF32Threads) {
        const int kk = t / D, c = t - kk * D;
        const int tok = block_token(g, kbox, base + kk);
        ks[kk][c] = k[head + (size_t)tok * D + c];
        vs[kk][c] = v[head + (size_t)tok * D + c];
      }
      __syncthreads();
      if (active) {
        for (int kk = 0; kk < nk; ++kk) {
          float dot = 0.f;
#pragma unroll
          for (int c = 0; c < D; ++c) dot = __builtin_fmaf(qr[c], ks[kk][c], dot);
          const float x = dot * scale;
          if (x > m) {
            const float alpha = expf(m - x);
            l = l * alpha + 1.0f;
#pragma unroll
            for (int c = 0; c < D; ++c) o[c] = __builtin_fmaf(o[c], alpha, vs[kk][c]);
            m = x;
          } else {
            const float p = expf(x - m);
            l += p;
#pragma unroll
            for (int c = 0; c < D; ++c) o[c] = __builtin_fmaf(p, vs[kk][c], o[c]);
          }
        }
      }
    }
  }
  if (active) {
    const int tok = block_token(g, qbox, qi);
    const float inv = l > 0.f ? 1.0f / l : 0.f;
#pragma unroll
    for (int c = 0; c < D; ++c) out[head + (size_t)tok * D + c] = o[c] * inv;
  }
}

}  // namespace

hipError_t launch_bsattn_bf16(const Geom& g, const void* qpack, const void* kpack, const void* vpack,
                              const int* row_ptr, const int* col_idx, long long col_capacity, float scale,
                              void* o, int* queue, int num_cus, hipStream_t s) {
  if (g.R == 0) return hipSuccess;
  queue_kernel<<<1, kQThreads, 0, s>>>(g.R, row_ptr, col_capacity, queue);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long items = (long long)g.R * ((g.P + kQTile - 1) / kQTile);
  long long grid = (long long)num_cus * 2;
  if (grid > items) grid = items;
  if (grid < 1) grid = 1;
  const float scale_log2 = scale * 1.4426950408889634f;
  if (g.d == 128)
    bsattn_bf16_kernel<128><<<(unsigned)grid, kThreads, 0, s>>>(
        g, (const uint16_t*)qpack, (const uint16_t*)kpack, (const uint16_t*)vpack, row_ptr, col_idx,
        col_capacity, scale_log2, (uint16_t*)o, queue);
  else
    bsattn_bf16_kernel<64><<<(unsigned)grid, kThreads, 0, s>>>(
        g, (const uint16_t*)qpack, (const uint16_t*)kpack, (const uint16_t*)vpack, row_ptr, col_idx,
        col_capacity, scale_log2, (uint16_t*)o, queue);
  return hipGetLastError();
}

hipError_t launch_bsattn_f32(const Geom& g, const float* q, const float* k, const float* v,
                             const int* row_ptr, const int* col_idx, long long col_capacity, float scale,
                             float* o, hipStream_t s) {
  if (g.R == 0) return hipSuccess;
  dim3 grid(g.R, (g.P + kF32Threads - 1) / kF32Threads);
  if (g.d == 128)
    bsattn_f32_kernel<128><<<grid, kF32Threads, 0, s>>>(g, q, k, v, row_ptr, col_idx, col_capacity, scale, o);
  else
    bsattn_f32_kernel<64><<<grid, kF32Threads, 0, s>>>(g, q, k, v, row_ptr, col_idx, col_capacity, scale, o);
  return hipGetLastError();
}

}  // namespace spade
