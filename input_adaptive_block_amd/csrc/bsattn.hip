// Flash block-sparse attention over the kept KV blocks.
//
// SPADE technical summary (gist.science), "Methodology 3. Head-wise Sparse
// Attention Execution": masks become a ranked block-sparse row format that the
// kernel walks sequentially, softmax is computed online so no dense attention
// matrix exists, and heads that share a blocking scheme are grouped into one
// launch to raise occupancy ("Head Grouping").  The pages' kernel targets
// Hopper (TMA, warp-group MMA); this one is written for CDNA4:
//
// * Work unit = twelve consecutive (row, 32-query subtile) items of one head,
//   one per wavefront: three rows of 120-token blocks, six of 64-token blocks,
//   up to twelve of small ones -- neighbouring Q blocks, whose kept KV sets
//   overlap heavily.  The unit streams the UNION of its rows' kept blocks once
//   (ascending block id, each entry with the mask of the rows keeping it);
//   each wavefront computes only on the blocks its own row keeps.  A K/V byte
//   fetched once serves every row of the unit that keeps its block, which
//   cuts L2 / Infinity-Cache traffic on video layers, where neighbouring rows
//   keep mostly the same blocks.  When the units would leave a last round
//   less than half full (a small layer has only a few units per CU), that
//   round's units go out as twice as many halves of six items each.
// * One persistent workgroup of 12 wavefronts per CU (three per SIMD) takes
//   units from one atomic counter in (head, row) order, so the units in
//   flight across the chip read the K/V of one or two heads, which stay in the
//   Infinity Cache.  With three wavefronts per SIMD, one wave's softmax runs
//   beside the others' MFMAs.
// * Scores are computed transposed, S^T = K Q^T, with
//   v_mfma_f32_32x32x16_bf16: each lane owns one query and 16 keys, so the row
//   sum is in-lane plus one permlane32 swap at the end, the lazy-rescale test
//   runs on each lane's own maximum (the two halves of a query exchange maxima
//   only when a lane clears it), and the S^T accumulator converted to bf16 is
//   directly the B operand of O^T += V^T P^T.  Q operands stay in registers
//   for the unit.
// * K and V come pre-packed (by the summarize kernel) in MFMA operand order:
//   a stage (two 32-key subtiles of K and of V, 32 KB at d = 128) is a
//   contiguous HBM -> LDS copy issued with global_load_lds_dwordx4 by eight
//   of the wavefronts, and every LDS operand read is a contiguous 1 KB
//   ds_read_b128 per wavefront (no bank conflicts).  Four stage slots form a
//   ring with one barrier per stage: stage s is computed while stages s+1 to
//   s+3 are in flight.  Each copying wave issues stage s+3 into the slot of
//   stage s-1 right after its own steps of stage s (every wave left that
//   slot before the barrier of stage s), so the copies are issued while the
//   other waves still compute.  Every wave walks the stages it computes with
//   a small cursor; only the copying waves also walk the stages they copy.
//   The youngest wave of a SIMD loses the MFMA arbitration and ends each stage
//   last, so the instructions between its steps are kept few.  Operands are
//   read just ahead of their MFMAs into small register rings, which keeps a
//   wavefront within the 168 registers that three wavefronts per SIMD allow.
//   The step is compiled twice: for any subtile (a per-key mask when fewer
//   than 32 keys are real), and for one with 24 real keys (the last subtile
//   of a 120-token block), which skips the mask and the padding's exps.
// * A wavefront raises its issue priority for its runs of MFMAs, so a wave
//   that reaches its MFMAs keeps the matrix pipe while the others run their
//   softmax arithmetic beside it.
// * Blocks that pad badly to 32-key subtiles (every block a multiple of 8
//   tokens, at least 32, and a full block 16 or more keys short of whole
//   subtiles, e.g. 72 -> 96) are walked densely instead: the unit's union is
//   one key stream cut into 32-key subtiles that may straddle two blocks.
//   Each lane's 16-byte copy is gathered from the block holding its key; K
//   rows are loaded with bits 2 and 3 of the key swapped and V is packed in
//   8-key groups, so that a lane's P operand and V operand hold the same
//   eight consecutive keys; a row computes the part of a subtile its kept
//   blocks cover, under a key-range mask.
// * fp32 online softmax in the exp2 domain with log2(e) folded into the scale;
//   the running max only moves when a score exceeds it by more than 2^8, which
//   bounds every p by 256 (exact in value, fewer rescales of the 64-register O
//   accumulator).  p is rounded to bf16 once and the row sum adds exactly the
//   rounded values, so normalisation matches the weights PV used.  The PV
//   MFMAs of the first 16 keys of a lane run while the exp of its second 16
//   is computed.
#include <type_traits>
#include "spade_internal.h"

namespace spade {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kCopyWaves = 8;                     // waves that issue the stage copies
constexpr int kWaves = 12;                        // one 32-query item per wave
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxUnitRows = kWaves;              // rows a unit's items can span
constexpr float kLazy = 8.0f;                     // log2 headroom before a rescale
constexpr bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};

// Work units: the (row, 32-query subtile) items of one head in order, one
// per wave, kWaves at a time.  A unit spans ceil(kWaves / nsub) rows or so
// (three rows of 120-token blocks, six of 64-token blocks), never more than
// kMaxUnitRows.
struct UnitMap {
  int nsub;        // 32-query subtiles per row (P / 32)
  int items;       // items per head = nblk * nsub
  int per_head;    // units per head = ceil(items / kWaves)
};

__host__ __device__ inline UnitMap unit_map(const Geom& g) {
  UnitMap u;
  u.nsub = g.P / 32;
  u.items = g.nblk * u.nsub;
  u.per_head = (u.items + kWaves - 1) / kWaves;
  return u;
}

// the attention kernel's unit counter, cleared on the launch stream before
// each launch (a kernel, so that the launch sequence can be captured)
__global__ void counter_reset_kernel(int* __restrict__ counter) { *counter = 0; }

// ---------------------------------------------------------------------------
// bf16 attention
// ---------------------------------------------------------------------------

// A walk over the unit's union list, one stage (two 32-key subtiles of one
// block) at a time: entry pos, its first subtile s0, the block's token count n
// and the entry word (block id | mask of the unit's rows keeping it << 12).
// The entry after pos is read one block ahead (ae, an), so that a new block
// never waits for its LDS read.
struct Cursor {
  int pos;
  int s0;
  int n;
  int word;
  uint32_t ae;
  uint32_t an;
};

__device__ inline void cursor_take(Cursor& c, const uint32_t* ul, const uint16_t* un, int cnt) {
  c.word = __builtin_amdgcn_readfirstlane((int)c.ae);
  c.n = __builtin_amdgcn_readfirstlane((int)c.an);
  const int pa = min(c.pos + 1, cnt - 1);
  c.ae = ul[pa];
  c.an = un[pa];
}

__device__ inline Cursor cursor_start(const uint32_t* ul, const uint16_t* un, int cnt) {
  Cursor c;
  c.pos = 0;
  c.s0 = 0;
  c.n = 0;
  c.word = 0;
  c.ae = ul[0];
  c.an = un[0];
  if (cnt > 0) cursor_take(c, ul, un, cnt);
  return c;
}

__device__ inline void cursor_next(Cursor& c, const uint32_t* ul, const uint16_t* un, int cnt) {
  c.s0 += 2;
  if (32 * c.s0 >= c.n) {
    c.s0 = 0;
    if (++c.pos < cnt) cursor_take(c, ul, un, cnt);
  }
}

// A walk over the unit's key stream when every block holds a multiple of 8
// tokens and at least 32: the kept blocks' keys back to back, one 32-key
// subtile at a time.  The subtile starts at key kb of union entry pos; when
// fewer than 32 of that entry's keys remain (b = n - kb < 32), its other
// keys are the first 32 - b of entry pos + 1.  The entry after pos is read
// one entry ahead (ae, an; zero past the last entry).
struct DCursor {
  int pos;
  int kb;
  int word;  // entry pos: block id | mask of the unit's rows keeping it << 12
  int n;     // entry pos: tokens (0 past the last entry)
  uint32_t ae;
  uint32_t an;
};

__device__ inline DCursor dcursor_start(const uint32_t* ul, const uint16_t* un, int cnt) {
  DCursor c;
  c.pos = 0;
  c.kb = 0;
  c.word = cnt > 0 ? __builtin_amdgcn_readfirstlane((int)ul[0]) : 0;
  c.n = cnt > 0 ? __builtin_amdgcn_readfirstlane((int)un[0]) : 0;
  c.ae = cnt > 1 ? ul[1] : 0u;
  c.an = cnt > 1 ? un[1] : 0u;
  return c;
}

__device__ inline void dcursor_next(DCursor& c, const uint32_t* ul, const uint16_t* un, int cnt) {
  c.kb += 32;
  if (c.kb >= c.n) {
    c.kb -= c.n;
    ++c.pos;
    c.word = __builtin_amdgcn_readfirstlane((int)c.ae);
    c.n = __builtin_amdgcn_readfirstlane((int)c.an);
    const bool more = c.pos + 1 < cnt;
    const int pa = more ? c.pos + 1 : 0;
    c.ae = more ? ul[pa] : 0u;
    c.an = more ? un[pa] : 0u;
  }
}

// Key order of a streamed K subtile: operand row r holds key r with bits 2
// and 3 swapped, so that the eight scores a lane turns into one P operand are
// eight consecutive keys, the keys its V operand holds (one 8-key group).
__device__ inline int dense_key_of_row(int r) { return (r & ~0xC) | ((r & 4) << 1) | ((r & 8) >> 1); }

// s_waitcnt immediate on gfx9: vmcnt in bits 3:0
// and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima (no wait).
constexpr int vm_wait_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }


template <int D, bool DENSE>
__global__ __launch_bounds__(kThreads, 1) void bsattn_bf16_kernel(
    Geom g, const uint16_t* __restrict__ qpack, const uint16_t* __restrict__ kpack,
    const uint16_t* __restrict__ vpack, const int* __restrict__ row_ptr, const int* __restrict__ col_idx,
    long long cap, float scale_log2, uint16_t* __restrict__ out, int* __restrict__ counter, int U, int Ufull) {
  constexpr int SUB = 32 * D;                  // bf16 elements of one 32-key subtile
  constexpr int STAGE_KB = 2 * SUB * 2 / 1024;  // 1 KB copies per tensor per stage (2 subtiles)
  constexpr int CPW = STAGE_KB / kCopyWaves;   // copies per copying wave per tensor
  constexpr int PER = 2 * CPW;                 // copy instructions per wave per stage
  constexpr int NC = D / 16;                   // K-chunks of S^T
  constexpr int NM = D / 32;                   // channel tiles of O^T
  static_assert(STAGE_KB % kCopyWaves == 0, "stage copies split evenly over the copying waves");
  // four stage slots; the copies into them are issued from inline asm, so the
  // compiler does not order the slot being read behind the copies in flight
  __shared__ __attribute__((aligned(1024))) uint16_t ring[4 * 2 * 2 * SUB];  // [slot][K,V][2 subtiles]
  // union list entries: block id | mask of the unit's rows keeping it << 12
  __shared__ uint32_t ulist[kMaxBlocks];
  __shared__ uint16_t ublkn[kMaxBlocks];  // tokens of each union entry's block
  // per-block row masks while the union is built (two blocks per word), in
  // the ring, which holds no stage between units
  uint32_t* const rowbits = reinterpret_cast<uint32_t*>(ring);
  static_assert(kMaxBlocks / 2 * 4 <= 4 * 2 * 2 * SUB * 2, "row masks fit in the ring");
  __shared__ int scanbuf[kThreads];
  __shared__ int s_unit;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: row-mask tests stay scalar
  const int half = lane >> 5;
  const UnitMap um = unit_map(g);

  for (;;) {
    if (tid == 0) {
      const int unit = atomicAdd(counter, 1);
      s_unit = unit < U ? unit : -1;
    }
    __syncthreads();
    const int unit = s_unit;
    if (unit < 0) break;
    // Code placement: these no-ops put the stage loop's code 16 bytes past a
    // 32-byte boundary (the first MFMA of the d = 128 kernel), the phase at
    // which that loop measures about 1 % faster than at the other 8-byte
    // phases; a host test checks the offset in the built code object.
    asm volatile("s_nop 0\n\ts_nop 0\n\ts_nop 0\n\ts_nop 0\n\ts_nop 0\n\ts_nop 0");

    // ids from Ufull on are halves of the last units, six items each (waves
    // 6 .. 11 idle): a last round that would keep only a few CUs busy is
    // spread over twice as many, each walking the smaller union of its rows
    const int whole = unit < Ufull ? unit : Ufull + ((unit - Ufull) >> 1);
    const int nit = unit < Ufull ? kWaves : kWaves / 2;  // items of this unit
    const int bh = whole / um.per_head;
    const int pi = whole - bh * um.per_head;
    const size_t head_off = (size_t)bh * g.nblk * (size_t)g.P * D;
    const int it0 = kWaves * pi + (unit >= Ufull && ((unit - Ufull) & 1) ? kWaves / 2 : 0);
    if (!head_active(g, bh) || it0 >= um.items) {
      // another scheme's head, or the empty second half of a head's last
      // unit: nothing to compute or write; s_unit is reused
      __syncthreads();
      continue;
    }

    // ---- the unit's union list of kept blocks, with row masks ----
    const int it_last = min(um.items, it0 + nit) - 1;
    const int row0 = it0 / um.nsub;
    const int nrows = it_last / um.nsub - row0 + 1;  // 1 .. kMaxUnitRows
    for (int t = tid; t < (g.nblk + 1) / 2; t += kThreads) rowbits[t] = 0u;
    __syncthreads();
    for (int m = 0; m < nrows; ++m) {
      const int r = bh * g.nblk + row0 + m;
      long long a = row_ptr[r], b = row_ptr[r + 1];
      a = a < 0 ? 0 : (a > cap ? cap : a);
      b = b < a ? a : (b > cap ? cap : b);
      for (long long e = a + tid; e < b; e += kThreads) {
        const int j = col_idx[e];
        if (j >= 0 && j < g.nblk) atomicOr(&rowbits[j >> 1], (1u << m) << (16 * (j & 1)));
      }
    }
    __syncthreads();
    auto row_mask = [&](int j) __attribute__((always_inline)) { return (rowbits[j >> 1] >> (16 * (j & 1))) & 0xFFFFu; };
    const int per = (g.nblk + kThreads - 1) / kThreads;
    const int jb = min(g.nblk, tid * per), je = min(g.nblk, jb + per);
    int cnt = 0;
    for (int j = jb; j < je; ++j) cnt += row_mask(j) != 0u;
    scanbuf[tid] = cnt;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {
      const int add = tid >= off ? scanbuf[tid - off] : 0;
      __syncthreads();
      scanbuf[tid] += add;
      __syncthreads();
    }
    {
      int w = scanbuf[tid] - cnt;
      for (int j = jb; j < je; ++j) {
        const uint32_t msk = row_mask(j);
        if (msk) {
          ublkn[w] = (uint16_t)block_box(g, j).n;
          ulist[w++] = (uint32_t)j | (msk << 12);
        }
      }
    }
    const int ucnt = scanbuf[kThreads - 1];
    __syncthreads();  // the ring is free again for the stage copies

    // ---- this wave's 32 queries ----
    const int my_it = it0 + wave;
    const bool has_item = wave < nit && my_it < um.items;
    const int my_i = has_item ? my_it / um.nsub : row0;
    const int qsub = has_item ? my_it - my_i * um.nsub : 0;
    const int my_row = my_i - row0;  // this wave's bit in the union masks
    const BlockBox qbox = block_box(g, my_i);
    const bool active = has_item && 32 * qsub < qbox.n;
    bf16x8 qop[NC];
    if (active) {
      const uint16_t* qp = qpack + ((size_t)bh * g.nblk + my_i) * (size_t)g.P * D + (size_t)qsub * SUB;
#pragma unroll
      for (int c = 0; c < NC; ++c) qop[c] = *reinterpret_cast<const bf16x8*>(qp + ((size_t)c * 64 + lane) * 8);
    }
    // the Q loads are the only loads the compiler tracks; retire them here so
    // that no wait inside the pipeline (which would also drain the stage
    // copies in flight) is needed for them
    __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
    f32x16 acc[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[m][v] = 0.f;
    // running max (exp2 domain); finite so that the first rescale factor is 0
    float mref = -1e30f;
    float mlazy = mref + kLazy;  // a score above this moves the running max
    float lsum = 0.f;
    // asynchronous HBM -> LDS copy of a stage into ring slot `slot`: always
    // two subtiles (the pack buffers carry one spare subtile at their end);
    // wave w copies KB w*CPW .. w*CPW+CPW-1 of K and of V, lane L's 16 bytes
    // land at 16 L.  M0 holds the wave's LDS destination.
    const uint32_t ring_lds = (uint32_t)(uintptr_t)(lds_void*)ring;
    auto issue = [&](const Cursor& st, int slot) __attribute__((always_inline)) {
      const size_t src = head_off + (size_t)(st.word & 0xFFF) * g.P * D + (size_t)st.s0 * SUB;
      const char* ks = reinterpret_cast<const char*>(kpack + src) + lane * 16;
      const char* vs = reinterpret_cast<const char*>(vpack + src) + lane * 16;
#pragma unroll
      for (int c = 0; c < CPW; ++c) {
        const int t = wave * CPW + c;
        const uint32_t kd = __builtin_amdgcn_readfirstlane(ring_lds + (uint32_t)(slot * 4 * SUB + t * 512) * 2u);
        const uint32_t vd = kd + 2 * SUB * 2;
        const char* kg = ks + t * 1024;
        const char* vg = vs + t * 1024;
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(kg), "s"(kd) : "memory", "m0");
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(vg), "s"(vd) : "memory", "m0");
      }
    };
    // One subtile of 32 keys at element offsets kx (K) / vx (V) of the ring:
    // S^T = K Q^T (8 MFMAs; each K operand read two MFMAs ahead into a ring of
    // three), the key mask of a partial subtile, the row max with the rare
    // lazy rescale, p = exp2(S scale - m) rounded to bf16 and its row sum,
    // then O^T += V^T P^T (8 MFMAs; V operands read two MFMAs ahead).  Three
    // wavefronts per SIMD overlap one wave's softmax with the others' MFMAs.
    //
    // VE (a compile-time constant) is the number of each lane's 16 scores that
    // are real keys when that does not depend on the lane (12 for 24 valid
    // keys); VE = 0 masks the keys from kvalid when it is below 32.
    auto step = [&](auto ve_c, int klo, int kvalid, int kx, int vx) __attribute__((always_inline)) {
      constexpr int VE = decltype(ve_c)::value;
      constexpr int NP = VE == 0 ? 8 : VE / 2;  // pairs of scores that can hold a real key
      const bf16x8* kl = reinterpret_cast<const bf16x8*>(ring + kx);
      const bf16x8* vl = reinterpret_cast<const bf16x8*>(ring + vx);
      bf16x8 kr[3];
      kr[0] = kl[lane];
      kr[1] = kl[64 + lane];
      f32x16 sx;
#pragma unroll
      for (int v = 0; v < 16; ++v) sx[v] = 0.f;
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        if (c + 2 < NC) kr[(c + 2) % 3] = kl[(c + 2) * 64 + lane];
        sx = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[c % 3], qop[c], sx, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_setprio(0);
      // V operand order of the PV MFMAs: i -> (channel tile i % NM, key chunk i / NM)
      bf16x8 vr[3];
      vr[0] = vl[(2 * (0 % NM) + 0 / NM) * 64 + lane];
      vr[1] = vl[(2 * (1 % NM) + 1 / NM) * 64 + lane];
      if constexpr (DENSE) {
        // keys outside [klo, kvalid) weigh nothing; key of element v:
        // 16 (v/8) + 8 half + v%8
        if (klo > 0 || kvalid < 32) {
          const int lo = klo - 8 * half, hi = kvalid - 8 * half;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int kv = 16 * (v >> 3) + (v & 7);
            if (kv < lo || kv >= hi) sx[v] = -__builtin_huge_valf();
          }
        }
      } else if (VE == 0 && kvalid < 32) {
        const int kk = kvalid - 4 * half;  // key of element v: 8 (v/4) + 4 half + v%4
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (8 * (v >> 2) + (v & 3) >= kk) sx[v] = -__builtin_huge_valf();
      }
      // row max as a tree of depth three (the scores are finite or -inf)
      auto max3 = [](float a, float b, float c) __attribute__((always_inline)) {
        return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
      };
      const float m0 = max3(sx[0], sx[1], sx[2]), m1 = max3(sx[3], sx[4], sx[5]);
      const float m2 = max3(sx[6], sx[7], sx[8]), m3 = max3(sx[9], sx[10], sx[11]);
      float mx;
      if constexpr (VE == 12) {
        mx = __builtin_elementwise_maximum(max3(m0, m1, m2), m3);
      } else {
        const float m4 = max3(sx[12], sx[13], sx[14]);
        mx = __builtin_elementwise_maximum(max3(m0, m1, m2), max3(m3, m4, sx[15]));
      }
      // each lane holds half of its query's keys: a lane whose own maximum
      // clears the threshold starts the (rare) exchange of the two halves
      if (__builtin_amdgcn_ballot_w64(mx * scale_log2 > mlazy)) {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        const float mnew = __builtin_elementwise_maximum(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * scale_log2;
        const bool need = mnew > mlazy;
        const float alpha = need ? __builtin_amdgcn_exp2f(mref - mnew) : 1.0f;
        lsum *= alpha;
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[m][v] *= alpha;
        mref = need ? mnew : mref;
        mlazy = mref + kLazy;
      }
      // first half of the weights (keys of the first 16-key chunk), then the
      // PV MFMAs of that chunk with the second half's exp beside them, then
      // those of the second chunk with the row sum beside them
      bf16x2 pr[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sx[2 * e], scale_log2, -mref));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sx[2 * e + 1], scale_log2, -mref));
        pr[e][0] = (__bf16)p0;
        pr[e][1] = (__bf16)p1;
      }
      const bf16x8 pk0 = __builtin_shufflevector(__builtin_shufflevector(pr[0], pr[1], 0, 1, 2, 3),
                                                 __builtin_shufflevector(pr[2], pr[3], 0, 1, 2, 3), 0, 1, 2, 3, 4,
                                                 5, 6, 7);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int i = 0; i < NM; ++i) {
        if (i + 2 < 2 * NM) vr[(i + 2) % 3] = vl[(2 * ((i + 2) % NM) + (i + 2) / NM) * 64 + lane];
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vr[i % 3], pk0, acc[i], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int e = 4 + i * 4 / NM; e < 4 + (i + 1) * 4 / NM; ++e) {
          if (e < NP) {
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sx[2 * e], scale_log2, -mref));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sx[2 * e + 1], scale_log2, -mref));
            pr[e][0] = (__bf16)p0;
            pr[e][1] = (__bf16)p1;
          } else {
            pr[e][0] = (__bf16)0.f;  // padding keys weigh nothing
            pr[e][1] = (__bf16)0.f;
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      const bf16x8 pk1 = __builtin_shufflevector(__builtin_shufflevector(pr[4], pr[5], 0, 1, 2, 3),
                                                 __builtin_shufflevector(pr[6], pr[7], 0, 1, 2, 3), 0, 1, 2, 3, 4,
                                                 5, 6, 7);
#pragma unroll
      for (int i = NM; i < 2 * NM; ++i) {
        const int m = i - NM;
        if (i + 2 < 2 * NM) vr[(i + 2) % 3] = vl[(2 * ((i + 2) % NM) + (i + 2) / NM) * 64 + lane];
        acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vr[i % 3], pk1, acc[m], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int e = (i - NM) * 8 / NM; e < (i - NM + 1) * 8 / NM; ++e)
          if (e < NP) lsum = __builtin_amdgcn_fdot2_f32_bf16(pr[e], kOnes2, lsum, false);
        // keeps the row-sum terms beside this MFMA: without it the compiler
        // sinks the whole chain of dependent dot2s past the end of the step
        asm volatile("" : "+v"(lsum));
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_setprio(0);
    };

    // Dense streaming: the stage's copies gather each lane's 16 bytes from the
    // block holding its key (K rows in dense_key_of_row order, V in 8-key
    // groups); wave w copies the chunks CPW w .. CPW w + CPW - 1 of the stage,
    // all in one of its two subtiles.  Advances k by the stage's two subtiles.
    auto dissue = [&](DCursor& k, int slot) __attribute__((always_inline)) {
      constexpr int CPS = D / 16;  // 1 KB chunks per subtile and tensor
      const int t0 = wave * CPW;
      const int sg = t0 / CPS;     // this wave's subtile of the stage (uniform)
      int blkA = 0, kbA = 0, b = 32, blkB = 0;
      bool valid = false;
      auto grab = [&]() __attribute__((always_inline)) {
        valid = k.pos < ucnt;
        blkA = k.word & 0xFFF;
        kbA = k.kb;
        b = k.n - k.kb;
        blkB = b < 32 ? (__builtin_amdgcn_readfirstlane((int)k.ae) & 0xFFF) : blkA;
      };
      if (sg == 0) grab();
      dcursor_next(k, ulist, ublkn, ucnt);
      if (sg == 1) grab();
      dcursor_next(k, ulist, ublkn, ucnt);
      if (!valid) {  // past the stream's end: any in-bounds tile (never computed)
        blkA = 0;
        kbA = 0;
        b = 32;
        blkB = 0;
      }
      const int r = lane & 31, h = lane >> 5;
      const int key = dense_key_of_row(r);
      const bool kin_b = key >= b;
      const int kk = kin_b ? key - b : kbA + key;
      const size_t ksrc = head_off + (size_t)(kin_b ? blkB : blkA) * g.P * D + (size_t)(kk >> 5) * SUB +
                          (size_t)((kk & 31) + 32 * h) * 8;
#pragma unroll
      for (int c = 0; c < CPW; ++c) {
        const int ch = (t0 + c) % CPS;  // K channel chunk; V chunk 2 m + kc
        const uint32_t kd = __builtin_amdgcn_readfirstlane(ring_lds + (uint32_t)(slot * 4 * SUB + sg * SUB + ch * 512) * 2u);
        const uint32_t vd = kd + 2 * SUB * 2;
        const int k8 = 16 * (ch & 1) + 8 * h;  // first of the lane's eight V keys
        const bool vin_b = k8 >= b;
        const int vk = vin_b ? k8 - b : kbA + k8;
        const size_t vsrc = head_off + (size_t)(vin_b ? blkB : blkA) * g.P * D + (size_t)(vk >> 5) * SUB +
                            (size_t)(((ch >> 1) * 2 + ((vk >> 4) & 1)) * 64 + ((vk >> 3) & 1) * 32 + r) * 8;
        const char* kg = reinterpret_cast<const char*>(kpack + ksrc) + ch * 1024;
        const char* vg = reinterpret_cast<const char*>(vpack + vsrc);
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(kg), "s"(kd) : "memory", "m0");
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(vg), "s"(vd) : "memory", "m0");
      }
    };

    // ---- stage ring of four slots: stage s is computed from slot s % 4
    // while stages s+1 and s+2 are in flight, and stage s+3 is issued at its
    // end; one barrier per stage ----
    // Every wave walks the stages it computes (cc); the copying waves also
    // walk the stages they copy (kc), three ahead.
    const bool copier = wave < kCopyWaves;
    int si = 0;      // stage computed next
    int issued = 0;  // stages this copying wave has issued
    bool did_prev = true;  // no LDS reads of this unit are outstanding yet
    // own copies of stage si have landed (those of the next two may still
    // fly); a wave that skipped the previous stage may still have reads of
    // the slot about to be refilled outstanding
    auto stage_wait = [&]() __attribute__((always_inline)) {
      if (copier) {
        const int fly = issued - si - 1;
        if (__builtin_expect(fly >= 2 && did_prev, 1)) {
          __builtin_amdgcn_s_waitcnt(vm_wait_imm(2 * PER));
        } else if (fly >= 2) {
          if (did_prev) __builtin_amdgcn_s_waitcnt(vm_wait_imm(2 * PER));
          else __builtin_amdgcn_s_waitcnt(vm_wait_imm(2 * PER) & ~(15 << 8));
        } else if (fly == 1) {
          if (did_prev) __builtin_amdgcn_s_waitcnt(vm_wait_imm(PER));
          else __builtin_amdgcn_s_waitcnt(vm_wait_imm(PER) & ~(15 << 8));
        } else {
          if (did_prev) __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
          else __builtin_amdgcn_s_waitcnt(vm_wait_imm(0) & ~(15 << 8));
        }
      } else if (!did_prev) {
        __builtin_amdgcn_s_waitcnt(vm_wait_imm(0) & ~(15 << 8));
      }
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };
    using any_t = std::integral_constant<int, 0>;
    if constexpr (!DENSE) {
      Cursor cc = cursor_start(ulist, ublkn, ucnt);
      Cursor kc = cc;
      if (copier) {
        for (int p = 0; p < 3 && kc.pos < ucnt; ++p) {
          issue(kc, issued & 3);
          ++issued;
          cursor_next(kc, ulist, ublkn, ucnt);
        }
      }
      while (cc.pos < ucnt) {
        stage_wait();
        did_prev = active && ((cc.word >> (12 + my_row)) & 1);
        if (did_prev) {
          const int kb = (si & 3) * 4 * SUB;
          using k24_t = std::integral_constant<int, 12>;
          // the stage's first subtile, then its second through the same code,
          // unless the second holds 24 keys (the last subtile of a 120-token
          // block), which has a step of its own
          const int nk = cc.n - 32 * cc.s0;
          int kx = kb, kv = min(32, nk), rest = nk - 32;
          for (;;) {
            step(any_t{}, 0, kv, kx, kx + 2 * SUB);
            if (rest <= 0) break;
            if (rest == 24) {
              step(k24_t{}, 0, 24, kb + SUB, kb + 3 * SUB);
              break;
            }
            kx = kb + SUB;
            kv = min(32, rest);
            rest = 0;
          }
        }
        // stage s+3 goes into the slot of stage s-1, which every wave left
        // before the barrier above
        if (copier && kc.pos < ucnt) {
          issue(kc, issued & 3);
          ++issued;
          cursor_next(kc, ulist, ublkn, ucnt);
        }
        cursor_next(cc, ulist, ublkn, ucnt);
        ++si;
      }
    } else {
      DCursor cc = dcursor_start(ulist, ublkn, ucnt);
      DCursor kc = cc;
      if (copier) {
        for (int p = 0; p < 3 && kc.pos < ucnt; ++p) {
          dissue(kc, issued & 3);
          ++issued;
        }
      }
      while (cc.pos < ucnt) {
        stage_wait();
        const int kb = (si & 3) * 4 * SUB;
        did_prev = false;
        // the stage's two subtiles through one copy of the step: this row's
        // keys of each are the part of entry pos (keys [0, b)) and of entry
        // pos + 1 (keys [b, 32)) that the row keeps
#pragma unroll 1
        for (int sg = 0; sg < 2; ++sg) {
          if (active && cc.pos < ucnt) {
            const int b = cc.n - cc.kb;
            const bool keep_a = (cc.word >> (12 + my_row)) & 1;
            int lo = 0, hi = keep_a ? 32 : 0;
            if (b < 32) {
              const bool keep_b = (__builtin_amdgcn_readfirstlane((int)cc.ae) >> (12 + my_row)) & 1;
              lo = keep_a ? 0 : b;
              hi = keep_b ? 32 : (keep_a ? b : 0);
            }
            if (lo < hi) {
              step(any_t{}, lo, hi, kb + sg * SUB, kb + (2 + sg) * SUB);
              did_prev = true;
            }
          }
          dcursor_next(cc, ulist, ublkn, ucnt);
        }
        if (copier && kc.pos < ucnt) {
          dissue(kc, issued & 3);
          ++issued;
        }
        ++si;
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
    __syncthreads();  // s_unit, the ring and ulist are reused by the next unit
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
  __shared__ uint8_t seen[kMaxBlocks];
  const int row = blockIdx.x;
  const int bh = row / g.nblk;
  const int i = row - bh * g.nblk;
  if (!head_active(g, bh)) return;  // another scheme's head (whole workgroup)
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
  for (int t = threadIdx.x; t < g.nblk; t += kF32Threads) seen[t] = 0;
  __syncthreads();
  for (long long kb = lo; kb < hi; ++kb) {
    const int j = col_idx[kb];
    if (j < 0 || j >= g.nblk) continue;
    // a row is a set of blocks: a repeated id is skipped
    const bool dup = seen[j] != 0;
    __syncthreads();
    if (threadIdx.x == 0) seen[j] = 1;
    __syncthreads();
    if (dup) continue;
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
                              void* o, int* counter, bool counter_cleared, int num_cus, hipStream_t s) {
  if (g.R == 0) return hipSuccess;
  const UnitMap um = unit_map(g);
  const int U = g.BH * um.per_head;
  if (!counter_cleared) {
    counter_reset_kernel<<<1, 1, 0, s>>>(counter);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // When the units would leave a last round less than half full (as for a
  // small layer of a few units per CU), the last round's units go out as
  // twice as many half units: Ufull whole units, then 2 (U - Ufull) halves.
  int Ufull = U;
  if (num_cus > 0) {
    const int rem = U % num_cus;
    if (rem > 0 && 2 * rem <= num_cus) Ufull = U - rem;
  }
  const int ids = Ufull + 2 * (U - Ufull);
  int grid = num_cus;  // one 12-wave workgroup per CU (LDS-limited)
  if (grid > ids) grid = ids;
  if (grid < 1) grid = 1;
  const float scale_log2 = scale * 1.4426950408889634f;
#define SPADE_BSATTN(DD, DN)                                                                                  \
  bsattn_bf16_kernel<DD, DN><<<grid, kThreads, 0, s>>>(g, (const uint16_t*)qpack, (const uint16_t*)kpack,           \
                                                     (const uint16_t*)vpack, row_ptr, col_idx, col_capacity,      \
                                                     scale_log2, (uint16_t*)o, counter, ids, Ufull)
  if (g.d == 128) {
    if (g.dense) SPADE_BSATTN(128, true);
    else SPADE_BSATTN(128, false);
  } else {
    if (g.dense) SPADE_BSATTN(64, true);
    else SPADE_BSATTN(64, false);
  }
#undef SPADE_BSATTN
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
