// spade_estimate_select_static: the estimate + select path with its scratch in
// a static device array instead of a caller's workspace, for callers that
// cannot allocate device memory.  The kernels are those of
// spade_estimate_select; only the source of the scratch differs.
#include <mutex>

#include "spade_internal.h"

// The selection scratch of one call (per-row counts, row bitmasks, scan chunk
// sums).  Each device holds its own copy, at its own address,
// from module load until the process ends.  In host code this name is only a
// stand-in for the symbol: its device address comes from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[SPADE_STATIC_SCRATCH_BYTES];

namespace spade {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // per device, filled on first use

// Device address of the current device's copy of `scratch`.
hipError_t scratch_address(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace
}  // namespace spade

extern "C" spade_status spade_estimate_select_static(const spade_problem* p, const float* q_mean,
                                                     const float* k_mean, const spade_budget* budget,
                                                     int32_t* row_ptr, int32_t* col_idx,
                                                     int64_t col_capacity, void* stream) {
  return spade::estimate_select_entry(p, q_mean, k_mean, budget, row_ptr, col_idx, col_capacity, nullptr,
                                      SPADE_STATIC_SCRATCH_BYTES, spade::scratch_address, (hipStream_t)stream);
}
