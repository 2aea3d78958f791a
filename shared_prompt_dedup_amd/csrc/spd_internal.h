// Internal helpers shared by the libspd translation units (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "spd.h"

namespace spd {

// Host-side bookkeeping -------------------------------------------------------

void set_last_hip_error(hipError_t e);

// Checks the launch that just happened on the calling thread.
inline spd_status check_launch() {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_last_hip_error(e);
    return SPD_ERR_HIP;
  }
  return SPD_OK;
}

#define SPD_TRY(expr)                     \
  do {                                    \
    spd_status _s = (expr);               \
    if (_s != SPD_OK) return _s;          \
  } while (0)

#define SPD_LAUNCH_CHECK() SPD_TRY(::spd::check_launch())

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Compute units of the current device (cached per device id).
int device_cu_count();

// Kernel timing (see spd_profile_begin in spd.h): no-ops unless a profile is
// active on the calling thread.
void prof_start(int kernel_id, hipStream_t st);
void prof_stop(int kernel_id, hipStream_t st);

// Validates the pointer fields of a plan that every consumer reads.
spd_status validate_plan(const spd_plan *plan);

// Device helpers --------------------------------------------------------------

constexpr int kWave = 64;

__device__ inline int lane_id() { return __lane_id(); }

// Inclusive prefix sum over a 64-lane wave.
__device__ inline int wave_inclusive_scan(int v) {
  const int lane = __lane_id();
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int n = __shfl_up(v, off, 64);
    if (lane >= off) v += n;
  }
  return v;
}

// Exclusive prefix sum over the whole block; `lds` needs blockDim/64 ints.
// Returns the thread's exclusive prefix and writes the block total.
__device__ inline int block_exclusive_scan(int v, int *lds, int &total) {
  const int lane = __lane_id();
  const int wid = threadIdx.x / kWave;
  const int nw = (blockDim.x + kWave - 1) / kWave;
  int inc = wave_inclusive_scan(v);
  __syncthreads();
  if (lane == kWave - 1) lds[wid] = inc;
  __syncthreads();
  int base = 0;
  total = 0;
  for (int w = 0; w < nw; ++w) {
    int s = lds[w];
    if (w < wid) base += s;
    total += s;
  }
  return base + inc - v;
}

}  // namespace spd
