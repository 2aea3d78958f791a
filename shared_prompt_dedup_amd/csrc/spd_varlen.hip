// Variable-length attention parameters (How Prompt Deduplication Works --
// "Flash Attention Integration"): cu_seqlens for varlen attention kernels,
// either read off a block-diagonal [total_q, total_kv] mask or taken from a
// plan (the two attention calls of Phase 2, "Split Attention Optimization").
//
// Mask conversion, three launches (each reads what the previous one wrote):
//   k_row_extent    one wave per row: first visible key, one past the last;
//   k_mask_owner    one block, rows from the end: the block a row belongs to is
//                   named by the first key of the nearest row at or after it
//                   that sees any key (a suffix scan with "leftmost non-empty",
//                   an associative operator);
//   k_mask_blocks   one block, rows in order: a block starts where that name
//                   changes; exclusive scan of the starts gives the indices;
//   k_mask_check    one thread per row: rows whose keys leave their block are
//                   counted, and each block's lengths feed the maxima.
#include <algorithm>
#include <climits>

#include "spd_internal.h"

namespace spd {
namespace {

constexpr int kScan = 1024;

__device__ inline int wave_max(int v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = max(v, __shfl_xor(v, off, 64));
  return v;
}

__device__ inline int wave_min(int v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = min(v, __shfl_xor(v, off, 64));
  return v;
}

// A key is visible when any byte of its esz-byte element is non-zero.
__global__ void __launch_bounds__(256) k_row_extent(const unsigned char *__restrict__ mask, int64_t Tq,
                                                    int row_bytes, int esz, int32_t *__restrict__ first,
                                                    int32_t *__restrict__ last) {
  const int lane = __lane_id();
  const int64_t nwaves = int64_t(gridDim.x) * 4;
  for (int64_t r = int64_t(blockIdx.x) * 4 + threadIdx.x / 64; r < Tq; r += nwaves) {
    const unsigned char *row = mask + r * int64_t(row_bytes);
    int lo = INT_MAX, hi = -1;
    for (int c = lane; c < row_bytes; c += 64) {
      if (row[c]) {
        lo = min(lo, c);
        hi = c;
      }
    }
    lo = wave_min(lo);
    hi = wave_max(hi);
    if (lane == 0) {
      first[r] = hi < 0 ? INT_MAX : lo / esz;
      last[r] = hi < 0 ? 0 : hi / esz + 1;
    }
  }
}

__global__ void __launch_bounds__(kScan) k_mask_owner(int Tq, const int32_t *__restrict__ first,
                                                      int32_t *__restrict__ owner) {
  __shared__ int lds[kScan / 64];
  const int lane = __lane_id(), wid = threadIdx.x / 64;
  // leftmost(a, b) = a unless a is empty (INT_MAX), else b
  int carry = INT_MAX;
  for (int c0 = (Tq - 1) / kScan * kScan; c0 >= 0; c0 -= kScan) {
    const int r = c0 + threadIdx.x;
    int v = r < Tq ? first[r] : INT_MAX;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int n = __shfl_down(v, off, 64);
      if (lane + off < 64 && v == INT_MAX) v = n;
    }
    __syncthreads();
    if (lane == 0) lds[wid] = v;
    __syncthreads();
    int after = carry, all = carry;
    for (int w = kScan / 64 - 1; w >= 0; --w) {
      if (lds[w] != INT_MAX) all = lds[w];
      if (w == wid + 1) after = all;
    }
    if (wid == kScan / 64 - 1) after = carry;
    if (r < Tq) owner[r] = v != INT_MAX ? v : after;
    carry = all;
  }
}

__global__ void __launch_bounds__(kScan) k_mask_blocks(int Tq, const int32_t *__restrict__ owner,
                                                       const int32_t *__restrict__ last, int32_t *__restrict__ cu_q,
                                                       int32_t *__restrict__ cu_k, int32_t *__restrict__ stats) {
  __shared__ int lds[kScan / 64];
  int base = 0, far = 0;
  for (int c0 = 0; c0 < Tq; c0 += kScan) {
    const int r = c0 + threadIdx.x;
    const int o = r < Tq ? owner[r] : INT_MAX;
    const bool start = o != INT_MAX && (r == 0 || owner[r - 1] != o);
    if (r < Tq) far = max(far, last[r]);
    int total;
    const int idx = base + block_exclusive_scan(start ? 1 : 0, lds, total);
    if (start) {
      cu_q[idx] = r;
      cu_k[idx] = o;
    }
    base += total;
  }
  __syncthreads();
  far = wave_max(far);
  if (__lane_id() == 0) lds[threadIdx.x / 64] = far;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 0; w < kScan / 64; ++w) far = max(far, lds[w]);
    const int n = base;
    if (n > 0) {
      cu_q[n] = Tq;
      cu_k[n] = far;
    } else {
      cu_q[0] = 0;
      cu_k[0] = 0;
    }
    stats[0] = n;
    stats[1] = 0;
    stats[2] = 0;
    stats[3] = 0;
  }
}

__global__ void __launch_bounds__(256) k_mask_check(int Tq, const int32_t *__restrict__ first,
                                                    const int32_t *__restrict__ last,
                                                    const int32_t *__restrict__ cu_q, const int32_t *__restrict__ cu_k,
                                                    int32_t *__restrict__ stats) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  const int n = stats[0];
  if (r >= Tq || n == 0) return;
  int lo = 0, hi = n - 1;          // block i with cu_q[i] <= r < cu_q[i + 1]
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (cu_q[mid] <= r) lo = mid;
    else hi = mid - 1;
  }
  const int i = lo;
  if (cu_q[i] == r) {
    atomicMax(&stats[1], cu_q[i + 1] - cu_q[i]);
    atomicMax(&stats[2], cu_k[i + 1] - cu_k[i]);
  }
  if (first[r] != INT_MAX && (first[r] != cu_k[i] || last[r] > cu_k[i + 1])) atomicAdd(&stats[3], 1);
}

// Exclusive scans of a plan's segment lengths: prompts [G], responses [B] and
// each sample's prompt + response [B]; maxima into maxes[0..2].
__global__ void __launch_bounds__(kScan) k_plan_varlen(int B, spd_plan plan, int32_t *__restrict__ cu_prompt,
                                                       int32_t *__restrict__ cu_q, int32_t *__restrict__ cu_k,
                                                       int32_t *__restrict__ maxes) {
  __shared__ int lds[kScan / 64];
  const int G = plan.counts[0];
  int bp = 0, bq = 0, bk = 0, mp = 0, mq = 0, mk = 0;
  for (int c0 = 0; c0 < B; c0 += kScan) {
    const int i = c0 + threadIdx.x;
    const int pl = i < G ? plan.prompt_len[i] : 0;
    const int rl = i < B ? plan.resp_len[i] : 0;
    const int kl = i < B ? plan.prompt_len[plan.group_of[i]] + rl : 0;
    mp = max(mp, pl);
    mq = max(mq, rl);
    mk = max(mk, kl);
    int tp, tq, tk;
    const int ep = block_exclusive_scan(pl, lds, tp);
    const int eq = block_exclusive_scan(rl, lds, tq);
    const int ek = block_exclusive_scan(kl, lds, tk);
    if (i < G) cu_prompt[i] = bp + ep;
    if (i < B) {
      cu_q[i] = bq + eq;
      cu_k[i] = bk + ek;
    }
    bp += tp;
    bq += tq;
    bk += tk;
  }
  __syncthreads();
  mp = wave_max(mp);
  mq = wave_max(mq);
  mk = wave_max(mk);
  __shared__ int red[3][kScan / 64];
  if (__lane_id() == 0) {
    red[0][threadIdx.x / 64] = mp;
    red[1][threadIdx.x / 64] = mq;
    red[2][threadIdx.x / 64] = mk;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 0; w < kScan / 64; ++w) {
      mp = max(mp, red[0][w]);
      mq = max(mq, red[1][w]);
      mk = max(mk, red[2][w]);
    }
    cu_prompt[G] = bp;
    cu_q[B] = bq;
    cu_k[B] = bk;
    maxes[0] = mp;
    maxes[1] = mq;
    maxes[2] = mk;
  }
}

}  // namespace
}  // namespace spd

using namespace spd;

extern "C" size_t spd_mask_varlen_workspace_bytes(int64_t total_q) {
  if (total_q < 1) return 0;
  return 3 * round_up(size_t(total_q) * 4, 256);
}

extern "C" spd_status spd_mask_to_varlen(const void *mask, int32_t mask_elem_bytes, int64_t total_q,
                                         int64_t total_kv, int32_t *cu_seqlens_q, int32_t *cu_seqlens_k,
                                         int32_t *stats, void *workspace, size_t workspace_bytes, void *stream) {
  if (!mask || !cu_seqlens_q || !cu_seqlens_k || !stats || total_q < 1 || total_kv < 1) return SPD_ERR_INVALID_ARG;
  if (mask_elem_bytes != 1 && mask_elem_bytes != 2 && mask_elem_bytes != 4 && mask_elem_bytes != 8)
    return SPD_ERR_INVALID_ARG;
  if (total_q >= INT_MAX || total_kv * mask_elem_bytes >= INT_MAX) return SPD_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < spd_mask_varlen_workspace_bytes(total_q)) return SPD_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  char *ws = static_cast<char *>(workspace);
  const size_t part = round_up(size_t(total_q) * 4, 256);
  int32_t *first = reinterpret_cast<int32_t *>(ws);
  int32_t *last = reinterpret_cast<int32_t *>(ws + part);
  int32_t *owner = reinterpret_cast<int32_t *>(ws + 2 * part);
  const int Tq = int(total_q);
  prof_start(SPD_K_MASK_VARLEN, st);
  const int64_t waves_grid = std::min<int64_t>((total_q + 3) / 4, int64_t(device_cu_count()) * 16);
  hipLaunchKernelGGL(k_row_extent, dim3(unsigned(std::max<int64_t>(1, waves_grid))), dim3(256), 0, st,
                     static_cast<const unsigned char *>(mask), total_q, int(total_kv * mask_elem_bytes),
                     int(mask_elem_bytes), first, last);
  SPD_LAUNCH_CHECK();
  hipLaunchKernelGGL(k_mask_owner, dim3(1), dim3(kScan), 0, st, Tq, first, owner);
  SPD_LAUNCH_CHECK();
  hipLaunchKernelGGL(k_mask_blocks, dim3(1), dim3(kScan), 0, st, Tq, owner, last, cu_seqlens_q, cu_seqlens_k, stats);
  SPD_LAUNCH_CHECK();
  hipLaunchKernelGGL(k_mask_check, dim3((Tq + 255) / 256), dim3(256), 0, st, Tq, first, last, cu_seqlens_q,
                     cu_seqlens_k, stats);
  SPD_LAUNCH_CHECK();
  prof_stop(SPD_K_MASK_VARLEN, st);
  return SPD_OK;
}

extern "C" spd_status spd_varlen_params(const spd_plan *plan, int32_t *cu_seqlens_prompt, int32_t *cu_seqlens_q,
                                        int32_t *cu_seqlens_k, int32_t *max_seqlens, void *stream) {
  SPD_TRY(validate_plan(plan));
  if (!cu_seqlens_prompt || !cu_seqlens_q || !cu_seqlens_k || !max_seqlens) return SPD_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(k_plan_varlen, dim3(1), dim3(kScan), 0, st, int(plan->B), *plan, cu_seqlens_prompt,
                     cu_seqlens_q, cu_seqlens_k, max_seqlens);
  SPD_LAUNCH_CHECK();
  return SPD_OK;
}
