// Variable-length attention parameters (How Prompt Deduplication Works --
// "Flash Attention Integration"): cu_seqlens for varlen attention kernels,
// either read off a block-diagonal [total_q, total_kv] mask or taken from a
// plan (the two attention calls of Phase 2, "Split Attention Optimization").
//
// Mask conversion, two launches:
//   k_row_extent    one wave per row: first visible key, one past the last
//                   (16 bytes per lane when rows are 16-byte multiples);
//   k_mask_scan     one block, three passes: rows from the end, the block a
//                   row belongs to is named by the first key of the nearest row
//                   at or after it that sees any key (a suffix scan with
//                   "leftmost non-empty", an associative operator); rows in
//                   order, a block starts where that name changes and an
//                   exclusive scan of the starts numbers them; then rows whose
//                   keys leave their block are counted and each block's
//                   lengths feed the maxima.
#include <algorithm>
#include <climits>

#include "spd_internal.h"

namespace spd {
namespace {

constexpr int kScan = 1024;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

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

// A key is visible when any byte of its esz-byte element is non-zero.  Rows
// whose byte length is a multiple of 16 are read 16 bytes per lane.
__global__ void __launch_bounds__(256) k_row_extent16(const u32x4 *__restrict__ mask, int64_t Tq, int row_vecs,
                                                      int esz, int32_t *__restrict__ first,
                                                      int32_t *__restrict__ last) {
  const int lane = __lane_id();
  const int64_t nwaves = int64_t(gridDim.x) * 4;
  for (int64_t r = int64_t(blockIdx.x) * 4 + threadIdx.x / 64; r < Tq; r += nwaves) {
    const u32x4 *row = mask + r * int64_t(row_vecs);
    int lo = INT_MAX, hi = -1;
#pragma unroll 4
    for (int c = lane; c < row_vecs; c += 64) {
      const u32x4 v = __builtin_nontemporal_load(row + c);
      const unsigned w[4] = {v[0], v[1], v[2], v[3]};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (w[j]) {     // little endian: byte k of the word is bits 8k .. 8k + 7
          const int b0 = 16 * c + 4 * j;
          lo = min(lo, b0 + (__builtin_ctz(w[j]) >> 3));
          hi = max(hi, b0 + ((31 - __builtin_clz(w[j])) >> 3));
        }
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

// The three passes below run in one block (k_mask_scan), each reading what
// the previous one wrote to global memory after a block barrier.  Each
// thread takes kItems consecutive rows: one block-wide scan per
// kScan * kItems rows.
constexpr int kItems = 16;

typedef int i32x4 __attribute__((ext_vector_type(4)));

// A thread's kItems consecutive values from row r0 on (16-byte loads when all
// are in range; the arrays start 256-byte aligned and r0 is a multiple of 16).
__device__ inline void load_items(const int32_t *__restrict__ a, int r0, int Tq, int fill, int (&v)[kItems]) {
  if (r0 + kItems <= Tq) {
#pragma unroll
    for (int q = 0; q < kItems / 4; ++q) {
      const i32x4 x = *reinterpret_cast<const i32x4 *>(a + r0 + 4 * q);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * q + e] = x[e];
    }
  } else {
#pragma unroll
    for (int j = 0; j < kItems; ++j) v[j] = r0 + j < Tq ? a[r0 + j] : fill;
  }
}

__device__ inline void store_items(int32_t *__restrict__ a, int r0, int Tq, const int (&v)[kItems]) {
  if (r0 + kItems <= Tq) {
#pragma unroll
    for (int q = 0; q < kItems / 4; ++q) {
      const i32x4 x = {v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
      *reinterpret_cast<i32x4 *>(a + r0 + 4 * q) = x;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kItems; ++j)
      if (r0 + j < Tq) a[r0 + j] = v[j];
  }
}

__device__ inline int block_max(int v, int *lds) {
  v = wave_max(v);
  __syncthreads();
  if (__lane_id() == 0) lds[threadIdx.x / 64] = v;
  __syncthreads();
  int m = lds[0];
  for (int w = 1; w < kScan / 64; ++w) m = max(m, lds[w]);
  return m;
}

// owner[r]: first visible key of the nearest row at or after r that sees any
// key (INT_MAX if none): a suffix scan with leftmost(a, b) = a unless a is
// empty, else b.
__device__ void mask_owner_pass(int Tq, const int32_t *__restrict__ first, int32_t *__restrict__ owner, int *lds) {
  const int lane = __lane_id(), wid = threadIdx.x / 64;
  constexpr int span = kScan * kItems;
  int carry = INT_MAX;
  for (int c0 = (Tq - 1) / span * span; c0 >= 0; c0 -= span) {
    const int r0 = c0 + threadIdx.x * kItems;
    int vals[kItems];
    load_items(first, r0, Tq, INT_MAX, vals);
    int agg = INT_MAX;
#pragma unroll
    for (int j = kItems - 1; j >= 0; --j)
      if (vals[j] != INT_MAX) agg = vals[j];
    int v = agg;          // leftmost non-empty of lanes lane .. 63
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int n = __shfl_down(v, off, 64);
      if (lane + off < 64 && v == INT_MAX) v = n;
    }
    int later = __shfl_down(v, 1, 64);     // of lanes lane + 1 .. 63
    if (lane == 63) later = INT_MAX;
    __syncthreads();
    if (lane == 0) lds[wid] = v;
    __syncthreads();
    int after = carry, all = carry;
    for (int w = kScan / 64 - 1; w >= 0; --w) {
      if (lds[w] != INT_MAX) all = lds[w];
      if (w == wid + 1) after = all;
    }
    if (wid == kScan / 64 - 1) after = carry;
    int cur = later != INT_MAX ? later : after;
#pragma unroll
    for (int j = kItems - 1; j >= 0; --j) {
      if (vals[j] != INT_MAX) cur = vals[j];
      vals[j] = cur;
    }
    store_items(owner, r0, Tq, vals);
    carry = all;
  }
}

// A block starts where the owner changes; an exclusive scan of the starts
// numbers them.  Returns the block count; cu_q[n], cu_k[n] close the lists.
// owner[r0] of each thread's first row r0 is replaced by the index of r0's
// block (no thread reads it again: a thread reads its own rows and the row
// before them).
__device__ int mask_blocks_pass(int Tq, int32_t *__restrict__ owner, const int32_t *__restrict__ last,
                                int32_t *__restrict__ cu_q, int32_t *__restrict__ cu_k, int *lds) {
  constexpr int span = kScan * kItems;
  int base = 0, far = 0;
  for (int c0 = 0; c0 < Tq; c0 += span) {
    const int r0 = c0 + threadIdx.x * kItems;
    int prev = r0 > 0 && r0 - 1 < Tq ? owner[r0 - 1] : INT_MAX;
    const int prev0 = prev;
    int vals[kItems], lv[kItems];
    load_items(owner, r0, Tq, INT_MAX, vals);
    load_items(last, r0, Tq, 0, lv);
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
      const int r = r0 + j;
      far = max(far, lv[j]);
      cnt += (vals[j] != INT_MAX && (r == 0 || prev != vals[j])) ? 1 : 0;
      prev = vals[j];
    }
    int total;
    int idx = base + block_exclusive_scan(cnt, lds, total);
    prev = prev0;
    if (r0 < Tq) owner[r0] = (vals[0] != INT_MAX && (r0 == 0 || prev0 != vals[0])) ? idx : idx - 1;
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
      const int r = r0 + j;
      if (vals[j] != INT_MAX && (r == 0 || prev != vals[j])) {
        cu_q[idx] = r;
        cu_k[idx] = vals[j];
        ++idx;
      }
      prev = vals[j];
    }
    base += total;
  }
  far = block_max(far, lds);
  if (threadIdx.x == 0) {
    if (base > 0) {
      cu_q[base] = Tq;
      cu_k[base] = far;
    } else {
      cu_q[0] = 0;
      cu_k[0] = 0;
    }
  }
  return base;
}

// Longest blocks, and rows whose visible keys leave their block's key range.
// blk[r0]: index of the block of each thread's first row (mask_blocks_pass).
__device__ void mask_check_pass(int Tq, int n, const int32_t *__restrict__ first, const int32_t *__restrict__ last,
                                const int32_t *__restrict__ blk, const int32_t *__restrict__ cu_q,
                                const int32_t *__restrict__ cu_k, int32_t *__restrict__ stats, int *lds) {
  int mq = 0, mk = 0, bad = 0;
  if (n > 0) {
    for (int r0 = threadIdx.x * kItems; r0 < Tq; r0 += kScan * kItems) {
      int f[kItems], l[kItems];
      load_items(first, r0, Tq, INT_MAX, f);
      load_items(last, r0, Tq, 0, l);
      int i = blk[r0];                     // cu_q[i] <= r0 < cu_q[i + 1]
      int qs = cu_q[i], qe = cu_q[i + 1], ks = cu_k[i], ke = cu_k[i + 1];
#pragma unroll
      for (int j = 0; j < kItems; ++j) {
        const int r = r0 + j;
        if (r < Tq) {
          if (r == qe) {                   // the next block starts here
            ++i;
            qs = qe;
            ks = ke;
            qe = cu_q[i + 1];
            ke = cu_k[i + 1];
          }
          if (r == qs) {
            mq = max(mq, qe - qs);
            mk = max(mk, ke - ks);
          }
          bad += (f[j] != INT_MAX && (f[j] != ks || l[j] > ke)) ? 1 : 0;
        }
      }
    }
  }
  mq = block_max(mq, lds);
  mk = block_max(mk, lds);
  int tot;
  block_exclusive_scan(bad, lds, tot);
  if (threadIdx.x == 0) {
    stats[0] = n;
    stats[1] = mq;
    stats[2] = mk;
    stats[3] = tot;
  }
}

__global__ void __launch_bounds__(kScan) k_mask_scan(int Tq, const int32_t *__restrict__ first,
                                                     const int32_t *__restrict__ last, int32_t *__restrict__ owner,
                                                     int32_t *__restrict__ cu_q, int32_t *__restrict__ cu_k,
                                                     int32_t *__restrict__ stats) {
  __shared__ int lds[kScan / 64];
  mask_owner_pass(Tq, first, owner, lds);
  __syncthreads();
  const int n = mask_blocks_pass(Tq, owner, last, cu_q, cu_k, lds);
  __syncthreads();
  mask_check_pass(Tq, n, first, last, owner, cu_q, cu_k, stats, lds);
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
  if (!aligned16(workspace)) return SPD_ERR_ALIGNMENT;
  hipStream_t st = static_cast<hipStream_t>(stream);
  char *ws = static_cast<char *>(workspace);
  const size_t part = round_up(size_t(total_q) * 4, 256);
  int32_t *first = reinterpret_cast<int32_t *>(ws);
  int32_t *last = reinterpret_cast<int32_t *>(ws + part);
  int32_t *owner = reinterpret_cast<int32_t *>(ws + 2 * part);
  const int Tq = int(total_q);
  prof_start(SPD_K_MASK_VARLEN, st);
  const int64_t waves_grid = std::min<int64_t>((total_q + 3) / 4, int64_t(device_cu_count()) * 16);
  const int64_t row_bytes = total_kv * mask_elem_bytes;
  if (row_bytes % 16 == 0 && aligned16(mask))
    hipLaunchKernelGGL(k_row_extent16, dim3(unsigned(std::max<int64_t>(1, waves_grid))), dim3(256), 0, st,
                       static_cast<const u32x4 *>(mask), total_q, int(row_bytes / 16), int(mask_elem_bytes), first,
                       last);
  else
    hipLaunchKernelGGL(k_row_extent, dim3(unsigned(std::max<int64_t>(1, waves_grid))), dim3(256), 0, st,
                       static_cast<const unsigned char *>(mask), total_q, int(row_bytes), int(mask_elem_bytes), first,
                       last);
  SPD_LAUNCH_CHECK();
  hipLaunchKernelGGL(k_mask_scan, dim3(1), dim3(kScan), 0, st, Tq, first, last, owner, cu_seqlens_q, cu_seqlens_k,
                     stats);
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
