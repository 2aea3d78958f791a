// Grouping, packing, row packing and reconstruction kernels plus their C-ABI
// entry points.  All of this is exact integer / byte work.
//
// How Prompt Deduplication Works:
//   Core Algorithm -- "Finding Prompt Groups", "Creating Deduplicated Batch",
//   "Reconstructing Original Batch"; "Working with Packed/Unpacked Sequences";
//   Phase 1 (prompt detection & deduplication) and Phase 3 (reconstruction).
#include <algorithm>
#include <mutex>
#include <vector>

#include <climits>

#include "spd_internal.h"

namespace spd {

namespace {
thread_local int g_last_hip_error = 0;
}

void set_last_hip_error(hipError_t e) { g_last_hip_error = static_cast<int>(e); }

int device_cu_count() {
  static std::mutex mu;
  static std::vector<int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (dev >= static_cast<int>(cache.size())) cache.resize(dev + 1, 0);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

spd_status validate_plan(const spd_plan *p) {
  if (!p) return SPD_ERR_INVALID_ARG;
  if (p->B < 1 || p->B > 65536 || p->S < 1 || p->P < 0 || p->P > p->S) return SPD_ERR_INVALID_ARG;
  if (p->B * p->S >= (int64_t(1) << 31)) return SPD_ERR_UNSUPPORTED;
  if (!p->group_of || !p->grp_off || !p->grp_idx || !p->rep || !p->prompt_off || !p->prompt_len ||
      !p->resp_off || !p->resp_len || !p->src || !p->dst || !p->seg_start || !p->counts)
    return SPD_ERR_INVALID_ARG;
  return SPD_OK;
}

// ----------------------------------------------------------------------------
// Grouping
// ----------------------------------------------------------------------------

// splitmix64 finalizer (Steele, Lea & Flood, "Fast splittable pseudorandom
// number generators", 2014): a bijective 64-bit mixer.
__device__ inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

typedef long long i64x2 __attribute__((ext_vector_type(2)));

// Prompt tokens hashed by one block of k_hash_rows.
constexpr int kHashChunk = 2048;

__device__ inline uint64_t token_term(int64_t id, int64_t t) {
  return mix64(static_cast<uint64_t>(id) + static_cast<uint64_t>(t + 1) * 0x9E3779B97F4A7C15ull);
}

// A row's hash is an order-dependent function of its P prompt ids: the
// wrapping sum over tokens t of mix64(id_t + (t + 1) * golden-ratio constant).
// It only narrows the candidates; equality is always decided by full
// comparison.  One block per (row, chunk of kHashChunk tokens) writes the
// chunk's part of the sum to part[row * nch + chunk]; a wrapping sum does not
// depend on the order its parts are added in.  VEC: rows start on 16-byte
// boundaries (S even), so token pairs (t, t + 1), t even, load as 16 bytes.
template <bool VEC>
__global__ void __launch_bounds__(256) k_hash_rows(const int64_t *__restrict__ ids, int64_t S, int64_t P, int nch,
                                                    uint64_t *__restrict__ part) {
  const int64_t b = blockIdx.x / nch;
  const int64_t t0 = int64_t(blockIdx.x % nch) * kHashChunk;
  const int64_t t1 = t0 + kHashChunk < P ? t0 + kHashChunk : P;
  const int64_t *row = ids + b * S;
  uint64_t h = 0;
  if (VEC) {
#pragma unroll 4
    for (int64_t t = t0 + 2 * int64_t(threadIdx.x); t < t1; t += 2 * blockDim.x) {
      if (t + 1 < t1) {
        const i64x2 x = *reinterpret_cast<const i64x2 *>(row + t);
        h += token_term(x.x, t) + token_term(x.y, t + 1);
      } else {
        h += token_term(row[t], t);
      }
    }
  } else {
    for (int64_t t = t0 + threadIdx.x; t < t1; t += blockDim.x) h += token_term(row[t], t);
  }
  __shared__ uint64_t wsum[4];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) h += __shfl_xor(h, off, 64);
  if (__lane_id() == 0) wsum[threadIdx.x / 64] = h;
  __syncthreads();
  if (threadIdx.x == 0) part[blockIdx.x] = wsum[0] + wsum[1] + wsum[2] + wsum[3];
}

__device__ inline uint64_t row_hash(const uint64_t *__restrict__ part, int nch, int r) {
  uint64_t h = 0;
  for (int c = 0; c < nch; ++c) h += part[int64_t(r) * nch + c];
  return h;
}

// One block per row b: rep_of[b] = the smallest c <= b whose prompt equals
// row b's.  Candidates are scanned in ascending order in chunks of 256; only
// equal hashes are compared in full (16-byte loads when VEC, as above).
template <bool VEC>
__global__ void __launch_bounds__(256) k_find_rep(const int64_t *__restrict__ ids, int64_t S, int64_t P, int nch,
                                                   const uint64_t *__restrict__ part,
                                                   int32_t *__restrict__ rep_of) {
  const int b = blockIdx.x;
  const uint64_t hb = row_hash(part, nch, b);
  const int64_t *rowb = ids + int64_t(b) * S;
  __shared__ int cand[256];
  for (int c0 = 0; c0 < b; c0 += 256) {
    const int c = c0 + threadIdx.x;
    cand[threadIdx.x] = (c < b && row_hash(part, nch, c) == hb) ? 1 : 0;
    __syncthreads();
    const int n = min(256, b - c0);
    for (int i = 0; i < n; ++i) {
      if (!cand[i]) continue;   // uniform: every thread reads the same flag
      const int64_t *rowc = ids + int64_t(c0 + i) * S;
      int diff = 0;
      if (VEC) {
        const int64_t P2 = P & ~int64_t(1);
#pragma unroll 4
        for (int64_t t = 2 * int64_t(threadIdx.x); t < P2; t += 2 * blockDim.x) {
          const i64x2 x = *reinterpret_cast<const i64x2 *>(rowc + t);
          const i64x2 y = *reinterpret_cast<const i64x2 *>(rowb + t);
          diff |= (x.x != y.x) | (x.y != y.y);
        }
        if ((P & 1) && threadIdx.x == 0) diff |= rowc[P - 1] != rowb[P - 1];
      } else {
        for (int64_t t = threadIdx.x; t < P; t += blockDim.x) diff |= (rowc[t] != rowb[t]);
      }
      if (!__syncthreads_or(diff)) {
        if (threadIdx.x == 0) rep_of[b] = c0 + i;
        return;
      }
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) rep_of[b] = b;
}

// Single block: number groups by first occurrence, build group_of, CSR
// offsets and the member lists (ascending), and counts[0] = G.
constexpr int kFinalThreads = 1024;
__global__ void __launch_bounds__(kFinalThreads) k_finalize_groups(int B, const int32_t *__restrict__ rep_of,
                                                                    int32_t *__restrict__ gid_of,
                                                                    int32_t *__restrict__ fill,
                                                                    spd_plan plan) {
  __shared__ int scan_tmp[kFinalThreads / 64];
  __shared__ int chunk_g[kFinalThreads];
  const int tid = threadIdx.x;
  // A: group ids for first members, in ascending order of the first member.
  int running = 0;
  for (int b0 = 0; b0 < B; b0 += kFinalThreads) {
    const int b = b0 + tid;
    const int is_rep = (b < B && rep_of[b] == b) ? 1 : 0;
    int total = 0;
    const int ex = block_exclusive_scan(is_rep, scan_tmp, total);
    if (is_rep) {
      gid_of[b] = running + ex;
      plan.rep[running + ex] = b;
    }
    running += total;
  }
  const int G = running;
  for (int g = tid; g < B; g += kFinalThreads) fill[g] = 0;
  __syncthreads();
  // B: group of every sample and member counts.
  for (int b = tid; b < B; b += kFinalThreads) {
    const int g = gid_of[rep_of[b]];
    plan.group_of[b] = g;
    atomicAdd(&fill[g], 1);
  }
  __syncthreads();
  // C: CSR offsets.
  int base = 0;
  for (int g0 = 0; g0 < G; g0 += kFinalThreads) {
    const int g = g0 + tid;
    const int c = g < G ? fill[g] : 0;
    int total = 0;
    const int ex = block_exclusive_scan(c, scan_tmp, total);
    if (g < G) plan.grp_off[g] = base + ex;
    base += total;
  }
  if (tid == 0) {
    plan.grp_off[G] = B;
    plan.counts[0] = G;
    plan.counts[4] = 0;    // no shared prefix unless spd_share_prefix finds one
    plan.counts[5] = 0;
  }
  __syncthreads();
  for (int g = tid; g < G; g += kFinalThreads) fill[g] = 0;
  __syncthreads();
  // D: stable placement of members (ascending sample index within a group).
  for (int b0 = 0; b0 < B; b0 += kFinalThreads) {
    const int b = b0 + tid;
    const int n = min(kFinalThreads, B - b0);
    const int g = b < B ? plan.group_of[b] : -1;
    chunk_g[tid] = g;
    __syncthreads();
    int rank = 0, later = 0, slot = -1;
    if (b < B) {
      for (int i = 0; i < n; ++i) {
        if (chunk_g[i] == g) {
          rank += (i < tid);
          later += (i > tid);
        }
      }
      slot = plan.grp_off[g] + fill[g] + rank;
    }
    __syncthreads();   // every thread has read fill[] for this chunk
    if (b < B) {
      plan.grp_idx[slot] = b;
      if (later == 0) fill[g] += rank + 1;
    }
    __syncthreads();
  }
}

// One block per (group slot, chunk of kHashChunk tokens): out[g] = the prompt
// ids of group g's first member; slots g >= G exit.  VEC: S and P even, so
// source and destination rows start on 16-byte boundaries.
template <bool VEC>
__global__ void __launch_bounds__(256) k_unique_prompts(const int64_t *__restrict__ ids, int64_t S, int64_t P,
                                                         int nch, const int32_t *__restrict__ rep,
                                                         const int32_t *__restrict__ counts,
                                                         int64_t *__restrict__ out) {
  const int g = blockIdx.x / nch;
  if (g >= counts[0]) return;
  const int64_t t0 = int64_t(blockIdx.x % nch) * kHashChunk;
  const int64_t t1 = t0 + kHashChunk < P ? t0 + kHashChunk : P;
  const int64_t *row = ids + int64_t(rep[g]) * S;
  int64_t *dst = out + int64_t(g) * P;
  if (VEC) {
    for (int64_t t = t0 + 2 * int64_t(threadIdx.x); t < t1; t += 2 * blockDim.x)
      *reinterpret_cast<i64x2 *>(dst + t) = *reinterpret_cast<const i64x2 *>(row + t);
  } else {
    for (int64_t t = t0 + threadIdx.x; t < t1; t += blockDim.x) dst[t] = row[t];
  }
}

// ----------------------------------------------------------------------------
// Packing
// ----------------------------------------------------------------------------

__device__ inline bool mask_at(const void *mask, int esz, int64_t i) {
  if (esz == 1) return static_cast<const int8_t *>(mask)[i] != 0;
  if (esz == 4) return static_cast<const int32_t *>(mask)[i] != 0;
  return static_cast<const int64_t *>(mask)[i] != 0;
}

// Padded packing (every column kept): segment lengths from the shapes alone.
__global__ void k_seg_lengths_dense(int64_t S, int64_t P, spd_plan plan) {
  const int64_t L0 = plan.counts[4];
  for (int b = threadIdx.x; b < plan.B; b += blockDim.x) {
    const int g = plan.group_of[b];
    plan.resp_len[b] = static_cast<int>(S - P);
    if (plan.rep[g] == b) plan.prompt_len[g] = static_cast<int>(P - L0);
    if (plan.rep[0] == b) plan.counts[5] = static_cast<int>(L0);
  }
}

// Unpadded packing works on chunks of kPackChunk columns of each sample's row,
// one block per (sample, chunk), each thread kPackPer consecutive columns.  A
// row's columns fall in three parts: the shared prefix [0, L0), the prompt
// [L0, P) and the response [P, S).  k_chunk_counts counts the kept columns
// of every (sample, chunk, part); k_chunk_bases turns them into exclusive
// scans over each (sample, part)'s chunks and the part totals into segment
// lengths; k_scatter_chunks then gives a kept column the rank of its chunk's
// base plus its rank inside the chunk.
constexpr int kPackChunk = 1024;
constexpr int kPackPer = kPackChunk / 256;

__device__ inline int pack_part(int64_t t, int64_t L0, int64_t P) { return t < L0 ? 0 : (t < P ? 1 : 2); }

// Sums of three per-thread values over a 256-thread block (red: 12 ints).
__device__ inline void block_sum3(int &v0, int &v1, int &v2, int *red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    v0 += __shfl_xor(v0, off, 64);
    v1 += __shfl_xor(v1, off, 64);
    v2 += __shfl_xor(v2, off, 64);
  }
  const int w = threadIdx.x / 64;
  __syncthreads();
  if (__lane_id() == 0) {
    red[3 * w] = v0;
    red[3 * w + 1] = v1;
    red[3 * w + 2] = v2;
  }
  __syncthreads();
  v0 = red[0] + red[3] + red[6] + red[9];
  v1 = red[1] + red[4] + red[7] + red[10];
  v2 = red[2] + red[5] + red[8] + red[11];
}

// cnt[(b * nch + c) * 3 + part]: kept columns of sample b's own row in chunk c.
__global__ void __launch_bounds__(256) k_chunk_counts(int64_t S, int64_t P, const void *mask, int esz, int nch,
                                                       spd_plan plan, int32_t *__restrict__ cnt) {
  __shared__ int red[12];
  const int b = blockIdx.x / nch, c = blockIdx.x % nch;
  const int64_t L0 = plan.counts[4];
  const int64_t t0 = int64_t(c) * kPackChunk + int64_t(threadIdx.x) * kPackPer;
  int v0 = 0, v1 = 0, v2 = 0;
#pragma unroll
  for (int i = 0; i < kPackPer; ++i) {
    const int64_t t = t0 + i;
    if (t < S) {
      const int k = mask_at(mask, esz, int64_t(b) * S + t) ? 1 : 0;
      const int part = pack_part(t, L0, P);
      v0 += part == 0 ? k : 0;
      v1 += part == 1 ? k : 0;
      v2 += part == 2 ? k : 0;
    }
  }
  block_sum3(v0, v1, v2, red);
  if (threadIdx.x < 3) cnt[(int64_t(b) * nch + c) * 3 + threadIdx.x] = threadIdx.x == 0 ? v0 : (threadIdx.x == 1 ? v1 : v2);
}

// One wave per (sample, part): cnt becomes the exclusive scan over the
// chunks of that sample's part; the totals give resp_len (every sample),
// prompt_len (a group's first member) and counts[5], the shared prefix's kept
// length (the first group's first member).
__global__ void __launch_bounds__(256) k_chunk_bases(int nch, spd_plan plan, int32_t *__restrict__ cnt) {
  const int pair = blockIdx.x * 4 + threadIdx.x / 64;
  if (pair >= 3 * plan.B) return;
  const int lane = __lane_id();
  const int b = pair / 3, part = pair % 3;
  int32_t *run = cnt + int64_t(b) * nch * 3 + part;
  int total = 0;
  for (int c0 = 0; c0 < nch; c0 += 64) {
    const int c = c0 + lane;
    const int x = c < nch ? run[3 * int64_t(c)] : 0;
    const int inc = wave_inclusive_scan(x);
    if (c < nch) run[3 * int64_t(c)] = total + inc - x;
    total += __shfl(inc, 63, 64);
  }
  if (lane != 0) return;
  if (part == 2) {
    plan.resp_len[b] = total;
  } else if (part == 1) {
    const int g = plan.group_of[b];
    if (plan.rep[g] == b) plan.prompt_len[g] = total;
  } else if (plan.rep[0] == b) {
    plan.counts[5] = total;
  }
}

// Single block: segment order [shared prefix][prompt g][members of g
// ascending]..., exclusive scan of segment lengths -> prompt_off / resp_off,
// counts[1] = T.
__global__ void __launch_bounds__(kFinalThreads) k_seg_offsets(int B, int32_t *__restrict__ seg, spd_plan plan) {
  __shared__ int scan_tmp[kFinalThreads / 64];
  const int G = plan.counts[0];
  const int nseg = G + B;
  for (int g = threadIdx.x; g < G; g += kFinalThreads) seg[plan.grp_off[g] + g] = plan.prompt_len[g];
  for (int i = threadIdx.x; i < B; i += kFinalThreads) {
    const int b = plan.grp_idx[i];
    seg[i + plan.group_of[b] + 1] = plan.resp_len[b];
  }
  __syncthreads();
  int base = plan.counts[5];     // rows of the shared prefix come first
  for (int s0 = 0; s0 < nseg; s0 += kFinalThreads) {
    const int s = s0 + threadIdx.x;
    const int len = s < nseg ? seg[s] : 0;
    int total = 0;
    const int ex = block_exclusive_scan(len, scan_tmp, total);
    __syncthreads();
    if (s < nseg) seg[s] = base + ex;
    base += total;
  }
  __syncthreads();
  for (int g = threadIdx.x; g < G; g += kFinalThreads) plan.prompt_off[g] = seg[plan.grp_off[g] + g];
  for (int i = threadIdx.x; i < B; i += kFinalThreads) {
    const int b = plan.grp_idx[i];
    plan.resp_off[b] = seg[i + plan.group_of[b] + 1];
  }
  if (threadIdx.x == 0) {
    plan.counts[1] = base;
    plan.counts[2] = 0;
    plan.counts[3] = 0;
  }
}

// Unpadded scatter, one block per (sample b, chunk c): dst for every (b, t)
// of the chunk; src, seg_start, dedup ids and positions for the packed rows
// b owns there (its response, its group's prompt when it is the first member,
// the shared prefix when it is the first group's first member).  A part's
// kept-ness comes from the row it is packed from: the prefix from the first
// group's first member, the prompt from the group's first member, the
// response from b.
__global__ void __launch_bounds__(256) k_scatter_chunks(int64_t S, int64_t P, const int64_t *__restrict__ ids,
                                                         const int64_t *__restrict__ pos, const void *mask, int esz,
                                                         int nch, spd_plan plan, const int32_t *__restrict__ cnt,
                                                         int64_t *__restrict__ dids, int64_t *__restrict__ dpos) {
  __shared__ int scan_tmp[4];
  const int b = blockIdx.x / nch, c = blockIdx.x % nch;
  const int g = plan.group_of[b];
  const int from0 = plan.rep[0], from1 = plan.rep[g];
  const int seg1 = plan.prompt_off[g], seg2 = plan.resp_off[b];
  const int64_t L0 = plan.counts[4];
  const int64_t t0 = int64_t(c) * kPackChunk + int64_t(threadIdx.x) * kPackPer;
  unsigned kept = 0;
  int n0 = 0, n1 = 0, n2 = 0;
#pragma unroll
  for (int i = 0; i < kPackPer; ++i) {
    const int64_t t = t0 + i;
    if (t < S) {
      const int part = pack_part(t, L0, P);
      const int from = part == 0 ? from0 : (part == 1 ? from1 : b);
      const int k = mask_at(mask, esz, int64_t(from) * S + t) ? 1 : 0;
      kept |= unsigned(k) << i;
      n0 += part == 0 ? k : 0;
      n1 += part == 1 ? k : 0;
      n2 += part == 2 ? k : 0;
    }
  }
  int tot;
  // rank in the part = the chunk's base in the row the part comes from + kept
  // columns of the part before this one in the chunk
  int r0 = block_exclusive_scan(n0, scan_tmp, tot) + cnt[(int64_t(from0) * nch + c) * 3];
  __syncthreads();
  int r1 = block_exclusive_scan(n1, scan_tmp, tot) + cnt[(int64_t(from1) * nch + c) * 3 + 1];
  __syncthreads();
  int r2 = block_exclusive_scan(n2, scan_tmp, tot) + cnt[(int64_t(b) * nch + c) * 3 + 2];
  int pads = 0;
#pragma unroll
  for (int i = 0; i < kPackPer; ++i) {
    const int64_t t = t0 + i;
    if (t < S) {
      const int part = pack_part(t, L0, P);
      const int64_t cell = int64_t(b) * S + t;
      if ((kept >> i) & 1) {
        const int rank = part == 0 ? r0++ : (part == 1 ? r1++ : r2++);
        const int seg = part == 0 ? 0 : (part == 1 ? seg1 : seg2);
        const int j = seg + rank;
        plan.dst[cell] = j;
        if (b == (part == 0 ? from0 : (part == 1 ? from1 : b))) {
          plan.src[j] = static_cast<int32_t>(cell);
          plan.seg_start[j] = seg;
          dids[j] = ids[cell];
          dpos[j] = pos[cell];
        }
      } else {
        plan.dst[cell] = -1;
        ++pads;
      }
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) pads += __shfl_xor(pads, off, 64);
  if (__lane_id() == 0 && pads) atomicAdd(&plan.counts[2], pads);
}

// Padded format (every column kept): a column's packed row is its offset in
// its segment, so one thread per batch cell, no scan.
__global__ void __launch_bounds__(256) k_scatter_dense(int64_t S, int64_t P, const int64_t *__restrict__ ids,
                                                        const int64_t *__restrict__ pos, const void *mask, int esz,
                                                        spd_plan plan, int64_t *__restrict__ dids,
                                                        int64_t *__restrict__ dpos) {
  const int64_t cells = plan.B * S;
  const int64_t L0 = plan.counts[4];
  int kept_pads = 0;
  for (int64_t c = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; c < cells; c += int64_t(gridDim.x) * blockDim.x) {
    const int b = static_cast<int>(c / S);
    const int64_t t = c - int64_t(b) * S;
    int j, from, seg;
    if (t < L0) {                 // shared prefix: packed from the first group's first sample
      from = plan.rep[0];
      j = static_cast<int>(t);
      seg = 0;
    } else if (t < P) {           // the group's prompt, from its first member
      const int g = plan.group_of[b];
      from = plan.rep[g];
      seg = plan.prompt_off[g];
      j = seg + static_cast<int>(t - L0);
    } else {                      // the sample's own response
      from = b;
      seg = plan.resp_off[b];
      j = seg + static_cast<int>(t - P);
    }
    plan.dst[c] = j;
    if (b == from) {
      plan.src[j] = static_cast<int32_t>(c);
      plan.seg_start[j] = seg;
      dids[j] = ids[c];
      dpos[j] = pos[c];
      if (mask) kept_pads += !mask_at(mask, esz, c);
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) kept_pads += __shfl_xor(kept_pads, off, 64);
  if (__lane_id() == 0 && kept_pads) atomicAdd(&plan.counts[3], kept_pads);
}

// ----------------------------------------------------------------------------
// Row movement: pack_rows and reconstruct.  One wave moves one row of
// row_bytes in 16-byte lanes; kU chunks per lane are loaded before any store
// so that each wave keeps several loads in flight.
// ----------------------------------------------------------------------------

constexpr int kRowThreads = 256;
constexpr int kU = 4;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Stores of output rows.  The [B, S, W] outputs of reconstruct and of the
// backward of pack_rows (2.2 GB on the 32K-prompt batch) measured 8-10%
// faster with plain stores; the [T, W] outputs of pack_rows and of the
// backward of reconstruct (a seventh of that, written while reading the large
// side) 10-12% faster with non-temporal ones, in the layer step.
__device__ inline void stream_store(u32x4 *p, const u32x4 &v) { __builtin_nontemporal_store(v, p); }
__device__ inline void plain_store(u32x4 *p, const u32x4 &v) { *p = v; }

// Non-temporal loads for inputs read once from cold HBM (pack_rows' [B,S,W]
// rows, reconstruct_bwd's gradient cells): measured 4% and 8% faster in the
// layer step.  Inputs that a kernel before just wrote (reconstruct's packed
// rows, pack_rows_bwd's) are read with plain loads, which hit the
// Infinity Cache more often and measured faster there.
__device__ inline u32x4 stream_load(const u32x4 *p) { return __builtin_nontemporal_load(p); }

// packed[j] = rows[src[j]]; with cell_row (another plan's dst), the input is
// that plan's packed layout: packed[j] = rows[cell_row[src[j]]], zeros where
// the cell has no row there.
__global__ void __launch_bounds__(kRowThreads) k_pack_rows(int64_t T, int64_t vec_per_row,
                                                            const int32_t *__restrict__ src,
                                                            const int32_t *__restrict__ cell_row,
                                                            const u32x4 *__restrict__ rows,
                                                            u32x4 *__restrict__ packed) {
  const int lane = __lane_id();
  const int64_t nwaves = int64_t(gridDim.x) * (kRowThreads / 64);
  const int64_t jfirst = int64_t(blockIdx.x) * (kRowThreads / 64) + threadIdx.x / 64;
  auto row_of = [&](int64_t j) -> int64_t { return cell_row ? cell_row[src[j]] : src[j]; };
  if (vec_per_row <= 64 * kU) {
    // as in k_reconstruct: the next row's loads go out before this row's stores
    u32x4 v[kU];
    auto load = [&](int64_t j, u32x4 (&x)[kU]) {
      const int64_t r = j < T ? row_of(j) : -1;
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t c = u * 64 + lane;
        x[u] = (c < vec_per_row && r >= 0) ? stream_load(rows + r * vec_per_row + c) : u32x4{0u, 0u, 0u, 0u};
      }
    };
    load(jfirst, v);
    for (int64_t j = jfirst; j < T; j += nwaves) {
      u32x4 vn[kU];
      load(j + nwaves, vn);
      u32x4 *out = packed + j * vec_per_row;
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t c = u * 64 + lane;
        if (c < vec_per_row) stream_store(out + c, v[u]);
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) v[u] = vn[u];
    }
    return;
  }
  for (int64_t j = jfirst; j < T; j += nwaves) {
    const int64_t r = row_of(j);
    const u32x4 *in = rows + r * vec_per_row;
    u32x4 *out = packed + j * vec_per_row;
    for (int64_t c0 = 0; c0 < vec_per_row; c0 += 64 * kU) {
      u32x4 v[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t c = c0 + u * 64 + lane;
        v[u] = (c < vec_per_row && r >= 0) ? stream_load(in + c) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t c = c0 + u * 64 + lane;
        if (c < vec_per_row) stream_store(out + c, v[u]);
      }
    }
  }
}

// Packed row j goes to every (b, t) that maps to it: for a prompt row, the
// same column t of every member of the group (read once, written n times);
// for a response row, its own (b, t).  Then, when unpad left cells that no
// packed row maps (counts[2] > 0), those read as zeros.
// SOURCE_ONLY (the backward of pack_rows): only the cell row j was packed from
// (src[j]) receives it; the other cells that map to j -- the group's other
// members' copies of a prompt row -- receive zeros.  Written by packed row like
// the forward, every output line is stored once.
template <bool SOURCE_ONLY>
__global__ void __launch_bounds__(kRowThreads) k_reconstruct(int64_t T, int64_t S, int64_t P,
                                                              int64_t vec_per_row, spd_plan plan,
                                                              const u32x4 *__restrict__ packed,
                                                              u32x4 *__restrict__ out) {
  const int lane = __lane_id();
  const int64_t nwaves = int64_t(gridDim.x) * (kRowThreads / 64);
  const int64_t jfirst = int64_t(blockIdx.x) * (kRowThreads / 64) + threadIdx.x / 64;
  // The readers of packed row j: samples members[m0 .. m1) (every sample for a
  // shared-prefix row; just b0 for a response row), column t.
  auto readers = [&](int64_t j, int64_t &b0, int64_t &t, int &m0, int &m1, const int32_t *&members,
                     bool &every_sample) {
    const int64_t s = plan.src[j];
    b0 = s / S;
    t = s - b0 * S;
    m0 = 0;
    m1 = 1;
    members = nullptr;
    every_sample = false;
    if (t < plan.counts[4]) {
      m1 = static_cast<int>(plan.B);
      every_sample = true;
    } else if (t < P) {
      const int g = plan.group_of[b0];
      m0 = plan.grp_off[g];
      m1 = plan.grp_off[g + 1];
      members = plan.grp_idx;
    }
  };
  auto store_row = [&](int64_t j, int64_t c0, const u32x4 (&v)[kU]) {
    int64_t b0, t;
    int m0, m1;
    const int32_t *members;
    bool every_sample;
    readers(j, b0, t, m0, m1, members, every_sample);
    for (int m = m0; m < m1; ++m) {
      const int64_t b = every_sample ? m : (members ? members[m] : b0);
      u32x4 *o = out + (b * S + t) * vec_per_row;
      const bool zero = SOURCE_ONLY && b != b0;
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t c = c0 + u * 64 + lane;
        if (c < vec_per_row) plain_store(o + c, zero ? u32x4{0u, 0u, 0u, 0u} : v[u]);
      }
    }
  };
  if (vec_per_row <= 64 * kU) {
    // One chunk covers a row: the next row's loads go out before this row's
    // stores, so waiting for them (the memory counter is in order) does not
    // wait for the stores.
    u32x4 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) v[u] = u32x4{0u, 0u, 0u, 0u};
    if (jfirst < T) {
#pragma unroll
      for (int u = 0; u < kU; ++u)
        if (u * 64 + lane < vec_per_row) v[u] = packed[jfirst * vec_per_row + u * 64 + lane];
    }
    for (int64_t j = jfirst; j < T; j += nwaves) {
      const int64_t jn = j + nwaves;
      u32x4 vn[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        vn[u] = u32x4{0u, 0u, 0u, 0u};
        if (jn < T && u * 64 + lane < vec_per_row) vn[u] = packed[jn * vec_per_row + u * 64 + lane];
      }
      store_row(j, 0, v);
#pragma unroll
      for (int u = 0; u < kU; ++u) v[u] = vn[u];
    }
  } else {
    for (int64_t j = jfirst; j < T; j += nwaves) {
      const u32x4 *in = packed + j * vec_per_row;
      for (int64_t c0 = 0; c0 < vec_per_row; c0 += 64 * kU) {
        u32x4 v[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int64_t c = c0 + u * 64 + lane;
          if (c < vec_per_row) v[u] = in[c];
        }
        store_row(j, c0, v);
      }
    }
  }
  if (plan.counts[2] != 0) {
    // This wave's cells are r = w, w + nwaves, ...: lane l reads the map of
    // the l-th of the next 64 at once, and the cells with none are zeroed.
    const int64_t cells = plan.B * S;
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int64_t r0 = int64_t(blockIdx.x) * (kRowThreads / 64) + threadIdx.x / 64; r0 < cells; r0 += 64 * nwaves) {
      const int64_t rl = r0 + lane * nwaves;
      uint64_t todo = __ballot(rl < cells && plan.dst[rl] < 0);
      while (todo) {
        const int l = __builtin_ctzll(todo);
        todo &= todo - 1;
        u32x4 *o = out + (r0 + int64_t(l) * nwaves) * vec_per_row;
        for (int64_t c = lane; c < vec_per_row; c += 64) plain_store(o + c, z);
      }
    }
  }
}

// Backward of reconstruct: packed row j receives the sum of the gradients of
// every (b, t) that reads it -- for a prompt row, column t of each member of
// the group, summed in ascending member order in fp32 and rounded once; for a
// response row, its own (b, t).  E is the element type (bf16 or fp32).
// With to_dst / to_src (another plan "to"), the gradient of cell (b, t) is the
// row to_dst[b*S+t] of a [T_to] input, and a cell counts only if it is that
// row's source (to_src[to_dst[c]] == c): the transpose of
// out[i] = in[plan.dst[to.src[i]]].
template <typename E>
__global__ void __launch_bounds__(kRowThreads) k_reconstruct_bwd(int64_t T, int64_t S, int64_t P,
                                                                  int64_t vec_per_row, spd_plan plan,
                                                                  const int32_t *__restrict__ to_dst,
                                                                  const int32_t *__restrict__ to_src,
                                                                  const u32x4 *__restrict__ dout,
                                                                  u32x4 *__restrict__ dpacked) {
  constexpr int EPV = 16 / sizeof(E);   // elements per 16-byte vector
  const int lane = __lane_id();
  const int64_t nwaves = int64_t(gridDim.x) * (kRowThreads / 64);
  for (int64_t j = int64_t(blockIdx.x) * (kRowThreads / 64) + threadIdx.x / 64; j < T; j += nwaves) {
    const int64_t s = plan.src[j];
    const int64_t b0 = s / S;
    const int64_t t = s - b0 * S;
    int m0 = 0, m1 = 1;
    const int32_t *members = nullptr;
    bool every_sample = false;      // a shared-prefix row: read by every sample
    if (t < plan.counts[4]) {
      m1 = static_cast<int>(plan.B);
      every_sample = true;
    } else if (t < P) {
      const int g = plan.group_of[b0];
      m0 = plan.grp_off[g];
      m1 = plan.grp_off[g + 1];
      members = plan.grp_idx;
    }
    u32x4 *o = dpacked + j * vec_per_row;
    for (int64_t c0 = 0; c0 < vec_per_row; c0 += 64 * kU) {
      float acc[kU][EPV];
#pragma unroll
      for (int u = 0; u < kU; ++u)
#pragma unroll
        for (int e = 0; e < EPV; ++e) acc[u][e] = 0.0f;
      for (int m = m0; m < m1; ++m) {
        const int64_t b = every_sample ? m : (members ? members[m] : b0);
        const int64_t cell = b * S + t;
        int64_t r = cell;
        if (to_dst) {
          r = to_dst[cell];
          if (r < 0 || to_src[r] != cell) continue;
        }
        const u32x4 *in = dout + r * vec_per_row;
        u32x4 v[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int64_t c = c0 + u * 64 + lane;
          v[u] = c < vec_per_row ? stream_load(in + c) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const auto x = __builtin_bit_cast(E __attribute__((ext_vector_type(EPV))), v[u]);
#pragma unroll
          for (int e = 0; e < EPV; ++e) acc[u][e] += static_cast<float>(x[e]);
        }
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t c = c0 + u * 64 + lane;
        E __attribute__((ext_vector_type(EPV))) y;
#pragma unroll
        for (int e = 0; e < EPV; ++e) y[e] = static_cast<E>(acc[u][e]);
        if (c < vec_per_row) stream_store(o + c, __builtin_bit_cast(u32x4, y));
      }
    }
  }
}

// Shared prefix: counts[4] = the number of leading prompt columns on which
// the first members of all groups agree (0 with fewer than two groups).
__global__ void k_prefix_init(int64_t P, spd_plan plan) {
  if (threadIdx.x == 0) plan.counts[4] = plan.counts[0] >= 2 ? static_cast<int32_t>(P) : 0;
}

// One block per group g >= 1: its first mismatch with group 0's prompt.
__global__ void __launch_bounds__(256) k_prefix_mismatch(const int64_t *__restrict__ ids, int64_t S, int64_t P,
                                                         spd_plan plan) {
  __shared__ int wmin[4];
  const int g = blockIdx.x + 1;
  if (g >= plan.counts[0]) return;
  const int64_t *a = ids + int64_t(plan.rep[0]) * S;
  const int64_t *c = ids + int64_t(plan.rep[g]) * S;
  int first = INT_MAX;
  for (int64_t t = threadIdx.x; t < P; t += blockDim.x)
    if (a[t] != c[t]) first = min(first, static_cast<int>(t));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) first = min(first, __shfl_xor(first, off, 64));
  if (__lane_id() == 0) wmin[threadIdx.x / 64] = first;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w) first = min(first, wmin[w]);
    if (first != INT_MAX) atomicMin(&plan.counts[4], first);
  }
}

// Every sample its own group: the plan of the non-deduplicated batch.
__global__ void k_singleton_groups(int B, spd_plan plan) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < B) {
    plan.group_of[b] = b;
    plan.grp_idx[b] = b;
    plan.rep[b] = b;
    plan.grp_off[b] = b;
  }
  if (b == 0) {
    plan.grp_off[B] = B;
    plan.counts[0] = B;
    plan.counts[4] = 0;
    plan.counts[5] = 0;
  }
}

int row_grid(int64_t rows) {
  const int64_t waves_per_block = kRowThreads / 64;
  const int64_t want = (rows + waves_per_block - 1) / waves_per_block;
  const int64_t cap = int64_t(device_cu_count()) * 16;
  return static_cast<int>(std::max<int64_t>(1, std::min(want, cap)));
}

}  // namespace spd

using namespace spd;

// ----------------------------------------------------------------------------
// C ABI
// ----------------------------------------------------------------------------

namespace {
// Hash chunks per row for prompts of at most P tokens (at least one).
int64_t hash_chunks(int64_t P) { return P > kHashChunk ? (P + kHashChunk - 1) / kHashChunk : 1; }
}  // namespace

extern "C" size_t spd_group_workspace_bytes(int64_t B, int64_t S) {
  if (B < 1 || S < 0) return 0;
  return round_up(size_t(B * hash_chunks(S)) * 8, 256) + 3 * round_up(size_t(B) * 4, 256);
}

extern "C" spd_status spd_group(const int64_t *input_ids, int64_t B, int64_t S, int64_t response_length,
                                const spd_plan *plan, int64_t *unique_prompts, void *workspace,
                                size_t workspace_bytes, void *stream) {
  SPD_TRY(validate_plan(plan));
  if (!input_ids || B != plan->B || S != plan->S || response_length < 0 || response_length > S ||
      plan->P != S - response_length)
    return SPD_ERR_INVALID_ARG;
  if (!aligned16(input_ids) || (unique_prompts && !aligned16(unique_prompts))) return SPD_ERR_ALIGNMENT;
  if (!workspace || workspace_bytes < spd_group_workspace_bytes(B, S)) return SPD_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t P = plan->P;
  char *ws = static_cast<char *>(workspace);
  uint64_t *hash_part = reinterpret_cast<uint64_t *>(ws);
  ws += round_up(size_t(B * hash_chunks(S)) * 8, 256);
  int32_t *rep_of = reinterpret_cast<int32_t *>(ws);
  ws += round_up(size_t(B) * 4, 256);
  int32_t *gid_of = reinterpret_cast<int32_t *>(ws);
  ws += round_up(size_t(B) * 4, 256);
  int32_t *fill = reinterpret_cast<int32_t *>(ws);

  const int nch = static_cast<int>(hash_chunks(P));
  const dim3 hgrid(static_cast<unsigned>(B * nch));
  if (S % 2 == 0) {
    hipLaunchKernelGGL(k_hash_rows<true>, hgrid, dim3(256), 0, st, input_ids, S, P, nch, hash_part);
    SPD_LAUNCH_CHECK();
    hipLaunchKernelGGL(k_find_rep<true>, dim3(B), dim3(256), 0, st, input_ids, S, P, nch, hash_part, rep_of);
  } else {
    hipLaunchKernelGGL(k_hash_rows<false>, hgrid, dim3(256), 0, st, input_ids, S, P, nch, hash_part);
    SPD_LAUNCH_CHECK();
    hipLaunchKernelGGL(k_find_rep<false>, dim3(B), dim3(256), 0, st, input_ids, S, P, nch, hash_part, rep_of);
  }
  SPD_LAUNCH_CHECK();
  hipLaunchKernelGGL(k_finalize_groups, dim3(1), dim3(kFinalThreads), 0, st, int(B), rep_of, gid_of, fill,
                     *plan);
  SPD_LAUNCH_CHECK();
  if (unique_prompts && P > 0) {
    if (S % 2 == 0 && P % 2 == 0)
      hipLaunchKernelGGL(k_unique_prompts<true>, hgrid, dim3(256), 0, st, input_ids, S, P, nch, plan->rep,
                         plan->counts, unique_prompts);
    else
      hipLaunchKernelGGL(k_unique_prompts<false>, hgrid, dim3(256), 0, st, input_ids, S, P, nch, plan->rep,
                         plan->counts, unique_prompts);
    SPD_LAUNCH_CHECK();
  }
  return SPD_OK;
}

// seg: 2 B ints (the segment-offset scan); cnt: 3 ints per (sample, chunk).
static int64_t pack_chunks(int64_t S) { return (S + kPackChunk - 1) / kPackChunk; }

extern "C" size_t spd_pack_workspace_bytes(int64_t B, int64_t S) {
  if (B < 1 || S < 1) return 0;
  return round_up(size_t(2 * B) * 4, 256) + round_up(size_t(B) * size_t(pack_chunks(S)) * 3 * 4, 256);
}

extern "C" spd_status spd_pack(const int64_t *input_ids, const int64_t *position_ids, const void *attention_mask,
                               int32_t mask_elem_bytes, int32_t use_unpad, spd_plan *plan,
                               int64_t *dedup_ids, int64_t *dedup_pos, void *workspace, size_t workspace_bytes,
                               void *stream) {
  SPD_TRY(validate_plan(plan));
  if (!input_ids || !position_ids || !dedup_ids || !dedup_pos) return SPD_ERR_INVALID_ARG;
  if (use_unpad != 0 && use_unpad != 1) return SPD_ERR_INVALID_ARG;
  if (use_unpad && !attention_mask) return SPD_ERR_INVALID_ARG;
  if (attention_mask && mask_elem_bytes != 1 && mask_elem_bytes != 4 && mask_elem_bytes != 8)
    return SPD_ERR_INVALID_ARG;
  if (!aligned16(input_ids) || !aligned16(position_ids) || !aligned16(dedup_ids) || !aligned16(dedup_pos))
    return SPD_ERR_ALIGNMENT;
  if (!workspace || workspace_bytes < spd_pack_workspace_bytes(plan->B, plan->S)) return SPD_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t B = plan->B, S = plan->S, P = plan->P;
  const int esz = attention_mask ? mask_elem_bytes : 1;
  int32_t *seg = static_cast<int32_t *>(workspace);
  // padded format with a mask: pads may sit among the packed rows, which the attention calls must not see
  plan->padded_with_mask = (!use_unpad && attention_mask) ? 1 : 0;
  const int nch = static_cast<int>(pack_chunks(S));
  int32_t *cnt = reinterpret_cast<int32_t *>(static_cast<char *>(workspace) + round_up(size_t(2 * B) * 4, 256));
  const unsigned chunk_blocks = static_cast<unsigned>(B * nch);
  if (use_unpad) {
    hipLaunchKernelGGL(k_chunk_counts, dim3(chunk_blocks), dim3(256), 0, st, S, P, attention_mask, esz, nch, *plan,
                       cnt);
    SPD_LAUNCH_CHECK();
    hipLaunchKernelGGL(k_chunk_bases, dim3(static_cast<unsigned>((3 * B + 3) / 4)), dim3(256), 0, st, nch, *plan,
                       cnt);
  } else {
    hipLaunchKernelGGL(k_seg_lengths_dense, dim3(1), dim3(256), 0, st, S, P, *plan);
  }
  SPD_LAUNCH_CHECK();
  hipLaunchKernelGGL(k_seg_offsets, dim3(1), dim3(kFinalThreads), 0, st, int(B), seg, *plan);
  SPD_LAUNCH_CHECK();
  if (use_unpad)
    hipLaunchKernelGGL(k_scatter_chunks, dim3(chunk_blocks), dim3(256), 0, st, S, P, input_ids, position_ids,
                       attention_mask, esz, nch, *plan, cnt, dedup_ids, dedup_pos);
  else
    hipLaunchKernelGGL(k_scatter_dense, dim3(unsigned(std::min<int64_t>((B * S + 255) / 256, 65536))), dim3(256),
                       0, st, S, P, input_ids, position_ids, attention_mask, esz, *plan, dedup_ids, dedup_pos);
  SPD_LAUNCH_CHECK();
  return SPD_OK;
}

extern "C" spd_status spd_pack_rows(const spd_plan *plan, int64_t T, const void *rows, int64_t row_bytes,
                                    void *packed, void *stream) {
  SPD_TRY(validate_plan(plan));
  if (!rows || (!packed && T != 0) || T < 0 || T > plan->B * plan->S || row_bytes <= 0) return SPD_ERR_INVALID_ARG;
  if (row_bytes % 16 || !aligned16(rows) || !aligned16(packed)) return SPD_ERR_ALIGNMENT;
  if (T == 0) return SPD_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  prof_start(SPD_K_PACK_ROWS, st);
  hipLaunchKernelGGL(k_pack_rows, dim3(row_grid(T)), dim3(kRowThreads), 0, st, T, row_bytes / 16, plan->src,
                     static_cast<const int32_t *>(nullptr), static_cast<const u32x4 *>(rows),
                     static_cast<u32x4 *>(packed));
  SPD_LAUNCH_CHECK();
  prof_stop(SPD_K_PACK_ROWS, st);
  return SPD_OK;
}

extern "C" spd_status spd_reconstruct(const spd_plan *plan, int64_t T, const void *packed, int64_t row_bytes,
                                      void *out, void *stream) {
  SPD_TRY(validate_plan(plan));
  if ((!packed && T != 0) || !out || T < 0 || T > plan->B * plan->S || row_bytes <= 0) return SPD_ERR_INVALID_ARG;
  if (row_bytes % 16 || !aligned16(packed) || !aligned16(out)) return SPD_ERR_ALIGNMENT;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t vpr = row_bytes / 16;
  prof_start(SPD_K_RECONSTRUCT, st);
  hipLaunchKernelGGL(k_reconstruct<false>, dim3(row_grid(plan->B * plan->S)), dim3(kRowThreads), 0, st, T,
                     plan->S, plan->P, vpr, *plan, static_cast<const u32x4 *>(packed), static_cast<u32x4 *>(out));
  SPD_LAUNCH_CHECK();
  prof_stop(SPD_K_RECONSTRUCT, st);
  return SPD_OK;
}

extern "C" spd_status spd_reconstruct_bwd(const spd_plan *plan, int64_t T, const void *dout, int64_t row_bytes,
                                          int32_t dtype, void *dpacked, void *stream) {
  SPD_TRY(validate_plan(plan));
  if (!dout || (!dpacked && T != 0) || T < 0 || T > plan->B * plan->S || row_bytes <= 0) return SPD_ERR_INVALID_ARG;
  if (dtype != SPD_F32 && dtype != SPD_BF16) return SPD_ERR_UNSUPPORTED;
  if (row_bytes % 16 || !aligned16(dout) || !aligned16(dpacked)) return SPD_ERR_ALIGNMENT;
  if (T == 0) return SPD_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t vpr = row_bytes / 16;
  prof_start(SPD_K_RECONSTRUCT_BWD, st);
  if (dtype == SPD_BF16)
    hipLaunchKernelGGL(k_reconstruct_bwd<__bf16>, dim3(row_grid(T)), dim3(kRowThreads), 0, st, T, plan->S, plan->P,
                       vpr, *plan, static_cast<const int32_t *>(nullptr), static_cast<const int32_t *>(nullptr),
                       static_cast<const u32x4 *>(dout), static_cast<u32x4 *>(dpacked));
  else
    hipLaunchKernelGGL(k_reconstruct_bwd<float>, dim3(row_grid(T)), dim3(kRowThreads), 0, st, T, plan->S, plan->P,
                       vpr, *plan, static_cast<const int32_t *>(nullptr), static_cast<const int32_t *>(nullptr),
                       static_cast<const u32x4 *>(dout), static_cast<u32x4 *>(dpacked));
  SPD_LAUNCH_CHECK();
  prof_stop(SPD_K_RECONSTRUCT_BWD, st);
  return SPD_OK;
}

extern "C" spd_status spd_pack_rows_bwd(const spd_plan *plan, int64_t T, const void *dpacked, int64_t row_bytes,
                                        void *drows, void *stream) {
  SPD_TRY(validate_plan(plan));
  if ((!dpacked && T != 0) || !drows || T < 0 || T > plan->B * plan->S || row_bytes <= 0) return SPD_ERR_INVALID_ARG;
  if (row_bytes % 16 || !aligned16(dpacked) || !aligned16(drows)) return SPD_ERR_ALIGNMENT;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t vpr = row_bytes / 16;
  prof_start(SPD_K_PACK_ROWS_BWD, st);
  hipLaunchKernelGGL(k_reconstruct<true>, dim3(row_grid(plan->B * plan->S)), dim3(kRowThreads), 0, st, T,
                     plan->S, plan->P, vpr, *plan, static_cast<const u32x4 *>(dpacked), static_cast<u32x4 *>(drows));
  SPD_LAUNCH_CHECK();
  prof_stop(SPD_K_PACK_ROWS_BWD, st);
  return SPD_OK;
}

extern "C" spd_status spd_share_prefix(const int64_t *input_ids, int64_t B, int64_t S, int64_t response_length,
                                       const spd_plan *plan, void *stream) {
  SPD_TRY(validate_plan(plan));
  if (!input_ids || B != plan->B || S != plan->S || response_length < 0 || response_length > S ||
      plan->P != S - response_length)
    return SPD_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(k_prefix_init, dim3(1), dim3(64), 0, st, plan->P, *plan);
  SPD_LAUNCH_CHECK();
  if (B > 1 && plan->P > 0) {
    hipLaunchKernelGGL(k_prefix_mismatch, dim3(unsigned(B - 1)), dim3(256), 0, st, input_ids, S, plan->P, *plan);
    SPD_LAUNCH_CHECK();
  }
  return SPD_OK;
}

extern "C" spd_status spd_group_singletons(int64_t B, int64_t S, int64_t response_length, const spd_plan *plan,
                                           void *stream) {
  SPD_TRY(validate_plan(plan));
  if (B != plan->B || S != plan->S || response_length < 0 || response_length > S ||
      plan->P != S - response_length)
    return SPD_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(k_singleton_groups, dim3((B + 255) / 256), dim3(256), 0, st, int(B), *plan);
  SPD_LAUNCH_CHECK();
  return SPD_OK;
}

namespace {
spd_status validate_pair(const spd_plan *to, int64_t T_to, const spd_plan *from, int64_t T_from) {
  SPD_TRY(validate_plan(to));
  SPD_TRY(validate_plan(from));
  if (to->B != from->B || to->S != from->S || to->P != from->P) return SPD_ERR_INVALID_ARG;
  if (T_to < 0 || T_to > to->B * to->S || T_from < 0 || T_from > from->B * from->S) return SPD_ERR_INVALID_ARG;
  return SPD_OK;
}
}  // namespace

extern "C" spd_status spd_repack_rows(const spd_plan *to, int64_t T_to, const spd_plan *from, int64_t T_from,
                                      const void *in, int64_t row_bytes, void *out, void *stream) {
  SPD_TRY(validate_pair(to, T_to, from, T_from));
  if ((!in && T_from != 0) || (!out && T_to != 0) || row_bytes <= 0) return SPD_ERR_INVALID_ARG;
  if (row_bytes % 16 || !aligned16(in) || !aligned16(out)) return SPD_ERR_ALIGNMENT;
  if (T_to == 0) return SPD_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(k_pack_rows, dim3(row_grid(T_to)), dim3(kRowThreads), 0, st, T_to, row_bytes / 16, to->src,
                     static_cast<const int32_t *>(from->dst), static_cast<const u32x4 *>(in),
                     static_cast<u32x4 *>(out));
  SPD_LAUNCH_CHECK();
  return SPD_OK;
}

extern "C" spd_status spd_repack_rows_bwd(const spd_plan *to, int64_t T_to, const spd_plan *from, int64_t T_from,
                                          const void *dout, int64_t row_bytes, int32_t dtype, void *din,
                                          void *stream) {
  SPD_TRY(validate_pair(to, T_to, from, T_from));
  if ((!dout && T_to != 0) || (!din && T_from != 0) || row_bytes <= 0) return SPD_ERR_INVALID_ARG;
  if (dtype != SPD_F32 && dtype != SPD_BF16) return SPD_ERR_UNSUPPORTED;
  if (row_bytes % 16 || !aligned16(dout) || !aligned16(din)) return SPD_ERR_ALIGNMENT;
  if (T_from == 0) return SPD_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t vpr = row_bytes / 16;
  if (dtype == SPD_BF16)
    hipLaunchKernelGGL(k_reconstruct_bwd<__bf16>, dim3(row_grid(T_from)), dim3(kRowThreads), 0, st, T_from,
                       from->S, from->P, vpr, *from, static_cast<const int32_t *>(to->dst),
                       static_cast<const int32_t *>(to->src), static_cast<const u32x4 *>(dout),
                       static_cast<u32x4 *>(din));
  else
    hipLaunchKernelGGL(k_reconstruct_bwd<float>, dim3(row_grid(T_from)), dim3(kRowThreads), 0, st, T_from,
                       from->S, from->P, vpr, *from, static_cast<const int32_t *>(to->dst),
                       static_cast<const int32_t *>(to->src), static_cast<const u32x4 *>(dout),
                       static_cast<u32x4 *>(din));
  SPD_LAUNCH_CHECK();
  return SPD_OK;
}

extern "C" const char *spd_status_string(spd_status s) {
  switch (s) {
    case SPD_OK: return "ok";
    case SPD_ERR_INVALID_ARG: return "invalid argument";
    case SPD_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case SPD_ERR_ALIGNMENT: return "pointer or row size not 16-byte aligned";
    case SPD_ERR_WORKSPACE: return "workspace missing or too small";
    case SPD_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

extern "C" int spd_last_hip_error(void) { return g_last_hip_error; }

extern "C" int spd_version(void) { return 100; }
