// Split attention: tile planning on the device and the C-ABI entry points.
//
// How Prompt Deduplication Works -- Phase 2, "Split Attention Optimization"
// (prompt-to-prompt once per unique prompt; response-to-full over its prompt
// and itself) and "Correctness & Gradients".
#include <algorithm>
#include <climits>
#include <mutex>
#include <vector>

#include "spd_attn.h"

// Scratch of spd_split_attn_fwd_noalloc: the forward's query-tile list and the
// planner's scratch, in place of a caller workspace.  Each device the library
// runs on holds its own copy until the process ends.  Host code never passes
// this name to a kernel: it is a host-side stand-in, and the device address
// comes from hipGetSymbolAddress (noalloc_scratch below).
static constexpr size_t kNoAllocScratchBytes = size_t(4) << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace spd {

namespace {

constexpr int kPlanThreads = 1024;
constexpr int kBuckets = 4096;

// Row one past the end of the response segment containing packed row x.
__device__ inline int segment_end(const spd_plan &plan, int x) {
  const int b = static_cast<int>(plan.src[x] / plan.S);
  return plan.resp_off[b] + plan.resp_len[b];
}

// Group g's rows: prompt [po, ro), responses [ro, re), clipped to [0, Tdev).
struct GroupRows {
  int po, ro, re, np, nr;
};

__device__ inline GroupRows group_rows(const spd_plan &plan, int g, int G, int Tdev, int TM) {
  GroupRows r;
  r.po = min(plan.prompt_off[g], Tdev);
  r.ro = min(r.po + plan.prompt_len[g], Tdev);
  r.re = (g + 1 < G) ? min(plan.prompt_off[g + 1], Tdev) : Tdev;
  r.re = max(r.re, r.ro);
  r.np = (r.ro - r.po + TM - 1) / TM;
  r.nr = (r.re - r.ro + TM - 1) / TM;
  return r;
}

// Chunks a key tile is cut into when its reader rows exceed `limit` (1: not
// split); *rows receives the reader rows per chunk.  A key tile's reader rows
// are its masked rows [u0, u1) followed by its unmasked rows [s0, e0).
__device__ inline int chunks_of(const Tile &t, int limit, int *rows) {
  const int U = (t.u1 - t.u0) + (t.e0 - t.s0);
  if (U <= limit || U < 2 * kSplitRows) {
    *rows = U;
    return 1;
  }
  const int want = min(kMaxChunks, (U + limit - 1) / limit);
  const int per = ((U + want - 1) / want + kSplitRows - 1) / kSplitRows * kSplitRows;
  *rows = per;
  return (U + per - 1) / per;
}

// One block: per-group tile counts and their exclusive scan (goff[0..G]),
// then one thread per tile (its group found by binary search over goff),
// then a counting sort by decreasing cost.
__device__ void build_tiles(const spd_plan &plan, int T, const TileJob &job) {
  const int TM = job.rows_per_tile, mode = job.mode, cap = job.cap;
  int *__restrict__ goff = job.goff;
  Tile *__restrict__ tmp = job.tmp;
  Tile *__restrict__ out = job.out;
  SplitGroup *__restrict__ splits = job.splits;
  int *__restrict__ arrivals = job.arrivals;
  const int max_slots = job.max_slots, blocks_per_tile = job.blocks_per_tile, n_cu = job.n_cu;
  __shared__ int scan_tmp[kPlanThreads / 64];
  __shared__ int hist[kBuckets];
  const int tid = threadIdx.x;
  const int G = plan.counts[0];
  const int Tdev = min(plan.counts[1], T);
  const int Lp = min(plan.counts[5], Tdev);       // shared prefix rows [0, Lp), first in the layout
  const int npre = (Lp + TM - 1) / TM;
  int base = npre;
  for (int g0 = 0; g0 < G; g0 += kPlanThreads) {
    const int g = g0 + tid;
    int cnt = 0;
    if (g < G) {
      const GroupRows r = group_rows(plan, g, G, Tdev, TM);
      cnt = r.np + r.nr;
    }
    int total = 0;
    const int ex = block_exclusive_scan(cnt, scan_tmp, total);
    if (g < G) goff[g] = base + ex;
    base += total;
  }
  if (tid == 0) goff[G] = base;
  __syncthreads();
  const int N = min(base, splits ? cap - max_slots : cap);
  for (int i = tid; i < N; i += kPlanThreads) {
    Tile t;
    t.grp = -1;
    if (i < npre) {           // the shared prefix: its own causal keys only
      t.r0 = i * TM;
      t.r1 = min(Lp, t.r0 + TM);
      t.kind = 0;
      t.v0 = t.v1 = 0;
      if (mode == kQueryTiles) {
        t.u0 = t.u1 = 0;
        t.s0 = 0;
        t.e0 = 0;
        t.cost = t.r1;
      } else {
        t.u0 = t.r0;
        t.u1 = Lp;
        t.s0 = Lp;
        t.e0 = Tdev;
        t.cost = (Lp - t.r0) + (Tdev - Lp);
      }
      t.slot = -1;
      out[i] = t;
      continue;
    }
    int lo = 0, hi = G - 1;   // last group whose first tile is <= i
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (goff[mid] <= i) lo = mid;
      else hi = mid - 1;
    }
    const int g = lo;
    const GroupRows r = group_rows(plan, g, G, Tdev, TM);
    const int j = i - goff[g];
    const bool prompt = j < r.np;
    t.r0 = (prompt ? r.po : r.ro) + (prompt ? j : j - r.np) * TM;
    t.r1 = min(prompt ? r.ro : r.re, t.r0 + TM);
    t.kind = prompt ? 0 : 1;
    if (mode == kQueryTiles) {
      t.v0 = 0;
      t.v1 = Lp;
      t.u0 = prompt ? 0 : r.po;
      t.u1 = prompt ? 0 : r.ro;
      t.s0 = plan.seg_start[t.r0];
      t.e0 = 0;
      t.cost = Lp + (t.u1 - t.u0) + (t.r1 - t.s0);
    } else {
      t.v0 = t.v1 = 0;
      t.u0 = t.r0;
      t.u1 = prompt ? r.ro : segment_end(plan, t.r1 - 1);
      t.s0 = prompt ? r.ro : 0;
      t.e0 = prompt ? r.re : 0;
      t.cost = (t.u1 - t.u0) + (t.e0 - t.s0);
    }
    t.slot = -1;
    out[i] = t;
  }
  __syncthreads();
  // When the heaviest key tile is about a CU's fair share of the blocks'
  // reader rows or more, the in-order dispatch cannot even the CUs out: tiles
  // above a limit are cut into chunks, the limit growing until the chunks fit
  // the partial-sum slots.  Below that, splitting only adds the partial sums'
  // traffic.
  int limit = INT_MAX;
  if (splits && n_cu > 0 && max_slots >= 2) {
    __shared__ long long red[kPlanThreads / 64];
    __shared__ int redmax[kPlanThreads / 64];
    long long tot = 0;
    int mx = 0;
    for (int i = tid; i < N; i += kPlanThreads) {
      tot += out[i].cost;
      mx = max(mx, out[i].cost);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      tot += __shfl_xor(tot, off, 64);
      mx = max(mx, __shfl_xor(mx, off, 64));
    }
    if (__lane_id() == 0) {
      red[tid / 64] = tot;
      redmax[tid / 64] = mx;
    }
    __syncthreads();
    tot = 0;
    for (int w = 0; w < kPlanThreads / 64; ++w) {
      tot += red[w];
      mx = max(mx, redmax[w]);
    }
    const long long share = tot * blocks_per_tile / n_cu;
    // chunks of half a share; of two thirds when the heaviest tile holds 1.4 to
    // 3 shares (fewer, larger chunks pack better there: dispatch model of the
    // planner's tile costs over the CUs)
    long long lim = LLONG_MAX;
    if (10LL * mx >= 9LL * share) lim = (10LL * mx >= 14LL * share && mx < 3LL * share) ? share * 2 / 3 : share / 2;
    lim = lim < 2048 ? 2048 : lim;
    for (int attempt = 0; attempt < 12; ++attempt) {
      int need = 0;
      for (int i = tid; i < N; i += kPlanThreads) {
        int rows;
        const int c = chunks_of(out[i], int(lim < INT_MAX ? lim : INT_MAX), &rows);
        need += c > 1 ? c : 0;
      }
      int total;
      block_exclusive_scan(need, scan_tmp, total);
      if (total <= max_slots) {
        limit = int(lim < INT_MAX ? lim : INT_MAX);
        break;
      }
      lim = lim / 2 * 3;
    }
  }
  int M = N;
  if (splits && limit != INT_MAX) {
    // expand into tmp: tile i -> c_i chunks at positions scanned over the tiles
    int pos_base = 0, slot_base = 0, grp_base = 0;
    for (int i0 = 0; i0 < N; i0 += kPlanThreads) {
      const int i = i0 + tid;
      Tile t;
      int rows = 0, c = 0;
      if (i < N) {
        t = out[i];
        c = chunks_of(t, limit, &rows);
      }
      int tp, ts, tg;
      const int pos = pos_base + block_exclusive_scan(c, scan_tmp, tp);
      const int slot0 = slot_base + block_exclusive_scan(c > 1 ? c : 0, scan_tmp, ts);
      const int grp = grp_base + block_exclusive_scan(c > 1 ? 1 : 0, scan_tmp, tg);
      if (i < N) {
        if (c == 1) {
          tmp[pos] = t;
        } else {
          const int Lu = t.u1 - t.u0, U = Lu + (t.e0 - t.s0);
          for (int j = 0; j < c; ++j) {
            const int a = j * rows, b = min(U, a + rows);   // reader rows [a, b) of [u0, u1) ++ [s0, e0)
            Tile ch = t;
            ch.u0 = t.u0 + min(a, Lu);
            ch.u1 = t.u0 + min(b, Lu);
            ch.s0 = t.s0 + max(a - Lu, 0);
            ch.e0 = t.s0 + max(b - Lu, 0);
            ch.cost = b - a;
            ch.slot = slot0 + j;
            ch.grp = grp;
            tmp[pos + j] = ch;
          }
          splits[grp] = SplitGroup{t.r0, t.r1, slot0, c};
          for (int h = 0; h < blocks_per_tile; ++h) arrivals[grp * blocks_per_tile + h] = 0;
        }
      }
      pos_base += tp;
      slot_base += ts;
      grp_base += tg;
    }
    M = pos_base;
  } else {
    for (int i = tid; i < N; i += kPlanThreads) tmp[i] = out[i];
  }
  __syncthreads();
  // counting sort by decreasing cost (order inside a bucket is free: it only
  // changes which block runs a tile first, never a result)
  int shift = 0;
  while ((Tdev >> shift) >= kBuckets) ++shift;
  for (int i = tid; i < kBuckets; i += kPlanThreads) hist[i] = 0;
  __syncthreads();
  for (int i = tid; i < M; i += kPlanThreads) {
    const int bkt = kBuckets - 1 - min(tmp[i].cost >> shift, kBuckets - 1);
    atomicAdd(&hist[bkt], 1);
  }
  __syncthreads();
  int c[4], s = 0;
  for (int e = 0; e < 4; ++e) {
    c[e] = hist[tid * 4 + e];
    s += c[e];
  }
  int total = 0;
  int ex = block_exclusive_scan(s, scan_tmp, total);
  __syncthreads();
  for (int e = 0; e < 4; ++e) {
    hist[tid * 4 + e] = ex;
    ex += c[e];
  }
  __syncthreads();
  __syncthreads();
  for (int i = tid; i < M; i += kPlanThreads) {
    const Tile t = tmp[i];
    const int bkt = kBuckets - 1 - min(t.cost >> shift, kBuckets - 1);
    out[atomicAdd(&hist[bkt], 1)] = t;
  }
  if (tid == 0) *job.n_out = M;
}

// Block b builds job b's list.
__global__ void __launch_bounds__(kPlanThreads) k_build_tiles(spd_plan plan, int T, TileJob j0, TileJob j1) {
  build_tiles(plan, T, blockIdx.x == 0 ? j0 : j1);
}

}  // namespace

spd_status launch_build_tiles(const spd_plan &plan, int64_t T, const TileJob &job, hipStream_t st,
                              const TileJob *second) {
  static_assert(kBuckets == 4 * kPlanThreads, "bucket scan assumes 4 buckets per thread");
  hipLaunchKernelGGL(k_build_tiles, dim3(second ? 2 : 1), dim3(kPlanThreads), 0, st, plan, int(T), job,
                     second ? *second : job);
  return check_launch();
}

namespace {

struct AttnWs {
  Tile *qtiles = nullptr, *ktiles = nullptr, *tmp = nullptr, *tmp2 = nullptr;
  int *counts = nullptr, *goff = nullptr, *goff2 = nullptr;
  float *Dbuf = nullptr, *L2buf = nullptr;
  int *segp = nullptr;
  SplitGroup *splits = nullptr;
  int *arrivals = nullptr;
  float *part_k = nullptr, *part_v = nullptr;
  int64_t capq = 0, capk = 0, Tp = 0;
  int slots = 0;
  size_t bytes = 0;
};

int q_rows(const spd_attn_desc &d) { return d.dtype == SPD_F32 ? kF32Rows : fwd_bf16_rows_per_tile(d); }
int dq_rows(const spd_attn_desc &d) { return d.dtype == SPD_F32 ? kF32Rows : dq_bf16_rows_per_tile(d); }
int k_rows(const spd_attn_desc &d) { return d.dtype == SPD_F32 ? kF32Rows : dkdv_bf16_rows_per_tile(d); }

// Forward workspace: [query tiles][scratch tiles][counts][group offsets].
AttnWs carve_fwd(const spd_attn_desc &d, int64_t B, int64_t T, void *base) {
  AttnWs w;
  w.capq = tile_capacity(B, T, q_rows(d));
  const size_t qb = round_up(size_t(w.capq) * sizeof(Tile), 256);
  char *p = static_cast<char *>(base);
  size_t off = 0;
  if (p) w.qtiles = reinterpret_cast<Tile *>(p + off);
  off += qb;
  if (p) w.tmp = reinterpret_cast<Tile *>(p + off);
  off += qb;
  if (p) w.counts = reinterpret_cast<int *>(p + off);
  off += 256;
  if (p) w.goff = reinterpret_cast<int *>(p + off);
  off += round_up(size_t(B + 1) * 4, 256);
  w.bytes = off;
  return w;
}

// Backward workspace: [-D: Hq*Tp floats][-lse/scale: Hq*Tp floats][segment ends: Tp ints]
//            [query tiles][key tiles][scratch tiles x 2][counts][group offsets x 2]
//            bf16 only: [split groups][arrival counters: slots x Hkv ints]
//                       [partial dK][partial dV] (slots x Hkv x 256 x D floats each)
AttnWs carve(const spd_attn_desc &d, int64_t B, int64_t T, void *base) {
  AttnWs w;
  const int rq = std::min(q_rows(d), dq_rows(d));
  w.slots = d.dtype == SPD_BF16 ? split_slots(d.num_kv_heads) : 0;
  w.capq = tile_capacity(B, T, rq);
  w.capk = tile_capacity(B, T, k_rows(d)) + w.slots;
  w.Tp = padded_rows(T);
  const size_t dbytes = round_up(size_t(d.num_q_heads) * size_t(w.Tp) * 4, 256);
  const size_t sbytes = round_up(size_t(w.Tp) * 4, 256);
  const size_t qb = round_up(size_t(w.capq) * sizeof(Tile), 256);
  const size_t kb = round_up(size_t(w.capk) * sizeof(Tile), 256);
  const size_t tb = std::max(qb, kb);
  char *p = static_cast<char *>(base);
  size_t off = 0;
  if (p) w.Dbuf = reinterpret_cast<float *>(p + off);
  off += dbytes;
  if (p) w.L2buf = reinterpret_cast<float *>(p + off);
  off += dbytes;
  if (p) w.segp = reinterpret_cast<int *>(p + off);
  off += sbytes;
  if (p) w.qtiles = reinterpret_cast<Tile *>(p + off);
  off += qb;
  if (p) w.ktiles = reinterpret_cast<Tile *>(p + off);
  off += kb;
  if (p) w.tmp = reinterpret_cast<Tile *>(p + off);
  off += tb;
  if (p) w.tmp2 = reinterpret_cast<Tile *>(p + off);
  off += tb;
  if (p) w.counts = reinterpret_cast<int *>(p + off);
  off += 256;
  if (p) w.goff = reinterpret_cast<int *>(p + off);
  off += round_up(size_t(B + 1) * 4, 256);
  if (p) w.goff2 = reinterpret_cast<int *>(p + off);
  off += round_up(size_t(B + 1) * 4, 256);
  if (w.slots) {
    const size_t pb = size_t(w.slots) * size_t(d.num_kv_heads) * size_t(k_rows(d)) * size_t(d.head_dim) * 4;
    if (p) w.splits = reinterpret_cast<SplitGroup *>(p + off);
    off += round_up(size_t(w.slots) * sizeof(SplitGroup), 256);
    if (p) w.arrivals = reinterpret_cast<int *>(p + off);
    off += round_up(size_t(w.slots) * size_t(d.num_kv_heads) * 4, 256);
    if (p) w.part_k = reinterpret_cast<float *>(p + off);
    off += pb;
    if (p) w.part_v = reinterpret_cast<float *>(p + off);
    off += pb;
  }
  w.bytes = off;
  return w;
}

spd_status validate_desc(const spd_attn_desc *d) {
  if (!d) return SPD_ERR_INVALID_ARG;
  if (d->num_q_heads < 1 || d->num_kv_heads < 1 || d->num_q_heads % d->num_kv_heads) return SPD_ERR_INVALID_ARG;
  if (!(d->softmax_scale > 0.0f)) return SPD_ERR_INVALID_ARG;
  if (d->dtype != SPD_F32 && d->dtype != SPD_BF16) return SPD_ERR_UNSUPPORTED;
  if (d->head_dim != 64 && d->head_dim != 128) return SPD_ERR_UNSUPPORTED;
  if (d->num_q_heads > 1024) return SPD_ERR_UNSUPPORTED;
  return SPD_OK;
}

// Checks shared by the forward and the backward (everything but the workspace).
spd_status validate_common(const spd_attn_desc *d, const spd_plan *plan, int64_t T) {
  SPD_TRY(validate_desc(d));
  SPD_TRY(validate_plan(plan));
  if (T < 0 || T > plan->B * plan->S) return SPD_ERR_INVALID_ARG;
  if (plan->padded_with_mask) return SPD_ERR_UNSUPPORTED;    // pads among the rows: attend on the unpadded plan
  if (int64_t(d->num_q_heads) * T * d->head_dim >= (int64_t(1) << 40)) return SPD_ERR_UNSUPPORTED;
  // K / V row offsets inside the kernels are 32-bit byte offsets from a head's first row
  const int64_t elt = d->dtype == SPD_F32 ? 4 : 2;
  if (T * int64_t(d->num_kv_heads) * d->head_dim * elt >= (int64_t(1) << 32)) return SPD_ERR_UNSUPPORTED;
  return SPD_OK;
}

// The forward after validation: the query-tile list in `workspace`, then the attention kernel.
spd_status fwd_launch(const spd_attn_desc *desc, const spd_plan *plan, int64_t T, const void *q, const void *k,
                      const void *v, void *o, float *lse, void *workspace, void *stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  AttnWs w = carve_fwd(*desc, plan->B, T, workspace);
  TileJob qj;
  qj.rows_per_tile = q_rows(*desc);
  qj.mode = kQueryTiles;
  qj.cap = int(w.capq);
  qj.goff = w.goff;
  qj.tmp = w.tmp;
  qj.out = w.qtiles;
  qj.n_out = w.counts;
  SPD_TRY(launch_build_tiles(*plan, T, qj, st));
  if (desc->dtype == SPD_F32)
    return attn_fwd_f32(*desc, *plan, T, w.qtiles, w.counts, w.capq, static_cast<const float *>(q),
                        static_cast<const float *>(k), static_cast<const float *>(v), static_cast<float *>(o), lse,
                        st);
  return attn_fwd_bf16(*desc, *plan, T, w.qtiles, w.counts, w.capq, q, k, v, o, lse, st);
}

// The scratch array's address on the current device, looked up once per
// device (with that device current) and kept.
spd_status noalloc_scratch(void **out) {
  static std::mutex mu;
  static std::vector<void *> addr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    set_last_hip_error(e);
    return SPD_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (dev >= static_cast<int>(addr.size())) addr.resize(dev + 1, nullptr);
  if (!addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      set_last_hip_error(e != hipSuccess ? e : hipErrorInvalidSymbol);
      return SPD_ERR_HIP;
    }
    addr[dev] = p;
  }
  *out = addr[dev];
  return SPD_OK;
}

}  // namespace
}  // namespace spd

using namespace spd;

extern "C" size_t spd_attn_workspace_bytes(const spd_attn_desc *desc, int64_t B, int64_t T) {
  if (validate_desc(desc) != SPD_OK || B < 1 || T < 0) return 0;
  return carve(*desc, B, T, nullptr).bytes;
}

extern "C" size_t spd_attn_fwd_workspace_bytes(const spd_attn_desc *desc, int64_t B, int64_t T) {
  if (validate_desc(desc) != SPD_OK || B < 1 || T < 0) return 0;
  return carve_fwd(*desc, B, T, nullptr).bytes;
}

extern "C" spd_status spd_split_attn_fwd(const spd_attn_desc *desc, const spd_plan *plan, int64_t T, const void *q,
                                         const void *k, const void *v, void *o, float *lse, void *workspace,
                                         size_t workspace_bytes, void *stream) {
  SPD_TRY(validate_common(desc, plan, T));
  if (!workspace || workspace_bytes < spd_attn_fwd_workspace_bytes(desc, plan->B, T)) return SPD_ERR_WORKSPACE;
  if (T == 0) return SPD_OK;      // no rows: the [T, ...] buffers may be NULL
  if (!q || !k || !v || !o || !lse) return SPD_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return SPD_ERR_ALIGNMENT;
  return fwd_launch(desc, plan, T, q, k, v, o, lse, workspace, stream);
}

extern "C" spd_status spd_split_attn_fwd_noalloc(const spd_attn_desc *desc, const spd_plan *plan, int64_t T,
                                                 const void *q, const void *k, const void *v, void *o, float *lse,
                                                 void *stream) {
  SPD_TRY(validate_common(desc, plan, T));
  if (spd_attn_fwd_workspace_bytes(desc, plan->B, T) > kNoAllocScratchBytes) return SPD_ERR_WORKSPACE;
  if (T == 0) return SPD_OK;      // no rows: the [T, ...] buffers may be NULL
  if (!q || !k || !v || !o || !lse) return SPD_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return SPD_ERR_ALIGNMENT;
  void *ws = nullptr;
  SPD_TRY(noalloc_scratch(&ws));
  // every scratch word the planner reads it writes first in the same call: nothing to clear
  return fwd_launch(desc, plan, T, q, k, v, o, lse, ws, stream);
}

extern "C" spd_status spd_split_attn_bwd(const spd_attn_desc *desc, const spd_plan *plan, int64_t T, const void *q,
                                         const void *k, const void *v, const void *o, const float *lse,
                                         const void *dout, void *dq, void *dk, void *dv, void *workspace,
                                         size_t workspace_bytes, void *stream) {
  SPD_TRY(validate_common(desc, plan, T));
  if (!workspace || workspace_bytes < spd_attn_workspace_bytes(desc, plan->B, T)) return SPD_ERR_WORKSPACE;
  if (T == 0) return SPD_OK;      // no rows: the [T, ...] buffers may be NULL
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return SPD_ERR_INVALID_ARG;
  for (const void *p : {q, k, v, o, static_cast<const void *>(lse), dout, static_cast<const void *>(dq),
                        static_cast<const void *>(dk), static_cast<const void *>(dv)})
    if (!aligned16(p)) return SPD_ERR_ALIGNMENT;
  hipStream_t st = static_cast<hipStream_t>(stream);
  AttnWs w = carve(*desc, plan->B, T, workspace);
  // both lists in one launch, one block each
  TileJob qj;
  qj.rows_per_tile = dq_rows(*desc);
  qj.mode = kQueryTiles;
  qj.cap = int(w.capq);
  qj.goff = w.goff;
  qj.tmp = w.tmp;
  qj.out = w.qtiles;
  qj.n_out = w.counts;
  TileJob kj;
  kj.rows_per_tile = k_rows(*desc);
  kj.mode = kKeyTiles;
  kj.cap = int(w.capk);
  kj.goff = w.goff2;
  kj.tmp = w.tmp2;
  kj.out = w.ktiles;
  kj.n_out = w.counts + 1;
  kj.splits = w.splits;
  kj.arrivals = w.arrivals;
  kj.max_slots = w.slots;
  kj.blocks_per_tile = desc->num_kv_heads;
  kj.n_cu = device_cu_count();
  SPD_TRY(launch_build_tiles(*plan, T, qj, st, &kj));
  if (desc->dtype == SPD_F32)
    return attn_bwd_f32(*desc, *plan, T, w.qtiles, w.counts, w.capq, w.ktiles, w.counts + 1, w.capk,
                        static_cast<const float *>(q), static_cast<const float *>(k), static_cast<const float *>(v),
                        static_cast<const float *>(o), lse, static_cast<const float *>(dout),
                        static_cast<float *>(dq), static_cast<float *>(dk), static_cast<float *>(dv), w.Dbuf, st);
  return attn_bwd_bf16(*desc, *plan, T, w.qtiles, w.counts, w.capq, w.ktiles, w.counts + 1, w.capk, q, k, v, o, lse,
                       dout, dq, dk, dv, w.Dbuf, w.L2buf, w.segp, w.Tp, w.splits, w.arrivals, w.part_k, w.part_v,
                       st);
}
