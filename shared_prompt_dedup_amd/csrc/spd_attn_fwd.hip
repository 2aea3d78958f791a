// bf16 split-attention forward on CDNA4 matrix cores.
//
// How Prompt Deduplication Works -- Phase 2, "Split Attention Optimization":
// each unique prompt attends causally to itself once (prompt-to-prompt); each
// response attends to its whole prompt and to its own causal prefix
// (response-to-full).  One block handles a query tile (never straddling a
// group or the prompt/response boundary) for the query heads of one kv head:
//   phase A (response tiles only): the group's prompt keys, no causal mask;
//   phase B: keys [s0, r1) of the tile's own rows, visible iff
//            seg_start[q] <= k <= q.
//
// Block: 12 waves (three per SIMD, so two waves' MFMAs overlap the third's
// softmax); wave w owns 32 query rows of one query head.  Per 64-key tile:
// K and V are copied to LDS by direct-to-LDS loads (a pair of tiles is read
// while the next pair loads, one barrier per pair), S^T = K Q^T puts one
// query per lane column so the row
// statistics are per-lane scalars, and O^T = V^T P^T reads V^T with
// transposing LDS reads.  The running maximum moves only when a tile exceeds
// it by more than 2^8 (numerator and denominator share the reference, so this
// is exact).  One rounding of O to bf16.
#include "spd_attn_dev.h"

namespace spd {
namespace {

using namespace dev;

constexpr int kFwdWaves = 12;          // three waves per SIMD (at most 168 VGPRs each)
constexpr int kFwdLoaders = 8;         // waves that issue the tile loads: a tile's 16-byte chunks split evenly over 8
constexpr int kFwdBN = 64;
constexpr float kRescaleSlack = 8.0f;
constexpr int kReadsAhead = 3;         // MFMAs an LDS operand read runs ahead of its use

template <int D, int HPW>
__global__ void __launch_bounds__(kFwdWaves * 64) k_fwd(const Tile *__restrict__ tiles,
                                                        const int *__restrict__ ntiles, int HG, int Hq, int Hkv,
                                                        int T, const __bf16 *__restrict__ q,
                                                        const __bf16 *__restrict__ k, const __bf16 *__restrict__ v,
                                                        __bf16 *__restrict__ o, float *__restrict__ lse,
                                                        const int *__restrict__ seg_start, float scale_log2) {
  constexpr int NW = kFwdWaves, BN = kFwdBN;
  constexpr int WPH = NW / HPW;          // waves per query head
  constexpr int KS = D / 16;             // contraction steps over head_dim
  constexpr int TB = BN * D * 2;         // bytes of one K or V tile
  constexpr int SLOTS = 4;               // 64-key slots: the pair of tiles being read, the pair loading
  __shared__ __attribute__((aligned(1024))) char smem[SLOTS * 2 * TB];   // [slot][K | V]

  const int tile_rank = blockIdx.x / HG;
  if (tile_rank >= *ntiles) return;
  const int hg = blockIdx.x % HG;
  const int ratio = Hq / Hkv;
  const int sub = ratio / HPW;
  const int kvh = hg / sub;
  const Tile t = tiles[tile_rank];
  const int wave = wave_id();
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5, col = lane & 31;
  const int h = kvh * ratio + (hg % sub) * HPW + wave / WPH;
  const int qw0 = t.r0 + (wave % WPH) * 32;                 // first row of this wave
  const int qlast = min(t.r1, qw0 + 32) - 1;                 // last valid row (< qw0: no rows)
  const int qrow = qw0 + col;
  const bool qvalid = qrow < t.r1;
  const int seg_q = qvalid ? seg_start[qrow] : 0x7fffffff;
  const int seg_hi = qlast >= qw0 ? seg_start[qlast] : 0x7fffffff;

  bf16x8 qf[KS];
  {
    const __bf16 *qp = q + (int64_t(qvalid ? qrow : t.r0) * Hq + h) * D + 8 * half;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = qvalid ? ld_global8(qp + 16 * ks) : zero8();
  }
  f32x16 oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) oacc[i] = zero16();
  float m_run = -1.0e30f, l_run = 0.0f;

  // Per-lane LDS offsets.  K reads (A operand of S^T): row 32 kb + col,
  // chunk 2 ks + half.  V^T reads: 16-lane group g = lane / 16 covers d
  // columns 32 dblk + 16 (g % 2) + i and rows 16 ks + 8 w + 4 (g / 2) + s / 4
  // (w = which half of the 8 contraction slots), s = lane % 16.
  int koff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) koff[ks] = swz_off<D>(col, 2 * ks + half);
  const int grp = lane >> 4, s16 = lane & 15;
  int voff[D / 32][2];
#pragma unroll
  for (int dblk = 0; dblk < D / 32; ++dblk)
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const int row = 8 * w + 4 * (grp >> 1) + (s16 >> 2);
      const int dcol = 32 * dblk + 16 * (grp & 1) + 4 * (s16 & 3);
      voff[dblk][w] = swz_off<D>(row, dcol >> 3) + ((dcol & 7) << 1);
    }

  // Unmasked keys -- the shared prefix [v0, v1), then the group's prompt
  // [u0, u1) -- form one virtual range [0, lenA): tile i < nA starts at virtual
  // key i * BN and only its copy maps virtual rows to real ones.  Then the
  // tile's own segment from s0.
  const int lenV = t.v1 - t.v0;
  const int lenA = lenV + (t.u1 - t.u0);
  const int nA = (lenA + BN - 1) / BN;
  const int nB = (t.r1 - t.s0 + BN - 1) / BN;
  const int n = nA + nB;
  auto kt_of = [&](int i) { return i < nA ? i * BN : t.s0 + (i - nA) * BN; };

  constexpr int NL = kFwdLoaders;
  auto issue = [&](int i) {
    if (wave >= NL) return;
    char *st = smem + (i % SLOTS) * 2 * TB;
    if (i < nA) {
      dma_rows2<BN, D, NL>(st, k, kt_of(i), lenV, t.v0, t.u0, T, Hkv, kvh, wave, lane);
      dma_rows2<BN, D, NL>(st + TB, v, kt_of(i), lenV, t.v0, t.u0, T, Hkv, kvh, wave, lane);
    } else {
      dma_rows<BN, D, NL>(st, k, kt_of(i), T, Hkv, kvh, wave, lane);
      dma_rows<BN, D, NL>(st + TB, v, kt_of(i), T, Hkv, kvh, wave, lane);
    }
  };
  wait_vm_all();
  for (int i = 0; i < 2 && i < n; ++i) issue(i);

  // One barrier per pair of tiles: past it, the pair's loads (issued during
  // the previous pair) have landed for every wave, and every wave is done with
  // the previous pair, whose slots then take the next one.  The next pair's
  // first tile is issued right after the barrier, its second between this
  // pair's two tiles, so the loading waves stall on half the burst at a time.
  // Waves w, w + 4 and w + 8 share a SIMD; at equal priority issue goes to
  // the oldest, which would take every matrix-core slot it can use and then
  // wait at the barrier while the others ran on.  So the priorities rank the
  // three by age in the pair's first tile (3, 2, 1) and in reverse in the
  // second (1, 2, 3).
  const int rank = wave / 4;   // 0: the oldest wave on its SIMD
  for (int j = 0; j < (n + 1) / 2; ++j) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (rank == 0) set_prio<3>();
    else if (rank == 1) set_prio<2>();
    else set_prio<1>();
    if (2 * j + 2 < n) issue(2 * j + 2);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = 2 * j + u;
      if (u == 1) {
        if (rank == 0) set_prio<1>();
        else if (rank == 2) set_prio<3>();
        if (2 * j + 3 < n) issue(2 * j + 3);
      }
      if (i >= n) break;
      const int kt = kt_of(i);
      const bool phaseA = i < nA;
      if (qlast < qw0 || (!phaseA && kt > qlast)) continue;   // nothing this wave can see
      const char *Ks = smem + (i % SLOTS) * 2 * TB;
      const char *Vs = Ks + TB;
      const bool need_mask = phaseA ? (kt + BN > lenA) : (kt + BN - 1 > qw0 || kt < seg_hi);

      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = zero16();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) s[kb] = mfma(ld_lds8(Ks + koff[ks] + kb * 32 * D * 2), qf[ks], s[kb]);
      }
      sched_reads_ahead<kReadsAhead, 2 * KS, 1>();
      if (need_mask) {
        keep_branch();
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kt + 32 * kb + c_row(r, half);
            const bool vis = phaseA ? (key < lenA) : (key <= qrow && key >= seg_q);
            s[kb][r] = vis ? s[kb][r] : -INFINITY;
          }
      }
      float mt = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[kb][r]);
      mt = fmaxf(mt, __shfl_xor(mt, 32)) * scale_log2;
      if (__any(mt > m_run + kRescaleSlack)) {
        const float mn = fmaxf(m_run, mt);
        const float alpha = __builtin_amdgcn_exp2f(m_run - mn);
        l_run *= alpha;
#pragma unroll
        for (int d = 0; d < D / 32; ++d) oacc[d] *= alpha;
        m_run = mn;
      }
      bf16x8 pf[4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][r], scale_log2, -m_run));
          l_run += p;
          pf[2 * kb + (r >> 3)][r & 7] = static_cast<__bf16>(p);
        }
      const char *vb[D / 32][2];
#pragma unroll
      for (int dblk = 0; dblk < D / 32; ++dblk)
#pragma unroll
        for (int w = 0; w < 2; ++w) vb[dblk][w] = opaque_lds(Vs + voff[dblk][w]);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int dblk = 0; dblk < D / 32; ++dblk) {
          const bf16x8 a = ld_lds_tr_pair(vb[dblk][0] + ks * 16 * D * 2, vb[dblk][1] + ks * 16 * D * 2);
          oacc[dblk] = mfma(a, pf[ks], oacc[dblk]);
        }
      sched_reads_ahead<kReadsAhead, 4 * (D / 32), 2>();
    }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (qvalid) {
    const float inv = 1.0f / l_tot;
    __bf16 *op = o + (int64_t(qrow) * Hq + h) * D;
#pragma unroll
    for (int dblk = 0; dblk < D / 32; ++dblk)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = static_cast<__bf16>(oacc[dblk][4 * rg + e] * inv);
        *reinterpret_cast<bf16x4 *>(op + 32 * dblk + 8 * rg + 4 * half) = w;
      }
    if (half == 0) lse[int64_t(h) * T + qrow] = (m_run + __log2f(l_tot)) * kLn2;
  }
}

int fwd_heads_per_block(const spd_attn_desc &d) {
  const int ratio = d.num_q_heads / d.num_kv_heads;
  return (ratio % 4 == 0) ? 4 : (ratio % 2 == 0 ? 2 : 1);
}

}  // namespace

int fwd_bf16_rows_per_tile(const spd_attn_desc &d) { return 32 * (kFwdWaves / fwd_heads_per_block(d)); }

spd_status attn_fwd_bf16(const spd_attn_desc &d, const spd_plan &plan, int64_t T, const Tile *tiles,
                         const int *ntiles, int64_t cap, const void *q, const void *k, const void *v, void *o,
                         float *lse, hipStream_t st) {
  const int hpw = fwd_heads_per_block(d);
  const int HG = d.num_q_heads / hpw;
  const dim3 grid(static_cast<unsigned>(cap * HG));
  const dim3 block(kFwdWaves * 64);
  const float sl2 = d.softmax_scale * kLog2e;
  const auto *qq = static_cast<const __bf16 *>(q);
  const auto *kk = static_cast<const __bf16 *>(k);
  const auto *vv = static_cast<const __bf16 *>(v);
  auto *oo = static_cast<__bf16 *>(o);
  prof_start(SPD_K_FWD, st);
#define SPD_FWD_LAUNCH(DD, HH)                                                                                  \
  hipLaunchKernelGGL((k_fwd<DD, HH>), grid, block, 0, st, tiles, ntiles, HG, d.num_q_heads, d.num_kv_heads, \
                     int(T), qq, kk, vv, oo, lse, plan.seg_start, sl2)
  if (d.head_dim == 128) {
    if (hpw == 4) SPD_FWD_LAUNCH(128, 4);
    else if (hpw == 2) SPD_FWD_LAUNCH(128, 2);
    else SPD_FWD_LAUNCH(128, 1);
  } else {
    if (hpw == 4) SPD_FWD_LAUNCH(64, 4);
    else if (hpw == 2) SPD_FWD_LAUNCH(64, 2);
    else SPD_FWD_LAUNCH(64, 1);
  }
#undef SPD_FWD_LAUNCH
  SPD_LAUNCH_CHECK();
  prof_stop(SPD_K_FWD, st);
  return SPD_OK;
}

}  // namespace spd
