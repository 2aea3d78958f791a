// bf16 split-attention backward on CDNA4 matrix cores.
//
// How Prompt Deduplication Works -- "Correctness & Gradients": gradients
// flow through the deduplicated computation.  With P = softmax(scale S),
// D = rowsum(dO * O), dP = dO V^T, dS = P (dP - D):
//   dq = scale dS K,  dk = scale dS^T Q,  dv = P^T dO.
// A prompt key's dk / dv sum over the prompt's own causal queries and over
// every response row of its group; query heads sharing a kv head add into it.
//
// k_bwd_pre: D and lse / scale per (head, row), and each row's segment end.
// k_dq: one block per query tile (as the forward), K and V tiles by
//   direct-to-LDS loads, S^T = K Q^T, dP^T = V dO^T, dq^T += K^T dS^T with
//   K^T read by transposing LDS reads.  The wave raises its issue priority
//   over its matrix-core phases, so they win ties against the other wave's
//   softmax (about 2% faster than without).
// k_dkdv: one block per 256-key tile and kv head; wave w owns keys
//   [r0 + 32 w, r0 + 32 w + 32) for every query row.  K of a wave's keys stays
//   in registers, V of the tile in LDS; Q and dO tiles of 64 query rows (plus
//   their LSE, D and segment starts) arrive by direct-to-LDS loads, double
//   buffered.  S = Q K^T and dP = dO V^T put one key per lane column, so P^T
//   and dS^T feed dv += P^T dO and dk += dS^T Q directly, with dO^T and Q^T
//   read by transposing LDS reads.  Of the two waves on a SIMD, the older
//   leads each 64-row block's first half and the younger its second (issue
//   priorities).  A tile the planner cut into chunks (a
//   prompt or prefix key read by far more rows than a CU's fair share) leaves
//   fp32 partial sums in numbered slots; an arrival counter per (tile, kv
//   head) elects the last chunk to finish, which adds the slots in chunk
//   order.  No float atomics: results are bitwise repeatable.
#include "spd_attn_dev.h"

namespace spd {
namespace {

using namespace dev;

constexpr int kWaves = 8;
constexpr int kBN = 64;      // keys per tile in k_dq
constexpr int kQB = 64;      // query rows per staged block in k_dkdv
constexpr int kDkdvKeys = 256;  // keys per k_dkdv tile (8 waves x 32)

// Per (head, row): nD = -sum_d dO O and nL = -lse / scale, so that
// P = exp2(c (s + nL)) with c = scale log2(e) and s the raw score Q.K, and
// dS = P (dP + nD); score and dP accumulators can start at nL and nD.  Per
// row: send = one past the last row of the row's segment (shared prefix, prompt
// or response).
// D and Ls have a row stride of Tp >= T + 64 so that 64-row blocks starting
// below T never leave them; the padding rows are set to 0 and every reader
// masks them.
// One block per (32-row chunk, group of HG heads): the block reads its rows'
// HG heads as contiguous runs of (row, head) pairs, stages the sums in LDS and
// writes each head's 32 rows of D and Ls as one 128-byte line, so no line is
// shared between blocks that may run on different XCDs.
template <int D>
__global__ void __launch_bounds__(256) k_bwd_pre(int Hq, int HG, int T, int Tp, float inv_scale,
                                                 const __bf16 *__restrict__ o, const __bf16 *__restrict__ dout,
                                                 const float *__restrict__ lse, spd_plan plan,
                                                 float *__restrict__ Dbuf, float *__restrict__ Lbuf,
                                                 int *__restrict__ send) {
  constexpr int LPR = D / 8;              // lanes per (row, head)
  constexpr int PPP = 256 / LPR;          // (row, head) pairs per pass of the block
  constexpr int R = 32;                   // rows per block
  __shared__ float sD[16 * R];
  const int ngrp = Hq / HG;
  const int h0 = (blockIdx.x % ngrp) * HG;
  const int r0 = (blockIdx.x / ngrp) * R;
  const int sub = threadIdx.x % LPR;
  // U passes' loads are issued before their reductions, so a thread keeps 2U
  // loads in flight; rows past T read row 0 (T >= 1) and count as zero, and
  // pairs past the block's R * HG load nothing.
  constexpr int U = 4;
  for (int p0 = 0; p0 < R * HG; p0 += U * PPP) {
    bf16x8 a[U], b[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p = p0 + u * PPP + threadIdx.x / LPR;   // pair: row r0 + p / HG, head h0 + p % HG
      const int row = r0 + p / HG, hh = p % HG;
      const int64_t off = (int64_t(row < T ? row : 0) * Hq + h0 + hh) * D + sub * 8;
      if (p < R * HG) {   // a block's last pass may hold fewer pairs than the pass has slots
        a[u] = ld_global8(o + off);
        b[u] = ld_global8(dout + off);
      } else {
        a[u] = zero8();
        b[u] = zero8();
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p = p0 + u * PPP + threadIdx.x / LPR;
      const int row = r0 + p / HG, hh = p % HG;
      float s = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) s = fmaf(static_cast<float>(a[u][e]), static_cast<float>(b[u][e]), s);
      s = row < T ? s : 0.0f;
#pragma unroll
      for (int off = LPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
      if (sub == 0 && p < R * HG) sD[hh * R + p / HG] = -s;
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < HG * R; idx += blockDim.x) {
    const int hh = idx / R, row = r0 + idx % R;
    const int64_t at = int64_t(h0 + hh) * Tp + row;
    if (row < T) {
      Dbuf[at] = sD[idx];
      Lbuf[at] = -lse[int64_t(h0 + hh) * T + row] * inv_scale;
    } else if (row < Tp) {       // padding rows [T, Tp) read as zeros
      Dbuf[at] = 0.0f;
      Lbuf[at] = 0.0f;
    }
  }
  if (h0 == 0 && threadIdx.x < R) {
    const int row = r0 + static_cast<int>(threadIdx.x);
    if (row < T) {
      const int src = plan.src[row];
      const int b = static_cast<int>(src / plan.S);
      const int64_t t = src - int64_t(b) * plan.S;
      int end;
      if (t < plan.counts[4]) {
        end = plan.counts[5];          // a row of the shared prefix
      } else if (t < plan.P) {
        const int g = plan.group_of[b];
        end = plan.prompt_off[g] + plan.prompt_len[g];
      } else {
        end = plan.resp_off[b] + plan.resp_len[b];
      }
      send[row] = end;
    }
  }
}

// ---------------------------------------------------------------------------- dq

template <int D, int HPW>
__global__ void __launch_bounds__(kWaves * 64) k_dq(const Tile *__restrict__ tiles, const int *__restrict__ ntiles,
                                                    int HG, int Hq, int Hkv, int T, const __bf16 *__restrict__ q,
                                                    const __bf16 *__restrict__ k, const __bf16 *__restrict__ v,
                                                    const float *__restrict__ Lbuf,
                                                    const __bf16 *__restrict__ dout, const float *__restrict__ Dbuf,
                                                    int Tp, __bf16 *__restrict__ dq,
                                                    const int *__restrict__ seg_start, float scale_log2,
                                                    float scale) {
  constexpr int NW = kWaves, BN = kBN;
  constexpr int WPH = NW / HPW;
  constexpr int KS = D / 16;
  constexpr int TB = BN * D * 2;
  constexpr int STAGES = 3;
  constexpr int PER = 2 * (BN * D / 8) / (NW * 64);
  __shared__ __attribute__((aligned(1024))) char smem[STAGES * 2 * TB];   // [stage][K | V]

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
  const int qw0 = t.r0 + (wave % WPH) * 32;
  const int qlast = min(t.r1, qw0 + 32) - 1;
  const int qrow = qw0 + col;
  const bool qvalid = qrow < t.r1;
  const int seg_q = qvalid ? seg_start[qrow] : 0x7fffffff;
  const int seg_hi = qlast >= qw0 ? seg_start[qlast] : 0x7fffffff;
  // P = exp2(c s + s_bias), dS = P (dP + dp_bias) with s_bias = -c lse/scale
  // = -lse log2(e) and dp_bias = -D (the arrays hold -lse/scale and -D); the
  // dP accumulator starts at dp_bias, so the MFMA adds it
  const float s_bias = qvalid ? Lbuf[int64_t(h) * Tp + qrow] * scale_log2 : 0.0f;
  const float dp_bias = qvalid ? Dbuf[int64_t(h) * Tp + qrow] : 0.0f;

  bf16x8 qf[KS], df[KS];
  {
    const int64_t off = (int64_t(qvalid ? qrow : t.r0) * Hq + h) * D + 8 * half;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks] = qvalid ? ld_global8(q + off + 16 * ks) : zero8();
      df[ks] = qvalid ? ld_global8(dout + off + 16 * ks) : zero8();
    }
  }
  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = zero16();

  int roff[KS];   // row reads of K / V: row 32 kb + col, chunk 2 ks + half
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) roff[ks] = swz_off<D>(col, 2 * ks + half);
  const int grp = lane >> 4, s16 = lane & 15;
  int toff[D / 32][2];   // K^T reads (transposing)
#pragma unroll
  for (int dblk = 0; dblk < D / 32; ++dblk)
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const int row = 8 * w + 4 * (grp >> 1) + (s16 >> 2);
      const int dcol = 32 * dblk + 16 * (grp & 1) + 4 * (s16 & 3);
      toff[dblk][w] = swz_off<D>(row, dcol >> 3) + ((dcol & 7) << 1);
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

  auto issue = [&](int i) {
    char *st = smem + (i % STAGES) * 2 * TB;
    if (i < nA) {
      dma_rows2<BN, D, NW>(st, k, kt_of(i), lenV, t.v0, t.u0, T, Hkv, kvh, wave, lane);
      dma_rows2<BN, D, NW>(st + TB, v, kt_of(i), lenV, t.v0, t.u0, T, Hkv, kvh, wave, lane);
    } else {
      dma_rows<BN, D, NW>(st, k, kt_of(i), T, Hkv, kvh, wave, lane);
      dma_rows<BN, D, NW>(st + TB, v, kt_of(i), T, Hkv, kvh, wave, lane);
    }
  };
  wait_vm_all();
  for (int i = 0; i < STAGES - 1 && i < n; ++i) issue(i);

  for (int i = 0; i < n; ++i) {
    wait_ring<STAGES, PER>(i, n);
    if (i + STAGES - 1 < n) issue(i + STAGES - 1);
    const int kt = kt_of(i);
    const bool phaseA = i < nA;
    if (qlast < qw0 || (!phaseA && kt > qlast)) continue;
    const char *Ks = smem + (i % STAGES) * 2 * TB;
    const char *Vs = Ks + TB;
    const bool need_mask = phaseA ? (kt + BN > lenA) : (kt + BN - 1 > qw0 || kt < seg_hi);
    const char *kb_[D / 32][2];   // K^T read bases of this tile
#pragma unroll
    for (int dblk = 0; dblk < D / 32; ++dblk)
#pragma unroll
      for (int w = 0; w < 2; ++w) kb_[dblk][w] = opaque_lds(Ks + toff[dblk][w]);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 s = zero16(), dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) dp[r] = dp_bias;   // the dP accumulator starts at -D
      __builtin_amdgcn_s_setprio(1);   // matrix-core phases win issue ties against the other wave's softmax
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s = mfma(ld_lds8(Ks + roff[ks] + kb * 32 * D * 2), qf[ks], s);
        dp = mfma(ld_lds8(Vs + roff[ks] + kb * 32 * D * 2), df[ks], dp);
      }
      sched_reads_ahead<3, 2 * KS, 1>();
      __builtin_amdgcn_s_setprio(0);
      if (need_mask) {
        keep_branch();
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kt + 32 * kb + c_row(r, half);
          const bool vis = phaseA ? (key < lenA) : (key <= qrow && key >= seg_q);
          s[r] = vis ? s[r] : -INFINITY;
        }
      }
      bf16x8 dsf[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[r], scale_log2, s_bias));
        dsf[r >> 3][r & 7] = static_cast<__bf16>(p * dp[r]);
      }
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int ks = 2 * kb + j;
#pragma unroll
        for (int dblk = 0; dblk < D / 32; ++dblk) {
          const bf16x8 a = ld_lds_tr_pair(kb_[dblk][0] + ks * 16 * D * 2, kb_[dblk][1] + ks * 16 * D * 2);
          acc[dblk] = mfma(a, dsf[j], acc[dblk]);
        }
      }
      sched_reads_ahead<2, 2 * (D / 32), 2>();
      __builtin_amdgcn_s_setprio(0);
    }
  }

  if (qvalid) {
    __bf16 *op = dq + (int64_t(qrow) * Hq + h) * D;
#pragma unroll
    for (int dblk = 0; dblk < D / 32; ++dblk)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = static_cast<__bf16>(acc[dblk][4 * rg + e] * scale);
        *reinterpret_cast<bf16x4 *>(op + 32 * dblk + 8 * rg + 4 * half) = w;
      }
  }
}

// ---------------------------------------------------------------------------- dk / dv

// Direct-to-LDS copy of one per-row float array for query rows [r0, r0 + 64):
// 16 lanes x 16 bytes.  r0 < T and the arrays' row stride Tp >= T + 64 keep
// the read inside them.
__device__ inline void dma_scalars(char *dst, const float *src, int lane) {
  if (lane < 16) dma16(src, static_cast<unsigned>(lane) * 16, dst);
}

template <int D>
__global__ void __launch_bounds__(kWaves * 64) k_dkdv(const Tile *__restrict__ tiles, const int *__restrict__ ntiles,
                                                      int Hq, int Hkv, int T, const __bf16 *__restrict__ q,
                                                      const __bf16 *__restrict__ k, const __bf16 *__restrict__ v,
                                                      const float *__restrict__ Lbuf,
                                                      const __bf16 *__restrict__ dout,
                                                      const float *__restrict__ Dbuf,
                                                      const int *__restrict__ send, int Tp, __bf16 *__restrict__ dk,
                                                      __bf16 *__restrict__ dv, const SplitGroup *__restrict__ splits,
                                                      int *__restrict__ arrivals, float *__restrict__ part_k,
                                                      float *__restrict__ part_v, float scale_log2, float scale) {
  constexpr int NW = kWaves, QB = kQB, BK = kDkdvKeys;   // 64 query rows per block, 256 keys per tile
  constexpr int KS = D / 16;
  constexpr int TB = QB * D * 2;                    // one Q or dO tile
  constexpr int STAGE = 2 * TB + 512;               // Q | dO | lse/scale, D (256 B each)
  constexpr int STAGES = 2;
  constexpr int PER = 2 * (QB * D / 8) / (NW * 64); // direct-to-LDS tile loads per wave per block
  constexpr int VT = BK * D * 2;                    // V rows of the tile's keys
  __shared__ __attribute__((aligned(1024))) char smem[STAGES * STAGE + VT];

  const int tile_rank = blockIdx.x / Hkv;
  if (tile_rank >= *ntiles) return;
  const int kvh = blockIdx.x % Hkv;
  const Tile t = tiles[tile_rank];
  const int wave = wave_id();
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5, col = lane & 31;
  const int kmin = t.r0 + 32 * wave;        // this wave's keys: kmin .. kmin + 31
  const int key = kmin + col;               // this lane's key column
  const bool kvalid = key < t.r1;
  const int ratio = Hq / Hkv;
  char *Vt = smem + STAGES * STAGE;
  // A masked query row sees this key iff key <= row < end of the key's segment
  // (a prompt key's masked rows are its own prompt's; a response key's are its
  // own response's).
  const int kend = kvalid ? send[key] : 0;
  // Segment ends never decrease with the key, so lane 0's (the wave's first
  // key) is the smallest; kmax is the wave's last valid key.
  const int kend0 = __builtin_amdgcn_readfirstlane(kend);
  const int kmax = min(kmin + 31, t.r1 - 1);

  bf16x8 kf[KS];
  {
    const int64_t off = (int64_t(kvalid ? key : t.r0) * Hkv + kvh) * D + 8 * half;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kf[ks] = kvalid ? ld_global8(k + off + 16 * ks) : zero8();
  }
  wait_vm_all();
  dma_rows<BK, D, NW>(Vt, v, t.r0, T, Hkv, kvh, wave, lane);
  f32x16 dka[D / 32], dva[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    dka[i] = zero16();
    dva[i] = zero16();
  }

  // A-operand row reads of Q / dO: row 32 m + col, chunk 2 ks + half (m = 32-row
  // half of the block, an immediate offset).  The V rows of this wave's keys
  // (row 32 wave + col) share the low row bits, so the same offsets apply.
  int roff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) roff[ks] = swz_off<D>(col, 2 * ks + half);
  const char *Vw = Vt + 32 * wave * D * 2;
  // dO^T / Q^T reads (transposing): rows 32 m + 16 j + 8 w + 4 (grp / 2) + s16 / 4
  const int grp = lane >> 4, s16 = lane & 15;
  int toff[D / 32][2];
#pragma unroll
  for (int dblk = 0; dblk < D / 32; ++dblk)
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const int row = 8 * w + 4 * (grp >> 1) + (s16 >> 2);
      const int dcol = 32 * dblk + 16 * (grp & 1) + 4 * (s16 & 3);
      toff[dblk][w] = swz_off<D>(row, dcol >> 3) + ((dcol & 7) << 1);
    }

  // Block order, per query head: the group's response rows (unmasked, the same
  // blocks for every prompt key tile of the group), then the masked rows from
  // the top down, so concurrently running tiles sweep the same rows together.
  const int nA = (t.u1 - t.u0 + QB - 1) / QB;   // masked query rows [u0, u1)
  const int nB = (t.e0 - t.s0 + QB - 1) / QB;   // unmasked query rows [s0, e0)
  const int nper = nA + nB;
  const int n = nper * ratio;
  auto blk_of = [&](int i, int &h, int &qb, bool &masked, int &qend) {
    const int hh = i / nper, j = i % nper;
    h = kvh * ratio + hh;
    masked = j >= nB;
    qb = masked ? t.u0 + (nper - 1 - j) * QB : t.s0 + j * QB;
    qend = masked ? t.u1 : t.e0;
  };
  auto issue = [&](int i) {
    int h, qb, qend;
    bool masked;
    blk_of(i, h, qb, masked, qend);
    // The younger wave of each SIMD issues the loads, each two waves' share:
    // the older leads the block's first half and starts its MFMAs at once.
    const int lw = wave - NW / 2;
    if (lw < 0) return;
    char *st = smem + (i % STAGES) * STAGE;
    dma_rows<QB, D, NW / 2>(st, q, qb, T, Hq, h, lw, lane);
    dma_rows<QB, D, NW / 2>(st + TB, dout, qb, T, Hq, h, lw, lane);
    if (lw == 0) dma_scalars(st + 2 * TB, Lbuf + int64_t(h) * Tp + qb, lane);
    if (lw == 1) dma_scalars(st + 2 * TB + 256, Dbuf + int64_t(h) * Tp + qb, lane);
  };

  // Waves w and w + NW / 2 share a SIMD, and at equal priority issue goes to
  // the older: wave w would take every matrix-core slot it can use, finish the
  // block first and wait at the barrier while its partner ran alone.  So the
  // older wave leads the block's first 32-row half (priority 2 over its
  // partner's 1) and yields in the second (0).
  const bool older = wave < NW / 2;
  if (!older) set_prio<1>();
  for (int i = 0; i < STAGES - 1 && i < n; ++i) issue(i);
  for (int i = 0; i < n; ++i) {
    // with two stages the ring waits for every load of the issuing waves
    static_assert(STAGES == 2, "the loading waves issue two waves' share: a deeper ring needs its own count");
    wait_ring<STAGES, PER>(i, n);
    if (older) set_prio<2>();
    if (i + STAGES - 1 < n) issue(i + STAGES - 1);
    int h, qb, qend;
    bool masked;
    blk_of(i, h, qb, masked, qend);
    if (masked && qb + QB - 1 < kmin) continue;     // every row of the block precedes every key
    const char *Qs = smem + (i % STAGES) * STAGE;
    const char *Ds = Qs + TB;
    const char *sL = Qs + 2 * TB;        // float entry e = row qb + e: lse / scale
    const char *sD = Qs + 2 * TB + 256;  // D
#pragma unroll
    for (int m = 0; m < QB / 32; ++m) {
      if (m == 1 && older) set_prio<0>();
      const int row0 = qb + 32 * m;
      if (row0 >= qend || (masked && row0 + 31 < kmin)) continue;
      const char *Qm = Qs + 32 * m * D * 2;
      const char *Dm = Ds + 32 * m * D * 2;
      // accumulators start at -lse/scale and -D of their rows: register r holds
      // row 32 m + 8 (r / 4) + 4 half + r % 4, four consecutive rows per group
      f32x16 s, dp;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int e = 32 * m + 8 * g + 4 * half;
        const f32x4 l4 = *reinterpret_cast<const f32x4 *>(sL + 4 * e);
        const f32x4 d4 = *reinterpret_cast<const f32x4 *>(sD + 4 * e);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          s[4 * g + j] = l4[j];
          dp[4 * g + j] = d4[j];
        }
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s = mfma(ld_lds8(Qm + roff[ks]), kf[ks], s);
        dp = mfma(ld_lds8(Dm + roff[ks]), ld_lds8(Vw + roff[ks]), dp);
      }
      // the 8 statistics reads, then Q / dO / V operands two steps (4 MFMAs) ahead
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 8 + 3 * 2, 0);
#pragma unroll
      for (int j = 0; j < KS - 2; ++j) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 3, 0);
      }
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 4, 0);
      // every (row, key) of the 32 x 32 block visible: rows inside the range,
      // and for masked rows all past the wave's last key and before the
      // earliest segment end among its keys
      const bool full = row0 + 31 < qend && (!masked || (row0 >= kmax && row0 + 31 < kend0));
      if (!full) {
        keep_branch();
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = row0 + c_row(r, half);
          bool vis = row < qend;
          if (masked) vis = vis && key <= row && row < kend;
          s[r] = vis ? s[r] : -INFINITY;
        }
      }
      bf16x8 pf[2], dsf[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(s[r] * scale_log2);
        pf[r >> 3][r & 7] = static_cast<__bf16>(p);
        dsf[r >> 3][r & 7] = static_cast<__bf16>(p * dp[r]);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int dblk = 0; dblk < D / 32; ++dblk) {
          const int o0 = toff[dblk][0] + (32 * m + 16 * j) * D * 2;
          const int o1 = toff[dblk][1] + (32 * m + 16 * j) * D * 2;
          const bf16x8 bdo = ld_lds_tr_pair(Ds + o0, Ds + o1);
          const bf16x8 bq = ld_lds_tr_pair(Qs + o0, Qs + o1);
          dva[dblk] = mfma(pf[j], bdo, dva[dblk]);
          dka[dblk] = mfma(dsf[j], bq, dka[dblk]);
        }
      sched_reads_ahead<2, 4 * (D / 32), 2>();
    }
  }

  // dv / dk: register r of dblk holds key row c_row(r, half) of the wave's 32
  // keys and column 32 dblk + col.  A chunk of a split tile leaves unscaled
  // fp32 sums in its slot instead; the tile's last chunk to arrive (for this kv
  // head) adds all its chunks' slots in chunk order.
  if (t.slot >= 0) {
    const int64_t sbase = (int64_t(t.slot) * Hkv + kvh) * BK;
#pragma unroll
    for (int dblk = 0; dblk < D / 32; ++dblk)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kr = 32 * wave + c_row(r, half);
        if (t.r0 + kr < t.r1) {
          const int64_t off = (sbase + kr) * D + 32 * dblk + col;
          part_k[off] = dka[dblk][r];
          part_v[off] = dva[dblk][r];
        }
      }
    __shared__ int is_last;
    const SplitGroup g = splits[t.grp];
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) is_last = atomicAdd(&arrivals[t.grp * Hkv + kvh], 1) == g.n - 1;
    __syncthreads();
    if (!is_last) return;
    __threadfence();
    constexpr int C4 = D / 4;
    const int64_t stride = int64_t(Hkv) * BK * D;   // one slot
    const int64_t src0 = (int64_t(g.slot0) * Hkv + kvh) * BK * D;
    for (int e = threadIdx.x; e < (t.r1 - t.r0) * C4; e += NW * 64) {
      const int kr = e / C4, c = 4 * (e % C4);
      const int64_t src = src0 + int64_t(kr) * D + c;
      f32x4 sk = *reinterpret_cast<const f32x4 *>(part_k + src);
      f32x4 sv = *reinterpret_cast<const f32x4 *>(part_v + src);
      for (int j = 1; j < g.n; ++j) {
        sk += *reinterpret_cast<const f32x4 *>(part_k + src + j * stride);
        sv += *reinterpret_cast<const f32x4 *>(part_v + src + j * stride);
      }
      const int64_t dst = (int64_t(t.r0 + kr) * Hkv + kvh) * D + c;
      bf16x4 ok, ov;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ok[i] = static_cast<__bf16>(sk[i] * scale);
        ov[i] = static_cast<__bf16>(sv[i]);
      }
      *reinterpret_cast<bf16x4 *>(dk + dst) = ok;
      *reinterpret_cast<bf16x4 *>(dv + dst) = ov;
    }
    return;
  }
#pragma unroll
  for (int dblk = 0; dblk < D / 32; ++dblk)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kk = kmin + c_row(r, half);
      if (kk < t.r1) {
        const int64_t off = (int64_t(kk) * Hkv + kvh) * D + 32 * dblk + col;
        dk[off] = static_cast<__bf16>(dka[dblk][r] * scale);
        dv[off] = static_cast<__bf16>(dva[dblk][r]);
      }
    }
}

int bwd_heads_per_block(const spd_attn_desc &d) {
  const int ratio = d.num_q_heads / d.num_kv_heads;
  return (ratio % 4 == 0) ? 4 : (ratio % 2 == 0 ? 2 : 1);
}

}  // namespace

int dq_bf16_rows_per_tile(const spd_attn_desc &d) { return 32 * (kWaves / bwd_heads_per_block(d)); }
int dkdv_bf16_rows_per_tile(const spd_attn_desc &) { return kDkdvKeys; }

spd_status attn_bwd_bf16(const spd_attn_desc &d, const spd_plan &plan, int64_t T, const Tile *qtiles, const int *nq,
                         int64_t capq, const Tile *ktiles, const int *nk, int64_t capk, const void *q, const void *k,
                         const void *v, const void *o, const float *lse, const void *dout, void *dq, void *dk,
                         void *dv, float *Dbuf, float *Lbuf, int *send, int64_t Tp, const SplitGroup *splits,
                         int *arrivals, float *part_k, float *part_v, hipStream_t st) {
  const auto *qq = static_cast<const __bf16 *>(q);
  const auto *kk = static_cast<const __bf16 *>(k);
  const auto *vv = static_cast<const __bf16 *>(v);
  const auto *oo = static_cast<const __bf16 *>(o);
  const auto *dd = static_cast<const __bf16 *>(dout);
  // Heads per block: the largest divisor of Hq up to 2.  Small blocks keep
  // the last round of the grid short (16 heads per block left a second round
  // of about 1/7 of the blocks on the 32K-prompt batch: 2 heads are 8% faster,
  // 1 head 16% slower).
  int hg = 2;
  while (d.num_q_heads % hg) --hg;
  // blocks cover rows [0, Tp): the padding rows are written as zeros
  const dim3 gpre(static_cast<unsigned>((Tp + 31) / 32 * (d.num_q_heads / hg)));
  prof_start(SPD_K_BWD_PRE, st);
  if (d.head_dim == 128)
    hipLaunchKernelGGL(k_bwd_pre<128>, gpre, dim3(256), 0, st, d.num_q_heads, hg, int(T), int(Tp),
                       1.0f / d.softmax_scale, oo, dd, lse, plan, Dbuf, Lbuf, send);
  else
    hipLaunchKernelGGL(k_bwd_pre<64>, gpre, dim3(256), 0, st, d.num_q_heads, hg, int(T), int(Tp),
                       1.0f / d.softmax_scale, oo, dd, lse, plan, Dbuf, Lbuf, send);
  SPD_LAUNCH_CHECK();
  prof_stop(SPD_K_BWD_PRE, st);

  const int hpw = bwd_heads_per_block(d);
  const int HG = d.num_q_heads / hpw;
  const float sl2 = d.softmax_scale * kLog2e;
  const dim3 block(kWaves * 64);
  const dim3 gq(static_cast<unsigned>(capq * HG));
  const dim3 gk(static_cast<unsigned>(capk * d.num_kv_heads));
  auto *dqq = static_cast<__bf16 *>(dq);
  auto *dkk = static_cast<__bf16 *>(dk);
  auto *dvv = static_cast<__bf16 *>(dv);
  prof_start(SPD_K_BWD_DQ, st);
#define SPD_DQ_LAUNCH(DD, HH)                                                                                     \
  hipLaunchKernelGGL((k_dq<DD, HH>), gq, block, 0, st, qtiles, nq, HG, d.num_q_heads, d.num_kv_heads, int(T), qq, \
                     kk, vv, Lbuf, dd, Dbuf, int(Tp), dqq, plan.seg_start, sl2, d.softmax_scale)
  if (d.head_dim == 128) {
    if (hpw == 4) SPD_DQ_LAUNCH(128, 4);
    else if (hpw == 2) SPD_DQ_LAUNCH(128, 2);
    else SPD_DQ_LAUNCH(128, 1);
  } else {
    if (hpw == 4) SPD_DQ_LAUNCH(64, 4);
    else if (hpw == 2) SPD_DQ_LAUNCH(64, 2);
    else SPD_DQ_LAUNCH(64, 1);
  }
#undef SPD_DQ_LAUNCH
  SPD_LAUNCH_CHECK();
  prof_stop(SPD_K_BWD_DQ, st);
  prof_start(SPD_K_BWD_DKDV, st);
  if (d.head_dim == 128)
    hipLaunchKernelGGL(k_dkdv<128>, gk, block, 0, st, ktiles, nk, d.num_q_heads, d.num_kv_heads, int(T), qq, kk, vv,
                       Lbuf, dd, Dbuf, send, int(Tp), dkk, dvv, splits, arrivals, part_k, part_v, sl2,
                       d.softmax_scale);
  else
    hipLaunchKernelGGL(k_dkdv<64>, gk, block, 0, st, ktiles, nk, d.num_q_heads, d.num_kv_heads, int(T), qq, kk, vv,
                       Lbuf, dd, Dbuf, send, int(Tp), dkk, dvv, splits, arrivals, part_k, part_v, sl2,
                       d.softmax_scale);
  SPD_LAUNCH_CHECK();
  prof_stop(SPD_K_BWD_DKDV, st);
  return SPD_OK;
}

}  // namespace spd
