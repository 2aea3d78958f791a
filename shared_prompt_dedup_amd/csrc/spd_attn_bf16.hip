// bf16 split attention on CDNA4 matrix cores (v_mfma_f32_32x32x16_bf16).
//
// How Prompt Deduplication Works -- Phase 2, "Split Attention Optimization";
// "Correctness & Gradients".  Each unique prompt attends causally to itself
// once; each response attends to its whole prompt and its own causal prefix;
// prompt keys collect dk / dv from their own causal queries and from every
// response of the group.
//
// MFMA 32x32x16 (wave64): lane l supplies row (l % 32) of A and column
// (l % 32) of B, each as 8 bf16 along the contraction; the fp32 result holds
// C[8 (r / 4) + 4 (l / 32) + (r % 4)][l % 32] in register r.  A result used
// again as an operand (probabilities P, dS) therefore lives as rows
// {4h..4h+3, 8+4h..8+4h+3} (h = l / 32) of each 16-wide contraction step,
// and the other operand of that product is laid out in LDS with each
// 16-group's middle two quads swapped so that a lane reads its 8 matching
// rows as one 16-byte vector.  That operand is the transpose of a row-major
// tile (V^T in the forward, K^T for dq, Q^T and dO^T for dk / dv); it is
// transposed on the way into LDS.
//
// Forward: S^T = K Q^T keeps one query per lane column, so the softmax row
// statistics are per-lane scalars (one cross-half max per key tile, the row
// sum combined once at the end), and O^T = V^T P^T accumulates in place.
// The running maximum is only moved when a tile's maximum exceeds it by more
// than 2^8 (exact: numerator and denominator share the reference).
#include "spd_attn.h"

namespace spd {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kNeg = -1.0e30f;      // score of a key a row does not see
constexpr float kVisibleFloor = -1.0e29f;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ inline f32x16 mfma(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ inline bf16x8 zero8() {
  bf16x8 z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = static_cast<__bf16>(0.0f);
  return z;
}

__device__ inline f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.0f;
  return z;
}

__device__ inline bf16x8 ld8(const __bf16 *p) { return *reinterpret_cast<const bf16x8 *>(p); }
__device__ inline bf16x8 lds8(const char *p) { return *reinterpret_cast<const bf16x8 *>(p); }

// Row (0..15) of a 16-row group after swapping its middle two quads.
__device__ inline int quad_perm(int quad) { return (quad == 1) ? 2 : (quad == 2 ? 1 : quad); }

// Row of register r of a 32x32 result, for lane half h.
__device__ inline int c_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// Copies rows [r0, r0 + ROWS) of a [*, H, D] tensor (head hh) into LDS,
// row-major with a byte stride of STR.  Rows >= T read as zero.
template <int ROWS, int D, int STR, int NT>
__device__ inline void stage_rows(char *dst, const __bf16 *src, int r0, int T, int H, int hh) {
  constexpr int CPR = D / 8;
  for (int c = threadIdx.x; c < ROWS * CPR; c += NT) {
    const int r = c / CPR, c8 = c % CPR;
    const int row = r0 + r;
    bf16x8 val = row < T ? ld8(src + (int64_t(row) * H + hh) * D + c8 * 8) : zero8();
    *reinterpret_cast<bf16x8 *>(dst + r * STR + c8 * 16) = val;
  }
}

// Copies the same rows transposed: dst[d][perm(row)] with a byte stride of
// STR per d, 4 rows x 8 columns per thread, written as 8-byte vectors.
template <int ROWS, int D, int STR, int NT>
__device__ inline void stage_rows_t(char *dst, const __bf16 *src, int r0, int T, int H, int hh) {
  constexpr int CPR = D / 8;
  for (int c = threadIdx.x; c < (ROWS / 4) * CPR; c += NT) {
    const int rq = c / CPR, dc = c % CPR;
    bf16x8 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = r0 + 4 * rq + i;
      v[i] = row < T ? ld8(src + (int64_t(row) * H + hh) * D + dc * 8) : zero8();
    }
    const int pos = 16 * (rq >> 2) + 4 * quad_perm(rq & 3);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      bf16x4 col4 = {v[0][e], v[1][e], v[2][e], v[3][e]};
      *reinterpret_cast<bf16x4 *>(dst + (dc * 8 + e) * STR + pos * 2) = col4;
    }
  }
}

constexpr int kThreads = 256;   // 4 waves
constexpr int kBN = 64;         // keys per LDS tile

// ---------------------------------------------------------------------------
// Backward preprocess: Dbuf[h, row] = sum_d dO[row, h, d] O[row, h, d]
// ---------------------------------------------------------------------------

template <int D>
__global__ void __launch_bounds__(256) k_rowdot_bf16(int64_t rows_x_heads, int Hq, int T, const __bf16 *__restrict__ o,
                                                     const __bf16 *__restrict__ dout, float *__restrict__ Dbuf) {
  constexpr int LPR = D / 8;          // lanes per (row, head)
  constexpr int RPW = 64 / LPR;       // (row, head) pairs per wave
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  const int64_t i = wave * RPW + lane / LPR;
  const int sub = lane % LPR;
  float s = 0.0f;
  if (i < rows_x_heads) {
    const bf16x8 a = ld8(o + i * D + sub * 8);
    const bf16x8 b = ld8(dout + i * D + sub * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) s = fmaf(static_cast<float>(a[e]), static_cast<float>(b[e]), s);
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
  if (i < rows_x_heads && sub == 0) {
    const int64_t row = i / Hq;
    const int h = static_cast<int>(i % Hq);
    Dbuf[int64_t(h) * T + row] = s;
  }
}

// ---------------------------------------------------------------------------
// dq: per query tile, over the same keys as the forward.
//   S^T = K Q^T, dP^T = V dO^T, dS^T = P^T (dP^T - D), dq^T += K^T dS^T.
// ---------------------------------------------------------------------------

template <int D, int HPW>
__global__ void __launch_bounds__(kThreads) k_dq_bf16(const Tile *__restrict__ tiles, const int *__restrict__ ntiles,
                                                      int HG, int Hq, int Hkv, int T, const __bf16 *__restrict__ q,
                                                      const __bf16 *__restrict__ k, const __bf16 *__restrict__ v,
                                                      const float *__restrict__ lse, const __bf16 *__restrict__ dout,
                                                      const float *__restrict__ Dbuf, __bf16 *__restrict__ dq,
                                                      const int *__restrict__ seg_start, float scale_log2,
                                                      float scale) {
  constexpr int WPH = 4 / HPW;
  constexpr int KS = D / 16;
  constexpr int KSTR = D * 2 + 16;
  constexpr int TSTR = kBN * 2 + 16;
  __shared__ __attribute__((aligned(16))) char smem[2 * kBN * KSTR + D * TSTR];
  char *Ks = smem;
  char *Vs = smem + kBN * KSTR;
  char *Kt = smem + 2 * kBN * KSTR;

  const int tile_rank = blockIdx.x / HG;
  if (tile_rank >= *ntiles) return;
  const int hg = blockIdx.x % HG;
  const int ratio = Hq / Hkv;
  const int sub = ratio / HPW;
  const int kvh = hg / sub;
  const Tile t = tiles[tile_rank];
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int half = lane >> 5, col = lane & 31;
  const int h = kvh * ratio + (hg % sub) * HPW + wave / WPH;
  const int qrow = t.r0 + (wave % WPH) * 32 + col;
  const bool qvalid = qrow < t.r1;
  const int seg_q = qvalid ? seg_start[qrow] : 0x7fffffff;
  const float lse2 = qvalid ? lse[int64_t(h) * T + qrow] * kLog2e : 0.0f;
  const float Dq = qvalid ? Dbuf[int64_t(h) * T + qrow] : 0.0f;

  bf16x8 qf[KS], df[KS];
  {
    const int64_t off = (int64_t(qvalid ? qrow : t.r0) * Hq + h) * D + 8 * half;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks] = qvalid ? ld8(q + off + 16 * ks) : zero8();
      df[ks] = qvalid ? ld8(dout + off + 16 * ks) : zero8();
    }
  }
  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = zero16();

  auto process = [&](int kt, bool prompt_keys, int klim) {
    __syncthreads();
    stage_rows<kBN, D, KSTR, kThreads>(Ks, k, kt, T, Hkv, kvh);
    stage_rows<kBN, D, KSTR, kThreads>(Vs, v, kt, T, Hkv, kvh);
    stage_rows_t<kBN, D, TSTR, kThreads>(Kt, k, kt, T, Hkv, kvh);
    __syncthreads();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 s = zero16(), dp = zero16();
      const char *kp = Ks + (32 * kb + col) * KSTR + 16 * half;
      const char *vp = Vs + (32 * kb + col) * KSTR + 16 * half;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s = mfma(lds8(kp + 32 * ks), qf[ks], s);
        dp = mfma(lds8(vp + 32 * ks), df[ks], dp);
      }
      bf16x8 dsf[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kt + 32 * kb + c_row(r, half);
        const bool vis = qvalid && (prompt_keys ? (key < klim) : (key <= qrow && key >= seg_q));
        const float p = vis ? exp2f(s[r] * scale_log2 - lse2) : 0.0f;
        dsf[r >> 3][r & 7] = static_cast<__bf16>(p * (dp[r] - Dq));
      }
#pragma unroll
      for (int dblk = 0; dblk < D / 32; ++dblk) {
        const char *ap = Kt + (32 * dblk + col) * TSTR + 16 * half + 64 * kb;
        acc[dblk] = mfma(lds8(ap), dsf[0], acc[dblk]);
        acc[dblk] = mfma(lds8(ap + 32), dsf[1], acc[dblk]);
      }
    }
  };

  for (int kt = t.u0; kt < t.u1; kt += kBN) process(kt, true, t.u1);
  for (int kt = t.s0; kt < t.r1; kt += kBN) process(kt, false, 0);

  if (qvalid) {
    __bf16 *op = dq + (int64_t(qrow) * Hq + h) * D;
#pragma unroll
    for (int dblk = 0; dblk < D / 32; ++dblk) {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        bf16x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = static_cast<__bf16>(acc[dblk][4 * rg + i] * scale);
        *reinterpret_cast<bf16x4 *>(op + 32 * dblk + 8 * rg + 4 * half) = w;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dk / dv: one block per (key tile of 128 keys, kv head); wave w owns keys
// [r0 + 32 w, r0 + 32 w + 32).  For every query head of the kv head and every
// block of 32 query rows that sees the tile:
//   S = Q K^T, dP = dO V^T (queries x keys, key per lane column),
//   P = exp(S - lse), dS = P (dP - D), dv += P^T dO, dk += dS^T Q.
// ---------------------------------------------------------------------------

constexpr int kQB = 32;   // query rows per step

template <int D>
__global__ void __launch_bounds__(kThreads) k_dkdv_bf16(const Tile *__restrict__ tiles, const int *__restrict__ ntiles,
                                                        int Hq, int Hkv, int T, const __bf16 *__restrict__ q,
                                                        const __bf16 *__restrict__ k, const __bf16 *__restrict__ v,
                                                        const float *__restrict__ lse,
                                                        const __bf16 *__restrict__ dout,
                                                        const float *__restrict__ Dbuf, __bf16 *__restrict__ dk,
                                                        __bf16 *__restrict__ dv, const int *__restrict__ seg_start,
                                                        float scale_log2, float scale) {
  constexpr int KS = D / 16;
  constexpr int RSTR = D * 2 + 16;     // row-major Q / dO tiles
  constexpr int TSTR = kQB * 2 + 16;   // transposed Q^T / dO^T tiles
  __shared__ __attribute__((aligned(16))) char smem[2 * kQB * RSTR + 2 * D * TSTR];
  __shared__ float s_lse[kQB], s_D[kQB];
  __shared__ int s_seg[kQB];
  char *Qs = smem;
  char *Ds = smem + kQB * RSTR;
  char *Qt = smem + 2 * kQB * RSTR;
  char *Dt = Qt + D * TSTR;

  const int tile_rank = blockIdx.x / Hkv;
  if (tile_rank >= *ntiles) return;
  const int kvh = blockIdx.x % Hkv;
  const Tile t = tiles[tile_rank];
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int half = lane >> 5, col = lane & 31;
  const int key = t.r0 + 32 * wave + col;
  const bool kvalid = key < t.r1;
  const int ratio = Hq / Hkv;

  bf16x8 kf[KS], vf[KS];
  {
    const int64_t off = (int64_t(kvalid ? key : t.r0) * Hkv + kvh) * D + 8 * half;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kf[ks] = kvalid ? ld8(k + off + 16 * ks) : zero8();
      vf[ks] = kvalid ? ld8(v + off + 16 * ks) : zero8();
    }
  }
  f32x16 dka[D / 32], dva[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    dka[i] = zero16();
    dva[i] = zero16();
  }

  auto process = [&](int h, int qb, int qend, bool masked) {
    __syncthreads();
    stage_rows<kQB, D, RSTR, kThreads>(Qs, q, qb, T, Hq, h);
    stage_rows<kQB, D, RSTR, kThreads>(Ds, dout, qb, T, Hq, h);
    stage_rows_t<kQB, D, TSTR, kThreads>(Qt, q, qb, T, Hq, h);
    stage_rows_t<kQB, D, TSTR, kThreads>(Dt, dout, qb, T, Hq, h);
    if (threadIdx.x < kQB) {
      const int row = qb + threadIdx.x;
      const bool ok = row < qend;
      s_lse[threadIdx.x] = ok ? lse[int64_t(h) * T + row] * kLog2e : 0.0f;
      s_D[threadIdx.x] = ok ? Dbuf[int64_t(h) * T + row] : 0.0f;
      s_seg[threadIdx.x] = ok ? (masked ? seg_start[row] : -1) : 0x7fffffff;
    }
    __syncthreads();
    f32x16 s = zero16(), dp = zero16();
    const char *qp = Qs + col * RSTR + 16 * half;
    const char *dpp = Ds + col * RSTR + 16 * half;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s = mfma(lds8(qp + 32 * ks), kf[ks], s);
      dp = mfma(lds8(dpp + 32 * ks), vf[ks], dp);
    }
    bf16x8 pf[2], dsf[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qi = c_row(r, half);
      const int row = qb + qi;
      const int sg = s_seg[qi];
      // masked rows: key <= row within the row's own segment; unmasked rows: all
      // (sg == -1); rows past the range: none (sg == INT_MAX)
      const bool vis = (sg < 0) || (key <= row && key >= sg);
      const float p = vis ? exp2f(s[r] * scale_log2 - s_lse[qi]) : 0.0f;
      pf[r >> 3][r & 7] = static_cast<__bf16>(p);
      dsf[r >> 3][r & 7] = static_cast<__bf16>(p * (dp[r] - s_D[qi]));
    }
#pragma unroll
    for (int dblk = 0; dblk < D / 32; ++dblk) {
      const char *dtp = Dt + (32 * dblk + col) * TSTR + 16 * half;
      const char *qtp = Qt + (32 * dblk + col) * TSTR + 16 * half;
      dva[dblk] = mfma(pf[0], lds8(dtp), dva[dblk]);
      dva[dblk] = mfma(pf[1], lds8(dtp + 32), dva[dblk]);
      dka[dblk] = mfma(dsf[0], lds8(qtp), dka[dblk]);
      dka[dblk] = mfma(dsf[1], lds8(qtp + 32), dka[dblk]);
    }
  };

  for (int hh = 0; hh < ratio; ++hh) {
    const int h = kvh * ratio + hh;
    for (int qb = t.u0; qb < t.u1; qb += kQB) process(h, qb, t.u1, true);
    for (int qb = t.s0; qb < t.e0; qb += kQB) process(h, qb, t.e0, false);
  }

  // dv / dk results: register r of dblk holds key row c_row(r, half) of the
  // wave's 32 keys and column 32 dblk + col.
#pragma unroll
  for (int dblk = 0; dblk < D / 32; ++dblk) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kk = t.r0 + 32 * wave + c_row(r, half);
      if (kk < t.r1) {
        const int64_t off = (int64_t(kk) * Hkv + kvh) * D + 32 * dblk + col;
        dk[off] = static_cast<__bf16>(dka[dblk][r] * scale);
        dv[off] = static_cast<__bf16>(dva[dblk][r]);
      }
    }
  }
}

int heads_per_block(const spd_attn_desc &d) {
  const int ratio = d.num_q_heads / d.num_kv_heads;
  return (ratio % 4 == 0) ? 4 : (ratio % 2 == 0 ? 2 : 1);
}

}  // namespace

int dq_bf16_rows_per_tile(const spd_attn_desc &d) { return 32 * (4 / heads_per_block(d)); }
int dkdv_bf16_rows_per_tile(const spd_attn_desc &) { return 128; }

#define SPD_DISPATCH_HPW(HPW_VAL, ...)            \
  switch (HPW_VAL) {                              \
    case 4: { constexpr int HPW = 4; __VA_ARGS__; } break; \
    case 2: { constexpr int HPW = 2; __VA_ARGS__; } break; \
    default: { constexpr int HPW = 1; __VA_ARGS__; } break; \
  }

spd_status attn_bwd_bf16(const spd_attn_desc &d, const spd_plan &plan, int64_t T, const Tile *qtiles, const int *nq,
                         int64_t capq, const Tile *ktiles, const int *nk, int64_t capk, const void *q, const void *k,
                         const void *v, const void *o, const float *lse, const void *dout, void *dq, void *dk,
                         void *dv, float *Dbuf, hipStream_t st) {
  const auto *qq = static_cast<const __bf16 *>(q);
  const auto *kk = static_cast<const __bf16 *>(k);
  const auto *vv = static_cast<const __bf16 *>(v);
  const auto *oo = static_cast<const __bf16 *>(o);
  const auto *dd = static_cast<const __bf16 *>(dout);
  const int64_t n = T * d.num_q_heads;
  const int rpw = 64 / (d.head_dim / 8);
  const int64_t waves = (n + rpw - 1) / rpw;
  const dim3 gpre(static_cast<unsigned>((waves + 3) / 4));
  prof_start(SPD_K_BWD_PRE, st);
  if (d.head_dim == 128)
    hipLaunchKernelGGL(k_rowdot_bf16<128>, gpre, dim3(256), 0, st, n, d.num_q_heads, int(T), oo, dd, Dbuf);
  else
    hipLaunchKernelGGL(k_rowdot_bf16<64>, gpre, dim3(256), 0, st, n, d.num_q_heads, int(T), oo, dd, Dbuf);
  SPD_LAUNCH_CHECK();
  prof_stop(SPD_K_BWD_PRE, st);
  const int hpw = heads_per_block(d);
  const int HG = d.num_q_heads / hpw;
  const float sl2 = d.softmax_scale * kLog2e;
  const dim3 gq(static_cast<unsigned>(capq * HG));
  const dim3 gk(static_cast<unsigned>(capk * d.num_kv_heads));
  auto *dqq = static_cast<__bf16 *>(dq);
  auto *dkk = static_cast<__bf16 *>(dk);
  auto *dvv = static_cast<__bf16 *>(dv);
  prof_start(SPD_K_BWD_DQ, st);
  if (d.head_dim == 128) {
    SPD_DISPATCH_HPW(hpw, hipLaunchKernelGGL((k_dq_bf16<128, HPW>), gq, dim3(kThreads), 0, st, qtiles, nq, HG,
                                             d.num_q_heads, d.num_kv_heads, int(T), qq, kk, vv, lse, dd, Dbuf, dqq,
                                             plan.seg_start, sl2, d.softmax_scale));
  } else {
    SPD_DISPATCH_HPW(hpw, hipLaunchKernelGGL((k_dq_bf16<64, HPW>), gq, dim3(kThreads), 0, st, qtiles, nq, HG,
                                             d.num_q_heads, d.num_kv_heads, int(T), qq, kk, vv, lse, dd, Dbuf, dqq,
                                             plan.seg_start, sl2, d.softmax_scale));
  }
  SPD_LAUNCH_CHECK();
  prof_stop(SPD_K_BWD_DQ, st);
  prof_start(SPD_K_BWD_DKDV, st);
  if (d.head_dim == 128)
    hipLaunchKernelGGL(k_dkdv_bf16<128>, gk, dim3(kThreads), 0, st, ktiles, nk, d.num_q_heads, d.num_kv_heads, int(T),
                       qq, kk, vv, lse, dd, Dbuf, dkk, dvv, plan.seg_start, sl2, d.softmax_scale);
  else
    hipLaunchKernelGGL(k_dkdv_bf16<64>, gk, dim3(kThreads), 0, st, ktiles, nk, d.num_q_heads, d.num_kv_heads, int(T),
                       qq, kk, vv, lse, dd, Dbuf, dkk, dvv, plan.seg_start, sl2, d.softmax_scale);
  SPD_LAUNCH_CHECK();
  prof_stop(SPD_K_BWD_DKDV, st);
  return SPD_OK;
}

}  // namespace spd
