// fp32 split attention: a plain-arithmetic path, one thread per row, meant
// for small problems and for checking the tile plan end to end in full fp32.
//
// How Prompt Deduplication Works -- Phase 2, "Split Attention Optimization";
// "Correctness & Gradients".  Forward: online softmax over the visible keys.
// Backward: D = rowsum(dO * O); P = exp(s - lse); dP = dO . v;
// dS = P (dP - D); dq = scale sum_k dS k; dk = scale sum_q dS q; dv = sum_q P dO.
#include "spd_attn.h"

namespace spd {
namespace {

__device__ inline bool sees(int key, int row, const int *seg_start) {
  return key <= row && key >= seg_start[row];
}

template <int D>
__global__ void __launch_bounds__(kF32Rows) k_fwd_f32(const Tile *__restrict__ tiles, const int *__restrict__ ntiles,
                                                      int Hq, int Hkv, int T, const float *__restrict__ q,
                                                      const float *__restrict__ k, const float *__restrict__ v,
                                                      float *__restrict__ o, float *__restrict__ lse,
                                                      const int *__restrict__ seg_start, float scale) {
  const int ti = blockIdx.x / Hq;
  const int h = blockIdx.x % Hq;
  if (ti >= *ntiles) return;
  const Tile t = tiles[ti];
  const int row = t.r0 + threadIdx.x;
  const bool valid = row < t.r1;
  const int kvh = h / (Hq / Hkv);
  float qv[D], acc[D];
  const float *qr = q + (int64_t(valid ? row : t.r0) * Hq + h) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    qv[d] = qr[d];
    acc[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  auto visit = [&](int key) {
    const float *kr = k + (int64_t(key) * Hkv + kvh) * D;
    const float *vr = v + (int64_t(key) * Hkv + kvh) * D;
    float s = 0.f;
#pragma unroll
    for (int d = 0; d < D; ++d) s = fmaf(qv[d], kr[d], s);
    s *= scale;
    const float mn = fmaxf(m, s);
    const float a = expf(m - mn);
    const float p = expf(s - mn);
    l = l * a + p;
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] = fmaf(p, vr[d], acc[d] * a);
    m = mn;
  };
  if (valid) {
    for (int key = t.v0; key < t.v1; ++key) visit(key);
    for (int key = t.u0; key < t.u1; ++key) visit(key);
    for (int key = t.s0; key <= row; ++key)
      if (sees(key, row, seg_start)) visit(key);
    const float inv = 1.f / l;
    float *orow = o + (int64_t(row) * Hq + h) * D;
#pragma unroll
    for (int d = 0; d < D; ++d) orow[d] = acc[d] * inv;
    lse[int64_t(h) * T + row] = m + logf(l);
  }
}

// D[h, row] = sum_d dO[row, h, d] * O[row, h, d]
template <typename In>
__global__ void __launch_bounds__(256) k_rowdot_f32(int64_t rows_x_heads, int D, const In *__restrict__ o,
                                                    const In *__restrict__ dout, int Hq, int T,
                                                    float *__restrict__ Dbuf) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= rows_x_heads) return;
  const int64_t row = i / Hq;
  const int h = static_cast<int>(i % Hq);
  const In *a = o + i * D;
  const In *b = dout + i * D;
  float s = 0.f;
  for (int d = 0; d < D; ++d) s = fmaf(static_cast<float>(a[d]), static_cast<float>(b[d]), s);
  Dbuf[int64_t(h) * T + row] = s;
}

template <int D>
__global__ void __launch_bounds__(kF32Rows) k_dq_f32(const Tile *__restrict__ tiles, const int *__restrict__ ntiles,
                                                     int Hq, int Hkv, int T, const float *__restrict__ q,
                                                     const float *__restrict__ k, const float *__restrict__ v,
                                                     const float *__restrict__ lse, const float *__restrict__ dout,
                                                     const float *__restrict__ Dbuf, float *__restrict__ dq,
                                                     const int *__restrict__ seg_start, float scale) {
  const int ti = blockIdx.x / Hq;
  const int h = blockIdx.x % Hq;
  if (ti >= *ntiles) return;
  const Tile t = tiles[ti];
  const int row = t.r0 + threadIdx.x;
  if (row >= t.r1) return;
  const int kvh = h / (Hq / Hkv);
  float qv[D], dov[D], acc[D];
  const float *qr = q + (int64_t(row) * Hq + h) * D;
  const float *dr = dout + (int64_t(row) * Hq + h) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    qv[d] = qr[d];
    dov[d] = dr[d];
    acc[d] = 0.f;
  }
  const float L = lse[int64_t(h) * T + row];
  const float Dr = Dbuf[int64_t(h) * T + row];
  auto visit = [&](int key) {
    const float *kr = k + (int64_t(key) * Hkv + kvh) * D;
    const float *vr = v + (int64_t(key) * Hkv + kvh) * D;
    float s = 0.f, dp = 0.f;
#pragma unroll
    for (int d = 0; d < D; ++d) {
      s = fmaf(qv[d], kr[d], s);
      dp = fmaf(dov[d], vr[d], dp);
    }
    const float p = expf(s * scale - L);
    const float ds = p * (dp - Dr);
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] = fmaf(ds, kr[d], acc[d]);
  };
  for (int key = t.v0; key < t.v1; ++key) visit(key);
  for (int key = t.u0; key < t.u1; ++key) visit(key);
  for (int key = t.s0; key <= row; ++key)
    if (sees(key, row, seg_start)) visit(key);
  float *out = dq + (int64_t(row) * Hq + h) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) out[d] = acc[d] * scale;
}

template <int D>
__global__ void __launch_bounds__(kF32Rows) k_dkdv_f32(const Tile *__restrict__ tiles, const int *__restrict__ ntiles,
                                                       int Hq, int Hkv, int T, const float *__restrict__ q,
                                                       const float *__restrict__ k, const float *__restrict__ v,
                                                       const float *__restrict__ lse, const float *__restrict__ dout,
                                                       const float *__restrict__ Dbuf, float *__restrict__ dk,
                                                       float *__restrict__ dv, const int *__restrict__ seg_start,
                                                       float scale) {
  const int ti = blockIdx.x / Hkv;
  const int kvh = blockIdx.x % Hkv;
  if (ti >= *ntiles) return;
  const Tile t = tiles[ti];
  const int key = t.r0 + threadIdx.x;
  if (key >= t.r1) return;
  const int ratio = Hq / Hkv;
  float kv[D], vv[D], ak[D], av[D];
  const float *kr = k + (int64_t(key) * Hkv + kvh) * D;
  const float *vr = v + (int64_t(key) * Hkv + kvh) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    kv[d] = kr[d];
    vv[d] = vr[d];
    ak[d] = 0.f;
    av[d] = 0.f;
  }
  for (int h = kvh * ratio; h < (kvh + 1) * ratio; ++h) {
    auto visit = [&](int row) {
      const float *qr = q + (int64_t(row) * Hq + h) * D;
      const float *dr = dout + (int64_t(row) * Hq + h) * D;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) {
        s = fmaf(qr[d], kv[d], s);
        dp = fmaf(dr[d], vv[d], dp);
      }
      const float p = expf(s * scale - lse[int64_t(h) * T + row]);
      const float ds = p * (dp - Dbuf[int64_t(h) * T + row]);
#pragma unroll
      for (int d = 0; d < D; ++d) {
        av[d] = fmaf(p, dr[d], av[d]);
        ak[d] = fmaf(ds, qr[d], ak[d]);
      }
    };
    for (int row = max(t.u0, key); row < t.u1; ++row)
      if (sees(key, row, seg_start)) visit(row);
    for (int row = t.s0; row < t.e0; ++row) visit(row);
  }
  float *ok = dk + (int64_t(key) * Hkv + kvh) * D;
  float *ov = dv + (int64_t(key) * Hkv + kvh) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    ok[d] = ak[d] * scale;
    ov[d] = av[d];
  }
}

}  // namespace

spd_status attn_fwd_f32(const spd_attn_desc &d, const spd_plan &plan, int64_t T, const Tile *tiles, const int *ntiles,
                        int64_t cap, const float *q, const float *k, const float *v, float *o, float *lse,
                        hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(cap * d.num_q_heads));
  prof_start(SPD_K_FWD, st);
  if (d.head_dim == 64)
    hipLaunchKernelGGL(k_fwd_f32<64>, grid, dim3(kF32Rows), 0, st, tiles, ntiles, d.num_q_heads, d.num_kv_heads,
                       int(T), q, k, v, o, lse, plan.seg_start, d.softmax_scale);
  else
    hipLaunchKernelGGL(k_fwd_f32<128>, grid, dim3(kF32Rows), 0, st, tiles, ntiles, d.num_q_heads, d.num_kv_heads,
                       int(T), q, k, v, o, lse, plan.seg_start, d.softmax_scale);
  SPD_LAUNCH_CHECK();
  prof_stop(SPD_K_FWD, st);
  return SPD_OK;
}

spd_status attn_bwd_f32(const spd_attn_desc &d, const spd_plan &plan, int64_t T, const Tile *qtiles, const int *nq,
                        int64_t capq, const Tile *ktiles, const int *nk, int64_t capk, const float *q,
                        const float *k, const float *v, const float *o, const float *lse, const float *dout,
                        float *dq, float *dk, float *dv, float *Dbuf, hipStream_t st) {
  const int64_t n = T * d.num_q_heads;
  hipLaunchKernelGGL(k_rowdot_f32<float>, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st, n,
                     d.head_dim, o, dout, d.num_q_heads, int(T), Dbuf);
  SPD_LAUNCH_CHECK();
  const dim3 gq(static_cast<unsigned>(capq * d.num_q_heads));
  const dim3 gk(static_cast<unsigned>(capk * d.num_kv_heads));
  if (d.head_dim == 64) {
    hipLaunchKernelGGL(k_dq_f32<64>, gq, dim3(kF32Rows), 0, st, qtiles, nq, d.num_q_heads, d.num_kv_heads, int(T),
                       q, k, v, lse, dout, Dbuf, dq, plan.seg_start, d.softmax_scale);
    SPD_LAUNCH_CHECK();
    hipLaunchKernelGGL(k_dkdv_f32<64>, gk, dim3(kF32Rows), 0, st, ktiles, nk, d.num_q_heads, d.num_kv_heads,
                       int(T), q, k, v, lse, dout, Dbuf, dk, dv, plan.seg_start, d.softmax_scale);
  } else {
    hipLaunchKernelGGL(k_dq_f32<128>, gq, dim3(kF32Rows), 0, st, qtiles, nq, d.num_q_heads, d.num_kv_heads, int(T),
                       q, k, v, lse, dout, Dbuf, dq, plan.seg_start, d.softmax_scale);
    SPD_LAUNCH_CHECK();
    hipLaunchKernelGGL(k_dkdv_f32<128>, gk, dim3(kF32Rows), 0, st, ktiles, nk, d.num_q_heads, d.num_kv_heads,
                       int(T), q, k, v, lse, dout, Dbuf, dk, dv, plan.seg_start, d.softmax_scale);
  }
  return check_launch();
}

}  // namespace spd
