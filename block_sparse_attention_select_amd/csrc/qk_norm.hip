// Attention-side q/k gemma RMSNorm and partial RoPE on gfx950, forward and
// backward.
//
// What is computed (miles docs "MiniMax-M3.1-Flash", section 1: per-head gemma
// q/k norm, RoPE on the first 64 dims, base 1e7; Megatron-Bridge "MiniMax-M3",
// Architecture Notes: gemma-style x * (1 + w), per-head QK RMSNorm, partial
// RoPE): for every head of q (and of k), at the token's sequence-local
// position p,
//     y = x * r * (1 + w),  r = 1 / sqrt(mean(x^2) + eps)   (128 dims)
//     z = RoPE_p(y)  (rotate-half on pairs (i, i+32), i < 32; dims >= 64 pass)
// rounded once to bf16; one [128] weight for q and one for k, shared by the
// heads.  Backward (vector-Jacobian product): dy = RoPE_p^T(dz) (rotation by
// -angle), g = dy * (1 + w), dx = r g - x r^3 sum(g x) / 128, and
// dw = sum over (token, head) of dy * x * r.
//
// Kernels:
//   qk_norm_rope_fwd_kernel  one wavefront per token: the angles once (fp64,
//                            rounded to fp32), then every q and k head;
//   qk_norm_rope_bwd_kernel  one wavefront per token, the same lane layout;
//                            each workgroup leaves its weight-gradient sums
//                            in a workspace row;
//   qk_norm_dw_stage1/2      sum those rows in workgroup order, in two
//                            stages (fixed order: bitwise deterministic).
// Lane l < 32 holds the RoPE pair (l, l + 32); lane l >= 32 dims 32 + l and
// 64 + l.  The forward keeps the indexer's arithmetic order, free of fused
// multiply-adds, so every step rounds once in fp32.
#include "msa_internal.h"

namespace msa {

namespace {

constexpr int kQkWaves = 4;

// cos / sin of this lane's RoPE pair at position pos (lanes >= 32: identity)
__device__ __forceinline__ void rope_angles(int lane, int pos, const RopeFreqs& fr, float& c, float& s) {
  c = 1.f;
  s = 0.f;
  if (lane < 32) {
    double sn, cs;
    sincos((double)pos * rope_freq_of(fr, lane), &sn, &cs);
    c = (float)cs;
    s = (float)sn;
  }
}

__global__ __launch_bounds__(64 * kQkWaves) void qk_norm_rope_fwd_kernel(
    const u16* __restrict__ q, int64_t q_st, int64_t q_sh, const u16* __restrict__ k, int64_t k_st, int64_t k_sh,
    const u16* __restrict__ w_q, const u16* __restrict__ w_k, float eps, RopeFreqs fr,
    const int32_t* __restrict__ cu, int S, int T, int Hq, int Hk, u16* __restrict__ qo, int64_t qo_st,
    int64_t qo_sh, u16* __restrict__ ko, int64_t ko_st, int64_t ko_sh) {
#pragma clang fp contract(off)
  const int t = blockIdx.x * kQkWaves + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  const int s = find_seq(cu, S, t);
  float c, sn;
  rope_angles(lane, t - cu[s], fr, c, sn);
  const int d0 = lane < 32 ? lane : 32 + lane;
  const int d1 = d0 + 32;
  for (int hh = 0; hh < Hq + Hk; ++hh) {
    const bool isq = hh < Hq;
    const int h = isq ? hh : hh - Hq;
    const u16* x = isq ? q + (int64_t)t * q_st + (int64_t)h * q_sh : k + (int64_t)t * k_st + (int64_t)h * k_sh;
    const u16* w = isq ? w_q : w_k;
    u16* out = isq ? qo + (int64_t)t * qo_st + (int64_t)h * qo_sh : ko + (int64_t)t * ko_st + (int64_t)h * ko_sh;
    const float x0 = bf2f(x[d0]);
    const float x1 = bf2f(x[d1]);
    float ss = x0 * x0 + x1 * x1;
    for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
    const float r = 1.0f / sqrtf(ss * (1.0f / 128.0f) + eps);
    float y0 = (x0 * r) * (1.0f + bf2f(w[d0]));
    float y1 = (x1 * r) * (1.0f + bf2f(w[d1]));
    if (lane < 32) {
      const float o0 = (y0 * c) - (y1 * sn);
      const float o1 = (y1 * c) + (y0 * sn);
      y0 = o0;
      y1 = o1;
    }
    out[d0] = f2bf(y0);
    out[d1] = f2bf(y1);
  }
}

// Wavefront w of workgroup b handles tokens b*4 + w, then + 4*gridDim.x, ...
// Its weight-gradient sums (this lane's two dims, for q and for k) are added
// across the four wavefronts in LDS and written to partial[b][256]
// (q: dims 0..127, k: 128..255).
__global__ __launch_bounds__(64 * kQkWaves) void qk_norm_rope_bwd_kernel(
    const u16* __restrict__ q, int64_t q_st, int64_t q_sh, const u16* __restrict__ k, int64_t k_st, int64_t k_sh,
    const u16* __restrict__ w_q, const u16* __restrict__ w_k, float eps, RopeFreqs fr,
    const int32_t* __restrict__ cu, int S, int T, int Hq, int Hk,
    const u16* __restrict__ dqh, int64_t dqh_st, int64_t dqh_sh, const u16* __restrict__ dkh, int64_t dkh_st,
    int64_t dkh_sh, u16* __restrict__ dq, int64_t dq_st, int64_t dq_sh, u16* __restrict__ dk, int64_t dk_st,
    int64_t dk_sh, float* __restrict__ partial) {
  __shared__ float red[kQkWaves][256];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int d0 = lane < 32 ? lane : 32 + lane;
  const int d1 = d0 + 32;
  const float wq0 = 1.0f + bf2f(w_q[d0]), wq1 = 1.0f + bf2f(w_q[d1]);
  const float wk0 = 1.0f + bf2f(w_k[d0]), wk1 = 1.0f + bf2f(w_k[d1]);
  float gq0 = 0.f, gq1 = 0.f, gk0 = 0.f, gk1 = 0.f;  // dw sums for dims d0, d1
  for (int t = blockIdx.x * kQkWaves + wave; t < T; t += gridDim.x * kQkWaves) {
    const int s = find_seq(cu, S, t);
    float c, sn;
    rope_angles(lane, t - cu[s], fr, c, sn);
    for (int hh = 0; hh < Hq + Hk; ++hh) {
      const bool isq = hh < Hq;
      const int h = isq ? hh : hh - Hq;
      const u16* x = isq ? q + (int64_t)t * q_st + (int64_t)h * q_sh : k + (int64_t)t * k_st + (int64_t)h * k_sh;
      const u16* dz = isq ? dqh + (int64_t)t * dqh_st + (int64_t)h * dqh_sh
                          : dkh + (int64_t)t * dkh_st + (int64_t)h * dkh_sh;
      u16* dx = isq ? dq + (int64_t)t * dq_st + (int64_t)h * dq_sh : dk + (int64_t)t * dk_st + (int64_t)h * dk_sh;
      const float x0 = bf2f(x[d0]), x1 = bf2f(x[d1]);
      const float z0 = bf2f(dz[d0]), z1 = bf2f(dz[d1]);
      float ss = x0 * x0 + x1 * x1;
      for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
      const float r = 1.0f / sqrtf(ss * (1.0f / 128.0f) + eps);
      // dy = RoPE^T(dz)
      const float dy0 = lane < 32 ? c * z0 + sn * z1 : z0;
      const float dy1 = lane < 32 ? c * z1 - sn * z0 : z1;
      const float g0 = dy0 * (isq ? wq0 : wk0), g1 = dy1 * (isq ? wq1 : wk1);
      float dot = g0 * x0 + g1 * x1;
      for (int m = 32; m >= 1; m >>= 1) dot += __shfl_xor(dot, m);
      const float k3 = r * r * r * dot * (1.0f / 128.0f);
      dx[d0] = f2bf(r * g0 - x0 * k3);
      dx[d1] = f2bf(r * g1 - x1 * k3);
      if (isq) {
        gq0 += dy0 * x0 * r;
        gq1 += dy1 * x1 * r;
      } else {
        gk0 += dy0 * x0 * r;
        gk1 += dy1 * x1 * r;
      }
    }
  }
  red[wave][d0] = gq0;
  red[wave][d1] = gq1;
  red[wave][128 + d0] = gk0;
  red[wave][128 + d1] = gk1;
  __syncthreads();
  const int i = threadIdx.x;  // 256 threads: one output each
  float acc = 0.f;
#pragma unroll
  for (int w = 0; w < kQkWaves; ++w) acc += red[w][i];
  partial[(int64_t)blockIdx.x * 256 + i] = acc;
}

// Fixed-order sums of the partial rows in two stages: workgroup j of the first
// stage adds rows 16j .. 16j+15 (in row order) into row j of `mid`; the second
// stage adds the rows of `mid` in order.  The sixteen loads of a stage are in
// flight together; the additions keep row order.
constexpr int kReduceRows = 16;
__global__ __launch_bounds__(256) void qk_norm_dw_stage1_kernel(const float* __restrict__ partial, int rows,
                                                                float* __restrict__ mid) {
  const int i = threadIdx.x;
  const int b0 = blockIdx.x * kReduceRows;
  float v[kReduceRows];
#pragma unroll
  for (int r = 0; r < kReduceRows; ++r) v[r] = b0 + r < rows ? partial[(int64_t)(b0 + r) * 256 + i] : 0.f;
  float acc = 0.f;
#pragma unroll
  for (int r = 0; r < kReduceRows; ++r) acc += v[r];
  mid[(int64_t)blockIdx.x * 256 + i] = acc;
}

__global__ __launch_bounds__(256) void qk_norm_dw_stage2_kernel(const float* __restrict__ mid, int rows,
                                                                float* __restrict__ dw_q, float* __restrict__ dw_k) {
  const int i = threadIdx.x;
  float acc = 0.f;
  for (int b0 = 0; b0 < rows; b0 += kReduceRows) {
    float v[kReduceRows];
#pragma unroll
    for (int r = 0; r < kReduceRows; ++r) v[r] = b0 + r < rows ? mid[(int64_t)(b0 + r) * 256 + i] : 0.f;
#pragma unroll
    for (int r = 0; r < kReduceRows; ++r) acc += v[r];
  }
  if (i < 128)
    dw_q[i] = acc;
  else
    dw_k[i - 128] = acc;
}

}  // namespace

int qk_norm_bwd_rows(int64_t T) {
  const int64_t wgs = (T + kQkWaves - 1) / kQkWaves;
  return (int)(wgs < kQkBwdMaxRows ? wgs : kQkBwdMaxRows);
}

void launch_qk_norm_fwd(const Sizes& z, const QkNormArgs& a, hipStream_t st) {
  KernelTimer timer("qk_norm_rope_fwd", st);
  qk_norm_rope_fwd_kernel<<<(unsigned)((z.T + kQkWaves - 1) / kQkWaves), 64 * kQkWaves, 0, st>>>(
      a.q, a.q_st, a.q_sh, a.k, a.k_st, a.k_sh, a.w_q, a.w_k, a.eps, rope_freqs(a.rope_base), a.cu, (int)z.S, (int)z.T,
      (int)z.Hq, (int)z.Hk, a.qo, a.qo_st, a.qo_sh, a.ko, a.ko_st, a.ko_sh);
}

void launch_qk_norm_bwd(const Sizes& z, const QkNormArgs& a, float* partial, hipStream_t st) {
  const int rows = qk_norm_bwd_rows(z.T);
  if (rows > 0) {
    KernelTimer timer("qk_norm_rope_bwd", st);
    qk_norm_rope_bwd_kernel<<<(unsigned)rows, 64 * kQkWaves, 0, st>>>(
        a.q, a.q_st, a.q_sh, a.k, a.k_st, a.k_sh, a.w_q, a.w_k, a.eps, rope_freqs(a.rope_base), a.cu, (int)z.S, (int)z.T,
        (int)z.Hq, (int)z.Hk, a.dqh, a.dqh_st, a.dqh_sh, a.dkh, a.dkh_st, a.dkh_sh, a.qo, a.qo_st, a.qo_sh, a.ko,
        a.ko_st, a.ko_sh, partial);
  }
  {
    KernelTimer timer("qk_norm_dw_reduce", st);
    const int mid_rows = (rows + kReduceRows - 1) / kReduceRows;
    float* mid = partial ? partial + (int64_t)kQkBwdMaxRows * 256 : nullptr;  // null only when rows == 0
    if (mid_rows > 0) qk_norm_dw_stage1_kernel<<<(unsigned)mid_rows, 256, 0, st>>>(partial, rows, mid);
    qk_norm_dw_stage2_kernel<<<1, 256, 0, st>>>(mid, mid_rows, a.dw_q, a.dw_k);
  }
}

}  // namespace msa
