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
//                            rounded to fp32), then its q and k heads, four
//                            rows at a time (16 lanes per row, 16-byte loads);
//   qk_norm_rope_bwd_kernel  one wavefront per token, the same lane layout;
//                            each workgroup leaves its weight-gradient sums
//                            in a workspace row;
//   qk_norm_dw_stage1/2      sum those rows in workgroup order, in two
//                            stages (fixed order: bitwise deterministic).
// The forward keeps the indexer's per-element arithmetic (square, sum, scale,
// add eps, sqrt, divide, multiply by x, by (1 + w); rotation as two products
// and one sum), free of fused multiply-adds, so every step rounds once in fp32;
// only the order of the 128-term sum of squares is the lane layout's.
#include "msa_internal.h"

namespace msa {

namespace {

constexpr int kQkWaves = 4;

// Lane layout: a wavefront works on four (token, head) rows at a time, row
// slot lane / 16; lane l = lane % 16 holds dims 8l .. 8l+7 (one 16-byte load).
// Lanes 0-3 hold dims 0..31, whose RoPE partners 32..63 sit in lanes 4-7
// (lane xor 4); lanes 8-15 hold the unrotated dims 64..127.  The RoPE angles
// of a token are formed once (lanes 0..31, fp64 from the host's fp64 inverse
// frequencies, rounded to fp32) and read back from LDS: lane l < 8 uses pairs
// 8 (l % 4) .. 8 (l % 4) + 7.
struct Row8 {
  float v[8];
};
__device__ __forceinline__ Row8 load_row8(const u16* p) {
  const u32x4 w = *reinterpret_cast<const u32x4*>(p);
  Row8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r.v[2 * i] = __uint_as_float(w[i] << 16);
    r.v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
  return r;
}
__device__ __forceinline__ void store_row8(u16* p, const float (&v)[8]) {
  u32x4 w;
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = (uint32_t)f2bf(v[2 * i]) | ((uint32_t)f2bf(v[2 * i + 1]) << 16);
  *reinterpret_cast<u32x4*>(p) = w;
}
// sum over the 16 lanes of a row slot
__device__ __forceinline__ float row_sum16(float x) {
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}
// the token's angles into LDS (cos at [0, 32), sin at [32, 64)), then this
// lane's eight pairs
__device__ __forceinline__ void token_angles(int lane, int pos, const RopeFreqs& fr, float* ang, float (&c)[8],
                                             float (&sn)[8]) {
  if (lane < 32) {
    double sd, cd;
    sincos((double)pos * rope_freq_of(fr, lane), &sd, &cd);
    ang[lane] = (float)cd;
    ang[32 + lane] = (float)sd;
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int pb = 8 * (lane & 3);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    c[i] = ang[pb + i];
    sn[i] = ang[32 + pb + i];
  }
}

__global__ __launch_bounds__(64 * kQkWaves) void qk_norm_rope_fwd_kernel(
    const u16* __restrict__ q, int64_t q_st, int64_t q_sh, const u16* __restrict__ k, int64_t k_st, int64_t k_sh,
    const u16* __restrict__ w_q, const u16* __restrict__ w_k, float eps, RopeFreqs fr,
    const int32_t* __restrict__ cu, int S, int T, int Hq, int Hk, u16* __restrict__ qo, int64_t qo_st,
    int64_t qo_sh, u16* __restrict__ ko, int64_t ko_st, int64_t ko_sh) {
#pragma clang fp contract(off)
  __shared__ float ang[kQkWaves][64];
  const int wave = threadIdx.x >> 6;
  const int t = blockIdx.x * kQkWaves + wave;
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  const int l = lane & 15, slot = lane >> 4;
  float wq1[8], wk1[8];  // (1 + w) of this lane's dims (the weights are only 2-byte aligned)
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    wq1[i] = 1.0f + bf2f(w_q[8 * l + i]);
    wk1[i] = 1.0f + bf2f(w_k[8 * l + i]);
  }
  const int s = find_seq(cu, S, t);
  float c[8], sn[8];
  token_angles(lane, t - cu[s], fr, ang[wave], c, sn);
  const int nrows = Hq + Hk;
  auto in_row = [&](int hh) -> const u16* {
    return hh < Hq ? q + (int64_t)t * q_st + (int64_t)hh * q_sh : k + (int64_t)t * k_st + (int64_t)(hh - Hq) * k_sh;
  };
  auto out_row = [&](int hh) -> u16* {
    return hh < Hq ? qo + (int64_t)t * qo_st + (int64_t)hh * qo_sh : ko + (int64_t)t * ko_st + (int64_t)(hh - Hq) * ko_sh;
  };
  for (int r0 = 0; r0 < nrows; r0 += 8) {
    // two rows per row slot, both loaded before either is used
    Row8 x[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int hh = min(r0 + 4 * e + slot, nrows - 1);
      x[e] = load_row8(in_row(hh) + 8 * l);
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int hh = r0 + 4 * e + slot;
      const bool isq = hh < Hq;
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) ss += x[e].v[i] * x[e].v[i];
      ss = row_sum16(ss);
      const float r = 1.0f / sqrtf(ss * (1.0f / 128.0f) + eps);
      float y[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = (x[e].v[i] * r) * (isq ? wq1[i] : wk1[i]);
      float o[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float p = __shfl_xor(y[i], 4);  // the RoPE partner dim (lanes 0-7)
        o[i] = l < 4 ? (y[i] * c[i]) - (p * sn[i]) : l < 8 ? (y[i] * c[i]) + (p * sn[i]) : y[i];
      }
      if (hh < nrows) store_row8(out_row(hh) + 8 * l, o);
    }
  }
}

// Wavefront w of workgroup b handles tokens b*4 + w, then + 4*gridDim.x, ...
// Its weight-gradient sums (this lane's eight dims, for q and for k) are added
// over the row slots and wavefronts in LDS, in a fixed order, and written to
// partial[b][256] (q: dims 0..127, k: 128..255).
__global__ __launch_bounds__(64 * kQkWaves) void qk_norm_rope_bwd_kernel(
    const u16* __restrict__ q, int64_t q_st, int64_t q_sh, const u16* __restrict__ k, int64_t k_st, int64_t k_sh,
    const u16* __restrict__ w_q, const u16* __restrict__ w_k, float eps, RopeFreqs fr,
    const int32_t* __restrict__ cu, int S, int T, int Hq, int Hk,
    const u16* __restrict__ dqh, int64_t dqh_st, int64_t dqh_sh, const u16* __restrict__ dkh, int64_t dkh_st,
    int64_t dkh_sh, u16* __restrict__ dq, int64_t dq_st, int64_t dq_sh, u16* __restrict__ dk, int64_t dk_st,
    int64_t dk_sh, float* __restrict__ partial) {
  __shared__ float ang[kQkWaves][64];
  __shared__ float red[4 * kQkWaves][256];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int l = lane & 15, slot = lane >> 4;
  float wq1[8], wk1[8];  // (1 + w) of this lane's dims (the weights are only 2-byte aligned)
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    wq1[i] = 1.0f + bf2f(w_q[8 * l + i]);
    wk1[i] = 1.0f + bf2f(w_k[8 * l + i]);
  }
  float gq[8], gk[8];  // dw sums for this lane's dims
#pragma unroll
  for (int i = 0; i < 8; ++i) gq[i] = gk[i] = 0.f;
  const int nrows = Hq + Hk;
  for (int t = blockIdx.x * kQkWaves + wave; t < T; t += gridDim.x * kQkWaves) {
    const int s = find_seq(cu, S, t);
    float c[8], sn[8];
    token_angles(lane, t - cu[s], fr, ang[wave], c, sn);
    for (int r0 = 0; r0 < nrows; r0 += 4) {
      const int hh = r0 + slot;
      const int hc = min(hh, nrows - 1);
      const bool isq = hc < Hq;
      const int h = isq ? hc : hc - Hq;
      const u16* x = isq ? q + (int64_t)t * q_st + (int64_t)h * q_sh : k + (int64_t)t * k_st + (int64_t)h * k_sh;
      const u16* dz = isq ? dqh + (int64_t)t * dqh_st + (int64_t)h * dqh_sh
                          : dkh + (int64_t)t * dkh_st + (int64_t)h * dkh_sh;
      const Row8 xv = load_row8(x + 8 * l);
      const Row8 zv = load_row8(dz + 8 * l);
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) ss += xv.v[i] * xv.v[i];
      ss = row_sum16(ss);
      const float r = 1.0f / sqrtf(ss * (1.0f / 128.0f) + eps);
      // dy = RoPE^T(dz)
      float dy[8], g[8];
      float dot = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float p = __shfl_xor(zv.v[i], 4);
        dy[i] = l < 4 ? c[i] * zv.v[i] + sn[i] * p : l < 8 ? c[i] * zv.v[i] - sn[i] * p : zv.v[i];
        g[i] = dy[i] * (isq ? wq1[i] : wk1[i]);
        dot += g[i] * xv.v[i];
      }
      dot = row_sum16(dot);
      const float k3 = r * r * r * dot * (1.0f / 128.0f);
      float dxv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) dxv[i] = r * g[i] - xv.v[i] * k3;
      if (hh < nrows) {
        u16* dx = isq ? dq + (int64_t)t * dq_st + (int64_t)h * dq_sh : dk + (int64_t)t * dk_st + (int64_t)h * dk_sh;
        store_row8(dx + 8 * l, dxv);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float a = dy[i] * xv.v[i] * r;
          if (isq)
            gq[i] += a;
          else
            gk[i] += a;
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    red[4 * wave + slot][8 * l + i] = gq[i];
    red[4 * wave + slot][128 + 8 * l + i] = gk[i];
  }
  __syncthreads();
  const int i = threadIdx.x;  // 256 threads: one output each
  float acc = 0.f;
#pragma unroll
  for (int w = 0; w < 4 * kQkWaves; ++w) acc += red[w][i];
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

void launch_qk_norm_bwd_k(const Sizes& z, const QkNormArgs& a, float* partial, int extra_rows, float* mid,
                          hipStream_t st) {
  const int rows_k = qk_norm_bwd_rows(z.T);
  if (rows_k > 0) {
    KernelTimer timer("qk_norm_rope_bwd", st);
    // no q rows: the kernel's q half of each partial row stays zero
    qk_norm_rope_bwd_kernel<<<(unsigned)rows_k, 64 * kQkWaves, 0, st>>>(
        nullptr, 0, 0, a.k, a.k_st, a.k_sh, a.w_q, a.w_k, a.eps, rope_freqs(a.rope_base), a.cu, (int)z.S, (int)z.T, 0,
        (int)z.Hk, nullptr, 0, 0, a.dkh, a.dkh_st, a.dkh_sh, nullptr, 0, 0, a.ko, a.ko_st, a.ko_sh, partial);
  }
  {
    KernelTimer timer("qk_norm_dw_reduce", st);
    const int rows = rows_k + extra_rows;
    const int mid_rows = (rows + kReduceRows - 1) / kReduceRows;
    if (mid_rows > 0) qk_norm_dw_stage1_kernel<<<(unsigned)mid_rows, 256, 0, st>>>(partial, rows, mid);
    qk_norm_dw_stage2_kernel<<<1, 256, 0, st>>>(mid, mid_rows, a.dw_q, a.dw_k);
  }
}

}  // namespace msa
