// Attention-side gemma RMSNorm and rotate-half RoPE applied inside the
// attention kernels (the fused entry points msa_attn_fwd_qknorm /
// msa_attn_bwd_qknorm): miles docs "MiniMax-M3.1-Flash", section 1 (per-head
// gemma q/k norm, RoPE on the first 64 of 128 dims, base 1e7);
// Megatron-Bridge "MiniMax-M3", Architecture Notes (x * (1 + w), partial RoPE).
//     y = x * r * (1 + w),  r = 1 / sqrt(mean(x^2) + eps)
//     z_i = y_i cos - y_{i+32} sin,  z_{i+32} = y_{i+32} cos + y_i sin   (i < 32)
// at the token's sequence-local position, rounded once to bf16.  The element
// arithmetic is the standalone norm kernel's (no fused multiply-adds); only
// the order of the 128-term sum of squares follows each caller's lane layout.
#pragma once
#include "msa_internal.h"

namespace msa {

// One row spread over the 8 consecutive lanes of a group: lane j holds dims
// 4j + e, 32 + 4j + e, 64 + 4j + e, 96 + 4j + e (x[4 * quarter + e]); c, s
// are the angles of pairs 4j + e.  On return x holds the bf16-rounded result.
__device__ __forceinline__ void norm_rope_row8(float (&x)[16], const float (&w1)[16], const float (&c)[4],
                                               const float (&s)[4], float eps) {
#pragma clang fp contract(off)
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) ss += x[i] * x[i];
#pragma unroll
  for (int m = 1; m < 8; m <<= 1) ss += __shfl_xor(ss, m);
  const float r = 1.0f / sqrtf(ss * (1.0f / 128.0f) + eps);
  float y[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) y[i] = (x[i] * r) * w1[i];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float a = (y[e] * c[e]) - (y[4 + e] * s[e]);
    const float b = (y[4 + e] * c[e]) + (y[e] * s[e]);
    y[e] = a;
    y[4 + e] = b;
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] = bf2f(f2bf(y[i]));
}

// cos / sin of pair i at position pos, from the fp64 angle (rounded to fp32)
__device__ __forceinline__ void rope_angle(const RopeFreqs& fr, int i, int pos, float& c, float& s) {
  double sd, cd;
  sincos((double)pos * rope_freq_of(fr, i), &sd, &cd);
  c = (float)cd;
  s = (float)sd;
}

// The token's RoPE angles for a wavefront: lanes 0..31 write cos / sin of
// pair `lane` to ang[lane], ang[32 + lane] (64 floats of LDS).
__device__ __forceinline__ void rope_angles_lds(const RopeFreqs& fr, int pos, int lane, float* ang) {
  if (lane < 32) {
    float c, s;
    rope_angle(fr, lane, pos, c, s);
    ang[lane] = c;
    ang[32 + lane] = s;
  }
}

// The 16 heads of one token held as MFMA B operands (lane li + 16 g holds
// dims 32 ds + 8 g + e of head li in qb[ds][e]): normalized per head (the sum
// of squares over the lane's 32 dims, then over the four lane groups) and
// rotated in place; pairs (i, i + 32) of dims i = 8 g + e sit in qb[0], qb[1]
// of the same lane.  w1(d) gives 1 + w of dim d; ang holds the token's angles
// (rope_angles_lds), visible to the wavefront.
template <class W1>
__device__ __forceinline__ void norm_rope_q_with(bf16x8 (&qb)[4], W1 w1, float eps, int lane, const float* ang) {
#pragma clang fp contract(off)
  const int g = lane >> 4;
  float x[4][8];
  float ss = 0.f;
#pragma unroll
  for (int ds = 0; ds < 4; ++ds)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[ds][e] = (float)qb[ds][e];
      ss += x[ds][e] * x[ds][e];
    }
  ss = sum_over_groups(ss);
  const float r = 1.0f / sqrtf(ss * (1.0f / 128.0f) + eps);
  float y[4][8];
#pragma unroll
  for (int ds = 0; ds < 4; ++ds)
#pragma unroll
    for (int e = 0; e < 8; ++e) y[ds][e] = (x[ds][e] * r) * w1(32 * ds + 8 * g + e);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float c = ang[8 * g + e], s = ang[32 + 8 * g + e];
    const float a = (y[0][e] * c) - (y[1][e] * s);
    const float b = (y[1][e] * c) + (y[0][e] * s);
    y[0][e] = a;
    y[1][e] = b;
  }
#pragma unroll
  for (int ds = 0; ds < 4; ++ds)
#pragma unroll
    for (int e = 0; e < 8; ++e) qb[ds][e] = (__bf16)y[ds][e];
}

}  // namespace msa
