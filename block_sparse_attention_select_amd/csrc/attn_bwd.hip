// Block-sparse GQA attention backward on gfx950.
//
// What is computed (radixark/miles PR #4581, kernel-tuning commit: gradients
// of the block-sparse kernel, dK/dV of a KV head summed over its query heads;
// the follow-up commit stores dV with V's own strides): with
// P = exp(scale q.k - LSE), dP = dO . v, Delta = rowsum(dO * O) and
// dS = P (dP - Delta):
//     dq   = scale * sum_j dS_j k_j                      (token-major pass)
//     dk_j = scale * sum dS q,  dv_j = sum P dO           (key-block-major pass)
// the key-block sums running over every (query, head) of the group that
// selected the block.
//
// Kernels:
//   bwd_prep_kernel     Delta, plus per-token transposed copies of q and dO
//                       ([d][16 heads]) used as MFMA operands by dK/dV;
//   attn_bwd_dq_kernel  one wavefront per (token, KV head), the forward's
//                       transposed-score layout (lane = head row);
//   attn_bwd_dkdv_kernel (attn_bwd_dkdv.hip) key-block-major dK/dV per chunk
//                       of selecting queries;
//   dkdv_reduce_kernel  sums the per-chunk slices of a block in chunk order
//                       (fixed order, no atomics: bitwise deterministic) and
//                       writes bf16 dK/dV with their own strides; blocks with a
//                       single chunk were finished by the dK/dV kernel.
#include "msa_internal.h"

namespace msa {

namespace {

// ---------------------------------------------------------------------------
// Delta and transposed q / dO.  One wavefront per (token, KV head).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_prep_kernel(
    const u16* __restrict__ o, int64_t o_st, int64_t o_sh,
    const u16* __restrict__ dO, int64_t do_st, int64_t do_sh,
    const u16* __restrict__ q, int64_t q_st, int64_t q_sh, int T, int Hk,
    float* __restrict__ delta, u16* __restrict__ qT, u16* __restrict__ doT) {
  __shared__ u16 tq[4][kHeadDim][kGroup + 2];
  __shared__ u16 tdo[4][kHeadDim][kGroup + 2];
  const int wl = threadIdx.x >> 6;
  const int wave_raw = blockIdx.x * 4 + wl;
  const int lane = threadIdx.x & 63;
  // Every wavefront reaches the barrier below; surplus ones redo the last
  // (token, head) without storing.
  const bool active = wave_raw < T * Hk;
  const int wave = active ? wave_raw : T * Hk - 1;
  const int t = wave / Hk;
  const int h = wave - t * Hk;
  const int head = lane >> 2;   // 0..15
  const int quarter = lane & 3; // 32 dims each
  const int hq = h * kGroup + head;
  const u16* orow = o + (int64_t)t * o_st + (int64_t)hq * o_sh + 32 * quarter;
  const u16* drow = dO + (int64_t)t * do_st + (int64_t)hq * do_sh + 32 * quarter;
  const u16* qrow = q + (int64_t)t * q_st + (int64_t)hq * q_sh + 32 * quarter;
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint4 ov = *reinterpret_cast<const uint4*>(orow + 8 * j);
    const uint4 dv = *reinterpret_cast<const uint4*>(drow + 8 * j);
    const uint4 qv = *reinterpret_cast<const uint4*>(qrow + 8 * j);
    const u16* op = reinterpret_cast<const u16*>(&ov);
    const u16* dp = reinterpret_cast<const u16*>(&dv);
    const u16* qp = reinterpret_cast<const u16*>(&qv);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      acc += bf2f(op[e]) * bf2f(dp[e]);
      tdo[wl][32 * quarter + 8 * j + e][head] = dp[e];
      tq[wl][32 * quarter + 8 * j + e][head] = qp[e];
    }
  }
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  if (active && quarter == 0) delta[(int64_t)t * (Hk * kGroup) + hq] = acc;
  __syncthreads();
  if (!active) return;
  // each lane writes two d rows of 16 heads (2 x 32 bytes) of each tensor
  const int64_t base = ((int64_t)t * Hk + h) * (kHeadDim * kGroup);
#pragma unroll
  for (int rr = 0; rr < 2; ++rr) {
    const int d = 2 * lane + rr;
    uint32_t wq[8], wd[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      wq[e] = (uint32_t)tq[wl][d][2 * e] | ((uint32_t)tq[wl][d][2 * e + 1] << 16);
      wd[e] = (uint32_t)tdo[wl][d][2 * e] | ((uint32_t)tdo[wl][d][2 * e + 1] << 16);
    }
    uint4* qdst = reinterpret_cast<uint4*>(qT + base + d * kGroup);
    uint4* ddst = reinterpret_cast<uint4*>(doT + base + d * kGroup);
    qdst[0] = make_uint4(wq[0], wq[1], wq[2], wq[3]);
    qdst[1] = make_uint4(wq[4], wq[5], wq[6], wq[7]);
    ddst[0] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
    ddst[1] = make_uint4(wd[4], wd[5], wd[6], wd[7]);
  }
}

// ---------------------------------------------------------------------------
// dQ.  One wavefront per (token, KV head); lane = head row (li), as in the
// forward.  dQ^T = K^T dS^T with K^T from the per-block transposed copy.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void attn_bwd_dq_kernel(
    const u16* __restrict__ q, int64_t q_st, int64_t q_sh,
    const u16* __restrict__ k, int64_t k_st, int64_t k_sh,
    const u16* __restrict__ v, int64_t v_st, int64_t v_sh,
    const u16* __restrict__ kt, const u16* __restrict__ dO, int64_t do_st, int64_t do_sh,
    const float* __restrict__ lse, const float* __restrict__ delta,
    const int32_t* __restrict__ blk_idx, const int32_t* __restrict__ cu, const int32_t* __restrict__ blkbase,
    int S, int T, int Hk, float scale_log2, float scale, u16* __restrict__ dq, int64_t dq_st, int64_t dq_sh) {
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int li = lane & 15;
  if (wave >= T * Hk) return;
  const int t = wave / Hk;
  const int h = wave - t * Hk;
  const int s = find_seq(cu, S, t);
  const int seq0 = cu[s];
  const int pos = t - seq0;
  const int b = pos / kBlock;
  const int gb0 = blkbase[s];
  const int my_blk = lane < kTopk ? blk_idx[(int64_t)wave * kTopk + lane] : -1;
  const int hq = h * kGroup + li;

  const u16* qrow = q + (int64_t)t * q_st + (int64_t)hq * q_sh;
  const u16* drow = dO + (int64_t)t * do_st + (int64_t)hq * do_sh;
  bf16x8 qb[4], db[4];
#pragma unroll
  for (int ds = 0; ds < 4; ++ds) {
    qb[ds] = load_bf16x8(qrow + 32 * ds + 8 * g);
    db[ds] = load_bf16x8(drow + 32 * ds + 8 * g);
  }
  const float l2 = lse[(int64_t)t * (Hk * kGroup) + hq];
  const bool live = l2 > -INFINITY;
  const float lse2 = live ? l2 * kLog2e : 0.f;
  const float dl = delta[(int64_t)t * (Hk * kGroup) + hq];

  f32x4 dqacc[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) dqacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int i = 0; i < kTopk; ++i) {
    const int c = __shfl(my_blk, i);
    if (c < 0 || c > b) continue;
    const int kstart = seq0 + kBlock * c;
    const bool diag = (c == b);
    f32x4 sacc[8], pacc[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int kl = 32 * (kk >> 1) + 8 * (li >> 2) + 4 * (kk & 1) + (li & 3);
      const int kg = min(kstart + kl, T - 1);
      const u16* krow = k + (int64_t)kg * k_st + (int64_t)h * k_sh;
      const u16* vrow = v + (int64_t)kg * v_st + (int64_t)h * v_sh;
      f32x4 a = {0.f, 0.f, 0.f, 0.f};
      f32x4 bb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) {
        a = mfma16x16x32(load_bf16x8(krow + 32 * ds + 8 * g), qb[ds], a);
        bb = mfma16x16x32(load_bf16x8(vrow + 32 * ds + 8 * g), db[ds], bb);
      }
      sacc[kk] = a;
      pacc[kk] = bb;
    }
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kl = 32 * (kk >> 1) + 8 * g + 4 * (kk & 1) + r;
        const float e = fast_exp2(sacc[kk][r] * scale_log2 - lse2);
        const float p = (!live || (diag && kBlock * c + kl > pos)) ? 0.f : e;
        sacc[kk][r] = p * (pacc[kk][r] - dl);
      }
    bf16x8 dsf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) dsf[ks] = pack_bf16x8(sacc[2 * ks], sacc[2 * ks + 1]);
    const u16* ktb = kt + ((int64_t)(gb0 + c) * Hk + h) * (kHeadDim * kBlock);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        dqacc[dt] = mfma16x16x32(load_bf16x8(ktb + ((dt * 4 + ks) * 64 + lane) * 8), dsf[ks], dqacc[dt]);
  }
  u16* out = dq + (int64_t)t * dq_st + (int64_t)hq * dq_sh;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<uint2*>(out + 16 * dt + 4 * g) = pack_bf16x4(dqacc[dt] * scale);
}

// ---------------------------------------------------------------------------
// Ordered reduction of the per-chunk slices of one (block, KV head).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void dkdv_reduce_kernel(
    const float* __restrict__ part_dk, const float* __restrict__ part_dv, const int32_t* __restrict__ item_count,
    const int32_t* __restrict__ itembase, const int32_t* __restrict__ blk_seq, const int32_t* __restrict__ blkbase,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ totals, int Hk, int items_cap, float scale,
    u16* __restrict__ dk, int64_t dk_st, int64_t dk_sh, u16* __restrict__ dv, int64_t dv_st, int64_t dv_sh) {
  const int gb = blockIdx.x;
  const int h = blockIdx.y;
  if (gb >= totals[0]) return;
  const int s = blk_seq[gb];
  const int c = gb - blkbase[s];
  const int seq0 = cu[s];
  const int L = cu[s + 1] - seq0;
  const int i0 = itembase[gb];
  const int i1 = min(itembase[gb + 1], items_cap);
  if (i1 - i0 == 1) return;  // a block with one work item was written by the dK/dV kernel itself
  for (int e = threadIdx.x * 4; e < kBlock * kHeadDim; e += 256 * 4) {
    const int key = e / kHeadDim;
    const int d = e - key * kHeadDim;
    const int kp = kBlock * c + key;
    if (kp >= L) continue;
    f32x4 adk = {0.f, 0.f, 0.f, 0.f};
    f32x4 adv = {0.f, 0.f, 0.f, 0.f};
    for (int it = i0; it < i1; ++it) {
      if (item_count[(int64_t)h * items_cap + it] == 0) continue;
      const int64_t off = ((int64_t)h * items_cap + it) * (kBlock * kHeadDim) + e;
      const float4 a = *reinterpret_cast<const float4*>(part_dk + off);
      const float4 b = *reinterpret_cast<const float4*>(part_dv + off);
      adk += f32x4{a.x, a.y, a.z, a.w};
      adv += f32x4{b.x, b.y, b.z, b.w};
    }
    *reinterpret_cast<uint2*>(dk + (int64_t)(seq0 + kp) * dk_st + (int64_t)h * dk_sh + d) = pack_bf16x4(adk * scale);
    *reinterpret_cast<uint2*>(dv + (int64_t)(seq0 + kp) * dv_st + (int64_t)h * dv_sh + d) = pack_bf16x4(adv);
  }
}

}  // namespace

void launch_attn_bwd(const Sizes& z, const BwdArgs& a, const PlanBufs& p, hipStream_t st) {
  const int T = (int)z.T, Hk = (int)z.Hk, S = (int)z.S;
  const unsigned wgs_tok = (unsigned)((z.T * z.Hk + 3) / 4);
  launch_block_transpose(z, a.k, a.k_st, a.k_sh, a.cu, p, a.kt, st);
  {
    KernelTimer timer("bwd_prep", st);
    bwd_prep_kernel<<<wgs_tok, 256, 0, st>>>(a.o, a.o_st, a.o_sh, a.dO, a.do_st, a.do_sh, a.q, a.q_st, a.q_sh, T, Hk,
                                             a.delta, a.qT, a.doT);
  }
  {
    KernelTimer timer("attn_bwd_dq", st);
    attn_bwd_dq_kernel<<<wgs_tok, 256, 0, st>>>(a.q, a.q_st, a.q_sh, a.k, a.k_st, a.k_sh, a.v, a.v_st, a.v_sh, a.kt,
                                                a.dO, a.do_st, a.do_sh, a.lse, a.delta, a.blk_idx, a.cu, p.blkbase, S,
                                                T, Hk, a.scale * kLog2e, a.scale, a.dq, a.dq_st, a.dq_sh);
  }
  launch_attn_bwd_dkdv(z, a, p, st);
  {
    KernelTimer timer("dkdv_reduce", st);
    dkdv_reduce_kernel<<<dim3((unsigned)z.nblk_cap, (unsigned)Hk), 256, 0, st>>>(
        a.part_dk, a.part_dv, a.item_count, p.itembase, p.blk_seq, p.blkbase, a.cu, p.totals, Hk, (int)z.items_cap,
        a.scale, a.dk, a.dk_st, a.dk_sh, a.dv, a.dv_st, a.dv_sh);
  }
}

}  // namespace msa
