// Block-sparse GQA attention forward on gfx950.
//
// What is computed (miles docs "MiniMax-M3.1-Flash", section 1: each query
// attends to its 16 selected 128-token blocks, index head h choosing for KV
// head h; radixark/miles PR #4581: QSA block-sparse kernel): for token t and
// query head g of KV head h, softmax(scale * q . k_j) v_j over the keys j <= t
// of the listed blocks, with the log-sum-exp saved for the backward.
//
// Layout of the work: one wavefront per (token, KV head).  The 16 query heads
// of the group are the 16 columns of every MFMA tile, so the token's shared
// block list drives one wavefront.  Scores are formed transposed,
// S^T[key][head] = K Q^T (A = K rows, B = the token's q held in registers),
// which leaves each lane with one head row: the online softmax needs only two
// cross-lane steps per block.  O^T = V^T P^T then takes P straight from the
// score registers (B operand) and V^T from a per-block transposed copy made
// by block_transpose_kernel, so every MFMA operand is one 16-byte load.
//
// Key order inside a 32-key step: score tile 2s holds keys 32s + 8g + {0..3}
// and tile 2s+1 keys 32s + 8g + {4..7} in lane group g = lane / 16, so the
// eight P values a lane owns are eight consecutive keys -- the same eight
// consecutive keys the V^T operand reads.
#include "msa_internal.h"

namespace msa {

namespace {

// Per-block transposed copy: xt[gb][h][d][key] (128 x 128 bf16), keys past the
// end of the sequence zero-filled.
__global__ __launch_bounds__(256) void block_transpose_kernel(const u16* __restrict__ x, int64_t st_t, int64_t st_h,
                                                              const int32_t* __restrict__ cu,
                                                              const int32_t* __restrict__ blkbase,
                                                              const int32_t* __restrict__ blk_seq,
                                                              const int32_t* __restrict__ totals, int Hk,
                                                              u16* __restrict__ xt) {
  __shared__ u16 tile[kBlock][kHeadDim + 8];
  const int gb = blockIdx.x;
  const int h = blockIdx.y;
  if (gb >= totals[0]) return;
  const int s = blk_seq[gb];
  const int c = gb - blkbase[s];
  const int seq0 = cu[s];
  const int L = cu[s + 1] - seq0;
  for (int i = threadIdx.x; i < kBlock * 16; i += 256) {
    const int key = i >> 4;
    const int ch = i & 15;
    const int kp = kBlock * c + key;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (kp < L) v = *reinterpret_cast<const uint4*>(x + (int64_t)(seq0 + kp) * st_t + (int64_t)h * st_h + ch * 8);
    *reinterpret_cast<uint4*>(&tile[key][ch * 8]) = v;
  }
  __syncthreads();
  u16* dst = xt + ((int64_t)gb * Hk + h) * (kHeadDim * kBlock);
  for (int i = threadIdx.x; i < kHeadDim * 16; i += 256) {
    const int d = i >> 4;
    const int kc = i & 15;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = (uint32_t)tile[8 * kc + 2 * e][d] | ((uint32_t)tile[8 * kc + 2 * e + 1][d] << 16);
    *reinterpret_cast<uint4*>(dst + d * kBlock + 8 * kc) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

__global__ __launch_bounds__(256) void attn_fwd_kernel(
    const u16* __restrict__ q, int64_t q_st, int64_t q_sh,
    const u16* __restrict__ k, int64_t k_st, int64_t k_sh,
    const u16* __restrict__ vt, const int32_t* __restrict__ blk_idx,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ blkbase, int S, int T, int Hk,
    float scale_log2, u16* __restrict__ o, int64_t o_st, int64_t o_sh, float* __restrict__ lse) {
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

  const u16* qrow = q + (int64_t)t * q_st + (int64_t)(h * kGroup + li) * q_sh;
  bf16x8 qb[4];
#pragma unroll
  for (int ds = 0; ds < 4; ++ds) qb[ds] = load_bf16x8(qrow + 32 * ds + 8 * g);

  f32x4 oacc[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  float l_run = 0.f;

  for (int i = 0; i < kTopk; ++i) {
    const int c = __shfl(my_blk, i);
    if (c < 0 || c > b) continue;
    const int kstart = seq0 + kBlock * c;
    const bool diag = (c == b);

    f32x4 st[8];
#pragma unroll
    for (int kt = 0; kt < 8; ++kt) {
      const int kl = 32 * (kt >> 1) + 8 * (li >> 2) + 4 * (kt & 1) + (li & 3);
      const int kg = min(kstart + kl, T - 1);
      const u16* krow = k + (int64_t)kg * k_st + (int64_t)h * k_sh;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) acc = mfma16x16x32(load_bf16x8(krow + 32 * ds + 8 * g), qb[ds], acc);
      st[kt] = acc;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 8; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kl = 32 * (kt >> 1) + 8 * g + 4 * (kt & 1) + r;
        float z = st[kt][r] * scale_log2;
        if (diag && kBlock * c + kl > pos) z = -INFINITY;
        st[kt][r] = z;
        mx = fmaxf(mx, z);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2f(m_run - m_new);
    float rs = 0.f;
#pragma unroll
    for (int kt = 0; kt < 8; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = exp2f(st[kt][r] - m_new);
        st[kt][r] = p;
        rs += p;
      }
    rs += __shfl_xor(rs, 16);
    rs += __shfl_xor(rs, 32);
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) oacc[dt] *= alpha;

    bf16x8 pf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) pf[ks] = pack_bf16x8(st[2 * ks], st[2 * ks + 1]);
    const u16* vtb = vt + ((int64_t)(gb0 + c) * Hk + h) * (kHeadDim * kBlock);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        oacc[dt] = mfma16x16x32(load_bf16x8(vtb + (16 * dt + li) * kBlock + 32 * ks + 8 * g), pf[ks], oacc[dt]);
  }

  const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
  u16* orow = o + (int64_t)t * o_st + (int64_t)(h * kGroup + li) * o_sh;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    *reinterpret_cast<uint2*>(orow + 16 * dt + 4 * g) = pack_bf16x4(oacc[dt] * inv);
  }
  if (g == 0) {
    lse[(int64_t)t * (Hk * kGroup) + h * kGroup + li] = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
  }
}

}  // namespace

void launch_block_transpose(const Sizes& z, const u16* x, int64_t st_t, int64_t st_h,
                            const int32_t* cu, const PlanBufs& p, u16* xt, hipStream_t st) {
  {
    KernelTimer timer("block_transpose", st);
    block_transpose_kernel<<<dim3((unsigned)z.nblk_cap, (unsigned)z.Hk), 256, 0, st>>>(
        x, st_t, st_h, cu, p.blkbase, p.blk_seq, p.totals, (int)z.Hk, xt);
  }
}

void launch_attn_fwd(const Sizes& z, const u16* q, int64_t q_st, int64_t q_sh,
                     const u16* k, int64_t k_st, int64_t k_sh, const u16* vt,
                     const int32_t* blk_idx, const int32_t* cu, const PlanBufs& p, float scale,
                     u16* o, int64_t o_st, int64_t o_sh, float* lse, hipStream_t st) {
  const int64_t waves = z.T * z.Hk;
  {
    KernelTimer timer("attn_fwd", st);
    attn_fwd_kernel<<<dim3((unsigned)((waves + 3) / 4)), 256, 0, st>>>(
        q, q_st, q_sh, k, k_st, k_sh, vt, blk_idx, cu, p.blkbase, (int)z.S, (int)z.T, (int)z.Hk,
        scale * kLog2e, o, o_st, o_sh, lse);
  }
}

}  // namespace msa
