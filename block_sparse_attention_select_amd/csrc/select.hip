// Frozen lightning-indexer block selection on gfx950.
//
// What is computed (miles docs "MiniMax-M3.1-Flash", section 1; Megatron-Bridge
// "MiniMax-M3", Architecture Notes; radixark/miles PR #4581 kernel tuning):
//   1. features: gemma RMSNorm x / sqrt(mean(x^2) + eps) * (1 + w), then
//      rotate-half RoPE on dims 0..63 at the sequence-local position, rounded
//      once to bf16;
//   2. score of causal block c for query i: max over keys j <= i of block c of
//      the bf16 feature dot product, accumulated in fp32 on the matrix cores;
//   3. selection: blocks 0..b when b < 16, else the own block b plus the 15
//      best of 0..b-1 (lower id first on equal scores), written ascending.
//
// Kernels: select_prologue (features), select_scores (MFMA + per-row block
// maximum), select_topk (wavefront arg-max rounds).
#include "msa_internal.h"

namespace msa {

namespace {

// ---------------------------------------------------------------------------
// 1. Features.  One wavefront per (token, head, q-or-k).  Lane l < 32 holds
// the RoPE pair (l, l + 32); lane l >= 32 holds dims 32 + l and 64 + l.
// The arithmetic order (square, sum, scale by 1/128, add eps, sqrt, divide,
// multiply by x, multiply by (1 + w); rotation as two products and one sum)
// is kept free of fused multiply-adds so every step rounds once in fp32.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void select_prologue_kernel(
    const u16* __restrict__ idx_q, int64_t sq_t, int64_t sq_h,
    const u16* __restrict__ idx_k, int64_t sk_t, int64_t sk_h,
    const u16* __restrict__ w_q, const u16* __restrict__ w_k, float eps, float rope_base,
    const int32_t* __restrict__ cu, int S, int T, int Hk,
    u16* __restrict__ qfeat, u16* __restrict__ kfeat) {
#pragma clang fp contract(off)
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (wave >= T * Hk * 2) return;
  const int which = wave & 1;
  const int th = wave >> 1;
  const int t = th / Hk;
  const int h = th - t * Hk;
  const int s = find_seq(cu, S, t);
  const int pos = t - cu[s];
  const u16* x = which ? idx_k + (int64_t)t * sk_t + (int64_t)h * sk_h
                       : idx_q + (int64_t)t * sq_t + (int64_t)h * sq_h;
  const u16* w = which ? w_k : w_q;
  u16* out = (which ? kfeat : qfeat) + ((int64_t)t * Hk + h) * kHeadDim;

  const int d0 = lane < 32 ? lane : 32 + lane;
  const int d1 = d0 + 32;
  const float x0 = bf2f(x[d0]);
  const float x1 = bf2f(x[d1]);
  float ss = x0 * x0 + x1 * x1;
  for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
  const float ms = ss * (1.0f / 128.0f);
  const float r = 1.0f / sqrtf(ms + eps);
  float y0 = (x0 * r) * (1.0f + bf2f(w[d0]));
  float y1 = (x1 * r) * (1.0f + bf2f(w[d1]));
  if (lane < 32) {
    const double inv_freq = pow((double)rope_base, -(double)(2 * lane) / 64.0);
    const double theta = (double)pos * inv_freq;
    double sn, cs;
    sincos(theta, &sn, &cs);
    const float c = (float)cs;
    const float sf = (float)sn;
    const float o0 = (y0 * c) - (y1 * sf);
    const float o1 = (y1 * c) + (y0 * sf);
    y0 = o0;
    y1 = o1;
  }
  out[d0] = f2bf(y0);
  out[d1] = f2bf(y1);
}

// ---------------------------------------------------------------------------
// 2. Block scores.  One workgroup (4 wavefronts) per (query block, chunk of
// kKeyChunk key blocks, head).  Wavefront w owns query rows 32w..32w+31 of
// the query block; its bf16 features stay in registers as MFMA A operands.
// Each key block (128 x 128 bf16) is staged in LDS with a 16-byte row pad so
// the B-operand reads of 16 consecutive keys hit distinct banks.
// ---------------------------------------------------------------------------
constexpr int kKeyChunk = 8;
constexpr int kRowPad = 17;  // uint4 per staged key row (16 data + 1 pad)

__global__ __launch_bounds__(256) void select_scores_kernel(
    const u16* __restrict__ qfeat, const u16* __restrict__ kfeat, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ blkbase, const int32_t* __restrict__ blk_seq,
    const int32_t* __restrict__ totals, int Hk, int nbmax, float* __restrict__ scores) {
  __shared__ uint4 ktile[kBlock * kRowPad];
  const int gb = blockIdx.x;
  const int kc = blockIdx.y;
  const int h = blockIdx.z;
  if (gb >= totals[0]) return;
  const int s = blk_seq[gb];
  const int qb = gb - blkbase[s];
  const int c0 = kc * kKeyChunk;
  if (c0 > qb) return;
  const int c1 = min(min(c0 + kKeyChunk, qb + 1), nbmax);  // nbmax bound holds when lengths <= max_seqlen
  const int seq0 = cu[s];
  const int L = cu[s + 1] - seq0;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int li = lane & 15;

  bf16x8 qa[2][4];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int qp = kBlock * qb + 32 * wave + 16 * rt + li;
    const u16* src = qfeat + ((int64_t)(seq0 + qp) * Hk + h) * kHeadDim;
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) qa[rt][ds] = qp < L ? load_bf16x8(src + 32 * ds + 8 * g) : zero_bf16x8();
  }

  for (int c = c0; c < c1; ++c) {
    __syncthreads();
    for (int i = threadIdx.x; i < kBlock * 16; i += 256) {
      const int key = i >> 4;
      const int ch = i & 15;
      const int kp = kBlock * c + key;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (kp < L) v = *reinterpret_cast<const uint4*>(kfeat + ((int64_t)(seq0 + kp) * Hk + h) * kHeadDim + ch * 8);
      ktile[key * kRowPad + ch] = v;
    }
    __syncthreads();

    float rmax[2][4];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) rmax[rt][r] = -INFINITY;

#pragma unroll
    for (int kt = 0; kt < 8; ++kt) {
      bf16x8 kb[4];
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) kb[ds] = __builtin_bit_cast(bf16x8, ktile[(16 * kt + li) * kRowPad + 4 * ds + g]);
      const int kp = kBlock * c + 16 * kt + li;
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ds = 0; ds < 4; ++ds) acc = mfma16x16x32(qa[rt][ds], kb[ds], acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int qp = kBlock * qb + 32 * wave + 16 * rt + 4 * g + r;
          const float v = kp <= qp ? acc[r] : -INFINITY;
          rmax[rt][r] = fmaxf(rmax[rt][r], v);
        }
      }
    }
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = rmax[rt][r];
        v = fmaxf(v, __shfl_xor(v, 1));
        v = fmaxf(v, __shfl_xor(v, 2));
        v = fmaxf(v, __shfl_xor(v, 4));
        v = fmaxf(v, __shfl_xor(v, 8));
        rmax[rt][r] = v;
      }
    if (li == 0) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int qp = kBlock * qb + 32 * wave + 16 * rt + 4 * g + r;
          if (qp < L) scores[((int64_t)(seq0 + qp) * Hk + h) * nbmax + c] = rmax[rt][r];
        }
    }
  }
}

// ---------------------------------------------------------------------------
// 3. Top-k.  One wavefront per (token, head): 15 rounds of a wavefront-wide
// arg-max over the block scores (score descending, id ascending), then the
// 16 ids are ranked to ascending order.
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool better(float av, int ai, float bv, int bi) {
  return av > bv || (av == bv && ai < bi);
}

__global__ __launch_bounds__(256) void select_topk_kernel(const float* __restrict__ scores,
                                                          const int32_t* __restrict__ cu, int S, int T,
                                                          int Hk, int nbmax, int32_t* __restrict__ blk_idx) {
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (wave >= T * Hk) return;
  const int t = wave / Hk;
  const int s = find_seq(cu, S, t);
  const int pos = t - cu[s];
  const int b = pos / kBlock;
  int32_t* out = blk_idx + (int64_t)wave * kTopk;
  if (b < kTopk) {
    if (lane < kTopk) out[lane] = lane <= b ? lane : -1;
    return;
  }
  const float* row = scores + (int64_t)wave * nbmax;
  constexpr int kPer = kMaxBlocks / 64;
  float v[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int c = lane + 64 * j;
    float x = -INFINITY;
    if (c < b && c < nbmax) {
      x = row[c];
      if (x != x) x = -INFINITY;  // NaN ranks last
    }
    v[j] = x;
  }
  unsigned taken = 0;
  int mine = -1;
  for (int k = 0; k < kTopk - 1; ++k) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int c = lane + 64 * j;
      if (c < b && !((taken >> j) & 1u) && better(v[j], c, bv, bi)) {
        bv = v[j];
        bi = c;
      }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      const float ov = __shfl_xor(bv, m);
      const int oi = __shfl_xor(bi, m);
      if (better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (lane == (bi & 63)) taken |= 1u << (bi >> 6);
    if (lane == k) mine = bi;
  }
  if (lane == kTopk - 1) mine = b;
  int rank = 0;
#pragma unroll
  for (int j = 0; j < kTopk; ++j) {
    const int o = __shfl(mine, j);
    rank += o < mine ? 1 : 0;
  }
  if (lane < kTopk) out[rank] = mine;
}

}  // namespace

void launch_select(const Sizes& z, const u16* idx_q, int64_t sq_t, int64_t sq_h,
                   const u16* idx_k, int64_t sk_t, int64_t sk_h, const u16* w_q, const u16* w_k,
                   float eps, float rope_base, const int32_t* cu, const PlanBufs& p,
                   u16* qfeat, u16* kfeat, float* scores, int32_t* blk_idx, hipStream_t st) {
  const int T = (int)z.T, Hk = (int)z.Hk, S = (int)z.S;
  const int64_t waves_pro = z.T * z.Hk * 2;
  {
    KernelTimer timer("select_prologue", st);
    select_prologue_kernel<<<dim3((unsigned)((waves_pro + 3) / 4)), 256, 0, st>>>(
        idx_q, sq_t, sq_h, idx_k, sk_t, sk_h, w_q, w_k, eps, rope_base, cu, S, T, Hk, qfeat, kfeat);
  }
  const unsigned kchunks = (unsigned)((z.nbmax + kKeyChunk - 1) / kKeyChunk);
  {
    KernelTimer timer("select_scores", st);
    select_scores_kernel<<<dim3((unsigned)z.nblk_cap, kchunks, (unsigned)Hk), 256, 0, st>>>(
        qfeat, kfeat, cu, p.blkbase, p.blk_seq, p.totals, Hk, (int)z.nbmax, scores);
  }
  const int64_t waves_top = z.T * z.Hk;
  {
    KernelTimer timer("select_topk", st);
    select_topk_kernel<<<dim3((unsigned)((waves_top + 3) / 4)), 256, 0, st>>>(scores, cu, S, T, Hk, (int)z.nbmax,
                                                                             blk_idx);
  }
}

}  // namespace msa
