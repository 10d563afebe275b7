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
// Kernels: select_prologue (features, and the pack's block numbering),
// select_scores (MFMA + per-row block maximum), select_topk (ranking).
#include "attn_stage.h"
#include "plan_blocks.h"

namespace msa {

namespace {

// ---------------------------------------------------------------------------
// 1. Features.  One wavefront per two tokens.  First the RoPE angles of both
// tokens, one per lane (lane l: token l / 32, pair l % 32; fp64 from the host's
// fp64 inverse frequencies, rounded to fp32), into LDS.  Then, per head, one
// pass over four rows {token 0, token 1} x {q, k}: lane group g = lane / 16
// holds row g (token g / 2, q for even g, k for odd g) and lane j = lane % 16
// its dims 8j .. 8j+7, one 16-byte load.  The sum of squares has a fixed
// order: eight partial sums over the dims of each residue mod 8, each adding
// its 16 squares in dim order (carried lane to lane by DPP), then the
// partials as ((0+1)+(2+3))+((4+5)+(6+7)); the rotation partner of dims
// 8j .. 8j+7 (j < 8) sits in lane j ^ 4.  Each operation is a separately rounded fp32 operation: no fused
// multiply-adds (norm: square, sum, scale by 1/128, add eps, sqrt, divide,
// multiply by x, multiply by (1 + w); rotation: two products and one sum).
// The sequence of a token comes from a ballot over cu_seqlens held one entry
// per lane (packs of up to 63 sequences; a binary search beyond).
// The launch has one more workgroup, which numbers the pack's blocks for the
// scoring kernel (plan_blocks).
// ---------------------------------------------------------------------------
constexpr int kProWaves = 4;

// Sequence of token t: lane l holds cu[l] (or INT_MAX past S) when S < 64.
__device__ __forceinline__ int seq_of(const int32_t* __restrict__ cu, int S, int cu_lane, int t) {
  if (S < 64) return __popcll(__ballot(cu_lane <= t)) - 1;
  return find_seq(cu, S, t);
}

// Lane i - 1's value within each 16-lane row; 0 in the row's first lane.
__device__ __forceinline__ float dpp_shr1(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x111, 0xF, 0xF, false));
}
// The value of the last lane of each 16-lane row, in every lane of the row.
__device__ __forceinline__ float row_lane15(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x10 | (0x0F << 5)));
}
// ds_swizzle in bit-mask mode: lane ^ m within each 32-lane half
template <int kMask>
__device__ __forceinline__ float swz_xor(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x1F | (kMask << 10)));
}

__global__ __launch_bounds__(64 * kProWaves) void select_prologue_kernel(
    const u16* __restrict__ idx_q, int64_t sq_t, int64_t sq_h,
    const u16* __restrict__ idx_k, int64_t sk_t, int64_t sk_h,
    const u16* __restrict__ w_q, const u16* __restrict__ w_k, float eps, RopeFreqs fr,
    const int32_t* __restrict__ cu, int S, int T, int Hk, int chunk, PlanBufs plan,
    u16* __restrict__ qfeat, u16* __restrict__ kfeat) {
#pragma clang fp contract(off)
  __shared__ __align__(16) float ang[kProWaves][2][2][32];  // [wave][token][cos, sin][pair]
  // workgroup 0 writes the plan, dispatched first so that it runs beside the
  // feature workgroups instead of after them
  if (blockIdx.x == 0) {
    __shared__ int sb[64 * kProWaves], si[64 * kProWaves];
    plan_blocks<64 * kProWaves, kBlock>(cu, S, chunk, plan.blkbase, plan.blk_seq, plan.seqitem, plan.totals, sb, si);
    return;
  }
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int t0 = ((blockIdx.x - 1) * kProWaves + wave) * 2;  // may be past T: such a wavefront stores nothing
  const int g = lane >> 4, j = lane & 15;
  const int tt = g >> 1, which = g & 1;
  const int t = t0 + tt;
  const bool ok = t < T;
  const int tc = min(t, T - 1);

  // this lane's row: the first head's 16 bytes are loaded before the lookups
  const u16* xb = which ? idx_k + (int64_t)tc * sk_t : idx_q + (int64_t)tc * sq_t;
  const int64_t x_sh = which ? sk_h : sq_h;
  u32x4 raw = *reinterpret_cast<const u32x4*>(xb + 8 * j);
  const int cu_lane = (S < 64 && lane <= S) ? cu[lane] : 0x7fffffff;
  const u16* wp = (which ? w_k : w_q) + 8 * j;
  float w1[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) w1[e] = 1.0f + bf2f(wp[e]);

  // RoPE angles of the two tokens (lane: token lane / 32, pair lane % 32)
  {
    const int ta = min(t0 + (lane >> 5), T - 1);
    const int sa = seq_of(cu, S, cu_lane, min(t0, T - 1));
    const int sb = seq_of(cu, S, cu_lane, min(t0 + 1, T - 1));
    const int cs0 = S < 64 ? __builtin_amdgcn_readlane(cu_lane, sa) : cu[sa];
    const int cs1 = S < 64 ? __builtin_amdgcn_readlane(cu_lane, sb) : cu[sb];
    const int pos = ta - (lane < 32 ? cs0 : cs1);
    double sn, cs;
    sincos((double)pos * rope_freq_of(fr, lane & 31), &sn, &cs);
    ang[wave][lane >> 5][0][lane & 31] = (float)cs;
    ang[wave][lane >> 5][1][lane & 31] = (float)sn;
  }
  __syncthreads();
  float c[8], sf[8];
  {
    const int f0 = 8 * (j & 3);
    const f32x4 c0 = *reinterpret_cast<const f32x4*>(&ang[wave][tt][0][f0]);
    const f32x4 c1 = *reinterpret_cast<const f32x4*>(&ang[wave][tt][0][f0 + 4]);
    const f32x4 s0 = *reinterpret_cast<const f32x4*>(&ang[wave][tt][1][f0]);
    const f32x4 s1 = *reinterpret_cast<const f32x4*>(&ang[wave][tt][1][f0 + 4]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      c[e] = c0[e];
      c[e + 4] = c1[e];
      sf[e] = s0[e];
      sf[e + 4] = s1[e];
    }
  }

  for (int h = 0; h < Hk; ++h) {
    if (h > 0) raw = *reinterpret_cast<const u32x4*>(xb + (int64_t)h * x_sh + 8 * j);
    float x[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = __uint_as_float(raw[e] << 16);
      x[2 * e + 1] = __uint_as_float(raw[e] & 0xFFFF0000u);
    }
    // sum of squares in a fixed order: partial e (e = 0..7) adds the squares
    // of dims e, e + 8, ..., e + 120 one after another, carried along the
    // row's lanes (lane m adds dim 8m + e, after lane m - 1); lane 15 then
    // combines the eight partials as ((0+1)+(2+3))+((4+5)+(6+7)), and the
    // row's lanes take its sum
    float part[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) part[e] = x[e] * x[e];
    const float sq0[8] = {part[0], part[1], part[2], part[3], part[4], part[5], part[6], part[7]};
#pragma unroll 1
    for (int m = 1; m < 16; ++m) {
#pragma unroll
      for (int e = 0; e < 8; ++e) part[e] = dpp_shr1(part[e]) + sq0[e];
    }
    float ss = ((part[0] + part[1]) + (part[2] + part[3])) + ((part[4] + part[5]) + (part[6] + part[7]));
    ss = row_lane15(ss);
    const float ms = ss * (1.0f / 128.0f);
    const float r = 1.0f / sqrtf(ms + eps);
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = (x[e] * r) * w1[e];
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      float v[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const float yp = swz_xor<4>(y[e + u]);  // the rotation partner (dims 8(j^4) + e + u)
        const float lo = (y[e + u] * c[e + u]) - (yp * sf[e + u]);
        const float hi = (y[e + u] * c[e + u]) + (yp * sf[e + u]);
        v[u] = j < 4 ? lo : (j < 8 ? hi : y[e + u]);
      }
      o[e / 2] = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
    }
    if (ok) {
      u16* out = (which ? kfeat : qfeat) + ((int64_t)t * Hk + h) * kHeadDim + 8 * j;
      *reinterpret_cast<u32x4*>(out) = u32x4{o[0], o[1], o[2], o[3]};
    }
  }
}

// ---------------------------------------------------------------------------
// 2. Block scores.  One workgroup (4 wavefronts) per (query block, chunk of
// key blocks, head).  Wavefront w owns query rows 32w..32w+31 of the
// query block; their bf16 features stay in registers as MFMA B operands of
// S^T = K Q^T, so a lane's accumulators are keys of one query and the block
// maximum is a per-lane maximum plus one exchange across the four row groups.
// Key blocks are copied into LDS in A-operand order with global_load_lds, the
// next one while the current one is used; each K operand read feeds the
// MFMAs of both 16-query tiles of the wavefront.  The chunk's maxima collect
// in LDS and leave as one contiguous run per query row.  Chunks are 8 key
// blocks, or 32 from 16k-token sequences on, where the fp32 score matrix
// outgrows the L2s: a row's 32 maxima then fill whole 128-byte lines (with
// 4-byte stores from eight separately scheduled workgroups per line, the
// unsharded 32k layer wrote the 134 MB matrix as 709 MB).
// ---------------------------------------------------------------------------
constexpr int kKeyChunk = 8;
constexpr int kMaxKeyChunk = 32;
constexpr int64_t kLongKeyChunkSeqlen = 16384;

__global__ __launch_bounds__(256) void select_scores_kernel(
    const u16* __restrict__ qfeat, const u16* __restrict__ kfeat, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ blkbase, const int32_t* __restrict__ blk_seq,
    const int32_t* __restrict__ totals, int Hk, int nbmax, int key_chunk, float* __restrict__ scores) {
  // run kt * 4 + ds, lane li + 16 g: key 16 kt + li, dims 32 ds + 8 g .. +7
  __shared__ u32x4 kst[2][32][64];
  // the workgroup's block maxima, [query][key block of the chunk], written out
  // as contiguous row segments once the chunk is done (64 + 16 KB of LDS: two
  // workgroups per CU)
  __shared__ float smax[kBlock * kMaxKeyChunk];
  const int gb = blockIdx.x;
  const int kc = blockIdx.y;
  const int h = blockIdx.z;
  if (gb >= totals[0]) return;
  const int s = blk_seq[gb];
  const int qb = gb - blkbase[s];
  const int c0 = kc * key_chunk;
  if (c0 > qb) return;
  const int c1 = min(min(c0 + key_chunk, qb + 1), nbmax);  // nbmax bound holds when lengths <= max_seqlen
  const int seq0 = cu[s];
  const int L = cu[s + 1] - seq0;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int li = lane & 15;

  bf16x8 qf[2][4];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int qp = kBlock * qb + 32 * wave + 16 * rt + li;
    const u16* src = qfeat + ((int64_t)(seq0 + qp) * Hk + h) * kHeadDim;
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) qf[rt][ds] = qp < L ? load_bf16x8(src + 32 * ds + 8 * g) : zero_bf16x8();
  }

  // wavefront w copies runs 8w .. 8w+7 (key tiles 2w, 2w+1); keys past the
  // sequence end repeat its last key (they are masked as later than every query)
  auto stage = [&](int c, int buf) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int kt = 2 * wave + e;
      const int kp = min(kBlock * c + 16 * kt + li, L - 1);
      const u16* src = kfeat + ((int64_t)(seq0 + kp) * Hk + h) * kHeadDim + 8 * g;
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) dma16(src + 32 * ds, lds_offset(&kst[buf][4 * kt + ds][0]));
    }
  };
  stage(c0, 0);
  wait_copies();
  wait_all_loads();
  __syncthreads();

  for (int c = c0; c < c1; ++c) {
    const int buf = (c - c0) & 1;
    if (c + 1 < c1) stage(c + 1, buf ^ 1);
    const bool diag = c == qb;
    float m0 = -INFINITY, m1 = -INFINITY;
    // two halves of four key tiles; the 16 K operands of the second half are
    // read while the first half's 32 MFMAs run, and consecutive MFMAs belong
    // to different accumulators
    bf16x8 ka[2][16];
#pragma unroll
    for (int i = 0; i < 16; ++i) ka[0][i] = __builtin_bit_cast(bf16x8, kst[buf][(i & 3) * 4 + (i >> 2)][lane]);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      f32x4 a0[4], a1[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) a0[kk] = a1[kk] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (hf == 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          ka[1][i] = __builtin_bit_cast(bf16x8, kst[buf][(4 + (i & 3)) * 4 + (i >> 2)][lane]);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        a0[i & 3] = mfma16x16x32(ka[hf][i], qf[0][i >> 2], a0[i & 3]);
        a1[i & 3] = mfma16x16x32(ka[hf][i], qf[1][i >> 2], a1[i & 3]);
      }
      if (hf == 0) {  // first half's reads, then one second-half read per two MFMAs
        __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        }
      }
      if (diag) {  // key 16kt + 4g + r against query 32w + 16rt + li of the same block
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = 16 * (4 * hf + kk) + 4 * g + r;
            if (key > 32 * wave + li) a0[kk][r] = -INFINITY;
            if (key > 32 * wave + 16 + li) a1[kk][r] = -INFINITY;
          }
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        m0 = fmaxf(m0, fmaxf(fmaxf(a0[kk][0], a0[kk][1]), fmaxf(a0[kk][2], a0[kk][3])));
        m1 = fmaxf(m1, fmaxf(fmaxf(a1[kk][0], a1[kk][1]), fmaxf(a1[kk][2], a1[kk][3])));
      }
    }
    m0 = max_over_groups(m0);
    m1 = max_over_groups(m1);
    if (g == 0) {
      smax[(32 * wave + li) * key_chunk + c - c0] = m0;
      smax[(32 * wave + 16 + li) * key_chunk + c - c0] = m1;
    }
    wait_copies();
    lds_barrier();
  }
  // rows of the query block past the sequence end are not stored
  const int n = c1 - c0;
  const int rows = min(kBlock, L - kBlock * qb);
  for (int i = threadIdx.x; i < rows * n; i += 256) {
    const int r = i / n, j = i - r * n;
    scores[((int64_t)(seq0 + kBlock * qb + r) * Hk + h) * nbmax + c0 + j] = smax[r * key_chunk + j];
  }
}

// ---------------------------------------------------------------------------
// 3. Top-k.  A wavefront ranks one (token, head) row at a time.  The
// candidates are blocks 0 .. b-1 (b = own block), or 1 .. b-1 when block 0 is
// forced in (then 14 are chosen instead of 15); order: score descending, id
// ascending, a NaN score after every number.  Lane l holds candidates
// l + 64 j as 32-bit keys that order like the scores (the float's bits made
// order-preserving as an unsigned integer, -0 as +0, NaN just below -inf; 0
// for a non-candidate).  The 15th largest key is found bit by bit, from the
// top: a bit is kept when at least 15 candidates' keys reach the value so far
// with that bit set (ballot counts, no cross-lane data movement), and the
// search ends early once exactly 15 do.  Chosen are the keys above it, then,
// lowest ids first, as many of the keys equal to it as are still missing;
// they are written in id order (ballot prefix counts), then the own block.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t order_key(float x) {
  if (x != x) return 0x007FFFFEu;  // NaN: below -inf (0x007FFFFF)
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  u = u == 0x80000000u ? 0u : u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The threshold search and the writes for a row with at most 64 kP
// candidates (its keys in registers, kP planes of 64).  The search stops as
// soon as exactly npick keys reach the value built so far: those are the
// chosen ones.  Otherwise it ends on the npick-th largest key itself, and ties
// with it are taken lowest ids first.
template <int kP>
__device__ __forceinline__ void topk_planes(const float* __restrict__ row, int b, float pre, int lane, int nbmax,
                                            int first, int npick, int32_t* __restrict__ out) {
  uint32_t key[kP];
#pragma unroll
  for (int j = 0; j < kP; ++j) {
    const int c = lane + 64 * j;
    key[j] = 0u;
    if (c >= first && c < b) key[j] = order_key(j == 0 ? pre : (c < nbmax ? row[c] : -INFINITY));
  }
  // every candidate's key is >= 0x007FFFFE and there are more than npick of them
  uint32_t thr = 0u;
  bool exact = false;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = thr | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < kP; ++j) cnt += __popcll(__ballot(key[j] >= cand));
    if (cnt >= npick) {
      thr = cand;
      if (cnt == npick) {
        exact = true;
        break;
      }
    }
  }
  int rem = 0;  // keys equal to thr still to take, lowest ids first
  if (!exact) {
    int above = 0;
#pragma unroll
    for (int j = 0; j < kP; ++j) above += __popcll(__ballot(key[j] > thr));
    rem = npick - above;
  }
  int base = first;
  const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
  for (int j = 0; j < kP; ++j) {
    uint64_t ch = __ballot(exact ? key[j] >= thr : key[j] > thr);
    if (rem > 0) {
      const uint64_t eq = __ballot(key[j] == thr);
      const int k = __popcll(eq);
      uint64_t take = eq;
      if (rem < k) {
        uint64_t rest = eq;
        for (int i = 0; i < rem; ++i) rest &= rest - 1ull;
        take = eq ^ rest;
      }
      rem = rem < k ? 0 : rem - k;
      ch |= take;
    }
    if ((ch >> lane) & 1ull) out[base + __popcll(ch & below)] = lane + 64 * j;
    base += __popcll(ch);
  }
  if (lane == 0) {
    if (first) out[0] = 0;
    out[kTopk - 1] = b;
  }
}

// row: the (token, head) row's scores; b: the token's own block; pre: this
// lane's score of candidate `lane` (loaded by the caller when b >= kTopk)
__device__ __forceinline__ void topk_row(const float* __restrict__ row, int b, float pre, int lane, int nbmax,
                                         int force_init, int32_t* __restrict__ out) {
  if (b < kTopk) {
    if (lane < kTopk) out[lane] = lane <= b ? lane : -1;
    return;
  }
  const int first = force_init ? 1 : 0;  // first candidate block
  const int npick = kTopk - 1 - first;    // blocks chosen by score
  static_assert(kMaxBlocks <= 64 * 16, "top-k planes");
  if (b <= 64)
    topk_planes<1>(row, b, pre, lane, nbmax, first, npick, out);
  else if (b <= 128)
    topk_planes<2>(row, b, pre, lane, nbmax, first, npick, out);
  else if (b <= 256)
    topk_planes<4>(row, b, pre, lane, nbmax, first, npick, out);
  else if (b <= 512)
    topk_planes<8>(row, b, pre, lane, nbmax, first, npick, out);
  else
    topk_planes<16>(row, b, pre, lane, nbmax, first, npick, out);
}

// One wavefront per kTopRows consecutive (token, head) rows; the scores of
// all its rows are loaded before any row is ranked.
constexpr int kTopRows = 1;

__global__ __launch_bounds__(256) void select_topk_kernel(const float* __restrict__ scores,
                                                          const int32_t* __restrict__ cu, int S, int T,
                                                          int Hk, int nbmax, int force_init,
                                                          int32_t* __restrict__ blk_idx) {
  const int lane = threadIdx.x & 63;
  const int64_t r0 = (int64_t)(blockIdx.x * 4 + (threadIdx.x >> 6)) * kTopRows;
  const int64_t nrows = (int64_t)T * Hk;
  if (r0 >= nrows) return;
  int b[kTopRows];
  float pre[kTopRows];
  const int cu_lane = (S < 64 && lane <= S) ? cu[lane] : 0x7fffffff;
#pragma unroll
  for (int e = 0; e < kTopRows; ++e) {
    const int64_t row = min(r0 + e, nrows - 1);
    const int t = (int)(row / Hk);
    const int s = seq_of(cu, S, cu_lane, t);
    const int cs = S < 64 ? __builtin_amdgcn_readlane(cu_lane, s) : cu[s];
    b[e] = __builtin_amdgcn_readfirstlane((t - cs) / kBlock);
    pre[e] = -INFINITY;
    if (b[e] >= kTopk && lane < b[e] && lane < nbmax) pre[e] = scores[row * nbmax + lane];
  }
#pragma unroll
  for (int e = 0; e < kTopRows; ++e)
    if (r0 + e < nrows)
      topk_row(scores + (r0 + e) * nbmax, b[e], pre[e], lane, nbmax, force_init, blk_idx + (r0 + e) * kTopk);
}

}  // namespace

void launch_select(const Sizes& z, const u16* idx_q, int64_t sq_t, int64_t sq_h,
                   const u16* idx_k, int64_t sk_t, int64_t sk_h, const u16* w_q, const u16* w_k,
                   float eps, float rope_base, const int32_t* cu, const PlanBufs& p,
                   bool force_init, u16* qfeat, u16* kfeat, float* scores, int32_t* blk_idx, hipStream_t st) {
  const int T = (int)z.T, Hk = (int)z.Hk, S = (int)z.S;
  {
    KernelTimer timer("select_prologue", st);
    const int64_t waves = (z.T + 1) / 2;
    select_prologue_kernel<<<dim3((unsigned)((waves + kProWaves - 1) / kProWaves + 1)), 64 * kProWaves, 0, st>>>(
        idx_q, sq_t, sq_h, idx_k, sk_t, sk_h, w_q, w_k, eps, rope_freqs(rope_base), cu, S, T, Hk, (int)z.chunk, p,
        qfeat, kfeat);
  }
  const int key_chunk = z.max_seqlen >= kLongKeyChunkSeqlen ? kMaxKeyChunk : kKeyChunk;
  const unsigned kchunks = (unsigned)((z.nbmax + key_chunk - 1) / key_chunk);
  {
    KernelTimer timer("select_scores", st);
    select_scores_kernel<<<dim3((unsigned)z.nblk_cap, kchunks, (unsigned)Hk), 256, 0, st>>>(
        qfeat, kfeat, cu, p.blkbase, p.blk_seq, p.totals, Hk, (int)z.nbmax, key_chunk, scores);
  }
  const int64_t waves_top = (z.T * z.Hk + kTopRows - 1) / kTopRows;
  {
    KernelTimer timer("select_topk", st);
    select_topk_kernel<<<dim3((unsigned)((waves_top + 3) / 4)), 256, 0, st>>>(scores, cu, S, T, Hk, (int)z.nbmax,
                                                                             force_init ? 1 : 0, blk_idx);
  }
}

}  // namespace msa
