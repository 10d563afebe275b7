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
// score registers (B operand) and V^T from the per-block transposed copy that
// block_prep_kernel writes, so every MFMA operand is one 16-byte load.
//
// Key order inside a 32-key step: score tile 2s holds keys 32s + 8g + {0..3}
// and tile 2s+1 keys 32s + 8g + {4..7} in lane group g = lane / 16, so the
// eight P values a lane owns are eight consecutive keys -- the same eight
// consecutive keys the V^T operand reads.
#include "attn_stage.h"
#include "plan_blocks.h"
#include "qk_rope.h"

namespace msa {

namespace {

// Forward tiles: kTPW tokens per wavefront (see the forward kernel below).
template <int kTPW>
struct FwdTile {
  static constexpr int kWaves = kTPW == 1 ? 16 : 8;
  static constexpr int kTok = kWaves * kTPW;        // tokens per tile
  static constexpr int kRuns = 64 / kWaves;         // K and V^T runs staged per wavefront
  static constexpr int kAhead = kTPW == 1 ? 8 : 4;  // operand reads ahead of the MFMAs (register budget)
  static constexpr int kMaxUnion = kTok * kTopk;
};

// Per-(global block, KV head) copies of K and V in the forward's staging
// order, so that every staged 1 KB run is one contiguous copy (a run of raw K
// rows would be sixteen 64-byte pieces).  Keys past the sequence end are zero.
//   kop: run kt*4 + ds, lane li + 16g holding K[key score_key(kt, li)][dims
//        32ds + 8g .. +7] -- the A operand of S^T = K Q^T;
//   vt:  run dt*4 + ks, lane li + 16g holding V[keys 32ks + 8g + 0..7][dim
//        16dt + li] -- the A operand of O^T = V^T P^T.
// kNorm: K is raw; its rows get the attention-side norm and RoPE (qk_rope.h)
// on the way into the staging copy.
template <bool kNorm>
__global__ __launch_bounds__(256) void block_prep_kernel(const u16* __restrict__ k, int64_t k_st, int64_t k_sh,
                                                         const u16* __restrict__ x, int64_t st_t, int64_t st_h,
                                                         const int32_t* __restrict__ cu, int S, int chunk,
                                                         int ntiles, int tile_tok, PlanBufs plan, int Hk,
                                                         QkNormParams nrm, u16* __restrict__ kop,
                                                         u16* __restrict__ xt) {
  // workgroup part p (of 4): K runs 8p .. 8p+7 (key tiles 2p, 2p+1) and the
  // V^T runs of dims 32p .. 32p+31 (runs 8p .. 8p+7).  The last workgroup of
  // the grid instead writes the plan (block numbering, tile launch order) for
  // the forward kernel, so the pass needs no plan launch of its own; the copy
  // workgroups locate their block from cu_seqlens directly.
  __shared__ u16 tile[kBlock][32 + 8];
  __shared__ int loc[2];
  const int gb = blockIdx.x;
  const int h = blockIdx.y;
  const int part = blockIdx.z;
  if (gb == (int)gridDim.x - 1) {
    if (h == 0 && part == 0) {
      __shared__ int sb[256], si[256], hist[kOrderBins], scu[kCuCache];
      plan_blocks<256, kBlock>(cu, S, chunk, plan.blkbase, plan.blk_seq, plan.seqitem, plan.totals, sb, si);
      // the order of the forward's tiles: tile_tok tokens each (ntiles of them)
      if (tile_tok == FwdTile<4>::kTok)
        plan_tile_order<256, 16, FwdTile<4>::kTok>(cu, S, ntiles, plan.tile_order, sb, hist, scu);
      else
        plan_tile_order<256, 16, FwdTile<1>::kTok>(cu, S, ntiles, plan.tile_order, sb, hist, scu);
    }
    return;
  }
  locate_block<kBlock>(cu, S, gb, loc);
  const int s = loc[0];
  if (s < 0) return;
  const int c = loc[1];
  const int seq0 = cu[s];
  const int L = cu[s + 1] - seq0;
  for (int i = threadIdx.x; i < kBlock * 4; i += 256) {
    const int key = i >> 2;
    const int ch = i & 3;
    const int kp = kBlock * c + key;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (kp < L)
      v = *reinterpret_cast<const u32x4*>(x + (int64_t)(seq0 + kp) * st_t + (int64_t)h * st_h + 32 * part + ch * 8);
    *reinterpret_cast<u32x4*>(&tile[key][ch * 8]) = v;
  }
  u16* kdst = kop + ((int64_t)gb * Hk + h) * (kHeadDim * kBlock);
  if constexpr (kNorm) {
    // the part's 32 keys (tiles 2p, 2p+1): each row normalized and rotated by
    // 8 lanes (norm_rope_row8), kept in LDS, then copied in run order
    __shared__ u16 krows[32][kHeadDim + 8];
    {
      const int row = threadIdx.x >> 3, j = threadIdx.x & 7;
      const int kp = kBlock * c + score_key(2 * part + (row >> 4), row & 15);
      float xv[16], w1[16], cs[4], sn[4];
      const u16* src = k + (int64_t)(seq0 + min(kp, L - 1)) * k_st + (int64_t)h * k_sh + 4 * j;
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const uint2 wv = *reinterpret_cast<const uint2*>(src + 32 * qd);
        xv[4 * qd] = __uint_as_float(wv.x << 16);
        xv[4 * qd + 1] = __uint_as_float(wv.x & 0xFFFF0000u);
        xv[4 * qd + 2] = __uint_as_float(wv.y << 16);
        xv[4 * qd + 3] = __uint_as_float(wv.y & 0xFFFF0000u);
#pragma unroll
        for (int e = 0; e < 4; ++e) w1[4 * qd + e] = 1.0f + bf2f(nrm.w_k[32 * qd + 4 * j + e]);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) rope_angle(nrm.fr, 4 * j + e, min(kp, L - 1), cs[e], sn[e]);
      norm_rope_row8(xv, w1, cs, sn, nrm.eps);
#pragma unroll
      for (int qd = 0; qd < 4; ++qd)
#pragma unroll
        for (int e = 0; e < 4; ++e) krows[row][32 * qd + 4 * j + e] = kp < L ? f2bf(xv[4 * qd + e]) : (u16)0;
    }
    __syncthreads();
    for (int i = 512 * part + threadIdx.x; i < 512 * part + 512; i += 256) {
      const int run = i >> 6, ln = i & 63;
      const int row = ((run >> 2) - 2 * part) * 16 + (ln & 15);
      *reinterpret_cast<u32x4*>(kdst + (int64_t)i * 8) =
          *reinterpret_cast<const u32x4*>(&krows[row][32 * (run & 3) + 8 * (ln >> 4)]);
    }
  } else {
    for (int i = 512 * part + threadIdx.x; i < 512 * part + 512; i += 256) {
      const int run = i >> 6, ln = i & 63;
      const int kp = kBlock * c + score_key(run >> 2, ln & 15);
      u32x4 v = {0u, 0u, 0u, 0u};
      if (kp < L)
        v = *reinterpret_cast<const u32x4*>(k + (int64_t)(seq0 + kp) * k_st + (int64_t)h * k_sh + 32 * (run & 3) +
                                            8 * (ln >> 4));
      *reinterpret_cast<u32x4*>(kdst + (int64_t)i * 8) = v;
    }
  }
  __syncthreads();
  u16* dst = xt + ((int64_t)gb * Hk + h) * (kHeadDim * kBlock);
  for (int i = 512 * part + threadIdx.x; i < 512 * part + 512; i += 256) {
    const int run = i >> 6;
    const int lane = i & 63;
    const int d = 16 * (run >> 2) + (lane & 15) - 32 * part;
    const int k0 = 32 * (run & 3) + 8 * (lane >> 4);
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = (uint32_t)tile[k0 + 2 * e][d] | ((uint32_t)tile[k0 + 2 * e + 1][d] << 16);
    *reinterpret_cast<u32x4*>(dst + (int64_t)i * 8) = u32x4{w[0], w[1], w[2], w[3]};
  }
}

// ---------------------------------------------------------------------------
// Forward.  One workgroup per (tile of consecutive tokens, KV head); each
// wavefront owns kTPW tokens of the tile (their q as MFMA B operands, their O
// accumulators and softmax state, all in registers).
//   * kTPW = 1: 16 wavefronts, 16-token tiles.  One token per wavefront keeps
//     a wavefront within 128 registers, so four of them share a SIMD and hide
//     each other's MFMA -> softmax -> MFMA dependency chains.
//   * kTPW = 4: 8 wavefronts of 4 tokens (two per SIMD, 256 registers),
//     32-token tiles.  For long sequences a 16-token tile's union is close to
//     every causal block while each staged block serves few of its tokens
//     (2.5 on the unsharded 32k layer), so the walk is paced by per-step costs;
//     the wider tile walks about 40 % fewer blocks per token there.
//   1. The union of the tile's selected blocks is built in LDS (a bitmap over
//      the tile's global block range, compacted in ascending order).
//   2. The workgroup walks that union.  Each block's K (A operand of
//      S^T = K Q^T) and V^T (A operand of O^T = V^T P^T) are copied into one of
//      two LDS buffers while the previous block is being used; every wavefront
//      then updates its tokens that selected the block.  K and V are read from
//      HBM/L2 once per tile instead of once per token.
// Each token meets its blocks in ascending order with either tile, so the
// results do not depend on the tile.
// ---------------------------------------------------------------------------
constexpr float kRescaleSlack = 8.f;  // log2 units
constexpr int kUnionWords = 34;  // a tile's blocks span fewer than 34 * 32 global ids


template <bool kDense, bool kNorm, int kTPW>
__global__ __launch_bounds__(64 * FwdTile<kTPW>::kWaves) void attn_fwd_kernel(
    const u16* __restrict__ q, int64_t q_st, int64_t q_sh,
    const u16* __restrict__ kop, const u16* __restrict__ vt, const int32_t* __restrict__ blk_idx,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ blkbase, const int32_t* __restrict__ blk_seq,
    const int32_t* __restrict__ tile_order, int S, int T, int Hk, float scale_log2, QkNormParams nrm,
    u16* __restrict__ o, int64_t o_st, int64_t o_sh, float* __restrict__ lse) {
  using Tile = FwdTile<kTPW>;
  constexpr int kTokPerWave = kTPW;
  constexpr int kFwdWaves = Tile::kWaves;
  constexpr int kTileTok = Tile::kTok;
  __shared__ u32x4 kbuf[2][32][64];
  __shared__ u32x4 vbuf[2][32][64];
  __shared__ uint32_t bitmap[kUnionWords];
  // a dense tile's union is up to one sequence's 1024 blocks plus one per later sequence
  constexpr int kUnionCap = kDense ? kUnionWords * 32 : Tile::kMaxUnion;
  __shared__ int ulist[kUnionCap];
  __shared__ int nunion;
  __shared__ float qang[kNorm ? kFwdWaves : 1][64];
  __shared__ float wq1[kNorm ? kHeadDim : 1];

  // workgroup b runs KV head b % Hk of the tile in launch slot b / Hk
  const int h = blockIdx.x % Hk;
  const int t0 = tile_order[blockIdx.x / Hk] * kTileTok;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int li = lane & 15;
  static_assert(!kNorm || kTokPerWave == 1, "the norm assumes one token per wavefront");
  static_assert(kTPW == 1 || kTPW == 4, "16- or 32-token tiles");

  // this lane's (token, slot): token kTokPerWave * wave + g % kTokPerWave, slot li
  const int tj = kTokPerWave * wave + g % kTokPerWave;
  const int t = t0 + tj;
  const bool tvalid = t < T;
  int s_t = 0, pos_t = 0, b_t = -1, my_gb = -1;
  if (tvalid) {
    s_t = find_seq(cu, S, t);
    pos_t = t - cu[s_t];
    b_t = pos_t / kBlock;
    if constexpr (!kDense) {
      const int c = blk_idx[((int64_t)t * Hk + h) * kTopk + li];
      if (c >= 0 && c <= b_t) my_gb = blkbase[s_t] + c;
    }
  }
  const int gb_lo = blkbase[find_seq(cu, S, t0)];

  // the token's q as B operands, loaded before the union build so the loads
  // overlap it
  int tok_t[kTokPerWave];
  bool tok_ok[kTokPerWave];
  bf16x8 qb[kTokPerWave][4];
#pragma unroll
  for (int j = 0; j < kTokPerWave; ++j) {
    tok_t[j] = t0 + kTokPerWave * wave + j;
    tok_ok[j] = tok_t[j] < T;
    const u16* qrow = q + (int64_t)min(tok_t[j], T - 1) * q_st + (int64_t)(h * kGroup + li) * q_sh;
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) qb[j][ds] = tok_ok[j] ? load_bf16x8(qrow + 32 * ds + 8 * g) : zero_bf16x8();
  }
  // the norm's angles and 1 + w_q, formed while the loads are in flight; the
  // union build's barriers publish them
  if constexpr (kNorm) {
    rope_angles_lds(nrm.fr, pos_t, lane, qang[wave]);
    if (threadIdx.x < kHeadDim) wq1[threadIdx.x] = 1.0f + bf2f(nrm.w_q[threadIdx.x]);
  }

  // 1. union of the tile's blocks
  if (threadIdx.x < kUnionWords) bitmap[threadIdx.x] = 0u;
  __syncthreads();
  if constexpr (kDense) {
    if (g < kTokPerWave && tvalid)
      for (int c = li; c <= b_t; c += 16) {
        const int rel = blkbase[s_t] + c - gb_lo;
        atomicOr(&bitmap[rel >> 5], 1u << (rel & 31));
      }
  } else if (g < kTokPerWave && my_gb >= 0 && my_gb - gb_lo < kUnionWords * 32) {
    atomicOr(&bitmap[(my_gb - gb_lo) >> 5], 1u << ((my_gb - gb_lo) & 31));
  }
  __syncthreads();
  if (wave == 0) {
    uint32_t bits = lane < kUnionWords ? bitmap[lane] : 0u;
    const int cnt = __popc(bits);
    int incl = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    int pos = incl - cnt;
    while (bits) {
      const int bit = __ffs(bits) - 1;
      ulist[pos++] = gb_lo + 32 * lane + bit;
      bits &= bits - 1u;
    }
    if (lane == 63) nunion = incl;
  }
  __syncthreads();
  const int nu = nunion;

  if constexpr (kNorm) norm_rope_q_with(qb[0], [&](int d) { return wq1[d]; }, nrm.eps, lane, qang[wave]);

  // per-token state (j = 0, 1 for tokens 2w, 2w+1)
  int tok_pos[kTokPerWave], tok_b[kTokPerWave], tok_base[kTokPerWave];
  f32x4 oacc[kTokPerWave][8];
  float m_run[kTokPerWave], l_run[kTokPerWave];
#pragma unroll
  for (int j = 0; j < kTokPerWave; ++j) {
    tok_pos[j] = __builtin_amdgcn_readlane(pos_t, 16 * j);
    tok_b[j] = __builtin_amdgcn_readlane(b_t, 16 * j);
    tok_base[j] = tok_ok[j] ? blkbase[__builtin_amdgcn_readlane(s_t, 16 * j)] : 0;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) oacc[j][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[j] = -INFINITY;
    l_run[j] = 0.f;
  }

  // 2. walk the union, staging block u+1 while block u is used.  The first
  // half of the wavefronts copies the K runs (kRuns each: keys score_key(w, .),
  // dims 32 ii ..), the second half the V^T runs; each copy is a scalar base
  // plus a lane offset.
  auto stage = [&](int u, int buf) {
    const int gb = __builtin_amdgcn_readfirstlane(ulist[u]);
    const int ln = fresh_lane();
    constexpr int kHalf = kFwdWaves / 2, kR = Tile::kRuns;
    if (wave < kHalf) {
      const u16* base = kop + (((int64_t)gb * Hk + h) * 32 + kR * wave) * 512;
#pragma unroll
      for (int ii = 0; ii < kR; ++ii) dma16s(base + 512 * ii, 16 * ln, lds_offset(&kbuf[buf][kR * wave + ii][0]));
    } else {
      const u16* base = vt + (((int64_t)gb * Hk + h) * 32 + kR * (wave - kHalf)) * 512;
#pragma unroll
      for (int ii = 0; ii < kR; ++ii)
        dma16s(base + 512 * ii, 16 * ln, lds_offset(&vbuf[buf][kR * (wave - kHalf) + ii][0]));
    }
  };
  if (nu > 0) stage(0, 0);
  wait_copies();
  wait_all_loads();
  __syncthreads();

  for (int u = 0; u < nu; ++u) {
    const int buf = u & 1;
    if (u + 1 < nu) stage(u + 1, buf ^ 1);
    const int gb = ulist[u];
    const uint64_t hits = kDense ? 0ull : __ballot(my_gb == gb);
#pragma unroll
    for (int j = 0; j < kTokPerWave; ++j) {
      if (kDense ? (gb < tok_base[j] || gb - tok_base[j] > tok_b[j]) : (((hits >> (16 * j)) & 0xFFFFull) == 0))
        continue;
      const int c = gb - tok_base[j];
      const bool diag = (c == tok_b[j]);
      // Two halves of 64 keys, each a full online-softmax update.  Base 2 on
      // the raw scores: the scale is folded into the exponent's FMA (scale > 0
      // keeps the max); masking only on the query's own block, where a half
      // that starts after the query is skipped.  The running max moves only
      // when a row's new max exceeds it by more than kRescaleSlack: until then
      // P stays below 2^kRescaleSlack, the sums stay consistent with the kept
      // max, and the accumulator rescale is skipped for the whole wavefront.
      // l_run holds this lane's share of the row sum (its keys 8g..8g+7 of
      // every 32); the four shares are added at the end.
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        if (diag && kBlock * c + 64 * hf > tok_pos[j]) break;
        // S^T for the half's four key tiles: the four accumulation chains are
        // interleaved (consecutive MFMAs independent) and the K operand reads
        // run kAhead ahead of the MFMAs that consume them.  The MFMA blocks run
        // at raised wave priority, so on a SIMD whose other wavefronts are in
        // their softmax the matrix unit is fed first (16k pack: 3 % faster)
        f32x4 st[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) st[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
        {
          __builtin_amdgcn_s_setprio(1);
          bf16x8 ka[16];
#pragma unroll
          for (int i = 0; i < 16; ++i)
            ka[i] = __builtin_bit_cast(bf16x8, kbuf[buf][(4 * hf + (i & 3)) * 4 + (i >> 2)][lane]);
#pragma unroll
          for (int i = 0; i < 16; ++i) st[i & 3] = mfma16x16x32(ka[i], qb[j][i >> 2], st[i & 3]);
          __builtin_amdgcn_sched_group_barrier(0x100, Tile::kAhead, 0);
#pragma unroll
          for (int i = 0; i < 16 - Tile::kAhead; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, Tile::kAhead, 0);
        }
        __builtin_amdgcn_s_setprio(0);
        float mx = -INFINITY;
        if (diag) {
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              if (kBlock * c + score_key(4 * hf + kt, 4 * g + r) > tok_pos[j]) st[kt][r] = -INFINITY;
              mx = fmaxf(mx, st[kt][r]);
            }
        } else {
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) mx = fmaxf(mx, st[kt][r]);
        }
        mx = max_over_groups(mx);
        const float m_cand = mx * scale_log2;
        const bool grow = m_cand > m_run[j] + kRescaleSlack;
        const float m_use = grow ? m_cand : m_run[j];
        const float alpha = grow ? fast_exp2(m_run[j] - m_cand) : 1.f;
        float rs = 0.f;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float p = fast_exp2(fmaf(st[kt][r], scale_log2, -m_use));
            st[kt][r] = p;
            rs += p;
          }
        l_run[j] = l_run[j] * alpha + rs;
        m_run[j] = m_use;
        if (__ballot(grow)) {
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) oacc[j][dt] *= alpha;
        }
        const bf16x8 pf0 = pack_bf16x8(st[0], st[1]);
        const bf16x8 pf1 = pack_bf16x8(st[2], st[3]);
        // O^T += V^T P^T: eight independent accumulators per sweep, V operand
        // reads kAhead ahead
        {
          __builtin_amdgcn_s_setprio(1);
          bf16x8 va[16];
#pragma unroll
          for (int i = 0; i < 16; ++i)
            va[i] = __builtin_bit_cast(bf16x8, vbuf[buf][(i & 7) * 4 + 2 * hf + (i >> 3)][lane]);
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[j][i & 7] = mfma16x16x32(va[i], i < 8 ? pf0 : pf1, oacc[j][i & 7]);
          __builtin_amdgcn_sched_group_barrier(0x100, Tile::kAhead, 0);
#pragma unroll
          for (int i = 0; i < 16 - Tile::kAhead; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, Tile::kAhead, 0);
        }
        __builtin_amdgcn_s_setprio(0);
      }
    }
    wait_copies();
    lds_barrier();
  }

#pragma unroll
  for (int j = 0; j < kTokPerWave; ++j) {
    l_run[j] = sum_over_groups(l_run[j]);
    if (!tok_ok[j]) continue;
    const float inv = l_run[j] > 0.f ? 1.0f / l_run[j] : 0.f;
    u16* orow = o + (int64_t)tok_t[j] * o_st + (int64_t)(h * kGroup + li) * o_sh;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<uint2*>(orow + 16 * dt + 4 * g) = pack_bf16x4(oacc[j][dt] * inv);
    if (g == 0)
      lse[(int64_t)tok_t[j] * (Hk * kGroup) + h * kGroup + li] =
          l_run[j] > 0.f ? (m_run[j] + __log2f(l_run[j])) * kLn2 : -INFINITY;
  }
}

}  // namespace

int fwd_tokens_per_wave(const Sizes& z, bool dense, bool nrm) {
  return (!dense && !nrm && z.max_seqlen >= kWideFwdSeqlen) ? 4 : 1;
}

void launch_block_prep(const Sizes& z, const u16* k, int64_t k_st, int64_t k_sh, const u16* v, int64_t v_st,
                       int64_t v_sh, const int32_t* cu, const PlanBufs& p, const QkNormParams* nrm, bool dense,
                       u16* kop, u16* vt, hipStream_t st) {
  KernelTimer timer("block_prep", st);
  const QkNormParams none{};
  auto kern = nrm ? block_prep_kernel<true> : block_prep_kernel<false>;
  const int tile = fwd_tokens_per_wave(z, dense, nrm != nullptr) == 4 ? FwdTile<4>::kTok : FwdTile<1>::kTok;
  kern<<<dim3((unsigned)(z.nblk_cap + 1), (unsigned)z.Hk, 4), 256, 0, st>>>(
      k, k_st, k_sh, v, v_st, v_sh, cu, (int)z.S, (int)z.chunk, (int)((z.T + tile - 1) / tile), tile, p, (int)z.Hk,
      nrm ? *nrm : none, kop, vt);
}

void launch_attn_fwd(const Sizes& z, const u16* q, int64_t q_st, int64_t q_sh,
                     const u16* kop, const u16* vt, const int32_t* blk_idx, const int32_t* cu, const PlanBufs& p,
                     float scale, u16* o, int64_t o_st, int64_t o_sh, float* lse, bool dense, const QkNormParams* nrm,
                     hipStream_t st) {
  KernelTimer timer("attn_fwd", st);
  const QkNormParams none{};
  const bool wide = fwd_tokens_per_wave(z, dense, nrm != nullptr) == 4;
  auto kern = wide ? attn_fwd_kernel<false, false, 4>
                   : (dense ? (nrm ? attn_fwd_kernel<true, true, 1> : attn_fwd_kernel<true, false, 1>)
                            : (nrm ? attn_fwd_kernel<false, true, 1> : attn_fwd_kernel<false, false, 1>));
  const int tile = wide ? FwdTile<4>::kTok : FwdTile<1>::kTok;
  const int waves = wide ? FwdTile<4>::kWaves : FwdTile<1>::kWaves;
  kern<<<(unsigned)(((z.T + tile - 1) / tile) * z.Hk), 64 * waves, 0, st>>>(
      q, q_st, q_sh, kop, vt, blk_idx, cu, p.blkbase, p.blk_seq, p.tile_order, (int)z.S, (int)z.T,
      (int)z.Hk, scale * kLog2e, nrm ? *nrm : none, o, o_st, o_sh, lse);
}

}  // namespace msa
