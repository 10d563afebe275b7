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
// Two pipelines.  Sparse layers (unless the caller asks for the recomputing
// form or the dS would exceed kDsBufMaxBytes): bwd_block_prep (K copies,
// plan) -> bwd_delta_kernel
// (Delta, -LSE log2(e), dK/dV item loads) -> dK/dV, which also writes every
// (selecting query, block)'s dS in bf16 -> dkdv_reduce -> attn_bwd_dq_ds_kernel
// (dQ = scale dS K from the stored dS, one product per selected block instead
// of three).  Dense layers, the fused attention-side norm and the recomputing
// form: bwd_block_prep (K and V copies) -> attn_bwd_dq_kernel (recomputes S
// and dP) -> dK/dV -> dkdv_reduce.
//
// Kernels:
//   attn_bwd_dq_kernel  token-major dQ, tiles of 16 tokens walking the union
//                       of their blocks with K, V and K^T staged in LDS; it
//                       also forms Delta = rowsum(dO * O) and -LSE * log2(e)
//                       for the dK/dV pass;
//   bwd_delta_kernel    Delta and -LSE * log2(e) per (token, query head), and
//                       the dK/dV item loads, ahead of the dK/dV pass;
//   attn_bwd_dq_ds_kernel token-major dQ from the dS the dK/dV pass stored:
//                       the same tiles and union walk with only K^T staged
//                       (bwd_block_prep writes it in operand order);
//   attn_bwd_dkdv_kernel (attn_bwd_dkdv.hip) key-block-major dK/dV per chunk
//                       of selecting queries;
//   dkdv_reduce_kernel  sums the per-chunk slices of a block in chunk order
//                       (fixed order, no atomics: bitwise deterministic) and
//                       writes bf16 dK/dV with their own strides; blocks with a
//                       single chunk were finished by the dK/dV kernel.
#include "attn_stage.h"
#include "plan_blocks.h"
#include "qk_rope.h"

namespace msa {

namespace {

// ---------------------------------------------------------------------------
// dQ.  Same tiling as the forward: one 16-wavefront workgroup per (tile of 16
// consecutive tokens, KV head), wavefront w owning token w (its q and dO as
// MFMA B operands and its dQ^T accumulators in registers, within 128 registers
// so that four wavefronts share a SIMD).  The
// workgroup walks the union of the tile's selected blocks; each block's K and
// V (A operands of S^T = K Q^T and dP^T = V dO^T) are copied into one of two
// LDS buffers while the previous block is used, and the K^T operands of
// dQ^T = K^T dS^T are read transposed from the same K copy.
// ---------------------------------------------------------------------------
constexpr int kTileTok = kAttnTile;

// Per-(global block, KV head) copies of K and V in the dQ pass's staging order,
// so every staged 1 KB run is one contiguous copy: run kt*4 + ds, slot l
// holding x[key score_key(kt, swz_slot(l) % 16)][dims 32ds + 8(l / 16) .. +7]
// (the swizzled stage the transposed K^T reads expect; keys past the sequence
// end are zero).  blockIdx.z: K (0-3) or V (4-7), a quarter of the runs each.
// kNorm: K is raw; its rows get the attention-side norm and RoPE (qk_rope.h)
// on the way into the copy, and the normalized rows are also written to khat
// ([T][Hk][128]) for the dK/dV pass.
// kKt (the stored-dS backward, K only): kop instead gets K^T in the operand
// order of dQ^T = K^T dS^T, run dt * 4 + q (dims 16 dt .., keys 32 q ..) with
// lane (dim 16 dt + l % 16, group l / 16) holding keys 32 q + 8 (l / 16) .. +7,
// transposed through an LDS tile of the part's 32 dims (workgroup part p:
// runs 8p .. 8p+7), so each dQ operand is one plain 16-byte LDS read.
template <bool kNorm, bool kKt = false>
__global__ __launch_bounds__(256) void bwd_block_prep_kernel(const u16* __restrict__ k, int64_t k_st, int64_t k_sh,
                                                             const u16* __restrict__ v, int64_t v_st, int64_t v_sh,
                                                             const int32_t* __restrict__ cu, int S, int chunk,
                                                             int ntiles, PlanBufs plan, int Hk, QkNormParams nrm,
                                                             u16* __restrict__ khat,
                                                             u16* __restrict__ kop, u16* __restrict__ vop,
                                                             int32_t* __restrict__ clear, int nclear) {
  __shared__ int loc[2];
  const int gb = blockIdx.x;
  const int h = blockIdx.y;
  // zero the dK/dV item-load counters the dQ pass accumulates
  {
    const int wg = (blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x;
    const int nwg = gridDim.x * gridDim.y * gridDim.z;
    for (int i = wg * 256 + threadIdx.x; i < nclear; i += nwg * 256) clear[i] = 0;
  }
  // the last workgroup of the grid writes the plan (block numbering, dK/dV
  // work items, tile launch order) for the kernels that follow; the copy
  // workgroups locate their block from cu_seqlens directly
  if (gb == (int)gridDim.x - 1) {
    if (h == 0 && blockIdx.z == 0) {
      __shared__ int sb[256], si[256], hist[kOrderBins], scu[kCuCache];
      plan_blocks<256, kBlock>(cu, S, chunk, plan.blkbase, plan.blk_seq, plan.seqitem, plan.totals, sb, si);
      plan_tile_order<256, 16>(cu, S, ntiles, plan.tile_order, sb, hist, scu);
    }
    return;
  }
  locate_block<kBlock>(cu, S, gb, loc);
  const int s = loc[0];
  if (s < 0) return;
  const int c = loc[1];
  const bool is_v = blockIdx.z >= 4;
  const int part = blockIdx.z & 3;  // runs 8 part .. 8 part + 7
  const u16* x = is_v ? v : k;
  const int64_t st_t = is_v ? v_st : k_st, st_h = is_v ? v_sh : k_sh;
  const int seq0 = cu[s];
  const int L = cu[s + 1] - seq0;
  u16* dst = (is_v ? vop : kop) + ((int64_t)gb * Hk + h) * (kHeadDim * kBlock);
  if constexpr (kKt) {
    static_assert(!kNorm, "the transposed copy serves the plain stored-dS backward");
    __shared__ u16 tile[kBlock][32 + 8];
    for (int i = threadIdx.x; i < kBlock * 4; i += 256) {
      const int key = i >> 2, ch = i & 3;
      const int kp = kBlock * c + key;
      u32x4 val = {0u, 0u, 0u, 0u};
      if (kp < L)
        val = *reinterpret_cast<const u32x4*>(k + (int64_t)(seq0 + kp) * k_st + (int64_t)h * k_sh + 32 * part + 8 * ch);
      *reinterpret_cast<u32x4*>(&tile[key][8 * ch]) = val;
    }
    __syncthreads();
    for (int i = 512 * part + threadIdx.x; i < 512 * part + 512; i += 256) {
      const int run = i >> 6, ln = i & 63;
      const int d = 16 * (run >> 2) + (ln & 15) - 32 * part;
      const int k0 = 32 * (run & 3) + 8 * (ln >> 4);
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = (uint32_t)tile[k0 + 2 * e][d] | ((uint32_t)tile[k0 + 2 * e + 1][d] << 16);
      *reinterpret_cast<u32x4*>(dst + (int64_t)i * 8) = u32x4{w[0], w[1], w[2], w[3]};
    }
    return;
  }
  if constexpr (kNorm) {
    if (!is_v) {
      // the part's 32 keys (tiles 2p, 2p+1): each row normalized and rotated
      // by 8 lanes, kept in LDS, then copied in run order
      __shared__ u16 krows[32][kHeadDim + 8];
      {
        const int row = threadIdx.x >> 3, j = threadIdx.x & 7;
        const int kp = kBlock * c + score_key(2 * part + (row >> 4), row & 15);
        const int kc = min(kp, L - 1);
        float xv[16], w1[16], cs[4], sn[4];
        const u16* src = k + (int64_t)(seq0 + kc) * k_st + (int64_t)h * k_sh + 4 * j;
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
        for (int e = 0; e < 4; ++e) rope_angle(nrm.fr, 4 * j + e, kc, cs[e], sn[e]);
        norm_rope_row8(xv, w1, cs, sn, nrm.eps);
        u16* hrow = khat + ((int64_t)(seq0 + kc) * Hk + h) * kHeadDim + 4 * j;
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          uint32_t pk[2];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const u16 b = kp < L ? f2bf(xv[4 * qd + e]) : (u16)0;
            krows[row][32 * qd + 4 * j + e] = b;
            if (e & 1)
              pk[e >> 1] |= (uint32_t)b << 16;
            else
              pk[e >> 1] = b;
          }
          if (kp < L) *reinterpret_cast<uint2*>(hrow + 32 * qd) = uint2{pk[0], pk[1]};
        }
      }
      __syncthreads();
      for (int i = 512 * part + threadIdx.x; i < 512 * part + 512; i += 256) {
        const int run = i >> 6, ln = i & 63;
        const int row = ((run >> 2) - 2 * part) * 16 + (swz_slot(ln) & 15);
        *reinterpret_cast<u32x4*>(dst + (int64_t)i * 8) =
            *reinterpret_cast<const u32x4*>(&krows[row][32 * (run & 3) + 8 * (ln >> 4)]);
      }
      return;
    }
  }
  for (int i = 512 * part + threadIdx.x; i < 512 * part + 512; i += 256) {
    const int run = i >> 6, ln = i & 63;
    const int kp = kBlock * c + score_key(run >> 2, swz_slot(ln) & 15);
    u32x4 val = {0u, 0u, 0u, 0u};
    if (kp < L)
      val = *reinterpret_cast<const u32x4*>(x + (int64_t)(seq0 + kp) * st_t + (int64_t)h * st_h + 32 * (run & 3) +
                                            8 * (ln >> 4));
    *reinterpret_cast<u32x4*>(dst + (int64_t)i * 8) = val;
  }
}
constexpr int kTokPerWave = 1;
constexpr int kDqWaves = kTileTok / kTokPerWave;
constexpr int kUnionWords = 34;
constexpr int kMaxUnion = kTileTok * kTopk;

// kDense: every causal key of the token's sequence (the dense layers), blk_idx unused.
// kNorm: q is raw.  The token's heads get the attention-side norm and RoPE
// (qk_rope.h) after loading, the normalized rows go to qhat ([T][Hq][128]) for
// the dK/dV pass, and the epilogue takes dq back through the norm:
//     dy = RoPE^T(dq_hat),  g = dy (1 + w),
//     dq = r g - x r^3 (g . x) / 128,   dw_q += sum over heads of dy x r
// with the dw_q sums of the workgroup's 16 tokens and 16 heads added in a fixed
// order into row (tile * Hk + head) of dwq_rows ([rows][256], columns
// 128..255 zero).
template <bool kDense, bool kNorm>
__global__ __launch_bounds__(64 * kDqWaves) void attn_bwd_dq_kernel(
    const u16* __restrict__ q, int64_t q_st, int64_t q_sh,
    const u16* __restrict__ kop, const u16* __restrict__ vop,
    const u16* __restrict__ o, int64_t o_st, int64_t o_sh,
    const u16* __restrict__ dO, int64_t do_st, int64_t do_sh, const float* __restrict__ lse,
    const int32_t* __restrict__ blk_idx, const int32_t* __restrict__ cu, const int32_t* __restrict__ blkbase,
    const int32_t* __restrict__ blk_seq, const int32_t* __restrict__ tile_order, int S, int T, int Hk,
    float scale_log2, float scale,
    u16* __restrict__ dq, int64_t dq_st, int64_t dq_sh, float* __restrict__ delta, float* __restrict__ nlse,
    const int32_t* __restrict__ seqitem, int chunk, int items_cap, int32_t* __restrict__ item_load,
    QkNormParams nrm, u16* __restrict__ qhat, float* __restrict__ dwq_rows) {
  __shared__ u32x4 kbuf[2][32][64];
  __shared__ float qang[kNorm ? kDqWaves : 1][64];
  __shared__ float wq1[kNorm ? kHeadDim : 1];
  static_assert(!kNorm || kTokPerWave == 1, "the norm assumes one token per wavefront");
  __shared__ u32x4 vbuf[2][32][64];
  __shared__ uint32_t bitmap[kUnionWords];
  // a dense tile's union is up to one sequence's 1024 blocks plus one per later sequence
  constexpr int kUnionCap = kDense ? kUnionWords * 32 : kMaxUnion;
  __shared__ int ulist[kUnionCap];
  __shared__ int nunion;

  // workgroup b runs KV head b % Hk of the tile in launch slot b / Hk
  const int h = blockIdx.x % Hk;
  const int tile_id = tile_order[blockIdx.x / Hk];
  const int t0 = tile_id * kTileTok;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int li = lane & 15;
  const int Hq = Hk * kGroup;

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
  // launch order of the dK/dV pass: count this token's selection of its block
  // toward work item (sequence, query chunk, block); the counters were zeroed
  // by the preceding prep kernel
  if constexpr (!kDense) {
    if (g < kTokPerWave && my_gb >= 0) {
      const int j = pos_t / chunk;
      const int item = seqitem[s_t] + (chunk / kBlock) * (j * (j + 1) / 2) + (my_gb - blkbase[s_t]);
      // items_cap is sized from max_seqlen: a sequence longer than that (a
      // broken caller contract) must not count past the array
      if (item < items_cap) atomicAdd(&item_load[(int64_t)h * items_cap + item], 1);
    }
  }

  // the token's q, dO, Delta and LSE, before the union build so the loads overlap it
  int tok_t[kTokPerWave], tok_pos[kTokPerWave], tok_b[kTokPerWave], tok_base[kTokPerWave];
  bool tok_ok[kTokPerWave];
  bf16x8 qb[kTokPerWave][4], db[kTokPerWave][4];
  f32x4 dqacc[kTokPerWave][8];
  float lse2[kTokPerWave], dl[kTokPerWave];
  bool live[kTokPerWave];
#pragma unroll
  for (int j = 0; j < kTokPerWave; ++j) {
    tok_t[j] = t0 + kTokPerWave * wave + j;
    tok_ok[j] = tok_t[j] < T;
    tok_pos[j] = __builtin_amdgcn_readlane(pos_t, 16 * j);
    tok_b[j] = __builtin_amdgcn_readlane(b_t, 16 * j);
    tok_base[j] = tok_ok[j] ? blkbase[__builtin_amdgcn_readlane(s_t, 16 * j)] : 0;
    const int tc = min(tok_t[j], T - 1);
    const u16* qrow = q + (int64_t)tc * q_st + (int64_t)(h * kGroup + li) * q_sh;
    const u16* drow = dO + (int64_t)tc * do_st + (int64_t)(h * kGroup + li) * do_sh;
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) {
      qb[j][ds] = tok_ok[j] ? load_bf16x8(qrow + 32 * ds + 8 * g) : zero_bf16x8();
      db[j][ds] = tok_ok[j] ? load_bf16x8(drow + 32 * ds + 8 * g) : zero_bf16x8();
    }
    const u16* orow = o + (int64_t)tc * o_st + (int64_t)(h * kGroup + li) * o_sh;
    bf16x8 ov[4];
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) ov[ds] = tok_ok[j] ? load_bf16x8(orow + 32 * ds + 8 * g) : zero_bf16x8();
    // the norm's angles and 1 + w_q, formed while the token's loads are in
    // flight; the union build's barriers publish them
    if constexpr (kNorm) {
      rope_angles_lds(nrm.fr, pos_t, lane, qang[wave]);
      if (threadIdx.x < kHeadDim) wq1[threadIdx.x] = 1.0f + bf2f(nrm.w_q[threadIdx.x]);
    }
    const int64_t row = (int64_t)tc * Hq + h * kGroup + li;
    const float l2 = lse[row];
    live[j] = tok_ok[j] && l2 > -INFINITY;
    lse2[j] = live[j] ? l2 * kLog2e : 0.f;
    // Delta = rowsum(dO * O) of head li: this lane's 32 dims (those of its dO
    // operand), then the four row groups
    float dsum = 0.f;
#pragma unroll
    for (int ds = 0; ds < 4; ++ds)
#pragma unroll
      for (int e = 0; e < 8; ++e) dsum += (float)db[j][ds][e] * (float)ov[ds][e];
    dl[j] = sum_over_groups(dsum);
    // Delta and -LSE in base 2 (-inf for a row without keys) for the dK/dV pass
    if (tok_ok[j] && g == 0) {
      delta[row] = dl[j];
      nlse[row] = l2 > -INFINITY ? -l2 * kLog2e : -INFINITY;
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) dqacc[j][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }


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
  const int nsteps = nunion;

  // step u: union block u.  Wavefronts 0-7 copy the four K runs of key tile w
  // (run 4w + ds: keys score_key(w, .), dims 32 ds ..), wavefronts 8-15 the
  // same runs of V; each copy is a scalar base plus a lane offset.
  static_assert(kDqWaves == 16, "four K or V runs per wavefront");
  auto stage = [&](int u, int buf) {
    const int gb = __builtin_amdgcn_readfirstlane(ulist[u]);
    const int ln = fresh_lane();
    const int tile = wave & 7;
    const bool is_k = wave < 8;
    u32x4* dst = is_k ? &kbuf[buf][4 * tile][0] : &vbuf[buf][4 * tile][0];
    const u16* base = (is_k ? kop : vop) + (((int64_t)gb * Hk + h) * 32 + 4 * tile) * 512;
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) dma16s(base + 512 * ds, 16 * ln, lds_offset(dst + 64 * ds));
  };
  if (nsteps > 0) stage(0, 0);
  if constexpr (kNorm) {
    norm_rope_q_with(qb[0], [&](int d) { return wq1[d]; }, nrm.eps, lane, qang[wave]);
    if (tok_ok[0]) {
      u16* hrow = qhat + ((int64_t)tok_t[0] * Hq + h * kGroup + li) * kHeadDim + 8 * g;
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) *reinterpret_cast<u32x4*>(hrow + 32 * ds) = __builtin_bit_cast(u32x4, qb[0][ds]);
    }
  }
  wait_copies();
  wait_all_loads();
  __syncthreads();

  for (int u = 0; u < nsteps; ++u) {
    const int buf = u & 1;
    if (u + 1 < nsteps) stage(u + 1, buf ^ 1);
    const int gb = ulist[u];
    const uint64_t hits = kDense ? 0ull : __ballot(my_gb == gb);
#pragma unroll
    for (int j = 0; j < kTokPerWave; ++j) {
      if (kDense ? (gb < tok_base[j] || gb - tok_base[j] > tok_b[j]) : (((hits >> (16 * j)) & 0xFFFFull) == 0))
        continue;
      const int c = gb - tok_base[j];
      const bool diag = (c == tok_b[j]);
      const int key0 = kBlock * c;
      // four quarters of 32 keys: S^T, dP^T, then dS^T as one B operand of
      // dQ^T; on the own block the quarters after the query are skipped
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        if (diag && key0 + 32 * qq > tok_pos[j]) break;
        // S^T and dP^T: four independent accumulation chains interleaved,
        // K / V operand reads eight ahead of the MFMAs that use them
        f32x4 sacc[2], pacc[2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          sacc[kk] = f32x4{0.f, 0.f, 0.f, 0.f};
          pacc[kk] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        {
          const int swz = swz_slot(lane);
          bf16x8 op[16];  // i = ds * 4 + kk * 2 + (0: K, 1: V)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int run = (2 * qq + ((i >> 1) & 1)) * 4 + (i >> 2);
            op[i] = __builtin_bit_cast(bf16x8, (i & 1) ? vbuf[buf][run][swz] : kbuf[buf][run][swz]);
          }
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int kk = (i >> 1) & 1, ds = i >> 2;
            if (i & 1)
              pacc[kk] = mfma16x16x32(op[i], db[j][ds], pacc[kk]);
            else
              sacc[kk] = mfma16x16x32(op[i], qb[j][ds], sacc[kk]);
          }
          __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
        }
        if (diag || !live[j]) {
#pragma unroll
          for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int key = key0 + score_key(2 * qq + kk, 4 * g + r);
              const float e = fast_exp2(fmaf(sacc[kk][r], scale_log2, -lse2[j]));
              const bool on = live[j] && key <= tok_pos[j];
              sacc[kk][r] = on ? e * (pacc[kk][r] - dl[j]) : 0.f;
            }
        } else {
#pragma unroll
          for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              sacc[kk][r] = fast_exp2(fmaf(sacc[kk][r], scale_log2, -lse2[j])) * (pacc[kk][r] - dl[j]);
        }
        const bf16x8 dsf = pack_bf16x8(sacc[0], sacc[1]);
        {
          // K^T operands read transposed from the K stage: keys 8g .. 8g+7 of
          // the quarter (tiles 2qq, 2qq+1, rows 4g .. 4g+3) at dim 16dt + li
          const uint32_t kq = lds_offset(&kbuf[buf][8 * qq][0]) + tr_lane_offset(fresh_lane());
          bf16x8 ta[8];
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) {
            const uint32_t off = kq + (dt >> 1) * 1024 + (dt & 1) * 512;
            const uint2 lo = read_tr16(off), hi = read_tr16(off + 4096);
            ta[dt] = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
          }
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) dqacc[j][dt] = mfma16x16x32(ta[dt], dsf, dqacc[j][dt]);
          __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
        }
      }
    }
    wait_copies();
    lds_barrier();
  }

  if constexpr (kNorm) {
    // the lane holds dims 16 dt + 4 g + r of head li; pairs (i, i + 32) of the
    // rotation sit in dt and dt + 2 of the same lane
#pragma clang fp contract(off)
    float x[8][4], dy[8][4];
    float ss = 0.f;
    {
      const int tc = min(tok_t[0], T - 1);
      const u16* qrow = q + (int64_t)tc * q_st + (int64_t)(h * kGroup + li) * q_sh;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const uint2 wv = *reinterpret_cast<const uint2*>(qrow + 16 * dt + 4 * g);
        x[dt][0] = __uint_as_float(wv.x << 16);
        x[dt][1] = __uint_as_float(wv.x & 0xFFFF0000u);
        x[dt][2] = __uint_as_float(wv.y << 16);
        x[dt][3] = __uint_as_float(wv.y & 0xFFFF0000u);
#pragma unroll
        for (int r = 0; r < 4; ++r) ss += x[dt][r] * x[dt][r];
      }
    }
    ss = sum_over_groups(ss);
    const float rr = 1.0f / sqrtf(ss * (1.0f / 128.0f) + nrm.eps);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) dy[dt][r] = dqacc[0][dt][r] * scale;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * dt + 4 * g + r;
        const float c = qang[wave][i], sn = qang[wave][32 + i];
        const float a = dy[dt][r], b = dy[dt + 2][r];
        dy[dt][r] = (c * a) + (sn * b);
        dy[dt + 2][r] = (c * b) - (sn * a);
      }
    float gr[8][4];
    float dot = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        gr[dt][r] = dy[dt][r] * wq1[16 * dt + 4 * g + r];
        dot += gr[dt][r] * x[dt][r];
      }
    dot = sum_over_groups(dot);
    const float k3 = rr * rr * rr * dot * (1.0f / 128.0f);
    if (tok_ok[0]) {
      u16* out = dq + (int64_t)tok_t[0] * dq_st + (int64_t)(h * kGroup + li) * dq_sh;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        f32x4 dx;
#pragma unroll
        for (int r = 0; r < 4; ++r) dx[r] = (rr * gr[dt][r]) - (x[dt][r] * k3);
        *reinterpret_cast<uint2*>(out + 16 * dt + 4 * g) = pack_bf16x4(dx);
      }
    }
    // dw_q: the token's 16 heads (the 16 lanes li of a row) added by a
    // shift-and-add scan within the row (DPP row_shr 1, 2, 4, 8 with zero
    // fill: lane li ends with the sum over heads 0..li, lane 15 with the
    // row's total), then the 16 tokens (wavefronts) in order; the K stage is
    // free by now
    float* red = reinterpret_cast<float*>(&kbuf[0][0][0]);  // [kDqWaves][128]
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float a = tok_ok[0] ? (dy[dt][r] * x[dt][r]) * rr : 0.f;
        a += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0x111, 0xF, 0xF, true));
        a += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0x112, 0xF, 0xF, true));
        a += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0x114, 0xF, 0xF, true));
        a += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0x118, 0xF, 0xF, true));
        if (li == 15) red[wave * kHeadDim + 16 * dt + 4 * g + r] = a;
      }
    __syncthreads();
    if (threadIdx.x < 256) {
      float acc = 0.f;
      if (threadIdx.x < kHeadDim)
#pragma unroll
        for (int w = 0; w < kDqWaves; ++w) acc += red[w * kHeadDim + threadIdx.x];
      dwq_rows[((int64_t)tile_id * Hk + h) * 256 + threadIdx.x] = acc;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kTokPerWave; ++j) {
      if (!tok_ok[j]) continue;
      u16* out = dq + (int64_t)tok_t[j] * dq_st + (int64_t)(h * kGroup + li) * dq_sh;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        *reinterpret_cast<uint2*>(out + 16 * dt + 4 * g) = pack_bf16x4(dqacc[j][dt] * scale);
    }
  }
}

// ---------------------------------------------------------------------------
// Delta = rowsum(dO * O) and -LSE * log2(e) (-inf for a row without keys) per
// (token, query head) for the dK/dV pass, and each (token, listed block)
// counted toward its dK/dV work item's load (the counters were zeroed by the
// prep kernel).  Workgroup per (16 consecutive tokens, KV head), wavefront w
// taking token w: lane (head li, group g) sums dims 32 ds + 8 g .. +7 of its
// head, the same lanes and order as the dQ kernel's prologue.  The counts of
// the tokens in the first token's (sequence, query chunk) are gathered in an
// LDS histogram over its blocks and added with one global atomic per block;
// other tokens (a tile crossing a chunk or sequence) add theirs directly.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void bwd_delta_kernel(
    const u16* __restrict__ o, int64_t o_st, int64_t o_sh, const u16* __restrict__ dO, int64_t do_st,
    int64_t do_sh, const float* __restrict__ lse, const int32_t* __restrict__ blk_idx,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ seqitem, int S, int T, int Hk, int chunk,
    int items_cap, float* __restrict__ delta, float* __restrict__ nlse, int32_t* __restrict__ item_load) {
  constexpr int kHistBins = kMaxBlocks;
  __shared__ int hist[kHistBins];
  const int h = blockIdx.y;
  const int t0 = blockIdx.x * 16;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int li = lane & 15;
  const int t = t0 + wave;
  for (int i = threadIdx.x; i < kHistBins; i += 1024) hist[i] = 0;
  const int s0 = find_seq(cu, S, t0);
  const int j0 = (t0 - cu[s0]) / chunk;
  const int base0 = seqitem[s0] + (chunk / kBlock) * (j0 * (j0 + 1) / 2);
  __syncthreads();
  if (t < T) {
    const u16* orow = o + (int64_t)t * o_st + (int64_t)(h * kGroup + li) * o_sh;
    const u16* drow = dO + (int64_t)t * do_st + (int64_t)(h * kGroup + li) * do_sh;
    bf16x8 db[4], ov[4];
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) {
      db[ds] = load_bf16x8(drow + 32 * ds + 8 * g);
      ov[ds] = load_bf16x8(orow + 32 * ds + 8 * g);
    }
    const int64_t row = (int64_t)t * (Hk * kGroup) + h * kGroup + li;
    const float l2 = lse[row];
    const int s = find_seq(cu, S, t);
    const int pos = t - cu[s];
    const int c = blk_idx[((int64_t)t * Hk + h) * kTopk + li];
    float dsum = 0.f;
#pragma unroll
    for (int ds = 0; ds < 4; ++ds)
#pragma unroll
      for (int e = 0; e < 8; ++e) dsum += (float)db[ds][e] * (float)ov[ds][e];
    const float dl = sum_over_groups(dsum);
    if (g == 0) {
      delta[row] = dl;
      nlse[row] = l2 > -INFINITY ? -l2 * kLog2e : -INFINITY;
      if (c >= 0 && c <= pos / kBlock) {
        const int j = pos / chunk;
        if (s == s0 && j == j0) {
          atomicAdd(&hist[c], 1);
        } else {
          const int item = seqitem[s] + (chunk / kBlock) * (j * (j + 1) / 2) + c;
          // items_cap is sized from max_seqlen: a sequence longer than that
          // (a broken caller contract) must not count past the array
          if (item < items_cap) atomicAdd(&item_load[(int64_t)h * items_cap + item], 1);
        }
      }
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kHistBins; i += 1024) {
    const int n = hist[i];
    if (n > 0 && base0 + i < items_cap) atomicAdd(&item_load[(int64_t)h * items_cap + base0 + i], n);
  }
}

// ---------------------------------------------------------------------------
// dQ from the stored dS.  The dK/dV pass left, for every (token, KV head,
// listed block), the block's bf16 dS as its score registers held it: quarter
// qq (keys 32 qq .. +31) as two runs of 64 lanes x 8 bytes, lane (key li,
// group g) of run x holding heads 4g .. 4g+3 of key 32 qq + 16 x + li
// (ds_buf[((t Hk + h) 16 + slot) 4 + qq][x][lane], slot = the block's first
// position in the token's list).  dQ^T = K^T dS^T wants dS^T as the B operand,
// lane (head s, group gg) holding keys 32 qq + 8 gg .. +7 of head s: each
// quarter is written to a 1 KB LDS slot of the wavefront and read back with
// ds_read_b64_tr_b16.  The tiling and union walk are the dQ kernel's with only
// K^T staged, from the prep kernel's copy in operand order (each A operand one
// 16-byte read), in a ring of four buffers: block u + 2 is copied while block
// u is used, and a barrier follows only every second step (there each
// wavefront waits for the copies of the next two blocks; 16k pack dQ 237 ->
// 224 us, unsharded 32k layer 4.16 -> 3.35 ms).  Each wavefront's dS loads
// run two of its own blocks ahead, and a step's own dS loads (issued after
// its copies) stay in flight across that wait (loads and copies complete in
// issue order).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64 * kDqWaves) void attn_bwd_dq_ds_kernel(
    const u16* __restrict__ kop, const u16* __restrict__ ds_buf, const int32_t* __restrict__ blk_idx,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ blkbase, const int32_t* __restrict__ tile_order,
    int S, int T, int Hk, float scale, u16* __restrict__ dq, int64_t dq_st, int64_t dq_sh) {
  __shared__ u32x4 kbuf[4][32][64];
  __shared__ u32x4 dsx[kDqWaves][1][64];
  __shared__ uint32_t bitmap[kUnionWords];
  __shared__ int ulist[kMaxUnion];
  __shared__ int nunion;

  const int h = blockIdx.x % Hk;
  const int tile_id = tile_order[blockIdx.x / Hk];
  const int t0 = tile_id * kTileTok;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int li = lane & 15;

  // The dS transpose.  Lane l loads bytes 16 l .. of the quarter (the 8-byte
  // pieces of lanes 2l, 2l+1 of run l / 32) and writes them to 16-byte slot
  // sigma(l) = l ^ 2 (l / 16 % 2) of the wavefront's 1 KB.  ds_read_b64_tr_b16
  // hands output lane i of a 16-lane group element e of source lane 4e + i/4,
  // whose 4 bf16 must then be heads 4(i/4) .. of one key: source lane j of
  // group gg points at key 8 gg + j/4 (+4 for the second read), heads
  // 4(j%4) .., i.e. at the piece of lane L = key % 16 + 16 (j%4) of run
  // key / 16, held by loading lane 32 (key / 16) + L / 2 at byte 8 (L % 2).
  // With sigma, the 32 reads of each half wavefront touch every bank once and
  // each 16-lane write touches 16 distinct slots.
  const uint32_t ds_wr = (uint32_t)(16 * (lane ^ (2 * (g & 1))));
  auto ds_rd = [&](int key) {
    const int L = (key & 15) + 16 * (li & 3);
    const int lp = 32 * (key >> 4) + (L >> 1);
    return (uint32_t)(16 * (lp ^ (2 * ((lp >> 4) & 1))) + 8 * (L & 1));
  };
  const uint32_t ds_rd0 = ds_rd(8 * g + (li >> 2)), ds_rd1 = ds_rd(8 * g + 4 + (li >> 2));

  const int t = t0 + wave;
  const bool tvalid = t < T;
  int s_t = 0, pos_t = 0, b_t = -1, my_gb = -1;
  if (tvalid && g == 0) {
    s_t = find_seq(cu, S, t);
    pos_t = t - cu[s_t];
    b_t = pos_t / kBlock;
    const int c = blk_idx[((int64_t)t * Hk + h) * kTopk + li];
    if (c >= 0 && c <= b_t) my_gb = blkbase[s_t] + c;
  }
  const int gb_lo = blkbase[find_seq(cu, S, t0)];
  const int tok_pos = __builtin_amdgcn_readlane(pos_t, 0);
  const int tok_b = __builtin_amdgcn_readlane(b_t, 0);
  const int tok_base = tvalid ? blkbase[__builtin_amdgcn_readlane(s_t, 0)] : 0;

  // the token's blocks in the order the walk meets them (ascending global id),
  // each at the first list position holding it: lane li (group 0) gets the
  // rank of its entry, or -1 for a hole or a repeat
  int rank = -1;
  {
    bool first = my_gb >= 0;
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (j < li && __builtin_amdgcn_readlane(my_gb, j) == my_gb) first = false;
    const int fg = first ? my_gb : 0x7fffffff;
    int r = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) r += __builtin_amdgcn_readlane(fg, j) < fg ? 1 : 0;
    if (first && g == 0) rank = r;
  }
  // the token's 16 x 4 KB of dS through a buffer resource: a load at an offset
  // past its 64 KB (no block of that rank, or no token) returns zeros without
  // reading memory, so every hit issues the same loads
  const __amdgpu_buffer_rsrc_t dsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(ds_buf + (((int64_t)(tvalid ? t : 0) * Hk + h) * kTopk) * 4 * 512), (short)0,
      tvalid ? kTopk * 4096 : 0, 0x00020000);
  // loads the dS of the k-th block the walk will meet (zeros when there is
  // none); non-temporal: each dS is read once
  constexpr int kNonTemporal = 2;  // the cache-policy bit of a streaming access
  auto load_ds = [&](int k, bf16x8* dst) {
    const uint64_t m = __ballot(rank == k);
    const int slot = m != 0ull ? __builtin_ctzll(m) : 0;
    // on the token's own block the quarters after the query are skipped by
    // the walk (and were not stored): they are not read either
    const int c = __builtin_amdgcn_readlane(my_gb, slot) - tok_base;
    const int qlast = m == 0ull ? -1 : (c == tok_b ? (tok_pos - kBlock * c) >> 5 : 3);
    const int off = slot * 4096 + 16 * fresh_lane();
#pragma unroll
    for (int qq = 0; qq < 4; ++qq)
      dst[qq] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                               dsrc, qq <= qlast ? off + 1024 * qq : kTopk * 4096, 0, kNonTemporal));
  };

  // union of the tile's blocks
  if (threadIdx.x < kUnionWords) bitmap[threadIdx.x] = 0u;
  __syncthreads();
  if (g == 0 && my_gb >= 0 && my_gb - gb_lo < kUnionWords * 32)
    atomicOr(&bitmap[(my_gb - gb_lo) >> 5], 1u << ((my_gb - gb_lo) & 31));
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
  const int nsteps = nunion;

  // wavefronts 0-7 copy the K^T runs 4w .. 4w+3 (dims 16 w .., the block's
  // four key quarters)
  const bool stager = wave < 8;
  auto stage = [&](int u, int buf) {
    if (!stager) return;
    const int gb = __builtin_amdgcn_readfirstlane(ulist[u]);
    const int ln = fresh_lane();
    const u16* base = kop + (((int64_t)gb * Hk + h) * 32 + 4 * wave) * 512;
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) dma16s(base + 512 * ds, 16 * ln, lds_offset(&kbuf[buf][4 * wave + ds][0]));
  };
  // three dS buffers in turn: block k's in buffer k % 3
  bf16x8 ds0[4], ds1[4], ds2[4];
#pragma unroll
  for (int qq = 0; qq < 4; ++qq) ds0[qq] = ds1[qq] = ds2[qq] = zero_bf16x8();
  load_ds(0, ds0);
  load_ds(1, ds1);
  f32x4 dqacc[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) dqacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (nsteps > 0) stage(0, 0);
  if (nsteps > 1) stage(1, 1);
  wait_copies();
  wait_all_loads();
  __syncthreads();

  int k = 0;              // blocks of the token met so far
  int buf = 0;            // u % 4
  int u = 0;
  auto is_hit = [&]() { return __ballot(my_gb == ulist[u]) != 0ull; };
  // block u + 2's copies into the buffer block u - 2 used; whether this
  // wavefront issued any
  auto stage_ahead = [&]() {
    if (u + 2 < nsteps) stage(u + 2, (buf + 2) & 3);
    return stager && u + 2 < nsteps;
  };
  // A barrier after every odd step (and the last): there each wavefront waits
  // for its copies of blocks u + 1 and u + 2 (issued in this step and the one
  // before), leaving only this step's dS loads (issued after them) in flight,
  // so both blocks are visible before the next two steps; the buffer a step
  // refills (block u - 2's) was released by the barrier after step u - 2 or
  // u - 1, whichever is odd.
  auto end_step = [&](bool staging, bool hit) {
    (void)staging;
    if ((u & 1) || u + 1 == nsteps) {
      if (hit)
        asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
      else
        wait_copies();
      lds_barrier();
    }
    buf = (buf + 1) & 3;
    ++u;
  };
  // steps up to the token's next block; false when the walk ends first
  auto skip_to_hit = [&]() {
    while (u < nsteps) {
      if (is_hit()) return true;
      end_step(stage_ahead(), false);
    }
    return false;
  };
  // the step of block k: its dS (loaded two blocks ago, in cur) times K^T;
  // block k + 2's dS loads into nxt (the buffer block k - 1 used)
  auto hit_step = [&](bf16x8 (&cur)[4], bf16x8 (&nxt)[4]) {
    // take cur before the next copy is issued, so that waiting for it never
    // waits for that copy
    asm volatile("" ::"v"(cur[0]), "v"(cur[1]), "v"(cur[2]), "v"(cur[3]));
    const bool staging = stage_ahead();
    load_ds(k + 2, nxt);
    const int c = ulist[u] - tok_base;
    const bool diag = (c == tok_b);
    const int key0 = kBlock * c;
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      if (diag && key0 + 32 * qq > tok_pos) break;
      bf16x8 bop;
      {
        const uint32_t slot = lds_offset(&dsx[wave][0][0]);
        dsx[wave][0][ds_wr / 16] = __builtin_bit_cast(u32x4, cur[qq]);
        const uint2 lo = read_tr16(slot + ds_rd0), hi = read_tr16(slot + ds_rd1);
        bop = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
      }
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        dqacc[dt] = mfma16x16x32(__builtin_bit_cast(bf16x8, kbuf[buf][4 * dt + qq][lane]), bop, dqacc[dt]);
    }
    ++k;
    end_step(staging, true);
  };
  // three phases, one per buffer role, so every buffer has one load site
  for (;;) {
    if (!skip_to_hit()) break;
    hit_step(ds0, ds2);
    if (!skip_to_hit()) break;
    hit_step(ds1, ds0);
    if (!skip_to_hit()) break;
    hit_step(ds2, ds1);
  }
  if (tvalid) {
    u16* out = dq + (int64_t)t * dq_st + (int64_t)(h * kGroup + li) * dq_sh;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<uint2*>(out + 16 * dt + 4 * g) = pack_bf16x4(dqacc[dt] * scale);
  }
}

// ---------------------------------------------------------------------------
// Ordered reduction of the per-chunk slices of one (block, KV head).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void dkdv_reduce_kernel(
    const float* __restrict__ part_dk, const float* __restrict__ part_dv, const int32_t* __restrict__ item_count,
    const int32_t* __restrict__ seqitem, const int32_t* __restrict__ blk_seq, const int32_t* __restrict__ blkbase,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ totals, int Hk, int chunk, int items_cap, float scale,
    u16* __restrict__ dk, int64_t dk_st, int64_t dk_sh, u16* __restrict__ dv, int64_t dv_st, int64_t dv_sh) {
  // eight keys per workgroup and up to eight chunk slices in flight per
  // thread, so a block summed over many chunks is not left to few threads
  // (16k pack 28.5 -> 25.4 us)
  constexpr int kKeys = 8;    // keys of the block per workgroup
  constexpr int kBatch = 8;   // chunk slices loaded before any is added
  const int gb = blockIdx.x;
  const int slice = blockIdx.y;
  const int h = blockIdx.z;
  if (gb >= totals[0]) return;
  const int s = blk_seq[gb];
  const int c = gb - blkbase[s];
  const int seq0 = cu[s];
  const int L = cu[s + 1] - seq0;
  const int nch = (L + chunk - 1) / chunk;
  const int jmin = (kBlock * c) / chunk;
  if (jmin == nch - 1) return;  // a block with one work item was written by the dK/dV kernel itself
  const int item0 = seqitem[s];
  const int m = chunk / kBlock;  // blocks per full chunk: chunk j's items start at item0 + m j (j + 1) / 2
  // this thread's 4 elements of the kKeys keys x 128 dims
  const int eg = slice * kKeys * kHeadDim + threadIdx.x * 4;
  const int kp = kBlock * c + eg / kHeadDim;
  f32x4 adk = f32x4{0.f, 0.f, 0.f, 0.f}, adv = adk;
  for (int j0 = jmin; j0 < nch; j0 += kBatch) {
    int cnt[kBatch];
    int64_t off[kBatch];
#pragma unroll
    for (int w = 0; w < kBatch; ++w) {
      const int j = min(j0 + w, nch - 1);
      const int it = item0 + m * (j * (j + 1) / 2) + c;
      const bool ok = j0 + w < nch && it < items_cap;
      const int itc = ok ? it : 0;
      cnt[w] = ok ? item_count[(int64_t)h * items_cap + itc] : 0;
      off[w] = ((int64_t)h * items_cap + itc) * (kBlock * kHeadDim);
    }
    f32x4 pk[kBatch], pv[kBatch];
#pragma unroll
    for (int w = 0; w < kBatch; ++w) {
      pk[w] = *reinterpret_cast<const f32x4*>(part_dk + off[w] + eg);
      pv[w] = *reinterpret_cast<const f32x4*>(part_dv + off[w] + eg);
    }
#pragma unroll
    for (int w = 0; w < kBatch; ++w)
      if (cnt[w] != 0) {
        adk += pk[w];
        adv += pv[w];
      }
  }
  if (kp < L) {
    const int d = eg % kHeadDim;
    *reinterpret_cast<uint2*>(dk + (int64_t)(seq0 + kp) * dk_st + (int64_t)h * dk_sh + d) = pack_bf16x4(adk * scale);
    *reinterpret_cast<uint2*>(dv + (int64_t)(seq0 + kp) * dv_st + (int64_t)h * dv_sh + d) = pack_bf16x4(adv);
  }
}

}  // namespace

void launch_attn_bwd(const Sizes& z, const BwdArgs& a, const PlanBufs& p, hipStream_t st) {
  const int T = (int)z.T, Hk = (int)z.Hk, S = (int)z.S;
  const QkNormParams none{};
  if (a.ds) {
    // sparse, no fused norm: dK/dV first (storing dS), then dQ from the stored dS
    {
      KernelTimer timer("bwd_block_prep", st);
      bwd_block_prep_kernel<false, true><<<dim3((unsigned)(z.nblk_cap + 1), (unsigned)Hk, 4), 256, 0, st>>>(
          a.k, a.k_st, a.k_sh, a.v, a.v_st, a.v_sh, a.cu, S, (int)z.chunk, (int)z.ntiles, p, Hk, none, nullptr,
          a.kop, nullptr, a.item_load, (int)(z.Hk * z.items_cap));
    }
    {
      KernelTimer timer("bwd_delta", st);
      bwd_delta_kernel<<<dim3((unsigned)((z.T + 15) / 16), (unsigned)Hk), 1024, 0, st>>>(
          a.o, a.o_st, a.o_sh, a.dO, a.do_st, a.do_sh, a.lse, a.blk_idx, a.cu, p.seqitem, S, T, Hk, (int)z.chunk,
          (int)z.items_cap, a.delta, a.nlse, a.item_load);
    }
    launch_attn_bwd_dkdv(z, a, p, st);
    {
      KernelTimer timer("dkdv_reduce", st);
      dkdv_reduce_kernel<<<dim3((unsigned)z.nblk_cap, kBlock / 8, (unsigned)Hk), 256, 0, st>>>(
          a.part_dk, a.part_dv, a.item_count, p.seqitem, p.blk_seq, p.blkbase, a.cu, p.totals, Hk, (int)z.chunk,
          (int)z.items_cap, a.scale, a.dk, a.dk_st, a.dk_sh, a.dv, a.dv_st, a.dv_sh);
    }
    {
      KernelTimer timer("attn_bwd_dq", st);
      attn_bwd_dq_ds_kernel<<<(unsigned)(z.ntiles * Hk), 64 * kDqWaves, 0, st>>>(
          a.kop, a.ds, a.blk_idx, a.cu, p.blkbase, p.tile_order, S, T, Hk, a.scale, a.dq, a.dq_st, a.dq_sh);
    }
    return;
  }
  {
    KernelTimer timer("bwd_block_prep", st);
    auto kern = a.nrm ? bwd_block_prep_kernel<true> : bwd_block_prep_kernel<false>;
    kern<<<dim3((unsigned)(z.nblk_cap + 1), (unsigned)Hk, 8), 256, 0, st>>>(
        a.k, a.k_st, a.k_sh, a.v, a.v_st, a.v_sh, a.cu, (int)z.S, (int)z.chunk, (int)z.ntiles, p, Hk,
        a.nrm ? *a.nrm : none, a.khat, a.kop, a.vop, a.item_load, (int)(z.Hk * z.items_cap));
  }
  {
    KernelTimer timer("attn_bwd_dq", st);
    auto kern = a.nrm ? (a.dense ? attn_bwd_dq_kernel<true, true> : attn_bwd_dq_kernel<false, true>)
                      : (a.dense ? attn_bwd_dq_kernel<true, false> : attn_bwd_dq_kernel<false, false>);
    kern<<<(unsigned)(z.ntiles * Hk), 64 * kDqWaves, 0, st>>>(
        a.q, a.q_st, a.q_sh, a.kop, a.vop, a.o, a.o_st, a.o_sh, a.dO, a.do_st,
        a.do_sh, a.lse, a.blk_idx, a.cu, p.blkbase, p.blk_seq, p.tile_order, S, T, Hk, a.scale * kLog2e, a.scale,
        a.dq, a.dq_st,
        a.dq_sh, a.delta, a.nlse, p.seqitem, (int)z.chunk, (int)z.items_cap, a.item_load, a.nrm ? *a.nrm : none,
        a.qhat, a.dwq_rows);
  }
  launch_attn_bwd_dkdv(z, a, p, st);
  {
    KernelTimer timer("dkdv_reduce", st);
    dkdv_reduce_kernel<<<dim3((unsigned)z.nblk_cap, kBlock / 8, (unsigned)Hk), 256, 0, st>>>(
        a.part_dk, a.part_dv, a.item_count, p.seqitem, p.blk_seq, p.blkbase, a.cu, p.totals, Hk, (int)z.chunk,
        (int)z.items_cap, a.scale, a.dk, a.dk_st, a.dk_sh, a.dv, a.dv_st, a.dv_sh);
  }
}

}  // namespace msa
