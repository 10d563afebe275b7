// Narrow-block variant of the block-sparse GQA attention on gfx950: the same
// attention as the wide kernels (attn_fwd.hip, attn_bwd*.hip) for the pages'
// second workload, 4-token blocks with head dim 256 and 12 query heads per KV
// head (radixark/miles PR #4581, kernel-tuning commit message: launch configs
// per block width, narrow = qwen3.8-next's 4-token blocks; 12 q / 1 kv head,
// D 256, 16k-token packs).
//
// What is computed is the wide variant's definition with 4-token blocks: for
// token t, query head g and KV head h = g / 12, the keys are every key j <= t
// of the blocks listed in blk_idx[t, h, :] (sequence-local 4-token block ids,
// any order, -1 padding; ids past t's own block are ignored, duplicates count
// once); O = softmax(scale q.k) v with the natural-log LSE; the backward gives
// dq, dk, dv of sum(O * dO).
//
// Tiling.  A query lists hundreds of 4-token blocks, far too small to stage
// one at a time, so keys are staged in tiles of 64 (16 blocks): the kernels
// walk key tiles and mask, per query, the blocks it did not list.  Selections
// arrive as a per-(token, KV head) bitmap over the sequence's blocks
// (qsa_bitmap_kernel), 16 bits per key tile.
//   forward   one 12-wavefront workgroup per (16 consecutive tokens, KV head):
//             the tile's 192 (token, head) rows packed 16 per wavefront as the
//             MFMA columns (q as B operands, O^T in registers), so no padding
//             heads are computed; the workgroup walks the union of its tokens'
//             key tiles with K and V^T staged in LDS, double buffered;
//   Delta     Delta = rowsum(dO*O) and -LSE * log2(e) per (token, head);
//   dK/dV     key-tile major: one workgroup per (sequence, query chunk, key
//             tile), four wavefronts of 16 keys with K and V in registers,
//             streaming the (selecting token, query head) rows of the chunk
//             through LDS 32 at a time, so a step mixes tokens and carries no
//             padding heads; chunk slices are summed in chunk order by
//             qsa_reduce_kernel (fixed order, no atomics).  It also stores the
//             bf16 dS of each (token, causal key tile, KV head, query head) it
//             covers as one whole 128-byte line (its 64 keys, zero where the
//             token listed nothing), at a slot found in closed form from the
//             token's position;
//   dQ        the forward's tiling and row packing over the stored dS: only K
//             is staged (K^T read transposed), and dQ^T = K^T dS^T is one
//             product per listed block instead of three.
#include "attn_stage.h"
#include "plan_blocks.h"

namespace msa {

namespace {

constexpr int kD = kQsaHeadDim;   // 256
constexpr int kG = kQsaGroup;     // 12
constexpr int kKT = kQsaKeyTile;  // 64
constexpr int kWords = kQsaWords; // 256
constexpr int kQTok = kAttnTile;  // tokens per forward / dQ workgroup (16)
constexpr int kRowWaves = kQTok * kG / 16;  // their wavefronts: the tile's 192 (token, head) rows, 16 each
constexpr int kDqTrAhead = 3;  // dQ: transposed K^T operands read ahead of their MFMAs
constexpr int kUnionWords = 32;   // a tile's key tiles span fewer than 1024 global ids
constexpr int kUnionMax = kUnionWords * 32;
constexpr float kRescaleSlack = 8.f;  // log2 units

// 16-bit mask of the blocks of key tile c (sequence-local) in a bitmap row.
__device__ __forceinline__ uint32_t tile_mask(const uint32_t* row, int c) {
  return (row[c >> 1] >> (16 * (c & 1))) & 0xFFFFu;
}

// ---------------------------------------------------------------------------
// Selection bitmaps: one wavefront per (token, KV head); bit b of the row is
// set when block b is listed and b <= the token's own block.
// ---------------------------------------------------------------------------
// Workgroup (0, 0) writes the plan (64-key tile numbering, dK/dV work items,
// token tile launch order) for the kernels that follow, so the narrow passes
// need no plan launch of their own; dispatched first, it runs beside the
// bitmap workgroups instead of after them.
// dS slots of the backward: a token at sequence position p owns one slot per
// key tile c <= p / 64, the slots of a sequence's tokens in position order, so
// the positions before p hold slots_before(p) of them.  dsbase (optional, the
// backward's) receives each sequence's first slot ([S+1], prefix sums).
__device__ __forceinline__ int64_t slots_before(int p) {
  const int a = p >> 6;
  return (int64_t)(a + 1) * (32 * a + (p & 63));
}

__global__ __launch_bounds__(256) void qsa_bitmap_kernel(const int32_t* __restrict__ blk_idx, int topk,
                                                         const int32_t* __restrict__ cu, int S, int T, int Hk,
                                                         int chunk, int ntiles, PlanBufs plan,
                                                         uint32_t* __restrict__ bits, int64_t* __restrict__ dsbase) {
  __shared__ uint32_t row[4][kWords];
  if (blockIdx.x == 0) {
    if (blockIdx.y == 0) {
      __shared__ int sb[256], si[256], hist[kOrderBins], scu[kCuCache];
      plan_blocks<256, kKT>(cu, S, chunk, plan.blkbase, plan.blk_seq, plan.seqitem, plan.totals, sb, si);
      plan_tile_order<256, 16>(cu, S, ntiles, plan.tile_order, sb, hist, scu);
      if (dsbase != nullptr) {
        // thread i sums a contiguous run of sequences; the 256 partial sums
        // are scanned, then each run is written out from its offset
        __shared__ int64_t part[256];
        const int per = (S + 255) / 256;
        const int s0 = threadIdx.x * per, s1 = min(s0 + per, S);
        int64_t sum = 0;
        for (int q = s0; q < s1; ++q) sum += slots_before(cu[q + 1] - cu[q]);
        part[threadIdx.x] = sum;
        __syncthreads();
        if (threadIdx.x == 0) {
          int64_t acc = 0;
          for (int i = 0; i < 256; ++i) {
            const int64_t x = part[i];
            part[i] = acc;
            acc += x;
          }
        }
        __syncthreads();
        int64_t acc = part[threadIdx.x];
        for (int q = s0; q < s1; ++q) {
          dsbase[q] = acc;
          acc += slots_before(cu[q + 1] - cu[q]);
        }
        if (threadIdx.x == 255) dsbase[S] = acc;
      }
    }
    return;
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = (blockIdx.x - 1) * 4 + wave;
  const int h = blockIdx.y;
  for (int i = lane; i < kWords; i += 64) row[wave][i] = 0u;
  __syncthreads();
  if (t < T) {
    const int s = find_seq(cu, S, t);
    const int b = (t - cu[s]) / kQsaBlock;
    const int32_t* ids = blk_idx + ((int64_t)t * Hk + h) * topk;
    for (int e = lane; e < topk; e += 64) {
      const int c = ids[e];
      if (c >= 0 && c <= b) atomicOr(&row[wave][c >> 5], 1u << (c & 31));
    }
  }
  __syncthreads();
  if (t < T) {
    const u32x4 x = {row[wave][4 * lane], row[wave][4 * lane + 1], row[wave][4 * lane + 2], row[wave][4 * lane + 3]};
    *reinterpret_cast<u32x4*>(bits + ((int64_t)t * Hk + h) * kWords + 4 * lane) = x;
  }
}

// ---------------------------------------------------------------------------
// Delta = rowsum(dO * O) and -LSE * log2(e) per (token, query head), ahead of
// the dK/dV pass: one wavefront per (token, KV head), 16 lanes per query head
// (16 dims a lane), four heads at a time.  Layout [T][Hk][16], heads past 12
// unused.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void qsa_delta_kernel(const u16* __restrict__ o, int64_t o_st, int64_t o_sh,
                                                        const u16* __restrict__ dO, int64_t do_st, int64_t do_sh,
                                                        const float* __restrict__ lse, int T, int Hk,
                                                        float* __restrict__ delta, float* __restrict__ nlse) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  const int h = blockIdx.y;
  if (t >= T) return;
  const int hg = lane >> 4, l16 = lane & 15;
#pragma unroll
  for (int pass = 0; pass < kG / 4; ++pass) {
    const int hh = 4 * pass + hg;
    const int hq = h * kG + hh;
    const u16* orow = o + (int64_t)t * o_st + (int64_t)hq * o_sh + 16 * l16;
    const u16* drow = dO + (int64_t)t * do_st + (int64_t)hq * do_sh + 16 * l16;
    const bf16x8 o0 = load_bf16x8(orow), o1 = load_bf16x8(orow + 8);
    const bf16x8 d0 = load_bf16x8(drow), d1 = load_bf16x8(drow + 8);
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) part = fmaf((float)d0[e], (float)o0[e], part);
#pragma unroll
    for (int e = 0; e < 8; ++e) part = fmaf((float)d1[e], (float)o1[e], part);
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) part += __shfl_xor(part, m);
    if (l16 == 0) {
      const int64_t slot = ((int64_t)t * Hk + h) * 16 + hh;
      delta[slot] = part;
      const float l2 = lse[(int64_t)t * (Hk * kG) + hq] * kLog2e;
      nlse[slot] = l2 > -INFINITY ? -l2 : -INFINITY;
    }
  }
}

// ---------------------------------------------------------------------------
// V^T of every (key tile, KV head) in the forward's operand order: run
// 2 dt + kc, lane li + 16 g holds V[key 32 kc + 8 g + e][dim 16 dt + li],
// e = 0..7 (zero past the sequence end).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void qsa_vt_kernel(const u16* __restrict__ v, int64_t v_st, int64_t v_sh,
                                                     const int32_t* __restrict__ cu,
                                                     const int32_t* __restrict__ ktbase,
                                                     const int32_t* __restrict__ kt_seq,
                                                     const int32_t* __restrict__ totals, int Hk,
                                                     u16* __restrict__ vt) {
  __shared__ __align__(16) u16 tile[kKT][kD + 8];
  const int gk = blockIdx.x, h = blockIdx.y;
  if (gk >= totals[0]) return;
  const int s = kt_seq[gk];
  const int c = gk - ktbase[s];
  const int seq0 = cu[s], L = cu[s + 1] - seq0;
  for (int i = threadIdx.x; i < kKT * kD / 8; i += 256) {
    const int key = i / (kD / 8), d8 = (i % (kD / 8)) * 8;
    const int kp = kKT * c + key;
    uint4 x = make_uint4(0u, 0u, 0u, 0u);
    if (kp < L) x = *reinterpret_cast<const uint4*>(v + (int64_t)(seq0 + kp) * v_st + (int64_t)h * v_sh + d8);
    *reinterpret_cast<uint4*>(&tile[key][d8]) = x;
  }
  __syncthreads();
  u16* dst = vt + ((int64_t)gk * Hk + h) * (32 * 64 * 8);
  for (int i = threadIdx.x; i < 32 * 64; i += 256) {
    const int run = i >> 6, ln = i & 63;
    const int d = 16 * (run >> 1) + (ln & 15);
    const int k0 = 32 * (run & 1) + 8 * (ln >> 4);
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = (uint32_t)tile[k0 + 2 * e][d] | ((uint32_t)tile[k0 + 2 * e + 1][d] << 16);
    *reinterpret_cast<u32x4*>(dst + (int64_t)i * 8) = u32x4{w[0], w[1], w[2], w[3]};
  }
}

// ---------------------------------------------------------------------------
// Copies of K per (key tile, KV head) in the stage order of the forward
// (plain) or the dQ pass (swizzled), so every staged 1 KB run is one
// contiguous copy: run kt*8 + ds, slot l holding k[key score_key(kt, r)][dims
// 32 ds + 8 (l / 16) .. +7] with r = l % 16 (plain) or swz_slot(l) % 16
// (swizzled); zero past the sequence end.  blockIdx.z: a quarter of the runs.
// ---------------------------------------------------------------------------
template <bool kSwizzled>
__global__ __launch_bounds__(256) void qsa_prep_kernel(const u16* __restrict__ k, int64_t k_st, int64_t k_sh,
                                                       const int32_t* __restrict__ cu,
                                                       const int32_t* __restrict__ ktbase,
                                                       const int32_t* __restrict__ kt_seq,
                                                       const int32_t* __restrict__ totals, int Hk,
                                                       u16* __restrict__ kop) {
  const int gk = blockIdx.x, h = blockIdx.y;
  if (gk >= totals[0]) return;
  const int part = blockIdx.z;
  const int s = kt_seq[gk];
  const int c = gk - ktbase[s];
  const int seq0 = cu[s], L = cu[s + 1] - seq0;
  u16* dst = kop + ((int64_t)gk * Hk + h) * (32 * 64 * 8);
  for (int i = 512 * part + threadIdx.x; i < 512 * part + 512; i += 256) {
    const int run = i >> 6, ln = i & 63;
    const int r = kSwizzled ? (swz_slot(ln) & 15) : (ln & 15);
    const int kp = kKT * c + score_key(run >> 3, r);
    u32x4 val = {0u, 0u, 0u, 0u};
    if (kp < L)
      val = *reinterpret_cast<const u32x4*>(k + (int64_t)(seq0 + kp) * k_st + (int64_t)h * k_sh + 32 * (run & 7) +
                                            8 * (ln >> 4));
    *reinterpret_cast<u32x4*>(dst + (int64_t)i * 8) = val;
  }
}

// ---------------------------------------------------------------------------
// Shared prologue of the token-major passes: the tile's kN tokens' bitmap rows
// into LDS and the ascending union of the global key tiles they touch, walked
// by kWaves wavefronts that do not each own a token: wavefront w reads the
// bitmap rows of tokens w, w + kWaves, ..., and each token's sequence position
// (-1 past the end of the pack) and its sequence's first global key tile are
// kept beside the rows.
// ---------------------------------------------------------------------------
template <int kN>
struct TileUnionRows {
  uint32_t bmap[kN][kWords];
  uint32_t ubits[kUnionWords];
  int ulist[kUnionMax];
  int tpos[kN];
  int tktb[kN];
  int64_t tslot[kN];  // the token's dS slot of key tile 0 (the backward's)
  int nunion;
};

template <int kN, int kWaves>
__device__ __forceinline__ void build_union_rows(TileUnionRows<kN>& tu, const uint32_t* __restrict__ bits,
                                                 const int32_t* __restrict__ cu, const int32_t* __restrict__ ktbase,
                                                 const int64_t* __restrict__ dsbase, int S, int T, int Hk, int h,
                                                 int t0, int wave, int lane) {
  const int gk_lo = ktbase[find_seq(cu, S, t0)];
  if (threadIdx.x < kUnionWords) tu.ubits[threadIdx.x] = 0u;
  __syncthreads();
  for (int j = wave; j < kN; j += kWaves) {
    const int t = t0 + j;
    const bool ok = t < T;
    int pos = -1, ktb = 0;
    int64_t slot = 0;
    if (ok) {
      const int s = find_seq(cu, S, t);
      pos = t - cu[s];
      ktb = ktbase[s];
      if (dsbase != nullptr) slot = dsbase[s] + slots_before(pos);
    }
    if (lane == 0) {
      tu.tpos[j] = pos;
      tu.tktb[j] = ktb;
      tu.tslot[j] = slot;
    }
    const uint32_t* brow = bits + ((int64_t)(ok ? t : 0) * Hk + h) * kWords;
    const int nw = ok ? (pos / kQsaBlock) / 32 + 1 : 0;
    for (int w = lane; w < kWords; w += 64) {
      const uint32_t x = w < nw ? brow[w] : 0u;
      tu.bmap[j][w] = x;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        if ((x >> (16 * hh)) & 0xFFFFu) {
          const int rel = ktb + 2 * w + hh - gk_lo;
          atomicOr(&tu.ubits[rel >> 5], 1u << (rel & 31));
        }
    }
  }
  __syncthreads();
  if (wave == 0) {
    uint32_t x = lane < kUnionWords ? tu.ubits[lane] : 0u;
    const int cnt = __popc(x);
    int incl = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    int pos = incl - cnt;
    while (x) {
      const int bit = __ffs(x) - 1;
      tu.ulist[pos++] = gk_lo + 32 * lane + bit;
      x &= x - 1u;
    }
    if (lane == 63) tu.nunion = incl;
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Forward.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64 * kRowWaves) void qsa_fwd_kernel(
    const u16* __restrict__ q, int64_t q_st, int64_t q_sh, const u16* __restrict__ kop,
    const u16* __restrict__ vt, const uint32_t* __restrict__ bits, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ ktbase, const int32_t* __restrict__ tile_order, int S, int T, int Hk,
    float scale_log2, u16* __restrict__ o, int64_t o_st, int64_t o_sh, float* __restrict__ lse) {
  // K runs kt * 8 + ds: keys score_key(kt, .) of the tile, dims 32 ds ..;
  // V^T runs 2 dt + kc as laid out by qsa_vt_kernel
  __shared__ u32x4 kbuf[2][32][64];
  __shared__ u32x4 vbuf[2][32][64];
  __shared__ TileUnionRows<kQTok> tu;

  // workgroup b: KV head b % Hk, 16-token tile in launch slot b / Hk
  const int h = blockIdx.x % Hk;
  const int t0 = tile_order[blockIdx.x / Hk] * kAttnTile;
  if (t0 >= T) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int li = lane & 15;
  // this lane's MFMA column: row 16 wave + li of the tile, head hd of token tk
  const int row = 16 * wave + li;
  const int tk = row / kG;
  const int hd = row - kG * tk;
  const int t = t0 + tk;
  const bool tok_ok = t < T;

  // q of this row as B operands, loaded before the union build so the loads
  // overlap it; O^T accumulators
  bf16x8 qb[8];
  {
    const u16* qrow = q + (int64_t)(tok_ok ? t : 0) * q_st + (int64_t)(h * kG + hd) * q_sh + 8 * g;
#pragma unroll
    for (int ds = 0; ds < 8; ++ds) qb[ds] = tok_ok ? load_bf16x8(qrow + 32 * ds) : zero_bf16x8();
  }
  build_union_rows<kQTok, kRowWaves>(tu, bits, cu, ktbase, nullptr, S, T, Hk, h, t0, wave, lane);
  const int nu = tu.nunion;
  const int pos_t = tu.tpos[tk];
  const int ktb_t = tu.tktb[tk];
  const int own_c = tok_ok ? pos_t / kKT : -1;
  f32x4 oacc[16];
#pragma unroll
  for (int dt = 0; dt < 16; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // staging of union step u: the tile's 32 K runs and 32 V^T runs, run
  // wave + 12 ii copied by wavefront `wave`
  auto stage = [&](int u, int buf) {
    const int gk = __builtin_amdgcn_readfirstlane(tu.ulist[u]);
    const int ln = fresh_lane();
    const u16* kbase = kop + ((int64_t)gk * Hk + h) * 32 * 512;
    const u16* vbase = vt + ((int64_t)gk * Hk + h) * 32 * 512;
#pragma unroll
    for (int ii = 0; ii < (64 + kRowWaves - 1) / kRowWaves; ++ii) {
      const int r = wave + kRowWaves * ii;
      if (r < 32)
        dma16s(kbase + 512 * r, 16 * ln, lds_offset(&kbuf[buf][r][0]));
      else if (r < 64)
        dma16s(vbase + 512 * (r - 32), 16 * ln, lds_offset(&vbuf[buf][r - 32][0]));
    }
  };
  if (nu > 0) stage(0, 0);
  wait_copies();
  wait_all_loads();
  __syncthreads();

  for (int u = 0; u < nu; ++u) {
    const int buf = u & 1;
    if (u + 1 < nu) stage(u + 1, buf ^ 1);
    // key tile of this row's sequence (when in range) and the blocks the row's
    // token lists in it; the wavefront works the tile when any of its rows does
    const int c = tu.ulist[u] - ktb_t;
    const uint32_t m16 = (c >= 0 && c <= own_c) ? tile_mask(tu.bmap[tk], c) : 0u;
    if (__ballot(m16 != 0u)) {
      const bool own = (c == own_c);
      const int plim = pos_t - kKT * c;  // causal: tile keys at index <= plim
      // S^T for the tile's four 16-key tiles: four chains interleaved, K
      // operand reads eight ahead of the MFMAs
      f32x4 st[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) st[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
      {
        // the MFMA blocks run at raised wave priority, so on a SIMD whose other
        // wavefronts are in their softmax the matrix unit is fed first
        __builtin_amdgcn_s_setprio(1);
        bf16x8 ka[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) ka[i] = __builtin_bit_cast(bf16x8, kbuf[buf][(i & 3) * 8 + (i >> 2)][lane]);
#pragma unroll
        for (int i = 0; i < 32; ++i) st[i & 3] = mfma16x16x32(ka[i], qb[i >> 2], st[i & 3]);
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
        for (int i = 0; i < 24; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
        __builtin_amdgcn_s_setprio(0);
      }
      // mask: accumulator row r of tile kt in lane group g is tile key
      // score_key(kt, 4g + r) = 32 (kt/2) + 8g + 4 (kt%2) + r, all four in
      // block 8 (kt/2) + 2g + kt%2
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const bool listed = (m16 >> (8 * (kt >> 1) + 2 * g + (kt & 1))) & 1u;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int kl = 32 * (kt >> 1) + 8 * g + 4 * (kt & 1) + r;
          const bool keep = listed && (!own || kl <= plim);
          st[kt][r] = keep ? st[kt][r] : -INFINITY;
          mx = fmaxf(mx, st[kt][r]);
        }
      }
      // online softmax in base 2 (scale folded into the exponent's FMA); the
      // running max moves only when it grows by more than kRescaleSlack.  A
      // row whose token lists nothing in this tile adds P = 0 (its max stays
      // -inf until its token lists a key, hence the 0 in the exponent then)
      mx = max_over_groups(mx);
      const float m_cand = mx * scale_log2;
      const bool grow = m_cand > m_run + kRescaleSlack;
      const float m_use = grow ? m_cand : m_run;
      const float alpha = grow ? fast_exp2(m_run - m_cand) : 1.f;
      const float m_sub = m_use > -INFINITY ? m_use : 0.f;
      float rs = 0.f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = fast_exp2(fmaf(st[kt][r], scale_log2, -m_sub));
          st[kt][r] = p;
          rs += p;
        }
      l_run = l_run * alpha + rs;
      m_run = m_use;
      if (__ballot(grow)) {
#pragma unroll
        for (int dt = 0; dt < 16; ++dt) oacc[dt] *= alpha;
      }
      const bf16x8 pf0 = pack_bf16x8(st[0], st[1]);
      const bf16x8 pf1 = pack_bf16x8(st[2], st[3]);
      // O^T += V^T P^T over the tile's two 32-key halves
      {
        __builtin_amdgcn_s_setprio(1);
        bf16x8 va[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) va[i] = __builtin_bit_cast(bf16x8, vbuf[buf][(i & 15) * 2 + (i >> 4)][lane]);
#pragma unroll
        for (int i = 0; i < 32; ++i) oacc[i & 15] = mfma16x16x32(va[i], i < 16 ? pf0 : pf1, oacc[i & 15]);
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
        for (int i = 0; i < 24; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
        __builtin_amdgcn_s_setprio(0);
      }
    }
    wait_copies();
    lds_barrier();
  }

  // l_run holds this lane's share of the row sum (its keys 8g.. of every 32)
  l_run = sum_over_groups(l_run);
  if (tok_ok) {
    const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
    u16* orow = o + (int64_t)t * o_st + (int64_t)(h * kG + hd) * o_sh;
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) *reinterpret_cast<uint2*>(orow + 16 * dt + 4 * g) = pack_bf16x4(oacc[dt] * inv);
    if (g == 0)
      lse[(int64_t)t * (Hk * kG) + h * kG + hd] = l_run > 0.f ? (m_run + __log2f(l_run)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// dQ from the dS the dK/dV pass stored.  The forward's tiling: 12 wavefronts
// per (16-token tile, KV head), lane column = row 16 wave + li of the tile
// (head hd of token tk), so no padding heads are computed, within the 168
// registers of three wavefronts per SIMD (dQ^T accumulators 64).  The union
// of the tile's key tiles is walked with K staged (swizzled, from the prep
// kernel's copy) and K^T read transposed; per 32-key half a lane's dS^T
// operand is keys 32 kc + 8g .. +7 of its row's dS line for the tile (slot
// tslot + c of the row's token), zero where the token lists nothing in the
// tile.  The lines are copied into LDS two steps ahead through a three-deep
// ring, K one step ahead; every wait in the walk is the step's own explicit
// one, which leaves the wavefront's last two copies (step u + 2's dS) in
// flight (copies complete in issue order).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64 * kRowWaves) void qsa_dq_ds_kernel(
    const u16* __restrict__ kop, const u16* ds, const int64_t* __restrict__ dsbase,
    const uint32_t* __restrict__ bits, const int32_t* __restrict__ cu, const int32_t* __restrict__ ktbase,
    const int32_t* __restrict__ tile_order, int S, int T, int Hk, float scale, u16* __restrict__ dq, int64_t dq_st,
    int64_t dq_sh) {
  // K runs kt * 8 + ds (keys score_key(kt, .), dims 32 ds ..), stored
  // swizzled (swz_slot) for the transposed K^T reads
  __shared__ u32x4 kbuf[2][32][64];
  // per wavefront and 32-key half, each lane's 8 keys of dS, three steps deep
  // (copied two steps ahead; each wavefront reads only its own slots)
  __shared__ u32x4 dsl[3][kRowWaves][2][64];
  __shared__ TileUnionRows<kQTok> tu;

  const int h = blockIdx.x % Hk;
  const int t0 = tile_order[blockIdx.x / Hk] * kAttnTile;
  if (t0 >= T) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int li = lane & 15;
  const int row = 16 * wave + li;
  const int tk = row / kG;
  const int hd = row - kG * tk;
  const int t = t0 + tk;
  const bool tok_ok = t < T;

  build_union_rows<kQTok, kRowWaves>(tu, bits, cu, ktbase, dsbase, S, T, Hk, h, t0, wave, lane);
  const int nu = tu.nunion;
  const int pos_t = tu.tpos[tk];
  const int ktb_t = tu.tktb[tk];
  const int own_c = tok_ok ? pos_t / kKT : -1;
  // this row's dS line of its token's key tile c: slot tslot + c
  const int64_t slot0 = tu.tslot[tk];
  f32x4 dqacc[16];
#pragma unroll
  for (int dt = 0; dt < 16; ++dt) dqacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // the row's listed blocks in step u's key tile
  auto tile_bits = [&](int u) -> uint32_t {
    const int c = tu.ulist[u] - ktb_t;
    return (c >= 0 && c <= own_c) ? tile_mask(tu.bmap[tk], c) : 0u;
  };
  // staging of union step u's K: the tile's 32 K runs, run wave + 12 ii
  // copied by wavefront `wave`
  auto stage_k = [&](int u, int buf) {
    const int gk = __builtin_amdgcn_readfirstlane(tu.ulist[u]);
    const int ln = fresh_lane();
    const u16* kbase = kop + ((int64_t)gk * Hk + h) * 32 * 512;
#pragma unroll
    for (int ii = 0; ii < (32 + kRowWaves - 1) / kRowWaves; ++ii) {
      const int r = wave + kRowWaves * ii;
      if (r < 32) dma16s(kbase + 512 * r, 16 * ln, lds_offset(&kbuf[buf][r][0]));
    }
  };
  // step u's dS: each lane's 16 bytes of its row's line per half, two copies
  // per wavefront whatever the masks (the row's token's first slot stands in
  // where its token lists nothing)
  auto stage_ds = [&](int u, int dbuf, uint32_t m16) {
    const int c = m16 != 0u ? tu.ulist[u] - ktb_t : 0;
    const u16* line = ds + (((slot0 + c) * Hk + h) * kG + hd) * kKT + 8 * g;
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) dma16(line + 32 * kc, lds_offset(&dsl[dbuf][wave][kc][0]));
  };
  uint32_t m_cur = 0u, m_n1 = 0u;
  if (nu > 0) {
    m_cur = tile_bits(0);
    stage_k(0, 0);
    stage_ds(0, 0, m_cur);
  }
  if (nu > 1) {
    m_n1 = tile_bits(1);
    stage_ds(1, 1, m_n1);
  }
  wait_copies();
  wait_all_loads();
  __syncthreads();

  int dbuf = 0;
  for (int u = 0; u < nu; ++u) {
    const int buf = u & 1;
    const bool ahead2 = u + 2 < nu;
    const uint32_t m_n2 = ahead2 ? tile_bits(u + 2) : 0u;
    if (u + 1 < nu) stage_k(u + 1, buf ^ 1);
    if (ahead2) stage_ds(u + 2, dbuf == 0 ? 2 : dbuf - 1, m_n2);
    if (__ballot(m_cur != 0u)) {
      const int c = tu.ulist[u] - ktb_t;
      const bool own = (c == own_c);
      const int plim = pos_t - kKT * c;
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        // a half no row has a causal key in holds only zero records
        if (!__ballot(m_cur != 0u && !(own && 32 * kc > plim))) continue;
        // dS^T operand: keys 32 kc + 8g .. +7 of the row (zero where its
        // token lists nothing in the tile: that line was never written)
        const u32x4 rec = dsl[dbuf][wave][kc][lane];
        const bool on = m_cur != 0u;
        const bf16x8 dsb =
            __builtin_bit_cast(bf16x8, u32x4{on ? rec[0] : 0u, on ? rec[1] : 0u, on ? rec[2] : 0u, on ? rec[3] : 0u});
        // K^T operands read transposed from the K stage: keys 8g .. 8g+7 of
        // the half (tiles 2kc, 2kc+1, rows 4g .. 4g+3) at dim 16 dt + li
        const uint32_t kq = lds_offset(&kbuf[buf][16 * kc][0]) + tr_lane_offset(fresh_lane());
        bf16x8 ta[16];
#pragma unroll
        for (int dt = 0; dt < 16; ++dt) {
          const uint32_t off = kq + (dt >> 1) * 1024 + (dt & 1) * 512;
          const uint2 lo = read_tr16(off), hi = read_tr16(off + 8192);
          ta[dt] = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
        }
#pragma unroll
        for (int dt = 0; dt < 16; ++dt) dqacc[dt] = mfma16x16x32(ta[dt], dsb, dqacc[dt]);
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * kDqTrAhead, 0);
#pragma unroll
        for (int i = 0; i < 16 - kDqTrAhead; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kDqTrAhead, 0);
      }
    }
    // step u + 1's K and dS have landed; step u + 2's dS (the wavefront's
    // last two copies) may still be in flight: copies complete in issue order
    if (ahead2)
      asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
    else
      wait_copies();
    lds_barrier();
    m_cur = m_n1;
    m_n1 = m_n2;
    dbuf = dbuf == 2 ? 0 : dbuf + 1;
  }

  if (tok_ok) {
    u16* out = dq + (int64_t)t * dq_st + (int64_t)(h * kG + hd) * dq_sh;
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) *reinterpret_cast<uint2*>(out + 16 * dt + 4 * g) = pack_bf16x4(dqacc[dt] * scale);
  }
}

// ---------------------------------------------------------------------------
// dK/dV.
// ---------------------------------------------------------------------------
constexpr int kPair = 2;  // 16-row tiles per staging round (one MFMA step of 32 rows)

// The selecting tokens' query heads are taken as one list of rows, row r being
// head r % 12 of selecting token r / 12, so that a 32-row MFMA step carries
// no padding heads (a step of two tokens would carry 8 of 32).  Stage layout
// of one 16-row tile (u32x4 units): [0, 512) q and [512, 1024) dO as
// [ds][slot], operand lane li + 16g of run ds (row li of the tile, dims
// 32 ds + 8g ..) at slot swz_slot(li + 16g); rows past the list's end repeat
// its last row (finite operands, masked).  Stats: the tile's 16 -LSE log2 e,
// then its 16 Delta.  Every lane reads its own row, so the copies take
// per-lane addresses.
__device__ __forceinline__ void stage_rows(int row0, int nrows, const int* sel, int tok0, int h, int Hk, int lane,
                                           uint32_t slot_lds, uint32_t stats_lds,
                                           const u16* __restrict__ q, int64_t q_st, int64_t q_sh,
                                           const u16* __restrict__ dO, int64_t do_st, int64_t do_sh,
                                           const float* __restrict__ nlse, const float* __restrict__ delta) {
  const int r = min(row0 + (swz_slot(lane) & 15), nrows - 1);
  const int n = r / kG;
  const int t = tok0 + (sel[n] & 0xFFFF);
  const int head = h * kG + (r - kG * n);
  const u16* qr = q + (int64_t)t * q_st + (int64_t)head * q_sh + 8 * (lane >> 4);
  const u16* dr = dO + (int64_t)t * do_st + (int64_t)head * do_sh + 8 * (lane >> 4);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    dma16(qr + 32 * i, slot_lds + i * 1024);
    dma16(dr + 32 * i, slot_lds + 8192 + i * 1024);
  }
  // lanes 0-15: -LSE of rows row0 + lane; lanes 16-31: Delta of rows row0 + lane - 16
  if (lane < 32) {
    const int rs = min(row0 + (lane & 15), nrows - 1);
    const int ns = rs / kG;
    const int ts = tok0 + (sel[ns] & 0xFFFF);
    dma4((lane < 16 ? nlse : delta) + ((int64_t)ts * Hk + h) * 16 + (rs - kG * ns), stats_lds);
  }
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void qsa_dkdv_kernel(
    const u16* __restrict__ q, int64_t q_st, int64_t q_sh, const u16* __restrict__ k, int64_t k_st, int64_t k_sh,
    const u16* __restrict__ v, int64_t v_st, int64_t v_sh, const u16* __restrict__ dO, int64_t do_st,
    int64_t do_sh, const float* __restrict__ nlse, const float* __restrict__ delta,
    const uint32_t* __restrict__ bits, const int64_t* __restrict__ dsbase, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ seqitem, const int32_t* __restrict__ totals, int S, int Hk, int chunk,
    int items_cap, float scale_log2, float scale, int32_t* __restrict__ item_count,
    float* __restrict__ part_dk, float* __restrict__ part_dv, u16* __restrict__ ds_out,
    u16* __restrict__ dk_out, int64_t dk_st, int64_t dk_sh, u16* __restrict__ dv_out, int64_t dv_st,
    int64_t dv_sh) {
  __shared__ u32x4 stage[2][kPair][1024];
  __shared__ __align__(16) float stats[2][kPair][32];
  __shared__ int sel[kQsaChunkMax];  // (position - p_begin) | (block mask << 16)
  // the dS of a round, [wavefront (16 keys)][row][key], stored during the next
  // round (double buffered: the next round's writes go to the other half)
  __shared__ __align__(16) u16 dsx[2][4][32][16];
  __shared__ int wcount[4];

  const int h = blockIdx.y;
  const int item = blockIdx.x;
  if (item >= totals[1]) return;
  // decode (sequence, query chunk j, key tile c)
  const int s = upper_index(seqitem, S, item);
  const int seq0 = cu[s];
  const int L = cu[s + 1] - seq0;
  const int nch = (L + chunk - 1) / chunk;
  int r = item - seqitem[s];
  int j = 0;
  for (;;) {
    const int cnt = (min((j + 1) * chunk, L) - 1) / kKT + 1;
    if (r < cnt) break;
    r -= cnt;
    ++j;
  }
  const int c = r;
  const int jmin = (kKT * c) / chunk;
  const bool single = (j == nch - 1) && (j == jmin);
  const int p_begin = max(j * chunk, kKT * c);
  const int p_end = min((j + 1) * chunk, L);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int li = lane & 15;

  // 1. the chunk's queries that listed a block of key tile c, in token order
  int nsel = 0;
  for (int p0 = p_begin; p0 < p_end; p0 += 256) {
    const int p = p0 + threadIdx.x;
    uint32_t m = 0u;
    if (p < p_end) m = tile_mask(bits + ((int64_t)(seq0 + p) * Hk + h) * kWords, c);
    const uint64_t bal = __ballot(m != 0u);
    const int before = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wcount[wave] = __popcll(bal);
    __syncthreads();
    int off = nsel;
    int tot = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      off += w < wave ? wcount[w] : 0;
      tot += wcount[w];
    }
    if (m != 0u) sel[off + before] = (p - p_begin) | (int)(m << 16);
    nsel += tot;
    __syncthreads();
  }
  if (threadIdx.x == 0) item_count[(int64_t)h * items_cap + item] = nsel;

  // 2. K and V of this wavefront's 16 keys as B operands (zero past the end)
  const int kbase = kKT * c + 16 * wave;
  bf16x8 kf[8], vf[8];
  {
    const int kp = kbase + li;
    const bool ok = kp < L;
    const u16* krow = k + (int64_t)(seq0 + min(kp, L - 1)) * k_st + (int64_t)h * k_sh + 8 * g;
    const u16* vrow = v + (int64_t)(seq0 + min(kp, L - 1)) * v_st + (int64_t)h * v_sh + 8 * g;
#pragma unroll
    for (int ds = 0; ds < 8; ++ds) {
      kf[ds] = ok ? load_bf16x8(krow + 32 * ds) : zero_bf16x8();
      vf[ds] = ok ? load_bf16x8(vrow + 32 * ds) : zero_bf16x8();
    }
  }
  f32x4 dk[16], dv[16];
#pragma unroll
  for (int dt = 0; dt < 16; ++dt) {
    dk[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    dv[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // 3. stream the selecting tokens' rows through LDS, 32 per MFMA step;
  // wavefronts 0 and 1 copy the two 16-row tiles of a round
  if (nsel > 0) {
    const int nrows = kG * nsel;
    const int nround = (nrows + 32 - 1) / 32;
    auto stage_round = [&](int bi, int buf) {
      if (wave < kPair)
        stage_rows(32 * bi + 16 * wave, nrows, sel, seq0 + p_begin, h, Hk, fresh_lane(),
                   lds_offset(&stage[buf][wave][0]), lds_offset(&stats[buf][wave][0]), q, q_st, q_sh, dO, do_st,
                   do_sh, nlse, delta);
    };
    // round b's dS from the stash into the dQ pass's slots: per (token, key
    // tile c, KV head, query head) the 64 keys' bf16 dS (zero where unlisted
    // or past the query), one 128-byte line written whole by eight threads,
    // non-temporal (the reduce that runs next keeps more of its slices cached:
    // qsa16k dK/dV 1441 -> 1416 us, reduce 116 -> 97 us)
    const int64_t seqslot = dsbase[s];
    auto flush = [&](int b) {
      const int R = threadIdx.x >> 3, j = threadIdx.x & 7;
      const int rrow = 32 * b + R;
      if (rrow < nrows) {
        const int n = rrow / kG;
        const int pos = p_begin + (sel[n] & 0xFFFF);
        const int64_t slot = seqslot + slots_before(pos) + c;
        __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(&dsx[b & 1][j >> 1][R][8 * (j & 1)]),
                                    reinterpret_cast<u32x4*>(ds_out +
                                                             ((slot * Hk + h) * kG + (rrow - kG * n)) * kKT + 8 * j));
      }
      asm volatile("" ::: "memory");
    };
    stage_round(0, 0);
    wait_copies();
    wait_all_loads();
    __syncthreads();
#pragma unroll 1
    for (int bi = 0; bi < nround; ++bi) {
      const int cur = bi & 1;
      if (bi + 1 < nround) stage_round(bi + 1, cur ^ 1);
      if (bi > 0) flush(bi - 1);
      // per tile tk, this lane's accumulator rows 4g .. 4g+3 (rows
      // 32 bi + 16 tk + 4g ..) belong to one token (12 is a multiple of 4);
      // rows past the list's end are masked out entirely
      int pos[2];
      uint32_t msk[2];
#pragma unroll
      for (int tk = 0; tk < 2; ++tk) {
        const int row = 32 * bi + 16 * tk + 4 * g;
        const int e = sel[min(row / kG, nsel - 1)];
        pos[tk] = p_begin + (e & 0xFFFF);
        msk[tk] = row < nrows ? ((uint32_t)e >> 16) : 0u;
      }
      // S = q K^T and dP = dO V^T per 16-row tile, turned into bf16 P and dS:
      // lane (key li, group g) keeps rows 4g .. 4g+3 of each tile, two per
      // dword, as the A operand of dV and dK (dwords 0-1 tile 0, 2-3 tile 1)
      u32x4 pw, sw;
      const int ln = fresh_lane();
      const int sl = swz_slot(ln);
      // the lane's key: kbase + li, in block (16 wave + li) / 4 of the tile
      const int kp = kbase + li;
#pragma unroll
      for (int tk = 0; tk < 2; ++tk) {
        const u32x4* b = stage[cur][tk];
        f32x4 sacc = {0.f, 0.f, 0.f, 0.f}, pacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ds = 0; ds < 8; ++ds) {
          const bf16x8 qa = __builtin_bit_cast(bf16x8, b[ds * 64 + sl]);
          const bf16x8 da = __builtin_bit_cast(bf16x8, b[512 + ds * 64 + sl]);
          sacc = mfma16x16x32(qa, kf[ds], sacc);
          pacc = mfma16x16x32(da, vf[ds], pacc);
        }
        const f32x4 nl = reinterpret_cast<const f32x4*>(stats[cur][tk])[ln >> 4];
        const f32x4 d4 = reinterpret_cast<const f32x4*>(stats[cur][tk] + 16)[ln >> 4];
        const bool on = ((msk[tk] >> (4 * wave + (li >> 2))) & 1u) && kp <= pos[tk];
        f32x4 e, d;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          e[rr] = on ? fast_exp2(fmaf(sacc[rr], scale_log2, nl[rr])) : 0.f;
          d[rr] = e[rr] * (pacc[rr] - d4[rr]);
        }
        pw[2 * tk] = pack_bf16x2(e[0], e[1]);
        pw[2 * tk + 1] = pack_bf16x2(e[2], e[3]);
        sw[2 * tk] = pack_bf16x2(d[0], d[1]);
        sw[2 * tk + 1] = pack_bf16x2(d[2], d[3]);
      }
      // the round's dS into the LDS stash; after the round's barrier it holds
      // all 64 keys of the round's rows
#pragma unroll
      for (int tk = 0; tk < 2; ++tk) {
        u16* col = &dsx[bi & 1][wave][16 * tk + 4 * g][li];
        col[0] = (u16)(sw[2 * tk] & 0xFFFFu);
        col[16] = (u16)(sw[2 * tk] >> 16);
        col[32] = (u16)(sw[2 * tk + 1] & 0xFFFFu);
        col[48] = (u16)(sw[2 * tk + 1] >> 16);
      }
      asm volatile("" ::: "memory");
      const bf16x8 pA = __builtin_bit_cast(bf16x8, pw);
      const bf16x8 sA = __builtin_bit_cast(bf16x8, sw);
      const uint32_t tro = tr_lane_offset(ln);
      const uint32_t q0 = lds_offset(stage[cur][0]) + tro, q1 = lds_offset(stage[cur][1]) + tro;
#pragma unroll
      for (int dt = 0; dt < 16; ++dt) {
        const uint32_t off = (dt >> 1) * 1024 + (dt & 1) * 512;
        const uint2 a0 = read_tr16(q0 + 8192 + off);
        const uint2 a1 = read_tr16(q1 + 8192 + off);
        const uint2 c0 = read_tr16(q0 + off);
        const uint2 c1 = read_tr16(q1 + off);
        const bf16x8 bdo = __builtin_bit_cast(bf16x8, u32x4{a0.x, a0.y, a1.x, a1.y});
        const bf16x8 bq = __builtin_bit_cast(bf16x8, u32x4{c0.x, c0.y, c1.x, c1.y});
        dv[dt] = mfma16x16x32(pA, bdo, dv[dt]);
        dk[dt] = mfma16x16x32(sA, bq, dk[dt]);
      }
      wait_copies();
      lds_barrier();
    }
    flush(nround - 1);
  }

  // 4. results: lane holds key kbase + 4g + r, dim 16 dt + li
  if (single) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int kp = kbase + 4 * g + rr;
      if (kp >= L) continue;
      u16* dkr = dk_out + (int64_t)(seq0 + kp) * dk_st + (int64_t)h * dk_sh + li;
      u16* dvr = dv_out + (int64_t)(seq0 + kp) * dv_st + (int64_t)h * dv_sh + li;
#pragma unroll
      for (int dt = 0; dt < 16; ++dt) {
        dkr[16 * dt] = f2bf(dk[dt][rr] * scale);
        dvr[16 * dt] = f2bf(dv[dt][rr]);
      }
    }
  } else if (nsel > 0) {
    const int64_t slice = ((int64_t)h * items_cap + item) * (kKT * kD);
#pragma unroll
    for (int dt = 0; dt < 16; ++dt)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int key = 16 * wave + 4 * g + rr;
        const int64_t off = slice + (int64_t)key * kD + 16 * dt + li;
        part_dk[off] = dk[dt][rr];
        part_dv[off] = dv[dt][rr];
      }
  }
}

// Ordered sum of the chunk slices of one (key tile, 16 keys, KV head).
constexpr int kRedBatch = 4;  // chunk slices in flight per reduce step

__global__ __launch_bounds__(256) void qsa_reduce_kernel(
    const float* __restrict__ part_dk, const float* __restrict__ part_dv, const int32_t* __restrict__ item_count,
    const int32_t* __restrict__ seqitem, const int32_t* __restrict__ kt_seq, const int32_t* __restrict__ ktbase,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ totals, int chunk, int items_cap, float scale,
    u16* __restrict__ dk, int64_t dk_st, int64_t dk_sh, u16* __restrict__ dv, int64_t dv_st, int64_t dv_sh) {
  const int gk = blockIdx.x;
  const int slice = blockIdx.y;
  const int h = blockIdx.z;
  if (gk >= totals[0]) return;
  const int s = kt_seq[gk];
  const int c = gk - ktbase[s];
  const int seq0 = cu[s];
  const int L = cu[s + 1] - seq0;
  const int nch = (L + chunk - 1) / chunk;
  const int jmin = (kKT * c) / chunk;
  if (jmin == nch - 1) return;  // a key tile with one work item was written by the dK/dV kernel
  const int item0 = seqitem[s];
  const int m = chunk / kKT;  // key tiles per full chunk: chunk j's items start at item0 + m j (j + 1) / 2
  // this thread's four 4-element groups of the 16 keys x 256 dims
  constexpr int kGroups = 16 * kD / 1024;
  int eg[kGroups], kp[kGroups];
#pragma unroll
  for (int u = 0; u < kGroups; ++u) {
    eg[u] = slice * 16 * kD + threadIdx.x * 4 + u * 1024;
    kp[u] = kKT * c + eg[u] / kD;
  }
  f32x4 adk[kGroups], adv[kGroups];
#pragma unroll
  for (int u = 0; u < kGroups; ++u) adk[u] = adv[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  // kRedBatch chunks at a time: their slices are loaded before any is added,
  // then added in chunk order (chunks whose item no query listed wrote nothing)
  for (int j0 = jmin; j0 < nch; j0 += kRedBatch) {
    int cnt[kRedBatch];
    int64_t off[kRedBatch];
#pragma unroll
    for (int w = 0; w < kRedBatch; ++w) {
      const int j = min(j0 + w, nch - 1);
      const int it = item0 + m * (j * (j + 1) / 2) + c;
      const bool ok = j0 + w < nch && it < items_cap;
      const int itc = ok ? it : 0;
      cnt[w] = ok ? item_count[(int64_t)h * items_cap + itc] : 0;
      off[w] = ((int64_t)h * items_cap + itc) * (kKT * kD);
    }
    f32x4 pk[kRedBatch][kGroups], pv[kRedBatch][kGroups];
#pragma unroll
    for (int w = 0; w < kRedBatch; ++w)
#pragma unroll
      for (int u = 0; u < kGroups; ++u) {
        pk[w][u] = *reinterpret_cast<const f32x4*>(part_dk + off[w] + eg[u]);
        pv[w][u] = *reinterpret_cast<const f32x4*>(part_dv + off[w] + eg[u]);
      }
#pragma unroll
    for (int w = 0; w < kRedBatch; ++w)
      if (cnt[w] != 0) {
#pragma unroll
        for (int u = 0; u < kGroups; ++u) {
          adk[u] += pk[w][u];
          adv[u] += pv[w][u];
        }
      }
  }
#pragma unroll
  for (int u = 0; u < kGroups; ++u) {
    if (kp[u] >= L) continue;
    const int d = eg[u] % kD;
    *reinterpret_cast<uint2*>(dk + (int64_t)(seq0 + kp[u]) * dk_st + (int64_t)h * dk_sh + d) =
        pack_bf16x4(adk[u] * scale);
    *reinterpret_cast<uint2*>(dv + (int64_t)(seq0 + kp[u]) * dv_st + (int64_t)h * dv_sh + d) = pack_bf16x4(adv[u]);
  }
}

void launch_bitmaps(const Sizes& z, const QsaArgs& a, const PlanBufs& p, int64_t* dsbase, hipStream_t st) {
  KernelTimer timer("qsa_bitmap", st);
  qsa_bitmap_kernel<<<dim3((unsigned)((z.T + 3) / 4 + 1), (unsigned)z.Hk), 256, 0, st>>>(
      a.blk_idx, a.topk, a.cu, (int)z.S, (int)z.T, (int)z.Hk, (int)z.chunk, (int)z.ntiles, p, a.bits, dsbase);
}

}  // namespace

void launch_qsa_fwd(const Sizes& z, const QsaArgs& a, const PlanBufs& p, hipStream_t st) {
  launch_bitmaps(z, a, p, nullptr, st);
  {
    KernelTimer timer("qsa_vt", st);
    qsa_vt_kernel<<<dim3((unsigned)z.nblk_cap, (unsigned)z.Hk), 256, 0, st>>>(
        a.v, a.v_st, a.v_sh, a.cu, p.blkbase, p.blk_seq, p.totals, (int)z.Hk, a.vt);
    qsa_prep_kernel<false><<<dim3((unsigned)z.nblk_cap, (unsigned)z.Hk, 4), 256, 0, st>>>(
        a.k, a.k_st, a.k_sh, a.cu, p.blkbase, p.blk_seq, p.totals, (int)z.Hk, a.kop);
  }
  KernelTimer timer("qsa_fwd", st);
  qsa_fwd_kernel<<<(unsigned)(z.ntiles * z.Hk), 64 * kRowWaves, 0, st>>>(
      a.q, a.q_st, a.q_sh, a.kop, a.vt, a.bits, a.cu, p.blkbase, p.tile_order, (int)z.S, (int)z.T, (int)z.Hk,
      a.scale * kLog2e, a.out_o, a.oo_st, a.oo_sh, a.out_lse);
}

void launch_qsa_bwd(const Sizes& z, const QsaArgs& a, const PlanBufs& p, hipStream_t st) {
  launch_bitmaps(z, a, p, a.dsbase, st);
  {
    // K in the dQ pass's swizzled stage order
    KernelTimer timer("qsa_prep", st);
    qsa_prep_kernel<true><<<dim3((unsigned)z.nblk_cap, (unsigned)z.Hk, 4), 256, 0, st>>>(
        a.k, a.k_st, a.k_sh, a.cu, p.blkbase, p.blk_seq, p.totals, (int)z.Hk, a.kop);
  }
  {
    KernelTimer timer("qsa_delta", st);
    qsa_delta_kernel<<<dim3((unsigned)((z.T + 3) / 4), (unsigned)z.Hk), 256, 0, st>>>(
        a.o, a.o_st, a.o_sh, a.dO, a.do_st, a.do_sh, a.lse, (int)z.T, (int)z.Hk, a.delta, a.nlse);
  }
  {
    KernelTimer timer("qsa_dkdv", st);
    qsa_dkdv_kernel<<<dim3((unsigned)z.items_cap, (unsigned)z.Hk), 256, 0, st>>>(
        a.q, a.q_st, a.q_sh, a.k, a.k_st, a.k_sh, a.v, a.v_st, a.v_sh, a.dO, a.do_st, a.do_sh, a.nlse, a.delta,
        a.bits, a.dsbase, a.cu, p.seqitem, p.totals, (int)z.S, (int)z.Hk, (int)z.chunk, (int)z.items_cap,
        a.scale * kLog2e, a.scale, a.item_count, a.part_dk, a.part_dv, a.ds, a.dk, a.dk_st, a.dk_sh, a.dv,
        a.dv_st, a.dv_sh);
  }
  {
    KernelTimer timer("qsa_reduce", st);
    qsa_reduce_kernel<<<dim3((unsigned)z.nblk_cap, kKT / 16, (unsigned)z.Hk), 256, 0, st>>>(
        a.part_dk, a.part_dv, a.item_count, p.seqitem, p.blk_seq, p.blkbase, a.cu, p.totals, (int)z.chunk,
        (int)z.items_cap, a.scale, a.dk, a.dk_st, a.dk_sh, a.dv, a.dv_st, a.dv_sh);
  }
  {
    KernelTimer timer("qsa_dq", st);
    qsa_dq_ds_kernel<<<(unsigned)(z.ntiles * z.Hk), 64 * kRowWaves, 0, st>>>(
        a.kop, a.ds, a.dsbase, a.bits, a.cu, p.blkbase, p.tile_order, (int)z.S, (int)z.T, (int)z.Hk, a.scale,
        a.dq, a.dq_st, a.dq_sh);
  }
}

}  // namespace msa
