// dK / dV of the block-sparse GQA attention, key-block-major, on gfx950.
//
// What is computed (radixark/miles PR #4581, kernel-tuning commit: the dK/dV
// kernel of a KV head sums over that head's query heads, each partial written
// to its own slice and the slices summed -- here in a fixed order):
//     dv_j = sum P dO,   dk_j = scale * sum dS q
// over every (query, head) of the group whose selected blocks include j's
// block, with P = exp(scale q.k - LSE) and dS = P (dO.v - Delta).
//
// One workgroup per (work item, KV head); a work item is one chunk of query
// positions of a sequence paired with one block those queries may select;
// items are launched heaviest first (dkdv_order_kernel).
//   1. The chunk's queries that selected the block are listed in token order
//      (wavefront ballots, so the list and every later sum are deterministic).
//   2. Each of the 4 wavefronts keeps 32 keys of K and V as MFMA B operands
//      and the 32 x 128 fp32 dK and dV sums in registers for the whole item.
//   3. Selecting tokens stream through LDS two at a time through a ring of
//      four slots: global_load_lds copies of the next two pairs are in
//      flight while one pair is used (the gathered rows come from HBM, whose
//      latency one pair of work does not cover), with a barrier after every
//      second pair.  Per token the stage holds q
//      and dO laid out so each MFMA A operand is one contiguous 1 KB read, plus
//      the token's 16 LSE and Delta values.
//   4. Two tokens (32 query rows) per MFMA step: S = q K^T and dP = dO V^T
//      (A from LDS, B from registers), then dV += P^T dO and dK += dS^T q
//      with P and dS taken straight from the score registers.  The B operands
//      of dV and dK (dO and q with the head rows as the contraction index) are
//      read from the same stage with ds_read_b64_tr_b16, which transposes 4x4
//      groups of 16-bit elements across lanes on the fly.
//   5. A block whose selecting queries all lie in one chunk writes bf16 dK/dV
//      itself; other blocks write fp32 slices that dkdv_reduce_kernel sums in
//      chunk order.
//   kWriteDs: every selecting (token, block)'s bf16 dS also goes to HBM as the
//      score registers hold it (two 8-byte stores per lane and token; on the
//      token's own block not the 32-key quarters past it), so the
//      token-major dQ pass needs one product per block (dQ = scale dS K)
//      instead of recomputing S and dP.
#include "attn_stage.h"

namespace msa {

namespace {

constexpr int kBatch = 2;  // tokens per staging round
constexpr int kNBuf = 4;   // staging ring: rounds bi+1, bi+2 in flight while bi is used

// Stage layout of one token (u32x4 units): [0,256) q and [256,512) dO as
// [ds][slot], operand lane li + 16g of run ds (row li, dims 32ds + 8g .. +7)
// at slot swz_slot(li + 16g); stats: 16 -LSE*log2(e) then 16 Delta values.
// Two wavefronts copy a token: part 0 the 4 q runs of 1 KB and the 128-byte
// stats run, part 1 the 4 dO runs.  Addresses are a wavefront-uniform base
// (the token's row, scalar registers) plus a per-lane byte offset (head, dims
// 8g..).
__device__ __forceinline__ void stage_part(int t, int part, int h, int Hk, int lane, uint32_t slot_lds, uint32_t stats_lds,
                                           const u16* __restrict__ q, int64_t q_st, int64_t q_sh,
                                           const u16* __restrict__ dO, int64_t do_st, int64_t do_sh,
                                           const float* __restrict__ nlse, const float* __restrict__ delta) {
  t = __builtin_amdgcn_readfirstlane(t);
  const int hr = swz_slot(lane) & 15;
  if (part == 0) {
    const uint32_t q_off = (uint32_t)(2 * (hr * q_sh + 8 * (lane >> 4)));
    const u16* qr = q + (int64_t)t * q_st + (int64_t)(h * kGroup) * q_sh;
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16s(qr + 32 * i, q_off, slot_lds + i * 1024);
    const int64_t row = (int64_t)t * (Hk * kGroup) + h * kGroup;
    if (lane < 16)
      dma4s(nlse + row, 4 * lane, stats_lds);
    else if (lane < 32)
      dma4s(delta + row - 16, 4 * lane, stats_lds);
  } else {
    const uint32_t do_off = (uint32_t)(2 * (hr * do_sh + 8 * (lane >> 4)));
    const u16* dr = dO + (int64_t)t * do_st + (int64_t)(h * kGroup) * do_sh;
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16s(dr + 32 * i, do_off, slot_lds + 4096 + i * 1024);
  }
}

// kDense: every token of the chunk at or after the block's first key selects it (blk_idx unused).
// kWriteDs (sparse only): ds_out[((t Hk + h) 16 + slot) 4 + w][half][lane][4]
// gets the token's bf16 dS for keys 32 w .. 32 w + 31 of the block, lane (key
// li, group g) holding heads 4g .. 4g+3 of key 32 w + 16 half + li, where slot
// is the block's first position in the token's list of selected blocks.
template <bool kDense, bool kWriteDs>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_bwd_dkdv_kernel(
    const u16* __restrict__ q, int64_t q_st, int64_t q_sh,
    const u16* __restrict__ k, int64_t k_st, int64_t k_sh,
    const u16* __restrict__ v, int64_t v_st, int64_t v_sh,
    const u16* __restrict__ dO, int64_t do_st, int64_t do_sh,
    const float* __restrict__ nlse, const float* __restrict__ delta,
    const int32_t* __restrict__ blk_idx, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ blkbase, const int32_t* __restrict__ blk_seq,
    const int32_t* __restrict__ seqitem, const int32_t* __restrict__ totals,
    int S, int Hk, int chunk, int items_cap, const int32_t* __restrict__ item_order, float scale_log2, float scale,
    int32_t* __restrict__ item_count, float* __restrict__ part_dk, float* __restrict__ part_dv,
    u16* __restrict__ dk_out, int64_t dk_st, int64_t dk_sh, u16* __restrict__ dv_out, int64_t dv_st, int64_t dv_sh,
    u16* __restrict__ ds_out) {
  static_assert(!(kDense && kWriteDs), "dS is stored for sparse layers only");
  __shared__ u32x4 stage[kNBuf][kBatch][512];
  __shared__ __align__(16) float stats[kNBuf][kBatch][32];
  // selecting tokens as (token << 4) | list slot of the block
  __shared__ int sel[kDkdvChunkMax];
  __shared__ int wcount[4];

  const int h = blockIdx.y;
  if ((int)blockIdx.x >= totals[1]) return;
  const int item = item_order[(int64_t)h * items_cap + blockIdx.x];
  // decode (sequence, query chunk j, block c) from the item index
  const int s = upper_index(seqitem, S, item);
  const int seq0 = cu[s];
  const int L = cu[s + 1] - seq0;
  const int nch = (L + chunk - 1) / chunk;
  int r = item - seqitem[s];
  int j = 0;
  for (;;) {
    const int cnt = (min((j + 1) * chunk, L) - 1) / kBlock + 1;
    if (r < cnt) break;
    r -= cnt;
    ++j;
  }
  const int c = r;
  const int jmin = (kBlock * c) / chunk;
  const bool single = (j == nch - 1) && (j == jmin);
  const int p_begin = max(j * chunk, kBlock * c);
  const int p_end = min((j + 1) * chunk, L);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int li = lane & 15;

  // 1. the chunk's queries that selected block c, in token order
  int nsel = 0;
  for (int p0 = p_begin; p0 < p_end; p0 += 256) {
    const int p = p0 + threadIdx.x;
    bool hit = false;
    int slot = 0;  // first list position holding block c
    if (kDense) {
      hit = p < p_end;
    } else if (p < p_end) {
      const int4* ids = reinterpret_cast<const int4*>(blk_idx + ((int64_t)(seq0 + p) * Hk + h) * kTopk);
      slot = kTopk;
#pragma unroll
      for (int jj = 3; jj >= 0; --jj) {
        const int4 x = ids[jj];
        slot = x.w == c ? 4 * jj + 3 : slot;
        slot = x.z == c ? 4 * jj + 2 : slot;
        slot = x.y == c ? 4 * jj + 1 : slot;
        slot = x.x == c ? 4 * jj : slot;
      }
      hit = slot < kTopk;
    }
    const uint64_t m = __ballot(hit);
    const int before = __popcll(m & ((1ull << lane) - 1ull));
    if (lane == 0) wcount[wave] = __popcll(m);
    __syncthreads();
    int off = nsel;
    int tot = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      off += w < wave ? wcount[w] : 0;
      tot += wcount[w];
    }
    if (hit) sel[off + before] = ((seq0 + p) << 4) | slot;
    nsel += tot;
    __syncthreads();
  }
  if (threadIdx.x == 0) item_count[(int64_t)h * items_cap + item] = nsel;

  // 2. K and V of this wavefront's 32 keys as B operands (zero past the sequence end)
  const int kbase = kBlock * c + 32 * wave;
  bf16x8 kf[2][4], vf[2][4];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int kp = kbase + 16 * kk + li;
    const bool ok = kp < L;
    const u16* krow = k + (int64_t)(seq0 + kp) * k_st + (int64_t)h * k_sh + 8 * g;
    const u16* vrow = v + (int64_t)(seq0 + kp) * v_st + (int64_t)h * v_sh + 8 * g;
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) {
      kf[kk][ds] = ok ? load_bf16x8(krow + 32 * ds) : zero_bf16x8();
      vf[kk][ds] = ok ? load_bf16x8(vrow + 32 * ds) : zero_bf16x8();
    }
  }
  f32x4 dk[2][8], dv[2][8];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      dk[kk][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
      dv[kk][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  // 3./4. stream the selecting tokens through LDS, two per MFMA step
  if (nsel > 0) {

    const int nbatch = (nsel + kBatch - 1) / kBatch;
    // slots past the end repeat the last token (finite operands, masked to zero)
    // wavefront w copies half of token w % 2 of a round: q and stats (w < 2) or dO
    auto stage_round = [&](int bi, int buf) {
      const int slot = wave & 1;
      stage_part(sel[min(bi * kBatch + slot, nsel - 1)] >> 4, wave >> 1, h, Hk, fresh_lane(),
                 lds_offset(&stage[buf][slot][0]), lds_offset(&stats[buf][slot][0]), q, q_st, q_sh, dO, do_st,
                 do_sh, nlse, delta);
    };
    // round bi + 2 is copied while round bi is used, into the slot of round
    // bi - 2; a barrier follows only every second round (16k pack 444 ->
    // 435 us): there every wavefront has waited for all its copies, rounds
    // bi + 1 and bi + 2 included, and the slot a round refills was released by
    // the barrier after round bi - 2 or bi - 1, whichever is odd
    for (int r = 0; r < kNBuf - 2 && r < nbatch; ++r) stage_round(r, r);
    wait_copies();
    wait_all_loads();
    __syncthreads();
    for (int bi = 0; bi < nbatch; ++bi) {
      const int cur = bi % kNBuf;
      const bool ahead = bi + kNBuf - 2 < nbatch;
      if (ahead) stage_round(bi + kNBuf - 2, (bi + kNBuf - 2) % kNBuf);
#pragma unroll 1
      for (int pp = 0; pp < kBatch / 2; ++pp) {
        const int n0 = bi * kBatch + 2 * pp;
        if (n0 < nsel) {
          // a missing second token is treated as a query at position -1 of
          // this block: every key is after it, so it contributes nothing
          const int tsel[2] = {sel[n0], n0 + 1 < nsel ? sel[n0 + 1] : -1};
          const int pos[2] = {(tsel[0] >> 4) - seq0, tsel[1] >= 0 ? (tsel[1] >> 4) - seq0 : -1};
          const u32x4* b[2] = {stage[cur][2 * pp], stage[cur][2 * pp + 1]};
          const float* st[2] = {stats[cur][2 * pp], stats[cur][2 * pp + 1]};

          // S = q K^T and dP = dO V^T per token, turned at once into bf16 P and
          // dS: lane (key li, group g) keeps rows 4g..4g+3 of each token, packed
          // two per dword as the A operand of dV and dK (dwords 0-1 token 0,
          // dwords 2-3 token 1).
          u32x4 pw[2], sw[2];
          const int ln = fresh_lane();
#pragma unroll
          for (int tk = 0; tk < 2; ++tk) {
            f32x4 sacc[2], pacc[2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
              sacc[kk] = f32x4{0.f, 0.f, 0.f, 0.f};
              pacc[kk] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int ds = 0; ds < 4; ++ds) {
              const bf16x8 qa = __builtin_bit_cast(bf16x8, b[tk][ds * 64 + swz_slot(ln)]);
              const bf16x8 da = __builtin_bit_cast(bf16x8, b[tk][256 + ds * 64 + swz_slot(ln)]);
#pragma unroll
              for (int kk = 0; kk < 2; ++kk) {
                sacc[kk] = mfma16x16x32(qa, kf[kk][ds], sacc[kk]);
                pacc[kk] = mfma16x16x32(da, vf[kk][ds], pacc[kk]);
              }
            }
            const f32x4 nl = reinterpret_cast<const f32x4*>(st[tk])[ln >> 4];
            const f32x4 d4 = reinterpret_cast<const f32x4*>(st[tk] + 16)[ln >> 4];
            f32x4 e[2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
              for (int r = 0; r < 4; ++r) e[kk][r] = fast_exp2(fmaf(sacc[kk][r], scale_log2, nl[r]));
            if (pos[tk] < kBlock * c + kBlock) {  // the query's own block (or no query): causal mask
#pragma unroll
              for (int kk = 0; kk < 2; ++kk) {
                const bool on = kbase + 16 * kk + li <= pos[tk];
#pragma unroll
                for (int r = 0; r < 4; ++r) e[kk][r] = on ? e[kk][r] : 0.f;
              }
            }
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
              f32x4 d;
#pragma unroll
              for (int r = 0; r < 4; ++r) d[r] = e[kk][r] * (pacc[kk][r] - d4[r]);
              pw[kk][2 * tk] = pack_bf16x2(e[kk][0], e[kk][1]);
              pw[kk][2 * tk + 1] = pack_bf16x2(e[kk][2], e[kk][3]);
              sw[kk][2 * tk] = pack_bf16x2(d[0], d[1]);
              sw[kk][2 * tk + 1] = pack_bf16x2(d[2], d[3]);
            }
            if constexpr (kWriteDs) {
              // a query before the wavefront's first key (on its own block)
              // has only zero dS here, which the dQ pass never reads
              if (tsel[tk] >= 0 && pos[tk] >= kbase) {
                // two 512-byte runs of register pairs: one 16-byte store per
                // lane would need the halves copied into four consecutive
                // registers, which this loop does not have to spare.  The
                // stores are non-temporal: the dS is read once, by a later
                // pass, and would otherwise push the gathered q / dO rows and
                // the chunk slices out of the caches (16k pack: dK/dV, reduce
                // and dQ 28 us faster)
                const int64_t row = ((int64_t)(tsel[tk] >> 4) * Hk + h) * kTopk + (tsel[tk] & 15);
                u16* dst = ds_out + (row * 4 + wave) * 512 + 4 * ln;
                __builtin_nontemporal_store(u32x2{sw[0][2 * tk], sw[0][2 * tk + 1]}, reinterpret_cast<u32x2*>(dst));
                __builtin_nontemporal_store(u32x2{sw[1][2 * tk], sw[1][2 * tk + 1]},
                                            reinterpret_cast<u32x2*>(dst + 256));
              }
              // keep the stores here: moved later, the dS registers would stay
              // live across the next token's products
              __builtin_amdgcn_sched_barrier(0);
            }
          }
          bf16x8 pA[2], sA[2];
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            pA[kk] = __builtin_bit_cast(bf16x8, pw[kk]);
            sA[kk] = __builtin_bit_cast(bf16x8, sw[kk]);
          }
          const uint32_t tro = tr_lane_offset(ln);
          const uint32_t q0 = lds_offset(b[0]) + tro, q1 = lds_offset(b[1]) + tro;
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) {
            const uint32_t off = (dt >> 1) * 1024 + (dt & 1) * 512;
            const uint2 a0 = read_tr16(q0 + 4096 + off);
            const uint2 a1 = read_tr16(q1 + 4096 + off);
            const uint2 c0 = read_tr16(q0 + off);
            const uint2 c1 = read_tr16(q1 + off);
            const bf16x8 bdo = __builtin_bit_cast(bf16x8, u32x4{a0.x, a0.y, a1.x, a1.y});
            const bf16x8 bq = __builtin_bit_cast(bf16x8, u32x4{c0.x, c0.y, c1.x, c1.y});
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
              dv[kk][dt] = mfma16x16x32(pA[kk], bdo, dv[kk][dt]);
              dk[kk][dt] = mfma16x16x32(sA[kk], bq, dk[kk][dt]);
            }
          }
        }
      }
      if ((bi & 1) || bi + 1 == nbatch) {
        wait_copies();
        lds_barrier();
      }
    }
  }

  // 5. results: lane holds key 32w + 16kk + 4g + r, dim 16dt + li
  if (single) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kp = kbase + 16 * kk + 4 * g + r;
        if (kp >= L) continue;
        u16* dkr = dk_out + (int64_t)(seq0 + kp) * dk_st + (int64_t)h * dk_sh + li;
        u16* dvr = dv_out + (int64_t)(seq0 + kp) * dv_st + (int64_t)h * dv_sh + li;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          dkr[16 * dt] = f2bf(dk[kk][dt][r] * scale);
          dvr[16 * dt] = f2bf(dv[kk][dt][r]);
        }
      }
  } else if (nsel > 0) {
    const int64_t slice = ((int64_t)h * items_cap + item) * (kBlock * kHeadDim);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = 32 * wave + 16 * kk + 4 * g + r;
          const int64_t off = slice + (int64_t)key * kHeadDim + 16 * dt + li;
          part_dk[off] = dk[kk][dt][r];
          part_dv[off] = dv[kk][dt][r];
        }
  }
}

// ---------------------------------------------------------------------------
// Launch order.  Items differ a lot in work (a chunk's own and nearby blocks
// are selected by most of its queries, far blocks by few), and in index order
// the heavy ones of the last sequence would run last.  The items are instead
// launched by decreasing number of selecting queries (longest job first), which
// only changes when each item runs, not what it computes.  For sparse layers
// the counters are zeroed by the backward prep kernel and filled by the dQ
// pass or the Delta kernel ahead of this one (one count per selecting query,
// head and block); the item of query
// chunk j of sequence s and its block c has index seqitem[s] +
// (chunk / kBlock) * j * (j + 1) / 2 + c.
// ---------------------------------------------------------------------------
// Dense layers: item (s, j, c) is selected by every query of chunk j at or
// after block c's first key.
__global__ __launch_bounds__(256) void dkdv_dense_load_kernel(const int32_t* __restrict__ cu,
                                                              const int32_t* __restrict__ seqitem,
                                                              const int32_t* __restrict__ totals, int S, int chunk,
                                                              int items_cap, int32_t* __restrict__ load) {
  const int item = blockIdx.x * 256 + threadIdx.x;
  const int h = blockIdx.y;
  if (item >= totals[1]) return;
  const int s = upper_index(seqitem, S, item);
  const int L = cu[s + 1] - cu[s];
  int r = item - seqitem[s];
  int j = 0;
  for (;;) {
    const int cnt = (min((j + 1) * chunk, L) - 1) / kBlock + 1;
    if (r < cnt) break;
    r -= cnt;
    ++j;
  }
  load[(int64_t)h * items_cap + item] = max(0, min((j + 1) * chunk, L) - max(j * chunk, kBlock * r));
}

// per KV head: counting sort of the items by decreasing load
constexpr int kLoadBins = kDkdvChunkMax + 1;
__global__ __launch_bounds__(1024) void dkdv_order_kernel(const int32_t* __restrict__ load,
                                                          const int32_t* __restrict__ totals, int items_cap,
                                                          int32_t* __restrict__ order) {
  __shared__ int bins[kLoadBins];
  __shared__ int wsum[16];
  const int h = blockIdx.x;
  const int n = totals[1];
  const int32_t* ld = load + (int64_t)h * items_cap;
  int32_t* od = order + (int64_t)h * items_cap;
  for (int b = threadIdx.x; b < kLoadBins; b += 1024) bins[b] = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += 1024) atomicAdd(&bins[kLoadBins - 1 - min(ld[i], kLoadBins - 1)], 1);
  __syncthreads();
  // exclusive scan of the bins (heaviest first), three bins per thread
  const int b0 = 3 * threadIdx.x;
  int v[3], run = 0;
#pragma unroll
  for (int e = 0; e < 3; ++e) {
    v[e] = b0 + e < kLoadBins ? bins[b0 + e] : 0;
    run += v[e];
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = run;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += wsum[w];
  int pos = base + incl - run;
  __syncthreads();
#pragma unroll
  for (int e = 0; e < 3; ++e) {
    if (b0 + e < kLoadBins) bins[b0 + e] = pos;
    pos += v[e];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += 1024) od[atomicAdd(&bins[kLoadBins - 1 - min(ld[i], kLoadBins - 1)], 1)] = i;
}

}  // namespace

void launch_attn_bwd_dkdv(const Sizes& z, const BwdArgs& a, const PlanBufs& p, hipStream_t st) {
  {
    KernelTimer timer("dkdv_order", st);
    // sparse: the selections per item were counted by an earlier pass; dense: a closed form
    if (a.dense)
      dkdv_dense_load_kernel<<<dim3((unsigned)((z.items_cap + 255) / 256), (unsigned)z.Hk), 256, 0, st>>>(
          a.cu, p.seqitem, p.totals, (int)z.S, (int)z.chunk, (int)z.items_cap, a.item_load);
    dkdv_order_kernel<<<(unsigned)z.Hk, 1024, 0, st>>>(a.item_load, p.totals, (int)z.items_cap, a.item_order);
  }
  KernelTimer timer("attn_bwd_dkdv", st);
  auto kern = a.dense ? attn_bwd_dkdv_kernel<true, false>
                      : (a.ds ? attn_bwd_dkdv_kernel<false, true> : attn_bwd_dkdv_kernel<false, false>);
  // with the attention-side norm fused in, the pass reads the normalized rows
  // the prep and dQ kernels wrote
  const int64_t D = kHeadDim;
  const u16* q = a.nrm ? a.qhat : a.q;
  const int64_t q_st = a.nrm ? z.Hq * D : a.q_st, q_sh = a.nrm ? D : a.q_sh;
  const u16* k = a.nrm ? a.khat : a.k;
  const int64_t k_st = a.nrm ? z.Hk * D : a.k_st, k_sh = a.nrm ? D : a.k_sh;
  kern<<<dim3((unsigned)z.items_cap, (unsigned)z.Hk), 256, 0, st>>>(
      q, q_st, q_sh, k, k_st, k_sh, a.v, a.v_st, a.v_sh, a.dO, a.do_st, a.do_sh, a.nlse,
      a.delta, a.blk_idx, a.cu, p.blkbase, p.blk_seq, p.seqitem, p.totals, (int)z.S, (int)z.Hk, (int)z.chunk,
      (int)z.items_cap, a.item_order, a.scale * kLog2e, a.scale, a.item_count, a.part_dk, a.part_dv, a.dk, a.dk_st, a.dk_sh, a.dv,
      a.dv_st, a.dv_sh, a.ds);
}

}  // namespace msa
