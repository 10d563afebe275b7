// Device-side plan of a THD pack: global block numbering, the dK/dV work
// items and the launch order of token tiles, computed from cu_seqlens on the
// GPU so that no offset ever travels back to the host (the pages' tile map is
// likewise built with no host sync: radixark/miles PR #4581, PR body).  It is
// written by one extra workgroup of the first kernel of each pass (the
// selection's feature kernel, the forward and backward prep kernels, the
// narrow variant's bitmap kernel); the kernels after it read it.
//
// Blocks are numbered pack-wide: sequence s owns global blocks
// blkbase[s] .. blkbase[s+1]-1, block c of s being blkbase[s] + c; blk_seq
// maps a global block back to its sequence.  The block width is a template
// parameter: 128-token blocks for the wide variant, 64-key tiles for the
// narrow one (whose 4-token blocks are grouped sixteen to a tile); "block"
// below means that unit.
//
// dK/dV work items are ordered by (sequence, query chunk, block): chunk j of a
// length-L sequence holds query positions [j*chunk, min((j+1)*chunk, L)) and
// forms one item with every block c that one of those queries may select,
// c = 0 .. (min((j+1)*chunk, L) - 1) / unit.  Consecutive items therefore read
// the same queries.  seqitem[s] is the first item of sequence s; totals =
// {blocks, items}.
//
// Token tiles (kAttnTile consecutive tokens of the pack, or the forward's
// wider tiles) are put in launch
// order by decreasing position of their first token within its sequence: a
// later query has more causal blocks to choose from, so its tile's union of
// selected blocks, and with it the tile's work, is larger.  Launching the
// long tiles first (longest-processing-time order) keeps the last wave of
// workgroups short.  Tiles of equal key may come in any order; the order only
// decides which workgroup runs when, never what any of them computes.
#pragma once
#include "msa_internal.h"

namespace msa {

template <int kUnit>
__device__ __forceinline__ int chunk_items(int L, int chunk, int j) {
  return (min((j + 1) * chunk, L) - 1) / kUnit + 1;
}

// Run by all kThreads threads of one workgroup; sb and si are LDS arrays of
// kThreads ints.  Ends with a workgroup barrier.
template <int kThreads, int kUnit>
__device__ __forceinline__ void plan_blocks(const int32_t* __restrict__ cu, int S, int chunk,
                                            int32_t* __restrict__ blkbase, int32_t* __restrict__ blk_seq,
                                            int32_t* __restrict__ seqitem, int32_t* __restrict__ totals,
                                            int* sb, int* si) {
  const int tid = threadIdx.x;
  int carry_b = 0, carry_i = 0;
  if (tid == 0) {
    blkbase[0] = 0;
    seqitem[0] = 0;
  }
  for (int base = 0; base < S; base += kThreads) {
    const int s = base + tid;
    int L = 0, nb = 0, ni = 0;
    if (s < S) {
      L = cu[s + 1] - cu[s];
      nb = (L + kUnit - 1) / kUnit;
      const int nch = (L + chunk - 1) / chunk;
      for (int j = 0; j < nch; ++j) ni += chunk_items<kUnit>(L, chunk, j);
    }
    sb[tid] = nb;
    si[tid] = ni;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {  // inclusive Hillis-Steele scan
      int a = tid >= off ? sb[tid - off] : 0;
      int b = tid >= off ? si[tid - off] : 0;
      __syncthreads();
      sb[tid] += a;
      si[tid] += b;
      __syncthreads();
    }
    if (s < S) {
      const int b0 = carry_b + sb[tid] - nb;
      blkbase[s + 1] = b0 + nb;
      seqitem[s + 1] = carry_i + si[tid];
      for (int c = 0; c < nb; ++c) blk_seq[b0 + c] = s;
    }
    carry_b += sb[kThreads - 1];
    carry_i += si[kThreads - 1];
    __syncthreads();
  }
  if (tid == 0) {
    totals[0] = carry_b;
    totals[1] = carry_i;
  }
}

constexpr int kOrderBins = 1024;  // tile order keys: one per 128-token block (131072 tokens)
constexpr int kCuCache = 4097;    // cu_seqlens entries held in LDS for the tile keys

// Order key of token tile i (kTile tokens a tile): block of its first token within that token's sequence.
template <int kTile>
__device__ __forceinline__ int tile_key(const int32_t* cu, int S, int i) {
  const int t0 = i * kTile;
  const int s = find_seq(cu, S, t0);
  return min((t0 - cu[s]) / kBlock, kOrderBins - 1);
}

// Token tiles (kTile tokens each) in launch order: a counting sort on tile_key, largest key first
// (a later query chooses among more blocks, so its tile's union, and work,
// is larger; the order within a key is free).  Run by all kThreads threads of
// one workgroup; sb: kThreads ints, hist: kOrderBins ints, scu: kCuCache ints
// of LDS.  kKeys tile keys per thread stay in registers between the passes.
template <int kThreads, int kKeys, int kTile = kAttnTile>
__device__ __forceinline__ void plan_tile_order(const int32_t* __restrict__ cu, int S, int ntiles,
                                                int32_t* __restrict__ tile_order, int* sb, int* hist, int* scu) {
  static_assert(kOrderBins % kThreads == 0, "whole bins per thread");
  constexpr int kBins = kOrderBins / kThreads;
  const int tid = threadIdx.x;
  const bool cached = S + 1 <= kCuCache;
  if (cached)
    for (int i = tid; i <= S; i += kThreads) scu[i] = cu[i];
  const int32_t* cus = cached ? (const int32_t*)scu : cu;
  for (int b = tid; b < kOrderBins; b += kThreads) hist[b] = 0;
  __syncthreads();
  int keys[kKeys];
#pragma unroll
  for (int e = 0; e < kKeys; ++e) {
    const int i = tid + e * kThreads;
    keys[e] = i < ntiles ? tile_key<kTile>(cus, S, i) : 0;
    if (i < ntiles) atomicAdd(&hist[keys[e]], 1);
  }
  for (int i = tid + kKeys * kThreads; i < ntiles; i += kThreads) atomicAdd(&hist[tile_key<kTile>(cus, S, i)], 1);
  __syncthreads();
  // thread tid owns scan slots kBins tid .. kBins tid + kBins - 1, slot j
  // holding key kOrderBins - 1 - j (largest key first)
  int cnt[kBins], sum = 0;
#pragma unroll
  for (int u = 0; u < kBins; ++u) {
    cnt[u] = hist[kOrderBins - 1 - (kBins * tid + u)];
    sum += cnt[u];
  }
  sb[tid] = sum;
  __syncthreads();
  for (int off = 1; off < kThreads; off <<= 1) {  // inclusive Hillis-Steele scan
    const int a = tid >= off ? sb[tid - off] : 0;
    __syncthreads();
    sb[tid] += a;
    __syncthreads();
  }
  int run = sb[tid] - sum;  // first launch slot of this thread's first key
#pragma unroll
  for (int u = 0; u < kBins; ++u) {
    hist[kOrderBins - 1 - (kBins * tid + u)] = run;
    run += cnt[u];
  }
  __syncthreads();
#pragma unroll
  for (int e = 0; e < kKeys; ++e) {
    const int i = tid + e * kThreads;
    if (i < ntiles) tile_order[atomicAdd(&hist[keys[e]], 1)] = i;
  }
  for (int i = tid + kKeys * kThreads; i < ntiles; i += kThreads)
    tile_order[atomicAdd(&hist[tile_key<kTile>(cus, S, i)], 1)] = i;
}

// Sequence and block index of global block gb (kUnit-token blocks), without
// the plan's tables: wavefront 0 scans the sequences' block counts, 64 at a
// time, and leaves {s, c} in loc (s = -1 when gb is past the pack's last
// block).  Ends with a workgroup barrier.
template <int kUnit>
__device__ __forceinline__ void locate_block(const int32_t* __restrict__ cu, int S, int gb, int* loc) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int carry = 0;
    for (int base = 0; base < S && carry <= gb; base += 64) {
      const int s = base + lane;
      const int nb = s < S ? (cu[s + 1] - cu[s] + kUnit - 1) / kUnit : 0;
      int incl = nb;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
      }
      const int first = carry + incl - nb;
      if (gb >= first && gb < first + nb) {
        loc[0] = s;
        loc[1] = gb - first;
      }
      carry += __shfl(incl, 63);
    }
    if (lane == 0 && carry <= gb) loc[0] = -1;
  }
  __syncthreads();
}

}  // namespace msa
