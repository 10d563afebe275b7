// Device-side plan of a THD pack: global block numbering and the dK/dV work
// items, computed from cu_seqlens on the GPU so that no offset ever travels
// back to the host (the pages' tile map is likewise built with no host sync:
// radixark/miles PR #4581, PR body).
//
// Blocks are numbered pack-wide: sequence s owns global blocks
// blkbase[s] .. blkbase[s+1]-1, block c of s being blkbase[s] + c.  The
// block width is a template parameter: 128-token blocks for the wide
// variant, 64-key tiles for the narrow one (whose 4-token blocks are grouped
// sixteen to a tile); "block" below means that unit.
//
// dK/dV work items are ordered by (sequence, query chunk, block): chunk j of a
// length-L sequence holds query positions [j*chunk, min((j+1)*chunk, L)) and
// forms one item with every block c that one of those queries may select,
// c = 0 .. (min((j+1)*chunk, L) - 1) / 128.  Consecutive items therefore read
// the same queries, which keeps them in L2 while the workgroups of a chunk run.
// seqitem[s] is the first item of sequence s.
//
// Token tiles (kAttnTile consecutive tokens of the pack) are put in launch
// order by decreasing position of their first token within its sequence: a
// later query has more causal blocks to choose from, so its tile's union of
// selected blocks, and with it the tile's work, is larger.  Launching the
// long tiles first (longest-processing-time order) keeps the last wave of
// workgroups short.  Tiles of equal key may come in any order; the order only
// decides which workgroup runs when, never what any of them computes.
#include "plan_blocks.h"

namespace msa {

namespace {

constexpr int kPlanThreads = 1024;

template <int kUnit>
__global__ __launch_bounds__(kPlanThreads) void plan_kernel(const int32_t* __restrict__ cu, int S, int chunk,
                                                             int ntiles, int32_t* __restrict__ blkbase,
                                                             int32_t* __restrict__ blk_seq,
                                                             int32_t* __restrict__ seqitem,
                                                             int32_t* __restrict__ totals,
                                                             int32_t* __restrict__ tile_order) {
  __shared__ int sb[kPlanThreads];
  __shared__ int si[kPlanThreads];
  __shared__ int hist[kOrderBins];
  __shared__ int scu[kCuCache];
  plan_blocks<kPlanThreads, kUnit>(cu, S, chunk, blkbase, blk_seq, seqitem, totals, sb, si);
  // ntiles = 0: the caller needs no tile order
  if (ntiles > 0) plan_tile_order<kPlanThreads, 8>(cu, S, ntiles, tile_order, sb, hist, scu);
}

}  // namespace

void launch_plan(const int32_t* cu, const Sizes& z, const PlanBufs& p, hipStream_t st, int unit, bool tiles) {
  KernelTimer timer("plan", st);
  const int nt = tiles ? (int)z.ntiles : 0;
  if (unit == kQsaKeyTile)
    plan_kernel<kQsaKeyTile><<<1, kPlanThreads, 0, st>>>(cu, (int)z.S, (int)z.chunk, nt, p.blkbase, p.blk_seq,
                                                        p.seqitem, p.totals, p.tile_order);
  else
    plan_kernel<kBlock><<<1, kPlanThreads, 0, st>>>(cu, (int)z.S, (int)z.chunk, nt, p.blkbase, p.blk_seq,
                                                   p.seqitem, p.totals, p.tile_order);
}

}  // namespace msa
