// Device-side plan of a THD pack: global block numbering and the dK/dV work
// items, computed from cu_seqlens on the GPU so that no offset ever travels
// back to the host (the pages' tile map is likewise built with no host sync:
// radixark/miles PR #4581, PR body).
//
// Blocks are numbered pack-wide: sequence s owns global blocks
// blkbase[s] .. blkbase[s+1]-1, block c of s being blkbase[s] + c.
//
// dK/dV work items are ordered by (sequence, query chunk, block): chunk j of a
// length-L sequence holds query positions [j*chunk, min((j+1)*chunk, L)) and
// forms one item with every block c that one of those queries may select,
// c = 0 .. (min((j+1)*chunk, L) - 1) / 128.  Consecutive items therefore read
// the same queries, which keeps them in L2 while the workgroups of a chunk run.
// seqitem[s] is the first item of sequence s.
#include "msa_internal.h"

namespace msa {

namespace {

constexpr int kPlanThreads = 1024;

__device__ __forceinline__ int chunk_items(int L, int chunk, int j) {
  return (min((j + 1) * chunk, L) - 1) / kBlock + 1;
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(const int32_t* __restrict__ cu, int S, int chunk,
                                                             int32_t* __restrict__ blkbase,
                                                             int32_t* __restrict__ blk_seq,
                                                             int32_t* __restrict__ seqitem,
                                                             int32_t* __restrict__ totals) {
  __shared__ int sb[kPlanThreads];
  __shared__ int si[kPlanThreads];
  const int tid = threadIdx.x;
  int carry_b = 0, carry_i = 0;
  if (tid == 0) {
    blkbase[0] = 0;
    seqitem[0] = 0;
  }
  for (int base = 0; base < S; base += kPlanThreads) {
    const int s = base + tid;
    int L = 0, nb = 0, ni = 0;
    if (s < S) {
      L = cu[s + 1] - cu[s];
      nb = (L + kBlock - 1) / kBlock;
      const int nch = (L + chunk - 1) / chunk;
      for (int j = 0; j < nch; ++j) ni += chunk_items(L, chunk, j);
    }
    sb[tid] = nb;
    si[tid] = ni;
    __syncthreads();
    for (int off = 1; off < kPlanThreads; off <<= 1) {  // inclusive Hillis-Steele scan
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
    carry_b += sb[kPlanThreads - 1];
    carry_i += si[kPlanThreads - 1];
    __syncthreads();
  }
  if (tid == 0) {
    totals[0] = carry_b;
    totals[1] = carry_i;
  }
}

}  // namespace

void launch_plan(const int32_t* cu, const Sizes& z, const PlanBufs& p, hipStream_t st) {
  {
    KernelTimer timer("plan", st);
    plan_kernel<<<1, kPlanThreads, 0, st>>>(cu, (int)z.S, (int)z.chunk, p.blkbase, p.blk_seq, p.seqitem, p.totals);
  }
}

}  // namespace msa
