// Device-side plan of a THD pack: global block numbering and the dK/dV work
// items, computed from cu_seqlens on the GPU so that no offset ever travels
// back to the host (the pages' tile map is likewise built with no host sync:
// radixark/miles PR #4581, PR body).
//
// Blocks are numbered pack-wide: sequence s owns global blocks
// blkbase[s] .. blkbase[s+1]-1, block c of s being blkbase[s] + c.  A dK/dV
// work item is one global block paired with one chunk of `chunk` consecutive
// query positions starting at the block itself (earlier queries cannot select
// it): block c of a length-L sequence has ceil((L - 128 c) / chunk) items.
#include "msa_internal.h"

namespace msa {

namespace {

constexpr int kPlanThreads = 1024;

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(const int32_t* __restrict__ cu, int S, int chunk,
                                                             int32_t* __restrict__ blkbase,
                                                             int32_t* __restrict__ blk_seq,
                                                             int32_t* __restrict__ itembase,
                                                             int32_t* __restrict__ totals) {
  __shared__ int sb[kPlanThreads];
  __shared__ int si[kPlanThreads];
  const int tid = threadIdx.x;
  int carry_b = 0, carry_i = 0;
  if (tid == 0) blkbase[0] = 0;
  for (int base = 0; base < S; base += kPlanThreads) {
    const int s = base + tid;
    int L = 0, nb = 0, ni = 0;
    if (s < S) {
      L = cu[s + 1] - cu[s];
      nb = (L + kBlock - 1) / kBlock;
      for (int c = 0; c < nb; ++c) ni += (L - kBlock * c + chunk - 1) / chunk;
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
      int it = carry_i + si[tid] - ni;
      blkbase[s + 1] = b0 + nb;
      for (int c = 0; c < nb; ++c) {
        blk_seq[b0 + c] = s;
        itembase[b0 + c] = it;
        it += (L - kBlock * c + chunk - 1) / chunk;
      }
    }
    carry_b += sb[kPlanThreads - 1];
    carry_i += si[kPlanThreads - 1];
    __syncthreads();
  }
  if (tid == 0) {
    itembase[carry_b] = carry_i;
    totals[0] = carry_b;
    totals[1] = carry_i;
  }
}

}  // namespace

void launch_plan(const int32_t* cu, const Sizes& z, const PlanBufs& p, hipStream_t st) {
  {
    KernelTimer timer("plan", st);
    plan_kernel<<<1, kPlanThreads, 0, st>>>(cu, (int)z.S, (int)z.chunk, p.blkbase, p.blk_seq, p.itembase, p.totals);
  }
}

}  // namespace msa
