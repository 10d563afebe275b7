// Block numbering and dK/dV work items of a THD pack, as a device function
// shared by the plan kernel and the selection's feature kernel (which runs it
// in one extra workgroup, so the selection needs no launch of its own for it).
//
// Sequence s owns global blocks blkbase[s] .. blkbase[s+1]-1 (kUnit tokens
// each); blk_seq maps a global block back to its sequence; seqitem[s] is the
// first dK/dV work item of sequence s (items: every (query chunk, block the
// chunk's queries may select) pair); totals = {blocks, items}.
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

}  // namespace msa
