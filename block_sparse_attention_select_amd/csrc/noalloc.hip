// Allocation-free block-sparse attention forward: msa_attn_fwd with its
// workspace (the pass plan and the per-block K / V^T staging copies) in a
// static device array instead of a caller-provided buffer, for callers that
// cannot allocate (code under HIP graph capture, tight serving loops).
//
// Each GPU the library runs on holds its own copy of `scratch` for the life of
// the process.  Its device address on the current device is looked up once
// with hipGetSymbolAddress and kept per device; host code only ever passes
// that address, never the array's name (which on the host is a stand-in, not
// a device address).  Every call on one GPU shares that GPU's array: calls
// that overlap on one GPU (two streams, two threads) race on it.  The forward
// writes every byte of its workspace it later reads (plan and staging copies
// are rebuilt on each call), so nothing needs clearing between calls.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/msa.h"

static __device__ __align__(256) unsigned char scratch[MSA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device (looked up on the first
// call on that device).
int scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MSA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MSA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MSA_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MSA_OK;
}

}  // namespace

extern "C" int msa_attn_fwd_noalloc(const msa_dims* dims, const void* q, int64_t q_st, int64_t q_sh,
                                    const void* k, int64_t k_st, int64_t k_sh, const void* v, int64_t v_st,
                                    int64_t v_sh, const int32_t* blk_idx, const int32_t* cu_seqlens,
                                    float softmax_scale, void* o, int64_t o_st, int64_t o_sh, float* lse,
                                    hipStream_t stream) {
  size_t need = 0;
  int st = msa_workspace_size(dims, MSA_OP_FWD, &need);
  if (st != MSA_OK) return st;
  if (need > (size_t)MSA_NOALLOC_SCRATCH_BYTES) return MSA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    st = scratch_on_current_device(&ws);
    if (st != MSA_OK) return st;
  }
  return msa_attn_fwd(dims, q, q_st, q_sh, k, k_st, k_sh, v, v_st, v_sh, blk_idx, cu_seqlens, softmax_scale, o,
                      o_st, o_sh, lse, ws, (size_t)MSA_NOALLOC_SCRATCH_BYTES, stream);
}
