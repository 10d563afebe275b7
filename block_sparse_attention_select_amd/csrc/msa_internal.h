// Internal declarations of the MSA HIP library: device helpers shared by the
// kernels, the workspace layout and the host-side launchers.  gfx950 only.
#pragma once

#include <cmath>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace msa {

constexpr int kHeadDim = 128;   // D
constexpr int kBlock = 128;     // keys per block
constexpr int kTopk = 16;       // selected blocks per query
constexpr int kGroup = 16;      // query heads per KV head
constexpr int kMaxBlocks = 1024;  // blocks per sequence this build handles (131072 tokens)

typedef uint16_t u16;

// ----------------------------------------------------------------------------
// Workspace layout (all offsets 256-byte aligned).  Computed identically by
// msa_workspace_size and by each operation.
// ----------------------------------------------------------------------------
struct Sizes {
  int64_t T, S, Hq, Hk, max_seqlen;
  int64_t nbmax;      // ceil(max_seqlen / 128): blocks of the longest sequence
  int64_t nblk_cap;   // bound on the total number of blocks of the pack
  int64_t chunk;      // query positions per dK/dV work item (a multiple of 128)
  int64_t items_cap;  // bound on the number of dK/dV work items per KV head
  int64_t ntiles;     // ceil(T / kAttnTile)
};

struct PlanBufs {
  int32_t* blkbase;   // [S+1]       first global block of each sequence
  int32_t* blk_seq;   // [nblk_cap]  sequence of each global block
  int32_t* seqitem;   // [S+1]       first dK/dV work item of each sequence
  int32_t* totals;    // [4]         {number of blocks, number of work items}
  int32_t* tile_order;  // [ntiles]  token tiles in launch order (longest expected work first)
};

// Tokens per workgroup tile of the token-major attention passes (forward, dQ).
constexpr int kAttnTile = 16;

// ----------------------------------------------------------------------------
// Device helpers
// ----------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
// Native 16-byte vector: unlike HIP's uint4 (a union-based struct) it stays in
// registers when copied around.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf2f(u16 h) { return __uint_as_float(((uint32_t)h) << 16); }
__device__ __forceinline__ u16 f2bf(float f) { return __builtin_bit_cast(u16, (__bf16)f); }

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 load_bf16x8(const u16* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

__device__ __forceinline__ bf16x8 zero_bf16x8() { return __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0)); }

// Two 4-element halves (8 bytes each) joined into one MFMA operand.
__device__ __forceinline__ bf16x8 load_bf16x4x2(const u16* lo, const u16* hi) {
  uint2 a = *reinterpret_cast<const uint2*>(lo);
  uint2 b = *reinterpret_cast<const uint2*>(hi);
  return __builtin_bit_cast(bf16x8, make_uint4(a.x, a.y, b.x, b.y));
}

__device__ __forceinline__ bf16x8 pack_bf16x8(f32x4 lo, f32x4 hi) {
  bf16x8 r;
  r[0] = (__bf16)lo[0]; r[1] = (__bf16)lo[1]; r[2] = (__bf16)lo[2]; r[3] = (__bf16)lo[3];
  r[4] = (__bf16)hi[0]; r[5] = (__bf16)hi[1]; r[6] = (__bf16)hi[2]; r[7] = (__bf16)hi[3];
  return r;
}

// Two floats to one dword of bf16 (round to nearest even), low half first.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, bf16x2{(__bf16)a, (__bf16)b});
}

__device__ __forceinline__ uint2 pack_bf16x4(f32x4 v) {
  uint32_t a = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
  uint32_t b = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
  return make_uint2(a, b);
}

// Largest s in [0, S) with cu[s] <= t (the sequence holding token t).
// RoPE inverse frequencies base^(-2i/64) of the 32 rotated pairs, computed
// once on the host in fp64 and passed by value to the kernels that rotate
struct RopeFreqs {
  double f[32];
};
inline RopeFreqs rope_freqs(float rope_base) {
  RopeFreqs r;
  for (int i = 0; i < 32; ++i) r.f[i] = std::pow((double)rope_base, -(double)(2 * i) / 64.0);
  return r;
}

// Parameters of the attention-side norm fused into the attention kernels:
// the [128] bf16 gemma weights of q and k (used as 1 + w), eps and the host's
// inverse RoPE frequencies.
struct QkNormParams {
  const u16* w_q;
  const u16* w_k;
  float eps;
  RopeFreqs fr;
};

// frequency of pair `lane` (lanes >= 32 get pair 0's, unused): a select
// chain over scalar registers, so the by-value table is never indexed
// per lane (which would put it in scratch memory)
__device__ __forceinline__ double rope_freq_of(const RopeFreqs& fr, int lane) {
  double f = fr.f[0];
#pragma unroll
  for (int i = 1; i < 32; ++i) f = lane == i ? fr.f[i] : f;
  return f;
}

__device__ __forceinline__ int find_seq(const int32_t* __restrict__ cu, int S, int t) {
  int lo = 0, hi = S;
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid;
  }
  return lo;
}

// Largest i in [0, n) with a[i] <= x, for non-decreasing a.
__device__ __forceinline__ int upper_index(const int32_t* __restrict__ a, int n, int x) {
  int lo = 0, hi = n;
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (a[mid] <= x) lo = mid; else hi = mid;
  }
  return lo;
}

// 2^x on the transcendental unit (v_exp_f32), branch-free; 2^-inf = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Lane exchanges across the four row groups of an MFMA accumulator column
// (lanes li, li+16, li+32, li+48).  v_permlane32_swap / v_permlane16_swap on
// two copies of x leave lane i holding x from lanes i and i^32 (resp. i^16) in
// the two results.  The second copy goes through an empty asm so the compiler
// cannot treat the two operands as one value and fold the cross-lane swap away.
__device__ __forceinline__ void swap32(float x, float& a, float& b) {
  uint32_t u = __builtin_bit_cast(uint32_t, x), v = u;
  asm volatile("" : "+v"(v));
  const auto r = __builtin_amdgcn_permlane32_swap(u, v, false, false);
  const uint32_t r0 = r[0], r1 = r[1];  // (bit_cast of a vector element reads element 0)
  a = __builtin_bit_cast(float, r0);
  b = __builtin_bit_cast(float, r1);
}
__device__ __forceinline__ void swap16(float x, float& a, float& b) {
  uint32_t u = __builtin_bit_cast(uint32_t, x), v = u;
  asm volatile("" : "+v"(v));
  const auto r = __builtin_amdgcn_permlane16_swap(u, v, false, false);
  const uint32_t r0 = r[0], r1 = r[1];  // (bit_cast of a vector element reads element 0)
  a = __builtin_bit_cast(float, r0);
  b = __builtin_bit_cast(float, r1);
}

// Maximum over the four row groups, in lane-swap VALU ops instead of LDS permutes.
__device__ __forceinline__ float max_over_groups(float x) {
  float a, b;
  swap32(x, a, b);
  swap16(fmaxf(a, b), a, b);
  return fmaxf(a, b);
}

// Sum over the four row groups.
__device__ __forceinline__ float sum_over_groups(float x) {
  float a, b;
  swap32(x, a, b);
  swap16(a + b, a, b);
  return a + b;
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ----------------------------------------------------------------------------
// Optional per-kernel timing: while msa_timing_enable(1) is in force, a
// KernelTimer records a HIP event pair around the launch it scopes.
// ----------------------------------------------------------------------------
class KernelTimer {
 public:
  KernelTimer(const char* name, hipStream_t st);
  ~KernelTimer();
  KernelTimer(const KernelTimer&) = delete;
  KernelTimer& operator=(const KernelTimer&) = delete;

 private:
  const char* name_;
  hipStream_t st_;
  hipEvent_t start_ = nullptr;
};

// ----------------------------------------------------------------------------
// Launchers (host functions, each defined next to its kernels).
// ----------------------------------------------------------------------------

void launch_select(const Sizes& z, const u16* idx_q, int64_t sq_t, int64_t sq_h,
                   const u16* idx_k, int64_t sk_t, int64_t sk_h, const u16* w_q, const u16* w_k,
                   float eps, float rope_base, const int32_t* cu, const PlanBufs& p,
                   bool force_init, u16* qfeat, u16* kfeat, float* scores, int32_t* blk_idx, hipStream_t st);

// Forward operand copies of K and V per (global block, KV head) (attn_fwd.hip).
// nrm: the attention-side norm fused into the prep (K) and forward (q)
// kernels, or nullptr for already normalized q and k.
void launch_block_prep(const Sizes& z, const u16* k, int64_t k_st, int64_t k_sh, const u16* v, int64_t v_st,
                       int64_t v_sh, const int32_t* cu, const PlanBufs& p, const QkNormParams* nrm, bool dense,
                       u16* kop, u16* vt, hipStream_t st);

// The forward's tile: 32 tokens (4 per wavefront) for sparse layers without
// the fused norm whose longest sequence is at least kWideFwdSeqlen tokens,
// else 16 (1 per wavefront).  launch_block_prep orders the tiles for it.
constexpr int64_t kWideFwdSeqlen = 12288;
int fwd_tokens_per_wave(const Sizes& z, bool dense, bool nrm);

void launch_attn_fwd(const Sizes& z, const u16* q, int64_t q_st, int64_t q_sh,
                     const u16* kop, const u16* vt,
                     const int32_t* blk_idx, const int32_t* cu, const PlanBufs& p, float scale,
                     u16* o, int64_t o_st, int64_t o_sh, float* lse, bool dense, const QkNormParams* nrm,
                     hipStream_t st);

// Attention-side q/k norm + RoPE.  Forward: q, k in, qo, ko out.  Backward:
// q, k (the forward's inputs) and dqh, dkh (gradients of its outputs) in,
// dx written to qo, ko; weight gradients to dw_q, dw_k.
struct QkNormArgs {
  const u16* q; int64_t q_st, q_sh;
  const u16* k; int64_t k_st, k_sh;
  const u16* w_q;
  const u16* w_k;
  float eps, rope_base;
  const int32_t* cu;
  const u16* dqh; int64_t dqh_st, dqh_sh;
  const u16* dkh; int64_t dkh_st, dkh_sh;
  u16* qo; int64_t qo_st, qo_sh;
  u16* ko; int64_t ko_st, ko_sh;
  float* dw_q;
  float* dw_k;
};
constexpr int kQkBwdMaxRows = 1024;  // workgroups of the backward (weight-gradient partial rows)
int qk_norm_bwd_rows(int64_t T);
void launch_qk_norm_fwd(const Sizes& z, const QkNormArgs& a, hipStream_t st);
void launch_qk_norm_bwd(const Sizes& z, const QkNormArgs& a, float* partial, hipStream_t st);
// The backward over the k rows alone (q's part done elsewhere): dkh in, dx to
// ko, partial rows [0, qk_norm_bwd_rows(T)) with a zero q half; then the
// weight-gradient sums over those rows and the extra_rows rows after them,
// through mid (one row per 16 rows summed).
void launch_qk_norm_bwd_k(const Sizes& z, const QkNormArgs& a, float* partial, int extra_rows, float* mid,
                          hipStream_t st);

struct BwdArgs {
  const u16* q; int64_t q_st, q_sh;
  const u16* k; int64_t k_st, k_sh;
  const u16* v; int64_t v_st, v_sh;
  const u16* o; int64_t o_st, o_sh;
  const float* lse;
  const u16* dO; int64_t do_st, do_sh;
  const int32_t* blk_idx;
  const int32_t* cu;
  float scale;
  bool dense;       // every causal key (blk_idx unused)
  u16* dq; int64_t dq_st, dq_sh;
  u16* dk; int64_t dk_st, dk_sh;
  u16* dv; int64_t dv_st, dv_sh;
  // workspace
  u16* kop;         // [nblk][Hk][32 runs][64 slots][8] K in the dQ pass's staging order
  u16* vop;         // the same for V
  float* delta;     // [T][Hq]
  float* nlse;      // [T][Hq] -LSE * log2(e), -inf for rows without keys
  int32_t* item_count;  // [Hk][items_cap]
  int32_t* item_load;   // [Hk][items_cap] selecting queries per item (launch order only)
  int32_t* item_order;  // [Hk][items_cap] items by decreasing load
  float* part_dk;   // [Hk][items_cap][128][128]
  float* part_dv;
  // sparse layers without the fused norm, when it fits kDsBufMaxBytes and the
  // caller did not ask for the recomputing form: the dK/dV pass stores every
  // (token, KV head, listed block)'s bf16 dS here
  // ([T][Hk][16][4 quarters][64 lanes][8]) and dQ is formed from it
  u16* ds = nullptr;
  // attention-side norm fused in (nrm != nullptr): q and k are raw; the prep
  // and dQ kernels normalize them (writing the normalized rows to khat and
  // qhat for the dK/dV pass), dq comes out for the raw q, and the dQ kernel
  // leaves one weight-gradient row per (tile, head, token slot) in dwq_rows
  // ([rows][256]: dw_q sums in columns 0..127, zeros in 128..255)
  const QkNormParams* nrm = nullptr;
  u16* qhat = nullptr;
  u16* khat = nullptr;
  float* dwq_rows = nullptr;
};

void launch_attn_bwd(const Sizes& z, const BwdArgs& a, const PlanBufs& p, hipStream_t st);
void launch_attn_bwd_dkdv(const Sizes& z, const BwdArgs& a, const PlanBufs& p, hipStream_t st);

// Largest number of query positions in one dK/dV work item.
constexpr int kDkdvChunkMax = 2048;

// Largest stored-dS buffer (16 blocks x 4 KB per token and KV head); longer
// packs take the backward that recomputes S and dP in the dQ pass.
constexpr int64_t kDsBufMaxBytes = int64_t(16) << 30;
constexpr int64_t kDsBytesPerRow = int64_t(kTopk) * kBlock * kGroup * 2;

// ----------------------------------------------------------------------------
// Narrow-block variant: 4-token blocks, head dim 256, 12 query heads per KV
// head (qsa_attn.hip).  Key tiles of 64 keys (16 blocks) are its unit of
// staging; Sizes::nblk_cap then counts key tiles and the plan's blkbase /
// blk_seq number key tiles.
// ----------------------------------------------------------------------------
constexpr int kQsaHeadDim = 256;
constexpr int kQsaBlock = 4;
constexpr int kQsaGroup = 12;
constexpr int kQsaKeyTile = 64;
constexpr int kQsaMaxSeqlen = 32768;
constexpr int kQsaMaxTopk = 1024;
constexpr int kQsaChunkMax = 1024;  // query positions per narrow dK/dV work item, at most
constexpr int kQsaWords = kQsaMaxSeqlen / kQsaBlock / 32;  // bitmap words per (token, KV head)

struct QsaArgs {
  const u16* q; int64_t q_st, q_sh;
  const u16* k; int64_t k_st, k_sh;
  const u16* v; int64_t v_st, v_sh;
  const u16* o; int64_t o_st, o_sh;
  const float* lse;
  const u16* dO; int64_t do_st, do_sh;
  const int32_t* blk_idx;
  int topk;
  const int32_t* cu;
  float scale;
  u16* out_o; int64_t oo_st, oo_sh;   // forward output
  float* out_lse;
  u16* dq; int64_t dq_st, dq_sh;
  u16* dk; int64_t dk_st, dk_sh;
  u16* dv; int64_t dv_st, dv_sh;
  // workspace
  uint32_t* bits;     // [T][Hk][kQsaWords] selected-block bitmaps
  int64_t* dsbase;    // [S+1] first dS slot of each sequence (backward)
  u16* vt;            // [key tiles][Hk][32 runs][64 lanes][8] V^T in MFMA operand order (forward)
  u16* kop;           // the same shape: K in the forward's (or, backward, the dQ pass's swizzled) stage order
  u16* ds;            // [slot][Hk][12][64] bf16 dS per (token, causal key tile) slot (backward)
  float* delta;       // [T][Hk][16] (heads past 12 unused)
  float* nlse;        // [T][Hk][16] -LSE * log2(e) (-inf for empty rows; heads past 12 unused)
  int32_t* item_count;  // [Hk][items_cap]
  float* part_dk;     // [Hk][items_cap][64][256]
  float* part_dv;
};
void launch_qsa_fwd(const Sizes& z, const QsaArgs& a, const PlanBufs& p, hipStream_t st);
void launch_qsa_bwd(const Sizes& z, const QsaArgs& a, const PlanBufs& p, hipStream_t st);

// Barrier for LDS traffic only: waits for this wavefront's LDS operations,
// then for every wavefront of the workgroup, without draining outstanding
// global loads (prefetches stay in flight across it).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace msa
