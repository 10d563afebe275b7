// C ABI of the MSA library: argument validation, workspace carving and the
// launch sequence of each operation on the caller's stream.  No host sync
// (except the explicit debug check) and no allocation; the only state is the
// optional kernel-timing event pool (timing.cpp), off unless enabled.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <vector>

#include "../../include/msa.h"
#include "msa_internal.h"

using msa::Sizes;
using msa::PlanBufs;
using msa::u16;

namespace {

constexpr size_t kAlign = 256;
constexpr int64_t kPartialBudget = int64_t(1) << 30;  // bytes of dK/dV chunk slices before chunks grow

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int check_dims(const msa_dims* d) {
  if (!d) return MSA_ERR_INVALID_ARG;
  if (d->total_tokens < 0 || d->num_seqs < 0 || d->max_seqlen < 0 || d->num_q_heads <= 0 ||
      d->num_kv_heads <= 0)
    return MSA_ERR_INVALID_ARG;
  if (d->total_tokens > 0 && (d->num_seqs < 1 || d->max_seqlen < 1)) return MSA_ERR_INVALID_ARG;
  if (d->max_seqlen > d->total_tokens && d->total_tokens > 0) return MSA_ERR_INVALID_ARG;
  if (d->head_dim != msa::kHeadDim || d->block_size != msa::kBlock || d->topk_blocks != msa::kTopk)
    return MSA_ERR_UNSUPPORTED;
  if (d->num_q_heads != msa::kGroup * d->num_kv_heads) return MSA_ERR_UNSUPPORTED;
  if (d->max_seqlen > MSA_MAX_SEQLEN) return MSA_ERR_UNSUPPORTED;
  if (d->num_kv_heads > 65535) return MSA_ERR_UNSUPPORTED;
  // 32-bit element counts inside the kernels
  if ((int64_t)d->total_tokens * d->num_q_heads * msa::kHeadDim >= (int64_t(1) << 31)) return MSA_ERR_UNSUPPORTED;
  return MSA_OK;
}

// Narrow-block variant: head_dim 256, block 4, 12 q heads per KV head,
// 1..1024 listed blocks per query, sequences up to 32768 tokens.
int check_qsa_dims(const msa_dims* d) {
  if (!d) return MSA_ERR_INVALID_ARG;
  if (d->total_tokens < 0 || d->num_seqs < 0 || d->max_seqlen < 0 || d->num_q_heads <= 0 ||
      d->num_kv_heads <= 0 || d->topk_blocks <= 0)
    return MSA_ERR_INVALID_ARG;
  if (d->total_tokens > 0 && (d->num_seqs < 1 || d->max_seqlen < 1)) return MSA_ERR_INVALID_ARG;
  if (d->max_seqlen > d->total_tokens && d->total_tokens > 0) return MSA_ERR_INVALID_ARG;
  if (d->head_dim != msa::kQsaHeadDim || d->block_size != msa::kQsaBlock || d->topk_blocks > msa::kQsaMaxTopk)
    return MSA_ERR_UNSUPPORTED;
  if (d->num_q_heads != msa::kQsaGroup * d->num_kv_heads) return MSA_ERR_UNSUPPORTED;
  if (d->max_seqlen > MSA_QSA_MAX_SEQLEN) return MSA_ERR_UNSUPPORTED;
  if (d->num_kv_heads > 65535) return MSA_ERR_UNSUPPORTED;
  if ((int64_t)d->total_tokens * d->num_q_heads * msa::kQsaHeadDim >= (int64_t(1) << 31)) return MSA_ERR_UNSUPPORTED;
  return MSA_OK;
}

// Grid and workspace bounds of a pack whose blocks (dK/dV work items, key
// numbering) are `unit` tokens wide, with `dhead` dims per head.  The dK/dV
// query chunk starts at `chunk0` tokens and doubles while the chunk slices
// would exceed kPartialBudget.
void size_blocks(Sizes& z, int64_t unit, int64_t dhead, int64_t chunk0, int64_t chunk_max = msa::kDkdvChunkMax) {
  // sum_s ceil(L_s / unit) <= (T + (unit - 1) S) / unit, and <= T
  int64_t cap = (z.T + (unit - 1) * z.S) / unit;
  if (cap > z.T) cap = z.T;
  if (cap < 1) cap = 1;
  z.nblk_cap = cap;
  z.ntiles = (z.T + msa::kAttnTile - 1) / msa::kAttnTile;
  // dK/dV work items: chunk j of a length-L sequence pairs with blocks
  // 0 .. (min((j+1)*chunk, L) - 1) / unit.  With n = ceil(L / chunk) chunks and
  // m = chunk / unit, a sequence has at most min(n * ceil(L / unit),
  // m * n * (n + 1) / 2) items; both sum over a pack to the bounds below.
  int64_t chunk = chunk0;
  for (;;) {
    const int64_t m = chunk / unit;
    const int64_t b1 = z.T * z.max_seqlen / (unit * chunk) + z.T / chunk + z.T / unit + 2 * z.S + 1;
    const int64_t b2 = z.T * z.max_seqlen / (2 * unit * chunk) + 3 * z.T / (2 * unit) + z.S * m + 1;
    const int64_t items = b1 < b2 ? b1 : b2;
    const int64_t bytes = items * z.Hk * unit * dhead * 4 * 2;
    if (bytes <= kPartialBudget || chunk >= chunk_max) {
      z.chunk = chunk;
      z.items_cap = items;
      break;
    }
    chunk *= 2;
  }
}

Sizes sizes_of_qsa(const msa_dims* d) {
  Sizes z;
  z.T = d->total_tokens;
  z.S = d->num_seqs;
  z.Hq = d->num_q_heads;
  z.Hk = d->num_kv_heads;
  z.max_seqlen = d->max_seqlen;
  z.nbmax = (z.max_seqlen + msa::kQsaKeyTile - 1) / msa::kQsaKeyTile;
  // dK/dV query chunks of 256 tokens: on the 16k narrow pack (512 listed
  // blocks per query) 512-token chunks took the dK/dV pass 1.79 ms against
  // 1.59 ms, while the reduce grew from 52 to 103 us; 128 gained nothing more
  size_blocks(z, msa::kQsaKeyTile, msa::kQsaHeadDim, 256, msa::kQsaChunkMax);
  return z;
}

Sizes sizes_of(const msa_dims* d) {
  Sizes z;
  z.T = d->total_tokens;
  z.S = d->num_seqs;
  z.Hq = d->num_q_heads;
  z.Hk = d->num_kv_heads;
  z.max_seqlen = d->max_seqlen;
  z.nbmax = (z.max_seqlen + msa::kBlock - 1) / msa::kBlock;
  // The dK/dV pass launches its items longest first over two workgroups per
  // CU (512 slots), and an item's work grows with its chunk: the item of a
  // chunk's own block is selected by every query of the chunk.  Chunks stay
  // at 512 tokens until a slot's share of the T * Hk * 16 selections exceeds
  // that (T * Hk / 32 > chunk), then grow with it up to 2048: fewer, longer
  // items, so fewer chunk slices for the reduce to sum, while no single item
  // outlasts a slot's share (16k pack 512, 32k pack 1024, 32k x 4 heads 2048).
  int64_t chunk0 = 512;
  while (chunk0 < msa::kDkdvChunkMax && 2 * chunk0 <= z.T * z.Hk / 32) chunk0 *= 2;
  size_blocks(z, msa::kBlock, msa::kHeadDim, chunk0);
  return z;
}

struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base((char*)b) {}
  template <typename T>
  T* take(size_t count) {
    T* p = base ? (T*)(base + off) : nullptr;
    off = align_up(off + count * sizeof(T));
    return p;
  }
};

PlanBufs carve_plan(Carver& c, const Sizes& z) {
  PlanBufs p;
  p.blkbase = c.take<int32_t>(z.S + 1);
  p.blk_seq = c.take<int32_t>(z.nblk_cap);
  p.seqitem = c.take<int32_t>(z.S + 1);
  p.totals = c.take<int32_t>(4);
  p.tile_order = c.take<int32_t>(z.ntiles);
  return p;
}

struct SelectWs {
  PlanBufs plan;
  u16* qfeat;
  u16* kfeat;
  float* scores;
};
SelectWs carve_select(Carver& c, const Sizes& z) {
  SelectWs w;
  w.plan = carve_plan(c, z);
  w.qfeat = c.take<u16>(z.T * z.Hk * msa::kHeadDim);
  w.kfeat = c.take<u16>(z.T * z.Hk * msa::kHeadDim);
  w.scores = c.take<float>(z.T * z.Hk * z.nbmax);
  return w;
}

struct FwdWs {
  PlanBufs plan;
  u16* kop;
  u16* vt;
};
FwdWs carve_fwd(Carver& c, const Sizes& z) {
  FwdWs w;
  w.plan = carve_plan(c, z);
  w.kop = c.take<u16>(z.nblk_cap * z.Hk * msa::kHeadDim * msa::kBlock);
  w.vt = c.take<u16>(z.nblk_cap * z.Hk * msa::kHeadDim * msa::kBlock);
  return w;
}

struct BwdWs {
  PlanBufs plan;
  u16* kop;
  u16* vop;
  float* delta;
  float* nlse;
  int32_t* item_count;
  int32_t* item_load;
  int32_t* item_order;
  float* part_dk;
  float* part_dv;
  u16* ds;  // stored dS, or null (the backward then recomputes S and dP for dQ)
};
// Whether the stored-dS buffer of a pack stays within its cap.
bool ds_fits(const Sizes& z) { return z.T * z.Hk * msa::kDsBytesPerRow <= msa::kDsBufMaxBytes; }
// with_ds: a sparse backward without the fused norm, which stores dS when it
// fits (the buffer is carved last, so the other layouts are its prefix)
BwdWs carve_bwd(Carver& c, const Sizes& z, bool with_ds) {
  BwdWs w;
  w.plan = carve_plan(c, z);
  w.kop = c.take<u16>(z.nblk_cap * z.Hk * msa::kHeadDim * msa::kBlock);
  w.vop = c.take<u16>(z.nblk_cap * z.Hk * msa::kHeadDim * msa::kBlock);
  w.delta = c.take<float>(z.T * z.Hq);
  w.nlse = c.take<float>(z.T * z.Hq);
  w.item_count = c.take<int32_t>(z.Hk * z.items_cap);
  w.item_load = c.take<int32_t>(z.Hk * z.items_cap);
  w.item_order = c.take<int32_t>(z.Hk * z.items_cap);
  w.part_dk = c.take<float>(z.Hk * z.items_cap * msa::kBlock * msa::kHeadDim);
  w.part_dv = c.take<float>(z.Hk * z.items_cap * msa::kBlock * msa::kHeadDim);
  w.ds = with_ds && ds_fits(z) ? c.take<u16>(z.T * z.Hk * (msa::kDsBytesPerRow / 2)) : nullptr;
  return w;
}

// Backward with the attention-side norm: the plain backward's workspace, the
// normalized q and k, their gradients, and the norm backward's partial rows.
struct BwdQkWs {
  BwdWs bwd;
  u16* qhat;        // [T][Hq][128] normalized q (written by the dQ kernel)
  u16* khat;        // [T][Hk][128] normalized k (written by the prep kernel)
  u16* dkhat;       // [T][Hk][128] gradient of the normalized k
  float* partial;   // weight-gradient rows: the k pass's, then one per (tile, KV head)
  float* mid;       // first-stage sums of those rows
};
int64_t qknorm_partial_rows(const Sizes& z) { return msa::kQkBwdMaxRows + z.ntiles * z.Hk; }
BwdQkWs carve_bwd_qknorm(Carver& c, const Sizes& z) {
  BwdQkWs w;
  w.bwd = carve_bwd(c, z, false);
  w.qhat = c.take<u16>(z.T * z.Hq * msa::kHeadDim);
  w.khat = c.take<u16>(z.T * z.Hk * msa::kHeadDim);
  w.dkhat = c.take<u16>(z.T * z.Hk * msa::kHeadDim);
  w.partial = c.take<float>(qknorm_partial_rows(z) * 256);
  w.mid = c.take<float>((qknorm_partial_rows(z) / 16 + 1) * 256);
  return w;
}

// The backward kernels of the wide variant on the given (normalized) q and k.
void launch_bwd_on(const Sizes& z, const BwdWs& w, const u16* q, int64_t q_st, int64_t q_sh, const u16* k,
                   int64_t k_st, int64_t k_sh, const u16* v, int64_t v_st, int64_t v_sh, const u16* o, int64_t o_st,
                   int64_t o_sh, const float* lse, const u16* dO, int64_t do_st, int64_t do_sh, const int32_t* blk_idx,
                   const int32_t* cu, float scale, bool dense, u16* dq, int64_t dq_st, int64_t dq_sh, u16* dk,
                   int64_t dk_st, int64_t dk_sh, u16* dv, int64_t dv_st, int64_t dv_sh, hipStream_t stream,
                   const msa::QkNormParams* nrm = nullptr, u16* qhat = nullptr, u16* khat = nullptr,
                   float* dwq_rows = nullptr) {
  msa::BwdArgs a;
  a.q = q; a.q_st = q_st; a.q_sh = q_sh;
  a.k = k; a.k_st = k_st; a.k_sh = k_sh;
  a.v = v; a.v_st = v_st; a.v_sh = v_sh;
  a.o = o; a.o_st = o_st; a.o_sh = o_sh;
  a.lse = lse;
  a.dO = dO; a.do_st = do_st; a.do_sh = do_sh;
  a.blk_idx = blk_idx;
  a.cu = cu;
  a.scale = scale;
  a.dense = dense;
  a.dq = dq; a.dq_st = dq_st; a.dq_sh = dq_sh;
  a.dk = dk; a.dk_st = dk_st; a.dk_sh = dk_sh;
  a.dv = dv; a.dv_st = dv_st; a.dv_sh = dv_sh;
  a.kop = w.kop;
  a.vop = w.vop;
  a.delta = w.delta;
  a.nlse = w.nlse;
  a.item_count = w.item_count;
  a.item_load = w.item_load;
  a.item_order = w.item_order;
  a.part_dk = w.part_dk;
  a.part_dv = w.part_dv;
  a.ds = w.ds;
  a.nrm = nrm;
  a.qhat = qhat;
  a.khat = khat;
  a.dwq_rows = dwq_rows;
  msa::launch_attn_bwd(z, a, w.plan, stream);
}

struct QsaFwdWs {
  PlanBufs plan;
  uint32_t* bits;
  u16* vt;
  u16* kop;
};
QsaFwdWs carve_qsa_fwd(Carver& c, const Sizes& z) {
  QsaFwdWs w;
  w.plan = carve_plan(c, z);
  w.bits = c.take<uint32_t>(z.T * z.Hk * msa::kQsaWords);
  w.vt = c.take<u16>(z.nblk_cap * z.Hk * msa::kQsaKeyTile * msa::kQsaHeadDim);
  w.kop = c.take<u16>(z.nblk_cap * z.Hk * msa::kQsaKeyTile * msa::kQsaHeadDim);
  return w;
}

struct QsaBwdWs {
  PlanBufs plan;
  uint32_t* bits;
  int64_t* dsbase;
  u16* kop;
  u16* ds;
  float* delta;
  float* nlse;
  int32_t* item_count;
  float* part_dk;
  float* part_dv;
};
// Bound on the narrow backward's dS slots: a token at position p owns p / 64 + 1
// (one per causal key tile), so a length-L sequence f(L) = sum over p < L.  f
// is convex, so over lengths <= max_seqlen M summing to T the sum is largest
// for T / M sequences of length M and one of T % M; nor does it exceed
// T * ceil(M / 64).
int64_t qsa_ds_slots(const Sizes& z) {
  const int64_t M = z.max_seqlen, T = z.T;
  if (T == 0 || M == 0) return 0;
  auto f = [](int64_t L) {
    const int64_t a = L / 64;
    return (a + 1) * (32 * a + L % 64);
  };
  const int64_t by_len = (T / M) * f(M) + f(T % M);
  const int64_t by_tok = T * ((M - 1) / 64 + 1);
  return by_len < by_tok ? by_len : by_tok;
}

QsaBwdWs carve_qsa_bwd(Carver& c, const Sizes& z) {
  QsaBwdWs w;
  w.plan = carve_plan(c, z);
  w.bits = c.take<uint32_t>(z.T * z.Hk * msa::kQsaWords);
  w.dsbase = c.take<int64_t>(z.S + 1);
  w.kop = c.take<u16>(z.nblk_cap * z.Hk * msa::kQsaKeyTile * msa::kQsaHeadDim);
  // one 128-byte dS line per (token, causal key tile, KV head, query head)
  w.ds = c.take<u16>(qsa_ds_slots(z) * z.Hk * msa::kQsaGroup * msa::kQsaKeyTile);
  w.delta = c.take<float>(z.T * z.Hk * 16);
  w.nlse = c.take<float>(z.T * z.Hk * 16);
  w.item_count = c.take<int32_t>(z.Hk * z.items_cap);
  w.part_dk = c.take<float>(z.Hk * z.items_cap * msa::kQsaKeyTile * msa::kQsaHeadDim);
  w.part_dv = c.take<float>(z.Hk * z.items_cap * msa::kQsaKeyTile * msa::kQsaHeadDim);
  return w;
}

size_t ws_bytes_for(const Sizes& z, int op) {
  Carver c(nullptr);
  switch (op) {
    case MSA_OP_SELECT: carve_select(c, z); break;
    case MSA_OP_FWD: carve_fwd(c, z); break;
    case MSA_OP_BWD: carve_bwd(c, z, true); break;
    case MSA_OP_BWD_RECOMPUTE: carve_bwd(c, z, false); break;
    case MSA_OP_QKNORM_BWD: c.take<float>((int64_t)(msa::kQkBwdMaxRows + msa::kQkBwdMaxRows / 16 + 1) * 256); break;
    case MSA_OP_QSA_FWD: carve_qsa_fwd(c, z); break;
    case MSA_OP_QSA_BWD: carve_qsa_bwd(c, z); break;
    case MSA_OP_BWD_QKNORM: carve_bwd_qknorm(c, z); break;
    default: return 0;
  }
  return c.off;
}

// A bf16 [T, H, 128] tensor view: 16-byte aligned base, non-negative strides
// that are multiples of 8 elements.  Inputs may broadcast (zero stride);
// outputs may not.
bool ok_view(const void* p, int64_t st_t, int64_t st_h, bool is_output) {
  if (!p || !aligned(p, 16)) return false;
  if (st_t < 0 || st_h < 0) return false;
  if (st_t % 8 != 0 || st_h % 8 != 0) return false;
  if (is_output && (st_t == 0 || st_h == 0)) return false;
  return true;
}
bool in_view(const void* p, int64_t st_t, int64_t st_h) { return ok_view(p, st_t, st_h, false); }
bool out_view(const void* p, int64_t st_t, int64_t st_h) { return ok_view(p, st_t, st_h, true); }

int check_ws(void* ws, size_t bytes, size_t need) {
  if (need == 0) return MSA_OK;
  if (!ws || !aligned(ws, kAlign) || bytes < need) return MSA_ERR_WORKSPACE;
  return MSA_OK;
}

int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? MSA_OK : MSA_ERR_HIP;
}

}  // namespace

extern "C" {

int msa_version(void) { return 100; }

const char* msa_status_string(int status) {
  switch (status) {
    case MSA_OK: return "MSA_OK";
    case MSA_ERR_INVALID_ARG: return "MSA_ERR_INVALID_ARG: null pointer, negative size, or bad stride/alignment";
    case MSA_ERR_UNSUPPORTED:
      return "MSA_ERR_UNSUPPORTED: needs head_dim=128, block_size=128, topk_blocks=16, num_q_heads=16*num_kv_heads, "
             "max_seqlen<=131072 (msa_qsa_*: head_dim=256, block_size=4, topk_blocks<=1024, "
             "num_q_heads=12*num_kv_heads, max_seqlen<=32768)";
    case MSA_ERR_WORKSPACE: return "MSA_ERR_WORKSPACE: workspace null, not 256-byte aligned, or too small";
    case MSA_ERR_HIP: return "MSA_ERR_HIP: the HIP runtime reported an error";
    default: return "unknown MSA status";
  }
}

int msa_workspace_size(const msa_dims* dims, int op, size_t* bytes) {
  if (!bytes) return MSA_ERR_INVALID_ARG;
  if (op == MSA_OP_QSA_FWD || op == MSA_OP_QSA_BWD) {
    int st = check_qsa_dims(dims);
    if (st != MSA_OK) return st;
    *bytes = dims->total_tokens == 0 ? 0 : ws_bytes_for(sizes_of_qsa(dims), op);
    return MSA_OK;
  }
  int st = check_dims(dims);
  if (st != MSA_OK) return st;
  if (op != MSA_OP_SELECT && op != MSA_OP_FWD && op != MSA_OP_BWD && op != MSA_OP_QKNORM_BWD &&
      op != MSA_OP_BWD_QKNORM && op != MSA_OP_BWD_RECOMPUTE)
    return MSA_ERR_INVALID_ARG;
  *bytes = dims->total_tokens == 0 ? 0 : ws_bytes_for(sizes_of(dims), op);
  return MSA_OK;
}

int msa_index_select(const msa_dims* dims, const void* idx_q, int64_t sq_t, int64_t sq_h, const void* idx_k,
                     int64_t sk_t, int64_t sk_h, const void* w_q, const void* w_k, float eps, float rope_base,
                     int32_t rope_dims, const int32_t* cu_seqlens, int32_t* blk_idx, void* workspace,
                     size_t workspace_bytes, hipStream_t stream) {
  return msa_index_select_ex(dims, idx_q, sq_t, sq_h, idx_k, sk_t, sk_h, w_q, w_k, eps, rope_base, rope_dims, 0u,
                             cu_seqlens, blk_idx, workspace, workspace_bytes, stream);
}

int msa_index_select_ex(const msa_dims* dims, const void* idx_q, int64_t sq_t, int64_t sq_h, const void* idx_k,
                        int64_t sk_t, int64_t sk_h, const void* w_q, const void* w_k, float eps, float rope_base,
                        int32_t rope_dims, uint32_t flags, const int32_t* cu_seqlens, int32_t* blk_idx,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_dims(dims);
  if (st != MSA_OK) return st;
  if (flags & ~MSA_SELECT_FORCE_INIT) return MSA_ERR_INVALID_ARG;
  if (rope_dims != 64) return MSA_ERR_UNSUPPORTED;
  if (!(eps >= 0.f) || !(rope_base > 1.f) || rope_base != rope_base) return MSA_ERR_INVALID_ARG;
  if (dims->total_tokens == 0) return MSA_OK;
  if (!in_view(idx_q, sq_t, sq_h) || !in_view(idx_k, sk_t, sk_h)) return MSA_ERR_INVALID_ARG;
  if (!w_q || !w_k || !aligned(w_q, 2) || !aligned(w_k, 2)) return MSA_ERR_INVALID_ARG;
  if (!cu_seqlens || !aligned(cu_seqlens, 4) || !blk_idx || !aligned(blk_idx, 16)) return MSA_ERR_INVALID_ARG;
  const Sizes z = sizes_of(dims);
  st = check_ws(workspace, workspace_bytes, ws_bytes_for(z, MSA_OP_SELECT));
  if (st != MSA_OK) return st;
  Carver c(workspace);
  SelectWs w = carve_select(c, z);
  msa::launch_select(z, (const u16*)idx_q, sq_t, sq_h, (const u16*)idx_k, sk_t, sk_h, (const u16*)w_q,
                     (const u16*)w_k, eps, rope_base, cu_seqlens, w.plan, (flags & MSA_SELECT_FORCE_INIT) != 0,
                     w.qfeat, w.kfeat, w.scores, blk_idx, stream);
  return launch_status();
}

int msa_attn_fwd(const msa_dims* dims, const void* q, int64_t q_st, int64_t q_sh, const void* k, int64_t k_st,
                 int64_t k_sh, const void* v, int64_t v_st, int64_t v_sh, const int32_t* blk_idx,
                 const int32_t* cu_seqlens, float softmax_scale, void* o, int64_t o_st, int64_t o_sh, float* lse,
                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return msa_attn_fwd_ex(dims, q, q_st, q_sh, k, k_st, k_sh, v, v_st, v_sh, blk_idx, cu_seqlens, softmax_scale, 0u,
                         o, o_st, o_sh, lse, workspace, workspace_bytes, stream);
}

int msa_attn_fwd_ex(const msa_dims* dims, const void* q, int64_t q_st, int64_t q_sh, const void* k, int64_t k_st,
                    int64_t k_sh, const void* v, int64_t v_st, int64_t v_sh, const int32_t* blk_idx,
                    const int32_t* cu_seqlens, float softmax_scale, uint32_t flags, void* o, int64_t o_st,
                    int64_t o_sh, float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_dims(dims);
  if (st != MSA_OK) return st;
  if (flags & ~MSA_ATTN_DENSE) return MSA_ERR_INVALID_ARG;
  const bool dense = (flags & MSA_ATTN_DENSE) != 0;
  if (!(softmax_scale > 0.f) || softmax_scale == INFINITY) return MSA_ERR_INVALID_ARG;
  if (dims->total_tokens == 0) return MSA_OK;
  if (!in_view(q, q_st, q_sh) || !in_view(k, k_st, k_sh) || !in_view(v, v_st, v_sh) || !out_view(o, o_st, o_sh))
    return MSA_ERR_INVALID_ARG;
  if ((!dense && (!blk_idx || !aligned(blk_idx, 16))) || !cu_seqlens || !aligned(cu_seqlens, 4) || !lse ||
      !aligned(lse, 16))
    return MSA_ERR_INVALID_ARG;
  const Sizes z = sizes_of(dims);
  st = check_ws(workspace, workspace_bytes, ws_bytes_for(z, MSA_OP_FWD));
  if (st != MSA_OK) return st;
  Carver c(workspace);
  FwdWs w = carve_fwd(c, z);
  msa::launch_block_prep(z, (const u16*)k, k_st, k_sh, (const u16*)v, v_st, v_sh, cu_seqlens, w.plan, nullptr,
                         dense, w.kop, w.vt, stream);
  msa::launch_attn_fwd(z, (const u16*)q, q_st, q_sh, w.kop, w.vt, dense ? nullptr : blk_idx,
                       cu_seqlens, w.plan, softmax_scale, (u16*)o, o_st, o_sh, lse, dense, nullptr, stream);
  return launch_status();
}

int msa_attn_bwd(const msa_dims* dims, const void* q, int64_t q_st, int64_t q_sh, const void* k, int64_t k_st,
                 int64_t k_sh, const void* v, int64_t v_st, int64_t v_sh, const void* o, int64_t o_st, int64_t o_sh,
                 const float* lse, const void* do_, int64_t do_st, int64_t do_sh, const int32_t* blk_idx,
                 const int32_t* cu_seqlens, float softmax_scale, void* dq, int64_t dq_st, int64_t dq_sh, void* dk,
                 int64_t dk_st, int64_t dk_sh, void* dv, int64_t dv_st, int64_t dv_sh, void* workspace,
                 size_t workspace_bytes, hipStream_t stream) {
  return msa_attn_bwd_ex(dims, q, q_st, q_sh, k, k_st, k_sh, v, v_st, v_sh, o, o_st, o_sh, lse, do_, do_st, do_sh,
                         blk_idx, cu_seqlens, softmax_scale, 0u, dq, dq_st, dq_sh, dk, dk_st, dk_sh, dv, dv_st, dv_sh,
                         workspace, workspace_bytes, stream);
}

int msa_attn_bwd_ex(const msa_dims* dims, const void* q, int64_t q_st, int64_t q_sh, const void* k, int64_t k_st,
                    int64_t k_sh, const void* v, int64_t v_st, int64_t v_sh, const void* o, int64_t o_st,
                    int64_t o_sh, const float* lse, const void* do_, int64_t do_st, int64_t do_sh,
                    const int32_t* blk_idx, const int32_t* cu_seqlens, float softmax_scale, uint32_t flags, void* dq,
                    int64_t dq_st, int64_t dq_sh, void* dk, int64_t dk_st, int64_t dk_sh, void* dv, int64_t dv_st,
                    int64_t dv_sh, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_dims(dims);
  if (st != MSA_OK) return st;
  if (flags & ~(MSA_ATTN_DENSE | MSA_ATTN_RECOMPUTE)) return MSA_ERR_INVALID_ARG;
  const bool dense = (flags & MSA_ATTN_DENSE) != 0;
  // the stored-dS pipeline, unless dense or asked to recompute
  const bool store_ds = !dense && !(flags & MSA_ATTN_RECOMPUTE);
  if (!(softmax_scale > 0.f) || softmax_scale == INFINITY) return MSA_ERR_INVALID_ARG;
  if (dims->total_tokens == 0) return MSA_OK;
  if (!in_view(q, q_st, q_sh) || !in_view(k, k_st, k_sh) || !in_view(v, v_st, v_sh) || !in_view(o, o_st, o_sh) ||
      !in_view(do_, do_st, do_sh) || !out_view(dq, dq_st, dq_sh) || !out_view(dk, dk_st, dk_sh) ||
      !out_view(dv, dv_st, dv_sh))
    return MSA_ERR_INVALID_ARG;
  if ((!dense && (!blk_idx || !aligned(blk_idx, 16))) || !cu_seqlens || !aligned(cu_seqlens, 4) || !lse ||
      !aligned(lse, 16))
    return MSA_ERR_INVALID_ARG;
  const Sizes z = sizes_of(dims);
  st = check_ws(workspace, workspace_bytes, ws_bytes_for(z, store_ds ? MSA_OP_BWD : MSA_OP_BWD_RECOMPUTE));
  if (st != MSA_OK) return st;
  Carver c(workspace);
  BwdWs w = carve_bwd(c, z, store_ds);
  launch_bwd_on(z, w, (const u16*)q, q_st, q_sh, (const u16*)k, k_st, k_sh, (const u16*)v, v_st, v_sh,
                (const u16*)o, o_st, o_sh, lse, (const u16*)do_, do_st, do_sh, dense ? nullptr : blk_idx,
                cu_seqlens, softmax_scale, dense, (u16*)dq, dq_st, dq_sh, (u16*)dk, dk_st, dk_sh, (u16*)dv, dv_st,
                dv_sh, stream);
  return launch_status();
}

int msa_attn_fwd_qknorm(const msa_dims* dims, const void* q, int64_t q_st, int64_t q_sh, const void* k,
                        int64_t k_st, int64_t k_sh, const void* v, int64_t v_st, int64_t v_sh, const void* w_q,
                        const void* w_k, float eps, float rope_base, int32_t rope_dims, const int32_t* blk_idx,
                        const int32_t* cu_seqlens, float softmax_scale, uint32_t flags, void* o, int64_t o_st,
                        int64_t o_sh, float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_dims(dims);
  if (st != MSA_OK) return st;
  if (flags & ~MSA_ATTN_DENSE) return MSA_ERR_INVALID_ARG;
  const bool dense = (flags & MSA_ATTN_DENSE) != 0;
  if (rope_dims != 64) return MSA_ERR_UNSUPPORTED;
  if (!(eps >= 0.f) || !(rope_base > 1.f) || rope_base != rope_base) return MSA_ERR_INVALID_ARG;
  if (!(softmax_scale > 0.f) || softmax_scale == INFINITY) return MSA_ERR_INVALID_ARG;
  if (dims->total_tokens == 0) return MSA_OK;
  if (!in_view(q, q_st, q_sh) || !in_view(k, k_st, k_sh) || !in_view(v, v_st, v_sh) || !out_view(o, o_st, o_sh))
    return MSA_ERR_INVALID_ARG;
  if (!w_q || !w_k || !aligned(w_q, 2) || !aligned(w_k, 2)) return MSA_ERR_INVALID_ARG;
  if ((!dense && (!blk_idx || !aligned(blk_idx, 16))) || !cu_seqlens || !aligned(cu_seqlens, 4) || !lse ||
      !aligned(lse, 16))
    return MSA_ERR_INVALID_ARG;
  const Sizes z = sizes_of(dims);
  st = check_ws(workspace, workspace_bytes, ws_bytes_for(z, MSA_OP_FWD));
  if (st != MSA_OK) return st;
  Carver c(workspace);
  FwdWs w = carve_fwd(c, z);
  const msa::QkNormParams nrm{(const u16*)w_q, (const u16*)w_k, eps, msa::rope_freqs(rope_base)};
  msa::launch_block_prep(z, (const u16*)k, k_st, k_sh, (const u16*)v, v_st, v_sh, cu_seqlens, w.plan, &nrm, dense,
                         w.kop, w.vt, stream);
  msa::launch_attn_fwd(z, (const u16*)q, q_st, q_sh, w.kop, w.vt, dense ? nullptr : blk_idx, cu_seqlens, w.plan,
                       softmax_scale, (u16*)o, o_st, o_sh, lse, dense, &nrm, stream);
  return launch_status();
}

int msa_attn_bwd_qknorm(const msa_dims* dims, const void* q, int64_t q_st, int64_t q_sh, const void* k,
                        int64_t k_st, int64_t k_sh, const void* v, int64_t v_st, int64_t v_sh, const void* w_q,
                        const void* w_k, float eps, float rope_base, int32_t rope_dims, const void* o, int64_t o_st,
                        int64_t o_sh, const float* lse, const void* do_, int64_t do_st, int64_t do_sh,
                        const int32_t* blk_idx, const int32_t* cu_seqlens, float softmax_scale, uint32_t flags,
                        void* dq, int64_t dq_st, int64_t dq_sh, void* dk, int64_t dk_st, int64_t dk_sh, void* dv,
                        int64_t dv_st, int64_t dv_sh, float* dw_q, float* dw_k, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  int st = check_dims(dims);
  if (st != MSA_OK) return st;
  if (flags & ~MSA_ATTN_DENSE) return MSA_ERR_INVALID_ARG;
  const bool dense = (flags & MSA_ATTN_DENSE) != 0;
  if (rope_dims != 64) return MSA_ERR_UNSUPPORTED;
  if (!(eps >= 0.f) || !(rope_base > 1.f) || rope_base != rope_base) return MSA_ERR_INVALID_ARG;
  if (!(softmax_scale > 0.f) || softmax_scale == INFINITY) return MSA_ERR_INVALID_ARG;
  if (!dw_q || !dw_k || !aligned(dw_q, 4) || !aligned(dw_k, 4)) return MSA_ERR_INVALID_ARG;
  if (dims->total_tokens == 0) {  // no rows: the weight gradients are zero
    msa::QkNormArgs a{};
    a.dw_q = dw_q;
    a.dw_k = dw_k;
    msa::launch_qk_norm_bwd(sizes_of(dims), a, nullptr, stream);
    return launch_status();
  }
  if (!in_view(q, q_st, q_sh) || !in_view(k, k_st, k_sh) || !in_view(v, v_st, v_sh) || !in_view(o, o_st, o_sh) ||
      !in_view(do_, do_st, do_sh) || !out_view(dq, dq_st, dq_sh) || !out_view(dk, dk_st, dk_sh) ||
      !out_view(dv, dv_st, dv_sh))
    return MSA_ERR_INVALID_ARG;
  if (!w_q || !w_k || !aligned(w_q, 2) || !aligned(w_k, 2)) return MSA_ERR_INVALID_ARG;
  if ((!dense && (!blk_idx || !aligned(blk_idx, 16))) || !cu_seqlens || !aligned(cu_seqlens, 4) || !lse ||
      !aligned(lse, 16))
    return MSA_ERR_INVALID_ARG;
  const Sizes z = sizes_of(dims);
  st = check_ws(workspace, workspace_bytes, ws_bytes_for(z, MSA_OP_BWD_QKNORM));
  if (st != MSA_OK) return st;
  Carver c(workspace);
  BwdQkWs w = carve_bwd_qknorm(c, z);
  const int64_t D = msa::kHeadDim;
  // the backward with the norm fused into its prep and dQ kernels (dq comes
  // out for the raw q, dk for the normalized k), then the norm's backward over
  // the k rows and the weight-gradient sums
  const msa::QkNormParams nrm{(const u16*)w_q, (const u16*)w_k, eps, msa::rope_freqs(rope_base)};
  const int rows_k = msa::qk_norm_bwd_rows(z.T);
  launch_bwd_on(z, w.bwd, (const u16*)q, q_st, q_sh, (const u16*)k, k_st, k_sh, (const u16*)v, v_st, v_sh,
                (const u16*)o, o_st, o_sh, lse, (const u16*)do_, do_st, do_sh, dense ? nullptr : blk_idx, cu_seqlens,
                softmax_scale, dense, (u16*)dq, dq_st, dq_sh, w.dkhat, z.Hk * D, D, (u16*)dv, dv_st, dv_sh, stream,
                &nrm, w.qhat, w.khat, w.partial + (int64_t)rows_k * 256);
  msa::QkNormArgs a{};
  a.k = (const u16*)k; a.k_st = k_st; a.k_sh = k_sh;
  a.w_q = (const u16*)w_q; a.w_k = (const u16*)w_k;
  a.eps = eps; a.rope_base = rope_base;
  a.cu = cu_seqlens;
  a.dkh = w.dkhat; a.dkh_st = z.Hk * D; a.dkh_sh = D;
  a.ko = (u16*)dk; a.ko_st = dk_st; a.ko_sh = dk_sh;
  a.dw_q = dw_q; a.dw_k = dw_k;
  msa::launch_qk_norm_bwd_k(z, a, w.partial, (int)(z.ntiles * z.Hk), w.mid, stream);
  return launch_status();
}

int msa_qsa_attn_fwd(const msa_dims* dims, const void* q, int64_t q_st, int64_t q_sh, const void* k, int64_t k_st,
                     int64_t k_sh, const void* v, int64_t v_st, int64_t v_sh, const int32_t* blk_idx,
                     const int32_t* cu_seqlens, float softmax_scale, void* o, int64_t o_st, int64_t o_sh, float* lse,
                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_qsa_dims(dims);
  if (st != MSA_OK) return st;
  if (!(softmax_scale > 0.f) || softmax_scale == INFINITY) return MSA_ERR_INVALID_ARG;
  if (dims->total_tokens == 0) return MSA_OK;
  if (!in_view(q, q_st, q_sh) || !in_view(k, k_st, k_sh) || !in_view(v, v_st, v_sh) || !out_view(o, o_st, o_sh))
    return MSA_ERR_INVALID_ARG;
  if (!blk_idx || !aligned(blk_idx, 4) || !cu_seqlens || !aligned(cu_seqlens, 4) || !lse || !aligned(lse, 16))
    return MSA_ERR_INVALID_ARG;
  const Sizes z = sizes_of_qsa(dims);
  st = check_ws(workspace, workspace_bytes, ws_bytes_for(z, MSA_OP_QSA_FWD));
  if (st != MSA_OK) return st;
  Carver c(workspace);
  QsaFwdWs w = carve_qsa_fwd(c, z);
  msa::QsaArgs a = {};
  a.q = (const u16*)q; a.q_st = q_st; a.q_sh = q_sh;
  a.k = (const u16*)k; a.k_st = k_st; a.k_sh = k_sh;
  a.v = (const u16*)v; a.v_st = v_st; a.v_sh = v_sh;
  a.blk_idx = blk_idx;
  a.topk = dims->topk_blocks;
  a.cu = cu_seqlens;
  a.scale = softmax_scale;
  a.out_o = (u16*)o; a.oo_st = o_st; a.oo_sh = o_sh;
  a.out_lse = lse;
  a.bits = w.bits;
  a.vt = w.vt;
  a.kop = w.kop;
  msa::launch_qsa_fwd(z, a, w.plan, stream);
  return launch_status();
}

int msa_qsa_attn_bwd(const msa_dims* dims, const void* q, int64_t q_st, int64_t q_sh, const void* k, int64_t k_st,
                     int64_t k_sh, const void* v, int64_t v_st, int64_t v_sh, const void* o, int64_t o_st,
                     int64_t o_sh, const float* lse, const void* do_, int64_t do_st, int64_t do_sh,
                     const int32_t* blk_idx, const int32_t* cu_seqlens, float softmax_scale, void* dq, int64_t dq_st,
                     int64_t dq_sh, void* dk, int64_t dk_st, int64_t dk_sh, void* dv, int64_t dv_st, int64_t dv_sh,
                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_qsa_dims(dims);
  if (st != MSA_OK) return st;
  if (!(softmax_scale > 0.f) || softmax_scale == INFINITY) return MSA_ERR_INVALID_ARG;
  if (dims->total_tokens == 0) return MSA_OK;
  if (!in_view(q, q_st, q_sh) || !in_view(k, k_st, k_sh) || !in_view(v, v_st, v_sh) || !in_view(o, o_st, o_sh) ||
      !in_view(do_, do_st, do_sh) || !out_view(dq, dq_st, dq_sh) || !out_view(dk, dk_st, dk_sh) ||
      !out_view(dv, dv_st, dv_sh))
    return MSA_ERR_INVALID_ARG;
  if (!blk_idx || !aligned(blk_idx, 4) || !cu_seqlens || !aligned(cu_seqlens, 4) || !lse || !aligned(lse, 16))
    return MSA_ERR_INVALID_ARG;
  const Sizes z = sizes_of_qsa(dims);
  st = check_ws(workspace, workspace_bytes, ws_bytes_for(z, MSA_OP_QSA_BWD));
  if (st != MSA_OK) return st;
  Carver c(workspace);
  QsaBwdWs w = carve_qsa_bwd(c, z);
  msa::QsaArgs a = {};
  a.q = (const u16*)q; a.q_st = q_st; a.q_sh = q_sh;
  a.k = (const u16*)k; a.k_st = k_st; a.k_sh = k_sh;
  a.v = (const u16*)v; a.v_st = v_st; a.v_sh = v_sh;
  a.o = (const u16*)o; a.o_st = o_st; a.o_sh = o_sh;
  a.lse = lse;
  a.dO = (const u16*)do_; a.do_st = do_st; a.do_sh = do_sh;
  a.blk_idx = blk_idx;
  a.topk = dims->topk_blocks;
  a.cu = cu_seqlens;
  a.scale = softmax_scale;
  a.dq = (u16*)dq; a.dq_st = dq_st; a.dq_sh = dq_sh;
  a.dk = (u16*)dk; a.dk_st = dk_st; a.dk_sh = dk_sh;
  a.dv = (u16*)dv; a.dv_st = dv_st; a.dv_sh = dv_sh;
  a.bits = w.bits;
  a.dsbase = w.dsbase;
  a.kop = w.kop;
  a.ds = w.ds;
  a.delta = w.delta;
  a.nlse = w.nlse;
  a.item_count = w.item_count;
  a.part_dk = w.part_dk;
  a.part_dv = w.part_dv;
  msa::launch_qsa_bwd(z, a, w.plan, stream);
  return launch_status();
}

int msa_qk_norm_rope_fwd(const msa_dims* dims, const void* q, int64_t q_st, int64_t q_sh, const void* k,
                         int64_t k_st, int64_t k_sh, const void* w_q, const void* w_k, float eps, float rope_base,
                         int32_t rope_dims, const int32_t* cu_seqlens, void* q_out, int64_t qo_st, int64_t qo_sh,
                         void* k_out, int64_t ko_st, int64_t ko_sh, hipStream_t stream) {
  int st = check_dims(dims);
  if (st != MSA_OK) return st;
  if (rope_dims != 64) return MSA_ERR_UNSUPPORTED;
  if (!(eps >= 0.f) || !(rope_base > 1.f) || rope_base != rope_base) return MSA_ERR_INVALID_ARG;
  if (dims->total_tokens == 0) return MSA_OK;
  if (!in_view(q, q_st, q_sh) || !in_view(k, k_st, k_sh) || !out_view(q_out, qo_st, qo_sh) ||
      !out_view(k_out, ko_st, ko_sh))
    return MSA_ERR_INVALID_ARG;
  if (!w_q || !w_k || !aligned(w_q, 2) || !aligned(w_k, 2) || !cu_seqlens || !aligned(cu_seqlens, 4))
    return MSA_ERR_INVALID_ARG;
  const Sizes z = sizes_of(dims);
  msa::QkNormArgs a{};
  a.q = (const u16*)q; a.q_st = q_st; a.q_sh = q_sh;
  a.k = (const u16*)k; a.k_st = k_st; a.k_sh = k_sh;
  a.w_q = (const u16*)w_q; a.w_k = (const u16*)w_k;
  a.eps = eps; a.rope_base = rope_base;
  a.cu = cu_seqlens;
  a.qo = (u16*)q_out; a.qo_st = qo_st; a.qo_sh = qo_sh;
  a.ko = (u16*)k_out; a.ko_st = ko_st; a.ko_sh = ko_sh;
  msa::launch_qk_norm_fwd(z, a, stream);
  return launch_status();
}

int msa_qk_norm_rope_bwd(const msa_dims* dims, const void* q, int64_t q_st, int64_t q_sh, const void* k,
                         int64_t k_st, int64_t k_sh, const void* w_q, const void* w_k, float eps, float rope_base,
                         int32_t rope_dims, const int32_t* cu_seqlens, const void* dq_hat, int64_t dqh_st,
                         int64_t dqh_sh, const void* dk_hat, int64_t dkh_st, int64_t dkh_sh, void* dq, int64_t dq_st,
                         int64_t dq_sh, void* dk, int64_t dk_st, int64_t dk_sh, float* dw_q, float* dw_k,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_dims(dims);
  if (st != MSA_OK) return st;
  if (rope_dims != 64) return MSA_ERR_UNSUPPORTED;
  if (!(eps >= 0.f) || !(rope_base > 1.f) || rope_base != rope_base) return MSA_ERR_INVALID_ARG;
  if (!dw_q || !dw_k || !aligned(dw_q, 4) || !aligned(dw_k, 4)) return MSA_ERR_INVALID_ARG;
  if (dims->total_tokens == 0) {  // no rows: the weight gradients are zero
    msa::QkNormArgs a{};
    a.dw_q = dw_q;
    a.dw_k = dw_k;
    msa::launch_qk_norm_bwd(sizes_of(dims), a, nullptr, stream);
    return launch_status();
  }
  if (!in_view(q, q_st, q_sh) || !in_view(k, k_st, k_sh) || !in_view(dq_hat, dqh_st, dqh_sh) ||
      !in_view(dk_hat, dkh_st, dkh_sh) || !out_view(dq, dq_st, dq_sh) || !out_view(dk, dk_st, dk_sh))
    return MSA_ERR_INVALID_ARG;
  if (!w_q || !w_k || !aligned(w_q, 2) || !aligned(w_k, 2) || !cu_seqlens || !aligned(cu_seqlens, 4))
    return MSA_ERR_INVALID_ARG;
  const Sizes z = sizes_of(dims);
  st = check_ws(workspace, workspace_bytes, ws_bytes_for(z, MSA_OP_QKNORM_BWD));
  if (st != MSA_OK) return st;
  msa::QkNormArgs a{};
  a.q = (const u16*)q; a.q_st = q_st; a.q_sh = q_sh;
  a.k = (const u16*)k; a.k_st = k_st; a.k_sh = k_sh;
  a.w_q = (const u16*)w_q; a.w_k = (const u16*)w_k;
  a.eps = eps; a.rope_base = rope_base;
  a.cu = cu_seqlens;
  a.dqh = (const u16*)dq_hat; a.dqh_st = dqh_st; a.dqh_sh = dqh_sh;
  a.dkh = (const u16*)dk_hat; a.dkh_st = dkh_st; a.dkh_sh = dkh_sh;
  a.qo = (u16*)dq; a.qo_st = dq_st; a.qo_sh = dq_sh;
  a.ko = (u16*)dk; a.ko_st = dk_st; a.ko_sh = dk_sh;
  a.dw_q = dw_q; a.dw_k = dw_k;
  msa::launch_qk_norm_bwd(z, a, (float*)workspace, stream);
  return launch_status();
}

int msa_check_cu_seqlens(const msa_dims* dims, const int32_t* cu_seqlens, hipStream_t stream) {
  int st = check_dims(dims);
  if (st != MSA_OK) return st;
  if (!cu_seqlens) return MSA_ERR_INVALID_ARG;
  const int S = dims->num_seqs;
  std::vector<int32_t> h((size_t)S + 1);
  if (hipMemcpyAsync(h.data(), cu_seqlens, sizeof(int32_t) * h.size(), hipMemcpyDeviceToHost, stream) != hipSuccess)
    return MSA_ERR_HIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return MSA_ERR_HIP;
  if (h[0] != 0 || h[S] != dims->total_tokens) return MSA_ERR_INVALID_ARG;
  for (int s = 0; s < S; ++s) {
    const int64_t len = (int64_t)h[s + 1] - h[s];
    if (len < 0 || len > dims->max_seqlen) return MSA_ERR_INVALID_ARG;
  }
  return MSA_OK;
}

}  // extern "C"
