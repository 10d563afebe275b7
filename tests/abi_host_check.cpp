// Host-side check of the C ABI, built against the address- and
// undefined-behaviour-sanitized build of the library (no GPU needed): every
// call below must return its status before anything is launched, so the
// device pointers are made-up, aligned addresses that are never dereferenced.
// Exits non-zero on the first unexpected status (or when a sanitizer fires).
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "msa.h"

static int failures = 0;

#define EXPECT(call, want)                                                                    \
  do {                                                                                        \
    const int got_ = (call);                                                                  \
    if (got_ != (want)) {                                                                     \
      fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #call, got_, (want)); \
      ++failures;                                                                             \
    }                                                                                         \
  } while (0)

static msa_dims dims(int T, int S, int L, int hq, int hk, int d = 128, int blk = 128, int topk = 16) {
  msa_dims x;
  x.total_tokens = T;
  x.num_seqs = S;
  x.max_seqlen = L;
  x.num_q_heads = hq;
  x.num_kv_heads = hk;
  x.head_dim = d;
  x.block_size = blk;
  x.topk_blocks = topk;
  return x;
}

static void* const F = (void*)0x7F0000000000ull;  // 256-byte aligned, never dereferenced
static void* off(size_t b) { return (char*)F + b; }
static const size_t BIG = (size_t)1 << 40;

int main() {
  const msa_dims d = dims(16384, 3, 7122, 16, 1);
  size_t n = 0;

  // workspace sizes and dims validation
  for (int op = MSA_OP_SELECT; op <= MSA_OP_BWD_RECOMPUTE; ++op) {
    if (op == MSA_OP_QSA_FWD || op == MSA_OP_QSA_BWD) continue;
    EXPECT(msa_workspace_size(&d, op, &n), MSA_OK);
    if (n == 0 || n % 256) {
      fprintf(stderr, "op %d: workspace %zu\n", op, n);
      ++failures;
    }
  }
  EXPECT(msa_workspace_size(&d, 99, &n), MSA_ERR_INVALID_ARG);
  EXPECT(msa_workspace_size(nullptr, MSA_OP_FWD, &n), MSA_ERR_INVALID_ARG);
  msa_dims bad = dims(16384, 3, 7122, 16, 1, 64);
  EXPECT(msa_workspace_size(&bad, MSA_OP_FWD, &n), MSA_ERR_UNSUPPORTED);
  bad = dims(16384, 3, 7122, 32, 1);
  EXPECT(msa_workspace_size(&bad, MSA_OP_FWD, &n), MSA_ERR_UNSUPPORTED);
  bad = dims(-1, 3, 7122, 16, 1);
  EXPECT(msa_workspace_size(&bad, MSA_OP_FWD, &n), MSA_ERR_INVALID_ARG);
  bad = dims(16384, 3, 20000, 16, 1);
  EXPECT(msa_workspace_size(&bad, MSA_OP_FWD, &n), MSA_ERR_INVALID_ARG);
  bad = dims(300000, 1, 200000, 16, 1);
  EXPECT(msa_workspace_size(&bad, MSA_OP_FWD, &n), MSA_ERR_UNSUPPORTED);
  const msa_dims empty = dims(0, 0, 0, 16, 1);
  EXPECT(msa_workspace_size(&empty, MSA_OP_BWD, &n), MSA_OK);
  const msa_dims layer = dims(32768, 1, 32768, 64, 4);
  EXPECT(msa_workspace_size(&layer, MSA_OP_BWD, &n), MSA_OK);
  const msa_dims qsa = dims(16384, 3, 7122, 12, 1, 256, 4, 512);
  EXPECT(msa_workspace_size(&qsa, MSA_OP_QSA_BWD, &n), MSA_OK);
  EXPECT(msa_workspace_size(&qsa, MSA_OP_FWD, &n), MSA_ERR_UNSUPPORTED);

  // forward
  size_t need_fwd = 0;
  msa_workspace_size(&d, MSA_OP_FWD, &need_fwd);
  auto fwd = [&](const void* q, int64_t q_st, const int32_t* blk, float scale, void* o_, int64_t o_sh, float* lse,
                 void* ws, size_t nb, const msa_dims* dd) {
    return msa_attn_fwd(dd, q, q_st, 128, F, 128, 128, F, 128, 128, blk, (const int32_t*)F, scale, o_, 2048, o_sh,
                        lse, ws, nb, nullptr);
  };
  const int32_t* B = (const int32_t*)F;
  float* Lp = (float*)F;
  EXPECT(fwd(nullptr, 2048, B, 0.088f, F, 128, Lp, F, BIG, &d), MSA_ERR_INVALID_ARG);
  EXPECT(fwd(off(2), 2048, B, 0.088f, F, 128, Lp, F, BIG, &d), MSA_ERR_INVALID_ARG);
  EXPECT(fwd(F, 2047, B, 0.088f, F, 128, Lp, F, BIG, &d), MSA_ERR_INVALID_ARG);
  EXPECT(fwd(F, 2048, B, 0.088f, F, 0, Lp, F, BIG, &d), MSA_ERR_INVALID_ARG);
  EXPECT(fwd(F, 2048, nullptr, 0.088f, F, 128, Lp, F, BIG, &d), MSA_ERR_INVALID_ARG);
  EXPECT(fwd(F, 2048, B, 0.088f, F, 128, (float*)off(4), F, BIG, &d), MSA_ERR_INVALID_ARG);
  EXPECT(fwd(F, 2048, B, 0.0f, F, 128, Lp, F, BIG, &d), MSA_ERR_INVALID_ARG);
  EXPECT(fwd(F, 2048, B, NAN, F, 128, Lp, F, BIG, &d), MSA_ERR_INVALID_ARG);
  EXPECT(fwd(F, 2048, B, 0.088f, F, 128, Lp, nullptr, BIG, &d), MSA_ERR_WORKSPACE);
  EXPECT(fwd(F, 2048, B, 0.088f, F, 128, Lp, off(16), BIG, &d), MSA_ERR_WORKSPACE);
  EXPECT(fwd(F, 2048, B, 0.088f, F, 128, Lp, F, need_fwd - 1, &d), MSA_ERR_WORKSPACE);
  EXPECT(fwd(nullptr, 2048, B, 0.088f, F, 128, Lp, nullptr, 0, &empty), MSA_OK);
  EXPECT(msa_attn_fwd_ex(&d, F, 2048, 128, F, 128, 128, F, 128, 128, B, B, 0.088f, 2u, F, 2048, 128, Lp, F, BIG,
                         nullptr),
         MSA_ERR_INVALID_ARG);

  // the allocation-free forward rejects a pack beyond its static scratch before anything else
  const msa_dims huge = dims(131072, 1, 131072, 32, 2);
  EXPECT(msa_attn_fwd_noalloc(&huge, nullptr, 0, 0, nullptr, 0, 0, nullptr, 0, 0, nullptr, nullptr, 0.1f, nullptr,
                              0, 0, nullptr, nullptr),
         MSA_ERR_WORKSPACE);

  // selection
  auto sel = [&](const void* iq, float base, int rope, int32_t* blk, void* ws, size_t nb, uint32_t flags,
                 const msa_dims* dd) {
    return msa_index_select_ex(dd, iq, 128, 128, F, 128, 128, F, F, 1e-6f, base, rope, flags, B, blk, ws, nb,
                               nullptr);
  };
  int32_t* Bo = (int32_t*)F;
  EXPECT(sel(F, 1e7f, 32, Bo, F, BIG, 0, &d), MSA_ERR_UNSUPPORTED);
  EXPECT(sel(F, 1.0f, 64, Bo, F, BIG, 0, &d), MSA_ERR_INVALID_ARG);
  EXPECT(sel(nullptr, 1e7f, 64, Bo, F, BIG, 0, &d), MSA_ERR_INVALID_ARG);
  EXPECT(sel(F, 1e7f, 64, (int32_t*)off(4), F, BIG, 0, &d), MSA_ERR_INVALID_ARG);
  EXPECT(sel(F, 1e7f, 64, Bo, F, 0, 0, &d), MSA_ERR_WORKSPACE);
  EXPECT(sel(F, 1e7f, 64, Bo, F, BIG, 2u, &d), MSA_ERR_INVALID_ARG);
  EXPECT(sel(F, 1e7f, 64, Bo, F, 0, MSA_SELECT_FORCE_INIT, &d), MSA_ERR_WORKSPACE);
  EXPECT(sel(nullptr, 1e7f, 64, Bo, nullptr, 0, 0, &empty), MSA_OK);

  // backward
  size_t need_bwd = 0;
  msa_workspace_size(&d, MSA_OP_BWD, &need_bwd);
  auto bwd = [&](int64_t dv_sh, const float* lse, size_t nb) {
    return msa_attn_bwd(&d, F, 2048, 128, F, 128, 128, F, 128, 128, F, 2048, 128, lse, F, 2048, 128, B, B, 0.088f,
                        F, 2048, 128, F, 128, 128, F, 128, dv_sh, F, nb, nullptr);
  };
  EXPECT(bwd(0, Lp, BIG), MSA_ERR_INVALID_ARG);
  EXPECT(bwd(128, nullptr, BIG), MSA_ERR_INVALID_ARG);
  EXPECT(bwd(128, Lp, need_bwd - 256), MSA_ERR_WORKSPACE);

  // the recompute flag: a smaller workspace (no stored-dS tail); unknown bits rejected
  size_t need_rc = 0;
  EXPECT(msa_workspace_size(&d, MSA_OP_BWD_RECOMPUTE, &need_rc), MSA_OK);
  if (!(need_rc > 0 && need_rc + (size_t)16384 * 65536 == need_bwd)) {
    fprintf(stderr, "recompute workspace %zu, stored-dS workspace %zu\n", need_rc, need_bwd);
    ++failures;
  }
  auto bwdx = [&](uint32_t flags, size_t nb) {
    return msa_attn_bwd_ex(&d, F, 2048, 128, F, 128, 128, F, 128, 128, F, 2048, 128, Lp, F, 2048, 128, B, B, 0.088f,
                           flags, F, 2048, 128, F, 128, 128, F, 128, 128, F, nb, nullptr);
  };
  EXPECT(bwdx(4u, BIG), MSA_ERR_INVALID_ARG);
  EXPECT(bwdx(MSA_ATTN_RECOMPUTE, need_rc - 256), MSA_ERR_WORKSPACE);
  EXPECT(bwdx(MSA_ATTN_DENSE, need_rc - 256), MSA_ERR_WORKSPACE);
  EXPECT(bwdx(0u, need_rc), MSA_ERR_WORKSPACE);

  // attention-side q/k norm
  EXPECT(msa_qk_norm_rope_fwd(&d, F, 2048, 128, F, 128, 128, F, F, 1e-6f, 1e7f, 32, B, F, 2048, 128, F, 128, 128,
                              nullptr),
         MSA_ERR_UNSUPPORTED);
  EXPECT(msa_qk_norm_rope_fwd(&d, F, 2048, 128, F, 128, 128, F, F, 1e-6f, 1e7f, 64, B, F, 2048, 0, F, 128, 128,
                              nullptr),
         MSA_ERR_INVALID_ARG);

  // narrow-block variant
  size_t need_q = 0;
  msa_workspace_size(&qsa, MSA_OP_QSA_FWD, &need_q);
  EXPECT(msa_qsa_attn_fwd(&qsa, nullptr, 3072, 256, F, 256, 256, F, 256, 256, B, B, 0.0625f, F, 3072, 256, Lp, F,
                          BIG, nullptr),
         MSA_ERR_INVALID_ARG);
  EXPECT(msa_qsa_attn_fwd(&qsa, F, 3072, 256, F, 256, 256, F, 256, 256, B, B, 0.0625f, F, 3072, 256, Lp, F,
                          need_q - 256, nullptr),
         MSA_ERR_WORKSPACE);
  EXPECT(msa_qsa_attn_fwd(&d, F, 3072, 256, F, 256, 256, F, 256, 256, B, B, 0.0625f, F, 3072, 256, Lp, F, BIG,
                          nullptr),
         MSA_ERR_UNSUPPORTED);

  // status strings and version
  for (int st = -4; st <= 0; ++st)
    if (strncmp(msa_status_string(st), "MSA_", 4) != 0) {
      fprintf(stderr, "status %d: %s\n", st, msa_status_string(st));
      ++failures;
    }
  if (!strstr(msa_status_string(7), "unknown")) ++failures;
  if (msa_version() < 100) ++failures;

  if (failures) {
    fprintf(stderr, "%d unexpected results\n", failures);
    return 1;
  }
  printf("abi host check: all statuses as expected\n");
  return 0;
}
