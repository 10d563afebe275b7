/*
 * msa.h -- C ABI of the MSA block-sparse attention hot path on AMD Instinct
 * MI355X (gfx950): the frozen lightning-indexer block selection and the GQA
 * block-sparse flash attention forward and backward over the selected blocks.
 *
 * What the operations compute is stated on these pages:
 *   [M31] miles docs, "MiniMax-M3.1-Flash", section 1 Model Introduction and
 *         section 5 Recipe Configuration (5.1 THD packing, 5.4 frozen indexer);
 *   [PR]  radixark/miles PR #4581, kernel-tuning commit message and PR body
 *         (per-block max-logit select, block-sparse attention fwd/bwd, dV
 *         stored with V's own strides, no host sync between select and attention);
 *   [MB]  NVIDIA Megatron-Bridge, "MiniMax-M3", Architecture Notes and Known
 *         Limitations (gemma RMSNorm x*(1+w), partial RoPE, 16 x 128 keys).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Tensors are THD-packed: token-major, then head, then the 128-wide head dim,
 * which must be contiguous (stride 1).  Token and head strides are given in
 * elements; they and every tensor pointer must keep 16-byte alignment (strides
 * multiples of 8 bf16 elements).  All tensor pointers, cu_seqlens and the
 * workspace are DEVICE pointers; msa_dims is read on the host.  bf16 means
 * 16-bit brain-float storage.
 *
 * cu_seqlens holds num_seqs+1 int32 offsets: cu[0] = 0, non-decreasing,
 * cu[num_seqs] = total_tokens, every length <= max_seqlen.  The library never
 * reads it back to the host (no host sync); it trusts this contract, which
 * msa_check_cu_seqlens can verify in debug builds of a caller.
 * Positions and 128-token blocks restart with every sequence ([M31] 5.1).
 *
 * Heads: query head g reads KV head g / (num_q_heads / num_kv_heads); index
 * head h selects the blocks of KV head h ([M31] section 1).  This build
 * supports head_dim = 128, block_size = 128, topk_blocks = 16 and exactly 16
 * query heads per KV head (one TP4 shard of MiniMax-M3 is 16 q / 1 kv).
 *
 * Ownership and execution: the caller allocates every input, output and the
 * workspace (size from msa_workspace_size).  The library allocates nothing
 * and keeps no pointer after a call returns.  Its only state between calls
 * is the optional kernel-timing pool of msa_timing_enable (off by default;
 * see below).
 * Work is enqueued on `stream` and runs asynchronously; outputs are
 * overwritten, never accumulated.  Identical inputs give bitwise identical
 * outputs.  Calls sharing one workspace must be ordered on one stream.
 *
 * Errors: every entry point returns MSA_OK (0) or a negative status.  On an
 * argument error nothing is launched.  MSA_ERR_HIP reports a launch failure
 * (hipGetLastError) after work may already have been enqueued.
 */
#ifndef MSA_H_
#define MSA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MSA_OK 0
#define MSA_ERR_INVALID_ARG (-1) /* null pointer, negative size, bad stride or alignment    */
#define MSA_ERR_UNSUPPORTED (-2) /* valid but outside this build: D/block/topk/group/limits   */
#define MSA_ERR_WORKSPACE (-3)   /* workspace null, misaligned (256 B) or smaller than needed */
#define MSA_ERR_HIP (-4)         /* the HIP runtime reported an error                         */

/* Selection flags of msa_index_select_ex. */
#define MSA_SELECT_FORCE_INIT 1u /* keep block 0 in every selection (the "init" rule) */

/* Attention flags of msa_attn_fwd_ex / msa_attn_bwd_ex. */
#define MSA_ATTN_DENSE 1u /* every causal key of the sequence; blk_idx is not read (may be NULL) */
/* msa_attn_bwd_ex only: the dQ pass recomputes S and dP instead of reading the
 * dS the dK/dV pass stores, so the workspace needs no dS tail
 * (msa_workspace_size(..., MSA_OP_BWD_RECOMPUTE)); same results within
 * rounding, slower, 64 KB less workspace per (token, KV head). */
#define MSA_ATTN_RECOMPUTE 2u

#define MSA_OP_SELECT 1
#define MSA_OP_FWD 2
#define MSA_OP_BWD 3
#define MSA_OP_QKNORM_BWD 4
#define MSA_OP_QSA_FWD 5
#define MSA_OP_QSA_BWD 6
#define MSA_OP_BWD_QKNORM 7
#define MSA_OP_BWD_RECOMPUTE 8 /* msa_attn_bwd_ex with MSA_ATTN_RECOMPUTE (or MSA_ATTN_DENSE) */

/* Longest sequence this build accepts (1024 blocks of 128 tokens). */
#define MSA_MAX_SEQLEN 131072
/* Longest sequence of the narrow-block entry points (8192 blocks of 4 tokens). */
#define MSA_QSA_MAX_SEQLEN 32768

typedef struct msa_dims {
  int32_t total_tokens; /* T = cu_seqlens[num_seqs]; 0 makes every call a no-op          */
  int32_t num_seqs;     /* S >= 1 when T > 0                                             */
  int32_t max_seqlen;   /* host-side bound on every sequence length, sizes the grids     */
  int32_t num_q_heads;  /* Hq = 16 * Hk                                                  */
  int32_t num_kv_heads; /* Hk = number of index heads                                    */
  int32_t head_dim;     /* must be 128                                                   */
  int32_t block_size;   /* must be 128                                                   */
  int32_t topk_blocks;  /* must be 16                                                    */
} msa_dims;

/*
 * Workspace bytes that operation `op` (MSA_OP_*) needs for `dims`, written to
 * *bytes.  The pointer passed to the operation must be 256-byte aligned.
 */
int msa_workspace_size(const msa_dims* dims, int op, size_t* bytes);

/*
 * Frozen lightning-indexer block selection ([M31] section 1; [PR] per-block
 * max-logit scores, rules and top-k; [MB] Architecture Notes for the norm).
 *
 * For token t at sequence-local position p (block b = p / 128) and index
 * head h:
 *   q~ = bf16( RoPE_p( RMSNorm(idx_q[t,h]) * (1 + w_q) ) ),
 *   k~_j likewise from idx_k[j,h] and w_k,
 * where RMSNorm(x) = x / sqrt(mean(x^2) + eps) over the 128 dims, and RoPE_p
 * rotates pairs (i, i+32), i < 32, of dims [0, 64) by p * rope_base^(-2i/64)
 * (rotate-half) leaving dims [64, 128) unchanged; norm and RoPE run in fp32
 * with fp64 angles.  Block c <= b scores max_{j in c, j <= t} q~ . k~_j
 * (fp32 accumulation).  Selection: blocks 0..b when b < 16, else block b
 * plus the 15 best of 0..b-1 (higher score first, lower id on equal scores).
 *
 *   idx_q   [T, Hk, 128] bf16, strides (sq_t, sq_h)
 *   idx_k   [T, Hk, 128] bf16, strides (sk_t, sk_h); sk_h = 0 shares one key head
 *   w_q,w_k [128] bf16 gemma weights (applied as 1 + w)
 *   eps (1e-6), rope_base (1e7), rope_dims (must be 64)
 *   blk_idx [T, Hk, 16] int32 output, contiguous: sequence-local block ids in
 *           ascending order, padded with -1 when b < 15.
 */
int msa_index_select(const msa_dims* dims,
                     const void* idx_q, int64_t sq_t, int64_t sq_h,
                     const void* idx_k, int64_t sk_t, int64_t sk_h,
                     const void* w_q, const void* w_k,
                     float eps, float rope_base, int32_t rope_dims,
                     const int32_t* cu_seqlens, int32_t* blk_idx,
                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * msa_index_select with selection flags ([PR] kernel-tuning commit message:
 * the indexer applies init/local/causal rules before top-k).  flags = 0 is
 * msa_index_select.  MSA_SELECT_FORCE_INIT reads "init" as a forced initial
 * block: when b >= 16, block 0 is kept like block b and the other 14 slots go
 * to the best of blocks 1..b-1 (same order); b < 16 is unchanged (all of
 * 0..b).  Unknown flag bits return MSA_ERR_INVALID_ARG.  Same workspace as
 * msa_index_select (MSA_OP_SELECT).
 */
int msa_index_select_ex(const msa_dims* dims,
                        const void* idx_q, int64_t sq_t, int64_t sq_h,
                        const void* idx_k, int64_t sk_t, int64_t sk_h,
                        const void* w_q, const void* w_k,
                        float eps, float rope_base, int32_t rope_dims, uint32_t flags,
                        const int32_t* cu_seqlens, int32_t* blk_idx,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Attention-side q/k norm and partial RoPE, forward ([M31] section 1: per-head
 * gemma q/k norm, RoPE on the first 64 dims, base 1e7; [MB] Architecture
 * Notes: per-head QK RMSNorm x * (1 + w), partial RoPE).  The step that
 * produces the q and k the attention entry points take.
 *
 * For every head of q (weights w_q) and of k (weights w_k), at token t's
 * sequence-local position p:
 *   out = bf16( RoPE_p( x / sqrt(mean(x^2) + eps) * (1 + w) ) )
 * with the same arithmetic as the indexer features of msa_index_select (fp32,
 * fp64 angles rounded to fp32, one rounding to bf16).
 *
 *   q [T, Hq, 128], k [T, Hk, 128] bf16 inputs, their own strides;
 *   w_q, w_k [128] bf16; q_out [T, Hq, 128], k_out [T, Hk, 128] bf16 outputs
 *   with their own strides (they may not alias the inputs).
 * No workspace.
 */
int msa_qk_norm_rope_fwd(const msa_dims* dims,
                         const void* q, int64_t q_st, int64_t q_sh,
                         const void* k, int64_t k_st, int64_t k_sh,
                         const void* w_q, const void* w_k,
                         float eps, float rope_base, int32_t rope_dims,
                         const int32_t* cu_seqlens,
                         void* q_out, int64_t qo_st, int64_t qo_sh,
                         void* k_out, int64_t ko_st, int64_t ko_sh, hipStream_t stream);

/*
 * Backward of msa_qk_norm_rope_fwd: given the forward's inputs q, k and the
 * gradients dq_hat, dk_hat of its outputs (e.g. msa_attn_bwd's dq, dk),
 *   dy = RoPE_p^T(dz), g = dy * (1 + w),
 *   dx = r g - x r^3 sum(g x) / 128,  r = 1 / sqrt(mean(x^2) + eps)
 * written as bf16 dq, dk (own strides), and the weight gradients
 *   dw[j] = sum over tokens and heads of dy_j x_j r
 * as fp32 dw_q[128], dw_k[128] (overwritten, summed in a fixed order).
 * Workspace: msa_workspace_size(..., MSA_OP_QKNORM_BWD).
 */
int msa_qk_norm_rope_bwd(const msa_dims* dims,
                         const void* q, int64_t q_st, int64_t q_sh,
                         const void* k, int64_t k_st, int64_t k_sh,
                         const void* w_q, const void* w_k,
                         float eps, float rope_base, int32_t rope_dims,
                         const int32_t* cu_seqlens,
                         const void* dq_hat, int64_t dqh_st, int64_t dqh_sh,
                         const void* dk_hat, int64_t dkh_st, int64_t dkh_sh,
                         void* dq, int64_t dq_st, int64_t dq_sh,
                         void* dk, int64_t dk_st, int64_t dk_sh,
                         float* dw_q, float* dw_k,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Attention with the attention-side q/k norm and partial RoPE fused in
 * (miles docs "MiniMax-M3.1-Flash", section 1: per-head gemma q/k norm and RoPE
 * on the first 64 dims ahead of the attention; Megatron-Bridge "MiniMax-M3",
 * Architecture Notes).  q and k are the raw projections [T, H, 128]; every
 * head row gets x * r * (1 + w) with r = 1 / sqrt(mean(x^2) + eps) and
 * rotate-half RoPE at its sequence-local position, rounded once to bf16 (the
 * arithmetic of msa_qk_norm_rope_fwd; only the order of the 128-term sum of
 * squares may differ, so q and k may differ from that kernel's by one bf16
 * unit in rare elements), and the block-sparse attention of msa_attn_fwd_ex
 * runs on the result.  w_q, w_k: [128] bf16 weights, 2-byte aligned; eps >= 0,
 * rope_base > 1, rope_dims must be 64; flags, outputs, strides and errors as
 * msa_attn_fwd_ex.
 *
 * msa_attn_fwd_qknorm: the forward kernels apply the norm themselves (K in the
 *   staging copy, q in the forward kernel's registers); the normalized q and k
 *   are never written.  Workspace: msa_workspace_size(dims, MSA_OP_FWD, ...).
 * msa_attn_bwd_qknorm: gradients with respect to the raw q and k (dq, dk with
 *   their own strides), dv, and the weight gradients dw_q, dw_k (fp32 [128],
 *   4-byte aligned, overwritten; sums over every (token, head) in a fixed
 *   order).  The norm is fused in: the backward's K prep kernel normalizes
 *   k, its dQ kernel normalizes q after loading and takes dq back through the
 *   norm in its epilogue (with that tile's dw_q sums); the normalized rows are
 *   kept in the workspace for the dK/dV pass, whose dk then goes through the
 *   norm's backward over the k rows.  Workspace: msa_workspace_size(dims, MSA_OP_BWD_QKNORM, ...).  With no
 *   tokens only dw_q, dw_k are written (zeros).
 */
int msa_attn_fwd_qknorm(const msa_dims* dims,
                        const void* q, int64_t q_st, int64_t q_sh,
                        const void* k, int64_t k_st, int64_t k_sh,
                        const void* v, int64_t v_st, int64_t v_sh,
                        const void* w_q, const void* w_k, float eps, float rope_base, int32_t rope_dims,
                        const int32_t* blk_idx, const int32_t* cu_seqlens, float softmax_scale, uint32_t flags,
                        void* o, int64_t o_st, int64_t o_sh, float* lse,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

int msa_attn_bwd_qknorm(const msa_dims* dims,
                        const void* q, int64_t q_st, int64_t q_sh,
                        const void* k, int64_t k_st, int64_t k_sh,
                        const void* v, int64_t v_st, int64_t v_sh,
                        const void* w_q, const void* w_k, float eps, float rope_base, int32_t rope_dims,
                        const void* o, int64_t o_st, int64_t o_sh, const float* lse,
                        const void* dO, int64_t do_st, int64_t do_sh,
                        const int32_t* blk_idx, const int32_t* cu_seqlens, float softmax_scale, uint32_t flags,
                        void* dq, int64_t dq_st, int64_t dq_sh,
                        void* dk, int64_t dk_st, int64_t dk_sh,
                        void* dv, int64_t dv_st, int64_t dv_sh,
                        float* dw_q, float* dw_k,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Block-sparse GQA attention forward ([M31] section 1: each query attends to
 * its selected blocks; [PR] QSA block-sparse kernel).
 *
 * For token t, query head g, KV head h = g / 16: the key set J is every key
 * j <= t of the blocks listed in blk_idx[t,h] (ids outside 0..b and -1 are
 * ignored; ids must be distinct).  O[t,g] = sum_j softmax_j(scale * q.k_j) v_j
 * with fp32 softmax and accumulation; LSE[t,g] = natural log of the softmax
 * denominator (the max-shifted sum), saved for the backward.  A row whose key
 * set is empty gets O = 0 and LSE = -inf.
 *
 *   q [T,Hq,128], k,v [T,Hk,128], o [T,Hq,128] bf16 with their own strides;
 *   blk_idx [T,Hk,16] int32 contiguous; lse [T,Hq] fp32 contiguous output.
 */
int msa_attn_fwd(const msa_dims* dims,
                 const void* q, int64_t q_st, int64_t q_sh,
                 const void* k, int64_t k_st, int64_t k_sh,
                 const void* v, int64_t v_st, int64_t v_sh,
                 const int32_t* blk_idx, const int32_t* cu_seqlens, float softmax_scale,
                 void* o, int64_t o_st, int64_t o_sh, float* lse,
                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Block-sparse GQA attention backward ([PR]: gradients of the block-sparse
 * kernel; dK/dV of a KV head are the sum over its query heads, reduced here
 * in a fixed order without atomics; dV is written with V's own strides).
 *
 * Gradients of sum(O * dO) over the same key sets as the forward, from the
 * forward's O and LSE:  P = exp(scale q.k - LSE), dP = dO.v,
 * Delta = rowsum(dO * O), dS = P (dP - Delta); dq = scale sum_j dS k_j;
 * dk_j = scale sum dS q and dv_j = sum P dO over every (query, head) of the
 * group that attends to key j.  The indexer is frozen ([M31] 5.4): there is
 * no gradient for the select inputs.
 *
 *   q, k, v, o, do_ as in the forward (each with its own strides), lse [T,Hq]
 *   fp32 from the forward; outputs dq [T,Hq,128], dk, dv [T,Hk,128] bf16
 *   with their own strides (dv need not share dk's layout).
 *
 * Workspace: msa_workspace_size(dims, MSA_OP_BWD).  When T * Hk <= 262144
 * it ends with 64 KB per (token, KV head) where the dK/dV pass stores each
 * selection's bf16 dS, from which dQ is then formed (16 GiB at that limit);
 * larger packs recompute S and dP in the dQ pass instead.  A dense call, or
 * one with MSA_ATTN_RECOMPUTE (msa_attn_bwd_ex), does not use that tail and
 * accepts a workspace without it (MSA_OP_BWD_RECOMPUTE).
 */
int msa_attn_bwd(const msa_dims* dims,
                 const void* q, int64_t q_st, int64_t q_sh,
                 const void* k, int64_t k_st, int64_t k_sh,
                 const void* v, int64_t v_st, int64_t v_sh,
                 const void* o, int64_t o_st, int64_t o_sh,
                 const float* lse,
                 const void* do_, int64_t do_st, int64_t do_sh,
                 const int32_t* blk_idx, const int32_t* cu_seqlens, float softmax_scale,
                 void* dq, int64_t dq_st, int64_t dq_sh,
                 void* dk, int64_t dk_st, int64_t dk_sh,
                 void* dv, int64_t dv_st, int64_t dv_sh,
                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Narrow-block variant of the block-sparse attention ([PR] kernel-tuning
 * commit message: the block-sparse kernel also runs qwen3.8-next's 4-token
 * blocks, 12 query heads per KV head, head dim 256).  Same definition as
 * msa_attn_fwd / msa_attn_bwd with these differences:
 *   dims: head_dim = 256, block_size = 4, topk_blocks = K in 1..1024 (the
 *         number of block ids listed per query), num_q_heads = 12 * num_kv_heads,
 *         max_seqlen <= MSA_QSA_MAX_SEQLEN; query head g reads KV head g / 12;
 *   blk_idx [T, Hk, K] int32 contiguous, sequence-local 4-token block ids in
 *         any order; ids below 0 and past the query's own block are ignored,
 *         a repeated id counts once; the own block is attended only if listed
 *         (the pages do not say how these blocks are chosen);
 *   q, o, do_, dq [T, Hq, 256] and k, v, dk, dv [T, Hk, 256] bf16 with their
 *         own strides (dim contiguous); lse [T, Hq] fp32.
 * Workspaces: msa_workspace_size(dims, MSA_OP_QSA_FWD / MSA_OP_QSA_BWD, ...).
 * The backward's holds dS for every (token, causal 64-key tile, KV head):
 * 1.5 KB each, so it grows with the square of the sequence lengths (about
 * 1.8 GB for 16384 tokens in sequences of up to 7122, 14 GB for one
 * 32768-token sequence with one KV head).
 * Errors, ownership, determinism and stream semantics as for msa_attn_*.
 */
int msa_qsa_attn_fwd(const msa_dims* dims,
                     const void* q, int64_t q_st, int64_t q_sh,
                     const void* k, int64_t k_st, int64_t k_sh,
                     const void* v, int64_t v_st, int64_t v_sh,
                     const int32_t* blk_idx, const int32_t* cu_seqlens, float softmax_scale,
                     void* o, int64_t o_st, int64_t o_sh, float* lse,
                     void* workspace, size_t workspace_bytes, hipStream_t stream);

int msa_qsa_attn_bwd(const msa_dims* dims,
                     const void* q, int64_t q_st, int64_t q_sh,
                     const void* k, int64_t k_st, int64_t k_sh,
                     const void* v, int64_t v_st, int64_t v_sh,
                     const void* o, int64_t o_st, int64_t o_sh,
                     const float* lse,
                     const void* do_, int64_t do_st, int64_t do_sh,
                     const int32_t* blk_idx, const int32_t* cu_seqlens, float softmax_scale,
                     void* dq, int64_t dq_st, int64_t dq_sh,
                     void* dk, int64_t dk_st, int64_t dk_sh,
                     void* dv, int64_t dv_st, int64_t dv_sh,
                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * msa_attn_fwd / msa_attn_bwd with attention flags.  flags = 0 is the plain
 * call.  MSA_ATTN_DENSE computes the same attention over every causal key of
 * the query's sequence instead of its listed blocks: the plain dense causal
 * attention of MiniMax-M3's first three layers ([PR] PR body: block-sparse
 * attention on the sparse layers, plain dense attention on the first three).
 * blk_idx is then ignored and may be NULL.  MSA_ATTN_RECOMPUTE (backward
 * only) trades speed for workspace, as described at its definition.
 * Unknown flag bits return MSA_ERR_INVALID_ARG.  Same workspaces
 * (MSA_OP_FWD / MSA_OP_BWD, or MSA_OP_BWD_RECOMPUTE) and conventions as the
 * plain calls.
 */
int msa_attn_fwd_ex(const msa_dims* dims,
                    const void* q, int64_t q_st, int64_t q_sh,
                    const void* k, int64_t k_st, int64_t k_sh,
                    const void* v, int64_t v_st, int64_t v_sh,
                    const int32_t* blk_idx, const int32_t* cu_seqlens, float softmax_scale, uint32_t flags,
                    void* o, int64_t o_st, int64_t o_sh, float* lse,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

int msa_attn_bwd_ex(const msa_dims* dims,
                    const void* q, int64_t q_st, int64_t q_sh,
                    const void* k, int64_t k_st, int64_t k_sh,
                    const void* v, int64_t v_st, int64_t v_sh,
                    const void* o, int64_t o_st, int64_t o_sh,
                    const float* lse,
                    const void* do_, int64_t do_st, int64_t do_sh,
                    const int32_t* blk_idx, const int32_t* cu_seqlens, float softmax_scale, uint32_t flags,
                    void* dq, int64_t dq_st, int64_t dq_sh,
                    void* dk, int64_t dk_st, int64_t dk_sh,
                    void* dv, int64_t dv_st, int64_t dv_sh,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Allocation-free forward, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, result and conventions as msa_attn_fwd, minus
 * the workspace: the forward's workspace lives in a static device array of
 * MSA_NOALLOC_SCRATCH_BYTES that each GPU holds until the process ends.  When
 * msa_workspace_size(dims, MSA_OP_FWD) exceeds that size the call returns
 * MSA_ERR_WORKSPACE before anything is launched (the array holds the forward's
 * workspace of up to about 1150 (128-token block, KV head) pairs: the 32768-
 * token, 4-KV-head layer fits).  The call allocates nothing; the first call on
 * a device looks the array's address up once.  All calls on one GPU share its
 * array: calls that overlap on one GPU (other streams, other threads) race
 * and must be serialized by the caller.
 */
#define MSA_NOALLOC_SCRATCH_BYTES (72u << 20)
int msa_attn_fwd_noalloc(const msa_dims* dims,
                         const void* q, int64_t q_st, int64_t q_sh,
                         const void* k, int64_t k_st, int64_t k_sh,
                         const void* v, int64_t v_st, int64_t v_sh,
                         const int32_t* blk_idx, const int32_t* cu_seqlens, float softmax_scale,
                         void* o, int64_t o_st, int64_t o_sh, float* lse, hipStream_t stream);

/* Static, human-readable text for a status code. */
const char* msa_status_string(int status);

/*
 * Debug check of the cu_seqlens contract.  Unlike every other entry point it
 * copies cu_seqlens to the host and synchronizes `stream`.  Returns MSA_OK,
 * MSA_ERR_INVALID_ARG when the offsets break the contract, or MSA_ERR_HIP.
 */
int msa_check_cu_seqlens(const msa_dims* dims, const int32_t* cu_seqlens, hipStream_t stream);

/*
 * Kernel timing, for benchmarks and profiling.  When enabled, every kernel the
 * library launches is bracketed by a pair of HIP events recorded on the launch
 * stream.  msa_timing_collect waits for the recorded events, then writes up to
 * `capacity` per-kernel totals (launch count and summed milliseconds, kernels
 * in first-launch order; `name` points to static storage) and the number
 * written to *count, and forgets what it reported.  Timing adds two event
 * records per launch; leave it off outside measurement.  Process-wide state,
 * guarded by a mutex.
 */
typedef struct msa_kernel_time {
  const char* name;
  int32_t launches;
  float total_ms;
} msa_kernel_time;

int msa_timing_enable(int enable);
int msa_timing_collect(msa_kernel_time* out, int32_t capacity, int32_t* count);

/* Library version, major * 10000 + minor * 100 + patch. */
int msa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H_ */
