"""GPU parity of the selection variants against the oracle.

The forced initial block (msa_index_select_ex with MSA_SELECT_FORCE_INIT; the
"init" of the pages' init/local/causal rules, radixark/miles PR #4581 commit
message, read as block 0 always kept): hand-derived planted cases, seeded
packs on both top-k paths (up to 64 candidate blocks, and more), and attention
forward + backward on the forced selection.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import synth
from parity import check_grad, check_out, check_select
from planted import load_planted

pytestmark = pytest.mark.gpu


def f32(t):
    return t.float().cpu().numpy()


def dev(t):
    return t.to("cuda")


def test_force_init_planted_golden(gpu_lib):
    P = load_planted()
    cu = torch.from_numpy(P["cu_seqlens"])
    args = (dev(P["idx_q"]), dev(P["idx_k"]), dev(P["w_q"]), dev(P["w_k"]), dev(cu), max(P["lengths"]))
    forced = gpu_lib.msa_index_select(*args, force_init=True).cpu().numpy()
    for t, ids, why in P["expected_force_init"]:
        assert list(forced[t, 0]) == ids, (t, why)
    plain = gpu_lib.msa_index_select(*args).cpu().numpy()
    for t, ids, why in P["expected"]:
        assert list(plain[t, 0]) == ids, (t, why)
    # every row: exact ties decided by the lower-id rule, as the oracle decides them
    res = O.index_select(f32(P["idx_q"]), f32(P["idx_k"]), f32(P["w_q"]), f32(P["w_k"]), P["cu_seqlens"],
                         force_init=True)
    bad = np.nonzero((forced != res.blk_idx).any(axis=(1, 2)))[0]
    assert bad.size == 0, f"{bad.size} rows differ from the oracle, first {bad[:8]}"


@pytest.mark.parametrize("lengths,hk,seed", [([2600, 700, 2300], 1, 51), ([3000, 1100], 2, 52), ([9000], 1, 53)])
def test_force_init_parity(gpu_lib, lengths, hk, seed):
    """[9000] has up to 70 candidate blocks: the arg-max-rounds path of top-k."""
    p = synth.make_custom_pack(lengths, num_q_heads=16 * hk, num_kv_heads=hk, seed=seed)
    res = O.index_select(f32(p.idx_q), f32(p.idx_k), f32(p.w_q), f32(p.w_k), p.cu_seqlens.numpy(), force_init=True,
                         keep_scores=True)
    g = gpu_lib.msa_index_select(dev(p.idx_q), dev(p.idx_k), dev(p.w_q), dev(p.w_k), dev(p.cu_seqlens),
                                 p.max_seqlen, force_init=True).cpu().numpy()
    check_select(res, g, f"force_init {lengths} hk={hk}", force_init=True)
    # block 0 is in every row
    assert (g[:, :, 0] == 0).all()


def test_force_init_attention(gpu_lib):
    """Forward and backward on the forced selection (oracle ids) against the oracle."""
    msa = gpu_lib
    p = synth.make_custom_pack([2700, 900], seed=54)
    cu = p.cu_seqlens.numpy()
    res = O.index_select(f32(p.idx_q), f32(p.idx_k), f32(p.w_q), f32(p.w_k), cu, force_init=True)
    blk = dev(torch.from_numpy(res.blk_idx))
    q, k, v, do = dev(p.q), dev(p.k), dev(p.v), dev(p.do)
    o, lse = msa.msa_attn_fwd(q, k, v, blk, dev(p.cu_seqlens), p.max_seqlen)
    dq, dk, dv = msa.msa_attn_bwd(q, k, v, o, lse, do, blk, dev(p.cu_seqlens), p.max_seqlen)
    torch.cuda.synchronize()
    s = 1 / math.sqrt(128)
    Ow, Lw = O.attention_forward(f32(p.q), f32(p.k), f32(p.v), res.blk_idx, cu, s)
    dQw, dKw, dVw = O.attention_backward(f32(p.q), f32(p.k), f32(p.v), f32(p.do), res.blk_idx, cu, s)
    check_out("force_init attn", f32(o), Ow, lse.cpu().numpy(), Lw)
    check_grad("force_init attn", "dQ", f32(dq), dQw)
    check_grad("force_init attn", "dK", f32(dk), dKw)
    check_grad("force_init attn", "dV", f32(dv), dVw)


def _select_workspace_features(msa, p, ws):
    """The q and k indexer features msa_index_select left in its workspace:
    the plan tables (blkbase [S+1], blk_seq [block bound], seqitem [S+1],
    totals [4], tile order [ceil(T/16)] int32), then q and k features
    [T, Hk, 128] bf16, each region starting on a 256-byte boundary."""
    T, Hk, _ = p.idx_q.shape
    S = p.cu_seqlens.numel() - 1
    up = lambda x: (x + 255) // 256 * 256
    off = 0
    for n in (S + 1, min((T + 127 * S) // 128, T), S + 1, 4, (T + 15) // 16):
        off = up(off + 4 * n)
    raw = ws.cpu().numpy()
    nbytes = T * Hk * 128 * 2
    qf = raw[off:off + nbytes].view(np.uint16).reshape(T, Hk, 128)
    kf = raw[up(off + nbytes):up(off + nbytes) + nbytes].view(np.uint16).reshape(T, Hk, 128)
    return qf, kf


@pytest.mark.parametrize("lengths,hk,seed", [([2600, 700, 2300], 1, 55), ([3000, 1100], 4, 56)])
def test_select_features_bitwise(gpu_lib, lengths, hk, seed):
    """The selection's q / k features (norm, RoPE, one bf16 rounding) equal the
    oracle's bit for bit: the norm's sum of squares runs in the oracle's fp32
    order, so the two only meet fp32 rounding differences in the scores."""
    msa = gpu_lib
    p = synth.make_custom_pack(lengths, num_q_heads=16 * hk, num_kv_heads=hk, seed=seed)
    T = p.idx_q.shape[0]
    need = msa.msa_workspace_size(msa.make_dims(T, len(lengths), p.max_seqlen, 16 * hk, hk), msa.MSA_OP_SELECT)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    msa.msa_index_select(dev(p.idx_q), dev(p.idx_k), dev(p.w_q), dev(p.w_k), dev(p.cu_seqlens), p.max_seqlen,
                         workspace=ws)
    torch.cuda.synchronize()
    gq, gk = _select_workspace_features(msa, p, ws)
    _, pos = O.sequence_layout(p.cu_seqlens.numpy())
    bits = lambda a: (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    for h in range(hk):
        wq = O.indexer_features(f32(p.idx_q)[:, h], f32(p.w_q), pos, 1e-6, 1e7, 64)
        wk = O.indexer_features(f32(p.idx_k)[:, h], f32(p.w_k), pos, 1e-6, 1e7, 64)
        assert np.array_equal(gq[:, h], bits(wq)), int((gq[:, h] != bits(wq)).sum())
        assert np.array_equal(gk[:, h], bits(wk)), int((gk[:, h] != bits(wk)).sum())
