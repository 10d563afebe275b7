"""GPU edge cases: empty packs and sequences, block lists the selector never
produces (unsorted, duplicated, out of range, missing own block), the
longest sequence this build accepts, and repeated calls that share one
workspace.  The oracle defines the expected result of each."""
import math

import numpy as np
import pytest
import torch

import oracle as O
import synth
from parity import check_grad, check_out, check_select

pytestmark = pytest.mark.gpu


def f32(t):
    return t.float().cpu().numpy()


def random_blocks(cu, hk, rng, k=16, junk=False):
    """Seeded block lists: own block plus up to 15 random earlier blocks.  With
    junk=True rows are shuffled and get duplicates, ids past the own block or
    the sequence, -1 holes, and sometimes lose the own block."""
    seq, pos = O.sequence_layout(cu)
    T = len(seq)
    blk = np.full((T, hk, k), -1, np.int32)
    for t in range(T):
        b = int(pos[t]) // 128
        for h in range(hk):
            ids = [b] + [int(x) for x in rng.permutation(b)[:k - 1]]
            if junk:
                r = rng.random()
                if r < 0.2 and len(ids) > 2:
                    ids[1] = ids[2]                      # duplicate
                elif r < 0.4:
                    ids[-1] = b + 1 + int(rng.integers(0, 5000))  # beyond the own block / sequence
                elif r < 0.5 and len(ids) > 1:
                    ids = ids[1:]                        # own block missing
                ids = list(rng.permutation(ids))
            blk[t, h, :len(ids)] = ids[:k]
    return blk


def run(msa, p, blk):
    g = lambda t: t.to("cuda")
    cu = g(p.cu_seqlens)
    q, k, v, do = g(p.q), g(p.k), g(p.v), g(p.do)
    b = g(torch.from_numpy(np.ascontiguousarray(blk)))
    o, lse = msa.msa_attn_fwd(q, k, v, b, cu, max(p.max_seqlen, 1))
    dq, dk, dv = msa.msa_attn_bwd(q, k, v, o, lse, do, b, cu, max(p.max_seqlen, 1))
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


def check(p, blk, out, rows=None, label="edge"):
    o, lse, dq, dk, dv = out
    cu = p.cu_seqlens.numpy()
    s = 1 / math.sqrt(128)
    Ow, Lw = O.attention_forward(f32(p.q), f32(p.k), f32(p.v), blk, cu, s, rows=rows)
    dQw, dKw, dVw = O.attention_backward(f32(p.q), f32(p.k), f32(p.v), f32(p.do), blk, cu, s, rows=rows)
    r = slice(None) if rows is None else rows
    on, ln = f32(o)[r], lse.cpu().numpy()[r]
    # rows with no key: O = 0 and LSE = -inf on both sides
    empty = np.isinf(Lw)
    assert np.array_equal(np.isinf(ln), empty)
    assert np.all(on[empty] == 0)
    check_out(label, on, Ow, ln, Lw)
    check_grad(label, "dQ", f32(dq)[r], dQw)
    if rows is None:
        check_grad(label, "dK", f32(dk), dKw)
        check_grad(label, "dV", f32(dv), dVw)


def test_empty_pack_is_a_noop(gpu_lib):
    msa = gpu_lib
    z = torch.zeros(0, 16, 128, dtype=torch.bfloat16, device="cuda")
    z1 = torch.zeros(0, 1, 128, dtype=torch.bfloat16, device="cuda")
    cu = torch.zeros(1, dtype=torch.int32, device="cuda")
    w = torch.zeros(128, dtype=torch.bfloat16, device="cuda")
    blk = msa.msa_index_select(z1, z1, w, w, cu, 0)
    assert blk.shape == (0, 1, 16)
    o, lse = msa.msa_attn_fwd(z, z1, z1, blk, cu, 0)
    dq, dk, dv = msa.msa_attn_bwd(z, z1, z1, o, lse, z, blk, cu, 0)
    torch.cuda.synchronize()


def test_empty_sequences_inside_a_pack(gpu_lib):
    p = synth.make_custom_pack([0, 300, 0, 0, 2200, 0, 5], seed=31)
    res = O.index_select(f32(p.idx_q), f32(p.idx_k), f32(p.w_q), f32(p.w_k), p.cu_seqlens.numpy(),
                         keep_scores=True)
    g = lambda t: t.to("cuda")
    blk = gpu_lib.msa_index_select(g(p.idx_q), g(p.idx_k), g(p.w_q), g(p.w_k), g(p.cu_seqlens), p.max_seqlen)
    check_select(res, blk.cpu().numpy(), "empty sequences")
    check(p, res.blk_idx, run(gpu_lib, p, res.blk_idx), label="empty sequences")


def test_unusual_block_lists(gpu_lib):
    """Unsorted, duplicated, out-of-range ids, -1 holes and missing own blocks."""
    rng = np.random.default_rng(32)
    p = synth.make_custom_pack([2600, 1300], num_q_heads=32, num_kv_heads=2, seed=32)
    blk = random_blocks(p.cu_seqlens.numpy(), 2, rng, junk=True)
    check(p, blk, run(gpu_lib, p, blk), label="unusual lists")


def test_longest_sequence(gpu_lib):
    """One 131072-token sequence (1024 blocks): select on sampled rows, attention
    on seeded block lists, checked on sampled rows."""
    msa = gpu_lib
    rng = np.random.default_rng(33)
    p = synth.make_custom_pack([131072], seed=33)
    rows = np.array([0, 127, 128, 2047, 2048, 65535, 65536, 131071] + list(rng.integers(0, 131072, 8)))
    res = O.index_select(f32(p.idx_q), f32(p.idx_k), f32(p.w_q), f32(p.w_k), p.cu_seqlens.numpy(), rows=rows,
                         keep_scores=True)
    g = lambda t: t.to("cuda")
    blk_g = msa.msa_index_select(g(p.idx_q), g(p.idx_k), g(p.w_q), g(p.w_k), g(p.cu_seqlens), 131072).cpu().numpy()
    check_select(res, blk_g, "longest sequence")
    blk = random_blocks(p.cu_seqlens.numpy(), 1, rng)
    check(p, blk, run(msa, p, blk), rows=np.unique(rows), label="longest sequence")


def test_shared_workspace_repeated_calls(gpu_lib):
    """A workspace reused across calls of different sizes leaves no trace."""
    msa = gpu_lib
    rng = np.random.default_rng(34)
    big = synth.make_custom_pack([3000, 2500], seed=34)
    small = synth.make_custom_pack([700, 90], seed=35)
    dims = msa.make_dims(big.total, 2, big.max_seqlen, 16, 1)
    ws = {op: torch.empty(msa.msa_workspace_size(dims, op), dtype=torch.uint8, device="cuda") for op in (1, 2, 3)}
    outs = []
    for p in (big, small, big):
        blk = random_blocks(p.cu_seqlens.numpy(), 1, rng if p is small else np.random.default_rng(36))
        g = lambda t: t.to("cuda")
        cu = g(p.cu_seqlens)
        b = g(torch.from_numpy(blk))
        q, k, v, do = g(p.q), g(p.k), g(p.v), g(p.do)
        sel = msa.msa_index_select(g(p.idx_q), g(p.idx_k), g(p.w_q), g(p.w_k), cu, p.max_seqlen, workspace=ws[1])
        o, lse = msa.msa_attn_fwd(q, k, v, b, cu, p.max_seqlen, workspace=ws[2])
        dq, dk, dv = msa.msa_attn_bwd(q, k, v, o, lse, do, b, cu, p.max_seqlen, workspace=ws[3])
        torch.cuda.synchronize()
        outs.append((sel, o, lse, dq, dk, dv))
        if p is small:
            check(p, blk, (o, lse, dq, dk, dv), label="shared workspace")
    for a, b in zip(outs[0], outs[2]):
        assert torch.equal(a, b)
