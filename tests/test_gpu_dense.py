"""GPU parity of the dense layers' attention (msa_attn_fwd_ex / msa_attn_bwd_ex with
MSA_ATTN_DENSE): every causal key of the sequence, checked against the oracle with
every causal block listed.  Tolerances as for the sparse path."""
import math

import numpy as np
import pytest
import torch

import oracle as O
import synth
from parity import check_grad, check_out

pytestmark = pytest.mark.gpu

SCALE = 1 / math.sqrt(128)


def f32(t):
    return t.float().cpu().numpy()


def dev(t):
    return t.to("cuda")


def all_blocks(cu, hk, width=None):
    seq, pos = O.sequence_layout(cu)
    nb = int(pos.max()) // 128 + 1 if width is None else width
    blk = np.full((len(seq), hk, nb), -1, np.int32)
    for t in range(len(seq)):
        blk[t, :, :pos[t] // 128 + 1] = np.arange(pos[t] // 128 + 1)
    return blk


def run(msa, p, blk=None):
    cu = dev(p.cu_seqlens)
    q, k, v, do = dev(p.q), dev(p.k), dev(p.v), dev(p.do)
    dense = blk is None
    b = None if dense else dev(torch.from_numpy(np.ascontiguousarray(blk)))
    o, lse = msa.msa_attn_fwd(q, k, v, b, cu, p.max_seqlen, dense=dense)
    dq, dk, dv = msa.msa_attn_bwd(q, k, v, o, lse, do, b, cu, p.max_seqlen, dense=dense)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


@pytest.mark.parametrize("lengths,hk,seed", [([3000, 1500, 200], 1, 61), ([2600, 130, 1], 2, 62)])
def test_dense_parity(gpu_lib, lengths, hk, seed):
    p = synth.make_custom_pack(lengths, num_q_heads=16 * hk, num_kv_heads=hk, seed=seed)
    cu = p.cu_seqlens.numpy()
    o, lse, dq, dk, dv = run(gpu_lib, p)
    blk = all_blocks(cu, hk)
    Ow, Lw = O.attention_forward(f32(p.q), f32(p.k), f32(p.v), blk, cu, SCALE)
    dQw, dKw, dVw = O.attention_backward(f32(p.q), f32(p.k), f32(p.v), f32(p.do), blk, cu, SCALE)
    label = f"dense {lengths} hk={hk}"
    check_out(label, f32(o), Ow, lse.cpu().numpy(), Lw)
    check_grad(label, "dQ", f32(dq), dQw)
    check_grad(label, "dK", f32(dk), dKw)
    check_grad(label, "dV", f32(dv), dVw)


def test_dense_equals_sparse_with_every_block_listed(gpu_lib):
    """Up to 2048 tokens every causal block fits in the 16 slots: the dense and the sparse
    kernels then walk the same blocks in the same order and agree bitwise."""
    p = synth.make_custom_pack([2048, 1000, 5, 77], seed=63)
    blk = all_blocks(p.cu_seqlens.numpy(), 1, width=16)
    a = run(gpu_lib, p)
    b = run(gpu_lib, p, blk)
    for x, y, n in zip(a, b, ("O", "LSE", "dQ", "dK", "dV")):
        assert torch.equal(x, y), n


def test_dense_long_sequence_sampled(gpu_lib):
    """One 8192-token sequence (64 blocks, all attended): sampled rows of O, LSE and dQ, and dK/dV
    of the last block (selected by its own 128 queries only) against the oracle."""
    p = synth.make_pack("single8k", 0)
    cu = p.cu_seqlens.numpy()
    o, lse, dq, dk, dv = run(gpu_lib, p)
    blk = all_blocks(cu, 1)
    rows = np.unique(np.concatenate([np.random.default_rng(64).integers(0, 8192, 24), [0, 127, 128, 8191]]))
    q, k, v, do = f32(p.q), f32(p.k), f32(p.v), f32(p.do)
    Ow, Lw = O.attention_forward(q, k, v, blk, cu, SCALE, rows=rows)
    dQw, _, _ = O.attention_backward(q, k, v, do, blk, cu, SCALE, rows=rows)
    check_out("dense single8k", f32(o)[rows], Ow, lse.cpu().numpy()[rows], Lw)
    check_grad("dense single8k", "dQ (sampled rows)", f32(dq)[rows], dQw)
    last = np.arange(8064, 8192)
    _, dKw, dVw = O.attention_backward(q, k, v, do, blk, cu, SCALE, rows=last)
    check_grad("dense single8k", "dK (last block)", f32(dk)[last], dKw[last])
    check_grad("dense single8k", "dV (last block)", f32(dv)[last], dVw[last])
