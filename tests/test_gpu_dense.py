"""GPU parity of the dense layers' attention (msa_attn_fwd_ex / msa_attn_bwd_ex with
MSA_ATTN_DENSE): every causal key of the sequence, checked against the oracle with
every causal block listed.  Tolerances as for the sparse path."""
import math

import numpy as np
import pytest
import torch

import oracle as O
import synth

pytestmark = pytest.mark.gpu

O_TOL = 2e-2
G_TOL = 1e-2
LSE_TOL = 1e-3
SCALE = 1 / math.sqrt(128)


def f32(t):
    return t.float().cpu().numpy()


def dev(t):
    return t.to("cuda")


def say(*a):
    print(*a, flush=True)


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


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
    eo = float(np.abs(f32(o) - Ow).max())
    el = float(np.abs(lse.cpu().numpy() - Lw).max())
    rq, rk, rv = rel(f32(dq), dQw), rel(f32(dk), dKw), rel(f32(dv), dVw)
    say(f"[dense {lengths} hk={hk}] O maxabs={eo:.3e} LSE maxabs={el:.3e} dQ rel={rq:.3e} dK rel={rk:.3e} "
        f"dV rel={rv:.3e}")
    assert eo <= O_TOL and el <= LSE_TOL
    assert rq <= G_TOL and rk <= G_TOL and rv <= G_TOL


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
    eo = float(np.abs(f32(o)[rows] - Ow).max())
    el = float(np.abs(lse.cpu().numpy()[rows] - Lw).max())
    rq = rel(f32(dq)[rows], dQw)
    last = np.arange(8064, 8192)
    _, dKw, dVw = O.attention_backward(q, k, v, do, blk, cu, SCALE, rows=last)
    rk, rv = rel(f32(dk)[last], dKw[last]), rel(f32(dv)[last], dVw[last])
    say(f"[dense single8k] O maxabs={eo:.3e} LSE maxabs={el:.3e} dQ rel={rq:.3e} last-block dK rel={rk:.3e} "
        f"dV rel={rv:.3e}")
    assert eo <= O_TOL and el <= LSE_TOL and rq <= G_TOL and rk <= G_TOL and rv <= G_TOL
