"""GPU checks of the ABI's contracts beyond parity.

* msa_check_cu_seqlens: the debug check of the cu_seqlens contract (a host copy
  after a stream sync) accepts valid offsets and rejects non-monotone,
  overlong, badly started or badly ended ones.
* Determinism across streams: the same call on two streams at once (separate
  outputs and workspaces) gives bitwise the outputs of a call on the default
  stream.
* Pack order: a sequence's selection and gradients do not depend on where it
  sits in the pack (positions and blocks restart per sequence): a shuffled pack
  gives bitwise the same per-sequence outputs, and matches the oracle.
* The binding rejects tensors of the wrong dtype, shape, layout or device
  before anything is launched.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import synth
from parity import check_grad, check_out, check_select, say

pytestmark = pytest.mark.gpu


def f32(t):
    return t.float().cpu().numpy()


def dev(t):
    return t.to("cuda")


def step(msa, p, stream=None):
    """select -> forward on the selection -> backward, on ``stream``."""
    s = stream or torch.cuda.current_stream()
    with torch.cuda.stream(s):
        cu = dev(p.cu_seqlens)
        args = [dev(t) for t in (p.idx_q, p.idx_k, p.w_q, p.w_k)]
        q, k, v, do = dev(p.q), dev(p.k), dev(p.v), dev(p.do)
        blk = msa.msa_index_select(*args, cu, p.max_seqlen)
        o, lse = msa.msa_attn_fwd(q, k, v, blk, cu, p.max_seqlen)
        dq, dk, dv = msa.msa_attn_bwd(q, k, v, o, lse, do, blk, cu, p.max_seqlen)
    return blk, o, lse, dq, dk, dv


def test_check_cu_seqlens(gpu_lib):
    msa = gpu_lib
    ok = torch.tensor([0, 300, 300, 1000, 1200], dtype=torch.int32, device="cuda")
    assert msa.msa_check_cu_seqlens(ok, 1200, 700) == msa.MSA_OK
    assert msa.msa_check_cu_seqlens(ok, 1200, 699) == msa.MSA_ERR_INVALID_ARG     # a length over max_seqlen
    assert msa.msa_check_cu_seqlens(ok, 1201, 700) == msa.MSA_ERR_INVALID_ARG     # cu[S] != T
    for bad in ([0, 300, 200, 1000, 1200],                                          # not monotone
                [5, 300, 300, 1000, 1200]):                                         # cu[0] != 0
        t = torch.tensor(bad, dtype=torch.int32, device="cuda")
        assert msa.msa_check_cu_seqlens(t, 1200, 800) == msa.MSA_ERR_INVALID_ARG, bad
    empty = torch.zeros(1, dtype=torch.int32, device="cuda")
    assert msa.msa_check_cu_seqlens(empty, 0, 0) == msa.MSA_OK


def test_two_streams_bitwise(gpu_lib):
    msa = gpu_lib
    p = synth.make_custom_pack([3100, 1700, 900], seed=71)
    ref = step(msa, p)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    a = step(msa, p, s1)
    b = step(msa, p, s2)
    torch.cuda.synchronize()
    for name, x, y, z in zip(("blk", "O", "LSE", "dQ", "dK", "dV"), ref, a, b):
        assert torch.equal(x, y) and torch.equal(x, z), name


def test_pack_order_does_not_matter(gpu_lib):
    msa = gpu_lib
    lengths = [2500, 700, 1900, 130, 1]
    p = synth.make_custom_pack(lengths, seed=72)
    perm = [3, 0, 4, 2, 1]
    cu = p.cu_seqlens.numpy()
    idx = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in perm])
    shuf = synth.make_custom_pack([lengths[s] for s in perm], seed=72)
    for name in ("q", "k", "v", "idx_q", "idx_k", "do"):
        setattr(shuf, name, getattr(p, name)[torch.from_numpy(idx)].contiguous())
    shuf.w_q, shuf.w_k = p.w_q, p.w_k
    a = [t.cpu() for t in step(msa, p)]
    b = [t.cpu() for t in step(msa, shuf)]
    torch.cuda.synchronize()
    for name, x, y in zip(("blk", "O", "LSE", "dQ", "dK", "dV"), a, b):
        assert torch.equal(x[torch.from_numpy(idx)], y), name
    # and the shuffled pack against the oracle
    cs = shuf.cu_seqlens.numpy()
    res = O.index_select(f32(shuf.idx_q), f32(shuf.idx_k), f32(shuf.w_q), f32(shuf.w_k), cs, keep_scores=True)
    check_select(res, b[0].numpy(), "shuffled pack")
    blk = b[0].numpy()
    sc = 1 / math.sqrt(128)
    Ow, Lw = O.attention_forward(f32(shuf.q), f32(shuf.k), f32(shuf.v), blk, cs, sc)
    dQw, dKw, dVw = O.attention_backward(f32(shuf.q), f32(shuf.k), f32(shuf.v), f32(shuf.do), blk, cs, sc)
    check_out("shuffled pack", f32(b[1]), Ow, b[2].numpy(), Lw)
    check_grad("shuffled pack", "dQ", f32(b[3]), dQw)
    check_grad("shuffled pack", "dK", f32(b[4]), dKw)
    check_grad("shuffled pack", "dV", f32(b[5]), dVw)


def test_binding_rejects_bad_tensors_before_launch(gpu_lib):
    msa = gpu_lib
    p = synth.make_custom_pack([600, 300], seed=73)
    cu = dev(p.cu_seqlens)
    q, k, v, do = dev(p.q), dev(p.k), dev(p.v), dev(p.do)
    iq, ik, wq, wk = dev(p.idx_q), dev(p.idx_k), dev(p.w_q), dev(p.w_k)
    blk = msa.msa_index_select(iq, ik, wq, wk, cu, p.max_seqlen)
    o, lse = msa.msa_attn_fwd(q, k, v, blk, cu, p.max_seqlen)
    torch.cuda.synchronize()
    with pytest.raises(ValueError, match="cu_seqlens"):
        msa.msa_index_select(iq, ik, wq, wk, cu.long(), p.max_seqlen)
    with pytest.raises(ValueError, match="cu_seqlens"):
        msa.msa_attn_fwd(q, k, v, blk, p.cu_seqlens, p.max_seqlen)              # host tensor
    with pytest.raises(ValueError, match="w_q"):
        msa.msa_index_select(iq, ik, wq.float(), wk, cu, p.max_seqlen)
    with pytest.raises(ValueError, match="blk_idx"):
        msa.msa_attn_fwd(q, k, v, blk.long(), cu, p.max_seqlen)
    with pytest.raises(ValueError, match="blk_idx"):
        msa.msa_attn_bwd(q, k, v, o, lse, do, blk[:, :, :8].contiguous(), cu, p.max_seqlen)
    with pytest.raises(ValueError, match="lse"):
        msa.msa_attn_bwd(q, k, v, o, lse[:, :8].contiguous(), do, blk, cu, p.max_seqlen)
    with pytest.raises(ValueError, match="lse"):
        msa.msa_attn_bwd(q, k, v, o, lse.double(), do, blk, cu, p.max_seqlen)
    with pytest.raises(ValueError):
        msa.msa_attn_bwd(q, k, v, o[:, :8], lse, do, blk, cu, p.max_seqlen)
    torch.cuda.synchronize()
    say("binding rejections raised before launch")
