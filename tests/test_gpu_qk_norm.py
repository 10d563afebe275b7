"""GPU parity of the attention-side q/k gemma norm + partial RoPE (forward and
backward) against the oracle: per-head norm with one [128] weight for q and
one for k, rotate-half RoPE on dims 0..63 at sequence-local positions (miles
docs "MiniMax-M3.1-Flash", section 1; Megatron-Bridge "MiniMax-M3",
Architecture Notes).  Also the whole chain raw q/k -> norm+RoPE -> block-sparse
attention forward/backward -> norm+RoPE backward."""
import math

import numpy as np
import pytest
import torch

import oracle as O
import synth
from parity import check_grad, rel

pytestmark = pytest.mark.gpu


def f32(t):
    return t.float().cpu().numpy()


def dev(t):
    return t.to("cuda")


def inputs(lengths, hq, hk, seed):
    p = synth.make_custom_pack(lengths, num_q_heads=hq, num_kv_heads=hk, seed=seed)
    g = torch.Generator().manual_seed(seed + 1000)
    wq = (0.1 * torch.randn(128, generator=g)).bfloat16()
    wk = (0.1 * torch.randn(128, generator=g)).bfloat16()
    dqh = torch.randn(p.q.shape, generator=g).bfloat16()
    dkh = torch.randn(p.k.shape, generator=g).bfloat16()
    return p, wq, wk, dqh, dkh


def test_qk_norm_rope_forward_parity(gpu_lib):
    p, wq, wk, _, _ = inputs([2300, 700], 32, 2, 61)
    cu = p.cu_seqlens.numpy()
    _, pos = O.sequence_layout(cu)
    # strided input views: q and k as slices of one fused buffer
    fused = torch.cat([p.q, p.k], dim=1)
    q, k = dev(fused)[:, :32], dev(fused)[:, 32:]
    qo, ko = gpu_lib.msa_qk_norm_rope_fwd(q, k, dev(wq), dev(wk), dev(p.cu_seqlens), p.max_seqlen)
    want_q = O.qk_norm_rope_forward(f32(p.q), f32(wq), pos)
    want_k = O.qk_norm_rope_forward(f32(p.k), f32(wk), pos)
    for got, want, name in ((f32(qo), want_q, "q"), (f32(ko), want_k, "k")):
        diff = np.abs(got - want)
        ulp = np.abs(want) * 2.0 ** -7 + 1e-30
        exact = float((diff == 0).mean())
        print(f"[qk fwd {name}] exact {exact:.5f} max diff / bf16 ulp {float((diff / ulp).max()):.2f}", flush=True)
        assert (diff <= ulp).all()          # at most one bf16 ulp (fp32 sum order of mean(x^2))
        assert exact >= 0.99


def test_qk_norm_rope_backward_parity_and_determinism(gpu_lib):
    p, wq, wk, dqh, dkh = inputs([2300, 700], 32, 2, 62)
    cu = p.cu_seqlens.numpy()
    _, pos = O.sequence_layout(cu)
    args = (dev(p.q), dev(p.k), dev(wq), dev(wk), dev(p.cu_seqlens), p.max_seqlen, dev(dqh), dev(dkh))
    dq, dk, dwq, dwk = gpu_lib.msa_qk_norm_rope_bwd(*args)
    dq2, dk2, dwq2, dwk2 = gpu_lib.msa_qk_norm_rope_bwd(*args)
    torch.cuda.synchronize()
    for a, b in ((dq, dq2), (dk, dk2), (dwq, dwq2), (dwk, dwk2)):
        assert torch.equal(a, b)
    dxq, dwq_w = O.qk_norm_rope_backward(f32(p.q), f32(wq), pos, f32(dqh))
    dxk, dwk_w = O.qk_norm_rope_backward(f32(p.k), f32(wk), pos, f32(dkh))
    r = (rel(dwq.cpu().numpy(), dwq_w), rel(dwk.cpu().numpy(), dwk_w))
    print(f"[qk bwd] dw_q rel {r[0]:.2e} dw_k rel {r[1]:.2e}", flush=True)
    check_grad("qk bwd", "dq", f32(dq), dxq)
    check_grad("qk bwd", "dk", f32(dk), dxk)
    assert r[0] <= 1e-4 and r[1] <= 1e-4


def test_qk_norm_rope_empty_pack(gpu_lib):
    z = torch.zeros(0, 16, 128, dtype=torch.bfloat16, device="cuda")
    z1 = torch.zeros(0, 1, 128, dtype=torch.bfloat16, device="cuda")
    w = torch.zeros(128, dtype=torch.bfloat16, device="cuda")
    cu = torch.zeros(1, dtype=torch.int32, device="cuda")
    gpu_lib.msa_qk_norm_rope_fwd(z, z1, w, w, cu, 0)
    dq, dk, dwq, dwk = gpu_lib.msa_qk_norm_rope_bwd(z, z1, w, w, cu, 0, z, z1)
    torch.cuda.synchronize()
    assert dwq.abs().sum().item() == 0 and dwk.abs().sum().item() == 0


def test_qk_norm_rope_with_attention_chain(gpu_lib):
    """raw q, k -> norm + RoPE -> attention fwd/bwd on the oracle's selection ->
    norm + RoPE backward, against the oracle's chain."""
    msa = gpu_lib
    p, wq, wk, _, _ = inputs([2600, 600], 16, 1, 63)
    cu = p.cu_seqlens.numpy()
    _, pos = O.sequence_layout(cu)
    res = O.index_select(f32(p.idx_q), f32(p.idx_k), f32(p.w_q), f32(p.w_k), cu)
    blk = dev(torch.from_numpy(res.blk_idx))
    cud = dev(p.cu_seqlens)
    qh, kh = msa.msa_qk_norm_rope_fwd(dev(p.q), dev(p.k), dev(wq), dev(wk), cud, p.max_seqlen)
    o, lse = msa.msa_attn_fwd(qh, kh, dev(p.v), blk, cud, p.max_seqlen)
    dqh, dkh, dv = msa.msa_attn_bwd(qh, kh, dev(p.v), o, lse, dev(p.do), blk, cud, p.max_seqlen)
    dq, dk, dwq, dwk = msa.msa_qk_norm_rope_bwd(dev(p.q), dev(p.k), dev(wq), dev(wk), cud, p.max_seqlen, dqh, dkh)
    torch.cuda.synchronize()
    s = 1 / math.sqrt(128)
    qh_w = O.qk_norm_rope_forward(f32(p.q), f32(wq), pos)
    kh_w = O.qk_norm_rope_forward(f32(p.k), f32(wk), pos)
    Ow, _ = O.attention_forward(qh_w, kh_w, f32(p.v), res.blk_idx, cu, s)
    dQh, dKh, dVw = O.attention_backward(qh_w, kh_w, f32(p.v), f32(p.do), res.blk_idx, cu, s)
    dxq, dwq_w = O.qk_norm_rope_backward(f32(p.q), f32(wq), pos, dQh)
    dxk, dwk_w = O.qk_norm_rope_backward(f32(p.k), f32(wk), pos, dKh)
    eo = float(np.abs(f32(o) - Ow).max())
    print(f"[qk chain] O maxabs {eo:.2e}", flush=True)
    assert eo <= 2e-2
    check_grad("qk chain", "dq", f32(dq), dxq)
    check_grad("qk chain", "dk", f32(dk), dxk)
    check_grad("qk chain", "dv", f32(dv), dVw)
    check_grad("qk chain", "dw_q", dwq.cpu().numpy()[None], dwq_w[None])
    check_grad("qk chain", "dw_k", dwk.cpu().numpy()[None], dwk_w[None])
