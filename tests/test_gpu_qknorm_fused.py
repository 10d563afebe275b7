"""The attention entry points with the attention-side q/k norm + partial RoPE
fused in (msa_attn_fwd_qknorm / msa_attn_bwd_qknorm) against the oracle's
chain: norm + RoPE of the raw q, k (miles docs "MiniMax-M3.1-Flash",
section 1), block-sparse attention forward/backward on the result, and the
norm's backward for dq, dk, dw_q, dw_k.  Tolerances as for the separate
passes (tests/test_gpu_qk_norm.py)."""
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


def inputs(lengths, hk, seed):
    p = synth.make_custom_pack(lengths, num_q_heads=16 * hk, num_kv_heads=hk, seed=seed)
    g = torch.Generator().manual_seed(seed + 1000)
    wq = (0.1 * torch.randn(128, generator=g)).bfloat16()
    wk = (0.1 * torch.randn(128, generator=g)).bfloat16()
    return p, wq, wk


def all_blocks(cu, hk):
    seq, pos = O.sequence_layout(cu)
    nb = int(pos.max()) // 128 + 1
    blk = np.full((len(seq), hk, nb), -1, np.int32)
    for t in range(len(seq)):
        blk[t, :, :pos[t] // 128 + 1] = np.arange(pos[t] // 128 + 1)
    return blk


@pytest.mark.parametrize("lengths,hk,seed,dense", [([2600, 600], 1, 81, False), ([1900, 130, 1], 2, 82, False),
                                                  ([2300, 700], 1, 83, True)])
def test_fused_norm_attention_matches_oracle_chain(gpu_lib, lengths, hk, seed, dense):
    msa = gpu_lib
    p, wq, wk = inputs(lengths, hk, seed)
    cu = p.cu_seqlens.numpy()
    _, pos = O.sequence_layout(cu)
    if dense:
        blk_np = all_blocks(cu, hk)
        blk = None
    else:
        res = O.index_select(f32(p.idx_q), f32(p.idx_k), f32(p.w_q), f32(p.w_k), cu)
        blk_np = res.blk_idx
        blk = dev(torch.from_numpy(blk_np))
    cud = dev(p.cu_seqlens)
    q, k, v, do = dev(p.q), dev(p.k), dev(p.v), dev(p.do)
    o, lse = msa.msa_attn_fwd_qknorm(q, k, v, dev(wq), dev(wk), blk, cud, p.max_seqlen, dense=dense)
    dq, dk, dv, dwq, dwk = msa.msa_attn_bwd_qknorm(q, k, v, dev(wq), dev(wk), o, lse, do, blk, cud, p.max_seqlen,
                                                   dense=dense)
    torch.cuda.synchronize()
    s = 1 / math.sqrt(128)
    qh_w = O.qk_norm_rope_forward(f32(p.q), f32(wq), pos)
    kh_w = O.qk_norm_rope_forward(f32(p.k), f32(wk), pos)
    Ow, Lw = O.attention_forward(qh_w, kh_w, f32(p.v), blk_np, cu, s)
    dQh, dKh, dVw = O.attention_backward(qh_w, kh_w, f32(p.v), f32(p.do), blk_np, cu, s)
    dxq, dwq_w = O.qk_norm_rope_backward(f32(p.q), f32(wq), pos, dQh)
    dxk, dwk_w = O.qk_norm_rope_backward(f32(p.k), f32(wk), pos, dKh)
    eo = float(np.abs(f32(o) - Ow).max())
    el = float(np.abs(lse.cpu().numpy() - Lw).max())
    r = (rel(f32(dq), dxq), rel(f32(dk), dxk), rel(f32(dv), dVw), rel(dwq.cpu().numpy(), dwq_w),
         rel(dwk.cpu().numpy(), dwk_w))
    print(f"[fused qknorm {lengths} hk={hk} dense={dense}] O maxabs {eo:.2e} LSE maxabs {el:.2e} dq {r[0]:.2e} "
          f"dk {r[1]:.2e} dv {r[2]:.2e} dw_q {r[3]:.2e} dw_k {r[4]:.2e}", flush=True)
    assert eo <= 2e-2 and el <= 1e-3
    label = f"fused qknorm {lengths} hk={hk} dense={dense}"
    check_grad(label, "dq", f32(dq), dxq)
    check_grad(label, "dk", f32(dk), dxk)
    check_grad(label, "dv", f32(dv), dVw)
    check_grad(label, "dw_q", dwq.cpu().numpy()[None], dwq_w[None])
    check_grad(label, "dw_k", dwk.cpu().numpy()[None], dwk_w[None])


def test_fused_forward_matches_separate_passes(gpu_lib):
    """The fused forward against msa_qk_norm_rope_fwd followed by msa_attn_fwd on the GPU: the normalized q
    and k may differ in the last bf16 bit where the 128-term sums of squares round differently, so the
    outputs agree to well inside the oracle tolerance rather than bitwise."""
    msa = gpu_lib
    p, wq, wk = inputs([3000, 900], 1, 84)
    cu = p.cu_seqlens.numpy()
    res = O.index_select(f32(p.idx_q), f32(p.idx_k), f32(p.w_q), f32(p.w_k), cu)
    blk = dev(torch.from_numpy(res.blk_idx))
    cud = dev(p.cu_seqlens)
    q, k, v = dev(p.q), dev(p.k), dev(p.v)
    o1, l1 = msa.msa_attn_fwd_qknorm(q, k, v, dev(wq), dev(wk), blk, cud, p.max_seqlen)
    qh, kh = msa.msa_qk_norm_rope_fwd(q, k, dev(wq), dev(wk), cud, p.max_seqlen)
    o2, l2 = msa.msa_attn_fwd(qh, kh, v, blk, cud, p.max_seqlen)
    torch.cuda.synchronize()
    do_ = float((o1.float() - o2.float()).abs().max())
    dl = float((l1 - l2).abs().max())
    same = float((o1 == o2).float().mean())
    print(f"[fused vs separate] O maxabs {do_:.2e} LSE maxabs {dl:.2e} identical O {same:.4f}", flush=True)
    assert do_ <= 5e-3 and dl <= 2e-4 and same >= 0.95


def test_fused_empty_pack_zero_weight_gradients(gpu_lib):
    z = torch.zeros(0, 16, 128, dtype=torch.bfloat16, device="cuda")
    z1 = torch.zeros(0, 1, 128, dtype=torch.bfloat16, device="cuda")
    w = torch.zeros(128, dtype=torch.bfloat16, device="cuda")
    cu = torch.zeros(1, dtype=torch.int32, device="cuda")
    blk = torch.zeros(0, 1, 16, dtype=torch.int32, device="cuda")
    lse = torch.zeros(0, 16, dtype=torch.float32, device="cuda")
    gpu_lib.msa_attn_fwd_qknorm(z, z1, z1, w, w, blk, cu, 1)
    *_, dwq, dwk = gpu_lib.msa_attn_bwd_qknorm(z, z1, z1, w, w, z, lse, z, blk, cu, 1)
    torch.cuda.synchronize()
    assert dwq.abs().sum().item() == 0 and dwk.abs().sum().item() == 0


def test_fused_backward_matches_separate_passes_and_repeats(gpu_lib):
    """The fused backward (norm in the prep and dQ kernels, dq taken back through the norm in the dQ
    epilogue) against msa_qk_norm_rope_fwd, msa_attn_bwd and msa_qk_norm_rope_bwd run one after another on
    the GPU, on q and k views with padded strides: the normalized rows may differ in the last bf16 bit
    (sum-of-squares order) and the fused dq skips one bf16 rounding of dq_hat, so they agree well inside the
    oracle tolerance.  A second call gives bitwise the same gradients (fixed-order sums)."""
    msa = gpu_lib
    p, wq, wk = inputs([2700, 520, 77], 2, 85)
    cu = p.cu_seqlens.numpy()
    res = O.index_select(f32(p.idx_q), f32(p.idx_k), f32(p.w_q), f32(p.w_k), cu)
    blk = dev(torch.from_numpy(res.blk_idx))
    cud = dev(p.cu_seqlens)
    T = p.q.shape[0]
    qpad = torch.zeros(T, 32, 160, dtype=torch.bfloat16, device="cuda")
    kpad = torch.zeros(T, 2, 192, dtype=torch.bfloat16, device="cuda")
    qpad[:, :, 16:144] = dev(p.q)
    kpad[:, :, 64:192] = dev(p.k)
    q, k = qpad[:, :, 16:144], kpad[:, :, 64:192]
    v, do = dev(p.v), dev(p.do)
    wqd, wkd = dev(wq), dev(wk)
    o, lse = msa.msa_attn_fwd_qknorm(q, k, v, wqd, wkd, blk, cud, p.max_seqlen)
    g1 = msa.msa_attn_bwd_qknorm(q, k, v, wqd, wkd, o, lse, do, blk, cud, p.max_seqlen)
    g2 = msa.msa_attn_bwd_qknorm(q, k, v, wqd, wkd, o, lse, do, blk, cud, p.max_seqlen)
    qh, kh = msa.msa_qk_norm_rope_fwd(q.contiguous(), k.contiguous(), wqd, wkd, cud, p.max_seqlen)
    dqh, dkh, dv_s = msa.msa_attn_bwd(qh, kh, v, o, lse, do, blk, cud, p.max_seqlen)
    dq_s, dk_s, dwq_s, dwk_s = msa.msa_qk_norm_rope_bwd(q.contiguous(), k.contiguous(), wqd, wkd, cud,
                                                        p.max_seqlen, dqh, dkh)
    torch.cuda.synchronize()
    repeat = all(torch.equal(a, b) for a, b in zip(g1, g2))
    r = [rel(f32(a), f32(b)) for a, b in zip(g1, (dq_s, dk_s, dv_s, dwq_s, dwk_s))]
    print(f"[fused vs separate bwd] dq {r[0]:.2e} dk {r[1]:.2e} dv {r[2]:.2e} dw_q {r[3]:.2e} dw_k {r[4]:.2e} "
          f"repeat bitwise {repeat}", flush=True)
    assert repeat
    assert max(r[:3]) <= 5e-3 and max(r[3:]) <= 1e-2
