"""GPU parity of the narrow-block variant (4-token blocks, head dim 256, 12 q
heads per KV head) through the C ABI (msa_qsa_attn_fwd / msa_qsa_attn_bwd)
against the CPU oracle (the same attention functions with block=4).

Tolerances as for the wide variant (tests/parity.py): O max-abs <= 2e-2, LSE
max-abs <= 1e-3, dQ, dK, dV relative Frobenius error <= 1e-2 per tensor plus a
per-row and a max-abs bound.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import synth
from parity import check_grad, check_out, say

pytestmark = pytest.mark.gpu

SCALE = 1 / math.sqrt(256)


def f32(t):
    return t.float().cpu().numpy()


def dev(t):
    return t.to("cuda")


def pack(lengths, hk, topk, seed):
    p = synth.make_custom_pack(lengths, num_q_heads=12 * hk, num_kv_heads=hk, seed=seed, head_dim=256,
                               block_size=4, topk_blocks=topk)
    blk = synth.random_block_lists(p.cu_seqlens.numpy(), hk, 4, topk, seed)
    return p, blk


def run(msa, p, blk_np):
    cu = dev(p.cu_seqlens)
    q, k, v, do = dev(p.q), dev(p.k), dev(p.v), dev(p.do)
    blk = dev(torch.from_numpy(np.ascontiguousarray(blk_np)))
    o, lse = msa.msa_qsa_attn_fwd(q, k, v, blk, cu, p.max_seqlen)
    dq, dk, dv = msa.msa_qsa_attn_bwd(q, k, v, o, lse, do, blk, cu, p.max_seqlen)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


def check_full(p, blk_np, out, label):
    o, lse, dq, dk, dv = out
    cu = p.cu_seqlens.numpy()
    Ow, Lw = O.attention_forward(f32(p.q), f32(p.k), f32(p.v), blk_np, cu, SCALE, block=4)
    dQw, dKw, dVw = O.attention_backward(f32(p.q), f32(p.k), f32(p.v), f32(p.do), blk_np, cu, SCALE, block=4)
    check_out(label, f32(o), Ow, lse.cpu().numpy(), Lw)
    check_grad(label, "dQ", f32(dq), dQw)
    check_grad(label, "dK", f32(dk), dKw)
    check_grad(label, "dV", f32(dv), dVw)


def test_qsa_dense_equality(gpu_lib):
    """64 blocks of 4 per query: sequences of at most 256 tokens attend to every causal key."""
    p, blk = pack([200, 56, 9], 1, 64, 51)
    assert (blk >= 0).sum(axis=2).max() <= 64
    out = run(gpu_lib, p, blk)
    check_full(p, blk, out, "qsa dense")
    # and the oracle with all blocks listed is dense causal attention (pinned on the CPU)
    seq, pos = O.sequence_layout(p.cu_seqlens.numpy())
    for t in range(0, len(seq), 17):
        assert list(blk[t, 0, :pos[t] // 4 + 1]) == list(range(pos[t] // 4 + 1))


@pytest.mark.parametrize("lengths,hk,topk,seed", [
    ([700, 1, 63, 65, 300], 1, 64, 52),   # ragged, 1-token and tile-edge sequences, tiles spanning sequences
    ([900, 500], 2, 32, 53),              # two KV heads, sparser lists
    ([1500], 1, 200, 54),                 # many key tiles in one sequence
])
def test_qsa_parity_sparse(gpu_lib, lengths, hk, topk, seed):
    p, blk = pack(lengths, hk, topk, seed)
    check_full(p, blk, run(gpu_lib, p, blk), f"qsa {lengths} hk={hk} K={topk}")


def test_qsa_unsorted_duplicate_and_foreign_ids(gpu_lib):
    """Lists in any order, with duplicates, -1 holes, ids past the own block and rows
    without their own block: the oracle's key set semantics (listed causal keys, once)."""
    p, blk = pack([600, 333], 1, 48, 55)
    rng = np.random.default_rng(56)
    seq, pos = O.sequence_layout(p.cu_seqlens.numpy())
    blk = blk.copy()
    for t in range(blk.shape[0]):
        row = blk[t, 0]
        r = rng.random()
        n = int((row >= 0).sum())
        if r < 0.2 and n > 2:
            row[1] = row[2]                                  # duplicate
        elif r < 0.4:
            row[-1] = pos[t] // 4 + 1 + int(rng.integers(0, 500))  # past the own block
        elif r < 0.5 and n > 1:
            row[row == pos[t] // 4] = -1                     # own block missing
        blk[t, 0] = rng.permutation(row)
    check_full(p, blk, run(gpu_lib, p, blk), "qsa junk lists")


def test_qsa_fullsize_sampled(gpu_lib):
    """The 16k benchmark pack (12 q / 1 kv, D 256, 512 blocks of 4 per query): sampled rows of
    O, LSE and dQ, and dK/dV of two key tiles (all their selecting queries) against the oracle."""
    p = synth.make_pack("qsa16k", 0)
    cu = p.cu_seqlens.numpy()
    blk = synth.random_block_lists(cu, 1, 4, 512, 0)
    o, lse, dq, dk, dv = run(gpu_lib, p, blk)
    seq, pos = O.sequence_layout(cu)
    rng = np.random.default_rng(57)
    rows = np.unique(np.concatenate([rng.integers(0, p.total, 40), cu[1:-1], cu[1:-1] - 1, [p.total - 1]]))
    q, k, v, do = f32(p.q), f32(p.k), f32(p.v), f32(p.do)
    Ow, Lw = O.attention_forward(q, k, v, blk, cu, SCALE, block=4, rows=rows)
    dQw, _, _ = O.attention_backward(q, k, v, do, blk, cu, SCALE, block=4, rows=rows)
    label = f"qsa16k rows={len(rows)}"
    check_out(label, f32(o)[rows], Ow, lse.cpu().numpy()[rows], Lw)
    check_grad(label, "dQ", f32(dq)[rows], dQw)
    # dK / dV of key tile c of sequence s come from every query that listed one of its blocks
    for s, c in [(0, 37), (2, 0)]:
        a, b = int(cu[s]), int(cu[s + 1])
        lo, hi = a + 64 * c, min(a + 64 * c + 64, b)
        tile_blocks = np.arange(16 * c, 16 * c + 16)
        sel = a + np.nonzero(np.isin(blk[a:b, 0, :], tile_blocks).any(axis=1))[0]
        _, dKw, dVw = O.attention_backward(q, k, v, do, blk, cu, SCALE, block=4, rows=sel)
        label = f"qsa16k key tile s={s} c={c} selectors={len(sel)}"
        check_grad(label, "dK", f32(dk)[lo:hi], dKw[lo:hi])
        check_grad(label, "dV", f32(dv)[lo:hi], dVw[lo:hi])


def test_qsa_deterministic(gpu_lib):
    p, blk = pack([800, 200], 1, 64, 58)
    a = run(gpu_lib, p, blk)
    b = run(gpu_lib, p, blk)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_qsa_empty_sequences_inside_a_pack(gpu_lib):
    """Zero-length sequences between ragged ones (repeated cu_seqlens entries)."""
    p, blk = pack([0, 300, 0, 5, 0, 130], 1, 40, 59)
    check_full(p, blk, run(gpu_lib, p, blk), "qsa empty sequences")


def test_qsa_empty_pack_is_a_noop(gpu_lib):
    cu = torch.zeros(1, dtype=torch.int32, device="cuda")
    z = torch.empty(0, 12, 256, dtype=torch.bfloat16, device="cuda")
    zk = torch.empty(0, 1, 256, dtype=torch.bfloat16, device="cuda")
    blk = torch.empty(0, 1, 8, dtype=torch.int32, device="cuda")
    o, lse = gpu_lib.msa_qsa_attn_fwd(z, zk, zk, blk, cu, 1)
    dq, dk, dv = gpu_lib.msa_qsa_attn_bwd(z, zk, zk, o, lse, z, blk, cu, 1)
    torch.cuda.synchronize()
    assert o.numel() == 0 and dq.numel() == 0


def test_qsa_longest_sequence_most_blocks(gpu_lib):
    """One 32768-token sequence (the narrow entry points' limit) with 1024 listed blocks per
    query (the K limit): sampled rows of O, LSE and dQ, and dK/dV of the last key tile."""
    p = synth.make_custom_pack([32768], num_q_heads=12, num_kv_heads=1, seed=60, head_dim=256, block_size=4,
                               topk_blocks=1024)
    cu = p.cu_seqlens.numpy()
    blk = synth.random_block_lists(cu, 1, 4, 1024, 60)
    o, lse, dq, dk, dv = run(gpu_lib, p, blk)
    rows = np.array([0, 63, 64, 4095, 4096, 16383, 32703, 32704, 32767] +
                    list(np.random.default_rng(61).integers(0, 32768, 8)))
    q, k, v, do = f32(p.q), f32(p.k), f32(p.v), f32(p.do)
    Ow, Lw = O.attention_forward(q, k, v, blk, cu, SCALE, block=4, rows=rows)
    dQw, _, _ = O.attention_backward(q, k, v, do, blk, cu, SCALE, block=4, rows=rows)
    check_out("qsa 32768 K=1024", f32(o)[rows], Ow, lse.cpu().numpy()[rows], Lw)
    check_grad("qsa 32768 K=1024", "dQ (sampled rows)", f32(dq)[rows], dQw)
    last = np.arange(32704, 32768)
    sel = np.nonzero(np.isin(blk[:, 0, :], np.arange(8176, 8192)).any(axis=1))[0]
    _, dKw, dVw = O.attention_backward(q, k, v, do, blk, cu, SCALE, block=4, rows=sel)
    check_grad(f"qsa 32768 K=1024 last tile ({len(sel)} selectors)", "dK", f32(dk)[last], dKw[last])
    check_grad(f"qsa 32768 K=1024 last tile ({len(sel)} selectors)", "dV", f32(dv)[last], dVw[last])
