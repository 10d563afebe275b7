"""The allocation-free forward (msa_attn_fwd_noalloc: the forward's workspace in
the library's static device scratch) against msa_attn_fwd with a caller
workspace, through the C ABI: bitwise equal O and LSE on two calls in a row,
the second on a smaller pack (the scratch keeps the first call's contents).
Run it alone in a fresh process or after the other GPU tests."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def blocks(p, rng):
    """Seeded block lists: the own block plus up to 15 random earlier blocks."""
    cu = p.cu_seqlens.numpy()
    blk = np.full((p.total, p.num_kv_heads, 16), -1, np.int32)
    for s in range(len(cu) - 1):
        for t in range(int(cu[s]), int(cu[s + 1])):
            b = (t - int(cu[s])) // 128
            for h in range(p.num_kv_heads):
                ids = sorted([b] + [int(x) for x in rng.permutation(b)[:15]])
                blk[t, h, :len(ids)] = ids
    return blk


def test_noalloc_forward_matches_workspace_forward(gpu_lib):
    msa = gpu_lib
    rng = np.random.default_rng(91)
    big = synth.make_custom_pack([3100, 2200, 700], num_q_heads=32, num_kv_heads=2, seed=91)
    small = synth.make_custom_pack([900, 130, 1], num_q_heads=32, num_kv_heads=2, seed=92)
    dev = lambda t: t.to("cuda")
    for p in (big, small):
        blk = dev(torch.from_numpy(blocks(p, rng)))
        cu = dev(p.cu_seqlens)
        q, k, v = dev(p.q), dev(p.k), dev(p.v)
        o_ref, lse_ref = msa.msa_attn_fwd(q, k, v, blk, cu, p.max_seqlen)
        torch.cuda.synchronize()
        o = torch.full_like(o_ref, 7.0)
        lse = torch.full_like(lse_ref, 7.0)
        msa.msa_attn_fwd_noalloc(q, k, v, blk, cu, p.max_seqlen, out=o, lse=lse)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), p.lengths
        assert torch.equal(lse, lse_ref), p.lengths
        print(f"[noalloc {p.lengths}] O and LSE bitwise equal to the workspace forward", flush=True)


def test_noalloc_rejects_a_pack_beyond_the_scratch(gpu_lib):
    msa = gpu_lib
    dims = msa.make_dims(131072, 1, 131072, 32, 2)          # 2 x 1024 blocks: 128 MiB of staging copies
    assert msa.msa_workspace_size(dims, msa.MSA_OP_FWD) > msa.MSA_NOALLOC_SCRATCH_BYTES
    st = msa.load().msa_attn_fwd_noalloc(dims, None, 0, 0, None, 0, 0, None, 0, 0, None, None, 0.1, None, 0, 0,
                                         None, None)
    assert st == msa.MSA_ERR_WORKSPACE
