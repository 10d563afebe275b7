"""GPU: the forward's two tiles give the same results.

Sparse layers whose longest sequence is at least 12288 tokens (the max_seqlen
bound) run the forward on 32-token tiles of 8 wavefronts x 4 tokens, shorter
ones on 16-token tiles of one token per wavefront.  Each token meets its
selected blocks in ascending order either way, so O and LSE must be bitwise
equal.  The packs hold at least 12288 tokens of short sequences (the bound
may not exceed the pack), so the same call with max_seqlen 12288 (which
only sizes grids and workspaces) runs the wide tile; the oracle checks
sampled rows, every row of the last (ragged) tile and a one-token sequence.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import synth
from parity import check_out

pytestmark = pytest.mark.gpu

WIDE_BOUND = 12288


def f32(t):
    return t.float().cpu().numpy()


def random_blocks(cu, hk, rng):
    """Own block plus up to 15 random earlier blocks, ascending."""
    _, pos = O.sequence_layout(cu)
    T = len(pos)
    blk = np.full((T, hk, 16), -1, np.int32)
    for t in range(T):
        b = int(pos[t]) // 128
        for h in range(hk):
            ids = sorted([b] + [int(x) for x in rng.permutation(b)[:15]])
            blk[t, h, :len(ids)] = ids
    return blk


@pytest.mark.parametrize("lengths,hk,seed", [([3000, 37, 1, 2600, 1111, 5611, 11], 1, 61),
                                             ([4099, 700, 7500], 2, 62)])
def test_wide_tile_bitwise_equal_and_oracle(gpu_lib, lengths, hk, seed):
    msa = gpu_lib
    p = synth.make_custom_pack(lengths, num_q_heads=16 * hk, num_kv_heads=hk, seed=seed)
    cu = p.cu_seqlens.numpy()
    rng = np.random.default_rng(seed)
    blk_np = random_blocks(cu, hk, rng)
    dev = torch.device("cuda:0")
    g = lambda t: t.to(dev)
    blk = g(torch.from_numpy(blk_np))
    q, k, v, cu_d = g(p.q), g(p.k), g(p.v), g(p.cu_seqlens)
    o16, l16 = msa.msa_attn_fwd(q, k, v, blk, cu_d, p.max_seqlen)
    o32, l32 = msa.msa_attn_fwd(q, k, v, blk, cu_d, max(WIDE_BOUND, p.max_seqlen))
    torch.cuda.synchronize()
    assert p.max_seqlen < WIDE_BOUND
    assert torch.equal(o16.view(torch.int16), o32.view(torch.int16))
    assert torch.equal(l16.view(torch.int32), l32.view(torch.int32))
    T = int(cu[-1])
    rows = set(int(x) for x in rng.integers(0, T, 48))
    rows.update(range(T - (T % 32 or 32), T))          # the last 32-token tile
    rows.update(int(c) for c in cu[:-1])               # every sequence's first token
    rows.update(int(c) - 1 for c in cu[1:])            # and its last
    rows = np.array(sorted(rows))
    Ow, Lw = O.attention_forward(f32(p.q), f32(p.k), f32(p.v), blk_np, cu, 1 / math.sqrt(128), rows=rows)
    check_out(f"wide tile {lengths} hk={hk}", f32(o32)[rows], Ow, l32.cpu().numpy()[rows], Lw)
