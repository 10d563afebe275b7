"""GPU parity at the benchmark's full sizes, in the launch configuration bench.py times.

For each workload (single 8k sequence, the 16k and 32k THD packs, the
unsharded 32k layer with 4 KV / index heads):
  * selection: every row of the GPU's msa_index_select against the oracle,
    exact except near ties (16th/17th scores within 1e-3 relative);
  * attention: the GPU runs forward + backward on the ORACLE's block ids over
    the whole pack; O, LSE and dQ are checked on sampled rows (sequence
    starts and ends, block edges, random rows), dK/dV on sampled key blocks
    (every query that selected the block recomputed by the oracle).
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import synth

pytestmark = pytest.mark.gpu

O_TOL, G_TOL, LSE_TOL, TIE = 2e-2, 1e-2, 1e-3, 1e-3


def f32(t):
    return t.float().cpu().numpy()


def say(*a):
    print(*a, flush=True)


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def sample_rows(lengths, rng, n_random=24):
    cu = np.concatenate([[0], np.cumsum(lengths)])
    rows = set()
    for s in range(len(lengths)):
        a, b = int(cu[s]), int(cu[s + 1])
        for p in (0, 1, 127, 128, 129, 2047, 2048, 2049, b - a - 1):
            if 0 <= p < b - a:
                rows.add(a + p)
    rows.update(int(x) for x in rng.integers(0, int(cu[-1]), n_random))
    return np.array(sorted(rows))


def sample_blocks(lengths, nkv, rng):
    """(seq, block, head) triples: the longest sequence's block 16 (first one
    chosen by top-k rather than by every later query), a middle block and its
    last (partial) block, and block 0 of the shortest sequence."""
    s = int(np.argmax(lengths))
    nb = (lengths[s] + 127) // 128
    h = int(rng.integers(0, nkv))
    out = [(s, min(16, nb - 1), h), (s, nb // 2, h), (s, nb - 1, h)]
    if len(lengths) > 1:
        out.append((int(np.argmin(lengths)), 0, h))
    return out


@pytest.mark.parametrize("config", ["single8k", "pack16k", "pack32k", "layer32k"])
def test_fullsize_parity(gpu_lib, config):
    msa = gpu_lib
    rng = np.random.default_rng(2024)
    p = synth.make_pack(config, 0)
    say(f"[{config}] lengths {p.lengths} heads {p.num_q_heads}/{p.num_kv_heads}")
    cu_np = p.cu_seqlens.numpy()
    dev = torch.device("cuda:0")
    g = lambda t: t.to(dev)

    # selection, every row
    res = O.index_select(f32(p.idx_q), f32(p.idx_k), f32(p.w_q), f32(p.w_k), cu_np)
    blk_gpu = msa.msa_index_select(g(p.idx_q), g(p.idx_k), g(p.w_q), g(p.w_k), g(p.cu_seqlens),
                                   p.max_seqlen).cpu().numpy()
    diff = (blk_gpu != res.blk_idx).any(axis=2)
    tie = res.near_tie(TIE)
    say(f"[{config}] select rows={diff.size} near-tie={int(tie.sum())} mismatch-in-ties={int((diff & tie).sum())} "
        f"mismatch-outside={int((diff & ~tie).sum())}")
    assert (diff & ~tie).sum() == 0

    # attention on the oracle's ids, whole pack, bench launch configuration
    blk = g(torch.from_numpy(res.blk_idx))
    cu = g(p.cu_seqlens)
    q, k, v, do = g(p.q), g(p.k), g(p.v), g(p.do)
    o, lse = msa.msa_attn_fwd(q, k, v, blk, cu, p.max_seqlen)
    dq, dk, dv = msa.msa_attn_bwd(q, k, v, o, lse, do, blk, cu, p.max_seqlen)
    torch.cuda.synchronize()
    qn, kn, vn, don = f32(p.q), f32(p.k), f32(p.v), f32(p.do)
    scale = 1 / math.sqrt(128)

    rows = sample_rows(p.lengths, rng)
    Ow, Lw = O.attention_forward(qn, kn, vn, res.blk_idx, cu_np, scale, rows=rows)
    dQw, _, _ = O.attention_backward(qn, kn, vn, don, res.blk_idx, cu_np, scale, rows=rows)
    eo = float(np.abs(f32(o)[rows] - Ow).max())
    el = float(np.abs(lse.cpu().numpy()[rows] - Lw).max())
    rq = rel(f32(dq)[rows], dQw)
    say(f"[{config}] {len(rows)} rows: O maxabs={eo:.3e} LSE maxabs={el:.3e} dQ rel={rq:.3e}")
    assert eo <= O_TOL and el <= LSE_TOL and rq <= G_TOL

    dkn, dvn = f32(dk), f32(dv)
    for (s, c, h) in sample_blocks(p.lengths, p.num_kv_heads, rng):
        sel = O.selectors_of_block(res.blk_idx, cu_np, s, c, h)
        _, dKw, dVw = O.attention_backward(qn, kn, vn, don, res.blk_idx, cu_np, scale, rows=sel, heads=[h])
        a = int(cu_np[s]) + 128 * c
        b = min(a + 128, int(cu_np[s + 1]))
        rk = rel(dkn[a:b, h], dKw[a:b, h])
        rv = rel(dvn[a:b, h], dVw[a:b, h])
        say(f"[{config}] block (seq {s}, {c}, head {h}): {len(sel)} selecting queries, dK rel={rk:.3e} dV rel={rv:.3e}")
        assert rk <= G_TOL and rv <= G_TOL
