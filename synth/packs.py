"""Seeded THD packs shaped like the workloads of the MiniMax-M3 pages.

The pages time the block-sparse attention and the indexer select on
"16k-token" and "32k-token" packs of one TP4 shard (16 query heads, one KV
head, head dim 128, 128-token blocks, top-16) -- radixark/miles PR #4581,
kernel-tuning commit message.  Sequences are packed token-major (THD,
``--qkv-format thd``; miles MiniMax-M3.1-Flash page, section 5.1).  The
pages do not publish their pack lengths, so packs are drawn here:

* lengths: ``numpy.random.default_rng(seed).integers(lo, hi, endpoint=True)``
  drawn until the running sum reaches the pack size, the last draw truncated
  so the pack is filled exactly;
* activations: one ``torch.Generator('cpu').manual_seed(seed)`` draws
  ``randn`` in fp32 in the fixed order q, k, v, idx_q, idx_k, dO, each cast to
  bf16; then the two gemma norm weights ``(0.1 * randn(128)).bf16()``.

The same tensors feed the oracle (upcast exactly to fp32/fp64) and the GPU.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np
import torch


@dataclass(frozen=True)
class PackConfig:
    name: str
    total: int                      # tokens in the pack
    lengths_lo: int                 # uniform length range (inclusive); lo == hi == total -> one sequence
    lengths_hi: int
    num_q_heads: int = 16
    num_kv_heads: int = 1
    head_dim: int = 128
    block_size: int = 128
    topk_blocks: int = 16
    description: str = ""


# The five workloads: a dense-equivalent single sequence, a single 8k
# sequence, the 16k headline pack, the 32k pack and the unsharded layer.
CONFIGS = {
    "dense1k": PackConfig("dense1k", 1024, 1024, 1024,
                          description="single 1024-token sequence; every causal block is selected"),
    "single8k": PackConfig("single8k", 8192, 8192, 8192,
                           description="single 8192-token sequence (64 blocks, 16 selected)"),
    "pack16k": PackConfig("pack16k", 16384, 1024, 8192,
                          description="16384-token THD pack, lengths U[1024, 8192]"),
    "pack32k": PackConfig("pack32k", 32768, 2048, 16384,
                          description="32768-token THD pack, lengths U[2048, 16384]"),
    "layer32k": PackConfig("layer32k", 32768, 32768, 32768, num_q_heads=64, num_kv_heads=4,
                           description="unsharded layer: one 32768-token sequence, 64 q / 4 kv / 4 index heads"),
    # Narrow-block variant (qwen3.8-next on the pages: 12 q / 1 kv head, head
    # dim 256, 4-token blocks, 16k-token packs).  The pages give no block count
    # per query; 512 blocks keep the 2048-key budget of the wide variant.
    "qsa16k": PackConfig("qsa16k", 16384, 1024, 8192, num_q_heads=12, num_kv_heads=1, head_dim=256,
                         block_size=4, topk_blocks=512,
                         description="16384-token THD pack, lengths U[1024, 8192], 12 q / 1 kv heads, "
                                     "D 256, 4-token blocks, 512 selected per query"),
}


def pack_lengths(total: int, lo: int, hi: int, seed: int) -> List[int]:
    """Sequence lengths of a pack: uniform draws until `total` is reached, last one truncated."""
    if lo == hi == total:
        return [total]
    rng = np.random.default_rng(seed)
    out: List[int] = []
    s = 0
    while s < total:
        x = int(rng.integers(lo, hi, endpoint=True))
        x = min(x, total - s)
        out.append(x)
        s += x
    return out


@dataclass
class Pack:
    """One synthetic pack.  Tensors are CPU bf16 (contiguous) unless noted."""
    lengths: List[int]
    cu_seqlens: torch.Tensor        # int32 [S+1]
    q: torch.Tensor                 # [T, Hq, D]
    k: torch.Tensor                 # [T, Hk, D]
    v: torch.Tensor                 # [T, Hk, D]
    idx_q: torch.Tensor             # [T, Hk, D]  (index head h selects for kv head h)
    idx_k: torch.Tensor             # [T, Hk, D]
    do: torch.Tensor                # [T, Hq, D]
    w_q: torch.Tensor               # [D] gemma weight, applied as (1 + w)
    w_k: torch.Tensor               # [D]
    num_q_heads: int
    num_kv_heads: int
    head_dim: int = 128
    block_size: int = 128
    topk_blocks: int = 16
    eps: float = 1e-6
    rope_base: float = 1e7
    rope_dims: int = 64
    seed: int = 0
    name: str = ""

    @property
    def total(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def max_seqlen(self) -> int:
        return max(self.lengths) if self.lengths else 0

    @property
    def softmax_scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))


def _draw(lengths: Sequence[int], hq: int, hk: int, d: int, seed: int,
          idx_k_heads: Optional[int] = None):
    T = int(sum(lengths))
    g = torch.Generator("cpu").manual_seed(seed)
    ikh = hk if idx_k_heads is None else idx_k_heads

    def rn(*shape):
        return torch.randn(*shape, generator=g, dtype=torch.float32).to(torch.bfloat16)

    q = rn(T, hq, d)
    k = rn(T, hk, d)
    v = rn(T, hk, d)
    idx_q = rn(T, hk, d)
    idx_k = rn(T, ikh, d)
    do = rn(T, hq, d)
    w_q = (0.1 * torch.randn(d, generator=g, dtype=torch.float32)).to(torch.bfloat16)
    w_k = (0.1 * torch.randn(d, generator=g, dtype=torch.float32)).to(torch.bfloat16)
    return q, k, v, idx_q, idx_k, do, w_q, w_k


def make_custom_pack(lengths: Sequence[int], num_q_heads: int = 16, num_kv_heads: int = 1,
                     seed: int = 0, head_dim: int = 128, block_size: int = 128,
                     topk_blocks: int = 16, name: str = "custom") -> Pack:
    lengths = [int(x) for x in lengths]
    cu = torch.tensor([0] + list(np.cumsum(lengths)), dtype=torch.int32)
    q, k, v, iq, ik, do, wq, wk = _draw(lengths, num_q_heads, num_kv_heads, head_dim, seed)
    return Pack(lengths=lengths, cu_seqlens=cu, q=q, k=k, v=v, idx_q=iq, idx_k=ik, do=do,
                w_q=wq, w_k=wk, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                head_dim=head_dim, block_size=block_size, topk_blocks=topk_blocks,
                seed=seed, name=name)


def make_pack(config: str, seed: int = 0) -> Pack:
    c = CONFIGS[config]
    lengths = pack_lengths(c.total, c.lengths_lo, c.lengths_hi, seed)
    p = make_custom_pack(lengths, c.num_q_heads, c.num_kv_heads, seed, c.head_dim,
                         c.block_size, c.topk_blocks, name=config)
    return p


def random_block_lists(cu_seqlens, num_kv_heads: int, block: int, topk: int, seed: int) -> np.ndarray:
    """Seeded block selections ``[T, Hk, topk]`` int32 for attention inputs.

    Query ``t`` at sequence-local position ``p`` owns block ``b = p // block``.
    With ``b + 1 <= topk`` it lists every block ``0..b``; otherwise its own
    block and ``topk - 1`` distinct blocks drawn uniformly from ``0..b-1``.
    Ids are sequence-local, ascending, ``-1`` padded.  The draws come from
    ``numpy.random.default_rng([seed, 7])``, one permutation per (token, head).
    """
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T = int(cu[-1])
    rng = np.random.default_rng([seed, 7])
    out = np.full((T, num_kv_heads, topk), -1, dtype=np.int32)
    for s in range(len(cu) - 1):
        for p in range(int(cu[s + 1] - cu[s])):
            t = int(cu[s]) + p
            b = p // block
            for h in range(num_kv_heads):
                if b + 1 <= topk:
                    out[t, h, :b + 1] = np.arange(b + 1)
                else:
                    ids = np.sort(np.concatenate([rng.permutation(b)[:topk - 1], [b]]))
                    out[t, h, :] = ids
    return out
