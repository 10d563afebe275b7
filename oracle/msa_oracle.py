"""Plain CPU oracle of the MSA block-sparse attention hot path.

TEST INFRASTRUCTURE ONLY.  This module states, slowly and in the order the
pages describe it, what the MSA path computes.  Only the tests, the
``smoke()`` check and the ``cpu_baseline`` leg of the benchmark may import it.
It shares no code, header, table or helper with the HIP library, and the
library never calls it.

Sources (cited by page and section; the pages are the authority):

* [M31] miles docs, "MiniMax-M3.1-Flash", section 1 (Model Introduction):
  a 4-head indexer of dim 128 with its own gemma q/k norm and RoPE scores
  every causal 128-token block by its maximum logit; each query attends to
  the 16 best blocks, its own block always included; index head h selects
  the blocks for KV head h; attention is GQA with RoPE on the first 64 of
  128 dims, base 1e7.  Section 5.1: sparse attention runs on THD packs.
  Section 5.4: the indexer is frozen (no gradient flows into it).
* [PR] radixark/miles PR #4581, kernel-tuning commit message and PR body:
  per-block max-logit scores, then rules and top-k; block-sparse attention
  forward and backward (dK/dV split over a KV head's query heads, summed).
* [MB] NVIDIA Megatron-Bridge, "MiniMax-M3", Architecture Notes: gemma-style
  RMSNorm ``x * (1 + w)``; partial RoPE on 64 of 128 channels.  Known
  Limitations: top-k blocks times block size is 2048 keys, so full causal
  attention is identical up to that length.

Readings where the pages are silent (each is listed with its reason in the
design notes of the repository):

* the norm is ``y = x * 1/sqrt(mean(x^2) + eps) * (1 + w)`` over the 128 dims
  of one head, eps = 1e-6, one [128] weight for q and one for k;
* RoPE is rotate-half on dims 0..63 with pairs (i, i+32) and angle
  ``p * base**(-2i/64)`` at the sequence-local position p;
* the indexer features are rounded once to bf16 (round to nearest even)
  after the fp32 norm and RoPE; the maximum logit is the plain dot product of
  those bf16 vectors (no scale, no ReLU, no head weights);
* a query in block b with b + 1 <= 16 takes all of blocks 0..b; otherwise its
  own block plus the 15 best of blocks 0..b-1, higher score first and the
  lower block id first on equal scores; ids are returned ascending, padded
  with -1;
* the optional forced initial block (the "init" of the pages' init/local/
  causal rules) keeps block 0 as well, leaving 14 slots for the best of
  blocks 1..b-1;
* attention keys for query i are the keys j <= i of its selected blocks in
  its own sequence; softmax scale 1/sqrt(128); query head g uses KV head
  g // (Hq / Hk);
* the narrow-block variant ([PR] kernel-tuning commit message: the same
  block-sparse kernel with 4-token blocks, head dim 256, 12 query heads per
  KV head) is the same attention with ``block=4``; the pages give neither its
  block count per query nor how its blocks are chosen, so its block lists
  are inputs (512 per query in the benchmark: the wide variant's 2048-key
  budget), and its softmax scale is 1/sqrt(256).

Precision.  The norm and RoPE run in fp32 with angles, cos and sin taken in
fp64 and rounded to fp32, because the bf16 rounding of the features is a
quantisation both sides must take in the same precision.  Block scores are
the exact dot products of the bf16 features (fp64 sums), rounded once to
fp32, and ranked in fp32.  Attention forward and backward run in fp64.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

F32 = np.float32
F64 = np.float64


# ---------------------------------------------------------------------------
# THD layout  ([M31] section 5.1: variable-length sequences packed token-major)
# ---------------------------------------------------------------------------

def sequence_layout(cu_seqlens: Sequence[int]) -> Tuple[np.ndarray, np.ndarray]:
    """Per-token sequence id and sequence-local position.

    ``cu_seqlens`` holds S+1 offsets starting at 0; token t belongs to the
    sequence s with cu[s] <= t < cu[s+1] and sits at position t - cu[s].
    Positions (and therefore blocks) restart with every sequence.
    """
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T = int(cu[-1])
    seq = np.empty(T, dtype=np.int64)
    pos = np.empty(T, dtype=np.int64)
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        seq[a:b] = s
        pos[a:b] = np.arange(b - a)
    return seq, pos


# ---------------------------------------------------------------------------
# bf16 rounding
# ---------------------------------------------------------------------------

def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 value (ties to even); returns fp32.

    bf16 keeps the upper 16 bits of an fp32 word.  Rounding adds half of the
    dropped range, plus one when the kept part is odd (ties to even).
    """
    x = np.ascontiguousarray(x, dtype=F32)
    u = x.view(np.uint32).astype(np.uint64)
    keep_odd = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + keep_odd) & np.uint64(0xFFFF0000)
    out = r.astype(np.uint32).view(F32).copy()
    nan = np.isnan(x)
    out[nan] = x[nan]
    return out


# ---------------------------------------------------------------------------
# Indexer prologue: gemma RMSNorm then partial rotate-half RoPE
# ([M31] section 1: "its own gemma q/k norm and RoPE"; [MB] Architecture Notes)
# ---------------------------------------------------------------------------

def gemma_rmsnorm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """Gemma-style RMSNorm in fp32: ``(x * 1/sqrt(mean(x^2) + eps)) * (1 + w)``.

    The mean runs over the last axis (one head's 128 dims).  Every operation
    is a separately rounded fp32 operation in the order written.
    """
    x = np.asarray(x, dtype=F32)
    w = np.asarray(w, dtype=F32)
    ms = (x * x).sum(axis=-1, dtype=F32) / F32(x.shape[-1])
    r = F32(1.0) / np.sqrt(ms + F32(eps))
    return (x * r[..., None]) * (F32(1.0) + w)


def rope_cos_sin(pos: np.ndarray, base: float, rope_dims: int) -> Tuple[np.ndarray, np.ndarray]:
    """cos and sin of the rotary angles, in fp64 then rounded to fp32.

    Pair i (0 <= i < rope_dims/2) turns by ``p * base**(-2i/rope_dims)`` at
    position p.
    """
    half = rope_dims // 2
    i = np.arange(half, dtype=F64)
    inv_freq = np.power(F64(base), -(2.0 * i) / F64(rope_dims))
    theta = np.asarray(pos, dtype=F64)[:, None] * inv_freq[None, :]
    return np.cos(theta).astype(F32), np.sin(theta).astype(F32)


def rope_rotate_half(y: np.ndarray, pos: np.ndarray, base: float, rope_dims: int) -> np.ndarray:
    """Rotate-half RoPE on dims [0, rope_dims) of the last axis; the rest pass through.

    With h = rope_dims/2: out[i] = y[i]*cos - y[i+h]*sin and
    out[i+h] = y[i+h]*cos + y[i]*sin, every product and sum rounded in fp32.
    ``y`` is [N, ..., D] with ``pos`` of length N.
    """
    y = np.asarray(y, dtype=F32)
    half = rope_dims // 2
    c, s = rope_cos_sin(pos, base, rope_dims)
    shape = (y.shape[0],) + (1,) * (y.ndim - 2) + (half,)
    c = c.reshape(shape)
    s = s.reshape(shape)
    y1 = y[..., :half]
    y2 = y[..., half:rope_dims]
    out = y.copy()
    out[..., :half] = (y1 * c) - (y2 * s)
    out[..., half:rope_dims] = (y2 * c) + (y1 * s)
    return out


def indexer_features(x: np.ndarray, w: np.ndarray, pos: np.ndarray, eps: float,
                     base: float, rope_dims: int, round_bf16: bool = True) -> np.ndarray:
    """Indexer q or k features: norm, RoPE, then one rounding to bf16.

    ``x`` is [N, H, D] (or [N, D]) fp32 holding bf16 values; returns fp32
    holding bf16 values (or the unrounded fp32 values with ``round_bf16=False``).
    """
    y = gemma_rmsnorm(x, w, eps)
    y = rope_rotate_half(y, pos, base, rope_dims)
    return round_to_bf16(y) if round_bf16 else y


# ---------------------------------------------------------------------------
# Per-block maximum logit  ([M31] section 1: "scores every causal 128-token
# block by its maximum logit"; [PR] per-block max-logit scores)
# ---------------------------------------------------------------------------

def block_max_scores(qf: np.ndarray, kf: np.ndarray, block: int,
                     rows: Optional[np.ndarray] = None, chunk: int = 512) -> np.ndarray:
    """Scores of one sequence and one index head.

    ``qf``, ``kf``: [L, D] features.  Returns fp32 [len(rows), n_blocks] with
    ``s[i, c] = max over keys j in block c with j <= i of qf[i] . kf[j]``,
    the dot products summed exactly (fp64) and rounded once to fp32, and -inf
    for blocks with no causal key (c > block of i).
    """
    L = qf.shape[0]
    nb = (L + block - 1) // block
    if rows is None:
        rows = np.arange(L)
    rows = np.asarray(rows, dtype=np.int64)
    out = np.full((len(rows), nb), -np.inf, dtype=F32)
    q64 = qf.astype(F64)
    k64 = kf.astype(F64)
    for a in range(0, len(rows), chunk):
        r = rows[a:a + chunk]
        hi = int(r.max()) + 1
        kb = (hi + block - 1) // block
        S = q64[r] @ k64[:hi].T                                  # [n, hi]
        S[np.arange(hi)[None, :] > r[:, None]] = -np.inf          # causal: j <= i
        pad = kb * block - hi
        if pad:
            S = np.concatenate([S, np.full((len(r), pad), -np.inf)], axis=1)
        out[a:a + chunk, :kb] = S.reshape(len(r), kb, block).max(axis=2).astype(F32)
    return out


def select_row(scores: np.ndarray, own: int, topk: int, force_init: bool = False) -> Tuple[List[int], float]:
    """Selection for one query whose own block is ``own``.

    Returns the ascending block ids and the relative gap between the last
    selected and the first unselected score among the blocks chosen by score
    (inf when every causal block fits, i.e. own + 1 <= topk).

    ``force_init`` is the "init" rule of the pages' init/local/causal rules
    ([PR] commit message), read as: block 0 is always kept, like the own block,
    and the remaining topk - 2 slots go to the best of blocks 1 .. own-1.
    """
    if own + 1 <= topk:
        return list(range(own + 1)), float("inf")
    first = 1 if force_init else 0
    forced = [0, own] if force_init else [own]
    n_pick = topk - len(forced)
    cand = np.arange(first, own)
    sc = scores[first:own].astype(F32)
    order = np.lexsort((cand, -sc.astype(F64)))       # score descending, id ascending
    keep = [int(c) for c in cand[order[:n_pick]]]
    s_last = F64(sc[order[n_pick - 1]])
    s_next = F64(sc[order[n_pick]])
    den = max(abs(s_last), abs(s_next))
    gap = abs(s_last - s_next) / den if den > 0 else 0.0
    return sorted(keep + forced), float(gap)


def selection_valid_within_ties(scores: np.ndarray, own: int, ids: Sequence[int], topk: int,
                                rel: float = 1e-3, force_init: bool = False) -> bool:
    """Whether ``ids`` is a correct selection for a query in block ``own``
    once near ties may go either way.

    The rule ([M31] section 1) fixes the forced blocks (the own block, plus
    block 0 under ``force_init``) and that every other chosen block scores at
    least as high as every causal block left out.  Two correct selections may
    differ only where the two scores are within ``rel`` of each other
    (relative to the larger magnitude): the near-tie exemption of the parity
    bar.  ``ids`` is a row of a block list: ascending, distinct, -1 padded.
    """
    ids = [int(c) for c in ids]
    got = [c for c in ids if c >= 0]
    if got != sorted(set(got)) or any(c > own for c in got) or ids[len(got):] != [-1] * (len(ids) - len(got)):
        return False
    if own + 1 <= topk:
        return got == list(range(own + 1))
    forced = {0, own} if force_init else {own}
    if len(got) != topk or not forced <= set(got):
        return False
    chosen = [c for c in got if c not in forced]
    left = [c for c in range(own) if c not in forced and c not in set(got)]
    lo = F64(min(scores[c] for c in chosen))
    hi = F64(max(scores[c] for c in left))
    if lo >= hi:
        return True
    return abs(lo - hi) / max(abs(lo), abs(hi)) < rel


@dataclass
class SelectResult:
    blk_idx: np.ndarray        # int32 [T, Hk, topk], ascending, -1 padded
    gap: np.ndarray            # fp64 [T, Hk]: relative 16th/17th gap (inf when nothing is decided)
    rows: np.ndarray           # token ids covered (all tokens unless sampled)
    scores: Optional[np.ndarray] = None   # fp32 [rows, Hk, blocks] block scores (-inf past own), if kept

    def near_tie(self, rel: float = 1e-3) -> np.ndarray:
        return self.gap < rel


def index_select(idx_q: np.ndarray, idx_k: np.ndarray, w_q: np.ndarray, w_k: np.ndarray,
                 cu_seqlens: Sequence[int], block: int = 128, topk: int = 16,
                 eps: float = 1e-6, rope_base: float = 1e7, rope_dims: int = 64,
                 rows: Optional[np.ndarray] = None, round_bf16: bool = True,
                 force_init: bool = False, keep_scores: bool = False) -> SelectResult:
    """Frozen lightning-indexer block selection ([M31] section 1, [PR]).

    ``idx_q``: [T, Hk, D]; ``idx_k``: [T, Hk, D] or [T, 1, D] (one key head
    shared by every index head).  Index head h selects the blocks for KV head
    h.  ``rows`` restricts the output to a subset of tokens (sampled checks);
    the returned arrays then follow ``rows``.  ``force_init`` keeps block 0 in
    every selection (see ``select_row``).  ``keep_scores`` also returns every
    row's block scores (for checking a selection that differs at a near tie).
    """
    idx_q = np.asarray(idx_q, dtype=F32)
    idx_k = np.asarray(idx_k, dtype=F32)
    T, Hk, D = idx_q.shape
    seq, pos = sequence_layout(cu_seqlens)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    all_rows = np.arange(T) if rows is None else np.asarray(sorted(set(int(r) for r in rows)), dtype=np.int64)
    blk = np.full((len(all_rows), Hk, topk), -1, dtype=np.int32)
    gap = np.full((len(all_rows), Hk), np.inf, dtype=F64)
    row_slot = {int(t): n for n, t in enumerate(all_rows)}
    if keep_scores:
        max_len = int(max(cu[1:] - cu[:-1])) if len(cu) > 1 else 0
        scores = np.full((len(all_rows), Hk, max(1, (max_len + block - 1) // block)), -np.inf, dtype=F32)
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        mine = all_rows[(all_rows >= a) & (all_rows < b)]
        if len(mine) == 0:
            continue
        hi = int(mine.max()) + 1
        p = pos[a:hi]
        for h in range(Hk):
            kh = h if idx_k.shape[1] > 1 else 0
            qf = indexer_features(idx_q[mine, h, :], w_q, pos[mine], eps, rope_base, rope_dims, round_bf16)
            kf = indexer_features(idx_k[a:hi, kh, :], w_k, p, eps, rope_base, rope_dims, round_bf16)
            # qf rows are the sampled queries; block_max_scores wants features indexed by position,
            # so scatter them into a buffer of the sequence prefix.
            qbuf = np.zeros((hi - a, D), dtype=F32)
            qbuf[mine - a] = qf
            sc = block_max_scores(qbuf, kf, block, rows=mine - a)
            for n, t in enumerate(mine):
                own = int(pos[t]) // block
                ids, g = select_row(sc[n], own, topk, force_init)
                slot = row_slot[int(t)]
                blk[slot, h, :len(ids)] = ids
                gap[slot, h] = g
                if keep_scores:
                    scores[slot, h, :sc.shape[1]] = sc[n]
    return SelectResult(blk_idx=blk, gap=gap, rows=all_rows, scores=scores if keep_scores else None)


# ---------------------------------------------------------------------------
# Block-sparse GQA attention, forward and backward
# ([M31] section 1; [PR] QSA block-sparse kernel forward/backward)
# ---------------------------------------------------------------------------

def key_set(i: int, blocks: Iterable[int], seq_start: int, pos_i: int, block: int) -> np.ndarray:
    """Global key indices query i attends to: keys j <= i of its listed blocks.

    Ids below 0 are padding.  A listed block entirely after the query
    contributes nothing.
    """
    out = []
    for c in sorted(set(int(c) for c in blocks if int(c) >= 0)):
        lo = c * block
        hi = min(c * block + block, pos_i + 1)
        if hi > lo:
            out.append(np.arange(seq_start + lo, seq_start + hi))
    if not out:
        return np.zeros(0, dtype=np.int64)
    return np.concatenate(out)


def attention_forward(q: np.ndarray, k: np.ndarray, v: np.ndarray, blk_idx: np.ndarray,
                      cu_seqlens: Sequence[int], scale: float, block: int = 128,
                      rows: Optional[Sequence[int]] = None,
                      heads: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """O = softmax(scale * q k^T) v over each query's selected causal keys, and LSE.

    ``q`` [T, Hq, D]; ``k``, ``v`` [T, Hk, D]; ``blk_idx`` [T, Hk, K] with
    sequence-local block ids.  Query head g reads KV head g // (Hq/Hk).
    Returns fp64 O [n, Hq, D] and natural-log LSE [n, Hq] for the tokens in
    ``rows`` (default: all).  A query with no key gets O = 0 and LSE = -inf.
    ``heads`` restricts the work to some KV heads (the other outputs stay 0).
    """
    T, Hq, D = q.shape
    Hk = k.shape[1]
    G = Hq // Hk
    seq, pos = sequence_layout(cu_seqlens)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    O = np.zeros((len(rows), Hq, D), dtype=F64)
    LSE = np.full((len(rows), Hq), -np.inf, dtype=F64)
    heads = range(Hk) if heads is None else heads
    for n, i in enumerate(rows):
        i = int(i)
        for h in heads:
            J = key_set(i, blk_idx[i, h], int(cu[seq[i]]), int(pos[i]), block)
            if len(J) == 0:
                continue
            Q = q[i, h * G:(h + 1) * G, :].astype(F64)             # [G, D]
            Kj = k[J, h, :].astype(F64)                              # [n, D]
            Vj = v[J, h, :].astype(F64)
            Z = scale * (Q @ Kj.T)                                   # [G, n]
            m = Z.max(axis=1, keepdims=True)
            E = np.exp(Z - m)
            l = E.sum(axis=1, keepdims=True)
            O[n, h * G:(h + 1) * G] = (E @ Vj) / l
            LSE[n, h * G:(h + 1) * G] = (m + np.log(l))[:, 0]
    return O, LSE


def attention_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray,
                       blk_idx: np.ndarray, cu_seqlens: Sequence[int], scale: float,
                       block: int = 128, rows: Optional[Sequence[int]] = None,
                       heads: Optional[Sequence[int]] = None
                       ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Gradients of sum(O * dO) with respect to q, k and v (fp64).

    With P = softmax(z) over the key set J of a query row and dP = dO . v_j,
    dS = P * (dP - sum_j P dP); dq = scale * sum_j dS_j k_j; each key gets
    dk_j += scale * dS_j q and dv_j += P_j dO, summed over every query head
    of its group and every query that selected its block.

    ``rows`` restricts the queries: dQ then covers those rows only and dK/dV
    hold only their contributions (useful to check one key block by passing
    every query that selected it).  ``heads`` restricts the work to some KV
    heads.
    """
    T, Hq, D = q.shape
    Hk = k.shape[1]
    G = Hq // Hk
    seq, pos = sequence_layout(cu_seqlens)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    dQ = np.zeros((len(rows), Hq, D), dtype=F64)
    dK = np.zeros((T, Hk, D), dtype=F64)
    dV = np.zeros((T, Hk, D), dtype=F64)
    heads = range(Hk) if heads is None else heads
    for n, i in enumerate(rows):
        i = int(i)
        for h in heads:
            J = key_set(i, blk_idx[i, h], int(cu[seq[i]]), int(pos[i]), block)
            if len(J) == 0:
                continue
            Q = q[i, h * G:(h + 1) * G, :].astype(F64)
            dO = do[i, h * G:(h + 1) * G, :].astype(F64)
            Kj = k[J, h, :].astype(F64)
            Vj = v[J, h, :].astype(F64)
            Z = scale * (Q @ Kj.T)
            Z = Z - Z.max(axis=1, keepdims=True)
            P = np.exp(Z)
            P /= P.sum(axis=1, keepdims=True)
            dP = dO @ Vj.T
            delta = (P * dP).sum(axis=1, keepdims=True)
            dS = P * (dP - delta)
            dQ[n, h * G:(h + 1) * G] = scale * (dS @ Kj)
            dK[J, h, :] += scale * (dS.T @ Q)
            dV[J, h, :] += P.T @ dO
    return dQ, dK, dV


def selectors_of_block(blk_idx: np.ndarray, cu_seqlens: Sequence[int], seq_id: int,
                       block_id: int, head: int) -> np.ndarray:
    """Tokens of sequence ``seq_id`` whose list for ``head`` contains ``block_id``."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    a, b = int(cu[seq_id]), int(cu[seq_id + 1])
    hit = (blk_idx[a:b, head, :] == block_id).any(axis=1)
    return a + np.nonzero(hit)[0]


# ---------------------------------------------------------------------------
# Attention-side q/k norm and partial RoPE  ([M31] section 1: "per-head gemma
# q/k norm, RoPE on the first 64 dims (base 1e7)"; [MB] Architecture Notes:
# per-head QK RMSNorm, gemma-style x * (1 + w), partial RoPE on 64 of 128
# channels).  The step applied to the attention's own q and k before the
# block-sparse kernel, forward and backward.
# ---------------------------------------------------------------------------

def qk_norm_rope_forward(x: np.ndarray, w: np.ndarray, pos: np.ndarray, eps: float = 1e-6,
                         base: float = 1e7, rope_dims: int = 64) -> np.ndarray:
    """q^ (or k^) = bf16(RoPE_p(RMSNorm(x) * (1 + w))) per head: the same
    arithmetic as the indexer features, on the attention's [N, H, 128] q or k
    with one [128] weight shared by the heads.  Returns fp32 holding bf16."""
    return indexer_features(x, w, pos, eps, base, rope_dims, round_bf16=True)


def qk_norm_rope_backward(x: np.ndarray, w: np.ndarray, pos: np.ndarray, dz: np.ndarray,
                          eps: float = 1e-6, base: float = 1e7,
                          rope_dims: int = 64) -> Tuple[np.ndarray, np.ndarray]:
    """Vector-Jacobian product of z = RoPE_p(y), y = x * r * (1 + w),
    r = 1 / sqrt(mean(x^2) + eps), in fp64 (with the same fp32 cos/sin as the
    forward).  ``x``, ``dz``: [N, H, D]; returns (dx [N, H, D], dw [D]).

    Written from the definition: RoPE is a rotation, so dy = RoPE_p^T(dz)
    (rotation by -angle); with g = dy * (1 + w), dx_k = r g_k - x_k r^3
    sum_j(g_j x_j) / D; and dw_j = sum over rows of dy_j x_j r.
    """
    x = np.asarray(x, dtype=F64)
    dz = np.asarray(dz, dtype=F64)
    w = np.asarray(w, dtype=F64)
    D = x.shape[-1]
    half = rope_dims // 2
    c, s = rope_cos_sin(pos, base, rope_dims)
    shape = (x.shape[0],) + (1,) * (x.ndim - 2) + (half,)
    c = c.astype(F64).reshape(shape)
    s = s.astype(F64).reshape(shape)
    dy = dz.copy()
    dy[..., :half] = c * dz[..., :half] + s * dz[..., half:rope_dims]
    dy[..., half:rope_dims] = -s * dz[..., :half] + c * dz[..., half:rope_dims]
    r = 1.0 / np.sqrt((x * x).mean(axis=-1) + eps)
    g = dy * (1.0 + w)
    dot = (g * x).sum(axis=-1)
    dx = r[..., None] * g - x * (r ** 3 * dot / D)[..., None]
    dw = (dy * x * r[..., None]).reshape(-1, D).sum(axis=0)
    return dx, dw
