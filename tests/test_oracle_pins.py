"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each test checks the oracle against something other than its own code:
a library routine (torch's bf16 cast, torch's CPU attention and autograd),
a closed form, a hand-derived golden fixture, an invariant of the method,
brute force on tiny inputs, or finite differences.  No GPU is needed.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import synth
from planted import load_planted

RNG = np.random.default_rng(1234)


def f32(t):
    return t.float().numpy()


# ---------------------------------------------------------------- bf16 rounding
def test_round_to_bf16_matches_torch_cast():
    x = RNG.standard_normal(200000).astype(np.float32) * np.float32(3.0)
    # exact ties: bit pattern with the low 16 bits equal to 0x8000
    ties = (RNG.integers(0, 2**15, 1000).astype(np.uint32) << 17 | 0x8000).view(np.float32)
    ties = ties[np.isfinite(ties)]
    x = np.concatenate([x, ties, np.array([0.0, -0.0, 1e-40, -3e38], dtype=np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    got = O.round_to_bf16(x)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


# ---------------------------------------------------------------- gemma RMSNorm
def test_rmsnorm_closed_forms():
    x = (RNG.standard_normal((64, 128)) * 2.5).astype(np.float32)
    eps = 1e-6
    w0 = np.zeros(128, np.float32)
    y = O.gemma_rmsnorm(x, w0, eps).astype(np.float64)
    ms = (x.astype(np.float64) ** 2).mean(axis=1)
    # mean(y^2) = mean(x^2) / (mean(x^2) + eps)
    np.testing.assert_allclose((y ** 2).mean(axis=1), ms / (ms + eps), rtol=2e-6)
    # (1 + w) with w = -1 kills the output; w = 1 doubles it exactly
    assert np.all(O.gemma_rmsnorm(x, -np.ones(128, np.float32), eps) == 0)
    assert np.array_equal(O.gemma_rmsnorm(x, np.ones(128, np.float32), eps), 2 * O.gemma_rmsnorm(x, w0, eps))
    # the weight scales channel d by (1 + w_d)
    w = (RNG.standard_normal(128) * 0.1).astype(np.float32)
    np.testing.assert_allclose(O.gemma_rmsnorm(x, w, eps), O.gemma_rmsnorm(x, w0, eps) * (1 + w), rtol=1e-6)


def test_indexer_features_norm_before_rope_closed_form():
    """The indexer's features are the norm first, then the rotation.  With x
    = e_0, 1 + w = 2 on dim 0 and 1 on dim 32, and angle theta on pair 0: norm
    first gives dim 32 = 2 r sin(theta) (r = 1 / sqrt(1/128 + eps)); rotating
    first would give r sin(theta) there, since the weight of dim 32 then
    scales the rotated component."""
    eps = 1e-6
    x = np.zeros((1, 128), np.float32)
    x[0, 0] = 1.0
    w = np.zeros(128, np.float32)
    w[0] = 1.0
    p = 3
    y = O.indexer_features(x, w, np.array([p]), eps, 1e7, 64, round_bf16=False).astype(np.float64)[0]
    r = 1.0 / math.sqrt(1.0 / 128.0 + eps)
    np.testing.assert_allclose(y[0], 2 * r * math.cos(p), rtol=1e-6)
    np.testing.assert_allclose(y[32], 2 * r * math.sin(p), rtol=1e-6)
    assert np.count_nonzero(y) == 2


# ---------------------------------------------------------------- RoPE
def test_rope_identity_at_position_zero_and_passthrough():
    y = RNG.standard_normal((5, 128)).astype(np.float32)
    out = O.rope_rotate_half(y, np.zeros(5, np.int64), 1e7, 64)
    assert np.array_equal(out, y)
    out = O.rope_rotate_half(y, np.arange(5) * 977, 1e7, 64)
    assert np.array_equal(out[:, 64:], y[:, 64:])


def test_rope_unit_vectors_give_rotation_angles():
    """e_i and e_{i+32} map to (cos t, sin t) and (-sin t, cos t) on dims (i, i+32),
    with t = p * base**(-i/32) -- the rotary definition with 64 rotated dims."""
    base = 1e7
    for p in [1, 3, 1000, 32767]:
        for i in [0, 1, 7, 16, 31]:
            e = np.zeros((1, 128), np.float32)
            e[0, i] = 1
            out = O.rope_rotate_half(e, np.array([p]), base, 64)[0].astype(np.float64)
            t = p * base ** (-i / 32.0)
            assert abs(out[i] - math.cos(t)) < 1e-7 and abs(out[i + 32] - math.sin(t)) < 1e-7
            nz = np.delete(np.arange(128), [i, i + 32])
            assert np.all(out[nz] == 0)
            e = np.zeros((1, 128), np.float32)
            e[0, i + 32] = 1
            out = O.rope_rotate_half(e, np.array([p]), base, 64)[0].astype(np.float64)
            assert abs(out[i] + math.sin(t)) < 1e-7 and abs(out[i + 32] - math.cos(t)) < 1e-7


def test_rope_matches_complex_multiplication():
    y = RNG.standard_normal((50, 128)).astype(np.float32)
    pos = RNG.integers(0, 32768, 50)
    out = O.rope_rotate_half(y, pos, 5e6, 64).astype(np.float64)
    z = y[:, :32].astype(np.float64) + 1j * y[:, 32:64].astype(np.float64)
    freqs = np.array([5e6 ** (-i / 32.0) for i in range(32)])
    zr = z * np.exp(1j * pos[:, None] * freqs[None, :])
    np.testing.assert_allclose(out[:, :32], zr.real, atol=3e-6)
    np.testing.assert_allclose(out[:, 32:64], zr.imag, atol=3e-6)


def test_rope_logits_depend_on_relative_position_only():
    q = RNG.standard_normal((20, 128)).astype(np.float32)
    k = RNG.standard_normal((20, 128)).astype(np.float32)
    pq = RNG.integers(0, 4000, 20)
    pk = RNG.integers(0, 4000, 20)
    for shift in [1, 517, 9000]:
        a = (O.rope_rotate_half(q, pq, 1e7, 64).astype(np.float64) * O.rope_rotate_half(k, pk, 1e7, 64)).sum(1)
        b = (O.rope_rotate_half(q, pq + shift, 1e7, 64).astype(np.float64) *
             O.rope_rotate_half(k, pk + shift, 1e7, 64)).sum(1)
        np.testing.assert_allclose(a, b, atol=5e-5 * np.abs(a).max())


# ---------------------------------------------------------------- block scores (brute force)
def test_block_max_scores_brute_force():
    L, D, B = 45, 16, 8
    qf = O.round_to_bf16(RNG.standard_normal((L, D)).astype(np.float32))
    kf = O.round_to_bf16(RNG.standard_normal((L, D)).astype(np.float32))
    got = O.block_max_scores(qf, kf, B)
    for i in range(L):
        for c in range((L + B - 1) // B):
            vals = [math.fsum(float(qf[i, d]) * float(kf[j, d]) for d in range(D))
                    for j in range(c * B, min(c * B + B, L)) if j <= i]
            want = np.float32(max(vals)) if vals else -np.inf
            assert got[i, c] == want, (i, c)


# ---------------------------------------------------------------- planted selection (golden)
def test_planted_selection_golden():
    P = load_planted()
    res = O.index_select(f32(P["idx_q"]), f32(P["idx_k"]), f32(P["w_q"]), f32(P["w_k"]),
                         P["cu_seqlens"], block=P["block"], topk=P["topk"])
    for t, ids, why in P["expected"]:
        assert list(res.blk_idx[t, 0]) == ids, (t, why)
    # the planted gaps are wide: no expected row is a near tie except the exact 3/9 tie
    assert res.gap[P["expected"][3][0], 0] > 1e-2


# Hand-built score row for the gap pins: blocks 0..19 precede the own block 20.
# The twenty scores, best first, are GAP_VALUES; block b holds rank GAP_RANK[b]
# (1 = best).  Consecutive values are spaced unevenly (2, 3, 4, ... apart), so a
# gap taken between the wrong pair of ranks gives a different number.
GAP_VALUES = [50, 48, 45, 41, 36, 30, 23, 15, 6, -4, -15, -27, -40, -54, -69, -85, -102, -120, -139, -159]
GAP_RANK = [1, 7, 16, 4, 12, 20, 2, 15, 9, 18, 5, 13, 3, 19, 10, 6, 17, 8, 14, 11]


def gap_row(rank_of, shift=0.0, own_score=-75.0):
    row = np.full(24, 1000.0, dtype=np.float32)      # blocks past the own block: never candidates
    for b, r in enumerate(rank_of):
        row[b] = GAP_VALUES[r - 1] + shift
    row[20] = own_score                                # the own block is forced, its score unused
    return row


def test_select_row_gap_hand_built():
    """The near-tie gap is |a - b| / max(|a|, |b|) between the last score-chosen
    block and the best block left out: with the own block forced, the 15th and
    16th best of blocks 0..19 (ranks 15 and 16: -69 and -85)."""
    ids, gap = O.select_row(gap_row(GAP_RANK), 20, 16)
    assert ids == sorted([b for b, r in enumerate(GAP_RANK) if r <= 15] + [20])
    assert gap == pytest.approx(16 / 85, rel=1e-12)
    # mixed signs: shifted by +71 the pair is (2, -14): |2 + 14| / 14, not (14 - 2) / 14
    _, gap = O.select_row(gap_row(GAP_RANK, shift=71.0, own_score=2.5), 20, 16)
    assert gap == pytest.approx(16 / 14, rel=1e-12)
    # the own block's score does not enter the ranking even when it sits between the pair
    for own_score in (-70.0, -80.0, 1e6, -1e6):
        assert O.select_row(gap_row(GAP_RANK, own_score=own_score), 20, 16)[1] == pytest.approx(16 / 85, rel=1e-12)
    # fewer than 16 earlier blocks: nothing is decided by score
    assert O.select_row(gap_row(GAP_RANK), 15, 16)[1] == math.inf


def test_select_row_gap_force_init_slot_count():
    """With the initial block forced, 14 slots go by score among blocks 1..19.
    Block 0 made the weakest: the gap falls between ranks 14 and 15 (-54, -69),
    not 15 and 16 as without the rule.  Block 0 made the best: it leaves the
    candidates, so ranks 2..15 are chosen and the gap is ranks 15/16 again."""
    rank = list(GAP_RANK)
    rank[0], rank[5] = rank[5], rank[0]                # block 0 now rank 20, block 5 rank 1
    ids, gap = O.select_row(gap_row(rank), 20, 16, force_init=True)
    assert ids == sorted([0, 20] + [b for b, r in enumerate(rank) if b > 0 and r <= 14])
    assert gap == pytest.approx(15 / 69, rel=1e-12)
    assert O.select_row(gap_row(rank), 20, 16)[1] == pytest.approx(16 / 85, rel=1e-12)
    ids, gap = O.select_row(gap_row(GAP_RANK), 20, 16, force_init=True)
    assert gap == pytest.approx(16 / 85, rel=1e-12)
    assert ids == sorted([b for b, r in enumerate(GAP_RANK) if r <= 15] + [20])


def test_planted_gap_closed_form():
    """The gap through the whole oracle on the planted pack.  With every logit
    position independent (content only in dims 64.., where RoPE is the
    identity), a key x*e64 + e65 against the query e64 scores, up to the bf16
    rounding of the features and eps, 128 * x / sqrt(x^2 + 1).  At block 16 of
    sequence 0 the 15th and 16th best peaks are x = -0.75 and x = -0.875, so
    the gap is about 0.0888; the neighbouring pairs would give 0.117 and 0.069.
    The planted exact tie (blocks 3 and 9 of sequence 2) has gap 0."""
    P = load_planted()
    res = O.index_select(f32(P["idx_q"]), f32(P["idx_k"]), f32(P["w_q"]), f32(P["w_k"]),
                         P["cu_seqlens"], block=P["block"], topk=P["topk"])
    s = lambda x: x / math.sqrt(x * x + 1)
    want = abs(s(-0.75) - s(-0.875)) / abs(s(-0.875))
    t16 = [t for t, _, why in P["expected"] if "block 16: own block kept" in why][0]
    assert res.gap[t16, 0] == pytest.approx(want, rel=2e-2)
    t_tie = [t for t, _, why in P["expected"] if "tie (identical peak keys)" in why][0]
    assert res.gap[t_tie, 0] == 0.0
    assert res.near_tie()[t_tie, 0] and not res.near_tie()[t16, 0]
    early = [t for t, ids, _ in P["expected"] if len([c for c in ids if c >= 0]) < 16]
    assert all(np.isinf(res.gap[t, 0]) and not res.near_tie()[t, 0] for t in early)


def test_selection_valid_within_ties_hand_built():
    """The checker used for rows where two correct selections may differ.  On
    the hand-built row: the oracle's own answer is valid; swapping the last
    chosen block (rank 15) for the first left out (rank 16) is valid only when
    the two scores are within 1e-3 relative; dropping the own block, a wrong
    count, a non-causal id or an unsorted row is never valid."""
    row = gap_row(GAP_RANK)
    ids, _ = O.select_row(row, 20, 16)
    pad = lambda xs: list(xs) + [-1] * (16 - len(xs))
    assert O.selection_valid_within_ties(row, 20, ids, 16)
    r15, r16 = GAP_RANK.index(15), GAP_RANK.index(16)
    swapped = sorted([c for c in ids if c != r15] + [r16])
    assert not O.selection_valid_within_ties(row, 20, swapped, 16)            # gap 16/85: far from a tie
    near = row.copy()
    near[r16] = np.float32(-69.05)                                              # gap 0.05/69 < 1e-3
    assert O.selection_valid_within_ties(near, 20, swapped, 16)
    near[r16] = np.float32(-69.1)                                               # gap 0.1/69 > 1e-3
    assert not O.selection_valid_within_ties(near, 20, swapped, 16)
    assert not O.selection_valid_within_ties(row, 20, sorted([c for c in ids if c != 20] + [r16]), 16)
    assert not O.selection_valid_within_ties(row, 20, pad(ids[:15]), 16)
    assert not O.selection_valid_within_ties(row, 20, sorted(ids[:15] + [21]), 16)
    assert not O.selection_valid_within_ties(row, 20, ids[::-1], 16)
    # below 16 causal blocks the answer is unique: blocks 0..b
    assert O.selection_valid_within_ties(row, 3, pad([0, 1, 2, 3]), 16)
    assert not O.selection_valid_within_ties(row, 3, pad([0, 1, 3]), 16)
    # under the initial-block rule block 0 must be present
    fi, _ = O.select_row(row, 20, 16, force_init=True)
    assert O.selection_valid_within_ties(row, 20, fi, 16, force_init=True)
    rank = list(GAP_RANK)
    rank[0], rank[5] = rank[5], rank[0]                # block 0 the weakest: plain selection drops it
    row0 = gap_row(rank)
    plain, _ = O.select_row(row0, 20, 16)
    assert 0 not in plain and O.selection_valid_within_ties(row0, 20, plain, 16)
    assert not O.selection_valid_within_ties(row0, 20, plain, 16, force_init=True)


def test_planted_selection_force_init_golden():
    """The forced initial block, on hand-derived planted cases."""
    P = load_planted()
    res = O.index_select(f32(P["idx_q"]), f32(P["idx_k"]), f32(P["w_q"]), f32(P["w_k"]),
                         P["cu_seqlens"], block=P["block"], topk=P["topk"], force_init=True)
    for t, ids, why in P["expected_force_init"]:
        assert list(res.blk_idx[t, 0]) == ids, (t, why)


def test_force_init_brute_force():
    """The forced initial block against an independent brute force: every
    (block 0, own block, 14-subset of 1..b-1) candidate set is ranked by the
    scores it keeps; the best set (highest sorted scores, lower ids on ties)
    must be the oracle's.  Tiny rows only (b = 16, 17)."""
    import itertools
    rng = np.random.default_rng(7)
    for trial in range(6):
        own = 16 + trial % 2
        sc = rng.integers(-3, 4, own).astype(np.float32)  # small integers: plenty of ties
        ids, _ = O.select_row(sc, own, 16, force_init=True)
        best = None
        for sub in itertools.combinations(range(1, own), 14):
            key = sorted(((-float(sc[c]), c) for c in sub))
            if best is None or key < best[0]:
                best = (key, sub)
        assert ids == sorted([0, own] + list(best[1])), (trial, ids)


def test_force_init_relation_to_plain_selection():
    """With block 0 among the plain choice the rule changes nothing; otherwise
    it replaces the weakest block chosen by score with block 0."""
    rng = np.random.default_rng(8)
    for trial in range(200):
        own = int(rng.integers(16, 80))
        sc = rng.standard_normal(own).astype(np.float32)
        if trial % 3 == 0:
            sc[0] = -10.0  # block 0 certainly not chosen by score
        plain, _ = O.select_row(sc, own, 16)
        forced, _ = O.select_row(sc, own, 16, force_init=True)
        if 0 in plain:
            assert forced == plain
        else:
            chosen = [c for c in plain if c != own]
            weakest = min(chosen, key=lambda c: (sc[c], -c))
            assert forced == sorted([c for c in plain if c != weakest] + [0])


# ---------------------------------------------------------------- selection invariants
def test_selection_invariants_random():
    p = synth.make_custom_pack([2600, 700, 2300], num_q_heads=2, num_kv_heads=2, seed=5)
    cu = p.cu_seqlens.numpy()
    res = O.index_select(f32(p.idx_q), f32(p.idx_k), f32(p.w_q), f32(p.w_k), cu)
    seq, pos = O.sequence_layout(cu)
    for h in range(2):
        scores = {}
        for s in range(3):
            a, b = int(cu[s]), int(cu[s + 1])
            qf = O.indexer_features(f32(p.idx_q)[a:b, h], f32(p.w_q), pos[a:b], 1e-6, 1e7, 64)
            kf = O.indexer_features(f32(p.idx_k)[a:b, h], f32(p.w_k), pos[a:b], 1e-6, 1e7, 64)
            scores[s] = O.block_max_scores(qf, kf, 128)
        for t in range(0, int(cu[-1]), 7):
            b = int(pos[t]) // 128
            ids = [int(c) for c in res.blk_idx[t, h] if c >= 0]
            assert b in ids
            assert len(ids) == min(16, b + 1)
            assert all(0 <= c <= b for c in ids) and ids == sorted(set(ids))
            if b >= 16:
                sc = scores[int(seq[t])][int(pos[t]) - 0]
                sel = [c for c in ids if c != b]
                uns = [c for c in range(b) if c not in ids]
                assert min(sc[sel]) >= max(sc[uns])


def test_bf16_feature_rounding_matters_only_near_ties():
    """Skipping the bf16 rounding of the features moves only rows whose 16th/17th
    scores sit within the bf16 rounding noise of the scores (a few 1e-3 relative):
    the rounding is a real part of the definition, and its effect is bounded."""
    p = synth.make_custom_pack([4096], seed=3)
    args = (f32(p.idx_q), f32(p.idx_k), f32(p.w_q), f32(p.w_k), p.cu_seqlens.numpy())
    a = O.index_select(*args)
    b = O.index_select(*args, round_bf16=False)
    diff = (a.blk_idx != b.blk_idx).any(axis=2)
    assert diff.sum() > 0
    assert np.all(a.gap[diff] < 1e-2)
    assert diff.sum() < 0.05 * np.isfinite(a.gap).sum()


# ---------------------------------------------------------------- attention helpers (torch references)
def _torch_dense(q, k, v, do, mask, scale):
    """Dense fp64 attention per kv group with a boolean mask [T, T]; torch autograd grads."""
    T, Hq, D = q.shape
    Hk = k.shape[1]
    G = Hq // Hk
    qt = torch.tensor(q, dtype=torch.float64, requires_grad=True)
    kt = torch.tensor(k, dtype=torch.float64, requires_grad=True)
    vt = torch.tensor(v, dtype=torch.float64, requires_grad=True)
    Q = qt.permute(1, 0, 2).unsqueeze(0)                                # [1, Hq, T, D]
    K = kt.permute(1, 0, 2).repeat_interleave(G, dim=0).unsqueeze(0)
    V = vt.permute(1, 0, 2).repeat_interleave(G, dim=0).unsqueeze(0)
    out = torch.nn.functional.scaled_dot_product_attention(
        Q, K, V, attn_mask=torch.tensor(mask)[None, None] if mask.ndim == 2 else torch.tensor(mask)[None],
        scale=scale)
    o = out[0].permute(1, 0, 2)
    (o * torch.tensor(do, dtype=torch.float64)).sum().backward()
    return o.detach().numpy(), qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


def _pack_np(lengths, hq, hk, seed):
    p = synth.make_custom_pack(lengths, num_q_heads=hq, num_kv_heads=hk, seed=seed)
    return p, f32(p.q), f32(p.k), f32(p.v), f32(p.do), p.cu_seqlens.numpy()


# ---------------------------------------------------------------- P1: dense equality up to 2048
def test_dense_equality_up_to_2048_tokens():
    """16 blocks x 128 = 2048 keys: at or below that length the method is full causal attention."""
    p, q, k, v, do, cu = _pack_np([1024, 640, 384], 4, 2, 11)
    sel = O.index_select(f32(p.idx_q), f32(p.idx_k), f32(p.w_q), f32(p.w_k), cu)
    seq, pos = O.sequence_layout(cu)
    for t in range(0, int(cu[-1]), 13):
        b = int(pos[t]) // 128
        assert list(sel.blk_idx[t, 0, :b + 1]) == list(range(b + 1))
    scale = 1 / math.sqrt(128)
    Ofw, LSE = O.attention_forward(q, k, v, sel.blk_idx, cu, scale)
    dQ, dK, dV = O.attention_backward(q, k, v, do, sel.blk_idx, cu, scale)
    for s in range(3):
        a, b = int(cu[s]), int(cu[s + 1])
        G = 2
        Q = torch.tensor(q[a:b], dtype=torch.float64).permute(1, 0, 2)[None]
        K = torch.tensor(k[a:b], dtype=torch.float64).permute(1, 0, 2).repeat_interleave(G, 0)[None]
        V = torch.tensor(v[a:b], dtype=torch.float64).permute(1, 0, 2).repeat_interleave(G, 0)[None]
        out, lse = torch.ops.aten._scaled_dot_product_flash_attention_for_cpu(Q, K, V, 0.0, True, scale=scale)
        np.testing.assert_allclose(Ofw[a:b], out[0].permute(1, 0, 2).numpy(), atol=1e-12)
        np.testing.assert_allclose(LSE[a:b], lse[0].permute(1, 0).numpy(), atol=1e-12)
        mask = np.tril(np.ones((b - a, b - a), dtype=bool))
        o_t, dq_t, dk_t, dv_t = _torch_dense(q[a:b], k[a:b], v[a:b], do[a:b], mask, scale)
        np.testing.assert_allclose(dQ[a:b], dq_t, atol=1e-10)
        np.testing.assert_allclose(dK[a:b], dk_t, atol=1e-10)
        np.testing.assert_allclose(dV[a:b], dv_t, atol=1e-10)


# ---------------------------------------------------------------- P2: masked dense attention
def test_sparse_equals_masked_dense_attention():
    p, q, k, v, do, cu = _pack_np([2400, 300], 4, 2, 21)
    sel = O.index_select(f32(p.idx_q), f32(p.idx_k), f32(p.w_q), f32(p.w_k), cu)
    T = int(cu[-1])
    seq, pos = O.sequence_layout(cu)
    scale = 1 / math.sqrt(128)
    Ofw, _ = O.attention_forward(q, k, v, sel.blk_idx, cu, scale)
    dQ, dK, dV = O.attention_backward(q, k, v, do, sel.blk_idx, cu, scale)
    # per kv head masks: mask[h, i, j] = same sequence, j <= i, block(j) listed for (i, h)
    Hk = 2
    G = 2
    mask = np.zeros((Hk, T, T), dtype=bool)
    for h in range(Hk):
        for i in range(T):
            s = seq[i]
            for c in sel.blk_idx[i, h]:
                if c < 0:
                    continue
                lo = int(cu[s]) + int(c) * 128
                hi = min(lo + 128, i + 1)
                mask[h, i, lo:hi] = True
    assert mask.sum() < np.tril(np.ones((T, T), bool)).sum() * Hk * 0.95  # really sparse
    full_mask = np.repeat(mask, G, axis=0)
    o_t, dq_t, dk_t, dv_t = _torch_dense(q, k, v, do, full_mask, scale)
    np.testing.assert_allclose(Ofw, o_t, atol=1e-11)
    np.testing.assert_allclose(dQ, dq_t, atol=1e-10)
    np.testing.assert_allclose(dK, dk_t, atol=1e-10)
    np.testing.assert_allclose(dV, dv_t, atol=1e-10)


# ---------------------------------------------------------------- dense layers beyond 16 blocks
def test_all_blocks_listed_equals_dense_causal_beyond_2048():
    """The dense first layers: with every causal block listed (24 > 16 of them) the oracle's attention
    is torch's causal flash attention (fp64), forward and backward."""
    p, q, k, v, do, cu = _pack_np([3000, 700], 2, 1, 31)
    seq, pos = O.sequence_layout(cu)
    nb = (max(p.lengths) + 127) // 128
    blk = np.full((int(cu[-1]), 1, nb), -1, np.int32)
    for t in range(int(cu[-1])):
        blk[t, 0, :pos[t] // 128 + 1] = np.arange(pos[t] // 128 + 1)
    scale = 1 / math.sqrt(128)
    Ofw, LSE = O.attention_forward(q, k, v, blk, cu, scale)
    dQ, dK, dV = O.attention_backward(q, k, v, do, blk, cu, scale, rows=np.arange(0, int(cu[-1]), 1))
    for s in range(2):
        a, b = int(cu[s]), int(cu[s + 1])
        Q = torch.tensor(q[a:b], dtype=torch.float64).permute(1, 0, 2)[None]
        K = torch.tensor(k[a:b], dtype=torch.float64).permute(1, 0, 2).repeat_interleave(2, 0)[None]
        V = torch.tensor(v[a:b], dtype=torch.float64).permute(1, 0, 2).repeat_interleave(2, 0)[None]
        out, lse = torch.ops.aten._scaled_dot_product_flash_attention_for_cpu(Q, K, V, 0.0, True, scale=scale)
        np.testing.assert_allclose(Ofw[a:b], out[0].permute(1, 0, 2).numpy(), atol=1e-12)
        np.testing.assert_allclose(LSE[a:b], lse[0].permute(1, 0).numpy(), atol=1e-12)
        mask = np.tril(np.ones((b - a, b - a), dtype=bool))
        o_t, dq_t, dk_t, dv_t = _torch_dense(q[a:b], k[a:b], v[a:b], do[a:b], mask, scale)
        np.testing.assert_allclose(dQ[a:b], dq_t, atol=1e-10)
        np.testing.assert_allclose(dK[a:b], dk_t, atol=1e-10)
        np.testing.assert_allclose(dV[a:b], dv_t, atol=1e-10)


# ---------------------------------------------------------------- narrow-block variant (4-token blocks)
def _narrow_pack(lengths, topk, seed):
    p = synth.make_custom_pack(lengths, num_q_heads=12, num_kv_heads=1, seed=seed, head_dim=256,
                               block_size=4, topk_blocks=topk)
    cu = p.cu_seqlens.numpy()
    blk = synth.random_block_lists(cu, 1, 4, topk, seed)
    return p, f32(p.q), f32(p.k), f32(p.v), f32(p.do), cu, blk


def test_narrow_dense_equality():
    """4-token blocks, 64 per query: sequences of at most 256 tokens see every causal key (12 q / 1 kv, D 256)."""
    p, q, k, v, do, cu, blk = _narrow_pack([200, 56], 64, 41)
    scale = 1 / math.sqrt(256)
    Ofw, LSE = O.attention_forward(q, k, v, blk, cu, scale, block=4)
    dQ, dK, dV = O.attention_backward(q, k, v, do, blk, cu, scale, block=4)
    for s in range(2):
        a, b = int(cu[s]), int(cu[s + 1])
        Q = torch.tensor(q[a:b], dtype=torch.float64).permute(1, 0, 2)[None]
        K = torch.tensor(k[a:b], dtype=torch.float64).permute(1, 0, 2).repeat_interleave(12, 0)[None]
        V = torch.tensor(v[a:b], dtype=torch.float64).permute(1, 0, 2).repeat_interleave(12, 0)[None]
        out, lse = torch.ops.aten._scaled_dot_product_flash_attention_for_cpu(Q, K, V, 0.0, True, scale=scale)
        np.testing.assert_allclose(Ofw[a:b], out[0].permute(1, 0, 2).numpy(), atol=1e-12)
        np.testing.assert_allclose(LSE[a:b], lse[0].permute(1, 0).numpy(), atol=1e-12)
        mask = np.tril(np.ones((b - a, b - a), dtype=bool))
        o_t, dq_t, dk_t, dv_t = _torch_dense(q[a:b], k[a:b], v[a:b], do[a:b], mask, scale)
        np.testing.assert_allclose(dQ[a:b], dq_t, atol=1e-10)
        np.testing.assert_allclose(dK[a:b], dk_t, atol=1e-10)
        np.testing.assert_allclose(dV[a:b], dv_t, atol=1e-10)


def test_narrow_sparse_equals_masked_dense():
    """4-token blocks, 16 per query out of up to 75: the key set is the listed blocks' causal keys."""
    p, q, k, v, do, cu, blk = _narrow_pack([300, 90], 16, 42)
    T = int(cu[-1])
    seq, pos = O.sequence_layout(cu)
    scale = 1 / math.sqrt(256)
    Ofw, _ = O.attention_forward(q, k, v, blk, cu, scale, block=4)
    dQ, dK, dV = O.attention_backward(q, k, v, do, blk, cu, scale, block=4)
    # mask[i, j]: same sequence, j <= i, and block (j - start) // 4 listed for i
    listed = np.zeros((T, 80), dtype=bool)
    for i in range(T):
        ids = blk[i, 0][blk[i, 0] >= 0]
        listed[i, ids] = True
    j = np.arange(T)
    same = seq[:, None] == seq[None, :]
    causal = j[None, :] <= j[:, None]
    jb = np.clip(pos[None, :] // 4, 0, 79)
    mask = same & causal & np.take_along_axis(listed, np.broadcast_to(jb, (T, T)), axis=1)
    assert mask.sum() < 0.5 * (same & causal).sum()
    o_t, dq_t, dk_t, dv_t = _torch_dense(q, k, v, do, np.repeat(mask[None], 12, axis=0), scale)
    np.testing.assert_allclose(Ofw, o_t, atol=1e-11)
    np.testing.assert_allclose(dQ, dq_t, atol=1e-10)
    np.testing.assert_allclose(dK, dk_t, atol=1e-10)
    np.testing.assert_allclose(dV, dv_t, atol=1e-10)


# ---------------------------------------------------------------- P3: finite differences
def test_backward_finite_differences():
    rng = np.random.default_rng(7)
    lengths, Hq, Hk, D, B, K = [37, 26], 2, 1, 16, 8, 3
    T = sum(lengths)
    cu = np.array([0, 37, 63])
    q = rng.standard_normal((T, Hq, D))
    k = rng.standard_normal((T, Hk, D))
    v = rng.standard_normal((T, Hk, D))
    do = rng.standard_normal((T, Hq, D))
    # a sparse selection: own block plus up to two random earlier blocks
    seq, pos = O.sequence_layout(cu)
    blk = np.full((T, Hk, K), -1, np.int32)
    for i in range(T):
        b = pos[i] // B
        earlier = rng.permutation(b)[:K - 1] if b > 0 else []
        ids = sorted([b] + [int(c) for c in earlier])
        blk[i, 0, :len(ids)] = ids
    scale = 0.37

    def loss(q_, k_, v_):
        o, _ = O.attention_forward(q_, k_, v_, blk, cu, scale, block=B)
        return float((o * do).sum())

    dQ, dK, dV = O.attention_backward(q, k, v, do, blk, cu, scale, block=B)
    h = 1e-6
    for name, x, g in [("q", q, dQ), ("k", k, dK), ("v", v, dV)]:
        for _ in range(3):
            u = rng.standard_normal(x.shape)
            xp, xm = x + h * u, x - h * u
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            an = float((g * u).sum())
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


# ---------------------------------------------------------------- P7: GQA closed form
def test_gqa_identical_heads_closed_form():
    rng = np.random.default_rng(8)
    cu = np.array([0, 300])
    T, D, G = 300, 128, 16
    q1 = rng.standard_normal((T, 1, D))
    do1 = rng.standard_normal((T, 1, D))
    k = rng.standard_normal((T, 1, D))
    v = rng.standard_normal((T, 1, D))
    seq, pos = O.sequence_layout(cu)
    blk = np.full((T, 1, 16), -1, np.int32)
    for i in range(T):
        b = pos[i] // 128
        blk[i, 0, :b + 1] = np.arange(b + 1)
    s = 1 / math.sqrt(128)
    o1, l1 = O.attention_forward(q1, k, v, blk, cu, s)
    dq1, dk1, dv1 = O.attention_backward(q1, k, v, do1, blk, cu, s)
    qG = np.repeat(q1, G, axis=1)
    doG = np.repeat(do1, G, axis=1)
    oG, lG = O.attention_forward(qG, k, v, blk, cu, s)
    dqG, dkG, dvG = O.attention_backward(qG, k, v, doG, blk, cu, s)
    np.testing.assert_allclose(oG, np.repeat(o1, G, axis=1), atol=1e-12)
    np.testing.assert_allclose(lG, np.repeat(l1, G, axis=1), atol=1e-12)
    np.testing.assert_allclose(dqG, np.repeat(dq1, G, axis=1), atol=1e-11)
    np.testing.assert_allclose(dkG, G * dk1, atol=1e-9)
    np.testing.assert_allclose(dvG, G * dv1, atol=1e-9)


# ---------------------------------------------------------------- P8: q = 0 closed form
def test_zero_query_uniform_attention_closed_form():
    rng = np.random.default_rng(9)
    lengths = [400, 170]
    cu = np.array([0, 400, 570])
    T, Hq, Hk, D, B, K = 570, 2, 1, 32, 32, 4
    q = np.zeros((T, Hq, D))
    k = rng.standard_normal((T, Hk, D))
    v = rng.standard_normal((T, Hk, D))
    do = rng.standard_normal((T, Hq, D))
    seq, pos = O.sequence_layout(cu)
    blk = np.full((T, Hk, K), -1, np.int32)
    for i in range(T):
        b = pos[i] // B
        ids = sorted(set([b] + [int(c) for c in rng.integers(0, b + 1, K - 1)]))
        blk[i, 0, :len(ids)] = ids
    o, lse = O.attention_forward(q, k, v, blk, cu, 0.2, block=B)
    dq, dk, dv = O.attention_backward(q, k, v, do, blk, cu, 0.2, block=B)
    dv_want = np.zeros_like(dv)
    for i in range(T):
        s = seq[i]
        keys = []
        for c in blk[i, 0]:
            if c >= 0:
                keys += [int(cu[s]) + j for j in range(c * B, min(c * B + B, pos[i] + 1))]
        n = len(keys)
        vm = v[keys, 0].mean(axis=0)
        for g in range(Hq):
            np.testing.assert_allclose(o[i, g], vm, atol=1e-12)
            assert abs(lse[i, g] - math.log(n)) < 1e-12
            # dS_j = (dP_j - mean dP) / n ; dq = scale * sum_j dS_j k_j
            dP = v[keys, 0] @ do[i, g]
            dS = (dP - dP.mean()) / n
            np.testing.assert_allclose(dq[i, g], 0.2 * (dS @ k[keys, 0]), atol=1e-12)
            dv_want[keys, 0] += do[i, g] / n
    assert np.all(dk == 0)
    np.testing.assert_allclose(dv, dv_want, atol=1e-12)


# ---------------------------------------------------------------- attention-side q/k norm + RoPE (f2)
def _qk_loss(x, w, pos, dz):
    """sum(dz * z) with z the unrounded fp32 forward (norm then RoPE)."""
    z = O.indexer_features(x, w, pos, 1e-6, 1e7, 64, round_bf16=False)
    return float((np.asarray(z, np.float64) * dz).sum())


def test_qk_norm_rope_backward_finite_differences():
    rng = np.random.default_rng(11)
    N, H, D = 3, 2, 128
    x = rng.standard_normal((N, H, D)).astype(np.float32)
    w = (0.3 * rng.standard_normal(D)).astype(np.float32)
    pos = np.array([0, 5, 1234])
    dz = rng.standard_normal((N, H, D))
    dx, dw = O.qk_norm_rope_backward(x, w, pos, dz)
    h = 1e-2
    for (n, hh, d) in [(0, 0, 3), (1, 1, 40), (2, 0, 70), (2, 1, 127), (1, 0, 31), (0, 1, 32)]:
        xp, xm = x.copy(), x.copy()
        xp[n, hh, d] += h
        xm[n, hh, d] -= h
        fd = (_qk_loss(xp, w, pos, dz) - _qk_loss(xm, w, pos, dz)) / (2 * h)
        assert abs(fd - dx[n, hh, d]) <= 2e-3 * max(1.0, abs(dx[n, hh, d])), (n, hh, d, fd, dx[n, hh, d])
    for d in [0, 17, 33, 64, 100]:
        wp, wm = w.copy(), w.copy()
        wp[d] += h
        wm[d] -= h
        fd = (_qk_loss(x, wp, pos, dz) - _qk_loss(x, wm, pos, dz)) / (2 * h)
        assert abs(fd - dw[d]) <= 2e-3 * max(1.0, abs(dw[d])), (d, fd, dw[d])


def test_qk_norm_rope_backward_closed_forms():
    rng = np.random.default_rng(12)
    N, H, D = 4, 3, 128
    x = rng.standard_normal((N, H, D)).astype(np.float32)
    dz = rng.standard_normal((N, H, D))
    pos = np.array([0, 1, 77, 4000])
    # eps = 0: RMSNorm is scale-invariant, so the gradient is orthogonal to x
    w = (0.2 * rng.standard_normal(D)).astype(np.float32)
    dx, _ = O.qk_norm_rope_backward(x, w, pos, dz, eps=0.0)
    assert np.abs((dx * x).sum(axis=-1)).max() < 1e-9 * np.abs(dx).max() * D
    # w = -1: y = 0 for every x, so dx = 0, while dw_j = sum dy_j x_j r
    dx, dw = O.qk_norm_rope_backward(x, -np.ones(D, np.float32), pos, dz)
    assert np.abs(dx).max() == 0.0
    assert np.abs(dw).max() > 0
    # position 0: RoPE is the identity, so with w = 0 the backward is RMSNorm's alone,
    # r (dz - x r^2 mean(dz x)), for every head
    dx0, dw0 = O.qk_norm_rope_backward(x[:1], np.zeros(D, np.float32), pos[:1], dz[:1])
    xx = x[0].astype(np.float64)
    r = 1 / np.sqrt((xx * xx).mean(axis=-1) + 1e-6)
    want = r[:, None] * dz[0] - xx * (r ** 3 * (dz[0] * xx).mean(axis=-1))[:, None]
    assert np.allclose(dx0[0], want, rtol=1e-12, atol=1e-12)
    assert np.allclose(dw0, (dz[0] * xx * r[:, None]).sum(axis=0), rtol=1e-12, atol=1e-12)
    # rotation: dims >= 64 pass through RoPE, so with x fixed and dz nonzero only
    # there, the result does not depend on the position
    dzh = dz.copy()
    dzh[..., :64] = 0
    a, _ = O.qk_norm_rope_backward(x, w, np.array([0, 0, 0, 0]), dzh)
    b, _ = O.qk_norm_rope_backward(x, w, pos, dzh)
    assert np.allclose(a, b, rtol=0, atol=0)
