"""Comparison helpers shared by the GPU parity tests (no arithmetic of the method).

Bars:
* selection: identical block sets on every row except near ties (oracle
  16th/17th relative gap < 1e-3).  A row that differs inside a near tie must
  still be a correct selection once near ties may go either way (checked with
  the oracle's scores); the count of such rows is printed and returned.
* O: max-abs <= 2e-2; LSE: max-abs <= 1e-3.
* dQ, dK, dV: Frobenius-relative <= 1e-2 per tensor, and element by element:
  every row (one token and head: 128 values) must satisfy
  ``|g - g*| <= ROW_REL * |g*| + ROW_ABS * rms_row(g*)`` in the 2-norm, where
  rms_row is the root-mean-square row norm of the reference tensor, and
  ``max|g - g*| <= MAX_REL * max|g*|`` over the tensor.  The bf16 output
  rounding alone is 2^-9 relative per element; bf16 P and dS operands add
  errors of the same order, so a correct kernel sits near 3e-3 per row.  A row
  that is wrong (dropped key, wrong block, stale value) is off by O(1) of its
  own norm and fails.
  dQ rows get a larger absolute floor (ROW_ABS_DQ).  A dQ row is
  scale * sum_j dS_j k_j over the query's keys, and the softmax makes
  sum_j dS_j = 0 exactly, so for a query with few keys (the first tokens of a
  sequence) the exact row is a small difference of large terms.  The kernel
  rounds each dS_j to bf16 (2^-9 relative) and takes Delta from the bf16 O; those
  errors do not cancel, which leaves an absolute error of about
  2^-9 * scale * sum_j |dS_j| |k_j| however small the exact row is: up to
  0.033 of the rms row norm on the tested packs.  dK and dV rows sum over many
  (query, head) pairs with no such constraint (worst 0.0016 of the rms).
"""
import numpy as np

import oracle as O

O_TOL = 2e-2
LSE_TOL = 1e-3
G_TOL = 1e-2
ROW_REL = 2e-2
ROW_ABS = 1e-2
ROW_ABS_DQ = 1e-1
MAX_REL = 2e-2
TIE = 1e-3


def say(*a):
    print(*a, flush=True)


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def grad_stats(got, want, row_abs=ROW_ABS):
    """(Frobenius rel, worst row ratio to its bound, max-abs / max|want|, text on the worst rows)."""
    g = np.asarray(got, np.float64)
    w = np.asarray(want, np.float64)
    d = g.shape[-1]
    g2, w2 = g.reshape(-1, d), w.reshape(-1, d)
    if not w2.size:
        return 0.0, 0.0, 0.0, ""
    wn = np.linalg.norm(w2, axis=1)
    en = np.linalg.norm(g2 - w2, axis=1)
    rms = float(np.sqrt(np.mean(wn * wn)))
    bound = ROW_REL * wn + row_abs * rms
    ratio = en / np.maximum(bound, 1e-30)
    worst = float(ratio.max())
    top = np.argsort(-ratio)[:3]
    lead = w.shape[:-1]
    info = "; ".join(f"row {np.unravel_index(i, lead)}: |err| {en[i]:.2e} |ref| {wn[i]:.2e}" for i in top)
    info += f"; rms row norm {rms:.2e}"
    mx = float(np.abs(w2).max())
    mrel = float(np.abs(g2 - w2).max() / max(mx, 1e-30))
    return rel(g, w), worst, mrel, info


def check_grad(label, name, got, want, tol=G_TOL):
    """Frobenius, per-row and max-abs bars for one gradient tensor.  A tensor
    named dQ / dq (a query gradient) takes the dQ row floor."""
    row_abs = ROW_ABS_DQ if name.lower().startswith("dq") else ROW_ABS
    fro, worst, mrel, info = grad_stats(got, want, row_abs)
    say(f"[{label}] {name}: rel {fro:.3e}, worst row {worst:.3f} of its bound, max-abs {mrel:.3e} of max")
    if worst > 0.5:
        say(f"[{label}] {name} worst rows: {info}")
    assert fro <= tol, (label, name, fro)
    assert worst <= 1.0, (label, name, worst)
    assert mrel <= MAX_REL, (label, name, mrel)
    return fro


def check_out(label, o, want_o, lse=None, want_lse=None):
    eo = float(np.abs(np.asarray(o, np.float64) - want_o).max()) if np.size(want_o) else 0.0
    msg = f"[{label}] O maxabs={eo:.3e}"
    el = 0.0
    if lse is not None:
        fin = np.isfinite(want_lse)
        assert np.array_equal(np.isfinite(lse), fin), label
        el = float(np.abs(np.asarray(lse)[fin] - want_lse[fin]).max()) if fin.any() else 0.0
        msg += f" LSE maxabs={el:.3e}"
    say(msg)
    assert eo <= O_TOL and el <= LSE_TOL, (label, eo, el)
    return eo, el


def check_select(res, gpu_blk, label, topk=16, force_init=False):
    """Selection parity; ``res`` from the oracle's index_select (with
    keep_scores=True, so rows differing inside a near tie can be validated).
    Returns (rows, near-tie rows, mismatches inside near ties)."""
    g = np.asarray(gpu_blk)[res.rows]
    diff = (g != res.blk_idx).any(axis=2)
    tie = res.near_tie(TIE)
    bad = diff & ~tie
    in_tie = diff & tie
    say(f"[{label}] select rows={diff.size} near-tie={int(tie.sum())} "
        f"mismatch-in-ties={int(in_tie.sum())} mismatch-outside={int(bad.sum())}")
    assert bad.sum() == 0, np.argwhere(bad)[:10]
    if in_tie.any():
        assert res.scores is not None, "keep_scores=True is needed to validate rows that differ inside ties"
        for n, h in np.argwhere(in_tie):
            own = int(max(c for c in res.blk_idx[n, h] if c >= 0))
            ok = O.selection_valid_within_ties(res.scores[n, h], own, list(g[n, h]), topk, TIE, force_init)
            assert ok, (label, int(res.rows[n]), int(h), list(g[n, h]), list(res.blk_idx[n, h]))
    return int(diff.size), int(tie.sum()), int(in_tie.sum())
