"""Acceptance rules for a top-k / dense-logits result against the oracle.

Test infrastructure (same rules as the rest of ``oracle/``). The rules:

(i)   validity, on every row: min(n, k) valid entries, distinct, inside
      [0, n), in the leading slots; the remaining k - min(n, k) slots hold -1
      (the API page's fused_mqa_topk_prefill: each index is the key minus
      the row's start, in no particular order; rows with fewer than k
      visible keys fill the unused slots with -1).
(ii)  set rule, on rows with n > k: with tau the oracle's k-th largest logit
      and tol = rel_tol * max|logit| of the row, every selected key has logit
      >= tau - tol and every visible unselected key has logit <= tau + tol.
      This accepts any resolution of ties at the boundary (the API page's
      use_fused_mqa_topk: which of several keys tied at the k-th score the
      fused op keeps depends on the order of its atomic updates).
(iii) dense logits: |gpu - oracle| <= tol on visible entries; -inf exactly
      where the oracle has -inf.
"""
from __future__ import annotations

import numpy as np

REL_TOL = 1e-5


def visible_ranges(starts, ends, keys):
    s = np.clip(np.asarray(starts, np.int64), 0, keys)
    e = np.clip(np.asarray(ends, np.int64), s, keys)
    return s, e


def check_valid(out: np.ndarray, starts, ends, keys: int, topk: int, rows=None):
    """Rule (i). out: [R, topk] int32 for rows `rows` (default: all).
    Returns a list of (row, message) failures (empty when valid)."""
    out = np.asarray(out)
    s, e = visible_ranges(starts, ends, keys)
    if rows is not None:
        rows = np.asarray(rows)
        s, e = s[rows], e[rows]
    else:
        rows = np.arange(out.shape[0])
    assert out.shape == (rows.shape[0], topk), out.shape
    n = e - s
    m = np.minimum(n, topk)
    fails = []
    slot = np.arange(topk)[None, :]
    lead = slot < m[:, None]
    # leading slots inside [0, n); trailing slots exactly -1
    bad_lead = lead & ((out < 0) | (out >= n[:, None]))
    bad_tail = (~lead) & (out != -1)
    for i in np.nonzero(bad_lead.any(axis=1) | bad_tail.any(axis=1))[0][:20]:
        fails.append((int(rows[i]), "index out of range or padding misplaced"))
    # distinctness of the leading entries
    srt = np.sort(np.where(lead, out, -1 - slot), axis=1)
    dup = (np.diff(srt, axis=1) == 0) & (srt[:, 1:] >= 0)
    for i in np.nonzero(dup.any(axis=1))[0][:20]:
        fails.append((int(rows[i]), "duplicate index"))
    return fails


def check_topk_row(sel_idx: np.ndarray, row_logits: np.ndarray, topk: int,
                   rel_tol: float = REL_TOL):
    """Rule (ii) for one row. row_logits: fp32 [n], the oracle's logits of the
    row's visible keys (position = key - start). sel_idx: the result's [topk]
    entries. Returns None when accepted, else a message."""
    n = row_logits.shape[0]
    if n <= topk:
        want = np.concatenate([np.arange(n), np.full(topk - n, -1)])
        got = np.concatenate([np.sort(sel_idx[:n]), sel_idx[n:]])
        return None if np.array_equal(got, want) else "short row not 0..n-1 then -1"
    if np.any(sel_idx < 0) or np.any(sel_idx >= n):
        return "index outside the visible range"
    if np.unique(sel_idx).shape[0] != topk:
        return "duplicate index"
    lg = row_logits.astype(np.float64)
    tau = np.partition(lg, n - topk)[n - topk]
    tol = rel_tol * float(np.max(np.abs(lg)))
    chosen = np.zeros(n, bool)
    chosen[sel_idx] = True
    lo = lg[chosen].min()
    hi = lg[~chosen].max()
    if lo < tau - tol:
        return f"selected logit {lo!r} below tau {tau!r} - tol {tol!r}"
    if hi > tau + tol:
        return f"unselected logit {hi!r} above tau {tau!r} + tol {tol!r}"
    return None


def check_lowkey_row(sel_row: np.ndarray, row_logits: np.ndarray, topk: int):
    """The deterministic tie rule for one row, on the oracle's logits of its
    visible keys (position = key - start): valid entries in ascending order,
    then -1; and no key left out scores exactly the smallest selected logit
    while being smaller than a selected key of that score (ties at the cut go
    to the smallest keys). Returns None when it holds, else a message."""
    sel_row = np.asarray(sel_row)
    n = row_logits.shape[0]
    m = min(n, topk)
    lead = sel_row[:m]
    if np.any(sel_row[m:] != -1):
        return "padding is not trailing -1"
    if m > 1 and np.any(np.diff(lead) <= 0):
        return "valid entries not in ascending key order"
    if n <= topk:
        return None
    chosen = np.zeros(n, bool)
    chosen[lead] = True
    cut = row_logits[chosen].min()
    at_cut = row_logits == cut
    taken = np.nonzero(at_cut & chosen)[0]
    left = np.nonzero(at_cut & ~chosen)[0]
    if left.size and taken.size and left.min() < taken.max():
        return (f"tie at the cut {cut!r}: key {int(left.min())} left out, "
                f"key {int(taken.max())} taken")
    return None


def check_lowkey(out_rows: np.ndarray, rows, oracle_problem, topk: int, batch: int = 16,
                 threads: int = 0):
    """check_lowkey_row on the given rows (oracle logits a batch at a time)."""
    import oracle  # test infrastructure: this module lives beside it

    rows = np.asarray(rows, np.int32)
    fails = []
    for lo in range(0, rows.shape[0], batch):
        rb = rows[lo:lo + batch]
        rng = [oracle_problem.visible(int(r)) for r in rb]
        c0 = min(s for s, _ in rng)
        c1 = max(e for _, e in rng)
        lg = oracle.logits(oracle_problem, rb, col0=c0, ncols=max(c1 - c0, 1), threads=threads)
        for i, r in enumerate(rb):
            s, e = rng[i]
            msg = check_lowkey_row(np.asarray(out_rows[lo + i]), lg[i, s - c0:e - c0], topk)
            if msg:
                fails.append((int(r), msg))
    return fails


def check_topk(out_rows: np.ndarray, rows, oracle_problem, topk: int,
               rel_tol: float = REL_TOL, batch: int = 16, threads: int = 0):
    """Rule (ii) on the given rows. out_rows: [len(rows), topk] result rows.
    The oracle's logits are computed a batch of rows at a time over the
    batch's union key range (bounded memory, all cores)."""
    import oracle  # test infrastructure: this module lives beside it

    rows = np.asarray(rows, np.int32)
    fails = []
    for lo in range(0, rows.shape[0], batch):
        rb = rows[lo:lo + batch]
        rng = [oracle_problem.visible(int(r)) for r in rb]
        c0 = min(s for s, _ in rng)
        c1 = max(e for _, e in rng)
        lg = oracle.logits(oracle_problem, rb, col0=c0, ncols=max(c1 - c0, 1), threads=threads)
        for i, r in enumerate(rb):
            s, e = rng[i]
            msg = check_topk_row(np.asarray(out_rows[lo + i]), lg[i, s - c0:e - c0], topk,
                                 rel_tol)
            if msg:
                fails.append((int(r), msg))
    return fails


def check_dense(gpu: np.ndarray, ref: np.ndarray, rel_tol: float = REL_TOL):
    """Rule (iii). gpu/ref: fp32 [R, C]. The tolerance of each row is rel_tol
    times the row's max |ref| over finite entries. Returns failures."""
    gpu = np.asarray(gpu, np.float32)
    ref = np.asarray(ref, np.float32)
    fails = []
    inf_ref = np.isneginf(ref)
    inf_gpu = np.isneginf(gpu)
    bad_inf = inf_ref != inf_gpu
    fin = ~inf_ref
    mx = np.where(fin, np.abs(ref), 0).max(axis=1, keepdims=True)
    with np.errstate(invalid="ignore"):
        diff = np.where(fin, np.abs(gpu.astype(np.float64) - ref.astype(np.float64)), 0)
    bad = (diff > rel_tol * mx) | bad_inf | np.isnan(gpu)
    for r in np.nonzero(bad.any(axis=1))[0][:20]:
        c = int(np.nonzero(bad[r])[0][0])
        fails.append((int(r), f"col {c}: gpu {gpu[r, c]!r} ref {ref[r, c]!r}"))
    return fails
