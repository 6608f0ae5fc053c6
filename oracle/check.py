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


# --------------------------------------------------------------------------
# DeepSeek-V4.1 two-level candidate selection (vLLM PR #60618, "Limitations
# of this PR -- TODOs"): the source layer also ranks blocks of 8 keys by their
# maximum score; consumer layers keep only the keys of given blocks before
# their top-k. Reading: blocks are 8 consecutive keys of the call's key
# numbering, block B = keys [8B, 8B + 8); a row names block B as B - s // 8
# (s its clamped start), and a block's score for a row is the maximum logit
# over the row's visible keys in it.

def masked_positions(s: int, e: int, blocks_row) -> np.ndarray:
    """Sorted distinct positions (key - s) of the row's visible keys that lie
    in its listed blocks (entries < 0 are padding)."""
    b = np.unique(np.asarray(blocks_row, np.int64))
    b = b[b >= 0]
    keys = ((b[:, None] + s // 8) * 8 + np.arange(8)[None, :]).reshape(-1)
    keys = keys[(keys >= s) & (keys < e)]
    return keys - s


def block_maxima(s: int, e: int, row_logits: np.ndarray) -> np.ndarray:
    """Block scores of a row: entry i is block s // 8 + i (i.e. named i), the
    maximum of row_logits (logits of keys s..e-1) over the block's visible
    keys; blocks i = 0 .. (e - 1) // 8 - s // 8 (none when e == s)."""
    if e <= s:
        return np.zeros(0, np.float64)
    b0 = s // 8
    nb = (e - 1) // 8 - b0 + 1
    full = np.full(nb * 8, -np.inf)
    full[s - 8 * b0: e - 8 * b0] = row_logits
    return full.reshape(nb, 8).max(1)


def check_select_row(sel: np.ndarray, values: np.ndarray, k: int, tol: float):
    """The acceptance rule on a compact set: sel holds indices into values;
    min(n, k) distinct valid ones then -1; every chosen value at least the
    k-th largest minus tol, every other at most it plus tol."""
    sel = np.asarray(sel)
    n = values.shape[0]
    m = min(n, k)
    lead, tail = sel[:m], sel[m:]
    if np.any(tail != -1):
        return "padding is not trailing -1"
    if np.any(lead < 0) or np.any(lead >= n):
        return "index outside the candidates"
    if np.unique(lead).shape[0] != m:
        return "duplicate index"
    if n <= k:
        return None
    v = values.astype(np.float64)
    tau = np.partition(v, n - k)[n - k]
    chosen = np.zeros(n, bool)
    chosen[lead] = True
    if v[chosen].min() < tau - tol:
        return f"selected value {v[chosen].min()!r} below tau {tau!r} - tol {tol!r}"
    if v[~chosen].max() > tau + tol:
        return f"unselected value {v[~chosen].max()!r} above tau {tau!r} + tol {tol!r}"
    return None


def _row_logits(oracle_problem, rows, threads=0):
    import oracle  # test infrastructure: this module lives beside it
    for r in np.asarray(rows, np.int32):
        s, e = oracle_problem.visible(int(r))
        lg = oracle.logits(oracle_problem, [int(r)], col0=s, ncols=max(e - s, 1),
                           threads=threads)[0, : e - s]
        yield int(r), s, e, lg


def check_topk_masked(out_rows, rows, oracle_problem, blocks, topk: int,
                      rel_tol: float = REL_TOL):
    """Consumer rows: out_rows[i] (key - s entries) must be the top-k of row
    rows[i]'s keys in its listed blocks (blocks[rows[i]])."""
    fails = []
    for i, (r, s, e, lg) in enumerate(_row_logits(oracle_problem, rows)):
        pos = masked_positions(s, e, blocks[r])
        out = np.asarray(out_rows[i])
        idx = np.full(out.shape, -1, np.int64)
        valid = out >= 0
        where = np.searchsorted(pos, out[valid])
        ok = (where < pos.shape[0]) & (pos[np.minimum(where, max(pos.shape[0] - 1, 0))] == out[valid]) \
            if pos.shape[0] else np.zeros(int(valid.sum()), bool)
        if not np.all(ok):
            fails.append((r, "selected key outside the row's blocks"))
            continue
        idx[valid] = where
        tol = rel_tol * float(np.max(np.abs(lg))) if lg.size else 0.0
        msg = check_select_row(idx, lg[pos].astype(np.float64), topk, tol)
        if msg:
            fails.append((r, msg))
    return fails


def check_blocks(out_blocks, rows, oracle_problem, nbo: int, rel_tol: float = REL_TOL):
    """Source rows: out_blocks[i] must name the nbo blocks of largest score of
    row rows[i] (block_maxima), unordered, -1 padded."""
    fails = []
    for i, (r, s, e, lg) in enumerate(_row_logits(oracle_problem, rows)):
        bm = block_maxima(s, e, lg)
        tol = rel_tol * float(np.max(np.abs(lg))) if lg.size else 0.0
        msg = check_select_row(np.asarray(out_blocks[i]), bm, nbo, tol)
        if msg:
            fails.append((r, msg))
    return fails
