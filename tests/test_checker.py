"""The acceptance checker must accept correct results, accept any tie
resolution, and reject planted mistakes. CPU only."""
import itertools

import numpy as np

import mqa_workloads as W
import oracle
from oracle import check


def _cfg1():
    wl = W.config(1)
    p = oracle.Problem(wl.q, wl.k, oracle.key_scales(wl.scale_bytes), wl.weights, wl.starts,
                       wl.ends)
    return wl, p


def test_checker_accepts_oracle_and_rejects_planted_mistakes():
    wl, p = _cfg1()
    rows = [0, 31, 63]
    idx, kth, mx = oracle.topk(p, rows, wl.topk)
    assert check.check_topk(idx, rows, p, wl.topk) == []
    assert check.check_valid(idx, wl.starts, wl.ends, wl.keys, wl.topk, rows=rows) == []
    # shuffled order is fine (the output is unordered)
    shuf = idx[:, ::-1].copy()
    assert check.check_topk(shuf, rows, p, wl.topk) == []
    # swap the best selected key for the worst visible key
    s, e = p.visible(0)
    lg = oracle.logits(p, [0], col0=s, ncols=e - s)[0]
    worst = int(np.argmin(lg))
    bad = idx.copy()
    bad[0, 0] = worst
    assert check.check_topk(bad, rows, p, wl.topk)
    # duplicate
    bad = idx.copy()
    bad[1, 5] = bad[1, 6]
    assert check.check_topk(bad, rows, p, wl.topk)
    assert check.check_valid(bad, wl.starts, wl.ends, wl.keys, wl.topk, rows=rows)
    # out of range
    bad = idx.copy()
    bad[2, 0] = e - s + 3
    assert check.check_topk(bad, rows, p, wl.topk)
    assert check.check_valid(bad, wl.starts, wl.ends, wl.keys, wl.topk, rows=rows)


def test_checker_padding_rules():
    starts = np.array([0, 0, 5], np.int32)
    ends = np.array([3, 0, 4], np.int32)
    good = np.array([[2, 0, 1, -1, -1], [-1] * 5, [-1] * 5], np.int32)
    assert check.check_valid(good, starts, ends, 10, 5) == []
    bad = good.copy()
    bad[0] = [2, -1, 1, 0, -1]          # padding not trailing
    assert check.check_valid(bad, starts, ends, 10, 5)
    bad = good.copy()
    bad[1, 0] = 0                       # empty row must be all -1
    assert check.check_valid(bad, starts, ends, 10, 5)


def test_checker_accepts_any_tie_resolution():
    lg = np.array([5, 3, 3, 3, 1, 0], np.float32)
    assert check.check_topk_row(np.array([0, 1]), lg, 2) is None
    assert check.check_topk_row(np.array([0, 3]), lg, 2) is None
    assert check.check_topk_row(np.array([0, 4]), lg, 2) is not None
    assert check.check_topk_row(np.array([1, 2]), lg, 2) is not None


def test_lowkey_checker_pins():
    # ties at the cut go to the smallest keys; valid entries ascending
    lg = np.array([5, 3, 3, 3, 1, 0], np.float32)
    assert check.check_lowkey_row(np.array([0, 1]), lg, 2) is None
    assert check.check_lowkey_row(np.array([0, 3]), lg, 2) is not None  # key 1 left out
    assert check.check_lowkey_row(np.array([1, 0]), lg, 2) is not None  # not ascending
    assert check.check_lowkey_row(np.array([0, 1, 2]), lg, 3) is None
    assert check.check_lowkey_row(np.array([0, 2, 3]), lg, 3) is not None
    # short rows: 0..n-1 then -1
    assert check.check_lowkey_row(np.array([0, 1, -1]), lg[:2], 3) is None
    assert check.check_lowkey_row(np.array([0, -1, 1]), lg[:2], 3) is not None
    # against brute force: the (value desc, key asc) choice, sorted, passes both
    # rules; every other correct tie resolution fails the tie rule only
    rng = np.random.default_rng(3)
    for _ in range(200):
        n, k = int(rng.integers(2, 12)), int(rng.integers(1, 6))
        k = min(k, n - 1)
        v = rng.integers(0, 4, size=n).astype(np.float32)
        order = sorted(range(n), key=lambda j: (-v[j], j))
        want = np.sort(np.array(order[:k], np.int32))
        assert np.array_equal(np.sort(oracle.select(v, k)), want)
        assert check.check_lowkey_row(want, v, k) is None
        assert check.check_topk_row(want, v, k) is None
        tau = v[order[k - 1]]
        ties = [j for j in range(n) if v[j] == tau]
        taken = [j for j in want if v[j] == tau]
        if len(ties) > len(taken):
            alt = sorted(set(want.tolist()) - {max(taken)} | {max(ties)})
            alt = np.array(alt, np.int32)
            assert check.check_topk_row(alt, v, k) is None
            assert check.check_lowkey_row(alt, v, k) is not None


def test_checker_tolerance_is_relative_to_row_max():
    lg = np.array([1000.0, 10.0, 10.0 - 5e-3, 9.0], np.float32)
    # tol = 1e-5 * 1000 = 1e-2: keys within 1e-2 of the k-th score may swap
    assert check.check_topk_row(np.array([0, 2]), lg, 2) is None
    lg2 = np.array([1000.0, 10.0, 10.0 - 5e-2, 9.0], np.float32)
    assert check.check_topk_row(np.array([0, 2]), lg2, 2) is not None


def test_dense_checker():
    ref = np.array([[1.0, -np.inf, 2.0], [100.0, 50.0, -np.inf]], np.float32)
    assert check.check_dense(ref.copy(), ref) == []
    g = ref.copy()
    g[1, 1] += 100.0 * 2e-5
    assert check.check_dense(g, ref)
    g = ref.copy()
    g[0, 1] = 0.0
    assert check.check_dense(g, ref)
    g = ref.copy()
    g[1, 1] += 100.0 * 5e-6
    assert check.check_dense(g, ref) == []


def test_near_tie_workload_separates_groups_beyond_tolerance():
    # the near-tie workload is only a discriminating GPU case if the oracle
    # puts group A strictly above group B by more than the checker's tolerance
    # (yet less than 8 * 2^-18 of the row's size, the select's margin floor),
    # every other key well below, and the checker rejects a B key in place of
    # an A key
    wl = W.extra_near_tie_groups()
    p = oracle.Problem(wl.q, wl.k, oracle.key_scales(wl.scale_bytes), wl.weights, wl.starts,
                       wl.ends)
    a, b = wl.groups["group_a"], wl.groups["group_b"]
    rest = np.setdiff1d(np.arange(wl.keys), np.concatenate([a, b]))
    lg = oracle.logits(p, [0, 1]).astype(np.float64)
    for r in range(2):
        la, lb, lr = lg[r, a], lg[r, b], lg[r, rest]
        assert la.min() == la.max() and lb.min() == lb.max()
        gap = (la[0] - lb[0]) / la[0]
        assert check.REL_TOL < gap < 8 * 2.0 ** -18, gap
        assert lr.max() < 0.5 * lb[0]
        sel = a[:wl.topk].copy()
        assert check.check_topk_row(sel, lg[r].astype(np.float32), wl.topk) is None
        sel[0] = b[0]
        assert check.check_topk_row(sel, lg[r].astype(np.float32), wl.topk) is not None


# ------------------------------------------------ two-level selection checks

def test_block_maxima_against_loops():
    rng = np.random.default_rng(0)
    for s, e in ((0, 64), (3, 50), (8, 9), (13, 13), (5, 200)):
        lg = rng.standard_normal(e - s)
        got = check.block_maxima(s, e, lg)
        want = []
        for b in range(s // 8, (e - 1) // 8 + 1 if e > s else s // 8):
            keys = [j for j in range(8 * b, 8 * b + 8) if s <= j < e]
            want.append(max(lg[j - s] for j in keys))
        assert np.array_equal(got, np.array(want)), (s, e)


def test_masked_positions_against_loops():
    s, e = 13, 90
    blocks = np.array([0, 3, -1, 10, 3, 2, -5])
    want = sorted({j - s for b in (0, 3, 10, 2) for j in range(8 * (b + s // 8), 8 * (b + s // 8) + 8)
                   if s <= j < e})
    assert check.masked_positions(s, e, blocks).tolist() == want


def test_select_row_rule_against_brute_force():
    rng = np.random.default_rng(1)
    for _ in range(200):
        n = int(rng.integers(1, 9))
        k = int(rng.integers(1, 6))
        v = rng.integers(0, 4, n).astype(np.float64)
        m = min(n, k)
        best = sorted(v, reverse=True)[m - 1] if m else None
        for sub in itertools.combinations(range(n), m):
            sel = np.array(list(sub) + [-1] * (k - m))
            # a subset is a correct top-k iff no left-out value beats a taken one
            taken = v[list(sub)]
            left = np.delete(v, list(sub))
            good = n <= k or (taken.min() >= (left.max() if left.size else -np.inf))
            assert (check.check_select_row(sel, v, k, 0.0) is None) == good, (v, k, sub)
    assert check.check_select_row(np.array([0, 0]), np.array([1.0, 2.0, 3.0]), 2, 0.0)
    assert check.check_select_row(np.array([2, -1, 1]), np.array([1.0, 2.0, 3.0]), 3, 0.0)
