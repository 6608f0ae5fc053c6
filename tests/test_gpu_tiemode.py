"""Deterministic tie mode (MQA_FLAG_DETERMINISTIC) through the C ABI: each
row's output is the k keys of largest exact score with ties at the k-th score
going to the smallest keys, in ascending key order. Checked against the oracle
(acceptance rule (ii) and the tie rule on the oracle's logits, exact where
keys repeat), across the fused path's internal routes (forced exact rescan,
forced bounded rescan, small slab cap: bitwise equal outputs) and across batch
compositions (the same rows in another order or another call: bitwise equal)."""
import numpy as np
import pytest
import torch

import fp8_mqa_logits_amd as mqa
import mqa_workloads as W
from oracle import check

from gpu_helpers import fused, oracle_problem, say, to_device

pytestmark = pytest.mark.gpu

TOL = 1e-5
DET = mqa.FLAG_DETERMINISTIC
ROUTES = (0, mqa.FLAG_FORCE_EXACT, mqa.FLAG_FORCE_RESCAN, mqa.FLAG_SMALL_CAP)


def _check_rows(o, wl, rows):
    assert not check.check_valid(o, wl.starts, wl.ends, wl.keys, wl.topk)
    p = oracle_problem(wl)
    fails = check.check_topk(o[rows], rows, p, wl.topk, TOL)
    assert not fails, fails[:5]
    fails = check.check_lowkey(o[rows], rows, p, wl.topk)
    assert not fails, fails[:5]


def _permuted(d, perm):
    pt = torch.from_numpy(perm.astype(np.int64)).to(d["q"].device)
    e = dict(d)
    for name in ("q", "weights", "starts", "ends"):
        e[name] = d[name].index_select(0, pt).contiguous()
    return e


def _routes_agree(d, wl):
    base = fused(d, wl.topk, flags=DET).cpu().numpy()
    for flags in ROUTES[1:]:
        say(f"  route flags={flags}")
        o = fused(d, wl.topk, flags=DET | flags).cpu().numpy()
        bad = np.nonzero((o != base).any(axis=1))[0]
        assert bad.size == 0, (flags, bad[:10])
    return base


@pytest.mark.parametrize("cfg", [1, 2])
def test_det_routes_and_batch_invariance(cfg):
    wl = W.config(cfg)
    say(f"case: deterministic mode, config {cfg}: routes {ROUTES}, reversed rows")
    d = to_device(wl)
    o = _routes_agree(d, wl)
    rows = np.arange(wl.rows) if cfg == 1 else W.sample_rows(wl, 128)
    _check_rows(o, wl, rows)
    perm = np.arange(wl.rows)[::-1].copy()
    o2 = fused(_permuted(d, perm), wl.topk, flags=DET).cpu().numpy()
    assert np.array_equal(o2, o[perm])


def test_det_repeated_keys():
    # keys repeated from 256 (vector, scale) pairs: exact ties at every rank
    wl = W.extra_repeated_keys()
    say(f"case: deterministic mode, {wl.name}: routes, all rows, every third row alone")
    d = to_device(wl)
    o = _routes_agree(d, wl)
    _check_rows(o, wl, np.arange(wl.rows))
    sub = np.arange(0, wl.rows, 3)
    o2 = fused(_permuted(d, sub), wl.topk, flags=DET).cpu().numpy()
    assert np.array_equal(o2, o[sub])


def test_det_edge_ranges():
    keys, topk = 5000, 512
    starts = [0, 0, 100, 4000, -50, 4990, 3000, 10, 0, 2500, 0, 0, 7, 700]
    ends = [5000, 512, 612, 4513, 900, 6000, 2000, 10, 513, 5000, 1, 4999, 4900, 701]
    rows = 77
    st = np.array((starts * 6)[:rows], np.int32)
    en = np.array((ends * 6)[:rows], np.int32)
    wl = W.custom(rows, keys, topk, st, en, seed=9)
    say("case: deterministic mode, edge ranges, 77 rows, all routes")
    d = to_device(wl)
    o = _routes_agree(d, wl)
    _check_rows(o, wl, np.arange(rows))


def test_det_config5_sampled():
    # 1M keys drawn from 16 vectors: thousands of keys tie at each row's cut
    wl = W.config(5)
    say(f"case: deterministic mode, {wl.name}: 64 sampled rows, rows 16..4111 alone")
    d = to_device(wl)
    ws = mqa.alloc_workspace(wl.rows)
    o = fused(d, wl.topk, flags=DET | mqa.FLAG_STATS, workspace=ws).cpu().numpy()
    say("stats", mqa.read_stats(ws))
    sub = np.arange(16, 4112)
    o2 = fused(_permuted(d, sub), wl.topk, flags=DET).cpu().numpy()
    del d
    assert np.array_equal(o2, o[sub])
    _check_rows(o, wl, W.sample_rows(wl, 64))
