"""The dense baseline's per-row top-k (mqa_topk_dense, vLLM PR #60618,
"Motivation": the top-k pass over the written logits) on crafted fp32 logits,
through the C ABI. The selection of given fp32 values is exact, so every row
is checked exactly: valid unique positions, min(n, k) of them, every selected
value at or above the k-th largest and every value above it selected. The
rows cover the three routes of the kernel: rows held in LDS (n <= 8192), the
sampled single pass, and its fall-back radix select (constant rows, few
distinct values, sorted and heavy-tailed rows)."""
import numpy as np
import pytest
import torch

import fp8_mqa_logits_amd as mqa

from gpu_helpers import say

pytestmark = pytest.mark.gpu


def _row(kind, n, rng):
    if kind == "gauss":
        return rng.standard_normal(n).astype(np.float32)
    if kind == "const":
        return np.full(n, 1.5, np.float32)
    if kind == "few":
        return rng.integers(0, 5, n).astype(np.float32)
    if kind == "asc":
        return np.sort(rng.standard_normal(n).astype(np.float32))
    if kind == "desc":
        return np.sort(rng.standard_normal(n).astype(np.float32))[::-1].copy()
    if kind == "tail":
        return rng.exponential(1.0, n).astype(np.float32) ** 4
    if kind == "neg":
        return -np.abs(rng.standard_normal(n).astype(np.float32)) - 1000.0
    raise ValueError(kind)


KINDS = ["gauss", "const", "few", "asc", "desc", "tail", "neg"]


def _check_row(o, vals, k, shift):
    n = vals.shape[0]
    sel = o[o >= 0]
    assert sel.shape[0] == min(n, k)
    assert (o[sel.shape[0]:] == -1).all()
    if n == 0:
        return
    pos = sel - shift
    assert pos.min() >= 0 and pos.max() < n
    assert np.unique(pos).shape[0] == pos.shape[0]
    if n <= k:
        return
    vk = np.sort(vals)[-k]
    got = vals[pos]
    assert (got >= vk).all()
    assert (got > vk).sum() == (vals > vk).sum()


@pytest.mark.parametrize("topk", [512, 2048])
def test_dense_topk_crafted(topk):
    rng = np.random.default_rng(11)
    keys, col0 = 140000, 3000
    ncols = keys - col0 - 1
    lens = [0, 100, topk, topk + 1, 5000, 8192, 8193, 20000, 65536, 136999]
    rows = []
    for n in lens:
        for kind in KINDS:
            rows.append((n, kind))
    R = len(rows)
    ld = (ncols + 3) // 4 * 4 + 4
    logits = np.full((R, ld), np.nan, np.float32)
    starts = np.zeros(R, np.int32)
    ends = np.zeros(R, np.int32)
    for r, (n, kind) in enumerate(rows):
        s = col0 + int(rng.integers(0, ncols - n + 1))  # ragged, unaligned offsets
        starts[r], ends[r] = s, s + n
        logits[r, s - col0:s - col0 + n] = _row(kind, n, rng)
    say(f"case: dense top-k of crafted logits, {R} rows, k={topk}")
    lg = torch.from_numpy(logits).cuda()[:, :ncols]
    out = mqa.mqa_topk_dense(lg, torch.from_numpy(starts).cuda(), torch.from_numpy(ends).cuda(),
                             topk, keys, col0=col0)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    for r, (n, kind) in enumerate(rows):
        s = int(starts[r])
        vals = logits[r, s - col0:s - col0 + n]
        try:
            _check_row(o[r], vals, topk, 0)
        except AssertionError:
            raise AssertionError(f"row {r}: n={n} kind={kind}")


def test_dense_topk_window_clips_range():
    # rows whose ranges start before or end after the window: only the
    # window's part of the range is ranked, output relative to the start
    rng = np.random.default_rng(12)
    keys, col0, ncols, k = 50000, 10000, 30000, 1024
    R = 6
    starts = np.array([0, 5000, 12000, 9000, 39000, 30000], np.int32)
    ends = np.array([50000, 41000, 38000, 12000, 50000, 30500], np.int32)
    logits = rng.standard_normal((R, ncols)).astype(np.float32)
    say("case: dense top-k, ranges clipped by the window")
    out = mqa.mqa_topk_dense(torch.from_numpy(logits).cuda(), torch.from_numpy(starts).cuda(),
                             torch.from_numpy(ends).cuda(), k, keys, col0=col0)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    for r in range(R):
        lo = max(int(starts[r]), col0)
        hi = min(int(ends[r]), col0 + ncols)
        vals = logits[r, lo - col0:max(hi, lo) - col0]
        # output is key - start; position in vals is key - lo
        _check_row(o[r], vals, k, lo - int(starts[r]))
