"""64 index heads (DeepSeek-V3.2's indexer; PR #60618 lists it as not yet
supported) through mqa_topk_prefill_heads, against the oracle with the same
64 heads, through the C ABI. A 64-head row runs as two 32-head halves whose
scores and error bounds are added; the deterministic mode must give the same
rows bit for bit whichever route (certified select, bounded rescan, exact
rescan) serves them."""
import numpy as np
import pytest
import torch

import fp8_mqa_logits_amd as mqa
import mqa_workloads as W
from oracle import check

from gpu_helpers import oracle_problem, say, to_device

pytestmark = pytest.mark.gpu
TOL = 1e-5


def _causal(rows, keys, first_end):
    ends = np.minimum(first_end + np.arange(rows), keys).astype(np.int32)
    return np.zeros(rows, np.int32), ends


def _ragged(rows, keys, seed):
    rng = np.random.default_rng(seed)
    s = rng.integers(0, keys // 4, rows).astype(np.int32)
    e = (s + rng.integers(0, keys, rows)).clip(max=keys).astype(np.int32)
    e[::17] = s[::17]  # empty rows
    e[5::23] = s[5::23] + 300  # short rows
    return s, e


def _run(wl, flags=0, ws=None):
    d = to_device(wl)
    out = mqa.mqa_topk_prefill(d["q"], d["k"], d["scales"], d["weights"], d["starts"], d["ends"],
                               wl.topk, flags=flags, workspace=ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


CASES = {
    "ragged_8k_k512": lambda: W.heads64(256, 8192, 512, *_ragged(256, 8192, 1), seed=1),
    "causal_32k_k1024": lambda: W.heads64(2048, 32768, 1024, *_causal(2048, 32768, 30721), seed=2),
}


@pytest.mark.parametrize("flags", [mqa.FLAG_DETERMINISTIC, 0])
@pytest.mark.parametrize("case", list(CASES))
def test_heads64_parity(case, flags):
    wl = CASES[case]()
    say(f"case: 64 heads {case}, flags={flags}")
    got = _run(wl, flags)
    assert not check.check_valid(got, wl.starts, wl.ends, wl.keys, wl.topk)
    rows = W.sample_rows(wl, 256)
    fails = check.check_topk(got[rows], rows, oracle_problem(wl), wl.topk, TOL)
    assert not fails, fails[:5]


def test_heads64_deterministic_routes_agree():
    wl = CASES["ragged_8k_k512"]()
    say("case: 64 heads, deterministic, default vs forced exact vs forced rescan")
    base = _run(wl, mqa.FLAG_DETERMINISTIC)
    for f in (mqa.FLAG_FORCE_EXACT, mqa.FLAG_FORCE_RESCAN, mqa.FLAG_SMALL_CAP):
        say(f"  route flag {f}")
        assert np.array_equal(_run(wl, mqa.FLAG_DETERMINISTIC | f), base), f


def test_heads64_full_size_sampled():
    # 16384 rows (two batches of 8192) x 131072 keys, top-2048, causal tail
    wl = W.heads64(16384, 131072, 2048, *_causal(16384, 131072, 114689), seed=3,
                   name="heads64_16384x131072_k2048")
    say(f"case: {wl.name}")
    d = to_device(wl)
    ws = torch.empty(mqa.workspace_size_heads(wl.rows, 64), dtype=torch.uint8, device="cuda")
    out = mqa.mqa_topk_prefill(d["q"], d["k"], d["scales"], d["weights"], d["starts"],
                               d["ends"], wl.topk, workspace=ws, flags=mqa.FLAG_STATS)
    torch.cuda.synchronize()
    st = mqa.read_stats(ws)  # the second batch's counters
    say(f"  stats {st}")
    got = out.cpu().numpy()
    assert not check.check_valid(got, wl.starts, wl.ends, wl.keys, wl.topk)
    rows = np.sort(np.concatenate([W.sample_rows(wl, 48), [0, 8191, 8192, 16383]]))
    fails = check.check_topk(got[rows], rows, oracle_problem(wl), wl.topk, TOL)
    assert not fails, fails[:5]
    assert st["rows_exact"] == 0 and st["bound_ratio_max"] < 1.0
