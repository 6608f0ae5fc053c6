"""The allocation-free entry point (mqa_topk_prefill_static, the library's own
device scratch) against mqa_topk_prefill with a workspace, through the C ABI:
two calls in a row, the second over a smaller input. In the deterministic mode
the two entry points must agree bitwise; in the default mode both must pass
the oracle's acceptance rule on every row (ties at the k-th score may be
taken differently)."""
import numpy as np
import pytest
import torch

import fp8_mqa_logits_amd as mqa
import mqa_workloads as W
from oracle import check

from gpu_helpers import oracle_problem, say, to_device

pytestmark = pytest.mark.gpu
TOL = 1e-5


def _both(wl, flags):
    d = to_device(wl)
    args = (d["q"], d["k"], d["scales"], d["weights"], d["starts"], d["ends"], wl.topk)
    ref = mqa.mqa_topk_prefill(*args, flags=flags)
    got = mqa.mqa_topk_prefill_static(*args, flags=flags)
    torch.cuda.synchronize()
    return ref.cpu().numpy(), got.cpu().numpy()


@pytest.mark.parametrize("flags", [mqa.FLAG_DETERMINISTIC, 0])
def test_static_entry_matches_workspace_entry(flags):
    # 2048 rows (two batches of the static scratch), then 64 rows
    for cfg in (2, 1):
        wl = W.config(cfg)
        say(f"case: static entry point, {wl.name}, flags={flags}")
        ref, got = _both(wl, flags)
        assert not check.check_valid(got, wl.starts, wl.ends, wl.keys, wl.topk)
        rows = np.arange(wl.rows)
        fails = check.check_topk(got, rows, oracle_problem(wl), wl.topk, TOL)
        assert not fails, fails[:5]
        if flags & mqa.FLAG_DETERMINISTIC:
            assert np.array_equal(ref, got)
        else:
            assert not check.check_topk(ref, rows, oracle_problem(wl), wl.topk, TOL)
