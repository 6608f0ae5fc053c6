"""The fused path reading its keys from the paged indexer cache
(mqa_topk_prefill_paged: 132 B per token, the e4m3 key rows of a page then
their UE8M0 scale words, pages through a block table) against the same path
over the gathered keys and decoded scales, through the C ABI. Under the
deterministic flag the two must agree bit for bit; in the default mode the
paged output must pass the oracle's acceptance rule on every (sampled) row.
The pages are a seeded permutation with spare pages of random bytes, so a key
read from the wrong page or slot changes the result."""
import numpy as np
import pytest
import torch

import fp8_mqa_logits_amd as mqa
import mqa_workloads as W
from oracle import check

from gpu_helpers import oracle_problem, say, to_device

pytestmark = pytest.mark.gpu
TOL = 1e-5


def _paged(wl, page, flags, seed=3, scale_bytes=None):
    sb = wl.scale_bytes if scale_bytes is None else scale_bytes
    cache, table = W.paged_cache(wl.k, sb, page, seed=seed)
    d = to_device(wl)
    if scale_bytes is not None:
        d["scales"] = mqa.mqa_key_scales(torch.from_numpy(np.ascontiguousarray(sb)).cuda())
    ref = mqa.mqa_topk_prefill(d["q"], d["k"], d["scales"], d["weights"], d["starts"],
                               d["ends"], wl.topk, flags=flags)
    got = mqa.mqa_topk_prefill_paged(d["q"], torch.from_numpy(cache).cuda(),
                                     torch.from_numpy(table).cuda(), page, wl.keys, d["weights"],
                                     d["starts"], d["ends"], wl.topk, flags=flags)
    torch.cuda.synchronize()
    return ref.cpu().numpy(), got.cpu().numpy()


def _ragged():
    # 5000 keys (a partial last page for every page size here), two requests
    # (the second from key 2048, a page boundary), ragged and empty ranges
    rows = 96
    starts = np.zeros(rows, np.int32)
    ends = np.zeros(rows, np.int32)
    starts[:48] = 0
    ends[:48] = np.linspace(300, 2048, 48).astype(np.int32)
    starts[48:] = 2048
    ends[48:] = np.linspace(2048, 5000, 48).astype(np.int32)
    ends[60] = 2048  # empty row
    return W.custom(rows, 5000, 512, starts, ends, seed=21, name="paged_ragged")


CASES = {
    "cfg1_p16": (lambda: W.config(1), 16),
    "cfg1_p64": (lambda: W.config(1), 64),
    "ragged_p4": (_ragged, 4),
    "ragged_p64": (_ragged, 64),
    "ragged_p1024": (_ragged, 1024),
    "cfg2_p64": (lambda: W.config(2), 64),
}


@pytest.mark.parametrize("flags", [mqa.FLAG_DETERMINISTIC, 0, mqa.FLAG_FORCE_RESCAN, mqa.FLAG_FORCE_EXACT])
@pytest.mark.parametrize("case", list(CASES))
def test_paged_matches_gathered(case, flags):
    make, page = CASES[case]
    wl = make()
    say(f"case: paged cache, {wl.name}, page {page}, flags={flags}")
    ref, got = _paged(wl, page, flags)
    assert not check.check_valid(got, wl.starts, wl.ends, wl.keys, wl.topk)
    rows = W.sample_rows(wl, 512)
    fails = check.check_topk(got[rows], rows, oracle_problem(wl), wl.topk, TOL)
    assert not fails, fails[:5]
    if flags & mqa.FLAG_DETERMINISTIC:
        assert np.array_equal(ref, got)


def test_paged_zero_scale_keys():
    # UE8M0 byte 0 decodes to a scale of +0.0: those keys score exactly 0
    wl = W.config(1)
    sb = wl.scale_bytes.copy()
    rng = np.random.default_rng(5)
    sb[rng.choice(wl.keys, wl.keys // 3, replace=False)] = 0
    say("case: paged cache, cfg1 with a third of the scales zero")
    ref, got = _paged(wl, 32, mqa.FLAG_DETERMINISTIC, scale_bytes=sb)
    assert np.array_equal(ref, got)
    wl0 = W.Workload(wl.name, wl.rows, wl.keys, wl.topk, wl.q, wl.k, sb, wl.weights, wl.starts,
                     wl.ends, wl.seed)
    fails = check.check_topk(got, np.arange(wl.rows), oracle_problem(wl0), wl.topk, TOL)
    assert not fails, fails[:5]


def test_paged_full_size_long_context():
    # 16384 rows x 131072 keys, top-2048, 64-token pages: bitwise equal to the
    # gathered call in the deterministic mode; oracle rule on sampled rows
    wl = W.config(3)
    say(f"case: paged cache, {wl.name}, page 64, deterministic")
    ref, got = _paged(wl, 64, mqa.FLAG_DETERMINISTIC)
    assert np.array_equal(ref, got)
    rows = W.sample_rows(wl, 64)
    fails = check.check_topk(got[rows], rows, oracle_problem(wl), wl.topk, TOL)
    assert not fails, fails[:5]
