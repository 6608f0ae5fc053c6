"""The decode-shaped fused path (mqa_topk_decode_paged: many requests of a
few query rows each, every request's keys in the paged indexer cache through
its own page-table row) against the oracle and against the prefill entry
point over the same keys gathered and concatenated, through the C ABI. Under
the deterministic flag the two entry points must agree bit for bit; in the
default mode the decode output must pass the oracle's acceptance rule.

Cases cover 1, 3, 8, 16 and 32 rows per request (four, two or one requests
per workgroup, with empty row slots below 8), rows with at most k visible
keys, top-512 and top-2048, page sizes 16..128, and calls whose few blocks
split their keys over several workgroups."""
import numpy as np
import pytest
import torch

import fp8_mqa_logits_amd as mqa
import mqa_workloads as W
from oracle import check

from gpu_helpers import oracle_problem, say, to_device

pytestmark = pytest.mark.gpu
TOL = 1e-5


def _lens(n, lo, hi, seed):
    return np.random.default_rng(seed).integers(lo, hi, n)


CASES = {
    "r8_k512": lambda: W.decode(16, 8, _lens(16, 2000, 30000, 1), 512, 64, seed=1),
    "r8_k2048_split": lambda: W.decode(12, 8, _lens(12, 9000, 40000, 2), 2048, 64, seed=2),
    "r1_short_mix": lambda: W.decode(40, 1, _lens(40, 300, 20000, 3), 512, 16, seed=3),
    "r3_p128": lambda: W.decode(10, 3, _lens(10, 1500, 12000, 4), 1024, 128, seed=4),
    "r16": lambda: W.decode(8, 16, _lens(8, 4000, 16000, 5), 512, 32, seed=5),
    "r32": lambda: W.decode(4, 32, _lens(4, 6000, 20000, 6), 512, 64, seed=6),
    "r8_many_requests": lambda: W.decode(300, 8, _lens(300, 600, 3000, 7), 512, 64, seed=7),
}


def _run(dw, flags):
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    got = mqa.mqa_topk_decode_paged(t(dw.q), t(dw.cache), t(dw.table), dw.page_size,
                                    t(dw.weights), t(dw.starts), t(dw.ends), dw.topk, dw.R,
                                    flags=flags)
    torch.cuda.synchronize()
    return got.cpu().numpy()


@pytest.mark.parametrize("flags", [mqa.FLAG_DETERMINISTIC, 0, mqa.FLAG_FORCE_RESCAN, mqa.FLAG_FORCE_EXACT])
@pytest.mark.parametrize("case", list(CASES))
def test_decode_matches_oracle_and_prefill(case, flags):
    dw = CASES[case]()
    g = dw.gathered()
    say(f"case: decode {case}: {dw.requests} requests x {dw.R} rows, {g.keys} keys, "
        f"top-{dw.topk}, page {dw.page_size}, flags={flags}")
    got = _run(dw, flags)
    assert not check.check_valid(got, dw.starts, dw.ends, int(dw.lens.max()), dw.topk)
    rows = W.sample_rows(g, 256)
    fails = check.check_topk(got[rows], rows, oracle_problem(g), dw.topk, TOL)
    assert not fails, fails[:5]
    if flags & mqa.FLAG_DETERMINISTIC:
        say("  against the prefill entry point on the gathered keys")
        d = to_device(g)
        ref = mqa.mqa_topk_prefill(d["q"], d["k"], d["scales"], d["weights"], d["starts"],
                                   d["ends"], dw.topk, flags=flags)
        torch.cuda.synchronize()
        assert np.array_equal(ref.cpu().numpy(), got)


def test_decode_stats_path():
    # every row served by the gate or the bounded rescan, none by the
    # streaming exact rescan, on i.i.d. inputs
    dw = CASES["r8_k512"]()
    say("case: decode r8_k512 path counters")
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    ws = torch.empty(mqa.workspace_size_decode(dw.requests, dw.R), dtype=torch.uint8,
                     device="cuda")
    mqa.mqa_topk_decode_paged(t(dw.q), t(dw.cache), t(dw.table), dw.page_size, t(dw.weights),
                              t(dw.starts), t(dw.ends), dw.topk, dw.R, workspace=ws,
                              flags=mqa.FLAG_STATS)
    st = mqa.read_stats(ws)
    say(f"  {st}")
    assert st["rows_exact"] == 0
    assert st["rows_gated"] + st["rows_short"] + st["rows_rescanned"] >= dw.rows - 8
    assert st["bound_ratio_max"] < 1.0


def test_decode_full_size_sampled():
    # the decode call the benchmark times: 512 requests x 8 rows x 131072
    # positions, top-2048, 64-token pages, inputs drawn on the device; every
    # row's output valid, and two seeded requests' rows against the oracle
    # over their own keys (read back through their page-table rows)
    req, R, ctx, k, P = 512, 8, 131072, 2048, 64
    say(f"case: decode full size {req} x {R} x {ctx}, top-{k}")
    d = W.decode_device(req, R, ctx, k, P, seed=1)
    got = mqa.mqa_topk_decode_paged(d["q"], d["cache"], d["table"], P, d["weights"],
                                    d["starts"], d["ends"], k, R)
    torch.cuda.synchronize()
    o = got.cpu().numpy()
    starts, ends = d["starts"].cpu().numpy(), d["ends"].cpu().numpy()
    assert not check.check_valid(o, starts, ends, ctx, k)
    for qi in np.random.default_rng(5).choice(req, 2, replace=False):
        rows = slice(qi * R, (qi + 1) * R)
        blob = d["cache"][d["table"][qi].long()].cpu().numpy()  # [pages, 132 P]
        keys = blob[:, :P * 128].reshape(-1, 128)[:ctx]
        sb = blob[:, P * 128:].reshape(-1, 4)[:ctx]
        wl = W.Workload(f"decode_request_{qi}", R, ctx, k, d["q"][rows].cpu().numpy(), keys, sb,
                        d["weights"][rows].cpu().numpy(), starts[rows], ends[rows], 0)
        say(f"  request {qi}: {R} rows against the oracle")
        fails = check.check_topk(o[rows], np.arange(R), oracle_problem(wl), k, TOL)
        assert not fails, fails[:5]
