"""DeepSeek-V4.1's two-level candidate selection (PR #60618, "Limitations of
this PR -- TODOs"), consumer layers: mqa_topk_masked keeps each row's keys
in its listed blocks of 8 and selects their top-k, checked against the
oracle's logits of the same keys, through the C ABI."""
import numpy as np
import pytest
import torch

import fp8_mqa_logits_amd as mqa
import mqa_workloads as W
from oracle import check

from gpu_helpers import oracle_problem, say, to_device

pytestmark = pytest.mark.gpu
TOL = 1e-5


def _blocks(wl, nb, seed, pad_every=0):
    """Per row nb distinct blocks among the row's visible ones (-1 padded
    when the row has fewer, and every pad_every-th entry of a row -1)."""
    rng = np.random.default_rng(seed)
    out = np.full((wl.rows, nb), -1, np.int32)
    for r in range(wl.rows):
        s = min(max(int(wl.starts[r]), 0), wl.keys)
        e = min(max(int(wl.ends[r]), s), wl.keys)
        if e <= s:
            continue
        nvis = (e - 1) // 8 - s // 8 + 1
        pick = rng.permutation(nvis)[:nb]
        out[r, :pick.shape[0]] = pick
        if pad_every:
            out[r, ::pad_every] = -1
    return out


def _run(wl, blocks, flags=0, topk=None):
    d = to_device(wl)
    out = mqa.mqa_topk_masked(d["q"], d["k"], d["scales"], d["weights"], d["starts"], d["ends"],
                              torch.from_numpy(blocks).cuda(), topk or wl.topk, flags=flags)
    torch.cuda.synchronize()
    return out.cpu().numpy()


CASES = {
    # 2048 blocks over a 32K-key causal chunk, top-512 (the consumer shape)
    "cfg2_2048blocks": lambda: (W.config(2), 2048, 0),
    # ragged and offset ranges (starts not multiples of 8), padded lists, and
    # rows whose kept keys number fewer than k
    "ragged_padded": lambda: (W.custom(96, 6000, 512, np.arange(96) * 7,
                                       np.minimum(np.arange(96) * 7 + 300 + np.arange(96) * 50, 6000),
                                       seed=5), 128, 5),
}


@pytest.mark.parametrize("flags", [mqa.FLAG_DETERMINISTIC, 0])
@pytest.mark.parametrize("case", list(CASES))
def test_masked_topk(case, flags):
    wl, nb, pad = CASES[case]()
    if wl.topk != 512:
        wl = W.Workload(wl.name, wl.rows, wl.keys, 512, wl.q, wl.k, wl.scale_bytes, wl.weights,
                        wl.starts, wl.ends, wl.seed)
    blocks = _blocks(wl, nb, 9, pad)
    say(f"case: masked top-k {case}, {nb} blocks per row, flags={flags}")
    got = _run(wl, blocks, flags)
    rows = W.sample_rows(wl, 96)
    fails = check.check_topk_masked(got[rows], rows, oracle_problem(wl), blocks, wl.topk, TOL)
    assert not fails, fails[:5]
    if flags & mqa.FLAG_DETERMINISTIC:
        for r in rows:
            v = got[r][got[r] >= 0]
            assert np.all(np.diff(v) > 0) and np.all(got[r][v.shape[0]:] == -1)


def test_masked_all_blocks_equals_unmasked():
    # listing every block of every row keeps every visible key: the result is
    # the plain top-k (bitwise, in the deterministic mode)
    wl = W.config(1)
    nvis = (wl.ends.astype(np.int64) - 1) // 8 - wl.starts // 8 + 1
    nb = int(nvis.max())
    blocks = np.full((wl.rows, nb), -1, np.int32)
    for r in range(wl.rows):
        blocks[r, :nvis[r]] = np.arange(nvis[r])[::-1]
    say("case: masked top-k with every block listed vs the fused path")
    got = _run(wl, blocks, mqa.FLAG_DETERMINISTIC)
    d = to_device(wl)
    ref = mqa.mqa_topk_prefill(d["q"], d["k"], d["scales"], d["weights"], d["starts"], d["ends"],
                               wl.topk, flags=mqa.FLAG_DETERMINISTIC)
    torch.cuda.synchronize()
    assert np.array_equal(got, ref.cpu().numpy())


# ------------------------------------------------------------ source layers

def _source(wl, topk, flags=0, ws=None):
    d = to_device(wl)
    out, ob = mqa.mqa_topk_prefill_blocks(d["q"], d["k"], d["scales"], d["weights"], d["starts"],
                                          d["ends"], topk, flags=flags, workspace=ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), ob.cpu().numpy()


SOURCES = {
    "cfg2_k512": lambda: W.config(2),
    "ragged_offsets": lambda: W.custom(128, 40000, 512, 3 + np.arange(128) * 11,
                                       np.minimum(3 + np.arange(128) * 11 + 2000 +
                                                  np.arange(128) * 300, 40000), seed=6),
    "repeated_keys": lambda: _repeated(),
    # few long rows: with the forced exact route every row's block maxima fit
    # the merge buffers, so the exact block scan splits the rows into pieces
    "few_long_rows": lambda: W.custom(8, 60000, 512, np.arange(8) * 13,
                                      60000 - np.arange(8) * 500, seed=10),
}


def _repeated():
    # keys drawn from 128 distinct vectors: block maxima tie everywhere, also
    # at the 2048th
    wl = W.custom(64, 40000, 512, np.zeros(64), np.full(64, 40000) - np.arange(64) * 100, seed=7)
    rng = np.random.default_rng(8)
    k = wl.k[rng.integers(0, 128, wl.keys)]
    sb = np.full_like(wl.scale_bytes, 126)
    return W.Workload("repeated_keys_64x40000", wl.rows, wl.keys, wl.topk, wl.q, k, sb,
                      wl.weights, wl.starts, wl.ends, wl.seed)


@pytest.mark.parametrize("flags", [mqa.FLAG_DETERMINISTIC, 0, mqa.FLAG_FORCE_RESCAN])
@pytest.mark.parametrize("case", list(SOURCES))
def test_source_blocks(case, flags):
    wl = SOURCES[case]()
    say(f"case: two-level source {case}, flags={flags}")
    out, ob = _source(wl, 512, flags)
    rows = W.sample_rows(wl, 64)
    p = oracle_problem(wl)
    fails = check.check_topk(out[rows], rows, p, 512, TOL)
    assert not fails, fails[:5]
    fails = check.check_blocks(ob[rows], rows, p, mqa.MAX_BLOCKS, TOL)
    assert not fails, fails[:5]
    if flags & mqa.FLAG_DETERMINISTIC:
        say("  against the exact block scan of every row (forced exact route)")
        out2, ob2 = _source(wl, 512, flags | mqa.FLAG_FORCE_EXACT)
        assert np.array_equal(ob, ob2) and np.array_equal(out, out2)
        for r in rows:
            v = ob[r][ob[r] >= 0]
            assert np.all(np.diff(v) > 0)


def test_source_then_consumer():
    # the consumer masks to the source's blocks: its keys lie in them and are
    # the top-512 of them
    wl = W.config(2)
    wl = W.Workload(wl.name, wl.rows, wl.keys, 512, wl.q, wl.k, wl.scale_bytes, wl.weights,
                    wl.starts, wl.ends, wl.seed)
    say("case: source blocks -> consumer mask")
    _, ob = _source(wl, 512)
    got = _run(wl, ob)
    rows = W.sample_rows(wl, 48)
    fails = check.check_topk_masked(got[rows], rows, oracle_problem(wl), ob, 512, TOL)
    assert not fails, fails[:5]


def test_source_full_size_sampled():
    # 16384 rows x 131072 keys (causal tail), top-512 keys and 2048 blocks
    wl = W.config(3)
    say(f"case: two-level source {wl.name}, top-512")
    ws = mqa.alloc_workspace(wl.rows)
    out, ob = _source(wl, 512, mqa.FLAG_STATS, ws)
    st = mqa.read_stats(ws)
    say(f"  stats {st}")
    rows = W.sample_rows(wl, 24)
    p = oracle_problem(wl)
    assert not check.check_topk(out[rows], rows, p, 512, TOL)
    assert not check.check_blocks(ob[rows], rows, p, mqa.MAX_BLOCKS, TOL)
    assert st["rows_block_scan"] <= wl.rows // 100
    # the consumer call the benchmark times: top-512 of each row's 2048 blocks
    say("  consumer on those blocks, top-512")
    got = _run(wl, ob, topk=512)
    fails = check.check_topk_masked(got[rows], rows, p, ob, 512, TOL)
    assert not fails, fails[:5]
