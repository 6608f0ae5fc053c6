"""Pins of the CPU oracle against facts that do not come from the oracle itself:
values worked by hand from the pages, a library decoder, closed forms, exact
identities and brute-force enumeration. CPU only."""
import itertools
import json
import os

import numpy as np
import pytest
import torch

import mqa_workloads as W
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def code_of(x: float) -> int:
    """e4m3 code of an exactly representable value (via the torch library)."""
    t = torch.tensor([x], dtype=torch.float32).to(torch.float8_e4m3fn)
    assert float(t.float()) == x, x
    return int(t.view(torch.uint8))


# ---------------------------------------------------------------- decoders

def test_e4m3_table_matches_library_decoder():
    tab = oracle.e4m3_table()
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    lib = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(lib)
    assert set(np.nonzero(nan)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(np.isnan(tab), nan)
    assert np.array_equal(tab[~nan], lib[~nan])
    # spot values of the OCP e4m3fn format
    assert tab[0x38] == 1.0 and tab[0xB8] == -1.0
    assert tab[0x01] == 2.0 ** -9 and tab[0x08] == 2.0 ** -6
    assert tab[0x7E] == 448.0 and tab[0xFE] == -448.0
    # every finite value is an integer multiple of 2^-9 (the exactness argument)
    fin = tab[~nan] * 512
    assert np.array_equal(fin, np.round(fin))


def test_ue8m0_decode_bit_pattern_rule():
    e = np.arange(0, 255, dtype=np.int64)
    b = np.repeat(e.astype(np.uint8)[:, None], 4, axis=1)
    got = oracle.key_scales(b)
    # the docstring's closed form 2**(e-127) for e >= 1; e = 0 gives +0.0
    # under the code's bit-pattern rule (e << 23 is the all-zero pattern)
    assert got[0] == 0.0 and not np.signbit(got[0])
    assert np.array_equal(got[1:].astype(np.float64), np.ldexp(1.0, e[1:] - 127))
    assert oracle.key_scales(np.array([[127] * 4], np.uint8))[0] == 1.0
    assert oracle.key_scales(np.array([[123] * 4], np.uint8))[0] == 0.0625
    # only the low byte of the little-endian int32 view counts
    assert oracle.key_scales(np.array([[126, 1, 2, 3]], np.uint8))[0] == 0.5


def test_e4m3_encoder_matches_library_rounding():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(200000) * 20, rng.standard_normal(20000) * 1e-2,
                        [0.0, 1.0625, 1.1875, 2 ** -10, 3 * 2 ** -11, 447.0, 448.0]])
    x = x.astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(W.encode_e4m3(x), ref)
    # saturation (the library instead returns NaN above 464)
    assert W.encode_e4m3(np.array([1e6, -1e6], np.float32)).tolist() == [0x7E, 0xFE]


# ---------------------------------------------------------------- dot products

def test_head_dots_closed_forms():
    big = code_of(448.0)
    q = np.full((32, 128), big, np.uint8)
    k = np.full(128, big, np.uint8)
    assert np.all(oracle.head_dots(q, k) == 128 * 448.0 * 448.0)
    k_neg = np.full(128, big | 0x80, np.uint8)
    assert np.all(oracle.head_dots(q, k_neg) == -128 * 200704.0)
    # one-hot: head h has only dim (3h+1) % 128 set; the key has dim d = d
    q = np.zeros((32, 128), np.uint8)
    k = np.zeros(128, np.uint8)
    tab = oracle.e4m3_table()
    for d in range(128):
        k[d] = (d * 7 + 3) % 0x7E
    for h in range(32):
        q[h, (3 * h + 1) % 128] = (h * 5 + 9) % 0x7E
    want = np.array([tab[q[h, (3 * h + 1) % 128]] * tab[k[(3 * h + 1) % 128]] for h in range(32)])
    assert np.array_equal(oracle.head_dots(q, k), want)


def test_head_dots_exact_against_library_matmul():
    # float64 BLAS products of e4m3 values are exact (products are multiples of
    # 2^-18 and every partial sum needs fewer than 53 bits), so a library
    # matmul in any order must agree bit for bit.
    rng = np.random.default_rng(5)
    tab = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    tab = tab.to(torch.float64).numpy()
    for trial in range(20):
        q = rng.integers(0, 256, size=(32, 128)).astype(np.uint8)
        k = rng.integers(0, 256, size=128).astype(np.uint8)
        q[(q & 0x7F) == 0x7F] = 0x7E
        k[(k & 0x7F) == 0x7F] = 0x7E
        want = tab[q] @ tab[k]
        assert np.array_equal(oracle.head_dots(q, k), want)


# ---------------------------------------------------------------- hand example

def _hand_problem(start=0, topk=512):
    g = json.load(open(os.path.join(GOLDEN, "hand_4key.json")))
    keys = np.zeros((4, 128), np.uint8)
    for j, (a, b) in enumerate(g["keys"]):
        keys[j, 0] = code_of(a)
        keys[j, 1] = code_of(b)
    q = np.zeros((1, 32, 128), np.uint8)
    for h, vec in g["query_heads"].items():
        q[0, int(h), 0] = code_of(vec[0])
        q[0, int(h), 1] = code_of(vec[1])
    w = np.full((1, 32), g["weights"]["other"], np.float32)
    w[0, 0] = g["weights"]["0"]
    w[0, 1] = g["weights"]["1"]
    sb = np.repeat(np.array(g["scale_exponent_bytes"], np.uint8)[:, None], 4, axis=1)
    scales = oracle.key_scales(sb)
    p = oracle.Problem(q, keys, scales, w, np.array([start], np.int32), np.array([4], np.int32))
    return g, p, q, keys, scales


def test_hand_example_logits_exact():
    g, p, q, keys, scales = _hand_problem()
    assert scales.tolist() == g["scales"]
    for j in range(4):
        s = oracle.head_dots(q[0], keys[j])
        assert s[0] == g["per_head_dots"]["0"][j]
        assert s[1] == g["per_head_dots"]["1"][j]
        assert np.all(s[2:] == 0)
    lg = oracle.logits(p, [0])[0]
    assert lg.tolist() == g["logits"]


def test_hand_example_selection_and_api_convention():
    g, p, *_ = _hand_problem()
    lg = oracle.logits(p, [0])[0]
    assert oracle.select(lg, 2).tolist() == g["top2_of_all_four"]
    assert oracle.select(lg[1:], 2).tolist() == g["top2_of_keys_1_to_3_relative"]
    idx, kth, mx = oracle.topk(p, [0], 512)
    want = g["api_k512_start0"]
    assert idx[0, :4].tolist() == want["valid"] and np.all(idx[0, 4:] == -1)
    assert (idx[0] == -1).sum() == want["pad"]
    assert np.isneginf(kth[0]) and mx[0] == 1.0
    g, p1, *_ = _hand_problem(start=1)
    idx, _, _ = oracle.topk(p1, [0], 512)
    want = g["api_k512_start1"]
    assert idx[0, :3].tolist() == want["valid"] and (idx[0] == -1).sum() == want["pad"]
    # dense logits: -inf before the start and past the last key
    dl = oracle.logits(p1, [0], col0=0, ncols=6)[0]
    assert np.isneginf(dl[0]) and dl[1:4].tolist() == g["logits"][1:] and np.all(np.isneginf(dl[4:]))


# ---------------------------------------------------------------- identities

def _random_problem(rows, keys, seed, scale_exps=None, wscale=1.0):
    wl = W.custom(rows, keys, 8, np.zeros(rows), np.full(rows, keys), seed=seed,
                  weight_scale=wscale)
    sb = wl.scale_bytes if scale_exps is None else W.ue8m0_bytes(scale_exps)
    return wl, oracle.Problem(wl.q, wl.k, oracle.key_scales(sb), wl.weights, wl.starts, wl.ends)


def test_relu_fold_identity():
    # sum_h w relu(s) = (sum_h w s + sum_h w |s|) / 2, checked per key from the
    # exact head dots; pins that relu sits on each head's dot, before weighting
    wl, p = _random_problem(4, 64, seed=11, scale_exps=np.zeros(64, np.int64))
    lg = oracle.logits(p, np.arange(4))
    for r in range(4):
        for j in range(64):
            s = oracle.head_dots(wl.q[r], wl.k[j])
            w = wl.weights[r].astype(np.float64)
            lin = float(np.dot(w, s))
            ab = float(np.dot(w, np.abs(s)))
            want = 0.5 * (lin + ab)
            assert abs(lg[r, j] - want) <= 2 ** -23 * max(abs(want), 1e-30) + 1e-30


def test_scale_bit_pattern_rule_is_exact_power_of_two():
    keys = 32
    e = np.array([(-4 + (j % 5)) for j in range(keys)], np.int64)
    wl, p1 = _random_problem(3, keys, seed=13, scale_exps=np.zeros(keys, np.int64))
    _, p2 = _random_problem(3, keys, seed=13, scale_exps=e)
    a = oracle.logits(p1, [0, 1, 2]).astype(np.float64)
    b = oracle.logits(p2, [0, 1, 2]).astype(np.float64)
    assert np.array_equal(b, a * np.ldexp(1.0, e)[None, :])


def test_weight_and_head_indexing():
    # q[r,h,:] is one-hot on dim h (value 1), w[r,h] = 1 only for h = r % 32:
    # then logit[r,j] = scale_j * relu(k[j, r % 32]). A transposed operand, a
    # wrong head or row index, or relu in the wrong place breaks this.
    rows, keys = 40, 24
    q = np.zeros((rows, 32, 128), np.uint8)
    for h in range(32):
        q[:, h, h] = code_of(1.0)
    w = np.zeros((rows, 32), np.float32)
    for r in range(rows):
        w[r, r % 32] = 1.0
    rng = np.random.default_rng(17)
    k = W.encode_e4m3(rng.standard_normal((keys, 128)).astype(np.float32))
    exps = rng.integers(-4, 1, size=keys)
    scales = oracle.key_scales(W.ue8m0_bytes(exps))
    p = oracle.Problem(q, k, scales, w, np.zeros(rows, np.int32), np.full(rows, keys, np.int32))
    lg = oracle.logits(p, np.arange(rows)).astype(np.float64)
    tab = oracle.e4m3_table()
    for r in range(rows):
        want = np.maximum(tab[k[:, r % 32]], 0.0) * scales.astype(np.float64)
        assert np.array_equal(lg[r], want)


def test_index_relative_to_start_and_clamping():
    # the best keys are planted; the answer must be key - start
    rows, keys, topk = 3, 600, 512
    wl, p = _random_problem(rows, keys, seed=19, scale_exps=np.zeros(keys, np.int64))
    k = wl.k.copy()
    k[:] = W.encode_e4m3(np.full((keys, 128), -0.5, np.float32))  # every dot <= 0 ...
    q = wl.q.copy()
    q[:] = code_of(1.0)
    w = np.ones((rows, 32), np.float32)
    planted = np.arange(100, 600, 1)[:topk]          # 500 keys: 100..599
    k[planted] = code_of(0.25)                       # positive dot
    p = oracle.Problem(q, k, oracle.key_scales(W.ue8m0_bytes(np.zeros(keys, np.int64))), w,
                       np.array([80, -5, 300], np.int32), np.array([600, 900, 200], np.int32))
    idx, kth, _ = oracle.topk(p, [0, 1, 2], topk)
    # row 0: [80, 600) has 520 visible keys, 500 planted + 12 of the zero-logit ones
    assert set(idx[0].tolist()) >= set((planted - 80).tolist())
    assert np.all(idx[0] >= 0) and np.all(idx[0] < 520)
    # row 1: start clamped to 0, end clamped to 600 (600 > 512 visible)
    assert set(idx[1].tolist()) >= set(planted.tolist())
    # row 2: end < start -> empty range: all -1
    assert np.all(idx[2] == -1)


def test_k_plus_four_exclusion():
    # k keys tie at logit 1.0 and 4 keys are below: exactly those 4 are excluded
    topk = 512
    n = topk + 4
    k = np.zeros((n, 128), np.uint8)
    k[:, 0] = code_of(1.0)
    low = np.array([5, 77, 300, 515])
    k[low, 0] = code_of(-1.0)
    k[low[2:], 0] = 0
    k[low[2:], 1] = code_of(2.0)
    q = np.zeros((1, 32, 128), np.uint8)
    q[0, 0, 0] = code_of(2.0)
    q[0, 1, 1] = code_of(1.0)
    w = np.zeros((1, 32), np.float32)
    w[0, 0], w[0, 1] = 0.5, -0.25
    scales = np.ones(n, np.float32)
    p = oracle.Problem(q, k, scales, w, np.array([0], np.int32), np.array([n], np.int32))
    lg = oracle.logits(p, [0])[0]
    assert set(np.nonzero(lg == 1.0)[0].tolist()) == set(range(n)) - set(low.tolist())
    idx, kth, _ = oracle.topk(p, [0], topk)
    assert set(idx[0].tolist()) == set(range(n)) - set(low.tolist())
    assert kth[0] == 1.0


# ---------------------------------------------------------------- selection

def _brute_force_best(v, kk):
    """The unique kk-subset whose every member beats every non-member under
    the total order (value descending, position ascending), by enumeration."""
    n = len(v)

    def beats(a, b):
        return v[a] > v[b] or (v[a] == v[b] and a < b)

    found = []
    for sub in itertools.combinations(range(n), kk):
        rest = [x for x in range(n) if x not in sub]
        if all(beats(a, b) for a in sub for b in rest):
            found.append(sub)
    assert len(found) == 1
    return set(found[0])


def test_selection_against_brute_force():
    rng = np.random.default_rng(23)
    for trial in range(150):
        n = int(rng.integers(1, 13))
        kk = int(rng.integers(1, min(6, n) + 1))
        # few distinct values so that ties are common
        v = rng.integers(-3, 4, size=n).astype(np.float32) * np.float32(0.5)
        got = oracle.select(v, kk)
        assert set(got.tolist()) == _brute_force_best(v, kk)
        assert len(set(got.tolist())) == kk


def test_selection_at_k512_against_library_sort():
    rng = np.random.default_rng(29)
    for trial in range(5):
        v = rng.standard_normal(4096).astype(np.float32)
        v[rng.integers(0, 4096, 300)] = v[7]   # plant ties
        got = oracle.select(v, 512)
        order = np.lexsort((np.arange(4096), -v.astype(np.float64)))
        assert got.tolist() == order[:512].tolist()


def test_thread_count_does_not_change_results():
    wl = W.config(1)
    p = oracle.Problem(wl.q, wl.k, oracle.key_scales(wl.scale_bytes), wl.weights, wl.starts,
                       wl.ends)
    rows = [0, 17, 63]
    a = oracle.topk(p, rows, 512, threads=1)
    b = oracle.topk(p, rows, 512, threads=8)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_rejects_out_of_contract_inputs():
    wl, p = _random_problem(2, 16, seed=31)
    bad = oracle.Problem(wl.q, wl.k, np.full(16, np.inf, np.float32), wl.weights, wl.starts,
                         wl.ends)
    with pytest.raises(ValueError):
        oracle.logits(bad, [0])
    q = wl.q.copy()
    q[0, 0, 0] = 0x7F
    bad = oracle.Problem(q, wl.k, p.scales, wl.weights, wl.starts, wl.ends)
    with pytest.raises(ValueError):
        oracle.topk(bad, [0], 8)


# ------------------------------------------------------------ 64 index heads

def _problem64(rows, keys, seed):
    rng = np.random.default_rng(seed)
    q = W.encode_e4m3(rng.standard_normal((rows, 64, 128)).astype(np.float32))
    k = W.encode_e4m3(rng.standard_normal((keys, 128)).astype(np.float32))
    sc = np.ldexp(1.0, rng.integers(-4, 1, keys)).astype(np.float32)
    w = (rng.standard_normal((rows, 64)) / 8).astype(np.float32)
    starts = np.zeros(rows, np.int32)
    ends = np.full(rows, keys, np.int32)
    return q, k, sc, w, starts, ends


def test_64_heads_brute_force_exact():
    # one row of 64 heads against 6 keys in exact rational arithmetic (the
    # formula summed over all 64 heads), rounded once to fp32
    from fractions import Fraction
    q, k, sc, w, s, e = _problem64(1, 6, 11)
    tab = oracle.e4m3_table()
    got = oracle.logits(oracle.Problem(q, k, sc, w, s, e), [0])[0]
    for j in range(6):
        tot = Fraction(0)
        for h in range(64):
            d = sum(Fraction(float(tab[q[0, h, i]])) * Fraction(float(tab[k[j, i]]))
                    for i in range(128))
            tot += Fraction(float(w[0, h])) * max(d, Fraction(0))
        assert got[j] == np.float32(float(tot * Fraction(float(sc[j])))), j


def test_64_heads_are_the_sum_of_two_32_head_halves():
    # linearity over heads: the 64-head logit is the 32-head logit of the
    # first half plus that of the second (each rounded once to fp32)
    q, k, sc, w, s, e = _problem64(8, 300, 12)
    full = oracle.logits(oracle.Problem(q, k, sc, w, s, e), np.arange(8)).astype(np.float64)
    a = oracle.logits(oracle.Problem(q[:, :32], k, sc, w[:, :32], s, e), np.arange(8))
    b = oracle.logits(oracle.Problem(q[:, 32:], k, sc, w[:, 32:], s, e), np.arange(8))
    a, b = a.astype(np.float64), b.astype(np.float64)
    tol = 2.0 ** -23 * (np.abs(a) + np.abs(b) + np.abs(full)) + 1e-30
    assert np.all(np.abs(full - (a + b)) <= tol)
    # and a half cannot stand in for the whole: dropping either half moves logits
    assert np.abs(full - a).max() > 1e-3 and np.abs(full - b).max() > 1e-3


def test_64_head_dots_closed_form():
    # head h selects dimension h % 128 with weight 2^(h % 4 - 1)
    q = np.zeros((64, 128), np.uint8)
    for h in range(64):
        q[h, h % 128] = code_of(2.0 ** (h % 4 - 1))
    kv = np.linspace(-3, 3, 128).astype(np.float32)
    k = W.encode_e4m3(kv)
    tab = oracle.e4m3_table()
    got = oracle.head_dots(q, k)
    want = np.array([2.0 ** (h % 4 - 1) * tab[k[h % 128]] for h in range(64)])
    assert np.array_equal(got, want)
