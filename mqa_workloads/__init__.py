"""Seeded synthetic inputs for the FP8 MQA-logits + top-k prefill path.

This module holds input generation only: random draws, the rounding of those
draws to e4m3 codes and UE8M0 exponent bytes, and the row ranges. It contains
none of the method's arithmetic (no decoding, no dot products, no selection),
and it is the only code shared by the CPU oracle side and the GPU side.

The workloads stand in for the pages' real serving captures (GLM-5.x indexer
inputs from MRCR and random prompts, vLLM PR #60618, "Performance"), which are
not available: q and k are N(0,1) rounded to e4m3, each key's UE8M0 scale is
2^e with e uniform in [-4, 0], and the per-row head weights are N(0,1)/sqrt(32).

Randomness: numpy's PCG64 generator, seed 0xF8A0 + config number, draws taken
in the fixed order q, k, scales, weights, special-row choices.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

HEADS = 32
DIM = 128
SEED_BASE = 0xF8A0


def encode_e4m3(x) -> np.ndarray:
    """Round real values to OCP e4m3fn codes: round to nearest, ties to even,
    magnitudes saturated at 448 (the largest finite e4m3 value)."""
    x = np.asarray(x)
    out = np.empty(x.shape, np.uint8)
    flat_in = x.reshape(-1)
    flat_out = out.reshape(-1)
    chunk = 1 << 22
    for lo in range(0, flat_in.shape[0], chunk):
        v = flat_in[lo:lo + chunk].astype(np.float64)
        sign = np.signbit(v).astype(np.uint8)
        a = np.minimum(np.abs(v), 448.0)
        _, e = np.frexp(a)                       # a = m * 2^e, m in [0.5, 1)
        ex = np.where(a > 0, e - 1, -6)          # floor(log2 a)
        ex = np.maximum(ex, -6)                  # below 2^-6: subnormal grid 2^-9
        qv = np.rint(np.ldexp(a, 3 - ex))        # integer on the 3-bit mantissa grid
        carry = qv >= 16
        ex = np.where(carry, ex + 1, ex)
        qv = np.where(carry, 8.0, qv)
        sub = qv < 8
        code = np.where(sub, qv, ((ex + 7) * 8) + (qv - 8)).astype(np.uint8)
        flat_out[lo:lo + chunk] = code | (sign << 7)
    return out


def ue8m0_bytes(exponents) -> np.ndarray:
    """[keys] int exponents e (scale 2^e) -> [keys, 4] uint8, four equal bytes
    127 + e, the layout of the gathered indexer K-cache scales."""
    e = np.asarray(exponents, np.int64)
    b = (127 + e).astype(np.uint8)
    return np.repeat(b[:, None], 4, axis=1)


@dataclasses.dataclass
class Workload:
    name: str
    rows: int
    keys: int
    topk: int
    q: np.ndarray            # uint8 [rows, 32, 128] e4m3 codes
    k: np.ndarray            # uint8 [keys, 128] e4m3 codes
    scale_bytes: np.ndarray  # uint8 [keys, 4] UE8M0 bytes
    weights: np.ndarray      # float32 [rows, 32]
    starts: np.ndarray       # int32 [rows]
    ends: np.ndarray         # int32 [rows]
    seed: int
    groups: dict = dataclasses.field(default_factory=dict)  # name -> int32 row ids

    def visible_pairs(self) -> int:
        s = np.clip(self.starts.astype(np.int64), 0, self.keys)
        e = np.clip(self.ends.astype(np.int64), s, self.keys)
        return int((e - s).sum())

    def hashes(self) -> dict:
        return {n: fnv1a(getattr(self, n)) for n in
                ("q", "k", "scale_bytes", "weights", "starts", "ends")}


def fnv1a(a: np.ndarray) -> str:
    """64-bit FNV-1a of an array's bytes, folded 8 bytes at a time (fast enough
    for 100 MB buffers); used only to log that two runs saw the same inputs."""
    b = np.ascontiguousarray(a).view(np.uint8).reshape(-1)
    pad = (-b.shape[0]) % 8
    if pad:
        b = np.concatenate([b, np.zeros(pad, np.uint8)])
    words = b.view(np.uint64)
    h = np.uint64(0xCBF29CE484222325)
    prime = np.uint64(0x100000001B3)
    # fold in blocks so that the loop runs in numpy, not per byte
    with np.errstate(over="ignore"):
        blk = 1 << 16
        for lo in range(0, words.shape[0], blk):
            w = words[lo:lo + blk]
            mult = np.uint64(1) + np.arange(w.shape[0], dtype=np.uint64) * np.uint64(2)
            h = (h ^ np.bitwise_xor.reduce(w * mult)) * prime
    return f"{int(h):016x}"


def _normal(rng, shape):
    return rng.standard_normal(shape, dtype=np.float32)


def _scales(rng, keys):
    return ue8m0_bytes(rng.integers(-4, 0, size=keys, endpoint=True))


def _weights(rng, rows):
    return (_normal(rng, (rows, HEADS)) / np.float32(math.sqrt(HEADS))).astype(np.float32)


def _causal(rows, keys, first_end, start=0):
    ends = (np.arange(rows, dtype=np.int64) + first_end).astype(np.int32)
    starts = np.full(rows, start, np.int32)
    assert int(ends[-1]) <= keys
    return starts, ends


def config(n: int) -> Workload:
    """The five benchmark configurations (1 tiny ... 5 stress at 1M keys)."""
    seed = SEED_BASE + n
    rng = np.random.Generator(np.random.PCG64(seed))
    if n == 1:
        rows, keys, topk = 64, 4096, 512
        q = encode_e4m3(_normal(rng, (rows, HEADS, DIM)))
        k = encode_e4m3(_normal(rng, (keys, DIM)))
        sb = _scales(rng, keys)
        w = _weights(rng, rows)
        starts, ends = _causal(rows, keys, 4033)
        return Workload("cfg1_tiny_64x4096_k512", rows, keys, topk, q, k, sb, w, starts, ends, seed)
    if n == 2:
        rows, keys, topk = 2048, 32768, 1024
        q = encode_e4m3(_normal(rng, (rows, HEADS, DIM)))
        k = encode_e4m3(_normal(rng, (keys, DIM)))
        sb = _scales(rng, keys)
        w = _weights(rng, rows)
        i = np.arange(rows, dtype=np.int64)
        req = i // 1024
        starts = (16384 * req).astype(np.int32)
        ends = (16384 * req + 15361 + (i % 1024)).astype(np.int32)
        return Workload("cfg2_2req_2048x32768_k1024", rows, keys, topk, q, k, sb, w, starts, ends,
                        seed)
    if n == 3:
        rows, keys, topk = 16384, 131072, 2048
        q = encode_e4m3(_normal(rng, (rows, HEADS, DIM)))
        k = encode_e4m3(_normal(rng, (keys, DIM)))
        sb = _scales(rng, keys)
        w = _weights(rng, rows)
        starts, ends = _causal(rows, keys, 114689)
        return Workload("cfg3_long_16384x131072_k2048", rows, keys, topk, q, k, sb, w, starts, ends,
                        seed)
    if n == 4:
        rows, keys, topk = 16384, 524288, 2048
        qf = _normal(rng, (rows, HEADS, DIM))
        qf[4096:8192] += np.float32(3.0)          # request 1: large common score offset
        q = encode_e4m3(qf)
        del qf
        k = encode_e4m3(_normal(rng, (keys, DIM)))
        sb = _scales(rng, keys)
        w = _weights(rng, rows)
        i = np.arange(rows, dtype=np.int64)
        req = i // 4096
        starts = (131072 * req).astype(np.int32)
        ends = (131072 * req + 126977 + (i % 4096)).astype(np.int32)
        return Workload("cfg4_4req_16384x524288_k2048", rows, keys, topk, q, k, sb, w, starts, ends,
                        seed, groups={"biased": np.arange(4096, 8192, dtype=np.int32)})
    if n == 5:
        rows, keys, topk = 16384, 1048576, 2048
        q = encode_e4m3(_normal(rng, (rows, HEADS, DIM)))
        # each key row is one of 16 distinct e4m3 vectors (heavy score ties)
        distinct = encode_e4m3(_normal(rng, (16, DIM)))
        choice = rng.integers(0, 16, size=keys)
        k = distinct[choice]
        sb = _scales(rng, keys)
        w = _weights(rng, rows)
        starts, ends = _causal(rows, keys, 1032193)
        nsel = int(0.05 * rows)                   # 819
        perm = rng.permutation(rows).astype(np.int32)
        short = np.sort(perm[:nsel])
        heavy = np.sort(perm[nsel:2 * nsel])
        lens = rng.integers(0, 2048, size=nsel)   # n in [0, 2047]
        starts[short] = (ends[short] - lens).astype(np.int32)
        w[heavy] *= np.float32(1e4)
        return Workload("cfg5_stress_16384x1048576_k2048", rows, keys, topk, q, k, sb, w, starts,
                        ends, seed, groups={"short": short, "heavy_weights": heavy})
    raise ValueError(f"no config {n}")


def sweep(keys: int, topk: int, rows: int = 16384, seed: int = SEED_BASE + 100) -> Workload:
    """Causal tail of a `keys`-key context: row i sees [0, keys - rows + 1 + i)."""
    rng = np.random.Generator(np.random.PCG64(seed + keys + topk))
    q = encode_e4m3(_normal(rng, (rows, HEADS, DIM)))
    k = encode_e4m3(_normal(rng, (keys, DIM)))
    sb = _scales(rng, keys)
    w = _weights(rng, rows)
    starts, ends = _causal(rows, keys, keys - rows + 1)
    return Workload(f"sweep_{rows}x{keys}_k{topk}", rows, keys, topk, q, k, sb, w, starts, ends,
                    seed)


def extra_common_offset(rows: int = 16384, keys: int = 131072, topk: int = 2048) -> Workload:
    """Config 3 shape with a true common score offset: k = e4m3(N(0,1) + 2) and
    every scale 1.0, so every head's dot carries the key-independent term
    2 * sum_d q[r,h,d]."""
    seed = SEED_BASE + 11
    rng = np.random.Generator(np.random.PCG64(seed))
    q = encode_e4m3(_normal(rng, (rows, HEADS, DIM)))
    k = encode_e4m3(_normal(rng, (keys, DIM)) + np.float32(2.0))
    sb = ue8m0_bytes(np.zeros(keys, np.int64))
    w = _weights(rng, rows)
    starts, ends = _causal(rows, keys, keys - rows + 1)
    return Workload(f"x1_offset_{rows}x{keys}_k{topk}", rows, keys, topk, q, k, sb, w, starts,
                    ends, seed)


def extra_elementwise_ties(rows: int = 16384, keys: int = 1048576, topk: int = 2048) -> Workload:
    """Config 5 shape with k drawn per element from 16 distinct e4m3 values."""
    seed = SEED_BASE + 12
    rng = np.random.Generator(np.random.PCG64(seed))
    q = encode_e4m3(_normal(rng, (rows, HEADS, DIM)))
    vals = encode_e4m3(_normal(rng, 16))
    k = vals[rng.integers(0, 16, size=(keys, DIM))]
    sb = _scales(rng, keys)
    w = _weights(rng, rows)
    starts, ends = _causal(rows, keys, keys - rows + 1)
    return Workload(f"x2_elemties_{rows}x{keys}_k{topk}", rows, keys, topk, q, k, sb, w, starts,
                    ends, seed)


def extra_near_tie_groups(rows: int = 64, keys: int = 65536, topk: int = 2048,
                          group: int = 9000) -> Workload:
    """Two groups of `group` identical keys each, at random positions, whose
    scores differ by about 2e-5 of their size (above the checker's tolerance,
    below the certified select's margin), every other key far below them.
    Head 0 of every query is (0.0390625, 1, ..., 1) and the other heads are
    zero; group A keys are all ones, group B keys are all ones except 0.9375 in
    dim 0, the remaining keys are e4m3(N(0,1) / 4); every scale is 1.0 and
    head 0's weight is uniform in [0.5, 2) (the other weights, N(0,1)/sqrt(32),
    multiply zero dots). The two groups together overfill a candidate slab,
    so the scan must drop group B by merging."""
    seed = SEED_BASE + 13
    rng = np.random.Generator(np.random.PCG64(seed))
    qf = np.zeros((rows, HEADS, DIM), np.float32)
    qf[:, 0, :] = 1.0
    qf[:, 0, 0] = 0.0390625
    q = encode_e4m3(qf)
    kf = _normal(rng, (keys, DIM)) / np.float32(4.0)
    perm = rng.permutation(keys)
    kf[perm[:group]] = 1.0
    kf[perm[group:2 * group]] = 1.0
    kf[perm[group:2 * group], 0] = 0.9375
    k = encode_e4m3(kf)
    sb = ue8m0_bytes(np.zeros(keys, np.int64))
    w = _weights(rng, rows)
    w[:, 0] = rng.uniform(0.5, 2.0, size=rows).astype(np.float32)
    starts = np.zeros(rows, np.int32)
    ends = np.full(rows, keys, np.int32)
    return Workload(f"x3_neartie_{rows}x{keys}_k{topk}", rows, keys, topk, q, k, sb, w, starts,
                    ends, seed, groups={"group_a": np.sort(perm[:group]).astype(np.int32),
                                        "group_b": np.sort(perm[group:2 * group]).astype(np.int32)})


def extra_repeated_keys(rows: int = 64, keys: int = 8192, topk: int = 512,
                        distinct: int = 256) -> Workload:
    """Keys drawn from `distinct` e4m3 vectors (each (vector, scale) pair
    repeats about keys / (distinct * 5) times), config-3 q, scale and weight
    distributions; row i sees [0, 6000 + 32 i). Small groups of tied scores
    sit everywhere, also at the rank where a full candidate slab is cut."""
    seed = SEED_BASE + 14
    rng = np.random.Generator(np.random.PCG64(seed))
    q = encode_e4m3(_normal(rng, (rows, HEADS, DIM)))
    vecs = encode_e4m3(_normal(rng, (distinct, DIM)))
    k = vecs[rng.integers(0, distinct, size=keys)]
    sb = _scales(rng, keys)
    w = _weights(rng, rows)
    starts = np.zeros(rows, np.int32)
    ends = (6000 + 32 * np.arange(rows)).astype(np.int32)
    assert int(ends[-1]) <= keys
    return Workload(f"x4_repkeys_{rows}x{keys}_k{topk}", rows, keys, topk, q, k, sb, w, starts,
                    ends, seed)


OUTLIER_PAIRS = ((3, 5), (12, 100), (40, 41), (66, 127))


def extra_outlier_channels(rows: int = 16384, keys: int = 131072, topk: int = 2048,
                           frac: float = 0.03) -> Workload:
    """Config 3 shape with heterogeneous key magnitudes: every query copies dim
    a into dim b for four pairs (a, b), and a fraction `frac` of the keys carry
    +448 in dim a and -448 in dim b of one pair (sign and pair random). The
    pair cancels in every exact dot product, so those keys score like the
    others, but each dominates its 8-dim group of products by far."""
    seed = SEED_BASE + 15
    rng = np.random.Generator(np.random.PCG64(seed))
    qf = _normal(rng, (rows, HEADS, DIM))
    for a, b in OUTLIER_PAIRS:
        qf[:, :, b] = qf[:, :, a]
    q = encode_e4m3(qf)
    del qf
    kf = _normal(rng, (keys, DIM))
    nout = int(frac * keys)
    idx = rng.choice(keys, size=nout, replace=False)
    which = rng.integers(0, len(OUTLIER_PAIRS), size=nout)
    sign = rng.choice(np.array([-1.0, 1.0], np.float32), size=nout)
    for i, (a, b) in enumerate(OUTLIER_PAIRS):
        sel = which == i
        kf[idx[sel], a] = 448.0 * sign[sel]
        kf[idx[sel], b] = -448.0 * sign[sel]
    k = encode_e4m3(kf)
    sb = _scales(rng, keys)
    w = _weights(rng, rows)
    starts, ends = _causal(rows, keys, keys - rows + 1)
    return Workload(f"x5_outliers_{rows}x{keys}_k{topk}", rows, keys, topk, q, k, sb, w, starts,
                    ends, seed)


def extra_truncation_worst(rows: int = 64, keys: int = 8192, topk: int = 512) -> Workload:
    """Near-worst case of the FP8 MFMA's truncation: one head per row (weight
    in [0.5, 2), the other heads zero). In every group of 8 dims the query
    holds a large value (1, 1.125 or 1.25) and seven values of 5..7 * 2^-9,
    the key a large value (0.5 .. 1.75) and seven values of 2..4 * 2^-9, so
    the seven small products of each group fall below the group's truncation
    grid. Scales 1; row i sees [0, 6000 + 32 i)."""
    seed = SEED_BASE + 16
    rng = np.random.Generator(np.random.PCG64(seed))
    big_q = encode_e4m3(np.array([1.0, 1.125, 1.25], np.float32))
    big_k = encode_e4m3(np.array([0.5, 0.75, 1.0, 1.25, 1.5, 1.75], np.float32))
    q = np.zeros((rows, HEADS, DIM), np.uint8)
    k = np.zeros((keys, DIM), np.uint8)
    for g in range(DIM // 8):
        q[:, 0, 8 * g] = big_q[rng.integers(0, 3, size=rows)]
        q[:, 0, 8 * g + 1: 8 * g + 8] = rng.integers(5, 8, size=(rows, 7))
        k[:, 8 * g] = big_k[rng.integers(0, 6, size=keys)]
        k[:, 8 * g + 1: 8 * g + 8] = rng.integers(2, 5, size=(keys, 7))
    sb = ue8m0_bytes(np.zeros(keys, np.int64))
    w = np.zeros((rows, HEADS), np.float32)
    w[:, 0] = rng.uniform(0.5, 2.0, size=rows).astype(np.float32)
    starts = np.zeros(rows, np.int32)
    ends = (6000 + 32 * np.arange(rows)).astype(np.int32)
    return Workload(f"x6_truncworst_{rows}x{keys}_k{topk}", rows, keys, topk, q, k, sb, w,
                    starts, ends, seed)


def custom(rows: int, keys: int, topk: int, starts, ends, seed: int = 1,
           q_offset: float = 0.0, weight_scale: float = 1.0, name: str = "custom") -> Workload:
    """Small hand-shaped inputs for edge-case tests (ragged ranges, empty rows)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = encode_e4m3(_normal(rng, (rows, HEADS, DIM)) + np.float32(q_offset))
    k = encode_e4m3(_normal(rng, (keys, DIM)))
    sb = _scales(rng, keys)
    w = (_weights(rng, rows) * np.float32(weight_scale)).astype(np.float32)
    return Workload(name, rows, keys, topk, q, k, sb, w,
                    np.asarray(starts, np.int32).copy(), np.asarray(ends, np.int32).copy(), seed)


def paged_cache(k: np.ndarray, scale_bytes: np.ndarray, page_size: int, seed: int = 3,
                spare_pages: int = 3):
    """Lay keys out in a paged indexer cache: each page holds page_size
    key rows (128 e4m3 bytes each), then their four scale bytes each. The
    pages of consecutive key runs go to a seeded random permutation of
    ceil(keys / page_size) + spare_pages pages; spare pages and unused slots
    are filled with random bytes. Returns (cache [pages, 132 * page_size]
    uint8, table [ceil(keys / page_size)] int32)."""
    keys = k.shape[0]
    used = -(-keys // page_size)
    rng = np.random.Generator(np.random.PCG64(seed))
    pages = used + spare_pages
    cache = rng.integers(0, 256, (pages, page_size * (DIM + 4)), dtype=np.uint8)
    table = rng.permutation(pages)[:used].astype(np.int32)
    for i in range(used):
        lo, hi = i * page_size, min(keys, (i + 1) * page_size)
        n = hi - lo
        page = cache[table[i]]
        page[: n * DIM] = k[lo:hi].reshape(-1)
        page[page_size * DIM: page_size * DIM + 4 * n] = scale_bytes[lo:hi].reshape(-1)
    return cache, table


@dataclasses.dataclass
class DecodeWorkload:
    """Decode-shaped inputs: `requests` requests of R query rows each (row r
    is row r % R of request r // R; row j of a request with context length L
    sees positions [0, L - (R - 1 - j)), as speculative tokens do), the keys
    of each request in a paged indexer cache, and the same keys gathered and
    concatenated (request q's keys at offset base[q]) for the oracle."""
    name: str
    requests: int
    R: int
    topk: int
    page_size: int
    q: np.ndarray            # uint8 [rows, 32, 128]
    weights: np.ndarray      # float32 [rows, 32]
    starts: np.ndarray       # int32 [rows], positions in the row's request
    ends: np.ndarray         # int32 [rows]
    lens: np.ndarray         # int32 [requests] context lengths
    base: np.ndarray         # int64 [requests] offsets into k_cat
    k_cat: np.ndarray        # uint8 [sum(lens), 128]
    sb_cat: np.ndarray       # uint8 [sum(lens), 4]
    cache: np.ndarray        # uint8 [pages, 132 * page_size]
    table: np.ndarray        # int32 [requests, table_stride], -1 past a request's pages
    seed: int

    @property
    def rows(self) -> int:
        return self.requests * self.R

    def visible_pairs(self) -> int:
        return int(np.maximum(self.ends.astype(np.int64) - self.starts, 0).sum())

    def gathered(self) -> Workload:
        """The same problem over the concatenated keys (ranges shifted by
        each row's request offset): outputs (key - start) are identical."""
        off = np.repeat(self.base, self.R).astype(np.int64)
        return Workload(self.name + "_gathered", self.rows, int(self.k_cat.shape[0]), self.topk,
                        self.q, self.k_cat, self.sb_cat, self.weights,
                        (self.starts + off).astype(np.int32), (self.ends + off).astype(np.int32),
                        self.seed)


def decode(requests: int, R: int, lens, topk: int, page_size: int = 64, seed: int = 1,
           spare_pages: int = 5, table_extra: int = 2, name: str = "decode") -> DecodeWorkload:
    """Seeded decode inputs with the given context lengths (one per request):
    config-3-like q, keys, scales and weights; each request's pages are taken
    from a random permutation of all pages (spare pages of random bytes in
    between), its table row lists them, then table_extra entries of -1."""
    rng = np.random.Generator(np.random.PCG64(SEED_BASE + 1000 + seed))
    lens = np.asarray(lens, np.int64)
    assert lens.shape == (requests,) and (lens >= 1).all()
    rows = requests * R
    q = encode_e4m3(_normal(rng, (rows, HEADS, DIM)))
    total = int(lens.sum())
    k_cat = encode_e4m3(_normal(rng, (total, DIM)))
    sb_cat = _scales(rng, total)
    w = _weights(rng, rows)
    base = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    j = np.tile(np.arange(R), requests)
    ends = (np.repeat(lens, R) - (R - 1 - j)).clip(0).astype(np.int32)
    starts = np.zeros(rows, np.int32)
    npg = -(-lens // page_size)
    pages = int(npg.sum()) + spare_pages
    cache = rng.integers(0, 256, (pages, page_size * (DIM + 4)), dtype=np.uint8)
    perm = rng.permutation(pages)
    stride = int(npg.max()) + table_extra
    table = np.full((requests, stride), -1, np.int32)
    at = 0
    for qi in range(requests):
        for i in range(int(npg[qi])):
            pg = int(perm[at])
            at += 1
            table[qi, i] = pg
            lo = int(base[qi]) + i * page_size
            n = min(page_size, int(lens[qi]) - i * page_size)
            cache[pg, : n * DIM] = k_cat[lo: lo + n].reshape(-1)
            cache[pg, page_size * DIM: page_size * DIM + 4 * n] = sb_cat[lo: lo + n].reshape(-1)
    return DecodeWorkload(name, requests, R, topk, page_size, q, w, starts, ends,
                          lens.astype(np.int32), base, k_cat, sb_cat, cache, table, seed)


def decode_device(requests: int, R: int, ctx: int, topk: int, page_size: int = 64,
                  seed: int = 1, device="cuda"):
    """Decode inputs generated on the device (torch's seeded generator), for
    benchmark sizes the host would take minutes to draw: every request has
    context ctx, q and keys are N(0,1) rounded to e4m3 by torch's
    round-to-nearest conversion, scale exponents uniform in [-4, 0], weights
    N(0,1)/sqrt(32), rows ranged as in decode(); request q's pages are
    q * (ctx / page_size) + i (one contiguous run of the cache each).
    Returns a dict of device tensors."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(SEED_BASE + 2000 + seed)
    rows = requests * R
    npg = -(-ctx // page_size)
    pages = requests * npg
    f8 = torch.float8_e4m3fn
    q = torch.randn((rows, HEADS, DIM), generator=g, device=device).to(f8).view(torch.uint8)
    w = (torch.randn((rows, HEADS), generator=g, device=device) / math.sqrt(HEADS)).float()
    cache = torch.empty((pages, page_size * (DIM + 4)), dtype=torch.uint8, device=device)
    for p0 in range(0, pages, 4096):
        p1 = min(pages, p0 + 4096)
        keys = torch.randn((p1 - p0, page_size * DIM), generator=g, device=device).to(f8)
        cache[p0:p1, : page_size * DIM] = keys.view(torch.uint8)
        e = torch.randint(123, 128, (p1 - p0, page_size, 1), generator=g, device=device,
                          dtype=torch.int32).to(torch.uint8)
        cache[p0:p1, page_size * DIM:] = e.expand(-1, -1, 4).reshape(p1 - p0, -1)
    table = torch.arange(pages, dtype=torch.int32, device=device).view(requests, npg)
    j = torch.arange(R, device=device).repeat(requests)
    ends = (ctx - (R - 1 - j)).clamp(min=0).to(torch.int32)
    starts = torch.zeros(rows, dtype=torch.int32, device=device)
    return {"q": q, "weights": w, "cache": cache, "table": table, "starts": starts, "ends": ends,
            "rows": rows, "pairs": int(ends.sum().item())}


def heads64(rows: int, keys: int, topk: int, starts, ends, seed: int = 1,
            name: str = "heads64") -> Workload:
    """64 index heads (DeepSeek-V3.2's indexer): q [rows, 64, 128] and weights
    [rows, 64] drawn like the 32-head workloads (weights N(0,1)/sqrt(64)),
    keys and scales as config 3; row ranges given."""
    rng = np.random.Generator(np.random.PCG64(SEED_BASE + 3000 + seed))
    q = encode_e4m3(_normal(rng, (rows, 64, DIM)))
    k = encode_e4m3(_normal(rng, (keys, DIM)))
    sb = _scales(rng, keys)
    w = (rng.standard_normal((rows, 64)) / math.sqrt(64)).astype(np.float32)
    return Workload(name, rows, keys, topk, q, k, sb, w, np.asarray(starts, np.int32).copy(),
                    np.asarray(ends, np.int32).copy(), seed)


def sample_rows(wl: Workload, n: int = 256, seed: int = 7) -> np.ndarray:
    """Seeded row sample for oracle checks of large workloads. With groups
    (config 5) it is stratified: half uniform over ungrouped rows, the rest
    split evenly over the groups."""
    if wl.rows <= n:
        return np.arange(wl.rows, dtype=np.int32)
    rng = np.random.Generator(np.random.PCG64(seed + wl.seed))
    if not wl.groups:
        return np.sort(rng.choice(wl.rows, size=n, replace=False)).astype(np.int32)
    grouped = np.concatenate(list(wl.groups.values()))
    rest = np.setdiff1d(np.arange(wl.rows), grouped)
    per = (n // 2) // len(wl.groups)
    picks = [rng.choice(rest, size=n - per * len(wl.groups), replace=False)]
    for g in wl.groups.values():
        picks.append(rng.choice(g, size=per, replace=False))
    return np.sort(np.concatenate(picks)).astype(np.int32)
