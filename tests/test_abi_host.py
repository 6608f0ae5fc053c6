"""Host-side checks of the C ABI: the library loads, exports every entry
point include/mqa_topk.h declares, and rejects bad arguments before touching
any device memory. No GPU needed (and nothing here launches work)."""
import ctypes
import os
import re

import pytest

import fp8_mqa_logits_amd as mqa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mqa_topk.h")

# fake, never-dereferenced device addresses (all checks fail before any use)
A16 = 0x10000
MIS = 0x10004


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[a-z_][a-z0-9_ ]*[ *]+(\w+)\(", text, flags=re.M)))


def test_header_declares_the_abi():
    names = declared_functions()
    assert set(names) == {"workspace_size", "mqa_topk_prefill", "mqa_topk_prefill_static",
                          "workspace_size_heads", "mqa_topk_prefill_heads", "mqa_topk_masked",
                          "mqa_topk_prefill_blocks",
                          "mqa_topk_prefill_paged", "workspace_size_paged",
                          "workspace_size_decode",
                          "mqa_topk_decode_paged", "mqa_logits_dense",
                          "mqa_topk_dense", "mqa_key_scales", "mqa_scan_time", "mqa_mfma_peak",
                          "mqa_fp8_mfma_probe",
                          "mqa_strerror"}


def test_binding_flags_match_the_header():
    text = open(HEADER).read()
    defs = {m.group(1): int(m.group(2)) for m in
            re.finditer(r"#define MQA_FLAG_(\w+) (\d+)u", text)}
    assert defs, "no MQA_FLAG_ defines found"
    for name, value in defs.items():
        assert getattr(mqa, "FLAG_" + name) == value, name
    assert len(set(defs.values())) == len(defs)


def test_library_exports_every_declared_symbol():
    lib = mqa.load()
    for n in declared_functions():
        assert hasattr(lib, n), n
    assert set(mqa.EXPORTS) == set(declared_functions())


def _prefill(**kw):
    a = dict(q=A16, k=A16, scales=A16, weights=A16, starts=A16, ends=A16, out=A16, rows=64,
             keys=4096, topk=512, ws=0x20000, wsb=1 << 40, flags=0)
    a.update(kw)
    P = ctypes.c_void_p
    return mqa.load().mqa_topk_prefill(P(a["q"]), P(a["k"]), P(a["scales"]), P(a["weights"]),
                                       P(a["starts"]), P(a["ends"]), P(a["out"]), a["rows"],
                                       a["keys"], a["topk"], P(a["ws"]), a["wsb"], a["flags"],
                                       None)


def test_prefill_null_align_shape_errors():
    assert _prefill(q=0) == 1
    assert _prefill(ws=0) == 1
    assert _prefill(k=MIS) == 2
    assert _prefill(out=MIS) == 2
    assert _prefill(starts=0x10002) == 2
    assert _prefill(ws=0x20080) == 2
    assert _prefill(rows=0) == 3
    assert _prefill(keys=0) == 3
    assert _prefill(keys=(1 << 20) + 1) == 3
    assert _prefill(topk=256) == 3
    assert _prefill(topk=4096) == 3


def test_dense_errors():
    P = ctypes.c_void_p
    L = mqa.load()

    def dense(**kw):
        a = dict(q=A16, logits=A16, ld=4096, rows=8, keys=4096, col0=0, ncols=4096)
        a.update(kw)
        return L.mqa_logits_dense(P(a["q"]), P(A16), P(A16), P(A16), P(A16), P(A16),
                                  P(a["logits"]), a["ld"], a["rows"], a["keys"], a["col0"],
                                  a["ncols"], None)

    assert dense(q=0) == 1
    assert dense(logits=MIS) == 2
    assert dense(ld=4095) == 3
    assert dense(ld=4098) == 3
    assert dense(col0=1) == 3        # window past the last key
    assert dense(ncols=0) == 3
    assert dense(col0=-1) == 3

    def topk(**kw):
        a = dict(logits=A16, ld=4096, col0=0, ncols=4096, out=A16, rows=8, keys=4096, topk=512)
        a.update(kw)
        return L.mqa_topk_dense(P(a["logits"]), a["ld"], a["col0"], a["ncols"], P(A16), P(A16),
                                P(a["out"]), a["rows"], a["keys"], a["topk"], None)

    assert topk(out=0) == 1
    assert topk(out=MIS) == 2
    assert topk(topk=100) == 3
    assert topk(ncols=5000) == 3
    assert L.mqa_key_scales(None, P(A16), 10, None) == 1
    assert L.mqa_key_scales(P(0x10001), P(A16), 10, None) == 2
    assert L.mqa_key_scales(P(A16), P(A16), 0, None) == 3
    assert L.mqa_scan_time(1, None) == 1


def _peak(out=A16, out_len=512 * 4, workgroups=4, iters=16):
    return mqa.load().mqa_mfma_peak(ctypes.c_void_p(out), out_len, workgroups, iters, None)


def test_mfma_peak_errors():
    assert _peak(out=0) == 1
    assert _peak(out=0x10002) == 2
    assert _peak(workgroups=0) == 3
    assert _peak(workgroups=65537, out_len=1 << 40) == 3
    assert _peak(iters=0) == 3
    assert _peak(iters=(1 << 20) + 1) == 3
    assert _peak(out_len=4 * 512 - 1) == 3


def test_strerror_covers_every_code():
    for c in range(0, 7):
        assert mqa.strerror(c)
    assert "unknown" in mqa.strerror(99)


def _no_gpu():
    import torch
    return not torch.cuda.is_available()


@pytest.mark.skipif(not _no_gpu(), reason="only meaningful on a host without a GPU")
def test_device_error_without_gpu():
    # valid arguments on a host with no HIP device: MQA_ERR_DEVICE, nothing launched
    assert _prefill() == 5
    assert mqa.load().workspace_size(64, 0) == 0
    v = ctypes.c_float(0.0)
    assert mqa.load().mqa_scan_time(1, ctypes.byref(v)) == 5
    assert _peak() == 5


def _static(**kw):
    a = dict(q=A16, k=A16, scales=A16, weights=A16, starts=A16, ends=A16, out=A16, rows=64,
             keys=4096, topk=512, flags=0)
    a.update(kw)
    P = ctypes.c_void_p
    return mqa.load().mqa_topk_prefill_static(P(a["q"]), P(a["k"]), P(a["scales"]),
                                              P(a["weights"]), P(a["starts"]), P(a["ends"]),
                                              P(a["out"]), a["rows"], a["keys"], a["topk"],
                                              a["flags"], None)


def test_static_prefill_errors():
    assert _static(q=0) == 1
    assert _static(out=0) == 1
    assert _static(weights=MIS) == 2
    assert _static(ends=0x10002) == 2
    assert _static(rows=0) == 3
    assert _static(keys=(1 << 20) + 1) == 3
    assert _static(topk=1000) == 3
    if _no_gpu():
        assert _static() == 5  # valid arguments, no device: nothing launched


def _paged(**kw):
    a = dict(q=A16, cache=A16, table=A16, page=64, pages=64, weights=A16, starts=A16, ends=A16,
             out=A16, rows=64, keys=4096, topk=512, ws=0x20000, wsb=1 << 40, flags=0)
    a.update(kw)
    P = ctypes.c_void_p
    return mqa.load().mqa_topk_prefill_paged(P(a["q"]), P(a["cache"]), P(a["table"]), a["page"],
                                             a["pages"], P(a["weights"]), P(a["starts"]),
                                             P(a["ends"]), P(a["out"]), a["rows"], a["keys"],
                                             a["topk"], P(a["ws"]), a["wsb"], a["flags"], None)


def test_paged_prefill_errors():
    assert _paged(cache=0) == 1
    assert _paged(table=0) == 1
    assert _paged(ws=0) == 1
    assert _paged(cache=MIS) == 2
    assert _paged(table=0x10002) == 2
    assert _paged(ws=0x20080) == 2
    for page in (0, 2, 48, 100, 1 << 21):
        assert _paged(page=page) == 3, page
    assert _paged(pages=0) == 3
    assert _paged(rows=0) == 3
    assert _paged(keys=(1 << 20) + 1) == 3
    assert _paged(topk=300) == 3
    if _no_gpu():
        assert _paged() == 5
        assert _paged(page=4) == 5
        assert _paged(page=1 << 20) == 5


def _decode(**kw):
    a = dict(q=A16, cache=A16, table=A16, stride=8, page=64, pages=64, weights=A16, starts=A16,
             ends=A16, out=A16, requests=16, R=8, topk=512, ws=0x20000, wsb=1 << 40, flags=0)
    a.update(kw)
    P = ctypes.c_void_p
    return mqa.load().mqa_topk_decode_paged(P(a["q"]), P(a["cache"]), P(a["table"]), a["stride"],
                                            a["page"], a["pages"], P(a["weights"]),
                                            P(a["starts"]), P(a["ends"]), P(a["out"]),
                                            a["requests"], a["R"], a["topk"], P(a["ws"]),
                                            a["wsb"], a["flags"], None)


def test_decode_errors():
    assert _decode(table=0) == 1
    assert _decode(out=0) == 1
    assert _decode(cache=MIS) == 2
    assert _decode(table=0x10001) == 2
    for kw in (dict(R=0), dict(R=33), dict(requests=0), dict(stride=0), dict(page=24),
               dict(pages=0), dict(topk=100), dict(requests=1 << 20, R=2)):
        assert _decode(**kw) == 3, kw
    assert mqa.load().workspace_size_decode(16, 8, 0) == 0 or not _no_gpu()
    assert mqa.load().workspace_size_decode(16, 33, 0) == 0
    if _no_gpu():
        assert _decode() == 5
        assert _decode(R=1, requests=4096) == 5


def test_heads_prefill_errors():
    P = ctypes.c_void_p

    def call(**kw):
        a = dict(q=A16, k=A16, scales=A16, weights=A16, starts=A16, ends=A16, out=A16,
                 rows=64, keys=4096, heads=64, topk=512, ws=0x20000, wsb=1 << 40)
        a.update(kw)
        return mqa.load().mqa_topk_prefill_heads(
            P(a["q"]), P(a["k"]), P(a["scales"]), P(a["weights"]), P(a["starts"]), P(a["ends"]),
            P(a["out"]), a["rows"], a["keys"], a["heads"], a["topk"], P(a["ws"]), a["wsb"], 0,
            None)
    assert call(q=0) == 1
    assert call(weights=MIS) == 2
    for h in (0, 16, 48, 96, 128):
        assert call(heads=h) == 3, h
    assert call(rows=0) == 3
    assert mqa.load().workspace_size_heads(64, 48, 0) == 0
    if _no_gpu():
        assert call() == 5
        assert call(heads=32) == 5


def test_masked_errors():
    P = ctypes.c_void_p

    def call(**kw):
        a = dict(q=A16, k=A16, scales=A16, weights=A16, starts=A16, ends=A16, blocks=A16, nb=2048,
                 out=A16, rows=64, keys=4096, topk=512, ws=0x20000, wsb=1 << 40)
        a.update(kw)
        return mqa.load().mqa_topk_masked(
            P(a["q"]), P(a["k"]), P(a["scales"]), P(a["weights"]), P(a["starts"]), P(a["ends"]),
            P(a["blocks"]), a["nb"], P(a["out"]), a["rows"], a["keys"], a["topk"], P(a["ws"]),
            a["wsb"], 0, None)
    assert call(blocks=0) == 1
    assert call(blocks=0x10002) == 2
    assert call(nb=0) == 3 and call(nb=2049) == 3
    assert call(topk=2047) == 3
    if _no_gpu():
        assert call() == 5


def test_fp8_probe_errors():
    P = ctypes.c_void_p
    L = mqa.load()
    assert L.mqa_fp8_mfma_probe(None, P(A16), None, P(A16), 4, None) == 1
    assert L.mqa_fp8_mfma_probe(P(MIS), P(A16), None, P(A16), 4, None) == 2
    assert L.mqa_fp8_mfma_probe(P(A16), P(A16), None, P(A16), 0, None) == 3


def test_binding_checks_every_shape_first():
    # CPU tensors: a wrong shape is reported before the device is looked at,
    # so these run without a GPU; the C ABI itself cannot see tensor sizes
    import torch
    rows, keys = 8, 600
    u8 = lambda *s: torch.zeros(s, dtype=torch.uint8)
    f32 = lambda *s: torch.zeros(s, dtype=torch.float32)
    i32 = lambda *s: torch.zeros(s, dtype=torch.int32)
    good = dict(q=u8(rows, 32, 128), k=u8(keys, 128), scales=f32(keys), weights=f32(rows, 32),
                starts=i32(rows), ends=i32(rows))
    bad = {"q": u8(rows, 16, 128), "k": u8(keys, 64), "scales": f32(keys - 1),
           "weights": f32(rows, 31), "starts": i32(rows + 1), "ends": i32(rows - 1)}
    for name, t in bad.items():
        args = dict(good, **{name: t})
        for fn in (mqa.mqa_topk_prefill, mqa.mqa_topk_prefill_static):
            with pytest.raises(ValueError, match="shape"):
                fn(args["q"], args["k"], args["scales"], args["weights"], args["starts"],
                   args["ends"], 512)
        with pytest.raises(ValueError, match="shape"):
            mqa.mqa_logits_dense(args["q"], args["k"], args["scales"], args["weights"],
                                 args["starts"], args["ends"])
    with pytest.raises(ValueError, match="shape"):
        mqa.mqa_topk_prefill(**good, topk=512, out=i32(rows, 511))
    with pytest.raises(ValueError, match="shape"):
        mqa.mqa_topk_dense(f32(rows, keys), i32(rows + 1), i32(rows), 512, keys)
    with pytest.raises(ValueError, match="shape"):
        mqa.mqa_topk_dense(f32(rows, keys), i32(rows), i32(rows), 512, keys, out=i32(rows, 4))
    with pytest.raises(ValueError):
        mqa.mqa_key_scales(u8(keys * 4))  # flat bytes, not [keys, 4]
    with pytest.raises(ValueError, match="shape"):
        mqa.mqa_key_scales(u8(keys, 3))
    with pytest.raises(ValueError, match="shape"):
        mqa.fp8_mfma_probe(u8(2, 16, 128), u8(3, 16, 128))
    # the paged entry: cache pages of 132 B per token, a long enough table
    pg = dict(q=u8(rows, 32, 128), cache=u8(10, 64 * 132), block_table=i32(10), page_size=64,
              keys=keys, weights=f32(rows, 32), starts=i32(rows), ends=i32(rows), topk=512)
    for name, t in (("cache", u8(10, 64 * 128)), ("weights", f32(rows, 30)),
                    ("starts", i32(rows + 2))):
        with pytest.raises(ValueError, match="shape"):
            mqa.mqa_topk_prefill_paged(**dict(pg, **{name: t}))
    with pytest.raises(ValueError, match="block_table"):
        mqa.mqa_topk_prefill_paged(**dict(pg, block_table=i32(9)))
    with pytest.raises(ValueError, match="page_size"):
        mqa.mqa_topk_prefill_paged(**dict(pg, page_size=48))
    # the decode entry: rows = requests * rows_per_request, a 2-D page table
    dc = dict(q=u8(16, 32, 128), cache=u8(10, 64 * 132), page_table=i32(2, 5), page_size=64,
              weights=f32(16, 32), starts=i32(16), ends=i32(16), topk=512, rows_per_request=8)
    with pytest.raises(ValueError, match="rows"):
        mqa.mqa_topk_decode_paged(**dict(dc, rows_per_request=4))
    with pytest.raises(ValueError, match="page_table"):
        mqa.mqa_topk_decode_paged(**dict(dc, page_table=i32(10)))
    for name, t in (("cache", u8(10, 64 * 131)), ("weights", f32(16, 31)), ("ends", i32(15))):
        with pytest.raises(ValueError, match="shape"):
            mqa.mqa_topk_decode_paged(**dict(dc, **{name: t}))


def test_paged_cache_layout_round_trips():
    # the paged-cache input builder: gathering each key back through the table
    # (page table[j // P], slot j % P: its 128 code bytes, then its scale word
    # at 128 P + 4 (j % P)) gives the gathered keys and scale bytes again
    import numpy as np
    import mqa_workloads as W
    rng = np.random.default_rng(0)
    keys = 1000
    k = rng.integers(0, 256, (keys, 128), dtype=np.uint8)
    sb = np.repeat(rng.integers(100, 130, (keys, 1), dtype=np.uint8), 4, axis=1)
    for P in (4, 64, 256):
        cache, table = W.paged_cache(k, sb, P, seed=P)
        assert cache.shape == (-(-keys // P) + 3, 132 * P) and table.shape == (-(-keys // P),)
        assert len(set(table.tolist())) == len(table)
        j = np.arange(keys)
        pg, sl = table[j // P], j % P
        kk = cache[pg[:, None], sl[:, None] * 128 + np.arange(128)]
        ss = cache[pg[:, None], 128 * P + 4 * sl[:, None] + np.arange(4)]
        assert np.array_equal(kk, k) and np.array_equal(ss, sb)


C_CALLER = r"""
#include <stdio.h>
#include "mqa_topk.h"

/* a C99 caller of the library: argument errors come back as codes, with
   nothing launched (NULL pointers, a bad row count) */
int main(void) {
  int rc = mqa_topk_prefill(NULL, NULL, NULL, NULL, NULL, NULL, NULL, 64, 4096, 512, NULL, 0,
                            0u, NULL);
  size_t ws = workspace_size(0, 0);
  int rd = mqa_logits_dense(NULL, NULL, NULL, NULL, NULL, NULL, NULL, 4096, 64, 4096, 0, 4096,
                            NULL);
  printf("%d %zu %d %s\n", rc, ws, rd, mqa_strerror(rc));
  return rc == MQA_ERR_NULL && ws == 0 && rd == MQA_ERR_NULL ? 0 : 1;
}
"""


def test_header_is_c_and_the_library_links_from_c(tmp_path):
    # the header compiles as C99 with warnings as errors, and a C program
    # links against the built library and gets its error codes
    import shutil
    import subprocess

    from fp8_mqa_logits_amd import build as b

    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "caller.c"
    src.write_text(C_CALLER)
    exe = tmp_path / "caller"
    subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
                    str(src), "-o", str(exe), b.LIB, "-Wl,-rpath," + os.path.dirname(b.LIB)],
                   check=True, capture_output=True, text=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.split()[:3] == [str(1), "0", str(1)]


def test_bench_refuses_several_gpus():
    # the benchmark is a one-GPU measurement: asked for more it says so and
    # exits before touching a device
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for argv, env in ((["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})):
        r = subprocess.run([sys.executable, os.path.join(root, "bench.py")] + argv,
                           capture_output=True, text=True, timeout=300,
                           env={**os.environ, **env})
        assert r.returncode != 0
        assert "one GPU" in r.stdout + r.stderr
