"""CPU oracle for FP8 MQA logits + per-row top-k (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product path (the HIP library and
its binding in ``fp8_mqa_logits_amd``) never does, and this package never
imports the product path. The arithmetic lives in ``mqa_oracle.cpp`` (plain
C++, built with g++); this module only marshals numpy arrays through ctypes.

What is computed, and which passage each step follows, is stated at the top of
``mqa_oracle.cpp``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mqa_oracle.cpp")
_LIB = os.path.join(_HERE, "libmqa_oracle.so")

HEADS = 32
DIM = 128


def build(force: bool = False) -> str:
    """Compile the oracle with g++ (plain host code, no GPU involved)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        cmd = ["g++", "-O3", "-std=c++17", "-ffp-contract=off", "-fPIC", "-shared",
               "-pthread", "-o", tmp, _SRC]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.oracle_e4m3_table.argtypes = [P]
        lib.oracle_e4m3_table.restype = None
        lib.oracle_key_scales.argtypes = [P, I64, P]
        lib.oracle_key_scales.restype = None
        I = ctypes.c_int
        lib.oracle_head_dots.argtypes = [P, P, P, I]
        lib.oracle_head_dots.restype = ctypes.c_int
        lib.oracle_logits.argtypes = [P, P, P, P, P, P, I64, I64, I, P, I64, I64, I64, P, I]
        lib.oracle_logits.restype = ctypes.c_int
        lib.oracle_topk.argtypes = [P, P, P, P, P, P, I64, I64, I, P, I64, I64, P, P, P, I]
        lib.oracle_topk.restype = ctypes.c_int
        lib.oracle_select.argtypes = [P, I64, I64, P]
        lib.oracle_select.restype = None
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def e4m3_table() -> np.ndarray:
    """float64 [256]: the value of every OCP e4m3fn code (NaN for 0x7F, 0xFF)."""
    out = np.empty(256, np.float64)
    _load().oracle_e4m3_table(_ptr(out))
    return out


def key_scales(scale_bytes: np.ndarray) -> np.ndarray:
    """UE8M0 scales [keys, 4] uint8 -> fp32 [keys] (bit pattern e << 23)."""
    b = _c(scale_bytes, np.uint8)
    assert b.ndim == 2 and b.shape[1] == 4
    out = np.empty(b.shape[0], np.float32)
    _load().oracle_key_scales(_ptr(b), b.shape[0], _ptr(out))
    return out


def head_dots(q_row: np.ndarray, k_row: np.ndarray) -> np.ndarray:
    """Exact per-head dots: q_row [H,128] e4m3 bytes (H = 32 or 64), k_row
    [128] -> float64 [H]."""
    heads = np.asarray(q_row).size // DIM
    q = _c(q_row, np.uint8).reshape(heads, DIM)
    k = _c(k_row, np.uint8).reshape(DIM)
    out = np.empty(heads, np.float64)
    if _load().oracle_head_dots(_ptr(q), _ptr(k), _ptr(out), heads) != 0:
        raise ValueError("oracle_head_dots: heads must be 32 or 64")
    return out


class Problem:
    """Host copies of one call's inputs (numpy), in the op's layouts."""

    def __init__(self, q, k, scales, weights, starts, ends):
        q = np.asarray(q)
        # 32 heads, or 64 (q [rows, 64, 128], weights [rows, 64])
        self.heads = q.shape[1] if q.ndim == 3 else HEADS
        assert self.heads in (32, 64), self.heads
        self.q = _c(q, np.uint8).reshape(-1, self.heads, DIM)
        self.k = _c(k, np.uint8).reshape(-1, DIM)
        self.scales = _c(scales, np.float32)
        self.weights = _c(weights, np.float32).reshape(-1, self.heads)
        self.starts = _c(starts, np.int32)
        self.ends = _c(ends, np.int32)
        self.rows = self.q.shape[0]
        self.keys = self.k.shape[0]
        assert self.scales.shape == (self.keys,)
        assert self.weights.shape[0] == self.rows
        assert self.starts.shape == (self.rows,) and self.ends.shape == (self.rows,)

    def _args(self):
        return (_ptr(self.q), _ptr(self.k), _ptr(self.scales), _ptr(self.weights),
                _ptr(self.starts), _ptr(self.ends), self.rows, self.keys, self.heads)

    def visible(self, r):
        """Clamped visible range (s, e) of row r."""
        s = min(max(int(self.starts[r]), 0), self.keys)
        e = min(max(int(self.ends[r]), s), self.keys)
        return s, e


def logits(p: Problem, rows, col0: int = 0, ncols: int | None = None,
           threads: int = 0) -> np.ndarray:
    """fp32 [len(rows), ncols] logits of the given rows over keys col0..col0+ncols-1;
    -inf outside each row's visible range."""
    sel = _c(rows, np.int32).reshape(-1)
    if ncols is None:
        ncols = p.keys - col0
    out = np.empty((sel.shape[0], ncols), np.float32)
    rc = _load().oracle_logits(*p._args(), _ptr(sel), sel.shape[0], col0, ncols,
                               _ptr(out), threads)
    if rc != 0:
        raise ValueError("oracle_logits: input outside the contract")
    return out


def topk(p: Problem, rows, k: int, threads: int = 0):
    """Per selected row: (idx [n_sel, k] int32 relative to start, -1 padded;
    kth [n_sel] fp32, the k-th largest logit or -inf; maxabs [n_sel] fp32)."""
    sel = _c(rows, np.int32).reshape(-1)
    idx = np.empty((sel.shape[0], k), np.int32)
    kth = np.empty(sel.shape[0], np.float32)
    mx = np.empty(sel.shape[0], np.float32)
    rc = _load().oracle_topk(*p._args(), _ptr(sel), sel.shape[0], k, _ptr(idx),
                             _ptr(kth), _ptr(mx), threads)
    if rc != 0:
        raise ValueError("oracle_topk: input outside the contract")
    return idx, kth, mx


def select(values: np.ndarray, k: int) -> np.ndarray:
    """The oracle's selection step alone: positions of the k largest values by
    (value descending, position ascending)."""
    v = _c(values, np.float32).reshape(-1)
    out = np.full(min(k, v.shape[0]), -1, np.int32)
    _load().oracle_select(_ptr(v), v.shape[0], k, _ptr(out))
    return out
