"""Python binding of libmqa_topk.so: FP8 MQA logits + per-row top-k on gfx950.

Argument marshalling only: every step of the path runs in the HIP kernels of
the library. PyTorch provides device memory and the current stream. The C ABI
and its contract are declared in include/mqa_topk.h. If the library is not
built, every entry point raises (there is no fallback).
"""
from __future__ import annotations

import ctypes
import os

import torch

from . import build as _build

HEADS = 32
HEAD_DIM = 128
MAX_KEYS = 1 << 20
TOPKS = (512, 1024, 2048)

FLAG_FORCE_EXACT = 1
FLAG_FORCE_GATE_MISS = 2
FLAG_SMALL_CAP = 4
FLAG_STATS = 8
FLAG_TIME_SCAN = 16
FLAG_FORCE_RESCAN = 32
FLAG_DETERMINISTIC = 64

ERR_NAMES = {0: "MQA_OK", 1: "MQA_ERR_NULL", 2: "MQA_ERR_ALIGN", 3: "MQA_ERR_SHAPE",
             4: "MQA_ERR_WORKSPACE", 5: "MQA_ERR_DEVICE", 6: "MQA_ERR_LAUNCH"}

EXPORTS = ("workspace_size", "mqa_topk_prefill", "mqa_topk_prefill_static",
           "workspace_size_heads", "mqa_topk_prefill_heads", "mqa_topk_masked",
           "mqa_topk_prefill_blocks",
           "mqa_topk_prefill_paged", "workspace_size_paged", "workspace_size_decode", "mqa_topk_decode_paged",
           "mqa_logits_dense",
           "mqa_topk_dense",
           "mqa_key_scales", "mqa_scan_time", "mqa_mfma_peak", "mqa_fp8_mfma_probe",
           "mqa_strerror")


class MQAError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {ERR_NAMES.get(code, code)} ({strerror(code)})")


_lib = None


def lib_path() -> str:
    return _build.LIB


def load() -> ctypes.CDLL:
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            raise RuntimeError(f"{_build.LIB} is missing: build it with "
                               "`python -m fp8_mqa_logits_amd.build` or __graft_entry__.build()")
        lib = ctypes.CDLL(_build.LIB)
        P, I, I64, SZ, U = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t,
                            ctypes.c_uint)
        lib.workspace_size.argtypes = [I, I]
        lib.workspace_size.restype = SZ
        lib.mqa_topk_prefill.argtypes = [P, P, P, P, P, P, P, I, I, I, P, SZ, U, P]
        lib.mqa_topk_prefill.restype = I
        lib.mqa_topk_prefill_blocks.argtypes = [P, P, P, P, P, P, P, P, I, I, I, P, SZ, U, P]
        lib.mqa_topk_prefill_blocks.restype = I
        lib.mqa_topk_masked.argtypes = [P, P, P, P, P, P, P, I, P, I, I, I, P, SZ, U, P]
        lib.mqa_topk_masked.restype = I
        lib.workspace_size_heads.argtypes = [I, I, I]
        lib.workspace_size_heads.restype = SZ
        lib.mqa_topk_prefill_heads.argtypes = [P, P, P, P, P, P, P, I, I, I, I, P, SZ, U, P]
        lib.mqa_topk_prefill_heads.restype = I
        lib.mqa_topk_prefill_static.argtypes = [P, P, P, P, P, P, P, I, I, I, U, P]
        lib.mqa_topk_prefill_static.restype = I
        lib.mqa_topk_prefill_paged.argtypes = [P, P, P, I, I, P, P, P, P, I, I, I, P, SZ, U, P]
        lib.mqa_topk_prefill_paged.restype = I
        lib.workspace_size_paged.argtypes = [I, I, I]
        lib.workspace_size_paged.restype = SZ
        lib.workspace_size_decode.argtypes = [I, I, I]
        lib.workspace_size_decode.restype = SZ
        lib.mqa_topk_decode_paged.argtypes = [P, P, P, I, I, I, P, P, P, P, I, I, I, P, SZ, U, P]
        lib.mqa_topk_decode_paged.restype = I
        lib.mqa_logits_dense.argtypes = [P, P, P, P, P, P, P, I64, I, I, I, I, P]
        lib.mqa_logits_dense.restype = I
        lib.mqa_topk_dense.argtypes = [P, I64, I, I, P, P, P, I, I, I, P]
        lib.mqa_topk_dense.restype = I
        lib.mqa_key_scales.argtypes = [P, P, I, P]
        lib.mqa_key_scales.restype = I
        lib.mqa_scan_time.argtypes = [I, P]
        lib.mqa_scan_time.restype = I
        lib.mqa_mfma_peak.argtypes = [P, I64, I, I, P]
        lib.mqa_mfma_peak.restype = I
        lib.mqa_fp8_mfma_probe.argtypes = [P, P, P, P, I, P]
        lib.mqa_fp8_mfma_probe.restype = I
        lib.mqa_strerror.argtypes = [I]
        lib.mqa_strerror.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def strerror(code: int) -> str:
    return load().mqa_strerror(int(code)).decode()


def _check(code: int, where: str):
    if code != 0:
        raise MQAError(code, where)


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device, stream=None):
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    return ctypes.c_void_p(s.cuda_stream)


def _need(t: torch.Tensor, name: str, dtypes, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must live on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _tensors(**named):
    for name, t in named.items():
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a tensor")


def _shape(t: torch.Tensor, shape: tuple, name: str):
    # the C ABI takes sizes, not tensors: a short tensor would be read or
    # written out of bounds on the device, so every shape is checked here
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")


FP8 = (torch.float8_e4m3fn, torch.uint8)


def workspace_size(rows: int, device: int | None = None) -> int:
    """Bytes of workspace one mqa_topk_prefill call over `rows` rows needs."""
    if device is None:
        device = torch.cuda.current_device()
    return int(load().workspace_size(int(rows), int(device)))


def alloc_workspace(rows: int, device=None) -> torch.Tensor:
    dev = torch.device("cuda", torch.cuda.current_device() if device is None else device)
    n = workspace_size(rows, dev.index)
    if n == 0:
        raise MQAError(5, "workspace_size")
    return torch.empty(n, dtype=torch.uint8, device=dev)


def workspace_size_heads(rows: int, heads: int, device: int | None = None) -> int:
    """Bytes of workspace one call over `rows` rows of `heads` heads needs."""
    if device is None:
        device = torch.cuda.current_device()
    return int(load().workspace_size_heads(int(rows), int(heads), int(device)))


def mqa_topk_prefill(q, k, scales, weights, starts, ends, topk: int, out=None, workspace=None,
                     flags: int = 0, stream=None) -> torch.Tensor:
    """Fused scores + per-row top-k. q [rows,H,128] e4m3 (or its uint8 bytes),
    H = 32 or 64 index heads, k [keys,128] e4m3, scales [keys] fp32, weights
    [rows,H] fp32, starts/ends [rows] int32; returns out [rows, topk] int32
    (key - start, -1 padded). 64 heads go through mqa_topk_prefill_heads."""
    _tensors(q=q, k=k, scales=scales, weights=weights, starts=starts, ends=ends)
    if q.dim() != 3 or k.dim() != 2:
        raise ValueError("q must be [rows,heads,128] and k [keys,128]")
    rows, keys = q.shape[0], k.shape[0]
    heads = q.shape[1]
    if heads not in (32, 64):
        raise ValueError(f"q: shape {tuple(q.shape)}, expected 32 or 64 heads")
    _shape(q, (rows, heads, HEAD_DIM), "q")
    _shape(k, (keys, HEAD_DIM), "k")
    _shape(scales, (keys,), "scales")
    _shape(weights, (rows, heads), "weights")
    _shape(starts, (rows,), "starts")
    _shape(ends, (rows,), "ends")
    if out is not None:
        _tensors(out=out)
        _shape(out, (rows, topk), "out")
    dev = q.device
    _need(q, "q", FP8, dev)
    _need(k, "k", FP8, dev)
    _need(scales, "scales", (torch.float32,), dev)
    _need(weights, "weights", (torch.float32,), dev)
    _need(starts, "starts", (torch.int32,), dev)
    _need(ends, "ends", (torch.int32,), dev)
    if out is None:
        out = torch.empty((rows, topk), dtype=torch.int32, device=dev)
    _need(out, "out", (torch.int32,), dev)
    _shape(out, (rows, topk), "out")
    if workspace is None:
        n = workspace_size_heads(rows, heads, dev.index)
        if n == 0:
            raise MQAError(5, "workspace_size_heads")
        workspace = torch.empty(n, dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", (torch.uint8,), dev)
    with torch.cuda.device(dev):
        if heads == HEADS:
            rc = load().mqa_topk_prefill(_ptr(q), _ptr(k), _ptr(scales), _ptr(weights),
                                         _ptr(starts), _ptr(ends), _ptr(out), rows, keys,
                                         int(topk), _ptr(workspace), workspace.numel(),
                                         int(flags), _stream(dev, stream))
            where = "mqa_topk_prefill"
        else:
            rc = load().mqa_topk_prefill_heads(_ptr(q), _ptr(k), _ptr(scales), _ptr(weights),
                                               _ptr(starts), _ptr(ends), _ptr(out), rows, keys,
                                               heads, int(topk), _ptr(workspace),
                                               workspace.numel(), int(flags),
                                               _stream(dev, stream))
            where = "mqa_topk_prefill_heads"
    _check(rc, where)
    return out


MAX_BLOCKS = 2048


def mqa_topk_prefill_blocks(q, k, scales, weights, starts, ends, topk: int, out=None,
                            out_blocks=None, workspace=None, flags: int = 0, stream=None):
    """Two-level selection, source layers: mqa_topk_prefill's output and each
    row's 2048 blocks of 8 keys of largest maximum score (block B = keys
    8B..8B+7, named B - start // 8, -1 padded). Returns (out, out_blocks)."""
    _tensors(q=q, k=k, scales=scales, weights=weights, starts=starts, ends=ends)
    if q.dim() != 3 or k.dim() != 2:
        raise ValueError("q must be [rows,32,128] and k [keys,128]")
    rows, keys = q.shape[0], k.shape[0]
    _shape(q, (rows, HEADS, HEAD_DIM), "q")
    _shape(k, (keys, HEAD_DIM), "k")
    _shape(scales, (keys,), "scales")
    _shape(weights, (rows, HEADS), "weights")
    _shape(starts, (rows,), "starts")
    _shape(ends, (rows,), "ends")
    for name, t, shp in (("out", out, (rows, topk)), ("out_blocks", out_blocks, (rows, MAX_BLOCKS))):
        if t is not None:
            _tensors(**{name: t})
            _shape(t, shp, name)
    dev = q.device
    for t, n, dt in ((q, "q", FP8), (k, "k", FP8), (scales, "scales", (torch.float32,)),
                     (weights, "weights", (torch.float32,)), (starts, "starts", (torch.int32,)),
                     (ends, "ends", (torch.int32,))):
        _need(t, n, dt, dev)
    if out is None:
        out = torch.empty((rows, topk), dtype=torch.int32, device=dev)
    if out_blocks is None:
        out_blocks = torch.empty((rows, MAX_BLOCKS), dtype=torch.int32, device=dev)
    _need(out, "out", (torch.int32,), dev)
    _need(out_blocks, "out_blocks", (torch.int32,), dev)
    if workspace is None:
        workspace = alloc_workspace(rows, dev.index)
    _need(workspace, "workspace", (torch.uint8,), dev)
    with torch.cuda.device(dev):
        rc = load().mqa_topk_prefill_blocks(_ptr(q), _ptr(k), _ptr(scales), _ptr(weights),
                                            _ptr(starts), _ptr(ends), _ptr(out), _ptr(out_blocks),
                                            rows, keys, int(topk), _ptr(workspace),
                                            workspace.numel(), int(flags), _stream(dev, stream))
    _check(rc, "mqa_topk_prefill_blocks")
    return out, out_blocks


def mqa_topk_masked(q, k, scales, weights, starts, ends, blocks, topk: int, out=None,
                    workspace=None, flags: int = 0, stream=None) -> torch.Tensor:
    """Two-level selection, consumer layers: the top-k of each row's keys in
    its listed blocks of 8 (blocks [rows, nb] int32, block j = keys
    8 (j + start // 8) .. + 7, entries < 0 padding, distinct otherwise).
    Other arguments as mqa_topk_prefill (32 heads)."""
    _tensors(q=q, k=k, scales=scales, weights=weights, starts=starts, ends=ends, blocks=blocks)
    if q.dim() != 3 or k.dim() != 2 or blocks.dim() != 2:
        raise ValueError("q must be [rows,32,128], k [keys,128] and blocks [rows, nb]")
    rows, keys, nb = q.shape[0], k.shape[0], blocks.shape[1]
    if nb < 1 or nb > MAX_BLOCKS:
        raise ValueError(f"blocks: shape {tuple(blocks.shape)}, nb must be in [1, {MAX_BLOCKS}]")
    _shape(q, (rows, HEADS, HEAD_DIM), "q")
    _shape(k, (keys, HEAD_DIM), "k")
    _shape(scales, (keys,), "scales")
    _shape(weights, (rows, HEADS), "weights")
    _shape(starts, (rows,), "starts")
    _shape(ends, (rows,), "ends")
    _shape(blocks, (rows, nb), "blocks")
    if out is not None:
        _tensors(out=out)
        _shape(out, (rows, topk), "out")
    dev = q.device
    for t, n, dt in ((q, "q", FP8), (k, "k", FP8), (scales, "scales", (torch.float32,)),
                     (weights, "weights", (torch.float32,)), (starts, "starts", (torch.int32,)),
                     (ends, "ends", (torch.int32,)), (blocks, "blocks", (torch.int32,))):
        _need(t, n, dt, dev)
    if out is None:
        out = torch.empty((rows, topk), dtype=torch.int32, device=dev)
    _need(out, "out", (torch.int32,), dev)
    if workspace is None:
        workspace = alloc_workspace(rows, dev.index)
    _need(workspace, "workspace", (torch.uint8,), dev)
    with torch.cuda.device(dev):
        rc = load().mqa_topk_masked(_ptr(q), _ptr(k), _ptr(scales), _ptr(weights), _ptr(starts),
                                    _ptr(ends), _ptr(blocks), nb, _ptr(out), rows, keys,
                                    int(topk), _ptr(workspace), workspace.numel(), int(flags),
                                    _stream(dev, stream))
    _check(rc, "mqa_topk_masked")
    return out


def mqa_topk_prefill_static(q, k, scales, weights, starts, ends, topk: int, out=None,
                            flags: int = 0, stream=None) -> torch.Tensor:
    """mqa_topk_prefill through the allocation-free entry point (the library's
    own device scratch; no workspace). Same arguments and result."""
    _tensors(q=q, k=k, scales=scales, weights=weights, starts=starts, ends=ends)
    if q.dim() != 3 or k.dim() != 2:
        raise ValueError("q must be [rows,32,128] and k [keys,128]")
    rows, keys = q.shape[0], k.shape[0]
    _shape(q, (rows, HEADS, HEAD_DIM), "q")
    _shape(k, (keys, HEAD_DIM), "k")
    _shape(scales, (keys,), "scales")
    _shape(weights, (rows, HEADS), "weights")
    _shape(starts, (rows,), "starts")
    _shape(ends, (rows,), "ends")
    if out is not None:
        _tensors(out=out)
        _shape(out, (rows, topk), "out")
    dev = q.device
    _need(q, "q", FP8, dev)
    _need(k, "k", FP8, dev)
    _need(scales, "scales", (torch.float32,), dev)
    _need(weights, "weights", (torch.float32,), dev)
    _need(starts, "starts", (torch.int32,), dev)
    _need(ends, "ends", (torch.int32,), dev)
    if out is None:
        out = torch.empty((rows, topk), dtype=torch.int32, device=dev)
    _need(out, "out", (torch.int32,), dev)
    with torch.cuda.device(dev):
        rc = load().mqa_topk_prefill_static(_ptr(q), _ptr(k), _ptr(scales), _ptr(weights),
                                            _ptr(starts), _ptr(ends), _ptr(out), rows, keys,
                                            int(topk), int(flags), _stream(dev, stream))
    _check(rc, "mqa_topk_prefill_static")
    return out


PAGE_ENTRY = HEAD_DIM + 4  # bytes per token in the paged indexer cache


def mqa_topk_prefill_paged(q, cache, block_table, page_size: int, keys: int, weights, starts,
                           ends, topk: int, out=None, workspace=None, flags: int = 0,
                           stream=None) -> torch.Tensor:
    """mqa_topk_prefill reading the keys from the paged indexer cache: cache
    [num_pages, page_size * 132] uint8 (per page: the e4m3 key rows, then the
    four UE8M0 bytes of each key), block_table [>= ceil(keys / page_size)]
    int32 (page of each run of page_size keys). Same result as
    mqa_topk_prefill on the gathered keys and decoded scales."""
    _tensors(q=q, cache=cache, block_table=block_table, weights=weights, starts=starts,
             ends=ends)
    if q.dim() != 3:
        raise ValueError("q must be [rows,32,128]")
    rows = q.shape[0]
    page_size, keys = int(page_size), int(keys)
    if page_size < 4 or page_size & (page_size - 1):
        raise ValueError("page_size must be a power of two >= 4")
    if keys < 1 or keys > MAX_KEYS:
        raise ValueError(f"keys must be in [1, {MAX_KEYS}]")
    if cache.dim() != 2:
        raise ValueError("cache must be [num_pages, page_size * 132]")
    num_pages = cache.shape[0]
    _shape(cache, (num_pages, page_size * PAGE_ENTRY), "cache")
    if block_table.dim() != 1 or block_table.shape[0] < -(-keys // page_size):
        raise ValueError(f"block_table must be 1-D with >= {-(-keys // page_size)} entries")
    _shape(q, (rows, HEADS, HEAD_DIM), "q")
    _shape(weights, (rows, HEADS), "weights")
    _shape(starts, (rows,), "starts")
    _shape(ends, (rows,), "ends")
    if out is not None:
        _tensors(out=out)
        _shape(out, (rows, topk), "out")
    dev = q.device
    _need(q, "q", FP8, dev)
    _need(cache, "cache", (torch.uint8,), dev)
    _need(block_table, "block_table", (torch.int32,), dev)
    _need(weights, "weights", (torch.float32,), dev)
    _need(starts, "starts", (torch.int32,), dev)
    _need(ends, "ends", (torch.int32,), dev)
    if out is None:
        out = torch.empty((rows, topk), dtype=torch.int32, device=dev)
    _need(out, "out", (torch.int32,), dev)
    if workspace is None:
        n = workspace_size_paged(rows, keys, dev.index)
        if n == 0:
            raise MQAError(5, "workspace_size_paged")
        workspace = torch.empty(n, dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", (torch.uint8,), dev)
    with torch.cuda.device(dev):
        rc = load().mqa_topk_prefill_paged(_ptr(q), _ptr(cache), _ptr(block_table), page_size,
                                           num_pages, _ptr(weights), _ptr(starts), _ptr(ends),
                                           _ptr(out), rows, keys, int(topk), _ptr(workspace),
                                           workspace.numel(), int(flags), _stream(dev, stream))
    _check(rc, "mqa_topk_prefill_paged")
    return out


def workspace_size_paged(rows: int, keys: int, device: int | None = None) -> int:
    """Bytes of workspace one mqa_topk_prefill_paged call needs."""
    if device is None:
        device = torch.cuda.current_device()
    return int(load().workspace_size_paged(int(rows), int(keys), int(device)))


def workspace_size_decode(requests: int, rows_per_request: int, device: int | None = None) -> int:
    """Bytes of workspace one mqa_topk_decode_paged call needs."""
    if device is None:
        device = torch.cuda.current_device()
    return int(load().workspace_size_decode(int(requests), int(rows_per_request), int(device)))


def mqa_topk_decode_paged(q, cache, page_table, page_size: int, weights, starts, ends, topk: int,
                          rows_per_request: int, out=None, workspace=None, flags: int = 0,
                          stream=None) -> torch.Tensor:
    """Decode-shaped fused scores + top-k over the paged indexer cache: q
    [requests * R, 32, 128] (row r is row r % R of request r // R), page_table
    [requests, table_stride] int32 (request q's position j is slot j % P of
    page page_table[q, j // P]), starts/ends [rows] int32 positions in the row's
    request. Returns out [rows, topk] int32 (position - start, -1 padded)."""
    _tensors(q=q, cache=cache, page_table=page_table, weights=weights, starts=starts, ends=ends)
    if q.dim() != 3:
        raise ValueError("q must be [rows,32,128]")
    rows = q.shape[0]
    R, page_size = int(rows_per_request), int(page_size)
    if R < 1 or R > 32:
        raise ValueError("rows_per_request must be in [1, 32]")
    if page_size < 4 or page_size & (page_size - 1):
        raise ValueError("page_size must be a power of two >= 4")
    if page_table.dim() != 2:
        raise ValueError("page_table must be [requests, table_stride]")
    requests, stride = page_table.shape
    if rows != requests * R:
        raise ValueError(f"q has {rows} rows, expected requests * rows_per_request = {requests * R}")
    if cache.dim() != 2:
        raise ValueError("cache must be [num_pages, page_size * 132]")
    num_pages = cache.shape[0]
    _shape(cache, (num_pages, page_size * PAGE_ENTRY), "cache")
    _shape(q, (rows, HEADS, HEAD_DIM), "q")
    _shape(weights, (rows, HEADS), "weights")
    _shape(starts, (rows,), "starts")
    _shape(ends, (rows,), "ends")
    if out is not None:
        _tensors(out=out)
        _shape(out, (rows, topk), "out")
    dev = q.device
    _need(q, "q", FP8, dev)
    _need(cache, "cache", (torch.uint8,), dev)
    _need(page_table, "page_table", (torch.int32,), dev)
    _need(weights, "weights", (torch.float32,), dev)
    _need(starts, "starts", (torch.int32,), dev)
    _need(ends, "ends", (torch.int32,), dev)
    if out is None:
        out = torch.empty((rows, topk), dtype=torch.int32, device=dev)
    _need(out, "out", (torch.int32,), dev)
    if workspace is None:
        n = workspace_size_decode(requests, R, dev.index)
        if n == 0:
            raise MQAError(5, "workspace_size_decode")
        workspace = torch.empty(n, dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", (torch.uint8,), dev)
    with torch.cuda.device(dev):
        rc = load().mqa_topk_decode_paged(_ptr(q), _ptr(cache), _ptr(page_table), stride,
                                          page_size, num_pages, _ptr(weights), _ptr(starts),
                                          _ptr(ends), _ptr(out), requests, R, int(topk),
                                          _ptr(workspace), workspace.numel(), int(flags),
                                          _stream(dev, stream))
    _check(rc, "mqa_topk_decode_paged")
    return out


def mqa_logits_dense(q, k, scales, weights, starts, ends, col0: int = 0, ncols: int | None = None,
                     logits=None, stream=None) -> torch.Tensor:
    """fp32 logits [rows, ncols] for keys col0 .. col0+ncols-1 (-inf where not visible)."""
    _tensors(q=q, k=k, scales=scales, weights=weights, starts=starts, ends=ends)
    if q.dim() != 3 or k.dim() != 2:
        raise ValueError("q must be [rows,32,128] and k [keys,128]")
    rows, keys = q.shape[0], k.shape[0]
    _shape(q, (rows, HEADS, HEAD_DIM), "q")
    _shape(k, (keys, HEAD_DIM), "k")
    _shape(scales, (keys,), "scales")
    _shape(weights, (rows, HEADS), "weights")
    _shape(starts, (rows,), "starts")
    _shape(ends, (rows,), "ends")
    dev = q.device
    for t, n, d in ((q, "q", FP8), (k, "k", FP8), (scales, "scales", (torch.float32,)),
                    (weights, "weights", (torch.float32,)), (starts, "starts", (torch.int32,)),
                    (ends, "ends", (torch.int32,))):
        _need(t, n, d, dev)
    if ncols is None:
        ncols = keys - col0
    if logits is None:
        ld = (ncols + 3) // 4 * 4
        logits = torch.empty((rows, ld), dtype=torch.float32, device=dev)[:, :ncols]
    if not isinstance(logits, torch.Tensor) or logits.device != dev:
        raise ValueError(f"logits must be a tensor on {dev}")
    ld = logits.stride(0)
    if logits.dtype != torch.float32 or logits.stride(1) != 1:
        raise ValueError("logits must be fp32 with unit column stride")
    _shape(logits, (rows, ncols), "logits")
    with torch.cuda.device(dev):
        rc = load().mqa_logits_dense(_ptr(q), _ptr(k), _ptr(scales), _ptr(weights), _ptr(starts),
                                     _ptr(ends), _ptr(logits), ld, rows, keys, int(col0),
                                     int(ncols), _stream(dev, stream))
    _check(rc, "mqa_logits_dense")
    return logits


def mqa_topk_dense(logits, starts, ends, topk: int, keys: int, col0: int = 0, out=None,
                   stream=None) -> torch.Tensor:
    """Per-row top-k of a logits window [rows, ncols] (columns = keys col0 ..)."""
    _tensors(logits=logits, starts=starts, ends=ends)
    if logits.dtype != torch.float32 or logits.dim() != 2 or logits.stride(1) != 1:
        raise ValueError("logits must be 2-D fp32 with unit column stride")
    rows, ncols = logits.shape
    _shape(starts, (rows,), "starts")
    _shape(ends, (rows,), "ends")
    if out is not None:
        _tensors(out=out)
        _shape(out, (rows, topk), "out")
    dev = logits.device
    _need(starts, "starts", (torch.int32,), dev)
    _need(ends, "ends", (torch.int32,), dev)
    if out is None:
        out = torch.empty((rows, topk), dtype=torch.int32, device=dev)
    _need(out, "out", (torch.int32,), dev)
    with torch.cuda.device(dev):
        rc = load().mqa_topk_dense(_ptr(logits), logits.stride(0), int(col0), int(ncols),
                                   _ptr(starts), _ptr(ends), _ptr(out), rows, int(keys),
                                   int(topk), _stream(dev, stream))
    _check(rc, "mqa_topk_dense")
    return out


def mqa_key_scales(scale_bytes, out=None, stream=None) -> torch.Tensor:
    """UE8M0 [keys,4] uint8 -> fp32 [keys] (bit pattern e << 23), on the GPU."""
    _tensors(scale_bytes=scale_bytes)
    if scale_bytes.dim() != 2:
        raise ValueError("scale_bytes must be [keys,4] uint8")
    keys = scale_bytes.shape[0]
    _shape(scale_bytes, (keys, 4), "scale_bytes")
    if out is not None:
        _tensors(out=out)
        _shape(out, (keys,), "out")
    dev = scale_bytes.device
    _need(scale_bytes, "scale_bytes", (torch.uint8,), dev)
    if out is None:
        out = torch.empty(keys, dtype=torch.float32, device=dev)
    _need(out, "out", (torch.float32,), dev)
    with torch.cuda.device(dev):
        rc = load().mqa_key_scales(_ptr(scale_bytes), _ptr(out), keys, _stream(dev, stream))
    _check(rc, "mqa_key_scales")
    return out


def scan_time_ms(last_n: int) -> float:
    """Total scan-kernel time (ms) of the last `last_n` calls made with
    FLAG_TIME_SCAN on the current device (waits for them to finish)."""
    v = ctypes.c_float(0.0)
    _check(load().mqa_scan_time(int(last_n), ctypes.byref(v)), "mqa_scan_time")
    return float(v.value)


def mfma_peak_tflops(workgroups: int = 2048, iters: int = 4096, repeats: int = 3) -> float:
    """FP8 MFMA rate (TFLOP/s) this GPU sustains on the scan's head-tile
    instruction: the best of `repeats` timed launches of the mqa_mfma_peak
    probe (after one untimed launch), timed with events on the current stream."""
    dev = torch.device("cuda", torch.cuda.current_device())
    out = torch.empty(workgroups * 512, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    lib = load()

    def launch():
        _check(lib.mqa_mfma_peak(_ptr(out), out.numel(), workgroups, iters, stream.cuda_stream),
               "mqa_mfma_peak")

    launch()
    best = 0.0
    for _ in range(repeats):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        launch()
        e1.record(stream)
        e1.synchronize()
        flop = workgroups * 8.0 * iters * 8 * 65536
        best = max(best, flop / (e0.elapsed_time(e1) / 1e3) / 1e12)
    if not torch.isfinite(out).all():
        raise RuntimeError("mqa_mfma_peak: non-finite probe sums")
    return best


def fp8_mfma_probe(a: torch.Tensor, b: torch.Tensor, ascale: torch.Tensor | None = None,
                   stream=None) -> torch.Tensor:
    """The FP8 MFMA's dot products of a [n,16,128] and b [n,16,128] e4m3 codes
    (uint8), out [n,16,16] fp32, with the A-scaled form when ascale [n,16,4]
    (E8M0 bytes per row and K block) is given."""
    _tensors(a=a, b=b)
    if a.dim() != 3:
        raise ValueError("a must be [n,16,128]")
    n = a.shape[0]
    _shape(a, (n, 16, HEAD_DIM), "a")
    _shape(b, (n, 16, HEAD_DIM), "b")
    if ascale is not None:
        _tensors(ascale=ascale)
        _shape(ascale, (n, 16, 4), "ascale")
    dev = a.device
    _need(a, "a", FP8, dev)
    _need(b, "b", FP8, dev)
    if ascale is not None:
        _need(ascale, "ascale", (torch.uint8,), dev)
    out = torch.empty((n, 16, 16), dtype=torch.float32, device=dev)
    with torch.cuda.device(dev):
        rc = load().mqa_fp8_mfma_probe(_ptr(a), _ptr(b), _ptr(ascale), _ptr(out), n,
                                       _stream(dev, stream))
    _check(rc, "mqa_fp8_mfma_probe")
    return out


def read_stats(workspace: torch.Tensor) -> dict:
    """The mqa_stats header of a workspace used with FLAG_STATS (synchronizes)."""
    h = workspace[:256].cpu().numpy().view("<u4")
    return {"rows_short": int(h[1]), "rows_gated": int(h[2]), "rows_exact": int(h[3]),
            "rows_rescanned": int(h[4]), "rows_undercount": int(h[5]),
            "compactions": int(h[6]), "rows_uncertified": int(h[7]),
            "candidates": int(h[8]) | (int(h[9]) << 32),
            "band_keys": int(h[10]) | (int(h[11]) << 32),
            "bound_ratio_max": float(h[12:13].view("<f4")[0]),
            # rows the select could not certify, by reason (counts, window
            # too far off, taken / dropped record reaching the k-th score,
            # admission bound reaching it)
            "fail_reasons": [int(h[26]), int(h[27]), int(h[28]), int(h[29])],
            # two-level source calls: rows the exact block scan served
            "rows_block_scan": int(h[32])}
