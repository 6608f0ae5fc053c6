// C ABI of libmqa_topk.so: argument checks, workspace layout and launches.
// The declarations and their contracts are in include/mqa_topk.h.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>
#include <mutex>

#include "launch.h"
#include "mqa_topk.h"

namespace {

constexpr size_t kAlign = 256;
constexpr int kHeaderWords = 64;

thread_local char g_err[256] = "";

size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct DeviceInfo {
  bool probed = false;
  bool ok = false;
  int cus = 0;
  int wg_per_cu = 0;
};

std::mutex g_mu;
DeviceInfo g_dev[64];

// Compute-unit count and persistent-grid occupancy of a gfx950 device.
const DeviceInfo* device_info(int device) {
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || device < 0 || device >= ndev || device >= 64) {
    (void)hipGetLastError();
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceInfo& d = g_dev[device];
  if (!d.probed) {
    d.probed = true;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) == hipSuccess &&
        std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) {
      int cur = 0;
      (void)hipGetDevice(&cur);
      (void)hipSetDevice(device);
      int occ = 0;
      if (mqa_fused_occupancy(&occ) == 0 && occ > 0) {
        d.ok = true;
        d.cus = prop.multiProcessorCount;
        d.wg_per_cu = occ;
      }
      (void)hipSetDevice(cur);
    }
    (void)hipGetLastError();
  }
  return d.ok ? &d : nullptr;
}

struct Layout {
  size_t header, order, xrow, xqueue, xflag, fqueue, fflag, rinfo, rqueue, rowinfo, seg, keyinfo,
      beta, slabE, slabI, tmpE, tmpI, kc, bqueue, total;
  int grid, nblocks;
};

// The kernels address a wave's score and key slab rows through one raw
// buffer whose byte range (the distance between the two slab arrays plus four
// rows) must stay below 2^31: a batch of kMaxBatchRows rows uses 1.09 GB.
static_assert((size_t)mqa::kMaxBatchRows * mqa::kSlabRow * 4 + 4 * mqa::kSlabRow * 4 + kAlign <
                  ((size_t)1 << 31),
              "slab range");

// Workspace of one batch of `nblocks` blocks of 32 row slots (at most
// kMaxBatchRows slots), plus room for kc_keys compacted keys (paged prefill).
Layout layout_blocks(int nblocks, const DeviceInfo& d, int kc_keys = 0) {
  Layout L{};
  L.grid = d.cus * d.wg_per_cu;
  L.nblocks = nblocks;
  const size_t rows_pad = (size_t)L.nblocks * mqa::kFusedBlockRows;
  size_t off = 0;
  L.header = off;
  off = align_up(off + kHeaderWords * 4);
  L.order = off;
  off = align_up(off + (size_t)L.nblocks * 4);
  L.xrow = off;
  off = align_up(off + rows_pad);
  L.xqueue = off;
  off = align_up(off + (size_t)L.nblocks * 4);
  L.xflag = off;
  off = align_up(off + (size_t)L.nblocks * 4);
  L.fqueue = off;
  off = align_up(off + (size_t)L.nblocks * 4);
  L.fflag = off;
  off = align_up(off + (size_t)L.nblocks * 4);
  L.rinfo = off;
  off = align_up(off + rows_pad * sizeof(mqa::RefineInfo));
  L.rqueue = off;
  off = align_up(off + 3 * rows_pad * 4);
  L.rowinfo = off;
  off = align_up(off + rows_pad * sizeof(mqa::RowInfo));
  L.seg = off;
  off = align_up(off + rows_pad * mqa::kMaxSeg * sizeof(mqa::SegInfo));
  L.keyinfo = off;  // per key, for the largest key count a call may have
  off = align_up(off + (size_t)MQA_MAX_KEYS * 8);
  L.beta = off;
  off = align_up(off + rows_pad * 4);
  const size_t slab = rows_pad * mqa::kSlabRow * 4;
  L.slabE = off;
  off = align_up(off + slab);
  L.slabI = off;
  off = align_up(off + slab);
  const size_t tmp = (size_t)L.grid * mqa::kFusedWaves * mqa::kTmp * 4;
  L.tmpE = off;
  off = align_up(off + tmp);
  L.tmpI = off;
  off = align_up(off + tmp);
  L.kc = off;
  off = align_up(off + (size_t)kc_keys * MQA_HEAD_DIM);
  L.bqueue = off;
  off = align_up(off + rows_pad * 4);
  L.total = off;
  return L;
}

// Workspace of one batch of `rows` rows (rows <= kMaxBatchRows).
Layout layout(int rows, const DeviceInfo& d, int kc_keys = 0) {
  return layout_blocks((rows + mqa::kFusedBlockRows - 1) / mqa::kFusedBlockRows, d, kc_keys);
}

// Decode layout: a request's rows in parts of up to 8 rows, four parts to a
// block; a batch holds at most kMaxBatchRows rows and kMaxBatchRows / 32
// blocks.
constexpr int kDecPack = 4;
int dec_parts(int rows_per_request) { return (rows_per_request + 7) / 8; }
int dec_blocks(int requests, int rows_per_request) {
  return (requests * dec_parts(rows_per_request) + kDecPack - 1) / kDecPack;
}
int dec_batch(int requests, int rows_per_request) {
  int b = mqa::kMaxBatchRows / rows_per_request;
  const int by_blocks = mqa::kMaxBatchRows / mqa::kFusedBlockRows * kDecPack /
                        dec_parts(rows_per_request);
  b = b < by_blocks ? b : by_blocks;
  return requests < b ? requests : b;
}

int batch_rows(int rows) { return rows < mqa::kMaxBatchRows ? rows : mqa::kMaxBatchRows; }

// Key segments per block (FusedParams.nseg): a power of two that gives about
// two work items per persistent workgroup when blocks are fewer, bounded so
// that a segment's part of a slab row (kSlabRow / nseg records) holds a merge
// of 2 * topk records plus two chunks.
int key_segments(int nblocks, int grid, int topk) {
  int s = 1;
  while (s < mqa::kMaxSeg && (size_t)nblocks * s < (size_t)2 * grid &&
         mqa::kSlabRow / (2 * s) >= 2 * topk + 128)
    s *= 2;
  return s;
}

int launch_error(int hip_code) {
  std::snprintf(g_err, sizeof(g_err), "HIP launch failed: %s",
                hipGetErrorString(static_cast<hipError_t>(hip_code)));
  return MQA_ERR_LAUNCH;
}

const DeviceInfo* current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  return device_info(dev);
}

bool topk_ok(int topk) { return topk == 512 || topk == 1024 || topk == 2048; }

// Per-device ring of event pairs recorded around the scan kernel by calls made
// with MQA_FLAG_TIME_SCAN (created on first use, kept until the process ends).
constexpr int kRing = 256;
struct TimingRing {
  bool made = false;
  hipEvent_t b[kRing], e[kRing];
  int next = 0, count = 0;
};
TimingRing g_ring[64];

// Event pair for the next timed call on `device`; false if events cannot be made.
bool ring_slot(int device, hipEvent_t* b, hipEvent_t* e) {
  std::lock_guard<std::mutex> lock(g_mu);
  TimingRing& r = g_ring[device];
  if (!r.made) {
    for (int i = 0; i < kRing; ++i) {
      if (hipEventCreate(&r.b[i]) != hipSuccess || hipEventCreate(&r.e[i]) != hipSuccess) {
        (void)hipGetLastError();
        return false;
      }
    }
    r.made = true;
  }
  *b = r.b[r.next];
  *e = r.e[r.next];
  r.next = (r.next + 1) % kRing;
  r.count = r.count < kRing ? r.count + 1 : kRing;
  return true;
}

// Where the keys come from: the dense k / scales arrays (table == nullptr) or
// the paged indexer cache k with its page table.
struct KeySource {
  const int32_t* table = nullptr;
  int page_shift = 0, num_pages = 0;
};

// Workspace pointers and the fields every batch shares.
void set_workspace(mqa::FusedParams& p, uint8_t* ws, const Layout& L) {
  p.header = reinterpret_cast<uint32_t*>(ws + L.header);
  p.order = reinterpret_cast<int32_t*>(ws + L.order);
  p.xrow = ws + L.xrow;
  p.xqueue = reinterpret_cast<int32_t*>(ws + L.xqueue);
  p.xflag = reinterpret_cast<uint32_t*>(ws + L.xflag);
  p.fqueue = reinterpret_cast<int32_t*>(ws + L.fqueue);
  p.fflag = reinterpret_cast<uint32_t*>(ws + L.fflag);
  p.rinfo = reinterpret_cast<mqa::RefineInfo*>(ws + L.rinfo);
  p.rqueue = reinterpret_cast<int32_t*>(ws + L.rqueue);
  p.rowinfo = reinterpret_cast<mqa::RowInfo*>(ws + L.rowinfo);
  p.seg = reinterpret_cast<mqa::SegInfo*>(ws + L.seg);
  p.keyinfo = reinterpret_cast<float*>(ws + L.keyinfo);
  p.beta = reinterpret_cast<float*>(ws + L.beta);
  p.slabE = reinterpret_cast<float*>(ws + L.slabE);
  p.slabI = reinterpret_cast<int32_t*>(ws + L.slabI);
  p.tmpE = reinterpret_cast<float*>(ws + L.tmpE);
  p.tmpI = reinterpret_cast<int32_t*>(ws + L.tmpI);
  p.kc = ws + L.kc;
  p.bqueue = reinterpret_cast<int32_t*>(ws + L.bqueue);
}

// Rows in batches of `batch` rows, one launch sequence each, in order on the
// stream (they share the workspace ws, which holds layout(batch)).
// hm = heads / 32: a batch of `batch` rows runs as batch * hm virtual rows
// (its workspace holds layout(batch * hm)).
int prefill_batches(const uint8_t* q, const uint8_t* k, const float* scales,
                    const float* weights, const int32_t* starts, const int32_t* ends,
                    int32_t* out, int rows, int keys, int topk, uint8_t* ws, int batch,
                    const DeviceInfo& d, unsigned flags, void* stream,
                    const KeySource& src = KeySource(), int hm = 1,
                    int32_t* blocks_out = nullptr) {
  const Layout L = layout(batch * hm, d, src.table ? keys : 0);
  hipEvent_t eb = nullptr, ee = nullptr;
  if (flags & MQA_FLAG_TIME_SCAN) {
    int dev = 0;
    (void)hipGetDevice(&dev);
    if (!ring_slot(dev, &eb, &ee)) return MQA_ERR_DEVICE;
  }
  for (int r0 = 0; r0 < rows; r0 += batch) {
    const int nr = rows - r0 < batch ? rows - r0 : batch;
    mqa::FusedParams p{};
    p.q = q + (size_t)r0 * hm * MQA_HEADS * MQA_HEAD_DIM;
    p.k = k;
    p.scales = scales;
    p.weights = weights + (size_t)r0 * hm * MQA_HEADS;
    p.starts = starts + r0;
    p.ends = ends + r0;
    p.out = out + (size_t)r0 * topk;
    p.rows = nr * hm;
    p.keys = keys;
    p.topk = topk;
    p.nblocks = (nr * hm + mqa::kFusedBlockRows - 1) / mqa::kFusedBlockRows;
    p.hm = hm;
    // a two-level source call gates for at least 2048 keys, so that its
    // candidates cover the 2048 blocks of its second output
    p.blocks_out = blocks_out ? blocks_out + (size_t)r0 * MQA_MAX_BLOCKS : nullptr;
    p.kgate = blocks_out && topk < MQA_MAX_BLOCKS ? MQA_MAX_BLOCKS : topk;
    p.flags = flags;
    set_workspace(p, ws, L);
    p.table = src.table;
    p.page_shift = src.page_shift;
    p.num_pages = src.num_pages;
    p.page_bytes = (int64_t)(MQA_HEAD_DIM + 4) << src.page_shift;
    p.dec_rows = 0;
    p.dec_parts = 1;
    p.nreq = 0;
    p.table_stride = 0;
    const int grid = L.grid < p.nblocks ? L.grid : p.nblocks;
    p.nseg = key_segments(p.nblocks, L.grid, topk);
    p.scan_grid = L.grid < p.nblocks * p.nseg ? L.grid : p.nblocks * p.nseg;
    // timing events: from the first batch's scan to the end of the last one
    const int rc = mqa_fused_launch(&p, grid, static_cast<hipStream_t>(stream),
                                    r0 == 0 ? eb : nullptr, r0 + nr >= rows ? ee : nullptr);
    if (rc != 0) return launch_error(rc);
  }
  return MQA_OK;
}

// Decode-shaped calls: batches of whole requests, one launch sequence each.
int decode_batches(const uint8_t* q, const uint8_t* cache, const int32_t* table,
                   int table_stride, int shift, int num_pages, const float* weights,
                   const int32_t* starts, const int32_t* ends, int32_t* out, int requests, int R,
                   int topk, uint8_t* ws, const DeviceInfo& d, unsigned flags, void* stream) {
  const int nb = dec_batch(requests, R);
  const Layout L = layout_blocks(dec_blocks(nb, R), d);
  const int64_t span = (int64_t)table_stride << shift;
  const int keys = span < MQA_MAX_KEYS ? (int)span : MQA_MAX_KEYS;
  hipEvent_t eb = nullptr, ee = nullptr;
  if (flags & MQA_FLAG_TIME_SCAN) {
    int dev = 0;
    (void)hipGetDevice(&dev);
    if (!ring_slot(dev, &eb, &ee)) return MQA_ERR_DEVICE;
  }
  for (int q0 = 0; q0 < requests; q0 += nb) {
    const int nq = requests - q0 < nb ? requests - q0 : nb;
    const int64_t r0 = (int64_t)q0 * R;
    mqa::FusedParams p{};
    p.q = q + r0 * MQA_HEADS * MQA_HEAD_DIM;
    p.k = cache;
    p.scales = nullptr;
    p.weights = weights + r0 * MQA_HEADS;
    p.starts = starts + r0;
    p.ends = ends + r0;
    p.out = out + r0 * topk;
    p.rows = nq * R;
    p.keys = keys;
    p.topk = topk;
    p.nblocks = dec_blocks(nq, R);
    p.flags = flags;
    set_workspace(p, ws, L);
    p.table = table + (int64_t)q0 * table_stride;
    p.page_shift = shift;
    p.num_pages = num_pages;
    p.page_bytes = (int64_t)(MQA_HEAD_DIM + 4) << shift;
    p.dec_rows = R;
    p.hm = 1;
    p.kgate = topk;
    p.blocks_out = nullptr;
    p.dec_parts = dec_parts(R);
    p.nreq = nq;
    p.table_stride = table_stride;
    const int grid = L.grid < p.nblocks ? L.grid : p.nblocks;
    p.nseg = key_segments(p.nblocks, L.grid, topk);
    p.scan_grid = L.grid < p.nblocks * p.nseg ? L.grid : p.nblocks * p.nseg;
    const int rc = mqa_fused_launch(&p, grid, static_cast<hipStream_t>(stream),
                                    q0 == 0 ? eb : nullptr, q0 + nq >= requests ? ee : nullptr);
    if (rc != 0) return launch_error(rc);
  }
  return MQA_OK;
}

int launch_error_text(const char* what) {
  std::snprintf(g_err, sizeof(g_err), "%s", what);
  return MQA_ERR_LAUNCH;
}

thread_local char g_ws_err[160] = "";

int workspace_error_text(const char* what) {
  std::snprintf(g_ws_err, sizeof(g_ws_err), "%s", what);
  return MQA_ERR_WORKSPACE;
}

}  // namespace

// The scratch of mqa_topk_prefill_static, for callers that cannot allocate:
// the workspace of one row batch, in device memory the library owns (each
// device the library runs on holds its own copy until the process ends).
// Host code never uses this name as an address: the device address of each
// device's copy comes from hipGetSymbolAddress (static_scratch).
constexpr size_t kStaticScratchBytes = (size_t)384 << 20;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {

void* g_scratch_ptr[64];
bool g_scratch_tried[64];

// Device address of `device`'s copy of the scratch (the device is current),
// looked up on its first use; nullptr if the lookup failed.
uint8_t* static_scratch(int device) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch_tried[device]) {
    g_scratch_tried[device] = true;
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) == hipSuccess && ptr &&
        reinterpret_cast<uintptr_t>(ptr) % kAlign == 0)
      g_scratch_ptr[device] = ptr;
    (void)hipGetLastError();
  }
  return static_cast<uint8_t*>(g_scratch_ptr[device]);
}

// Rows per batch of the static entry point: the largest multiple of 32 (at
// most one full batch) whose workspace fits the scratch; 0 if none does.
int static_batch(const DeviceInfo& d) {
  int b = mqa::kMaxBatchRows;
  while (b >= mqa::kFusedBlockRows && layout(b, d).total > kStaticScratchBytes)
    b -= mqa::kFusedBlockRows;
  return b >= mqa::kFusedBlockRows ? b : 0;
}

}  // namespace

extern "C" {

size_t workspace_size(int rows, int device) {
  if (rows < 1 || rows > MQA_MAX_ROWS) return 0;
  const DeviceInfo* d = device_info(device);
  if (!d) return 0;
  return layout(batch_rows(rows), *d).total;
}

int mqa_topk_prefill(const uint8_t* q, const uint8_t* k, const float* scales,
                     const float* weights, const int32_t* starts, const int32_t* ends,
                     int32_t* out, int rows, int keys, int topk, void* workspace,
                     size_t workspace_bytes, unsigned flags, void* stream) {
  if (!q || !k || !scales || !weights || !starts || !ends || !out || !workspace)
    return MQA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(scales, 16) || !aligned(weights, 16) ||
      !aligned(out, 16) || !aligned(starts, 4) || !aligned(ends, 4) || !aligned(workspace, 256))
    return MQA_ERR_ALIGN;
  if (rows < 1 || rows > MQA_MAX_ROWS || keys < 1 || keys > MQA_MAX_KEYS || !topk_ok(topk))
    return MQA_ERR_SHAPE;
  const DeviceInfo* d = current_device();
  if (!d) return MQA_ERR_DEVICE;
  const int batch = batch_rows(rows);
  if (workspace_bytes < layout(batch, *d).total) {
    g_ws_err[0] = 0;
    return MQA_ERR_WORKSPACE;
  }
  return prefill_batches(q, k, scales, weights, starts, ends, out, rows, keys, topk,
                         static_cast<uint8_t*>(workspace), batch, *d, flags, stream);
}

int mqa_topk_prefill_static(const uint8_t* q, const uint8_t* k, const float* scales,
                            const float* weights, const int32_t* starts, const int32_t* ends,
                            int32_t* out, int rows, int keys, int topk, unsigned flags,
                            void* stream) {
  if (!q || !k || !scales || !weights || !starts || !ends || !out) return MQA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(scales, 16) || !aligned(weights, 16) ||
      !aligned(out, 16) || !aligned(starts, 4) || !aligned(ends, 4))
    return MQA_ERR_ALIGN;
  if (rows < 1 || rows > MQA_MAX_ROWS || keys < 1 || keys > MQA_MAX_KEYS || !topk_ok(topk))
    return MQA_ERR_SHAPE;
  const DeviceInfo* d = current_device();
  if (!d) return MQA_ERR_DEVICE;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return MQA_ERR_DEVICE;
  }
  uint8_t* ws = static_scratch(dev);
  if (!ws) return launch_error_text("hipGetSymbolAddress of the static scratch failed");
  const int batch = static_batch(*d);
  if (batch < 1)
    return workspace_error_text("the static scratch cannot hold one 32-row batch on this device");
  return prefill_batches(q, k, scales, weights, starts, ends, out, rows, keys, topk, ws, batch,
                         *d, flags, stream);
}

int mqa_topk_prefill_paged(const uint8_t* q, const uint8_t* cache, const int32_t* block_table,
                           int page_size, int num_pages, const float* weights,
                           const int32_t* starts, const int32_t* ends, int32_t* out, int rows,
                           int keys, int topk, void* workspace, size_t workspace_bytes,
                           unsigned flags, void* stream) {
  if (!q || !cache || !block_table || !weights || !starts || !ends || !out || !workspace)
    return MQA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(cache, 16) || !aligned(block_table, 4) ||
      !aligned(weights, 16) || !aligned(out, 16) || !aligned(starts, 4) || !aligned(ends, 4) ||
      !aligned(workspace, 256))
    return MQA_ERR_ALIGN;
  int shift = 0;
  while (shift < 20 && (1 << shift) < page_size) ++shift;
  if (rows < 1 || rows > MQA_MAX_ROWS || keys < 1 || keys > MQA_MAX_KEYS || !topk_ok(topk) ||
      page_size < 4 || page_size > MQA_MAX_KEYS || (1 << shift) != page_size || num_pages < 1)
    return MQA_ERR_SHAPE;
  const DeviceInfo* d = current_device();
  if (!d) return MQA_ERR_DEVICE;
  const int batch = batch_rows(rows);
  if (workspace_bytes < layout(batch, *d, keys).total) {
    g_ws_err[0] = 0;
    return MQA_ERR_WORKSPACE;
  }
  KeySource src;
  src.table = block_table;
  src.page_shift = shift;
  src.num_pages = num_pages;
  return prefill_batches(q, cache, nullptr, weights, starts, ends, out, rows, keys, topk,
                         static_cast<uint8_t*>(workspace), batch, *d, flags, stream, src);
}

int mqa_topk_prefill_blocks(const uint8_t* q, const uint8_t* k, const float* scales,
                            const float* weights, const int32_t* starts, const int32_t* ends,
                            int32_t* out, int32_t* out_blocks, int rows, int keys, int topk,
                            void* workspace, size_t workspace_bytes, unsigned flags,
                            void* stream) {
  if (!q || !k || !scales || !weights || !starts || !ends || !out || !out_blocks || !workspace)
    return MQA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(scales, 16) || !aligned(weights, 16) ||
      !aligned(out, 16) || !aligned(out_blocks, 16) || !aligned(starts, 4) || !aligned(ends, 4) ||
      !aligned(workspace, 256))
    return MQA_ERR_ALIGN;
  if (rows < 1 || rows > MQA_MAX_ROWS || keys < 1 || keys > MQA_MAX_KEYS || !topk_ok(topk))
    return MQA_ERR_SHAPE;
  const DeviceInfo* d = current_device();
  if (!d) return MQA_ERR_DEVICE;
  const int batch = batch_rows(rows);
  if (workspace_bytes < layout(batch, *d).total) {
    g_ws_err[0] = 0;
    return MQA_ERR_WORKSPACE;
  }
  return prefill_batches(q, k, scales, weights, starts, ends, out, rows, keys, topk,
                         static_cast<uint8_t*>(workspace), batch, *d, flags, stream, KeySource(),
                         1, out_blocks);
}

int mqa_topk_masked(const uint8_t* q, const uint8_t* k, const float* scales, const float* weights,
                    const int32_t* starts, const int32_t* ends, const int32_t* blocks, int nb,
                    int32_t* out, int rows, int keys, int topk, void* workspace,
                    size_t workspace_bytes, unsigned flags, void* stream) {
  if (!q || !k || !scales || !weights || !starts || !ends || !blocks || !out || !workspace)
    return MQA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(scales, 16) || !aligned(weights, 16) ||
      !aligned(out, 16) || !aligned(starts, 4) || !aligned(ends, 4) || !aligned(blocks, 4) ||
      !aligned(workspace, 256))
    return MQA_ERR_ALIGN;
  if (rows < 1 || rows > MQA_MAX_ROWS || keys < 1 || keys > MQA_MAX_KEYS || !topk_ok(topk) ||
      nb < 1 || nb > MQA_MAX_BLOCKS)
    return MQA_ERR_SHAPE;
  const DeviceInfo* d = current_device();
  if (!d) return MQA_ERR_DEVICE;
  const int batch = batch_rows(rows);
  const Layout L = layout(batch, *d);
  if (workspace_bytes < L.total) {
    g_ws_err[0] = 0;
    return MQA_ERR_WORKSPACE;
  }
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  for (int r0 = 0; r0 < rows; r0 += batch) {
    const int nr = rows - r0 < batch ? rows - r0 : batch;
    mqa::FusedParams p{};
    p.q = q + (size_t)r0 * MQA_HEADS * MQA_HEAD_DIM;
    p.k = k;
    p.scales = scales;
    p.weights = weights + (size_t)r0 * MQA_HEADS;
    p.starts = starts + r0;
    p.ends = ends + r0;
    p.out = out + (size_t)r0 * topk;
    p.rows = nr;
    p.keys = keys;
    p.topk = topk;
    p.flags = flags;
    p.hm = 1;
    p.kgate = topk;
    set_workspace(p, ws, L);
    const int rc = mqa_masked_launch(&p, blocks + (size_t)r0 * nb, nb,
                                     static_cast<hipStream_t>(stream));
    if (rc != 0) return launch_error(rc);
  }
  return MQA_OK;
}

size_t workspace_size_heads(int rows, int heads, int device) {
  if (rows < 1 || rows > MQA_MAX_ROWS || (heads != 32 && heads != 64)) return 0;
  const DeviceInfo* d = device_info(device);
  if (!d) return 0;
  const int hm = heads / 32;
  const int batch = rows < mqa::kMaxBatchRows / hm ? rows : mqa::kMaxBatchRows / hm;
  return layout(batch * hm, *d).total;
}

int mqa_topk_prefill_heads(const uint8_t* q, const uint8_t* k, const float* scales,
                           const float* weights, const int32_t* starts, const int32_t* ends,
                           int32_t* out, int rows, int keys, int heads, int topk,
                           void* workspace, size_t workspace_bytes, unsigned flags,
                           void* stream) {
  if (!q || !k || !scales || !weights || !starts || !ends || !out || !workspace)
    return MQA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(scales, 16) || !aligned(weights, 16) ||
      !aligned(out, 16) || !aligned(starts, 4) || !aligned(ends, 4) || !aligned(workspace, 256))
    return MQA_ERR_ALIGN;
  if (rows < 1 || rows > MQA_MAX_ROWS || keys < 1 || keys > MQA_MAX_KEYS || !topk_ok(topk) ||
      (heads != 32 && heads != 64))
    return MQA_ERR_SHAPE;
  const DeviceInfo* d = current_device();
  if (!d) return MQA_ERR_DEVICE;
  const int hm = heads / 32;
  const int batch = rows < mqa::kMaxBatchRows / hm ? rows : mqa::kMaxBatchRows / hm;
  if (workspace_bytes < layout(batch * hm, *d).total) {
    g_ws_err[0] = 0;
    return MQA_ERR_WORKSPACE;
  }
  return prefill_batches(q, k, scales, weights, starts, ends, out, rows, keys, topk,
                         static_cast<uint8_t*>(workspace), batch, *d, flags, stream,
                         KeySource(), hm);
}

size_t workspace_size_paged(int rows, int keys, int device) {
  if (rows < 1 || rows > MQA_MAX_ROWS || keys < 1 || keys > MQA_MAX_KEYS) return 0;
  const DeviceInfo* d = device_info(device);
  if (!d) return 0;
  return layout(batch_rows(rows), *d, keys).total;
}

size_t workspace_size_decode(int requests, int rows_per_request, int device) {
  if (requests < 1 || rows_per_request < 1 || rows_per_request > 32 ||
      (int64_t)requests * rows_per_request > MQA_MAX_ROWS)
    return 0;
  const DeviceInfo* d = device_info(device);
  if (!d) return 0;
  return layout_blocks(dec_blocks(dec_batch(requests, rows_per_request), rows_per_request), *d)
      .total;
}

int mqa_topk_decode_paged(const uint8_t* q, const uint8_t* cache, const int32_t* page_table,
                          int table_stride, int page_size, int num_pages, const float* weights,
                          const int32_t* starts, const int32_t* ends, int32_t* out, int requests,
                          int rows_per_request, int topk, void* workspace, size_t workspace_bytes,
                          unsigned flags, void* stream) {
  if (!q || !cache || !page_table || !weights || !starts || !ends || !out || !workspace)
    return MQA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(cache, 16) || !aligned(page_table, 4) ||
      !aligned(weights, 16) || !aligned(out, 16) || !aligned(starts, 4) || !aligned(ends, 4) ||
      !aligned(workspace, 256))
    return MQA_ERR_ALIGN;
  int shift = 0;
  while (shift < 20 && (1 << shift) < page_size) ++shift;
  if (requests < 1 || rows_per_request < 1 || rows_per_request > 32 ||
      (int64_t)requests * rows_per_request > MQA_MAX_ROWS || !topk_ok(topk) ||
      page_size < 4 || page_size > MQA_MAX_KEYS || (1 << shift) != page_size || num_pages < 1 ||
      table_stride < 1)
    return MQA_ERR_SHAPE;
  const DeviceInfo* d = current_device();
  if (!d) return MQA_ERR_DEVICE;
  const int nb = dec_batch(requests, rows_per_request);
  if (workspace_bytes < layout_blocks(dec_blocks(nb, rows_per_request), *d).total) {
    g_ws_err[0] = 0;
    return MQA_ERR_WORKSPACE;
  }
  return decode_batches(q, cache, page_table, table_stride, shift, num_pages, weights, starts,
                        ends, out, requests, rows_per_request, topk,
                        static_cast<uint8_t*>(workspace), *d, flags, stream);
}

int mqa_logits_dense(const uint8_t* q, const uint8_t* k, const float* scales,
                     const float* weights, const int32_t* starts, const int32_t* ends,
                     float* logits, int64_t ld, int rows, int keys, int col0, int ncols,
                     void* stream) {
  if (!q || !k || !scales || !weights || !starts || !ends || !logits) return MQA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(scales, 16) || !aligned(weights, 16) ||
      !aligned(logits, 16) || !aligned(starts, 4) || !aligned(ends, 4))
    return MQA_ERR_ALIGN;
  if (rows < 1 || rows > MQA_MAX_ROWS || keys < 1 || keys > MQA_MAX_KEYS || col0 < 0 ||
      ncols < 1 || (int64_t)col0 + ncols > keys || ld < ncols || ld % 4 != 0)
    return MQA_ERR_SHAPE;
  if (!current_device()) return MQA_ERR_DEVICE;
  mqa::DenseParams p{q, k, scales, weights, starts, ends, logits, ld, rows, keys, col0, ncols};
  const int rc = mqa_dense_logits_launch(&p, static_cast<hipStream_t>(stream));
  if (rc != 0) return launch_error(rc);
  return MQA_OK;
}

int mqa_topk_dense(const float* logits, int64_t ld, int col0, int ncols, const int32_t* starts,
                   const int32_t* ends, int32_t* out, int rows, int keys, int topk,
                   void* stream) {
  if (!logits || !starts || !ends || !out) return MQA_ERR_NULL;
  if (!aligned(logits, 16) || !aligned(out, 16) || !aligned(starts, 4) || !aligned(ends, 4))
    return MQA_ERR_ALIGN;
  if (rows < 1 || rows > MQA_MAX_ROWS || keys < 1 || keys > MQA_MAX_KEYS || col0 < 0 ||
      ncols < 1 || (int64_t)col0 + ncols > keys || ld < ncols || ld % 4 != 0 || !topk_ok(topk))
    return MQA_ERR_SHAPE;
  if (!current_device()) return MQA_ERR_DEVICE;
  mqa::DenseTopkParams p{logits, ld, col0, ncols, starts, ends, out, rows, keys, topk};
  const int rc = mqa_dense_topk_launch(&p, static_cast<hipStream_t>(stream));
  if (rc != 0) return launch_error(rc);
  return MQA_OK;
}

int mqa_key_scales(const uint8_t* scale_bytes, float* scales, int keys, void* stream) {
  if (!scale_bytes || !scales) return MQA_ERR_NULL;
  if (!aligned(scale_bytes, 4) || !aligned(scales, 4)) return MQA_ERR_ALIGN;
  if (keys < 1 || keys > MQA_MAX_KEYS) return MQA_ERR_SHAPE;
  if (!current_device()) return MQA_ERR_DEVICE;
  const int rc = mqa_key_scales_launch(scale_bytes, scales, keys, static_cast<hipStream_t>(stream));
  if (rc != 0) return launch_error(rc);
  return MQA_OK;
}

// The probe's launcher (probe.hip).
extern "C" int mqa_mfma_peak_launch(float* out, int workgroups, int iters, hipStream_t stream);

int mqa_mfma_peak(float* out, int64_t out_len, int workgroups, int iters, void* stream) {
  if (!out) return MQA_ERR_NULL;
  if (!aligned(out, 4)) return MQA_ERR_ALIGN;
  if (workgroups < 1 || workgroups > 65536 || iters < 1 || iters > (1 << 20) ||
      out_len < (int64_t)workgroups * 512)
    return MQA_ERR_SHAPE;
  if (!current_device()) return MQA_ERR_DEVICE;
  const int rc = mqa_mfma_peak_launch(out, workgroups, iters, static_cast<hipStream_t>(stream));
  if (rc != 0) return launch_error(rc);
  return MQA_OK;
}

extern "C" int mqa_fp8_mfma_probe_launch(const uint8_t* a, const uint8_t* b, const uint8_t* sa,
                                         float* out, int ncases, hipStream_t stream);

int mqa_fp8_mfma_probe(const uint8_t* a, const uint8_t* b, const uint8_t* ascale, float* out,
                       int ncases, void* stream) {
  if (!a || !b || !out) return MQA_ERR_NULL;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(out, 4)) return MQA_ERR_ALIGN;
  if (ncases < 1 || ncases > (1 << 20)) return MQA_ERR_SHAPE;
  if (!current_device()) return MQA_ERR_DEVICE;
  const int rc = mqa_fp8_mfma_probe_launch(a, b, ascale, out, ncases,
                                           static_cast<hipStream_t>(stream));
  if (rc != 0) return launch_error(rc);
  return MQA_OK;
}

int mqa_scan_time(int last_n, float* total_ms) {
  if (!total_ms) return MQA_ERR_NULL;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return MQA_ERR_DEVICE;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  const TimingRing& r = g_ring[dev];
  if (last_n < 1 || last_n > r.count) return MQA_ERR_SHAPE;
  double sum = 0.0;
  for (int i = 1; i <= last_n; ++i) {
    const int s = (r.next - i + kRing) % kRing;
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(r.e[s]);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.b[s], r.e[s]);
    if (e != hipSuccess) return launch_error((int)e);
    sum += ms;
  }
  *total_ms = (float)sum;
  return MQA_OK;
}

const char* mqa_strerror(int code) {
  switch (code) {
    case MQA_OK: return "ok";
    case MQA_ERR_NULL: return "a required pointer is NULL";
    case MQA_ERR_ALIGN: return "a pointer is not aligned as the contract requires";
    case MQA_ERR_SHAPE: return "a size or shape argument is outside the contract";
    case MQA_ERR_WORKSPACE:
      return g_ws_err[0] ? g_ws_err : "the workspace is smaller than workspace_size(rows, device)";
    case MQA_ERR_DEVICE: return "no current HIP device, or it is not gfx950";
    case MQA_ERR_LAUNCH: return g_err[0] ? g_err : "HIP launch failed";
    default: return "unknown error code";
  }
}

}  // extern "C"
