// Kernel parameter blocks and launch entry points shared by the kernel
// translation units and the C ABI (api.hip). Host-visible plain structs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mqa {

// Per-row state handed from the gate to the scan and from the scan to the
// select kernel.
struct RowInfo {
  float thr;   // admission threshold
  int cnt;     // candidates in the row's slab
  int mode;    // how the row is served (fused.hip RowMode)
  int strict;  // 1: candidates had to beat thr strictly (a merge raised it, or a
               // bounded-rescan round admits scores above its bound only)
  int above;   // bounded rescan: keys scoring strictly above thr
  int filled;  // bounded rescan: output slots [k - filled, k) already hold ties of thr
};

// Per-(row, key segment) state of a split scan (nseg > 1): the segment's
// final admission bound and its candidate count in the segment's part of the
// row's slab.
struct SegInfo {
  float thr;  // every candidate of the segment scores >= thr, every other key <= thr
  int cnt;
};

// Per-row hand-over from the gate to its fine pass (fused_refine_kernel):
// the coarse histogram's reference and scale, the crowded threshold bin (-1:
// the row needs no fine pass), the sample count still needed inside it and
// the next sampled coarse bin below it.
struct RefineInfo {
  float m0, inv;
  int bin, need, next;
};

struct FusedParams {
  const uint8_t* q;
  const uint8_t* k;  // [keys][128] e4m3; with a page table: the paged indexer cache
  const float* scales;
  const float* weights;
  const int32_t* starts;
  const int32_t* ends;
  int32_t* out;
  int rows, keys, topk, nblocks;
  // Key segments per block: with few blocks each block's key range is split
  // into nseg segments scanned as separate work items (nblocks * nseg items
  // over scan_grid persistent workgroups), each into its own part of the
  // rows' slabs; 1 otherwise.
  int nseg, scan_grid;
  unsigned flags;
  uint32_t* header;  // 64 words: stats + claim counter
  int32_t* order;    // [nblocks] heaviest-first block order
  uint8_t* xrow;     // [rows] 1 = the row needs the exact rescan
  int32_t* xqueue;   // [nblocks] blocks queued for the exact rescan
  int32_t* fqueue;   // [nblocks] blocks queued for the gate's fine pass
  uint32_t* fflag;   // [nblocks] 1 = the block is queued for the fine pass
  RefineInfo* rinfo; // [rows]
  int32_t* rqueue;   // [3][nblocks * 32] rows queued for the three bounded-rescan rounds
  uint32_t* xflag;   // [nblocks] 1 = the block is queued
  RowInfo* rowinfo;  // [rows]
  SegInfo* seg;      // [nblocks * 32 rows][kMaxSeg] (nseg > 1)
  // FP8 score error bounds (written by the prologue): an FP8-scored key j of
  // row r is within beta[r] * nhat_j of its exact score. keyinfo[2j] is key
  // j's scale, keyinfo[2j + 1] its nhat, which keeps only its top 12 bits
  // (the low 20 are zero) so that it travels in the upper bits of a
  // candidate record's key word.
  float* keyinfo;    // [keys][2]
  float* beta;       // [rows]
  // Paged indexer cache (table != nullptr): key j lives in page
  // table[j >> page_shift] of k (clamped to [0, num_pages)), slot
  // j & (2^page_shift - 1); a page of P = 2^page_shift tokens holds their
  // P x 128 e4m3 codes, then their P 4-byte UE8M0 scale words
  // (page_bytes = 132 P). scales is unused then: the prologue decodes the
  // scales into keyinfo and copies the keys to kc, and the kernels after it
  // read kc like gathered keys.
  const int32_t* table;
  int page_shift, num_pages;
  int64_t page_bytes;
  uint8_t* kc;  // [keys][128] paged prefill: the keys compacted by the prologue
  // Decode-shaped calls (dec_rows > 0): nreq requests of dec_rows rows each
  // (row r belongs to request r / dec_rows); request q's key positions map
  // to pages through table row q (table_stride entries). A request's rows
  // form dec_parts parts of up to 8 rows, and blocks pack four parts; keys
  // is the positions' bound, and keyinfo is unused.
  int dec_rows, dec_parts, nreq, table_stride;
  // Index heads / 32 (1, or 2 for 64 heads). With 64 heads a row r runs as
  // the virtual rows 2r (its lead: state, candidates, output) and 2r + 1 (its
  // partner: heads 32..63), each read as a 32-head row of q and weights; rows
  // counts virtual rows, and starts/ends/out are indexed by r.
  int hm;
  // The gate's key target (topk, or at least 2048 when blocks_out is set)
  // and the merges' keep count 2 * kgate.
  int kgate;
  // Two-level source calls: [rows][2048] block output (nullptr otherwise),
  // and the queue of rows for the exact block scan [rows].
  int32_t* blocks_out;
  int32_t* bqueue;
  float* slabE;      // [nblocks * 32 rows][kSlabRow] candidate scores
  int32_t* slabI;    // [nblocks * 32 rows][kSlabRow] candidate keys
  float* tmpE;       // [grid][8 waves][kTmp] merge buffers
  int32_t* tmpI;
};

struct DenseParams {
  const uint8_t* q;
  const uint8_t* k;
  const float* scales;
  const float* weights;
  const int32_t* starts;
  const int32_t* ends;
  float* logits;
  int64_t ld;
  int rows, keys, col0, ncols;
};

struct DenseTopkParams {
  const float* logits;
  int64_t ld;
  int col0, ncols;
  const int32_t* starts;
  const int32_t* ends;
  int32_t* out;
  int rows, keys, topk;
};

constexpr int kFusedBlockRows = 32;
constexpr int kTmp = 10240;  // merge-buffer records per wave
// Records per slab row: a capacity of 16384 plus room for one more chunk of
// 64 records past it (rows stay 1 KiB aligned).
constexpr int kSlabRow = 16384 + 256;
constexpr int kFusedWaves = 8;
constexpr int kMaxSeg = 8;
// Rows per launch sequence: larger calls run in batches of this many rows
// (the workspace holds one batch's candidate slabs, 1.09 GB).
constexpr int kMaxBatchRows = 16384;
// A candidate record's key word: the key in the low 20 bits (keys < 2^20),
// the key's nhat bit pattern in the others.
constexpr uint32_t kKeyMask = 0xFFFFFu;

}  // namespace mqa

extern "C" {
// scan_begin/scan_end: optional events recorded around the scan kernel.
int mqa_fused_launch(const mqa::FusedParams* p, int grid, hipStream_t stream,
                     hipEvent_t scan_begin, hipEvent_t scan_end);
int mqa_fused_occupancy(int* wg_per_cu);
int mqa_masked_launch(const mqa::FusedParams* p, const int32_t* blocks, int nb,
                      hipStream_t stream);
int mqa_dense_logits_launch(const mqa::DenseParams* p, hipStream_t stream);
int mqa_dense_topk_launch(const mqa::DenseTopkParams* p, hipStream_t stream);
int mqa_key_scales_launch(const uint8_t* b, float* s, int keys, hipStream_t stream);
}
