/*
 * mqa_topk.h -- C ABI of the MI355X (gfx950) FP8 MQA-logits + top-k prefill
 * library (libmqa_topk.so).
 *
 * The operation (vLLM API page "fused_mqa_topk", fused_mqa_topk_prefill; vLLM
 * PR #60618, "What this PR does"): for every query row r and every visible key
 * j in [start_r, end_r),
 *
 *     logit[r,j] = scale_j * sum_{h<32} w[r,h] * relu(q[r,h,:] . k[j,:])
 *
 * with q [rows,32,128] and k [keys,128] in OCP FP8 e4m3 (e4m3fn), scale_j the
 * fp32 decoded from a UE8M0 byte e as the bit pattern e << 23 (same page,
 * fused_mqa_topk_key_scales) and w [rows,32] fp32; then return each row's k
 * largest keys (k = 512, 1024 or 2048) as key - start_r, in no particular
 * order, with -1 in the slots a row with fewer than k visible keys leaves.
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     allocates no device memory and keeps no state between calls (apart from
 *     the event ring of MQA_FLAG_TIME_SCAN).
 *   - Every call is asynchronous on `stream` (a hipStream_t; 0 is the null
 *     stream). A return of MQA_OK means the work was queued.
 *   - On any error code nothing has been launched.
 *   - Nothing traps or aborts, on the host or on the device.
 *   - starts/ends are read on the device. A row's range is clamped there to
 *     s = clamp(start, 0, keys), e = clamp(end, s, keys); an empty range gives
 *     an all -1 output row.
 *   - Output rows hold min(n, k) distinct valid entries in slots [0, min(n,k))
 *     and -1 in the remaining slots (n = e - s). Order is otherwise unspecified;
 *     among keys tied at the k-th score any subset may be returned.
 */
#ifndef MQA_TOPK_H
#define MQA_TOPK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define MQA_OK 0
#define MQA_ERR_NULL 1      /* a required pointer is NULL */
#define MQA_ERR_ALIGN 2     /* q, k, scales, weights, out/logits not 16-B aligned;
                               starts/ends not 4-B aligned; workspace not 256-B aligned */
#define MQA_ERR_SHAPE 3     /* rows < 1, keys < 1 or > MQA_MAX_KEYS, topk not in
                               {512,1024,2048}, or a bad column window / leading dim */
#define MQA_ERR_WORKSPACE 4 /* workspace_bytes < workspace_size(rows, device) */
#define MQA_ERR_DEVICE 5    /* no current HIP device, or it is not gfx950 */
#define MQA_ERR_LAUNCH 6    /* a HIP launch failed; mqa_strerror names the HIP error */

#define MQA_HEADS 32
#define MQA_HEAD_DIM 128
#define MQA_MAX_KEYS (1 << 20) /* 1M keys per call (PR #60618, "Limitations") */
#define MQA_MAX_ROWS (1 << 20)
#define MQA_MAX_BLOCKS 2048    /* blocks of 8 keys per row of the two-level selection */

/* Test-only flags for mqa_topk_prefill (0 in normal use). The output never
 * depends on them: they force the exact fallback (PR #60618, "What this PR
 * does": exact rescan) so that tests can reach it. */
#define MQA_FLAG_FORCE_EXACT 1u     /* every row takes the exact streaming rescan */
#define MQA_FLAG_FORCE_GATE_MISS 2u /* the gate admits nothing: every gated row falls back */
#define MQA_FLAG_SMALL_CAP 4u       /* per-row candidate slab limited to topk + 128
                                       (a merge past topk / (2 S) + 64 records per key
                                       segment when a call with few rows splits each
                                       block's keys into S segments) */
#define MQA_FLAG_STATS 8u           /* fill the mqa_stats header of the workspace */
#define MQA_FLAG_TIME_SCAN 16u      /* record HIP events around the scan kernel (see
                                       mqa_scan_time); a benchmarking aid */
#define MQA_FLAG_FORCE_RESCAN 32u   /* every gated row skips the certified select and
                                       is redone by the bounded rescan from an open
                                       bound */
#define MQA_FLAG_DETERMINISTIC 64u  /* deterministic, batch-invariant selection (API
                                       page, use_fused_mqa_topk: batch-invariant serving
                                       stays on the dense path there because which tied
                                       k-th-score keys the fused op keeps depends on its
                                       atomics' order): a
                                       row's output is the k keys of largest
                                       exact score, ties at the k-th score going to the
                                       smallest keys, listed in ascending key order
                                       (then the -1 padding); certificates are strict,
                                       and one more launch sorts the rows */

/* Counters written to the first bytes of the workspace when MQA_FLAG_STATS is
 * set (read them after the stream has finished the call). A call over more
 * than 16384 rows runs in batches of 16384 rows that share the workspace; the
 * counters then describe the last batch. */
typedef struct mqa_stats {
  uint32_t claim_counter;   /* internal: blocks claimed (== number of blocks) */
  uint32_t rows_short;      /* rows with n <= k (no scoring) */
  uint32_t rows_gated;      /* rows served by the gate + certified select */
  uint32_t rows_exact;      /* rows served by the exact streaming rescan */
  uint32_t rows_rescanned;  /* uncertified rows redone by the bounded rescan */
  uint32_t rows_undercount; /* gated rows with fewer than k candidates */
  uint32_t compactions;     /* slab merges (keep the best records, raise the threshold) */
  uint32_t rows_uncertified;/* gated rows whose k-th exact score fell outside the window
                               the select cut its candidates' error intervals against */
  uint64_t candidates;      /* candidates emitted by gated rows */
  uint64_t band_keys;       /* keys rescored exactly around the rows' k-th scores */
  float bound_ratio_max;    /* largest |exact - FP8 score| / proven error bound among
                               the rescored keys (below 1 whenever the bound holds) */
} mqa_stats;

/*
 * Bytes of device workspace one mqa_topk_prefill call over `rows` query rows
 * needs on HIP device `device` (the pages' get_fused_mqa_topk_workspaces, API
 * page "fused_mqa_topk"). It holds the block order, per-row state and queues,
 * one candidate slab of 16640 (score, key) records per row of a batch of up
 * to 16384 rows (1.09 GB for a full batch), and per-wave merge buffers of
 * 10240 records for every workgroup the device runs at once; it grows with
 * rows up to 16384 and with the device's compute-unit count. Returns 0 if the
 * device does not exist or is not gfx950, or rows is out of range.
 */
size_t workspace_size(int rows, int device);

/*
 * The fused path (API page "fused_mqa_topk", fused_mqa_topk_prefill; PR
 * #60618, "What this PR does"): scores every visible key of every row and
 * writes each row's top-k without writing the [rows, keys] logits.
 *   q        [rows,32,128] e4m3 bytes, row-major, 16-B aligned
 *   k        [keys,128]    e4m3 bytes, row-major, 16-B aligned
 *   scales   [keys] fp32 (decoded UE8M0, >= 0), 16-B aligned
 *   weights  [rows,32] fp32, 16-B aligned
 *   starts, ends [rows] int32, 4-B aligned
 *   out      [rows,topk] int32, 16-B aligned (written entirely)
 *   rows in [1, MQA_MAX_ROWS], keys in [1, MQA_MAX_KEYS], topk in {512,1024,2048}
 *   workspace: >= workspace_size(rows, current device) bytes, 256-B aligned;
 *     scratch owned by this call until the stream reaches its end (calls that
 *     share one workspace must be ordered on one stream). No prior contents
 *     are needed: the call resets what it uses.
 *   flags: 0, or MQA_FLAG_* bits (test-only).
 * Returns MQA_OK or an MQA_ERR_* code (checked in the order NULL, ALIGN,
 * SHAPE, DEVICE, WORKSPACE).
 */
int mqa_topk_prefill(const uint8_t* q, const uint8_t* k, const float* scales,
                     const float* weights, const int32_t* starts, const int32_t* ends,
                     int32_t* out, int rows, int keys, int topk, void* workspace,
                     size_t workspace_bytes, unsigned flags, void* stream);

/*
 * Source layers of DeepSeek-V4.1's two-level candidate selection (PR #60618,
 * "Limitations of this PR -- TODOs": the source layer also writes, per row,
 * the top 2048 blocks of 8 keys ranked by their maximum score). Writes out
 * exactly as mqa_topk_prefill, and
 *   out_blocks [rows, MQA_MAX_BLOCKS] int32, 16-B aligned: the row's 2048
 *     blocks of largest score, unordered, -1 padded when the row has fewer
 *     blocks. Block B is keys 8B .. 8B + 7 of the key numbering; its score
 *     for a row is the maximum exact logit over the row's visible keys in
 *     it; the row names it B - s / 8 (s the row's clamped start), as
 *     mqa_topk_masked reads it. MQA_FLAG_DETERMINISTIC: ties at the 2048th
 *     score go to the smallest blocks, and the row is sorted.
 * The call gates for at least 2048 keys, so that the key candidates cover the
 * blocks; rows they do not certify get an exact scan of their keys. Other
 * arguments, the workspace (>= workspace_size(rows, device)) and the return
 * codes as for mqa_topk_prefill (32 heads).
 */
int mqa_topk_prefill_blocks(const uint8_t* q, const uint8_t* k, const float* scales,
                            const float* weights, const int32_t* starts, const int32_t* ends,
                            int32_t* out, int32_t* out_blocks, int rows, int keys, int topk,
                            void* workspace, size_t workspace_bytes, unsigned flags,
                            void* stream);

/*
 * Consumer layers of DeepSeek-V4.1's two-level candidate selection (PR
 * #60618, "Limitations of this PR -- TODOs": they mask their scores to the
 * source layer's blocks of 8 keys before the top-k). Row r keeps only the
 * keys of its listed blocks: entry j of blocks[r] names keys
 * 8 (j + s / 8) .. 8 (j + s / 8) + 7, s the row's clamped start (the naming of
 * the source layer's block output), those inside the row's visible range;
 * entries < 0 are padding. The row's output is the top-k of its kept keys by
 * exact score (key - s, unordered, -1 padded when it keeps fewer than topk
 * keys); MQA_FLAG_DETERMINISTIC sorts it by key and gives ties at the k-th
 * score to the smallest keys.
 *   blocks   [rows, nb] int32, 4-B aligned, nb in [1, MQA_MAX_BLOCKS]; a
 *            row's non-negative entries must be distinct
 *   workspace >= workspace_size(rows, device) bytes, 256-B aligned
 * Other arguments and return codes as for mqa_topk_prefill (32 heads).
 */
int mqa_topk_masked(const uint8_t* q, const uint8_t* k, const float* scales, const float* weights,
                    const int32_t* starts, const int32_t* ends, const int32_t* blocks, int nb,
                    int32_t* out, int rows, int keys, int topk, void* workspace,
                    size_t workspace_bytes, unsigned flags, void* stream);

/*
 * Bytes of device workspace one mqa_topk_prefill_heads call over `rows` rows
 * of `heads` index heads needs on HIP device `device` (heads 32: the same as
 * workspace_size). Returns 0 for a bad device or size, or heads not 32 or 64.
 */
size_t workspace_size_heads(int rows, int heads, int device);

/*
 * mqa_topk_prefill with 32 or 64 index heads (64: DeepSeek-V3.2's indexer, PR
 * #60618, "Limitations of this PR -- TODOs"):
 *     logit[r,j] = scale_j * sum_{h<heads} w[r,h] * relu(q[r,h,:] . k[j,:])
 *   q        [rows, heads, 128] e4m3, 16-B aligned
 *   weights  [rows, heads] fp32, 16-B aligned
 *   heads    32 or 64
 * Every other argument, the workspace (>= workspace_size_heads(rows, heads,
 * device) bytes), the flags, the output and the return codes as for
 * mqa_topk_prefill. A 64-head row runs as two 32-head halves whose scores
 * are added before any selection (its FP8 error bound is the sum of the
 * halves' bounds); calls run in batches of at most 8192 such rows.
 */
int mqa_topk_prefill_heads(const uint8_t* q, const uint8_t* k, const float* scales,
                           const float* weights, const int32_t* starts, const int32_t* ends,
                           int32_t* out, int rows, int keys, int heads, int topk,
                           void* workspace, size_t workspace_bytes, unsigned flags,
                           void* stream);

/*
 * mqa_topk_prefill without a workspace argument and without any allocation,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc). Same
 * arguments, contract and results as mqa_topk_prefill; its scratch is a
 * 384 MiB array in device memory that the library holds on each device it
 * runs on until the process ends, so the rows run in batches that fit it
 * (about 1600 rows per batch on a 256-CU device; a call over more rows runs
 * the batches one after another on `stream`). Every call on a device uses the
 * same scratch: calls that overlap on one device (other streams, other
 * threads) race and must not be made. Nothing needs clearing before a call.
 * MQA_FLAG_STATS writes its counters into that scratch, where the caller
 * cannot read them. Returns MQA_OK, MQA_ERR_NULL, MQA_ERR_ALIGN,
 * MQA_ERR_SHAPE, MQA_ERR_DEVICE, MQA_ERR_WORKSPACE (the scratch cannot hold
 * one 32-row batch on this device) or MQA_ERR_LAUNCH (also when the
 * scratch's device address cannot be looked up).
 */
int mqa_topk_prefill_static(const uint8_t* q, const uint8_t* k, const float* scales,
                            const float* weights, const int32_t* starts, const int32_t* ends,
                            int32_t* out, int rows, int keys, int topk, unsigned flags,
                            void* stream);

/*
 * Bytes of device workspace one mqa_topk_prefill_paged call over `rows` rows
 * and `keys` keys needs on HIP device `device`: workspace_size(rows, device)
 * plus 128 bytes per key for the keys compacted out of the pages. Returns 0
 * if the device does not exist or is not gfx950, or the sizes are out of
 * range.
 */
size_t workspace_size_paged(int rows, int keys, int device);

/*
 * The fused path reading the keys straight from the paged indexer K-cache, the
 * UE8M0 decode fused (PR #60618, "Motivation": an indexer cache entry is 132 B
 * per token, a 128-byte e4m3 key and a 4-byte scale; API page,
 * fused_mqa_topk_key_scales, for the scale word). Key j of the call (the same
 * key numbering as mqa_topk_prefill's k, which starts/ends and the output refer
 * to) is slot j % page_size of page block_table[j / page_size].
 *   cache        [num_pages][page_size * 132] bytes, 16-B aligned: page p holds
 *                its page_size keys' e4m3 rows ([page_size][128]), then their
 *                scale words ([page_size][4] bytes, four equal UE8M0 bytes e;
 *                the scale is the fp32 with bit pattern (e & 0xFF) << 23; e =
 *                255, which decodes to +inf, is outside the contract)
 *   block_table  [ceil(keys / page_size)] int32, 4-B aligned; an entry outside
 *                [0, num_pages) is clamped into it (the call's result is then
 *                unspecified, but nothing reads outside the cache)
 *   page_size    a power of two in [4, MQA_MAX_KEYS]; num_pages >= 1
 * Several requests share one call as with mqa_topk_prefill: the caller lays
 * their keys out in the key numbering (each request's first key at a
 * multiple of page_size, its pages in its table order) and gives every row
 * its request's range. The first kernel reads every key once from its page
 * (for its error bound and its decoded scale) and copies it into the
 * workspace, where the later kernels, which read each key once per block of
 * rows, find it contiguous. Workspace: >= workspace_size_paged(rows, keys,
 * current device) bytes, 256-B aligned. Flags, output and return codes as for
 * mqa_topk_prefill, whose results it reproduces on the gathered keys and
 * decoded scales (bit for bit under MQA_FLAG_DETERMINISTIC).
 */
int mqa_topk_prefill_paged(const uint8_t* q, const uint8_t* cache, const int32_t* block_table,
                           int page_size, int num_pages, const float* weights,
                           const int32_t* starts, const int32_t* ends, int32_t* out, int rows,
                           int keys, int topk, void* workspace, size_t workspace_bytes,
                           unsigned flags, void* stream);

/*
 * Bytes of device workspace one mqa_topk_decode_paged call over `requests`
 * requests of `rows_per_request` rows needs on HIP device `device`: the
 * mqa_topk_prefill workspace of one batch of requests (a batch holds at most
 * 16384 rows and 512 workgroups; a workgroup holds four parts of up to 8 rows
 * of a request each). Returns 0 if the device
 * does not exist or is not gfx950, or the sizes are out of range.
 */
size_t workspace_size_decode(int requests, int rows_per_request, int device);

/*
 * The fused path shaped for decode (PR #60618's review thread, the decode
 * follow-up: many requests of a few query rows each, such as speculative
 * tokens, each request with its own long context): row r is row r % R of
 * request r / R (R = rows_per_request), and sees positions [s, e) of its own
 * request's keys, s and e the row's starts/ends clamped to [0, K], K =
 * min(table_stride * page_size, MQA_MAX_KEYS). Position j of request i is
 * slot j % page_size of cache page page_table[i * table_stride + j /
 * page_size] (the cache layout of mqa_topk_prefill_paged; an entry outside
 * [0, num_pages) is clamped into it, and entries past a request's visible
 * positions are never used for its results). Each row's output holds its
 * top-k positions as position - s, unordered, -1 padded, with the conventions
 * of mqa_topk_prefill (flags included).
 *   q        [requests * R, 32, 128] e4m3, 16-B aligned
 *   cache    [num_pages][page_size * 132] bytes, 16-B aligned
 *   page_table [requests][table_stride] int32, 4-B aligned
 *   weights  [requests * R, 32] fp32; starts, ends [requests * R] int32
 *   out      [requests * R, topk] int32, 16-B aligned
 *   requests >= 1, R in [1, 32], requests * R <= MQA_MAX_ROWS, table_stride
 *   >= 1, page_size a power of two in [4, MQA_MAX_KEYS], num_pages >= 1,
 *   topk in {512, 1024, 2048}
 *   workspace: >= workspace_size_decode(requests, R, current device) bytes,
 *   256-B aligned, owned by the call until the stream reaches its end.
 * Requests run in batches (workspace_size_decode) in order on `stream`. The
 * rows of a part of a request (up to 8 rows) share its key copies; a request
 * of R rows reads its keys ceil(R / 8) times, and R not a multiple of 8 leaves
 * row slots of a workgroup empty. Returns MQA_OK or an MQA_ERR_*
 * code (checked in the order NULL, ALIGN, SHAPE, DEVICE, WORKSPACE).
 */
int mqa_topk_decode_paged(const uint8_t* q, const uint8_t* cache, const int32_t* page_table,
                          int table_stride, int page_size, int num_pages, const float* weights,
                          const int32_t* starts, const int32_t* ends, int32_t* out, int requests,
                          int rows_per_request, int topk, void* workspace,
                          size_t workspace_bytes, unsigned flags, void* stream);

/*
 * Dense logits (the first half of the dense path the fused op replaces: PR
 * #60618, "Motivation"; API page, fused_mqa_topk_prefill names the
 * fp8_mqa_logits + top_k_per_row_prefill pair): writes
 *   logits[r * ld + c] = logit[r, col0 + c]   for c in [0, ncols)
 * as fp32, and -inf where col0 + c lies outside row r's visible range.
 *   logits: [rows, ld] fp32, 16-B aligned, ld >= ncols, ld % 4 == 0
 *   col0 >= 0, ncols >= 1, col0 + ncols <= keys
 * Other arguments as for mqa_topk_prefill.
 */
int mqa_logits_dense(const uint8_t* q, const uint8_t* k, const float* scales,
                     const float* weights, const int32_t* starts, const int32_t* ends,
                     float* logits, int64_t ld, int rows, int keys, int col0, int ncols,
                     void* stream);

/*
 * Dense per-row top-k (the second half of the dense path): for each row r,
 * the topk largest logits among columns c whose key col0 + c lies in the
 * row's visible range [s, e) and inside the window [col0, col0 + ncols);
 * writes key - s, unordered, -1 padded (slots [n', topk) when the row has
 * n' <= topk such columns, in which case slots [0, n') hold 0..n'-1 shifted
 * by max(0, col0 - s)).
 *   logits [rows, ld] fp32 as written by mqa_logits_dense; out [rows, topk].
 */
int mqa_topk_dense(const float* logits, int64_t ld, int col0, int ncols,
                   const int32_t* starts, const int32_t* ends, int32_t* out, int rows,
                   int keys, int topk, void* stream);

/*
 * UE8M0 key-scale decode (API page, fused_mqa_topk_key_scales): the gathered
 * indexer K-cache scales [keys,4] uint8 (four equal bytes per key) viewed as a
 * little-endian int32, low byte e -> fp32 with bit pattern e << 23 (e = 0 gives
 * +0.0, e = 255 gives +inf, which is outside the contract of the other calls).
 *   scale_bytes: [keys,4] uint8, 4-B aligned; scales: [keys] fp32, 4-B aligned.
 */
int mqa_key_scales(const uint8_t* scale_bytes, float* scales, int keys, void* stream);

/*
 * Total GPU time, in milliseconds, of the scan kernel (the dominant kernel of
 * mqa_topk_prefill) over the last `last_n` calls made on the current device
 * with MQA_FLAG_TIME_SCAN, from HIP events recorded on the call's stream just
 * before and after that kernel. The library keeps one ring of 256 event pairs
 * per device, created on the first timed call and kept until the process ends.
 * Blocks until the last of those calls has finished.
 *   last_n in [1, number of timed calls so far on this device, at most 256]
 * Returns MQA_OK, MQA_ERR_NULL (total_ms NULL), MQA_ERR_SHAPE (last_n out of
 * range), MQA_ERR_DEVICE or MQA_ERR_LAUNCH (an event query failed).
 */
int mqa_scan_time(int last_n, float* total_ms);

/*
 * FP8 MFMA throughput probe (a benchmarking aid; the pages give no peak for the
 * part they measure on, so the scan's MFMA fraction is also read against the
 * rate this machine sustains). Launches `workgroups` workgroups of 512 threads
 * on `stream`; each of their 8 waves issues `iters` rounds of 8 independent
 * v_mfma_f32_16x16x128_f8f6f4 (the instruction of the scan's head tiles) on
 * register operands and writes one float per thread to `out` (the sums, so that
 * nothing is optimised away). FP8 flop per launch: workgroups * 8 * iters * 8 *
 * 65536. The caller times the launch (events on `stream`).
 *   out: device, caller-owned, >= workgroups * 512 floats (out_len), 4-B aligned;
 *   workgroups in [1, 65536]; iters in [1, 2^20].
 * Returns MQA_OK, MQA_ERR_NULL, MQA_ERR_ALIGN, MQA_ERR_SHAPE (sizes out of range
 * or out_len too small), MQA_ERR_DEVICE or MQA_ERR_LAUNCH; nothing is launched
 * on an error.
 */
int mqa_mfma_peak(float* out, int64_t out_len, int workgroups, int iters, void* stream);

/*
 * FP8 MFMA precision probe (a test aid: the fused path's error bounds rest on
 * how this instruction rounds). Runs the scan's instruction forms on caller
 * operands, one 16x16 product per case:
 *   out[c][m][n] = sum_d a[c][m][d] * b[c][n][d]   (as the MFMA computes it)
 * with v_mfma_f32_16x16x128_f8f6f4 (ascale NULL) or, with ascale, its scaled
 * form, a[c][m][d] taking the E8M0 scale ascale[c][m][blk] of the 32-wide
 * K block blk that holds d (the block of dims {0-15, 32-47}, {64-79, 96-111},
 * {16-31, 48-63} or {80-95, 112-127}) and b scale 1.
 *   a, b: [ncases][16][128] OCP e4m3 bytes, 16-B aligned; ascale: NULL or
 *   [ncases][16][4] bytes; out: [ncases][16][16] fp32, 4-B aligned; all
 *   device pointers owned by the caller; ncases in [1, 2^20].
 * Returns MQA_OK, MQA_ERR_NULL, MQA_ERR_ALIGN, MQA_ERR_SHAPE, MQA_ERR_DEVICE
 * or MQA_ERR_LAUNCH; asynchronous on `stream`.
 */
int mqa_fp8_mfma_probe(const uint8_t* a, const uint8_t* b, const uint8_t* ascale, float* out,
                       int ncases, void* stream);

/* Human-readable text of a return code (for MQA_ERR_LAUNCH it names the HIP
 * error of the failing call on this thread). Never NULL. */
const char* mqa_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* MQA_TOPK_H */
