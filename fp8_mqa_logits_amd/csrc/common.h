// Device building blocks shared by the fused and dense kernels (gfx950 only).
//
// Scoring tile (FP8 MFMA 16x16x128, measured operand layouts on gfx950):
//   A operand (one 16-head half of one query row): lane l holds head
//     16*hh + (l % 16), bytes [32*(l/16), 32*(l/16) + 32) of its 128-dim vector.
//   B operand (16 keys): lane l holds key (l % 16), the same 32-byte K slice.
//   C (fp32 16x16): lane l, element v holds head 4*(l/16) + v, key (l % 16).
// One query row against 64 keys is 4 key sub-tiles x 2 head halves = 8 MFMAs.
// Each lane then owns 8 heads of 4 keys; it applies relu and the head weights
// (vLLM PR #60618, "What this PR does": per-head relu, weighted head sum), and
// two permlane swap+add steps leave lane l holding the unscaled score of key l
// of the 64-key chunk.
//
// Precision (measured on gfx950): the FP8 MFMA sums its products in groups of
// 8 and truncates each product toward zero on a grid of 2^(e - 13), e being
// the exponent of the group's largest product, so its dot products carry
// errors of up to ~2^-12 of sum|q_d k_d|. The bf16 MFMA, fed the same e4m3
// values converted exactly to bf16, accumulates them to fp32 accuracy. The
// scan therefore ranks with FP8 scores, and every score that decides the
// result near a row's k-th key is recomputed with score_chunk_exact below.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mqa {

constexpr int kHeads = 32;
constexpr int kDim = 128;
constexpr int kWave = 64;
constexpr int kChunk = 64;                 // keys per LDS stage
constexpr int kChunkBytes = kChunk * kDim; // 8 KiB
// Word 3 of an unswizzled buffer resource on gfx950: 32-bit data format.
// Raw (stride 0): offsets are bytes and stores past num_records bytes are
// dropped; structured (stride > 0): a store addresses record `vindex` and
// records past num_records are dropped.
constexpr int kBufferFlags = 0x00020000;

// Structured-buffer dword store (the LLVM intrinsic has no clang builtin):
// writes v at base + soffset + voffset + stride * vindex.
__device__ void struct_buffer_store_b32(uint32_t v, __amdgpu_buffer_rsrc_t rsrc, int vindex,
                                        int voffset, int soffset, int aux)
    __asm("llvm.amdgcn.struct.ptr.buffer.store.i32");
constexpr int kCap = 16384;                // candidate slab capacity per row
constexpr int kMaxTopk = 2048;

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

__device__ __forceinline__ v4f mfma_fp8(v8i a, v8i b, v4f c) {
  // cbsz = blgp = 0: both operands OCP e4m3. Scale operands 0 make the
  // compiler emit the unscaled v_mfma_f32_16x16x128_f8f6f4 (no scale-load
  // prefix instruction); the scaled form is only needed for the fold terms.
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ v4f mfma_bf16(v8bf a, v8bf b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 8 e4m3 bytes (two dwords) -> 8 bf16, exact (every e4m3 value is a bf16).
__device__ __forceinline__ v8bf fp8x8_to_bf16(int lo, int hi) {
  const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.f, false);
  const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.f, true);
  const v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.f, false);
  const v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.f, true);
  return v8bf{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Index of the calling wave in its workgroup, as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0)); }

// LDS placement of a 64-key chunk: key j's 16-byte slice c (0..7) lives at
// slot (c ^ swz(j)) of its 128-byte row, so that the 16 lanes reading one
// slice of 16 different keys touch 16 different bank groups.
__device__ __forceinline__ int swz(int j) { return (j & 7) ^ ((j >> 3) & 1); }

// Order-preserving map fp32 -> uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t fkey(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float kfloat(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

// Query operands of one row: qa[hh] for heads 16*hh .. 16*hh+15.
struct QueryRow {
  v8i qa[2];
  float w[8];  // w[r, 16*hh + 4*(l/16) + v] at index 4*hh + v
};

// wmul scales the weights as they are loaded (the FP8 scorers take w / 2, the
// relu fold's factor 1/2; exact scorers take w).
__device__ __forceinline__ void load_query(QueryRow& qr, const uint8_t* __restrict__ q,
                                           const float* __restrict__ weights, int64_t r,
                                           float wmul = 1.f) {
  const int l = lane_id();
  const int g = l >> 4;
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const uint8_t* p = q + (r * kHeads + 16 * hh + (l & 15)) * kDim + 32 * g;
    const uint4 x0 = *reinterpret_cast<const uint4*>(p);
    const uint4 x1 = *reinterpret_cast<const uint4*>(p + 16);
    qr.qa[hh] = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                    (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
    const float4 wv = *reinterpret_cast<const float4*>(weights + r * kHeads + 16 * hh + 4 * g);
    qr.w[4 * hh + 0] = wv.x * wmul;
    qr.w[4 * hh + 1] = wv.y * wmul;
    qr.w[4 * hh + 2] = wv.z * wmul;
    qr.w[4 * hh + 3] = wv.w * wmul;
  }
}

// B operands of the 4 key sub-tiles of a chunk staged in LDS.
struct KeyTile {
  v8i kb[4];
};

// Each 16-byte slice is read as one vector from a single byte offset off the
// chunk base. The shallow address chain matters: the compiler tags an LDS
// access with its variable's alias scope only when it can trace the address
// back to the variable in a few steps, and an untagged read waits for every
// direct global->LDS copy in flight, the next stage's included.
__device__ __forceinline__ void load_keys_lds(KeyTile& kt, const uint8_t* lds_chunk) {
  const int l = lane_id();
  const int g = l >> 4;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int j = 16 * t + (l & 15);
    const v4i x0 = *reinterpret_cast<const v4i*>(lds_chunk + (j * kDim + 16 * ((2 * g) ^ swz(j))));
    const v4i x1 =
        *reinterpret_cast<const v4i*>(lds_chunk + (j * kDim + 16 * ((2 * g + 1) ^ swz(j))));
    kt.kb[t] = __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
  }
}

// relu of an fp32 value as an integer max of its bit pattern (negative floats
// have the sign bit set, so they compare below 0): one VALU op, no NaN
// canonicalization.
__device__ __forceinline__ float relu(float x) {
  return __int_as_float(__builtin_elementwise_max(__float_as_int(x), 0));
}

// The 8 head-dot tiles of one query row against a 64-key chunk.
struct RowAcc {
  v4f a[4][2];
};

__device__ __forceinline__ void mfma_row(RowAcc& acc, const QueryRow& qr, const KeyTile& kt) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const v4f z = {0.f, 0.f, 0.f, 0.f};
    acc.a[t][0] = mfma_fp8(qr.qa[0], kt.kb[t], z);
    acc.a[t][1] = mfma_fp8(qr.qa[1], kt.kb[t], z);
  }
}

// Weighted relu sum over the lane's 8 heads of each sub-tile, then two
// permlane swap+add steps: lane l ends with the unscaled score of key l.
template <class Row>
__device__ __forceinline__ float reduce_heads(const Row& qr, const RowAcc& acc) {
  float part[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    float s = 0.f;
#pragma unroll
    for (int v = 0; v < 4; ++v) s = __builtin_fmaf(qr.w[v], relu(acc.a[t][0][v]), s);
#pragma unroll
    for (int v = 0; v < 4; ++v) s = __builtin_fmaf(qr.w[4 + v], relu(acc.a[t][1][v]), s);
    part[t] = s;
  }
  // lanes 0-31 | 32-63 hold head groups {0,1} | {2,3}; fold them pairwise
  const auto s02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[0]),
                                                    __float_as_uint(part[2]), false, false);
  const auto s13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[1]),
                                                    __float_as_uint(part[3]), false, false);
  const float y02 = __uint_as_float(s02[0]) + __uint_as_float(s02[1]);
  const float y13 = __uint_as_float(s13[0]) + __uint_as_float(s13[1]);
  const auto s4 = __builtin_amdgcn_permlane16_swap(__float_as_uint(y02), __float_as_uint(y13),
                                                   false, false);
  return __uint_as_float(s4[0]) + __uint_as_float(s4[1]);
}

// ---------------------------------------------------------------------------
// relu fold (vLLM PR #60618, "What this PR does"): relu(s) = (s + |s|) / 2, so
//   sum_h w_h relu(s_h) = ( sum_h w_h s_h + sum_h w_h |s_h| ) / 2
// and the linear half is one dot product of the key with the folded query
// f = sum_h w_h q_h. The factor 1/2 is exact and is carried by the operands:
// the weights are loaded halved and the fold terms' MFMA scale is halved. f (fp32) is carried as 4 e4m3 terms, each with a
// power-of-two scale per 32-element block of the MFMA's K order (its E8M0 A
// scales):
// term t encodes what terms 0..t-1 left over, so the sum of the terms
// matches f to about 2^-16 of each block's largest magnitude. The 4 terms of
// the wave's 4 rows are the 16 A rows of one extra MFMA per 16 keys: M row
// 4t + r = term t of row r, so that lane group g receives term g of every
// row (output register r: row r). Each row's head epilogue starts its
// lane's |s| accumulation from that term, and the cross-lane head reduction
// sums the 4 terms together with the 4 head groups.

struct FoldOp {
  v8i fa;      // this lane's 32 e4m3 codes: M row (l%16), dims 32*(l/16) ..
  int fscale;  // E8M0 scale byte of those codes
};

__device__ __forceinline__ float e4m3_to_f32(int word, int byte) {
  switch (byte) {
    case 0: return __builtin_amdgcn_cvt_f32_fp8(word, 0);
    case 1: return __builtin_amdgcn_cvt_f32_fp8(word, 1);
    case 2: return __builtin_amdgcn_cvt_f32_fp8(word, 2);
    default: return __builtin_amdgcn_cvt_f32_fp8(word, 3);
  }
}

// Builds this lane's fold operand for the wave's rows rows[0..3] (-1: unused
// row, zero terms). Lane l covers row (l%16)%4, term (l%16)/4, dims
// 32*(l/16) .. +31.
__device__ __forceinline__ void build_fold(FoldOp& fo, const uint8_t* __restrict__ q,
                                           const float* __restrict__ weights, const int* rows) {
  const int l = lane_id();
  const int m = l & 15;
  const int rr = m & 3;
  const int term = m >> 2;
  const int g = l >> 4;
  int row = rows[0];
#pragma unroll
  for (int i = 1; i < 4; ++i)
    if (rr == i) row = rows[i];
  float rho[32];
#pragma unroll
  for (int d = 0; d < 32; ++d) rho[d] = 0.f;
  if (row >= 0) {
    for (int h = 0; h < kHeads; ++h) {
      const float wv = weights[(int64_t)row * kHeads + h];
      const int* qp = reinterpret_cast<const int*>(q + ((int64_t)row * kHeads + h) * kDim + 32 * g);
#pragma unroll
      for (int d4 = 0; d4 < 8; ++d4) {
        const int word = qp[d4];
#pragma unroll
        for (int b = 0; b < 4; ++b)
          rho[4 * d4 + b] = __builtin_fmaf(wv, e4m3_to_f32(word, b), rho[4 * d4 + b]);
      }
    }
  }
  // Scale blocks follow the MFMA's K order: lane group g's bytes 0-15 and
  // 16-31 fall in the 32-wide blocks g/2 and 2 + g/2, each shared with the
  // same half of lane group g^1; block b's scale for A row m is read from
  // lane 16*b + m (both measured on gfx950).
  int codes[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  int e_kept[2] = {0, 0};
  auto exponent_for = [](float mx) {  // smallest e with mx * 2^-e <= 448
    int e = 0;
    if (mx > 0.f) {
      int ex;
      (void)__builtin_frexpf(mx / 448.f, &ex);
      e = ex;
      if (__builtin_ldexpf(448.f, e) < mx) e += 1;
      if (__builtin_ldexpf(448.f, e - 1) >= mx) e -= 1;
    }
    return e < -100 ? -100 : (e > 100 ? 100 : e);
  };
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    float hm[2] = {0.f, 0.f};
#pragma unroll
    for (int d = 0; d < 32; ++d) hm[d >> 4] = __builtin_fmaxf(hm[d >> 4], __builtin_fabsf(rho[d]));
    int e[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) e[h] = exponent_for(__builtin_fmaxf(hm[h], __shfl_xor(hm[h], 16, 64)));
    int cw[8];
#pragma unroll
    for (int d4 = 0; d4 < 8; ++d4) {
      const int h = d4 >> 2;
      const float down = __builtin_ldexpf(1.f, -e[h]);
      const float up = __builtin_ldexpf(1.f, e[h]);
      int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(rho[4 * d4] * down, rho[4 * d4 + 1] * down, 0, false);
      w0 = __builtin_amdgcn_cvt_pk_fp8_f32(rho[4 * d4 + 2] * down, rho[4 * d4 + 3] * down, w0, true);
      cw[d4] = w0;
#pragma unroll
      for (int b = 0; b < 4; ++b) rho[4 * d4 + b] -= e4m3_to_f32(w0, b) * up;
    }
    if (t == term) {
#pragma unroll
      for (int d4 = 0; d4 < 8; ++d4) codes[d4] = cw[d4];
      e_kept[0] = e[0];
      e_kept[1] = e[1];
    }
  }
  // the scale this lane supplies: block g, whose halves live in lane groups
  // {0,1} (blocks 0, 2) or {2,3} (blocks 1, 3)
  const int from_g2 = __shfl(e_kept[0], m + 32, 64);  // block 1: half 0 of group 2
  const int from_g0 = __shfl(e_kept[1], m, 64);       // block 2: half 1 of group 0
  const int es = g == 0 ? e_kept[0] : (g == 1 ? from_g2 : (g == 2 ? from_g0 : e_kept[1]));
  fo.fa = v8i{codes[0], codes[1], codes[2], codes[3], codes[4], codes[5], codes[6], codes[7]};
  fo.fscale = 126 + es;  // the MFMA applies f / 2: the relu fold's factor 1/2
}

// The fold terms of the wave's 4 rows for a 64-key chunk: 4 scaled MFMAs
// (one per 16-key sub-tile); ft[t][r] in lane group g is term g of row r for
// key 16t + l%16.
struct FoldTerms {
  v4f ft[4];
};

__device__ __forceinline__ void fold_terms(FoldTerms& f, const FoldOp& fo, const KeyTile& kt) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const v4f z = {0.f, 0.f, 0.f, 0.f};
    f.ft[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fo.fa, kt.kb[t], z, 0, 0, 0,
                                                               fo.fscale, 0, 127);
  }
}

// Linear half plus weighted |s| sum of row r: per sub-tile, the lane's fold
// term of row r plus its 8 heads (one abs-modified FMA per head), reduced
// across lane groups like reduce_heads (4 terms + 32 heads). With halved
// weights and fold terms this is the unscaled score itself.
__device__ __forceinline__ float reduce_heads_abs(const QueryRow& qr, const RowAcc& acc,
                                                  const FoldTerms& f, int r) {
  float part[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    float s = f.ft[t][r];
#pragma unroll
    for (int v = 0; v < 4; ++v) s = __builtin_fmaf(qr.w[v], __builtin_fabsf(acc.a[t][0][v]), s);
#pragma unroll
    for (int v = 0; v < 4; ++v)
      s = __builtin_fmaf(qr.w[4 + v], __builtin_fabsf(acc.a[t][1][v]), s);
    part[t] = s;
  }
  const auto s02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[0]),
                                                    __float_as_uint(part[2]), false, false);
  const auto s13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[1]),
                                                    __float_as_uint(part[3]), false, false);
  const float y02 = __uint_as_float(s02[0]) + __uint_as_float(s02[1]);
  const float y13 = __uint_as_float(s13[0]) + __uint_as_float(s13[1]);
  const auto s4 = __builtin_amdgcn_permlane16_swap(__float_as_uint(y02), __float_as_uint(y13),
                                                   false, false);
  return __uint_as_float(s4[0]) + __uint_as_float(s4[1]);
}

// Unscaled scores sum_h w[r,h] * relu(q[r,h,:] . k[j,:]) of the 64 keys of a
// chunk (key j = lane id) for one query row, with the head dots taken by the
// bf16 MFMA (16x16x32) on the exactly converted e4m3 values: fp32-accurate.
// Each lane's 32 bytes (dims 32g .. 32g+31) feed 4 K-steps of 8 elements;
// A and B use the same dim order, so every dot product covers all 128 dims.
__device__ __forceinline__ float score_chunk_exact(const QueryRow& qr, const KeyTile& kt) {
  RowAcc acc;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    v4f a0 = {0.f, 0.f, 0.f, 0.f};
    v4f a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const v8bf bk = fp8x8_to_bf16(kt.kb[t][2 * st], kt.kb[t][2 * st + 1]);
      a0 = mfma_bf16(fp8x8_to_bf16(qr.qa[0][2 * st], qr.qa[0][2 * st + 1]), bk, a0);
      a1 = mfma_bf16(fp8x8_to_bf16(qr.qa[1][2 * st], qr.qa[1][2 * st + 1]), bk, a1);
    }
    acc.a[t][0] = a0;
    acc.a[t][1] = a1;
  }
  return reduce_heads(qr, acc);
}

// A query row with its e4m3 values converted to bf16 once, for scorers that
// score many chunks exactly against one row (the conversion otherwise costs
// 128 of the ~270 VALU instructions of each score_chunk_exact call). The
// products, their order and the reduction are score_chunk_exact's, so both
// give the same bits.
struct QueryRowB {
  v8bf qb[2][4];
  float w[8];
};

__device__ __forceinline__ void to_bf16(QueryRowB& b, const QueryRow& qr) {
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
    for (int st = 0; st < 4; ++st)
      b.qb[hh][st] = fp8x8_to_bf16(qr.qa[hh][2 * st], qr.qa[hh][2 * st + 1]);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) b.w[i] = qr.w[i];
}

__device__ __forceinline__ float score_chunk_exact(const QueryRowB& qb, const KeyTile& kt) {
  RowAcc acc;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    v4f a0 = {0.f, 0.f, 0.f, 0.f};
    v4f a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const v8bf bk = fp8x8_to_bf16(kt.kb[t][2 * st], kt.kb[t][2 * st + 1]);
      a0 = mfma_bf16(qb.qb[0][st], bk, a0);
      a1 = mfma_bf16(qb.qb[1][st], bk, a1);
    }
    acc.a[t][0] = a0;
    acc.a[t][1] = a1;
  }
  return reduce_heads(qb, acc);
}

// B operands of up to 64 arbitrary keys read straight from global memory:
// lane l loads key idx[16t + l%16] of sub-tile t (bytes 32*(l/16) ..).
__device__ __forceinline__ void load_keys_gather(KeyTile& kt, const uint8_t* __restrict__ k,
                                                 const int* keyidx) {
  const int l = lane_id();
  const int g = l >> 4;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int64_t key = keyidx[t];
    const uint8_t* p = k + key * kDim + 32 * g;
    const uint4 x0 = *reinterpret_cast<const uint4*>(p);
    const uint4 x1 = *reinterpret_cast<const uint4*>(p + 16);
    kt.kb[t] = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                   (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
  }
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ int wave_max_i(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const int u = __shfl_xor(v, o, 64);
    v = u > v ? u : v;
  }
  return v;
}
__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = __builtin_fminf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
// Inclusive prefix sum over the wave's lanes.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int l = lane_id();
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o, 64);
    if (l >= o) v += t;
  }
  return v;
}

__device__ __forceinline__ int rank_in_mask(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
}

// ---------------------------------------------------------------------------
// One level of a wave-level radix select: hist[0..nb) holds the counts of the
// current digit among the records matching the prefix; find the digit of the
// `need`-th largest record. Returns the digit; `above` receives the number of
// records in higher digits and `cnt` the count of the chosen digit.
__device__ __forceinline__ int radix_digit(const uint32_t* hist, int nb, int need, int& above,
                                           int& cnt) {
  const int l = lane_id();
  const int per = nb / kWave;
  int mine = 0;
  for (int b = 0; b < per; ++b) mine += (int)hist[nb - 1 - (l * per + b)];
  const int incl = wave_incl_scan(mine);
  const int excl = incl - mine;
  const uint64_t hit = __ballot(incl >= need);
  const int src = hit ? __builtin_ctzll(hit) : 63;  // hit != 0: the total is >= need
  int digit = 0, ab = 0, ct = 0;
  if (l == src) {
    int c = excl;
    for (int b = 0; b < per; ++b) {
      const int bin = nb - 1 - (l * per + b);
      const int h = (int)hist[bin];
      if (c + h >= need) {
        digit = bin;
        ab = c;
        ct = h;
        break;
      }
      c += h;
    }
  }
  above = __shfl(ab, src, 64);
  cnt = __shfl(ct, src, 64);
  return __shfl(digit, src, 64);
}

// Histogram of one radix level over E[0..n) restricted to a prefix.
__device__ __forceinline__ void radix_hist(const float* __restrict__ E, int n, uint32_t prefix,
                                           uint32_t pmask, int sh, uint32_t dmask, int nb,
                                           uint32_t* hist) {
  const int l = lane_id();
  for (int b = l; b < nb; b += kWave) hist[b] = 0;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  for (int i = l; i < n; i += kWave) {
    const uint32_t key = fkey(E[i]);
    if ((key & pmask) == prefix) atomicAdd(&hist[(key >> sh) & dmask], 1u);
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// The rank-th largest of E[0..n) (1 <= rank <= n), exactly, by a three-level
// radix select (11, 11 and 10 bits of the order-preserving key).
__device__ float wave_kth_value(const float* __restrict__ E, int n, int rank, uint32_t* hist) {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  uint32_t prefix = 0, pmask = 0;
  int need = rank;
  const int shifts[3] = {21, 10, 0};
  const int widths[3] = {11, 11, 10};
  for (int lev = 0; lev < 3; ++lev) {
    const int sh = shifts[lev];
    const uint32_t dmask = (1u << widths[lev]) - 1u;
    const int nb = 1 << widths[lev];
    radix_hist(E, n, prefix, pmask, sh, dmask, nb, hist);
    int above, cnt;
    const int digit = radix_digit(hist, nb, need, above, cnt);
    need -= above;
    prefix |= (uint32_t)digit << sh;
    pmask |= dmask << sh;
    __builtin_amdgcn_wave_barrier();
  }
  return kfloat(prefix);
}

// ---------------------------------------------------------------------------
// The `need` best of nb <= 256 records (E, I)[0..nb) by exact comparison:
// record i takes slot rank(i) = #{j : E[j] > E[i] or (E[j] == E[i] and
// j < i)} when rank(i) < need. Lane l holds records l, l + 64, ... in
// registers; every record's score is broadcast once (readlane into a scalar)
// and compared with the lane's. Returns the smallest selected score.
template <class Emit>
__device__ float small_select(const float* __restrict__ E, const int* __restrict__ I, int nb,
                              int need, Emit emit) {
  const int l = lane_id();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  float v[4];
  int rank[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int i = kWave * s + l;
    v[s] = i < nb ? E[i] : 0.f;
    rank[s] = 0;
  }
#pragma unroll
  for (int s2 = 0; s2 < 4; ++s2) {
    const int cnt = nb - kWave * s2 < kWave ? nb - kWave * s2 : kWave;
    for (int jl = 0; jl < cnt; ++jl) {
      const float ej = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v[s2]), jl));
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if (kWave * s >= nb) break;
        // record j = 64 s2 + jl against record i = 64 s + l: j < i for s > s2,
        // j > i for s < s2, and jl < l for s == s2
        if (s > s2)
          rank[s] += ej >= v[s] ? 1 : 0;
        else if (s < s2)
          rank[s] += ej > v[s] ? 1 : 0;
        else
          rank[s] += (ej > v[s] || (ej == v[s] && jl < l)) ? 1 : 0;
      }
    }
  }
  float tau = __builtin_inff();
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int i = kWave * s + l;
    if (i < nb && rank[s] < need) {
      emit(rank[s], v[s], I[i]);
      tau = __builtin_fminf(tau, v[s]);
    }
  }
  return wave_min(tau);
}

// First bin b (scanning bins 0, 1, ... of hist[0..nb)) whose cumulative count
// reaches `need`; `before` receives the count of bins < b. Returns nb - 1 when
// the total is below `need`.
__device__ __forceinline__ int first_bin_reaching(const uint32_t* hist, int nb, int need,
                                                  int& before) {
  const int l = lane_id();
  const int per = nb / kWave;
  int mine = 0;
  for (int b = 0; b < per; ++b) mine += (int)hist[l * per + b];
  const int incl = wave_incl_scan(mine);
  const int excl = incl - mine;
  const uint64_t hit = __ballot(incl >= need);
  if (hit == 0) {
    before = __shfl(incl, 63, 64) - (int)hist[nb - 1];
    return nb - 1;
  }
  const int src = __builtin_ctzll(hit);
  int bin = nb - 1, bf = 0;
  if (l == src) {
    int c = excl;
    for (int b = 0; b < per; ++b) {
      const int h = (int)hist[l * per + b];
      if (c + h >= need) {
        bin = l * per + b;
        bf = c;
        break;
      }
      c += h;
    }
  }
  before = __shfl(bf, src, 64);
  return __shfl(bin, src, 64);
}

// ---------------------------------------------------------------------------
// Radix search of the wave-level selects below: the order-preserving key of
// the k-th best of E[0..n) (n > k) is found 11, 11 and 10 bits at a time in
// an LDS histogram of 2048 words private to the wave. On return the records
// whose key matches `prefix` under `pmask` are the ties of the k-th best
// (pmask stops short of all 32 bits when every record matching the prefix so
// far belongs to the best k), records above the prefix are all among the best
// k, and `need` of the ties complete them.
__device__ __forceinline__ void radix_search(const float* __restrict__ E, int n, int k,
                                             uint32_t* hist, uint32_t& prefix, uint32_t& pmask,
                                             int& need) {
  prefix = 0;
  pmask = 0;
  need = k;
  bool done = false;
  const int shifts[3] = {21, 10, 0};
  const int widths[3] = {11, 11, 10};
  for (int lev = 0; lev < 3 && !done; ++lev) {
    const int sh = shifts[lev];
    const uint32_t dmask = (1u << widths[lev]) - 1u;
    const int nb = 1 << widths[lev];
    radix_hist(E, n, prefix, pmask, sh, dmask, nb, hist);
    int above, cnt;
    const int digit = radix_digit(hist, nb, need, above, cnt);
    need -= above;
    prefix |= (uint32_t)digit << sh;
    pmask |= dmask << sh;
    if (cnt == need) done = true;
    __builtin_amdgcn_wave_barrier();
  }
}

// Wave-level exact top-k select over n (score, key) records held in global
// memory (E[i], I[i]), then one output pass. Records strictly above the
// selected prefix are all taken; records equal to it fill the remaining slots
// in slab order (any subset of ties at the k-th score is a correct answer).
// `emit(slot, score, key)` is called once per selected record with distinct
// slots in [0, min(n, k)). Returns the smallest selected score (or +inf when
// nothing is selected).
template <class Emit>
__device__ float wave_select(const float* __restrict__ E, const int* __restrict__ I, int n,
                             int k, uint32_t* hist, Emit emit) {
  const int l = lane_id();
  // the records were stored by this wave: make them visible to all its lanes
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  if (n <= k) {
    float mn = __builtin_inff();
    for (int i = l; i < n; i += kWave) {
      const float e = E[i];
      emit(i, e, I[i]);
      mn = __builtin_fminf(mn, e);
    }
    return wave_min(mn);
  }
  uint32_t prefix, pmask;
  int need;
  radix_search(E, n, k, hist, prefix, pmask, need);
  // output: strictly-above records fill slots [0, k - need), ties the rest
  const int n_above = k - need;
  int taken_above = 0, taken_tie = 0;
  float mn = __builtin_inff();
  for (int i0 = 0; i0 < n; i0 += kWave) {
    const int i = i0 + l;
    uint32_t key = 0;
    float e = 0.f;
    if (i < n) {
      e = E[i];
      key = fkey(e);
    }
    const bool in = i < n;
    const bool up = in && (key & pmask) > prefix;
    const bool tie = in && (key & pmask) == prefix;
    const uint64_t mu = __ballot(up);
    const uint64_t mt = __ballot(tie);
    if (up) {
      const int slot = taken_above + rank_in_mask(mu);
      if (slot < n_above) {
        emit(slot, e, I[i]);
        mn = __builtin_fminf(mn, e);
      }
    }
    if (tie) {
      const int rk = taken_tie + rank_in_mask(mt);
      if (rk < need) {
        emit(n_above + rk, e, I[i]);
        mn = __builtin_fminf(mn, e);
      }
    }
    taken_above += __popcll(mu);
    taken_tie += __popcll(mt);
  }
  return wave_min(mn);
}

// The k best of n records by (score descending, key ascending): every record
// scoring above the k-th best score tau, then the ties of tau with the
// smallest keys (keys are distinct and below 2^20). tau is found by
// wave_kth_value; the cut among the ties by a two-level radix select over the
// key bits (10 + 10) in the same LDS histogram. emit(slot, score, key) fills
// slots [0, min(n, k)): above-tau records first, then the ties. Returns tau
// (+inf when n == 0). Score comparisons are float comparisons (-0 == +0).
template <class Emit>
__device__ float wave_select_lowkey(const float* __restrict__ E, const int* __restrict__ I, int n,
                                    int k, uint32_t* hist, Emit emit) {
  const int l = lane_id();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  if (n <= k) {
    float mn = __builtin_inff();
    for (int i = l; i < n; i += kWave) {
      const float e = E[i];
      emit(i, e, I[i]);
      mn = __builtin_fminf(mn, e);
    }
    return wave_min(mn);
  }
  const float tau = wave_kth_value(E, n, k, hist);
  int gt = 0;
  for (int i = l; i < n; i += kWave) gt += E[i] > tau ? 1 : 0;
  gt = wave_sum(gt);
  // the need-th smallest key among the records scoring tau
  int rem = k - gt;
  uint32_t kpre = 0, kmask = 0;
  for (int lev = 0; lev < 2; ++lev) {
    const int sh = lev == 0 ? 10 : 0;
    constexpr uint32_t dmask = 1023u;
    constexpr int nb = 1024;
    for (int b = l; b < nb; b += kWave) hist[b] = 0;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    for (int i = l; i < n; i += kWave) {
      const uint32_t key = (uint32_t)I[i];
      if (E[i] == tau && (key & kmask) == kpre) atomicAdd(&hist[(key >> sh) & dmask], 1u);
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    int before;
    const int bin = first_bin_reaching(hist, nb, rem, before);
    rem -= before;
    kpre |= (uint32_t)bin << sh;
    kmask |= dmask << sh;
    __builtin_amdgcn_wave_barrier();
  }
  const uint32_t kcut = kpre;  // the last tie taken
  int taken_above = 0, taken_tie = 0;
  for (int i0 = 0; i0 < n; i0 += kWave) {
    const int i = i0 + l;
    const bool in = i < n;
    const float e = in ? E[i] : 0.f;
    const int key = in ? I[i] : 0;
    const bool up = in && e > tau;
    const bool tie = in && e == tau && (uint32_t)key <= kcut;
    const uint64_t mu = __ballot(up);
    const uint64_t mt = __ballot(tie);
    if (up) emit(taken_above + rank_in_mask(mu), e, key);
    if (tie) emit(gt + taken_tie + rank_in_mask(mt), e, key);
    taken_above += __popcll(mu);
    taken_tie += __popcll(mt);
  }
  return tau;
}

// The best k of n > k records as wave_select picks them, widened by every
// record tied with the k-th best while no more than `room` (>= k) records
// are taken in all. emit(slot, score, key) fills slots [0, taken); returns
// taken. `bound` receives a score that every record left out is at most
// (and every taken record beats): the best left-out score when all ties were
// taken, else the k-th best score itself (then exactly k are taken).
template <class Emit>
__device__ int wave_select_ties(const float* __restrict__ E, const int* __restrict__ I, int n,
                                int k, int room, uint32_t* hist, float& bound, Emit emit) {
  const int l = lane_id();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  uint32_t prefix, pmask;
  int need;
  radix_search(E, n, k, hist, prefix, pmask, need);
  const int n_above = k - need;
  const int tie_room = room - n_above;
  int taken_above = 0, taken_tie = 0;
  float below = -__builtin_inff();
  for (int i0 = 0; i0 < n; i0 += kWave) {
    const int i = i0 + l;
    uint32_t key = 0;
    float e = 0.f;
    if (i < n) {
      e = E[i];
      key = fkey(e);
    }
    const bool in = i < n;
    const bool up = in && (key & pmask) > prefix;
    const bool tie = in && (key & pmask) == prefix;
    const uint64_t mu = __ballot(up);
    const uint64_t mt = __ballot(tie);
    if (up) emit(taken_above + rank_in_mask(mu), e, I[i]);
    if (tie) {
      const int rk = taken_tie + rank_in_mask(mt);
      if (rk < tie_room) emit(n_above + rk, e, I[i]);
    }
    if (in && !up && !tie) below = __builtin_fmaxf(below, e);
    taken_above += __popcll(mu);
    taken_tie += __popcll(mt);
  }
  if (taken_tie <= tie_room) {
    bound = wave_max(below);
    return n_above + taken_tie;
  }
  // more ties than room: the prefix is the whole key of the k-th best score
  bound = kfloat(prefix);
  return k;
}

}  // namespace mqa
