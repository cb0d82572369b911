// Shared device helpers for the gfx950 DSA kernels: vector types, MFMA
// wrappers, key-row addressing (contiguous / batched / paged) and the
// order-preserving float -> uint32 key used by top-k.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef short v2s __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// D = A(16x128 fp8 e4m3) * B(128x16 fp8 e4m3) + C, unit scales.  Lane l
// supplies A row (l % 16) / B column (l % 16), 32 consecutive k values starting
// at 32 * (l / 16) (the same k set for A and B, so the contraction covers all
// 128 k).  C/D: lane l holds column l % 16, rows 4*(l/16) + i.  The sums are
// not fp32-accurate: products are truncated in groups of 8 k (see the FP8
// scoring pass in indexer.hip).
__device__ __forceinline__ v4f mfma_f8_16x16x128(v8i a, v8i b, v4f c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// D = A(16x32 bf16) * B(32x16 bf16) + C.  Lane l supplies A row (l % 16) /
// B column (l % 16), k values 8*(l/16) .. +7.  C/D: lane l holds column
// l % 16, rows 4*(l/16) + i.  Products are exact and the accumulation is
// fp32-accurate.
__device__ __forceinline__ v4f mfma_bf16_16x16x32(v8bf a, v8bf b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Widens 8 FP8 E4M3 values (two dwords) to bf16.  Every E4M3 value is
// exactly representable in bf16, so this is exact.
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
__device__ __forceinline__ v8bf e4m3x8_to_bf16(int lo, int hi) {
  const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return (v8bf){a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// D = A(32x16 bf16) * B(16x32 bf16) + C.  Lane l supplies A row (l % 32) and
// B column (l % 32), k values 8*(l/32) .. +7.  C/D: lane l holds column
// l % 32, rows 8*(r/4) + 4*(l/32) + (r%4) for r = 0..15.
__device__ __forceinline__ v16f mfma_bf16_32x32x16(v8bf a, v8bf b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------------------ addressing
// Row index (into a [rows, dim] array) of token s of sequence b, or -1 when
// the token has no backing row.
// group_row(b, g): row of token g of a 64-aligned group g .. g+63 whose tokens
// sit in consecutive rows (true for every layout here, pages being 64 tokens),
// or -1 when the group has no backing rows.
// Two-phase form of row(): lookup(b, s) issues the layout's loads with no
// branch (indexes clamped into range, valid for any s), row_of(b, s, look)
// finishes; several lookups can then be in flight together.
struct AddrSingle {  // one contiguous sequence of n rows
  int64_t n;
  __device__ __forceinline__ int64_t row(int64_t /*b*/, int64_t s) const { return (s >= 0 && s < n) ? s : -1; }
  __device__ __forceinline__ int64_t group_row(int64_t b, int64_t g) const { return row(b, g); }
  __device__ __forceinline__ int32_t lookup(int64_t, int64_t) const { return 0; }
  __device__ __forceinline__ int64_t row_of(int64_t b, int64_t s, int32_t) const { return row(b, s); }
};
struct AddrBatched {  // [B, stride] contiguous sequences
  int64_t stride;
  __device__ __forceinline__ int64_t row(int64_t b, int64_t s) const {
    return (s >= 0 && s < stride) ? b * stride + s : -1;
  }
  __device__ __forceinline__ int64_t group_row(int64_t b, int64_t g) const { return row(b, g); }
  __device__ __forceinline__ int32_t lookup(int64_t, int64_t) const { return 0; }
  __device__ __forceinline__ int64_t row_of(int64_t b, int64_t s, int32_t) const { return row(b, s); }
};
struct AddrPaged {  // pool of pages addressed through a page table
  const int32_t* page_table;
  int32_t max_pages;
  int32_t page_shift;  // log2(page_size)
  int64_t n_pages;
  __device__ __forceinline__ int64_t row(int64_t b, int64_t s) const {
    if (s < 0) return -1;
    int64_t lp = s >> page_shift;
    if (lp >= max_pages) return -1;
    int32_t p = page_table[b * max_pages + lp];
    if (p < 0 || p >= n_pages) return -1;
    return ((int64_t)p << page_shift) + (s & ((1 << page_shift) - 1));
  }
  __device__ __forceinline__ int64_t group_row(int64_t b, int64_t g) const { return row(b, g); }
  __device__ __forceinline__ int32_t lookup(int64_t b, int64_t s) const {
    const int64_t lp = s < 0 ? 0 : min(s >> page_shift, (int64_t)max_pages - 1);
    return page_table[b * max_pages + lp];
  }
  __device__ __forceinline__ int64_t row_of(int64_t /*b*/, int64_t s, int32_t p) const {
    if (s < 0 || (s >> page_shift) >= max_pages || p < 0 || p >= n_pages) return -1;
    return ((int64_t)p << page_shift) + (s & ((1 << page_shift) - 1));
  }
};

// ------------------------------------------------------------------ top-k keys
// Monotone map of fp32 to uint32: a > b (as floats) <=> key(a) > key(b);
// -0 is first canonicalised to +0 so the two compare equal.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, kWave); }

}  // namespace dsa
