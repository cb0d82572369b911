// Lightning indexer on gfx950 matrix cores.
//
// Computes the index score of DeepSeek-V3.2's lightning indexer ("DeepSeek-
// V3.2" report walk-through, §2.1.1, index-score equation):
//   I[t, s] = sum_j w[t, j] * ReLU(q_I[t, j, :] . k_I[s, :])
// with FP8 E4M3 inputs (few heads, 128-dim keys: analysis article §1.2).
//
// Precision: gfx950's FP8 MFMA keeps only ~14 bits when it sums products
// (measured: errors up to 1e-4 of sum|products| per instruction), which is
// far from fp32.  The FP8 operands are therefore widened to bf16 in
// registers (exact: every E4M3 value is a bf16 value) and contracted on the
// bf16 MFMA, whose products are exact and whose sums are fp32-accurate.
//
// Mapping: the head-by-key dot products of one query are 16x32 by 32x16 bf16
// MFMAs per (16-head tile, 16-key block), four k-steps for d = 128; heads sit
// on the MFMA rows so a lane holds 4 heads of one key and the head sum is
// mostly in-lane.  ReLU and the w-weighting are fused into the accumulator
// epilogue (fp32), and the remaining sum over the four lane groups is a 4x4
// transposing reduction that leaves each lane with one finished score of a
// 64-key group, so stores are fully coalesced.  Keys are streamed (never the
// L x L matrix): the prefill kernel stages 64-key groups in LDS (widened to
// bf16 once per workgroup) and shares them across the workgroup's query
// rows; the decode kernel streams each key once from HBM.
#include <type_traits>

#include "common.h"
#include "indexer_exact.h"
#include "launch.h"

namespace dsa {

// ---------------------------------------------------------------- prefill
// Workgroup = NW waves x QW query rows, one key chunk of `key_chunk` keys.
// grid.x: query blocks of NW*QW rows; grid.y: key chunks.  Key s of the
// sequence is row addr.row(0, s) of k_idx (a contiguous sequence, or pages
// of a pool through one page-table row); a key without a backing row scores
// as a zero key.
template <int NW, int QW, int NT, class Addr>
__global__ __launch_bounds__(64 * NW, 1) void indexer_prefill_kernel(
    const uint8_t* __restrict__ q_idx, const float* __restrict__ w, const uint8_t* __restrict__ k_idx, Addr addr,
    int64_t T, int64_t N, int32_t H_I, int64_t q_pos0, float* __restrict__ scores, int64_t ld,
    int32_t key_chunk, int32_t fill_masked) {
  constexpr int QB = NW * QW;
  constexpr int kStageBytes = 64 * kIdxD / (64 * NW);  // FP8 bytes each thread stages per group
  static_assert(kStageBytes == 16 || kStageBytes == 32, "staging covers a 64-key group");
  __shared__ __attribute__((aligned(16))) uint8_t kbuf[2][64 * kKeyStride];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int64_t r0 = (int64_t)blockIdx.x * QB;
  if (r0 >= T) return;
  const int64_t r_last = min(r0 + QB, T) - 1;
  const int64_t n_comp_all = min(q_pos0 + r_last + 1, N);  // keys past this are masked for every row
  const int64_t c0 = (int64_t)blockIdx.y * key_chunk;
  const int64_t c_end = min(c0 + key_chunk, fill_masked ? N : n_comp_all);
  if (c0 >= c_end) return;
  const int64_t n_comp = min(c_end, n_comp_all);

  Frag a[QW][NT];
  float wr[QW][NT][4];
  int64_t nq[QW];
#pragma unroll
  for (int q = 0; q < QW; ++q) {
    const int64_t r = r0 + wave * QW + q;
    const bool valid = r < T;
    nq[q] = valid ? min(q_pos0 + r + 1, N) : 0;
    load_query<NT>(q_idx, w, r, valid, H_I, col, grp, a[q], wr[q]);
  }

  // staging: lane l of wave w moves FP8 bytes [32*(l/16), +32) of key
  // 16*w + l%16 of a 64-key group and stores them widened to bf16 (the same
  // shape as the operand reads, which keeps the LDS writes cheap)
  static_assert(NW == 4, "staging maps 256 threads onto 64 keys x 4 slices");
  const int st_key = 16 * wave + (lane & 15), st_off = kStageBytes * (lane >> 4);
  auto stage_load = [&](int64_t kg, v4i& s0, v4i& s1) {
    const int64_t s = kg + st_key;
    s0 = (v4i){0, 0, 0, 0};
    s1 = s0;
    const int64_t row = s < n_comp ? addr.row(0, s) : -1;
    if (row >= 0) {
      const v4i* p = (const v4i*)(k_idx + row * kIdxD + st_off);
      s0 = p[0];
      if (kStageBytes == 32) s1 = p[1];
    }
  };
  auto stage_store = [&](int bufi, v4i s0, v4i s1) {
    v8bf* row = (v8bf*)(&kbuf[bufi][st_key * kKeyStride]);
    const int c0 = st_off / 8;  // bf16 chunk of FP8 byte st_off
    row[kchunk(st_key, c0 + 0)] = e4m3x8_to_bf16(s0.x, s0.y);
    row[kchunk(st_key, c0 + 1)] = e4m3x8_to_bf16(s0.z, s0.w);
    row[kchunk(st_key, c0 + 2)] = e4m3x8_to_bf16(s1.x, s1.y);
    row[kchunk(st_key, c0 + 3)] = e4m3x8_to_bf16(s1.z, s1.w);
  };

  v4i s0, s1;
  stage_load(c0, s0, s1);
  int buf = 0;
  for (int64_t kg = c0; kg < c_end; kg += 64) {
    if (kg < n_comp) stage_store(buf, s0, s1);
    __syncthreads();
    if (kg + 64 < n_comp) stage_load(kg + 64, s0, s1);
    const int64_t s = kg + lane;
    if (kg < n_comp) {
      float part[QW][4];
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        // key 16*blk + col, chunks 4*grp + st (dims 32*grp + 8*st ..)
        const int key = 16 * blk + col;
        const v8bf* row = (const v8bf*)(&kbuf[buf][key * kKeyStride]);
        Frag b;
#pragma unroll
        for (int st = 0; st < 4; ++st) b.s[st] = row[kchunk(key, 4 * grp + st)];
#pragma unroll
        for (int q = 0; q < QW; ++q) part[q][blk] = head_sum<NT>(a[q], wr[q], b);
      }
#pragma unroll
      for (int q = 0; q < QW; ++q) {
        const float v = group_transpose_reduce(part[q][0], part[q][1], part[q][2], part[q][3], grp);
        const int64_t r = r0 + wave * QW + q;
        if (r < T && s < c_end) {
          if (s < nq[q])
            scores[r * ld + s] = v;
          else if (fill_masked)
            scores[r * ld + s] = -INFINITY;
        }
      }
    } else {
#pragma unroll
      for (int q = 0; q < QW; ++q) {
        const int64_t r = r0 + wave * QW + q;
        if (r < T && s < c_end) scores[r * ld + s] = -INFINITY;
      }
    }
    buf ^= 1;
  }
}

// ---------------------------------------------------------------- decode
// Workgroup = one query (sequence b = grid.y) and one chunk of `key_chunk`
// keys; the 4 waves take interleaved 64-key groups, loading each key once.
// The FP8 keys stream straight from HBM into registers, software pipelined:
// the row of group i+2 is resolved (one page lookup per 64-key group, which
// always lies in one page) and the keys of group i+1 are loaded while group
// i is on the matrix cores.
template <int NT, class Addr>
__global__ __launch_bounds__(256) void indexer_decode_kernel(const uint8_t* __restrict__ q_idx,
                                                             const float* __restrict__ w,
                                                             const uint8_t* __restrict__ keys, Addr addr,
                                                             const int32_t* __restrict__ ctx_len,
                                                             int64_t max_ctx, int32_t H_I,
                                                             float* __restrict__ scores, int64_t ld,
                                                             int32_t key_chunk) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int64_t b = blockIdx.y;
  const int64_t c0 = (int64_t)blockIdx.x * key_chunk;
  const int64_t c_end = min(c0 + key_chunk, max_ctx);
  if (c0 >= c_end) return;
  int64_t n = ctx_len[b];
  n = n < 0 ? 0 : (n > max_ctx ? max_ctx : n);
  if (c0 >= n) {  // the whole chunk lies past the context: only the -inf fill
    for (int64_t s = c0 + tid; s < c_end; s += 256) scores[b * ld + s] = -INFINITY;
    return;
  }

  Frag a[NT];
  float wr[NT][4];
  load_query<NT>(q_idx, w, b, true, H_I, col, grp, a, wr);

  // groups of this wave: kg(i) = c0 + 64*wave + 256*i, the first nv of them
  // holding keys of the context.  Lane i resolves the row of group i up
  // front (one page lookup per 64-key group, which always lies in one page),
  // so no key load waits on a lookup.
  const int64_t kg0 = c0 + 64 * wave;
  const int ng = kg0 < c_end ? (int)((c_end - kg0 + 255) / 256) : 0;
  const int nv = kg0 < n ? min(ng, (int)((n - kg0 + 255) / 256)) : 0;
  auto kg_of = [&](int i) { return kg0 + 256 * (int64_t)i; };
  int64_t my_base = -1;
  if (lane < ng && kg_of(lane) < n) my_base = addr.group_row(b, kg_of(lane));
  auto base_of = [&](int i) -> int64_t {
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)my_base, i);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)((uint64_t)my_base >> 32), i);
    return (int64_t)(((uint64_t)hi << 32) | lo);
  };
  // Unpredicated loads: keys past the context re-read the group's last valid
  // key (same page), and a group without a row reads row 0; their scores
  // are masked in finish().
  auto load = [&](int i, v4i (&raw)[4][2]) {
    const int64_t base = base_of(i);
    const int64_t last = n - 1 - kg_of(i);  // >= 0 whenever base >= 0
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
      const int64_t j = 16 * blk + col;
      const int64_t r = base >= 0 ? base + (j < last ? j : last) : 0;
      const v4i* p = (const v4i*)(keys + r * kIdxD + 32 * grp);
      raw[blk][0] = p[0];
      raw[blk][1] = p[1];
    }
  };
  auto finish = [&](int i, const v4i (&raw)[4][2]) {
    const int64_t s = kg_of(i) + lane;
    float part[4];
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) part[blk] = head_sum<NT>(a, wr, widen32(raw[blk][0], raw[blk][1]));
    const float v = group_transpose_reduce(part[0], part[1], part[2], part[3], grp);
    if (s < c_end) scores[b * ld + s] = (s < n && base_of(i) >= 0) ? v : -INFINITY;
  };

  // keys of the next two groups in flight while one group is on the matrix cores
  v4i ra[4][2], rb[4][2], rc[4][2];
  if (nv > 0) load(0, ra);
  if (nv > 1) load(1, rb);
  for (int i = 0; i < nv; i += 3) {
    if (i + 2 < nv) load(i + 2, rc);
    finish(i, ra);
    if (i + 1 >= nv) break;
    if (i + 3 < nv) load(i + 3, ra);
    finish(i + 1, rb);
    if (i + 2 >= nv) break;
    if (i + 4 < nv) load(i + 4, rb);
    finish(i + 2, rc);
  }
  for (int i = nv; i < ng; ++i) {  // groups past the context
    const int64_t s = kg_of(i) + lane;
    if (s < c_end) scores[b * ld + s] = -INFINITY;
  }
}

// ---------------------------------------------------------------- FP8 scoring pass
// The fused prefill first scores every causal pair on the FP8 matrix cores and
// keeps those approximate scores only to decide which keys need an exact score:
// its top-k (topk.hip) rescores, with the exact arithmetic above, every key
// whose approximate score lies within the error bound below of the row's
// threshold, so the selection is the one the exact scores give.
//
// Approximate score: c~[j, s] = q_I[t, j] . k_I[s] on the 16x16x128 FP8 MFMA
// (E4M3 operands as stored, unit scales); R = ReLU(c~) rounded toward zero to
// f16; I~[s] = sum_j f16(w_j) R[j, s] on the 16x16x32 f16 MFMA (fp32 sums).
//
// Error bound (|I~ - I| for the exact-route score I), from the FP8 MFMA's
// accumulation as measured on gfx950: the 128 products of a dot product are
// summed in 16 groups of 8 consecutive dims; inside a group every product is
// truncated toward zero at 13 bits below 2^e_ref, e_ref = the largest
// exponent-field sum E(q) + E(k) over the group (subnormals and zero count as
// E = -6), the truncated products are summed exactly, and the group sums are
// added in fp32.  So with MQ[j, g] and MK[s, g] the powers of two of the
// largest exponent field in group g of q_I[t, j] and of k_I[s],
//   |c~ - c| < 8 * 2^-13 * sum_g MQ[j, g] MK[s, g] (1 + 2^-5)
// (the fp32 additions included).  ReLU does not increase the error; the f16
// rounding of R (toward zero) and of w (to nearest) add at most
// (2^-10 + 2^-11)(1 + 2^-20) of sum_j w_j R_j, which the f16 MFMA's fp32 sums
// keep below 2^-9 I~; the exact route's own fp32 rounding (at most 2^-18 of
// sum_j |w_j| sum_i |q k|, and |q k| < 4 MQ MK) is below 2^-3 of the first term.  With W[g] = sum_j |w_j| MQ[j, g] and S[s] = sum_g MK[s, g]:
//   |I~[s] - I[s]| <= fac * S[s] + 1.0625 2^-9 I~[s] + eps,
//   fac = 1.25 * 2^-10 * max_g W[g],  eps = the f16 underflow terms.
// The stored score is f16(I~ * 2^-s), s chosen per row so that the row's
// largest possible |I~| fits f16's range.
// Rows with a negative or non-finite weight, or whose dot products could pass
// f16's range, are flagged and take the exact route whole.

// Largest exponent field (as 2^E, E >= -6) among the four E4M3 bytes of x.
__device__ __forceinline__ uint32_t max_exp_field(uint32_t x) {
  const uint32_t e0 = (x >> 3) & 15, e1 = (x >> 11) & 15, e2 = (x >> 19) & 15, e3 = (x >> 27) & 15;
  return max(max(e0, e1), max(e2, e3));
}
__device__ __forceinline__ float exp_field_pow2(uint32_t e) {  // 2^(max(e, 1) - 7)
  return __uint_as_float((max(e, 1u) - 7u + 127u) << 23);
}
// |E4M3 value|, exact in fp32
__device__ __forceinline__ float e4m3_abs(uint32_t b) {
  const uint32_t e = (b >> 3) & 15, m = b & 7;
  return e == 0 ? (float)m * 0x1p-9f : (float)(8 + m) * __uint_as_float((e - 10u + 127u) << 23);
}

// One thread per key: S[s], and over all keys the largest S and the largest
// |k_I| (as float bits; positive floats order like their bit patterns).  Key
// s is row addr.row(0, s) of k_idx; a key without a backing row is a zero key.
template <class Addr>
__global__ __launch_bounds__(256) void fp8_key_bounds_kernel(const uint8_t* __restrict__ k_idx, Addr addr, int64_t N,
                                                             float* __restrict__ key_s, uint32_t* __restrict__ glob) {
  const int64_t s = (int64_t)blockIdx.x * 256 + threadIdx.x;
  float S = 0.f;
  uint32_t kmax = 0;
  if (s < N) {
    const int64_t row = addr.row(0, s);
    const v4i* p = (const v4i*)(k_idx + (row < 0 ? 0 : row) * kIdxD);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const v4i z = {0, 0, 0, 0};
      const v4i v = row < 0 ? z : p[c];
      S += exp_field_pow2(max(max_exp_field(v.x), max_exp_field(v.y)));
      S += exp_field_pow2(max(max_exp_field(v.z), max_exp_field(v.w)));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t x = (uint32_t)v[i];
#pragma unroll
        for (int b = 0; b < 4; ++b) kmax = max(kmax, (x >> (8 * b)) & 0x7Fu);
      }
    }
    key_s[s] = S;
  }
  // a NaN code (S.1111.111) anywhere among the keys makes the largest |k_I|
  // infinite, which sends every row of the call down the exact route
  uint32_t sb = __float_as_uint(S), kb = __float_as_uint(kmax == 0x7Fu ? INFINITY : e4m3_abs(kmax));
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    sb = max(sb, (uint32_t)__shfl_xor((int)sb, d, 64));
    kb = max(kb, (uint32_t)__shfl_xor((int)kb, d, 64));
  }
  if ((threadIdx.x & 63) == 0) {
    atomicMax(&glob[0], sb);
    atomicMax(&glob[1], kb);
  }
}

// One wave per query row, lane j = head j: fac, eps and the exact-route flag
// of the row (see the FP8 scoring pass comment).
__global__ __launch_bounds__(256) void fp8_row_bounds_kernel(const uint8_t* __restrict__ q_idx,
                                                             const float* __restrict__ w, int64_t T, int32_t H_I,
                                                             const uint32_t* __restrict__ glob,
                                                             float* __restrict__ row_fac, float* __restrict__ row_eps,
                                                             int32_t* __restrict__ row_flag,
                                                             float* __restrict__ row_scale) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float kmax = __uint_as_float(glob[1]);
  float mq[16];
  float sum_abs = 0.f, wj = 0.f;
  bool bad = false;
  if (lane < H_I) {
    wj = w[t * H_I + lane];
    bad = !(wj >= 0.f && wj <= 65504.f);
    const v4i* p = (const v4i*)(q_idx + (t * H_I + lane) * kIdxD);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const v4i v = p[c];
      mq[2 * c] = exp_field_pow2(max(max_exp_field(v.x), max_exp_field(v.y)));
      mq[2 * c + 1] = exp_field_pow2(max(max_exp_field(v.z), max_exp_field(v.w)));
#pragma unroll
      for (int i = 0; i < 4; ++i) {  // exact conversions, two values each; a NaN code gives NaN
        const v2f lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(v[i], 1.0f, false);
        const v2f hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(v[i], 1.0f, true);
        sum_abs += (__builtin_fabsf(lo[0]) + __builtin_fabsf(lo[1])) + (__builtin_fabsf(hi[0]) + __builtin_fabsf(hi[1]));
      }
    }
  } else {
#pragma unroll
    for (int g = 0; g < 16; ++g) mq[g] = 0.f;
  }
  const float aw = bad ? 0.f : wj;
  const float cmax = sum_abs * kmax;  // bound on |c| and |c~| of this head (NaN codes: NaN)
  bad = bad || !(cmax <= 60000.f);
  // f16 underflow: a weight below 2^-14 may flush to zero (error w |c|), and
  // a rectified dot product below 2^-14 likewise (error 2^-14 w)
  float eps = (aw < 0x1p-14f ? aw * cmax : 0.f) + 0x1p-14f * aw;
  float imax = aw * cmax;  // bound on the row's |I~|
  // W[g] = sum over heads of aw * mq[g] for the 16 groups, then their max:
  // a transposed reduction -- each exchange halves the groups a lane keeps
  // (lane bit 5 picks groups 8..15, bit 4 the upper four of those, ...) --
  // leaves W[8 b5 + 4 b4 + 2 b3 + b2] summed over the other lane bits
  float x[16];
#pragma unroll
  for (int g = 0; g < 16; ++g) x[g] = aw * mq[g];
#pragma unroll
  for (int half = 8, d = 32; half >= 1; half >>= 1, d >>= 1) {
    const bool up = (lane & d) != 0;
#pragma unroll
    for (int i = 0; i < half; ++i) {
      const float keep = up ? x[i + half] : x[i];
      const float give = up ? x[i] : x[i + half];
      x[i] = keep + __shfl_xor(give, d, 64);
    }
  }
  float wsum = x[0];
  wsum += __shfl_xor(wsum, 2, 64);
  wsum += __shfl_xor(wsum, 1, 64);
  float wmax = wsum;
#pragma unroll
  for (int d = 4; d <= 32; d <<= 1) wmax = fmaxf(wmax, __shfl_xor(wmax, d, 64));
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    eps += __shfl_xor(eps, d, 64);
    imax += __shfl_xor(imax, d, 64);
  }
  const bool any_bad = __any(bad);
  if (lane == 0) {
    // the stored score is I~ * 2^-s in f16: the smallest s >= 0 that keeps the
    // row's largest possible |I~| below 60000 after scaling; rounding it to
    // f16 (to nearest) adds 2^-11 |I~| (in the relative term) and at most
    // 2^(s - 25) in f16's subnormal range
    int sc = 0;
    const float lim = imax * (1.f + 0x1p-8f);
    while (sc < 120 && ldexpf(lim, -sc) > 60000.f) ++sc;
    row_scale[t] = ldexpf(1.f, sc);
    row_fac[t] = 1.25f * 0x1p-10f * wmax * (1.f + 0x1p-16f);
    row_eps[t] = (eps + ldexpf(1.f, sc - 24) + 0x1p-20f) * (1.f + 0x1p-16f);
    row_flag[t] = any_bad ? 1 : 0;
  }
}

// Approximate scores of the causal pairs of a 4-row query block (one row per
// wave) over one chunk of `key_chunk` keys; the candidates (s <= pos) are
// written, as f16 I~ * 2^-s (row_scale = 2^s, rounded to nearest) in the
// first half of each fp32 row of the tile (with up to three slots past the
// last candidate, inside the row, that nothing reads).  64-key groups of FP8 keys are staged in LDS as stored (128-byte
// rows whose 16-byte chunks are XOR-swizzled by key, so the operand reads of
// 16 keys x one chunk are free of bank conflicts) and shared by the 4 rows.
// Per 16-key block: one 16x16x128 FP8 MFMA per 16-head tile (heads on the
// rows, keys on the columns), R packed to f16 pairs, then the head sum as
// 16x16x32 f16 MFMAs with R as the A operand (keys on the rows, the lane's 8
// heads of two tiles on the k dim) and the weights as the B operand, placed
// in column b for block b: the four blocks accumulate into one 16x16 result
// whose column b holds block b's scores, so lane (g, b) ends with the scores of
// keys 16 b + 4 g .. +3 and stores them as one 16-byte write.
template <int NT, class Addr>
__global__ __launch_bounds__(256) void indexer_fp8_prefill_kernel(
    const uint8_t* __restrict__ q_idx, const float* __restrict__ w, const uint8_t* __restrict__ k_idx, Addr addr,
    int64_t T, int64_t N, int32_t H_I, int64_t q_pos0, const float* __restrict__ row_scale,
    float* __restrict__ scores, int64_t ld, int32_t key_chunk) {
  constexpr int NS = (NT + 1) / 2;  // f16 k-steps of the head sum, two head tiles each
  __shared__ __attribute__((aligned(16))) uint8_t kbuf[2][64 * kIdxD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int64_t r0 = (int64_t)blockIdx.x * 4;
  if (r0 >= T) return;
  const int64_t r_last = min(r0 + 4, T) - 1;
  const int64_t n_comp = min(q_pos0 + r_last + 1, N);  // keys past this are no row's candidates
  const int64_t c0 = (int64_t)blockIdx.y * key_chunk;
  const int64_t c_end = min(c0 + key_chunk, n_comp);
  if (c0 >= c_end) return;
  const int64_t r = r0 + wave;
  const bool valid = r < T;
  const int64_t nq = valid ? min(q_pos0 + r + 1, N) : 0;
  const float inv_scale = valid ? 1.f / row_scale[r] : 1.f;  // a power of two: exact

  v8i a[NT];
#pragma unroll
  for (int tl = 0; tl < NT; ++tl) {
    const int head = 16 * tl + col;
    a[tl] = (valid && head < H_I) ? *(const v8i*)(q_idx + ((r * H_I + head) * kIdxD + 32 * grp)) : (v8i){};
  }
  // B operands of the head sum: step st, k-slot 8 grp + e holds head
  // 16 (2 st + e / 4) + 4 grp + e % 4 (the rows this lane holds of tiles 2 st
  // and 2 st + 1); block b's operand has the weights in column b only.
  v8h wb[4][NS];
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    v8h wv;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int head = 16 * (2 * st + e / 4) + 4 * grp + (e & 3);
      wv[e] = (valid && head < H_I) ? (_Float16)w[r * H_I + head] : (_Float16)0.f;
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) wb[b][st] = col == b ? wv : (v8h){};
  }

  const int st_key = 16 * wave + col;
  auto slot = [](int key, int ch) { return ch ^ ((key >> 1) & 7); };
  // key s of the sequence is row addr.row(0, s); a 64-key group lies in one
  // page, so one lookup per group (a group without a backing row stages zeros).
  // Contiguous keys load unpredicated: a key past c_end (only in the chunk's
  // last group) re-reads key c_end - 1, and its score is never read.
  auto stage_load = [&](int64_t kg, v4i& s0, v4i& s1) {
    const int64_t s = kg + st_key;
    if constexpr (std::is_same_v<Addr, AddrSingle>) {
      const v4i* p = (const v4i*)(k_idx + (s < c_end ? s : c_end - 1) * kIdxD + 32 * grp);
      s0 = p[0];
      s1 = p[1];
      return;
    }
    const int64_t grow = addr.group_row(0, kg);
    if (s < c_end && grow >= 0) {
      const v4i* p = (const v4i*)(k_idx + (grow + st_key) * kIdxD + 32 * grp);
      s0 = p[0];
      s1 = p[1];
    } else {
      s0 = (v4i){0, 0, 0, 0};
      s1 = s0;
    }
  };
  auto stage_store = [&](int bi, v4i s0, v4i s1) {
    v4i* row = (v4i*)(&kbuf[bi][st_key * kIdxD]);
    row[slot(st_key, 2 * grp)] = s0;
    row[slot(st_key, 2 * grp + 1)] = s1;
  };
  auto relu_pk = [](float x, float y) -> uint32_t {
    // f16 pair rounded toward zero; ReLU as a signed 16-bit max with 0 (a
    // negative f16, -0 included, has its sign bit set)
    const auto h = __builtin_amdgcn_cvt_pkrtz(x, y);
    const v2s v = __builtin_elementwise_max(__builtin_bit_cast(v2s, h), (v2s){0, 0});
    return __builtin_bit_cast(uint32_t, v);
  };

  v4i s0, s1;
  stage_load(c0, s0, s1);
  int buf = 0;
  for (int64_t kg = c0; kg < c_end; kg += 64) {
    stage_store(buf, s0, s1);
    __syncthreads();
    if (kg + 64 < c_end) stage_load(kg + 64, s0, s1);
    v4f d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int key = 16 * b + col;
      const v4i* row = (const v4i*)(&kbuf[buf][key * kIdxD]);
      const v4i lo = row[slot(key, 2 * grp)], hi = row[slot(key, 2 * grp + 1)];
      const v8i bk = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      v4f c[NT];
#pragma unroll
      for (int tl = 0; tl < NT; ++tl) c[tl] = mfma_f8_16x16x128(a[tl], bk, (v4f){0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        const int t0 = 2 * st, t1 = 2 * st + 1;
        v4i ra;
        ra.x = (int)relu_pk(c[t0][0], c[t0][1]);
        ra.y = (int)relu_pk(c[t0][2], c[t0][3]);
        ra.z = t1 < NT ? (int)relu_pk(c[t1 < NT ? t1 : t0][0], c[t1 < NT ? t1 : t0][1]) : 0;
        ra.w = t1 < NT ? (int)relu_pk(c[t1 < NT ? t1 : t0][2], c[t1 < NT ? t1 : t0][3]) : 0;
        d = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, ra), wb[b][st], d, 0, 0, 0);
      }
    }
    if (valid && col < 4) {
      const int64_t s = kg + 16 * col + 4 * grp;
      _Float16* dst = reinterpret_cast<_Float16*>(scores + r * ld) + s;
      const _Float16 h0 = (_Float16)(d[0] * inv_scale), h1 = (_Float16)(d[1] * inv_scale);
      const _Float16 h2 = (_Float16)(d[2] * inv_scale), h3 = (_Float16)(d[3] * inv_scale);
      // a group of four that crosses the row's last candidate is stored
      // whole: the slots past it lie inside the row's stride and are never read
      if (s < nq) *(v4h*)dst = (v4h){h0, h1, h2, h3};
    }
    buf ^= 1;
  }
}

// ---------------------------------------------------------------- launchers
namespace {
constexpr int kPrefillNW = 4;
constexpr int kPrefillQW = 1;
constexpr int kPrefillChunk = 8192;
// keys per decode workgroup (8 groups of 64 per wave): measured on MI355X, 2048 balances
// ragged contexts (32 sequences of 5.8K..127K keys: 77 us against 90 us with 4096) at
// about the same time for uniform ones (64 x 32K: 66 us against 64 us)
constexpr int kDecodeChunk = 2048;

template <int NT, class Addr>
hipError_t prefill_nt(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, Addr addr, int64_t T, int64_t N,
                      int32_t H_I, int64_t q_pos0, float* scores, int64_t ld, bool fill, hipStream_t st) {
  constexpr int QB = kPrefillNW * kPrefillQW;
  const int64_t n_all = fill ? N : std::min<int64_t>(q_pos0 + T, N);
  dim3 grid((unsigned)((T + QB - 1) / QB), (unsigned)((n_all + kPrefillChunk - 1) / kPrefillChunk));
  if (grid.x == 0 || grid.y == 0) return hipSuccess;
  hipLaunchKernelGGL((indexer_prefill_kernel<kPrefillNW, kPrefillQW, NT, Addr>), grid, dim3(64 * kPrefillNW), 0, st,
                     q_idx, w, k_idx, addr, T, N, H_I, q_pos0, scores, ld, kPrefillChunk, fill ? 1 : 0);
  return hipGetLastError();
}

template <class Addr>
hipError_t prefill_dispatch(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, Addr addr, int64_t T,
                            int64_t N, int32_t H_I, int64_t q_pos0, float* scores, int64_t ld, bool fill,
                            hipStream_t st) {
  switch ((H_I + 15) / 16) {
    case 1: return prefill_nt<1>(q_idx, w, k_idx, addr, T, N, H_I, q_pos0, scores, ld, fill, st);
    case 2: return prefill_nt<2>(q_idx, w, k_idx, addr, T, N, H_I, q_pos0, scores, ld, fill, st);
    case 3: return prefill_nt<3>(q_idx, w, k_idx, addr, T, N, H_I, q_pos0, scores, ld, fill, st);
    default: return prefill_nt<4>(q_idx, w, k_idx, addr, T, N, H_I, q_pos0, scores, ld, fill, st);
  }
}

template <int NT, class Addr>
hipError_t decode_nt(const uint8_t* q_idx, const float* w, const uint8_t* keys, Addr addr,
                     const int32_t* ctx_len, int64_t B, int64_t max_ctx, int32_t H_I, float* scores, int64_t ld,
                     hipStream_t st) {
  dim3 grid((unsigned)((max_ctx + kDecodeChunk - 1) / kDecodeChunk), (unsigned)B);
  if (grid.x == 0 || grid.y == 0) return hipSuccess;
  hipLaunchKernelGGL((indexer_decode_kernel<NT, Addr>), grid, dim3(256), 0, st, q_idx, w, keys, addr, ctx_len,
                     max_ctx, H_I, scores, ld, kDecodeChunk);
  return hipGetLastError();
}

template <class Addr>
hipError_t decode_dispatch(const uint8_t* q_idx, const float* w, const uint8_t* keys, Addr addr,
                           const int32_t* ctx_len, int64_t B, int64_t max_ctx, int32_t H_I, float* scores,
                           int64_t ld, hipStream_t st) {
  const int nt = (H_I + 15) / 16;
  switch (nt) {
    case 1: return decode_nt<1>(q_idx, w, keys, addr, ctx_len, B, max_ctx, H_I, scores, ld, st);
    case 2: return decode_nt<2>(q_idx, w, keys, addr, ctx_len, B, max_ctx, H_I, scores, ld, st);
    case 3: return decode_nt<3>(q_idx, w, keys, addr, ctx_len, B, max_ctx, H_I, scores, ld, st);
    default: return decode_nt<4>(q_idx, w, keys, addr, ctx_len, B, max_ctx, H_I, scores, ld, st);
  }
}
}  // namespace

hipError_t launch_indexer_prefill(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, int64_t T,
                                  int64_t N, int32_t H_I, int64_t q_pos0, float* scores, int64_t ld,
                                  bool fill_masked, const PagedArgs* paged, hipStream_t st) {
  if (paged) {
    AddrPaged ad{paged->page_table, paged->max_pages, __builtin_ctz((unsigned)paged->page_size), paged->n_pages};
    return prefill_dispatch(q_idx, w, k_idx, ad, T, N, H_I, q_pos0, scores, ld, fill_masked, st);
  }
  return prefill_dispatch(q_idx, w, k_idx, AddrSingle{N}, T, N, H_I, q_pos0, scores, ld, fill_masked, st);
}

hipError_t launch_indexer_decode(const uint8_t* q_idx, const float* w, const uint8_t* keys, int64_t stride,
                                 const PagedArgs* paged, const int32_t* ctx_len, int64_t B, int64_t max_ctx,
                                 int32_t H_I, float* scores, int64_t ld, hipStream_t st) {
  if (paged) {
    AddrPaged ad{paged->page_table, paged->max_pages, __builtin_ctz((unsigned)paged->page_size),
                 paged->n_pages};
    return decode_dispatch(q_idx, w, keys, ad, ctx_len, B, max_ctx, H_I, scores, ld, st);
  }
  AddrBatched ad{stride};
  return decode_dispatch(q_idx, w, keys, ad, ctx_len, B, max_ctx, H_I, scores, ld, st);
}

hipError_t launch_fp8_bounds(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, int64_t T, int64_t N,
                             int32_t H_I, float* key_s, uint32_t* glob, float* row_fac, float* row_eps,
                             int32_t* row_flag, float* row_scale, const PagedArgs* paged, hipStream_t st) {
  hipError_t e = launch_zero_f32(reinterpret_cast<float*>(glob), 2, st);
  if (e != hipSuccess) return e;
  const dim3 kgrid((unsigned)((N + 255) / 256));
  if (paged) {
    const AddrPaged ad{paged->page_table, paged->max_pages, __builtin_ctz((unsigned)paged->page_size),
                       paged->n_pages};
    hipLaunchKernelGGL(fp8_key_bounds_kernel<AddrPaged>, kgrid, dim3(256), 0, st, k_idx, ad, N, key_s, glob);
  } else {
    hipLaunchKernelGGL(fp8_key_bounds_kernel<AddrSingle>, kgrid, dim3(256), 0, st, k_idx, AddrSingle{N}, N, key_s,
                       glob);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(fp8_row_bounds_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, st, q_idx, w, T, H_I, glob,
                     row_fac, row_eps, row_flag, row_scale);
  return hipGetLastError();
}

namespace {
template <int NT, class Addr>
hipError_t fp8_prefill_nt(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, Addr addr, int64_t T, int64_t N,
                          int32_t H_I, int64_t q_pos0, const float* row_scale, float* scores, int64_t ld,
                          hipStream_t st) {
  const int64_t n_all = std::min<int64_t>(q_pos0 + T, N);
  dim3 grid((unsigned)((T + 3) / 4), (unsigned)((n_all + kPrefillChunk - 1) / kPrefillChunk));
  if (grid.x == 0 || grid.y == 0) return hipSuccess;
  hipLaunchKernelGGL((indexer_fp8_prefill_kernel<NT, Addr>), grid, dim3(256), 0, st, q_idx, w, k_idx, addr, T, N,
                     H_I, q_pos0, row_scale, scores, ld, kPrefillChunk);
  return hipGetLastError();
}

template <class Addr>
hipError_t fp8_prefill_dispatch(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, Addr addr, int64_t T,
                                int64_t N, int32_t H_I, int64_t q_pos0, const float* row_scale, float* scores,
                                int64_t ld, hipStream_t st) {
  switch ((H_I + 15) / 16) {
    case 1: return fp8_prefill_nt<1>(q_idx, w, k_idx, addr, T, N, H_I, q_pos0, row_scale, scores, ld, st);
    case 2: return fp8_prefill_nt<2>(q_idx, w, k_idx, addr, T, N, H_I, q_pos0, row_scale, scores, ld, st);
    case 3: return fp8_prefill_nt<3>(q_idx, w, k_idx, addr, T, N, H_I, q_pos0, row_scale, scores, ld, st);
    default: return fp8_prefill_nt<4>(q_idx, w, k_idx, addr, T, N, H_I, q_pos0, row_scale, scores, ld, st);
  }
}
}  // namespace

hipError_t launch_indexer_fp8_prefill(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, int64_t T,
                                      int64_t N, int32_t H_I, int64_t q_pos0, const float* row_scale, float* scores,
                                      int64_t ld, const PagedArgs* paged, hipStream_t st) {
  if (paged) {
    const AddrPaged ad{paged->page_table, paged->max_pages, __builtin_ctz((unsigned)paged->page_size),
                       paged->n_pages};
    return fp8_prefill_dispatch(q_idx, w, k_idx, ad, T, N, H_I, q_pos0, row_scale, scores, ld, st);
  }
  return fp8_prefill_dispatch(q_idx, w, k_idx, AddrSingle{N}, T, N, H_I, q_pos0, row_scale, scores, ld, st);
}

}  // namespace dsa
