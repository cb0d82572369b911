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
#include "common.h"
#include "launch.h"

namespace dsa {

constexpr int kIdxD = 128;       // indexer head dim
constexpr int kKeyStride = 256;  // LDS row of a staged bf16 key (bytes): 16 chunks of 16 bytes

// 16-byte chunk slot of chunk c of staged key `key` (a swizzle chosen by
// measuring LDS bank conflicts on gfx950: the operand reads below -- 16
// consecutive keys x 4 chunk groups per instruction -- are conflict-free).
__device__ __forceinline__ int kchunk(int key, int c) { return c ^ (((key & 3) << 2) | ((key >> 2) & 3)); }

// On entry lane (g, c) = (lane/16, lane%16) holds its partial for key
// 16*b + c of a 64-key group in p[b]; returns the sum over all four lane
// groups for key 16*g + c.
// The exchanges are VALU lane swaps: v_permlane32_swap(x, y) trades the upper
// half-wave of x with the lower half-wave of y, so after swapping (p0, p2)
// every lower lane holds (p0, partner p0) and every upper lane (partner p2,
// p2); v_permlane16_swap does the same between odd and even 16-lane rows.
__device__ __forceinline__ float group_transpose_reduce(float p0, float p1, float p2, float p3, int) {
  const auto s02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p2), false, false);
  const auto s13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p1), __float_as_uint(p3), false, false);
  const float a0 = __uint_as_float(s02[0]) + __uint_as_float(s02[1]);  // rows 0-1: keys of p0; rows 2-3: of p2
  const float a1 = __uint_as_float(s13[0]) + __uint_as_float(s13[1]);
  const auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(a0), __float_as_uint(a1), false, false);
  return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}

// A lane's 32 FP8 values (dims 32*g .. 32*g+31 of one vector) as the four
// bf16 k-steps of the MFMA: step s covers dims 32*g + 8*s .. +7.  A and B
// use the same dim <-> (lane group, step, slot) map, so the contraction
// covers all 128 dims.
struct Frag {
  v8bf s[4];
};

__device__ __forceinline__ Frag widen32(v4i lo, v4i hi) {
  Frag f;
  f.s[0] = e4m3x8_to_bf16(lo.x, lo.y);
  f.s[1] = e4m3x8_to_bf16(lo.z, lo.w);
  f.s[2] = e4m3x8_to_bf16(hi.x, hi.y);
  f.s[3] = e4m3x8_to_bf16(hi.z, hi.w);
  return f;
}

template <int NT>
__device__ __forceinline__ void load_query(const uint8_t* __restrict__ q_idx, const float* __restrict__ w,
                                           int64_t r, bool valid, int32_t H_I, int col, int grp, Frag (&a)[NT],
                                           float (&wr)[NT][4]) {
#pragma unroll
  for (int tl = 0; tl < NT; ++tl) {
    const int head = 16 * tl + col;
    if (valid && head < H_I) {
      const v4i* p = (const v4i*)(q_idx + ((r * H_I + head) * kIdxD + 32 * grp));
      a[tl] = widen32(p[0], p[1]);
    } else {
#pragma unroll
      for (int st = 0; st < 4; ++st) a[tl].s[st] = (v8bf){};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hw = 16 * tl + 4 * grp + i;
      wr[tl][i] = (valid && hw < H_I) ? 0.5f * w[r * H_I + hw] : 0.f;
    }
  }
}

// Weighted, rectified head sum of one query against one 16-key block.
// wr holds w/2: w * ReLU(c) = (|c| + c) * (w/2) exactly (the doubling and the
// halving are exact), which is one add with an abs source modifier plus one
// FMA per element -- fmaxf would cost an extra canonicalisation.  The 4*NT
// elements of a lane accumulate in two FMA chains.
template <int NT>
__device__ __forceinline__ float head_sum(const Frag (&a)[NT], const float (&wr)[NT][4], const Frag& b) {
  v4f c[NT];
#pragma unroll
  for (int tl = 0; tl < NT; ++tl) c[tl] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int st = 0; st < 4; ++st) {
#pragma unroll
    for (int tl = 0; tl < NT; ++tl) c[tl] = mfma_bf16_16x16x32(a[tl].s[st], b.s[st], c[tl]);
  }
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int tl = 0; tl < NT; ++tl) {
    s0 = fmaf(__builtin_fabsf(c[tl][0]) + c[tl][0], wr[tl][0], s0);
    s1 = fmaf(__builtin_fabsf(c[tl][1]) + c[tl][1], wr[tl][1], s1);
    s0 = fmaf(__builtin_fabsf(c[tl][2]) + c[tl][2], wr[tl][2], s0);
    s1 = fmaf(__builtin_fabsf(c[tl][3]) + c[tl][3], wr[tl][3], s1);
  }
  return s0 + s1;
}

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

  Frag a[NT];
  float wr[NT][4];
  load_query<NT>(q_idx, w, b, true, H_I, col, grp, a, wr);

  // groups of this wave: kg(i) = c0 + 64*wave + 256*i.  Lane i resolves the
  // row of group i up front (one page lookup per 64-key group, which always
  // lies in one page), so no key load waits on a lookup.
  const int64_t kg0 = c0 + 64 * wave;
  const int ng = kg0 < c_end ? (int)((c_end - kg0 + 255) / 256) : 0;
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
  if (ng > 0) load(0, ra);
  if (ng > 1) load(1, rb);
  for (int i = 0; i < ng; i += 3) {
    if (i + 2 < ng) load(i + 2, rc);
    finish(i, ra);
    if (i + 1 >= ng) break;
    if (i + 3 < ng) load(i + 3, ra);
    finish(i + 1, rb);
    if (i + 2 >= ng) break;
    if (i + 4 < ng) load(i + 4, rb);
    finish(i + 2, rc);
  }
}

// ---------------------------------------------------------------- launchers
namespace {
constexpr int kPrefillNW = 4;
constexpr int kPrefillQW = 1;
constexpr int kPrefillChunk = 8192;
constexpr int kDecodeChunk = 4096;  // keys per decode workgroup: 16 groups of 64 per wave

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

}  // namespace dsa
