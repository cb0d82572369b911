// Exact lightning-indexer arithmetic shared by the prefill and decode score
// kernels and by the fused prefill's top-k, which rescores the keys near each
// row's threshold with these same functions (so those scores are bit-identical
// to the score kernels' output).
//
// Index score ("DeepSeek-V3.2" report walk-through, §2.1.1, index-score
// equation): I[t, s] = sum_j w[t, j] * ReLU(q_I[t, j, :] . k_I[s, :]), FP8 E4M3
// inputs.  Each FP8 value is widened to bf16 (exact) and the head-by-key dot
// products run on the bf16 MFMA (exact products, fp32-accurate sums); heads
// sit on the MFMA rows, so a lane holds 4 heads of one key per 16-head tile.
// ReLU and the weight are fused into the accumulator epilogue and the sum
// over the four lane groups is a 4x4 transposing reduction, which leaves each
// lane one finished score of a 64-key group.  The score of a key does not
// depend on where in the group it sits: every key takes the same MFMA
// sequence, the same in-lane order over heads and the same ((g0 + g2) +
// (g1 + g3)) order over lane groups.
#pragma once
#include "common.h"

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

// Query row r (its H_I heads and weights) in the A layout of head_sum; heads
// past H_I, and every head when !valid, are zero.  All loads are issued
// unconditionally -- an invalid row reads row 0 (valid memory whenever a
// kernel runs) and a padding head reads head H_I-1 -- and zeroed by selects,
// so the NT query tiles and the weights are in flight together: one memory
// round trip rather than one per tile.
template <int NT>
__device__ __forceinline__ void load_query(const uint8_t* __restrict__ q_idx, const float* __restrict__ w,
                                           int64_t r, bool valid, int32_t H_I, int col, int grp, Frag (&a)[NT],
                                           float (&wr)[NT][4]) {
  const int64_t rr = valid ? r : 0;
  v4i lo[NT], hi[NT];
  float wv[NT][4];
#pragma unroll
  for (int tl = 0; tl < NT; ++tl) {
    const int head = min(16 * tl + col, H_I - 1);
    const v4i* p = (const v4i*)(q_idx + ((rr * H_I + head) * kIdxD + 32 * grp));
    lo[tl] = p[0];
    hi[tl] = p[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) wv[tl][i] = w[rr * H_I + min(16 * tl + 4 * grp + i, H_I - 1)];
  }
#pragma unroll
  for (int tl = 0; tl < NT; ++tl) {
    const bool hv = valid && 16 * tl + col < H_I;
    const v4i z = {0, 0, 0, 0};
    a[tl] = widen32(hv ? lo[tl] : z, hv ? hi[tl] : z);
#pragma unroll
    for (int i = 0; i < 4; ++i) wr[tl][i] = (valid && 16 * tl + 4 * grp + i < H_I) ? 0.5f * wv[tl][i] : 0.f;
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

}  // namespace dsa
