// Indexer KL loss of DeepSeek-V3.2's sparse training stage on gfx950.
//
// "DeepSeek-V3.2" report walk-through §2.3.2: with the selected set S_t of
// query t fixed, the indexer is trained with
//   L^I = sum_t KL( p_{t,S_t} || Softmax(I_{t,S_t}) ),
// where the target p_{t,:} is built as in §2.3.1: the main attention scores
// of all heads are summed and L1-normalised along the sequence.  Here the
// attention scores are each head's softmax over S_t, so with lse_h the
// attention's log-sum-exp of head h:
//   P_h(s) = exp(scale * q_h . kv_s - lse_h),   p(s) = (1/H) sum_h P_h(s),
//   KL_t   = sum_s p(s) ln p(s) - sum_s p(s) I(s) + LSE_I * sum_s p(s),
// LSE_I = ln sum_{s in S_t} exp(I(s)).  (sum_s p(s) is 1 up to rounding; it
// is kept so the loss is the divergence of the normalised distributions the
// kernel actually formed.)
//
// Mapping.  One workgroup of 4 waves per query.  Wave w owns heads
// 32w .. 32w+31 as the N side of 32x32x16 bf16 MFMAs and keeps all 36 query
// k-steps in registers; selected latent rows arrive 32 at a time in a
// three-stage LDS ring, two blocks ahead, through the global->LDS DMA (the band-major, swizzled
// layout of the attention kernel).  Per block the logit product gives each
// lane one head over 16 keys; the probabilities go to an LDS tile
// [32 keys x 128 heads] and eight threads per key sum them over the heads.
// The indexer scores of the selected entries are gathered once into LDS.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace dsa {

namespace {
constexpr int kDqk = 576;
constexpr int kBlk = 32;
constexpr int kBufBytes = kBlk * kDqk * 2;  // 36864 bytes per stage
constexpr int kBand = 4096;                 // bytes per 8-chunk band of a stage
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kHeadsPerWave = 32;
constexpr int kMaxHeads = kWaves * kHeadsPerWave;
constexpr int kDmaPerWave = 9;
constexpr int kKSteps = kDqk / 16;
constexpr int kMaxK = 4096;
constexpr int kPf = 3;  // key-tile reads in flight

typedef __attribute__((address_space(3))) void* lds_ptr;
typedef __attribute__((address_space(3))) uint8_t* lds_u8_ptr;

// chunk-slot swizzle of a 128-byte band row (as in the attention kernel:
// conflict-free for the 16-byte key-tile reads of 32 rows)
__device__ __forceinline__ int swz(int r) { return ((r >> 2) ^ (2 * r)) & 7; }

// The three stages arrive restrict-qualified, so the compiler sees that the
// stage being read is not the one a DMA is writing; step(cur, ahead, blk)
// reads block blk from cur and fills `ahead` with block blk + 2.
template <class Step>
__device__ __forceinline__ void run_triple(uint8_t* __restrict__ sa, uint8_t* __restrict__ sb,
                                           uint8_t* __restrict__ sc, int nb, Step& step) {
  for (int blk = 0; blk < nb; blk += 3) {
    step(sa, sc, blk);
    if (blk + 1 < nb) step(sb, sa, blk + 1);
    if (blk + 2 < nb) step(sc, sb, blk + 2);
  }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += shfl_xor_f(v, m);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, shfl_xor_f(v, m));
  return v;
}
}  // namespace

struct KlParams {
  const uint16_t* q;
  const uint16_t* kv;
  uint32_t kv_bytes;  // extent of the latent rows when below 4 GiB (buffer DMA), else 0
  const int32_t* idx;
  const float* lse;
  const float* scores;
  int64_t ld;
  int64_t N;
  int32_t H;
  int32_t k;
  float scale_log2;  // scale * log2(e)
  float* kl;
};

template <bool kBufDma>
__global__ __launch_bounds__(kThreads, 1) void indexer_kl_kernel(KlParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t st0[kBufBytes];
  __shared__ __attribute__((aligned(16))) uint8_t st1[kBufBytes];
  __shared__ __attribute__((aligned(16))) uint8_t st2[kBufBytes];
  __shared__ int32_t rows[kMaxK];                          // latent row of every entry (-1: skipped)
  __shared__ float isel[kMaxK];                            // indexer score of every entry
  __shared__ __attribute__((aligned(16))) float pbuf[kBlk * kMaxHeads];  // P of one block, [key][head]
  __shared__ float red[3 * kWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hn = lane & 31, hh = lane >> 5;
  const int64_t t = blockIdx.x;
  const int32_t* idx_row = p.idx + t * (int64_t)p.k;
  const int nb = (p.k + kBlk - 1) / kBlk;

  // ---- selected rows and their indexer scores; LSE_I over the valid ones
  float imax = -INFINITY;
  for (int e = tid; e < nb * kBlk; e += kThreads) {
    int32_t row = -1;
    float sc = -INFINITY;
    if (e < p.k) {
      const int32_t s = idx_row[e];
      if (s >= 0 && s < p.N) {
        row = s;
        sc = p.scores[t * p.ld + s];
      }
    }
    rows[e] = row;
    isel[e] = sc;
    imax = fmaxf(imax, sc);
  }
  imax = wave_max(imax);
  if (lane == 0) red[wave] = imax;
  __syncthreads();
  imax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float isum = 0.f;
  for (int e = tid; e < nb * kBlk; e += kThreads)
    if (rows[e] >= 0) isum += expf(isel[e] - imax);
  isum = wave_sum(isum);
  __syncthreads();
  if (lane == 0) red[wave] = isum;

  // ---- query rows of this wave's heads (all 36 k-steps; B layout of the
  // logit MFMA: k-step ks of lane (head hn, half hh) is dims 16ks + 8hh ..)
  const int head = kHeadsPerWave * wave + hn;
  const bool hv = head < p.H;
  v8bf qf[kKSteps];
  {
    const uint16_t* qrow = p.q + (t * p.H + (hv ? head : p.H - 1)) * (int64_t)kDqk + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
      const v8bf v = *(const v8bf*)(qrow + 16 * ks);
      qf[ks] = hv ? v : (v8bf){};
    }
  }
  const float lse_l2 = hv ? p.lse[t * p.H + head] * 1.44269504088896340736f : 0.f;
  __syncthreads();
  const float lse_i = imax + logf(red[0] + red[1] + red[2] + red[3]);  // -inf for an empty row

  // ---- gather: wave w moves rows 8w .. 8w+7 of a block, one DMA per band
  const int g_row = 8 * wave + (lane >> 3);
  const int g_chunk = (lane & 7) ^ swz(g_row);
  const __amdgpu_buffer_rsrc_t kv_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.kv, (short)0, (int)p.kv_bytes, 0x00020000);
  auto gather = [&](uint8_t* base, int blk) {
    int32_t row = rows[blk * kBlk + g_row];
    row = row < 0 ? 0 : row;  // skipped entries read row 0 (masked later)
    if constexpr (kBufDma) {
      const uint32_t voff = (uint32_t)row * (kDqk * 2) + 16 * g_chunk;
#pragma unroll
      for (int bd = 0; bd < kDmaPerWave; ++bd)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(kv_rsrc, (lds_ptr)(base + bd * kBand + wave * 1024), 16,
                                                 voff + 128 * bd, 0, 0, 0);
    } else {
      const uint16_t* src = p.kv + ((uint64_t)(uint32_t)row * kDqk + 8 * g_chunk);
#pragma unroll
      for (int bd = 0; bd < kDmaPerWave; ++bd)
        __builtin_amdgcn_global_load_lds((const void*)(src + 64 * bd), (lds_ptr)(base + bd * kBand + wave * 1024),
                                         16, 0, 0);
    }
  };
  // key tile of k-step ks: lane (row hn, half hh) reads chunk 2ks + hh of its row
  uint32_t k_addr[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) k_addr[q] = (uint32_t)(hn * 128 + (((2 * q + hh) ^ swz(hn)) << 4));
  auto read_k = [&](const lds_u8_ptr base, int ks) {
    return *(const __attribute__((address_space(3))) v8bf*)(base + k_addr[ks & 3] + kBand * (ks >> 2));
  };

  float ent = 0.f, cross = 0.f, psum = 0.f;  // per key-owning thread, over all blocks
  const int rkey = tid >> 3, rpart = tid & 7;  // head-sum role: key rkey, heads 16*rpart .. +15

  auto step = [&](uint8_t* cur, uint8_t* ahead, int blk) {
    // this wave's DMA of blk landed (the one of blk+1 may still be in
    // flight); the barrier makes every wave's land and frees `ahead` (read in
    // the previous step) and pbuf (read there too)
    if (blk + 1 < nb)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kDmaPerWave) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    if (blk + 2 < nb) gather(ahead, blk + 2);
    const lds_u8_ptr kb = (lds_u8_ptr)cur;
    v16f acc = {};
    v8bf abuf[kPf + 1];
#pragma unroll
    for (int ks = 0; ks < kPf; ++ks) abuf[ks] = read_k(kb, ks);
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
      if (ks + kPf < kKSteps) abuf[(ks + kPf) % (kPf + 1)] = read_k(kb, ks + kPf);
      acc = mfma_bf16_32x32x16(abuf[ks % (kPf + 1)], qf[ks], acc);
    }
    // lane (head, hh) holds keys 8*(r/4) + 4*hh + r%4 of the block
    const uint32_t valid = (uint32_t)(__ballot(rows[blk * kBlk + (lane & 31)] >= 0) & 0xFFFFFFFFull);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 8 * (r >> 2) + 4 * hh + (r & 3);
      const bool ok = hv && ((valid >> key) & 1);
      pbuf[key * kMaxHeads + head] = ok ? __builtin_amdgcn_exp2f(fmaf(acc[r], p.scale_log2, -lse_l2)) : 0.f;
    }
    // bare barrier after the LDS writes: a fenced one would also wait for the DMA just issued
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    // sum over the heads: 8 threads per key, 16 heads each
    const v4f* src = (const v4f*)(pbuf + rkey * kMaxHeads + 16 * rpart);
    const v4f a = src[0], b2 = src[1], c = src[2], d = src[3];
    float v = ((a[0] + a[1]) + (a[2] + a[3])) + ((b2[0] + b2[1]) + (b2[2] + b2[3])) +
              (((c[0] + c[1]) + (c[2] + c[3])) + ((d[0] + d[1]) + (d[2] + d[3])));
    v += shfl_xor_f(v, 1);
    v += shfl_xor_f(v, 2);
    v += shfl_xor_f(v, 4);
    const int e = blk * kBlk + rkey;
    if (rpart == 0 && rows[e] >= 0) {
      const float ps = v / (float)p.H;
      if (ps > 0.f) ent += ps * logf(ps);
      cross += ps * isel[e];
      psum += ps;
    }
  };
  if (nb > 0) gather(st0, 0);
  if (nb > 1) gather(st1, 1);
  run_triple(st0, st1, st2, nb, step);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  ent = wave_sum(ent);
  cross = wave_sum(cross);
  psum = wave_sum(psum);
  __syncthreads();
  if (lane == 0) {
    red[wave] = ent;
    red[kWaves + wave] = cross;
    red[2 * kWaves + wave] = psum;
  }
  __syncthreads();
  if (tid == 0) {
    float se = 0.f, sc = 0.f, sp = 0.f;
    for (int w = 0; w < kWaves; ++w) {
      se += red[w];
      sc += red[kWaves + w];
      sp += red[2 * kWaves + w];
    }
    p.kl[t] = sp > 0.f ? se - sc + sp * lse_i : 0.f;
  }
}

// ---------------------------------------------------------------- dense warm-up loss
// "DeepSeek-V3.2" report walk-through §2.3.1 (dense warm-up stage): the same
// divergence with the target built from the dense attention over every causal
// key s <= pos(t) and the indexer softmax over the same keys,
//   L^I = sum_t KL( p_{t,:} || Softmax(I_{t,:}) ).
// One workgroup of 8 waves per pair of consecutive queries: waves 0-3 hold the
// heads of the first, waves 4-7 of the second, and every 32-key block is
// gathered once for both (the two queries' causal ranges differ by one key).
// Three passes over the keys:
//   0. LSE_I of each query's score row (an online log-sum-exp per thread);
//   1. each head's dense log-sum-exp lse_h over all its keys (the logit MFMAs
//      of the sparse-stage kernel with an online maximum and sum per head);
//   2. the sparse-stage step with S_t = all keys and P_h(s) = exp(z - lse_h).
// Key blocks stream through a three-stage LDS ring, two blocks ahead; the
// block's indexer scores arrive with its latent rows by the same DMA.
struct DenseKlParams {
  const uint16_t* q;
  const uint16_t* kv;
  uint32_t kv_bytes;  // extent of the latent rows when below 4 GiB (buffer DMA), else 0
  const float* scores;
  uint32_t s_bytes;   // extent of the score rows when below 4 GiB, else 0
  int64_t ld;
  int64_t N;
  int64_t T;
  int64_t q_pos0;
  int32_t H;
  float scale_log2;  // scale * log2(e)
  float* kl;
  float* lse;  // optional: the dense lse [T, H] (natural log)
};

constexpr int kDq = 2;                  // queries per workgroup
constexpr int kDThreads = kDq * kThreads;
constexpr int kDStages = 3;

// (m, l) <- log-sum-exp merge of two partial (max, sum of exp(x - max)) pairs
__device__ __forceinline__ void lse_merge(float& m, float& l, float m2, float l2) {
  const float mm = fmaxf(m, m2);
  if (mm == -INFINITY) return;  // both empty
  l = l * expf(m - mm) + l2 * expf(m2 - mm);
  m = mm;
}

template <bool kBufDma>
__global__ __launch_bounds__(kDThreads, 1) void indexer_dense_kl_kernel(DenseKlParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t st0[kBufBytes];
  __shared__ __attribute__((aligned(16))) uint8_t st1[kBufBytes];
  __shared__ __attribute__((aligned(16))) uint8_t st2[kBufBytes];
  __shared__ __attribute__((aligned(16))) float sst[kDStages][kDq * kBlk];  // scores of a block's keys
  __shared__ __attribute__((aligned(16))) float pbuf[kDq][kBlk * kMaxHeads];  // P of one block, [key][head]
  __shared__ float red[kDq][3 * kWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qs = wave >> 2, qw = wave & 3;  // query slot, wave within the query
  const int hn = lane & 31, hh = lane >> 5;
  const int64_t t0 = (int64_t)kDq * blockIdx.x;
  const int64_t t = t0 + qs;
  const bool tv = t < p.T;
  const int64_t n = tv ? min(p.q_pos0 + t + 1, p.N) : 0;                    // this query's keys
  const int64_t n_wg = min(p.q_pos0 + min(t0 + kDq, p.T), p.N);             // the workgroup's keys (>= 1)
  const int nb = (int)((n_wg + kBlk - 1) / kBlk);
  const float* srow = p.scores + (tv ? t : t0) * p.ld;

  // ---- pass 0: LSE_I over the query's score row
  {
    float im = -INFINITY, il = 0.f;
    for (int64_t s = tid & (kThreads - 1); s < n; s += kThreads) lse_merge(im, il, srow[s], 1.f);
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) lse_merge(im, il, shfl_xor_f(im, d), shfl_xor_f(il, d));
    if (lane == 0) {
      red[qs][qw] = im;
      red[qs][kWaves + qw] = il;
    }
  }

  // ---- query rows of this wave's heads (as in the sparse-stage kernel)
  const int head = kHeadsPerWave * qw + hn;
  const bool hv = tv && head < p.H;
  v8bf qf[kKSteps];
  {
    const uint16_t* qrow = p.q + ((tv ? t : t0) * p.H + (head < p.H ? head : p.H - 1)) * (int64_t)kDqk + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
      const v8bf v = *(const v8bf*)(qrow + 16 * ks);
      qf[ks] = hv ? v : (v8bf){};
    }
  }
  __syncthreads();
  float lse_i;
  {
    float im = red[qs][0], il = red[qs][kWaves];
    for (int w = 1; w < kWaves; ++w) lse_merge(im, il, red[qs][w], red[qs][kWaves + w]);
    lse_i = im + logf(il);
  }
  __syncthreads();

  // ---- gather (waves 0-3): rows 8w .. 8w+7 of a block, one DMA per band, and
  // (wave 0) the 2 x 32 scores of the block's keys; rows past n_wg re-read the last
  const bool gatherer = wave < kWaves;
  const int g_row = 8 * qw + (lane >> 3);
  const int g_chunk = (lane & 7) ^ swz(g_row);
  const __amdgpu_buffer_rsrc_t kv_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.kv, (short)0, (int)p.kv_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t s_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.scores, (short)0, (int)p.s_bytes, 0x00020000);
  // score DMA of lane l: key 32*blk + l%32 of query t0 + l/32 (clamped inside that query's row)
  const int64_t s_t = min(t0 + (lane >> 5), p.T - 1);
  const int64_t s_n = min(p.q_pos0 + s_t + 1, p.N);
  auto gather = [&](uint8_t* base, int blk, int stage) {
    if (!gatherer) return;
    const int64_t row = min((int64_t)blk * kBlk + g_row, n_wg - 1);
    const int64_t skey = min((int64_t)blk * kBlk + (lane & 31), s_n - 1);
    if constexpr (kBufDma) {
      const uint32_t voff = (uint32_t)row * (kDqk * 2) + 16 * g_chunk;
#pragma unroll
      for (int bd = 0; bd < kDmaPerWave; ++bd)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(kv_rsrc, (lds_ptr)(base + bd * kBand + qw * 1024), 16,
                                                 voff + 128 * bd, 0, 0, 0);
      if (wave == 0)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(s_rsrc, (lds_ptr)&sst[stage][0], 4,
                                                 (uint32_t)((s_t * p.ld + skey) * 4), 0, 0, 0);
    } else {
      const uint16_t* src = p.kv + ((uint64_t)row * kDqk + 8 * g_chunk);
#pragma unroll
      for (int bd = 0; bd < kDmaPerWave; ++bd)
        __builtin_amdgcn_global_load_lds((const void*)(src + 64 * bd), (lds_ptr)(base + bd * kBand + qw * 1024),
                                         16, 0, 0);
      if (wave == 0)
        __builtin_amdgcn_global_load_lds((const void*)(p.scores + s_t * p.ld + skey), (lds_ptr)&sst[stage][0], 4,
                                         0, 0);
    }
  };
  // wait for this wave's DMA of block blk; one later block's DMA (kDmaPerWave
  // row DMAs, plus wave 0's score DMA) may stay in flight
  constexpr int kScoreDma = 1;
  static_assert(kDmaPerWave + kScoreDma <= 63, "vmcnt field");
  auto wait_block = [&](int blk) {
    if (blk + 1 < nb) {
      if (wave == 0)
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kDmaPerWave + kScoreDma) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kDmaPerWave) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __builtin_amdgcn_s_barrier();
  };
  uint32_t k_addr[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) k_addr[q] = (uint32_t)(hn * 128 + (((2 * q + hh) ^ swz(hn)) << 4));
  auto read_k = [&](const lds_u8_ptr base, int ks) {
    return *(const __attribute__((address_space(3))) v8bf*)(base + k_addr[ks & 3] + kBand * (ks >> 2));
  };
  auto logits = [&](const lds_u8_ptr kb) {
    v16f acc = {};
    v8bf abuf[kPf + 1];
#pragma unroll
    for (int ks = 0; ks < kPf; ++ks) abuf[ks] = read_k(kb, ks);
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
      if (ks + kPf < kKSteps) abuf[(ks + kPf) % (kPf + 1)] = read_k(kb, ks + kPf);
      acc = mfma_bf16_32x32x16(abuf[ks % (kPf + 1)], qf[ks], acc);
    }
    return acc;
  };
  auto prologue = [&]() {
    gather(st0, 0, 0);
    if (nb > 1) gather(st1, 1, 1);
  };

  // ---- pass 1: dense lse of each head (log2 units; both lanes of a head agree)
  float mrun = -INFINITY, lrun = 0.f;
  auto step1 = [&](uint8_t* cur, uint8_t* ahead, int blk) {
    wait_block(blk);
    if (blk + 2 < nb) gather(ahead, blk + 2, (blk + 2) % kDStages);
    const v16f acc = logits((lds_u8_ptr)cur);
    // accumulator r of this lane is key 32*blk + 8*(r/4) + 4*hh + r%4; keys from n on are masked
    const int64_t kb = (int64_t)blk * kBlk + 4 * hh;
    float bm = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (kb + 8 * (r >> 2) + (r & 3) < n) bm = fmaxf(bm, acc[r] * p.scale_log2);
    bm = fmaxf(bm, shfl_xor_f(bm, 32));
    if (bm > mrun) {
      lrun *= __builtin_amdgcn_exp2f(mrun - bm);
      mrun = bm;
    }
    float ls = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (kb + 8 * (r >> 2) + (r & 3) < n) ls += __builtin_amdgcn_exp2f(fmaf(acc[r], p.scale_log2, -mrun));
    lrun += ls + shfl_xor_f(ls, 32);
  };
  prologue();
  run_triple(st0, st1, st2, nb, step1);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();  // every wave is done with the stages
  const float lse_l2 = mrun + log2f(lrun);
  if (p.lse && hv && hh == 0) p.lse[t * p.H + head] = lse_l2 * 0.69314718055994530942f;

  // ---- pass 2: the sparse-stage step over all keys
  float ent = 0.f, cross = 0.f, psum = 0.f;
  const int rq = tid >> 8, rkey = (tid >> 3) & 31, rpart = tid & 7;  // head-sum role: query rq, key rkey
  const int64_t n_r = min(p.q_pos0 + t0 + rq + 1, p.N);
  const bool rv = t0 + rq < p.T;
  float* pq = pbuf[qs];
  auto step2 = [&](uint8_t* cur, uint8_t* ahead, int blk) {
    wait_block(blk);
    if (blk + 2 < nb) gather(ahead, blk + 2, (blk + 2) % kDStages);
    const v16f acc = logits((lds_u8_ptr)cur);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 8 * (r >> 2) + 4 * hh + (r & 3);
      const bool ok = hv && (int64_t)blk * kBlk + key < n;
      pq[key * kMaxHeads + head] = ok ? __builtin_amdgcn_exp2f(fmaf(acc[r], p.scale_log2, -lse_l2)) : 0.f;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    const v4f* src = (const v4f*)(&pbuf[rq][0] + rkey * kMaxHeads + 16 * rpart);
    const v4f a = src[0], b2 = src[1], c = src[2], d = src[3];
    float v = ((a[0] + a[1]) + (a[2] + a[3])) + ((b2[0] + b2[1]) + (b2[2] + b2[3])) +
              (((c[0] + c[1]) + (c[2] + c[3])) + ((d[0] + d[1]) + (d[2] + d[3])));
    v += shfl_xor_f(v, 1);
    v += shfl_xor_f(v, 2);
    v += shfl_xor_f(v, 4);
    const int64_t e = (int64_t)blk * kBlk + rkey;
    if (rpart == 0 && rv && e < n_r) {
      const float ps = v / (float)p.H;
      if (ps > 0.f) ent += ps * logf(ps);
      cross += ps * sst[blk % kDStages][rq * kBlk + rkey];
      psum += ps;
    }
  };
  prologue();
  run_triple(st0, st1, st2, nb, step2);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  ent = wave_sum(ent);
  cross = wave_sum(cross);
  psum = wave_sum(psum);
  __syncthreads();
  if (lane == 0) {  // a wave's key owners all belong to query rq = wave / 4
    red[qs][qw] = ent;
    red[qs][kWaves + qw] = cross;
    red[qs][2 * kWaves + qw] = psum;
  }
  __syncthreads();
  if (tid == 0 || tid == kThreads) {
    const int r = tid / kThreads;
    float se = 0.f, sc = 0.f, sp = 0.f;
    for (int w = 0; w < kWaves; ++w) {
      se += red[r][w];
      sc += red[r][kWaves + w];
      sp += red[r][2 * kWaves + w];
    }
    if (t0 + r < p.T) {
      // LSE_I of query r: the lse_i of any of its waves (this thread is in wave 4r)
      p.kl[t0 + r] = se - sc + sp * lse_i;
    }
  }
}

hipError_t launch_indexer_dense_kl(const uint16_t* q, const uint16_t* kv, int64_t N, const float* scores, int64_t ld,
                                   int64_t T, int64_t q_pos0, int32_t H, float scale, float* kl, float* lse,
                                   hipStream_t st) {
  if (T <= 0) return hipSuccess;
  DenseKlParams p;
  p.q = q;
  p.kv = kv;
  const uint64_t extent = (uint64_t)N * kDqk * 2;
  p.kv_bytes = extent < 0xFFFFFFFFull ? (uint32_t)extent : 0u;
  p.scores = scores;
  const uint64_t s_extent = (uint64_t)T * ld * 4;
  p.s_bytes = s_extent < 0xFFFFFFFFull ? (uint32_t)s_extent : 0u;
  p.ld = ld;
  p.N = N;
  p.T = T;
  p.q_pos0 = q_pos0;
  p.H = H;
  p.scale_log2 = scale * 1.44269504088896340736f;
  p.kl = kl;
  p.lse = lse;
  const dim3 grid((unsigned)((T + kDq - 1) / kDq));
  if (p.kv_bytes != 0 && p.s_bytes != 0)
    hipLaunchKernelGGL(indexer_dense_kl_kernel<true>, grid, dim3(kDThreads), 0, st, p);
  else
    hipLaunchKernelGGL(indexer_dense_kl_kernel<false>, grid, dim3(kDThreads), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_indexer_kl(const uint16_t* q, const uint16_t* kv, int64_t N, const int32_t* idx,
                             const float* lse, const float* scores, int64_t ld, int64_t T, int32_t H, int32_t k,
                             float scale, float* kl, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  KlParams p;
  p.q = q;
  p.kv = kv;
  const uint64_t extent = (uint64_t)N * kDqk * 2;
  p.kv_bytes = extent < 0xFFFFFFFFull ? (uint32_t)extent : 0u;
  p.idx = idx;
  p.lse = lse;
  p.scores = scores;
  p.ld = ld;
  p.N = N;
  p.H = H;
  p.k = k;
  p.scale_log2 = scale * 1.44269504088896340736f;
  p.kl = kl;
  if (p.kv_bytes != 0)
    hipLaunchKernelGGL(indexer_kl_kernel<true>, dim3((unsigned)T), dim3(kThreads), 0, st, p);
  else
    hipLaunchKernelGGL(indexer_kl_kernel<false>, dim3((unsigned)T), dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace dsa
