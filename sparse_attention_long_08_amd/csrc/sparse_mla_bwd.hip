// Backward of the sparse MLA-MQA attention on gfx950 bf16 matrix cores.
//
// The sparse training stage trains the main model through the sparse
// attention ("DeepSeek-V3.2" report walk-through, §2.3.2), so the attention
// over the selected rows (§2.1.2 attention equation, MQA form of §2.2) needs
// its gradient.  Per query t, head h and selected row s, with dO = dL/dout:
//   P    = exp(scale * q[t,h] . kv[s] - lse[t,h])        (recomputed)
//   dP   = dO[t,h] . kv[s][:512]
//   D    = dO[t,h] . out[t,h]          (= sum_s P dP for the forward's out)
//   dS   = scale * P * (dP - D)
//   dq[t,h]  = sum_s dS kv[s]
//   dkv[s]  += sum_h dS q[t,h]  +  sum_h P dO[t,h]   (second term: dims < 512)
//
// Two kernels per tile of queries:
//
// mla_bwd_dq_kernel: one workgroup of 4 waves per (query, 64-head half);
// wave w owns 16 heads.  The selected latent rows are gathered 32 at a time
// into LDS by DMA (band-major stages with an XOR swizzle, as the forward
// kernel lays them out), double buffered.  Per block it forms S^T = K Q^T and
// dP^T = V dO^T on 16x16x32 MFMAs (keys on the rows, heads on the columns,
// so each lane owns one head and four keys per tile), then P and dS in
// registers, accumulates dq^T += K^T dS^T (36 tiles of 16 latent dims; the
// K^T operand is read transposed with ds_read_b64_tr_b16 and dS^T is the
// lane's own values, with the key order of the two agreeing) and stores P
// and dS as bf16 to a workspace laid out [query][entry][head].
//
// mla_bwd_dkv_kernel: one workgroup of 8 waves per query; each wave owns
// four or five 16-column tiles of the 576 latent dims.  It holds q and dO of
// all heads in the B layout of the head contraction (heads on k), streams
// the P and dS tiles of each 32-entry block through LDS by DMA, forms
//   addend_block = dS^T q + P^T dO          (32 entries x 576 dims)
// and stores it, one bf16 row per (query, entry) (rounded to nearest: 2^-9
// of each addend, against the 2^-7 tolerance of the gradients).
//
// dkv sums the addends over every (query, entry) that selected a row, so it
// is a scatter.  Instead of atomics (whose adds all travel to the memory
// side, since 75 MB of dkv rows fit no L2), the tile's entries are grouped by
// cache row through an inverted index (count, scan, fill) and
// dkv_reduce_kernel sums each row's addends with one wave per row.
#include "common.h"
#include "launch.h"

namespace dsa {
namespace {

constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kBlk = 32;                    // selected rows per block
constexpr int kStage = kBlk * kDqk * 2;     // 36864 bytes of gathered rows
constexpr int kBand = 4096;                 // one 8-chunk band of all 32 rows
constexpr int kDmaPerWave = kStage / kBand; // one DMA per band, eight rows per wave
constexpr int kStoreTiles = 2;              // 16-key tiles of a block
constexpr int kStoreRows = 4;               // accumulator rows per lane and tile
constexpr int kStoresPerStep = 2 * kStoreTiles * kStoreRows;  // P and dS of every (tile, row)
static_assert(kStage == kDmaPerWave * kBand, "a stage is whole bands");
static_assert(kStoreTiles * 16 == kBlk, "a block is two 16-key tiles");
// vmcnt is a 6-bit field: the deepest wait below must fit it
static_assert(kDmaPerWave + 2 * kStoresPerStep + kDmaPerWave <= 63, "vmcnt field");
constexpr int kThreads = 256;               // 4 waves
constexpr int kMaxK = 4096;
constexpr int kQSteps = kDqk / 32;          // 18 k-steps of the logit product
constexpr int kVSteps = kDv / 32;           // 16 k-steps of the dP product
constexpr int kCt = kDqk / 16;              // 36 dq tiles of 16 latent dims
constexpr int kKvWaves = 8;                 // waves of the dkv kernel (two per SIMD)
constexpr int kKvThreads = 64 * kKvWaves;
constexpr int kTilesPerWave = 5;            // dkv column tiles per wave, at most

// Column tile (16 latent dims) of slot ci of dkv wave w, or -1.  Waves 0..3
// take tiles 5w .. 5w+4; wave 4+i takes 20+3i .. 22+3i and the rope tile
// 32+i, so the two waves on one SIMD share out 17 tile products (a rope tile
// has no value term).
__device__ __forceinline__ int kv_tile(int w, int ci) {
  if (w < 4) return 5 * w + ci;
  const int i = w - 4;
  return ci < 3 ? 20 + 3 * i + ci : (ci == 3 ? 32 + i : -1);
}
constexpr int kPRow = 256;                  // LDS bytes per entry row of a P / dS tile (128 heads)

typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4s* lds_v4s_ptr;
typedef __attribute__((address_space(3))) void* lds_ptr;
typedef __attribute__((address_space(3))) uint8_t* lds_u8_ptr;
typedef __attribute__((address_space(3))) const v8bf* lds_v8bf_cptr;

// XOR swizzle of the 16-byte slot within a 128-byte band row (the forward
// kernel's layout).
__device__ __forceinline__ int swz(int r) { return ((r >> 2) ^ (2 * r)) & 7; }

__device__ __forceinline__ __bf16 to_bf16(float x) { return (__bf16)x; }

struct BwdParams {
  const uint16_t* q;     // [T, H, 576]
  const uint16_t* kv;    // [N, 576]
  const int32_t* idx;    // [T, k]
  const float* out;      // [T, H, 512]
  const float* lse;      // [T, H]
  const uint16_t* dout;  // [T, H, 512]
  int64_t T;
  int64_t N;
  int32_t H;
  int32_t Hp;            // heads padded to a multiple of 32 (k-steps of the head contraction)
  int32_t Hs;            // heads padded to a multiple of 64: the workspace row (one slot per dq-kernel lane)
  int32_t k;
  int32_t kp;            // k rounded up to whole blocks: entry stride of pbuf / dsbuf
  uint32_t kv_bytes;     // extent of kv when below 4 GiB (buffer-form DMA), else 0
  float scale;
  float scale_log2;      // scale * log2(e)
  float* dq;             // [T, H, 576]
  uint16_t* pbuf;        // [T, kp, Hs] bf16 P (entries k .. kp-1 and heads H .. Hs-1 are padding)
  uint16_t* dsbuf;       // [T, kp, Hs] bf16 dS (scale folded in)
  uint16_t* addend;      // [T, k, 576] bf16: each entry's contribution to its cache row
};

// Resolves the entries of query t to cache rows (-1: skipped), padded with
// -1 to whole blocks.
__device__ __forceinline__ void load_rows(const BwdParams& p, int64_t t, int32_t* rows, int nb) {
  for (int e = threadIdx.x; e < nb * kBlk; e += blockDim.x) {
    int32_t r = -1;
    if (e < p.k) {
      const int32_t s = p.idx[t * (int64_t)p.k + e];
      if (s >= 0 && s < p.N) r = s;
    }
    rows[e] = r;
  }
}

// Drives a three-stage ring; the stages arrive restrict-qualified so that
// the compiler sees the stage being read is not the one a DMA is filling.
template <class Step>
__device__ __forceinline__ void run_ring3(uint8_t* __restrict__ sa, uint8_t* __restrict__ sb,
                                          uint8_t* __restrict__ sc, int nb, Step& step) {
  for (int blk = 0; blk < nb; blk += 3) {
    step(sa, sc, blk);
    if (blk + 1 < nb) step(sb, sa, blk + 1);
    if (blk + 2 < nb) step(sc, sb, blk + 2);
  }
}

// ---------------------------------------------------------------- dq kernel
template <bool kBufDma>
__global__ __launch_bounds__(kThreads, 1) void mla_bwd_dq_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t stage0[kStage];
  __shared__ __attribute__((aligned(16))) uint8_t stage1[kStage];
  __shared__ __attribute__((aligned(16))) uint8_t stage2[kStage];
  __shared__ int32_t rows[kMaxK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hn = lane & 15, qd = lane >> 4;

  // Workgroups b and b+8 land on the same XCD: with two head halves they
  // take the two halves of one query, so its gathered rows are shared in L2.
  const int n_half = (p.Hp + 63) / 64;
  int64_t t;
  int half;
  if (n_half == 2) {
    const int64_t b = blockIdx.x;
    half = (int)((b >> 3) & 1);
    t = (b >> 4) * 8 + (b & 7);
  } else {
    half = 0;
    t = blockIdx.x;
  }
  if (t >= p.T) return;
  const int head = 64 * half + 16 * wave + hn;
  // a wave whose heads are all padding computes zeros, stores them to its
  // own padding slots and joins every barrier
  const bool hv = head < p.H;
  const int nb = (p.k + kBlk - 1) / kBlk;
  load_rows(p, t, rows, nb);

  // q and dO of this lane's head in the B layout of 16x16x32 MFMAs: k-step
  // ks holds dims 32*ks + 8*qd .. +7.  D = dO . out over the same dims,
  // summed over the four lanes of the head.
  const int hc = hv ? head : 0;
  v8bf qf[kQSteps], df[kVSteps];
  float dsum = 0.f;
  {
    const uint16_t* qrow = p.q + (t * p.H + hc) * (int64_t)kDqk + 8 * qd;
#pragma unroll
    for (int ks = 0; ks < kQSteps; ++ks) {
      const v8bf v = *(const v8bf*)(qrow + 32 * ks);
      qf[ks] = hv ? v : (v8bf){};
    }
    const uint16_t* drow = p.dout + (t * p.H + hc) * (int64_t)kDv + 8 * qd;
    const float* orow = p.out + (t * p.H + hc) * (int64_t)kDv + 8 * qd;
#pragma unroll
    for (int ks = 0; ks < kVSteps; ++ks) {
      const v8bf v = *(const v8bf*)(drow + 32 * ks);
      const float4 o0 = *(const float4*)(orow + 32 * ks);
      const float4 o1 = *(const float4*)(orow + 32 * ks + 4);
      df[ks] = hv ? v : (v8bf){};
      dsum += (float)v[0] * o0.x + (float)v[1] * o0.y + (float)v[2] * o0.z + (float)v[3] * o0.w +
              (float)v[4] * o1.x + (float)v[5] * o1.y + (float)v[6] * o1.z + (float)v[7] * o1.w;
    }
    dsum += shfl_xor_f(dsum, 16);
    dsum += shfl_xor_f(dsum, 32);
  }
  const float lse_l2 = hv ? p.lse[t * p.H + hc] * 1.4426950408889634f : 0.f;
  __syncthreads();  // rows[]

  // Gather of one block: wave w moves rows 8w .. 8w+7, one DMA per band;
  // lane L carries row 8w + L/8 into slot L%8 of the band.
  const int g_row = 8 * wave + (lane >> 3);
  const int g_chunk = (lane & 7) ^ swz(g_row);
  // the buffer form of the DMA leaves the compiler's LDS wait counting exact
  const __amdgpu_buffer_rsrc_t kv_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.kv, (short)0, (int)p.kv_bytes, 0x00020000);
  auto gather = [&](uint8_t* base, int blk) {
    int32_t row = rows[blk * kBlk + g_row];
    row = row < 0 ? 0 : row;  // skipped entries read row 0; P = 0 masks them
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

  // Key order.  Row m of a 16-key tile of S^T holds key 16kt + kperm(m):
  // the groups of four rows are placed in the order 0, 3, 1, 2.  With it the
  // lanes that the LDS serves together (for the 16-byte key-tile reads and
  // the 8-byte transposed reads, whether it serves 8 or 16 of the first and
  // 16 or 32 of the second per cycle) reach distinct banks under the stage
  // swizzle; in plain order the transposed reads of rows r and r+4 collide.
  auto kperm = [](int m) { return (m & 3) | (((0x2130 >> (4 * (m >> 2))) & 0xF) << 2); };

  // Operand offsets.  Key tile kt, k-step ks (A of S^T and dP^T): lane (row
  // hn, qd) reads key 16kt + kperm(hn), chunk 4ks + qd = band ks/2, slot
  // (4(ks%2) + qd) ^ swz(key).
  uint32_t k_off[2][2];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const int r = 16 * kt + kperm(hn);
      k_off[kt][par] = (uint32_t)(r * 128 + (((4 * par + qd) ^ swz(r)) << 4));
    }
  // K^T tile ct (A of dq^T): the B operand dS^T of lane (head, qd) holds, at
  // k-slot 8qd + i, accumulator row 4qd + i of tile 0 (i < 4) or 4qd + i - 4
  // of tile 1, i.e. its own accumulator values.  ds_read_b64_tr_b16 gives
  // lane i of a 16-lane group column i of the 4 x 16 block whose rows lane
  // 4*rho + c addresses at columns 4c .. 4c+3, so group qd reads keys
  // kperm(4qd + rho) (and 16 + kperm(4qd + rho)) at dims 16ct + 4c: chunk
  // 2ct + c/2, byte 8(c%2).
  uint32_t t_off[2][4];
  {
    const int rho = hn >> 2, c = hn & 3;
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int r = 16 * hi + kperm(4 * qd + rho);
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4)
        t_off[hi][c4] = (uint32_t)(r * 128 + (((2 * c4 + (c >> 1)) ^ swz(r)) << 4) + 8 * (c & 1));
    }
  }

  v4f dqa[kCt];
#pragma unroll
  for (int ct = 0; ct < kCt; ++ct) dqa[ct] = (v4f){0.f, 0.f, 0.f, 0.f};

  // workspace rows of this query (uniform base, 32-bit per-lane offsets)
  uint16_t* const pdst = p.pbuf + (t * (int64_t)p.kp) * p.Hs;
  uint16_t* const sdst = p.dsbuf + (t * (int64_t)p.kp) * p.Hs;
  uint32_t st_off[2][4];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int r = 0; r < 4; ++r) st_off[kt][r] = (uint32_t)((16 * kt + kperm(4 * qd + r)) * p.Hs + head);

  // Wait for this wave's DMA of block blk.  Vector memory operations retire
  // in issue order, so what was issued after that DMA may stay in flight:
  // for block 0 the prologue's DMA of block 1; for block 1 step 0's DMA of
  // block 2 and its stores; for later blocks the stores of steps blk-2 and
  // blk-1 and step blk-1's DMA of block blk+1 (each DMA only if that block
  // exists).
  constexpr int kW0 = kDmaPerWave;                       // step 0, block 1 in flight
  constexpr int kW1 = kStoresPerStep + kDmaPerWave;      // step 1, block 2 in flight
  constexpr int kW2 = 2 * kStoresPerStep + kDmaPerWave;  // later steps, block blk+1 in flight
  auto wait_block = [&](int blk) {
    if (blk == 0) {
      if (nb > 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kW0) : "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    } else if (blk == 1) {
      if (nb > 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kW1) : "memory");
      else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kStoresPerStep) : "memory");
    } else {
      if (blk + 1 < nb) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kW2) : "memory");
      else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kStoresPerStep) : "memory");
    }
    __builtin_amdgcn_s_barrier();
  };

  auto step = [&](uint8_t* __restrict__ cur, uint8_t* __restrict__ ahead, int blk) {
    wait_block(blk);  // block blk landed everywhere; block blk-1's stage is free
    if (blk + 2 < nb) gather(ahead, blk + 2);
    const lds_u8_ptr base = (lds_u8_ptr)cur;
    // logits and dP of the block; key tiles are read kPf k-steps ahead
    constexpr int kPf = 3;
    auto rd_k = [&](int kt, int ks) { return *(lds_v8bf_cptr)(base + (ks >> 1) * kBand + k_off[kt][ks & 1]); };
    auto rd_t = [&](int ct) {
      const uint32_t off = (ct >> 2) * kBand;
      const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(base + off + t_off[0][ct & 3]));
      const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(base + off + t_off[1][ct & 3]));
      return __builtin_bit_cast(v8bf, (v8s){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
    };
    v4f sacc[2] = {(v4f){0.f, 0.f, 0.f, 0.f}, (v4f){0.f, 0.f, 0.f, 0.f}};
    v4f pacc[2] = {(v4f){0.f, 0.f, 0.f, 0.f}, (v4f){0.f, 0.f, 0.f, 0.f}};
    v8bf ab[kPf + 1][2];
#pragma unroll
    for (int i = 0; i < kPf; ++i) {
      ab[i][0] = rd_k(0, i);
      ab[i][1] = rd_k(1, i);
    }
#pragma unroll
    for (int ks = 0; ks < kQSteps; ++ks) {
      if (ks + kPf < kQSteps) {
        ab[(ks + kPf) % (kPf + 1)][0] = rd_k(0, ks + kPf);
        ab[(ks + kPf) % (kPf + 1)][1] = rd_k(1, ks + kPf);
      }
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const v8bf a = ab[ks % (kPf + 1)][kt];
        sacc[kt] = mfma_bf16_16x16x32(a, qf[ks], sacc[kt]);
        if (ks < kVSteps) pacc[kt] = mfma_bf16_16x16x32(a, df[ks < kVSteps ? ks : 0], pacc[kt]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // the first transposed key tiles of the dq product do not depend on dS
    v8bf tb[kPf + 1];
#pragma unroll
    for (int i = 0; i < kPf; ++i) tb[i] = rd_t(i);
    // P and dS; lane holds keys 16kt + kperm(4qd + r) of its head
    float pv[2][4], dv[2][4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = blk * kBlk + 16 * kt + kperm(4 * qd + r);
        const bool valid = hv && rows[e] >= 0;
        const float pr = valid ? __builtin_amdgcn_exp2f(fmaf(sacc[kt][r], p.scale_log2, -lse_l2)) : 0.f;
        pv[kt][r] = pr;
        dv[kt][r] = p.scale * pr * (pacc[kt][r] - dsum);
      }
    const v8bf bop = (v8bf){to_bf16(dv[0][0]), to_bf16(dv[0][1]), to_bf16(dv[0][2]), to_bf16(dv[0][3]),
                            to_bf16(dv[1][0]), to_bf16(dv[1][1]), to_bf16(dv[1][2]), to_bf16(dv[1][3])};
    // kStoresPerStep stores per lane and block, issued by every wave (a wave of padding
    // heads writes the zeros of its own padding slots), so the wait counts
    // above are exact; entries k .. kp-1 are padding rows
    uint16_t* const pb = pdst + (int64_t)blk * kBlk * p.Hs;
    uint16_t* const sb = sdst + (int64_t)blk * kBlk * p.Hs;
#pragma unroll
    for (int kt = 0; kt < kStoreTiles; ++kt)
#pragma unroll
      for (int r = 0; r < kStoreRows; ++r) {
        pb[st_off[kt][r]] = __builtin_bit_cast(uint16_t, to_bf16(pv[kt][r]));
        sb[st_off[kt][r]] = __builtin_bit_cast(uint16_t, to_bf16(dv[kt][r]));
      }
    // dq^T += K^T dS^T
#pragma unroll
    for (int ct = 0; ct < kCt; ++ct) {
      if (ct + kPf < kCt) tb[(ct + kPf) % (kPf + 1)] = rd_t(ct + kPf);
      dqa[ct] = mfma_bf16_16x16x32(tb[ct % (kPf + 1)], bop, dqa[ct]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  if (nb > 0) gather(stage0, 0);
  if (nb > 1) gather(stage1, 1);
  run_ring3(stage0, stage1, stage2, nb, step);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  if (hv) {
    float* drow = p.dq + (t * p.H + head) * (int64_t)kDqk + 4 * qd;
#pragma unroll
    for (int ct = 0; ct < kCt; ++ct) *(float4*)(drow + 16 * ct) = make_float4(dqa[ct][0], dqa[ct][1], dqa[ct][2], dqa[ct][3]);
  }
}

// ---------------------------------------------------------------- dkv kernel
__global__ __launch_bounds__(kKvThreads, 1) void mla_bwd_dkv_kernel(BwdParams p) {
  // [stage][P, dS][32 entries x 128 heads] bf16, slot of chunk c in row j at c ^ (j % 16)
  __shared__ __attribute__((aligned(16))) uint8_t pst[2][2][kBlk * kPRow];
  __shared__ __attribute__((aligned(16))) uint8_t stg[32 * 2 * kDqk];  // one 32-head chunk of q or dO
  __shared__ int32_t rows[kMaxK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hn = lane & 15, qd = lane >> 4;
  const int64_t t = blockIdx.x;
  if (t >= p.T) return;
  const int nb = (p.k + kBlk - 1) / kBlk;
  load_rows(p, t, rows, nb);
  // Head chunks past Hp are never loaded: zero them once in both stages so
  // that the k-steps over them multiply zeros (q and dO are zero there too).
  if (p.Hp < 128) {
    for (int i = tid; i < 2 * 2 * kBlk * 16; i += kKvThreads) {
      const int c = i & 15, j = (i >> 4) & 31, arr = (i >> 9) & 1, sidx = i >> 10;
      const int chunk = c ^ (j & 15);
      if (8 * chunk >= p.Hp) *(v4i*)&pst[sidx][arr][j * kPRow + 16 * c] = (v4i){0, 0, 0, 0};
    }
  }

  // q and dO in the B layout of the head contraction: slot ci covers dims
  // 16 kv_tile(w, ci) + hn; k-step kh holds heads 32kh + 8qd .. +7.  Each
  // 32-head chunk of q (then of dO) is staged row-major in LDS and read back
  // transposed with ds_read_b64_tr_b16 (lane i of a 16-lane group receives
  // column i of the 4 x 16 block whose rows lane 4*rho + c addresses at
  // columns 4c .. 4c+3): group qd reads heads 8qd + rho and 8qd + 4 + rho.
  v8bf qc[kTilesPerWave][4], dc[kTilesPerWave][4];
  {
    const int rho = hn >> 2, c = hn & 3;
#pragma unroll
    for (int kh = 0; kh < 4; ++kh) {
#pragma unroll
      for (int arr = 0; arr < 2; ++arr) {
        const int width = arr ? kDv : kDqk;
        const int cpr = width / 8;  // 16-byte chunks per head row
        const uint16_t* src = arr ? p.dout : p.q;
        for (int i = tid; i < 32 * cpr; i += kKvThreads) {
          const int r = i / cpr, ch = i - r * cpr, h = 32 * kh + r;
          v4i v = (v4i){0, 0, 0, 0};
          if (h < p.H) v = *(const v4i*)(src + (t * p.H + h) * (int64_t)width + 8 * ch);
          *(v4i*)&stg[r * (2 * kDqk) + 16 * ch] = v;
        }
        __syncthreads();
#pragma unroll
        for (int ci = 0; ci < kTilesPerWave; ++ci) {
          const int tile = kv_tile(wave, ci);
          v8bf val = (v8bf){};
          if (tile >= 0 && (!arr || tile < kDv / 16)) {
            const uint32_t col_b = (uint32_t)(2 * (16 * tile + 4 * c));
            const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_v4s_ptr)((lds_u8_ptr)stg + (8 * qd + rho) * (2 * kDqk) + col_b));
            const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_v4s_ptr)((lds_u8_ptr)stg + (8 * qd + 4 + rho) * (2 * kDqk) + col_b));
            val = __builtin_bit_cast(v8bf, (v8s){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
          }
          if (arr) dc[ci][kh] = val;
          else qc[ci][kh] = val;
        }
        __syncthreads();
      }
    }
  }
  __syncthreads();  // rows[]

  // DMA of the P and dS rows of one block: 16 instructions of 4 entry rows
  // each (instruction ii: array ii/8, rows 4(ii%8) .. +3), wave w issuing ii =
  // w and w + 8; lane L fills row 4(ii%8) + L/16, slot L%16 with chunk
  // (L%16) ^ row%16 (chunks past Hp/8 are not loaded and stay zero).
  auto gather = [&](int sidx, int blk) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ii = wave + kKvWaves * i;
      const int arr = ii >> 3, j0 = 4 * (ii & 7);
      const int j = j0 + (lane >> 4);
      const int c = (lane & 15) ^ (j & 15);
      int e = blk * kBlk + j;
      e = e < p.k ? e : p.k - 1;
      if (8 * c < p.Hp) {
        const int64_t off = (t * (int64_t)p.kp + e) * p.Hs + 8 * c;
        const uint16_t* src = arr ? p.dsbuf : p.pbuf;
        __builtin_amdgcn_global_load_lds((const void*)(src + off), (lds_ptr)(&pst[sidx][arr][0] + j0 * kPRow), 16,
                                         0, 0);
      }
    }
  };

  auto step = [&](int sidx, int blk) {
    const lds_u8_ptr pb = (lds_u8_ptr)&pst[sidx][0][0];
    const lds_u8_ptr sb = (lds_u8_ptr)&pst[sidx][1][0];
    v4f acc[2][kTilesPerWave];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int ci = 0; ci < kTilesPerWave; ++ci) acc[kt][ci] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kh = 0; kh < 4; ++kh) {
      v8bf ap[2], as[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const uint32_t off = (uint32_t)((16 * kt + hn) * kPRow + (((4 * kh + qd) ^ hn) << 4));
        ap[kt] = *(lds_v8bf_cptr)(pb + off);
        as[kt] = *(lds_v8bf_cptr)(sb + off);
      }
#pragma unroll
      for (int ci = 0; ci < kTilesPerWave; ++ci) {
        const int tile = kv_tile(wave, ci);
        if (tile < 0) continue;
        const bool has_v = tile < kDv / 16;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          acc[kt][ci] = mfma_bf16_16x16x32(as[kt], qc[ci][kh], acc[kt][ci]);
          if (has_v) acc[kt][ci] = mfma_bf16_16x16x32(ap[kt], dc[ci][kh], acc[kt][ci]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);  // one k-step of operands live at a time
    }
    // addend rows: lane (dim 16 tile + hn, qd) holds entries 16kt + 4qd + r
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = blk * kBlk + 16 * kt + 4 * qd + r;
        if (e < p.k) {
          uint16_t* dst = p.addend + (t * (int64_t)p.k + e) * kDqk + hn;
#pragma unroll
          for (int ci = 0; ci < kTilesPerWave; ++ci) {
            const int tile = kv_tile(wave, ci);
            if (tile >= 0) dst[16 * tile] = __builtin_bit_cast(uint16_t, to_bf16(acc[kt][ci][r]));
          }
        }
      }
  };

  if (nb > 0) gather(0, 0);
  for (int blk = 0; blk < nb; ++blk) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (blk + 1 < nb) gather((blk + 1) & 1, blk + 1);
    step(blk & 1, blk);
  }
}

// ---------------------------------------------------------------- inverted index
// Entries of the tile (e = t*k + j) grouped by cache row: count per row,
// exclusive scan into offsets (cursor starts as a copy), fill the list.
__global__ void csr_count_kernel(const int32_t* __restrict__ idx, int64_t n_ent, int64_t N,
                                 int32_t* __restrict__ count) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n_ent; e += (int64_t)gridDim.x * blockDim.x) {
    const int32_t s = idx[e];
    if (s >= 0 && s < N) atomicAdd(count + s, 1);
  }
}

// One workgroup of 1024 threads: thread i sums a contiguous chunk, the 1024
// chunk sums are scanned across the workgroup (within each wave by shuffles,
// then over the 16 wave totals), and each thread writes its chunk's offsets.
__global__ __launch_bounds__(1024) void csr_scan_kernel(int32_t* __restrict__ count, int32_t* __restrict__ offsets,
                                                        int64_t N) {
  __shared__ int32_t wave_sum[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t chunk = (N + 1023) / 1024;
  const int64_t b = tid * chunk < N ? tid * chunk : N, e = b + chunk < N ? b + chunk : N;
  int32_t sum = 0;
  for (int64_t i = b; i < e; ++i) sum += count[i];
  int32_t incl = sum;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int32_t v = __shfl_up(incl, d, 64);
    if (lane >= d) incl += v;
  }
  if (lane == 63) wave_sum[wave] = incl;
  __syncthreads();
  int32_t before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) {
    const int32_t v = wave_sum[w];
    before += w < wave ? v : 0;
    total += v;
  }
  if (tid == 0) offsets[N] = total;
  int32_t run = before + incl - sum;
  for (int64_t i = b; i < e; ++i) {
    const int32_t c = count[i];
    offsets[i] = run;
    count[i] = run;  // becomes the fill cursor
    run += c;
  }
}

__global__ void csr_fill_kernel(const int32_t* __restrict__ idx, int64_t n_ent, int64_t N,
                                int32_t* __restrict__ cursor, int32_t* __restrict__ list) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n_ent; e += (int64_t)gridDim.x * blockDim.x) {
    const int32_t s = idx[e];
    if (s >= 0 && s < N) list[atomicAdd(cursor + s, 1)] = (int32_t)e;
  }
}

// dkv[s] += sum of the (bf16) addend rows listed for s, in fp32: one wave per
// cache row.  Lane l holds dims 4l..4l+3 of the first and second 256-dim
// halves of the row and, for l < 16, of the 64 rope dims, so a row is three
// 8-byte loads per lane; list entries are fetched 64 at a time and kRedRows
// rows are in flight.
constexpr int kRedRows = 8;

struct Bf16x4 {
  float v[4];
};

__device__ __forceinline__ Bf16x4 bf16x4_to_f32(uint2 w) {
  Bf16x4 r;
  r.v[0] = __uint_as_float(w.x << 16);
  r.v[1] = __uint_as_float(w.x & 0xFFFF0000u);
  r.v[2] = __uint_as_float(w.y << 16);
  r.v[3] = __uint_as_float(w.y & 0xFFFF0000u);
  return r;
}

__global__ __launch_bounds__(256) void dkv_reduce_kernel(const int32_t* __restrict__ offsets,
                                                         const int32_t* __restrict__ list,
                                                         const uint16_t* __restrict__ addend,
                                                         float* __restrict__ dkv, int64_t N) {
  const int lane = threadIdx.x & 63;
  const int64_t s = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (s >= N) return;
  const int32_t b = offsets[s], e = offsets[s + 1];
  if (b == e) return;
  const bool rope = lane < 16;
  float acc[3][4];
#pragma unroll
  for (int c = 0; c < 3; ++c)
#pragma unroll
    for (int x = 0; x < 4; ++x) acc[c][x] = 0.f;
  for (int32_t i0 = b; i0 < e; i0 += 64) {
    const int32_t n = e - i0 < 64 ? e - i0 : 64;
    const int32_t mine = lane < n ? list[i0 + lane] : 0;
    int32_t j = 0;
    for (; j + kRedRows <= n; j += kRedRows) {
      uint2 w[kRedRows][3];
#pragma unroll
      for (int u = 0; u < kRedRows; ++u) {
        const uint2* r = reinterpret_cast<const uint2*>(addend + (int64_t)__shfl(mine, j + u, 64) * kDqk) + lane;
        w[u][0] = r[0];
        w[u][1] = r[64];
        w[u][2] = rope ? r[128] : make_uint2(0u, 0u);
      }
#pragma unroll
      for (int u = 0; u < kRedRows; ++u)
#pragma unroll
        for (int c = 0; c < 3; ++c) {
          const Bf16x4 f = bf16x4_to_f32(w[u][c]);
#pragma unroll
          for (int x = 0; x < 4; ++x) acc[c][x] += f.v[x];
        }
    }
    for (; j < n; ++j) {
      const uint2* r = reinterpret_cast<const uint2*>(addend + (int64_t)__shfl(mine, j, 64) * kDqk) + lane;
      uint2 w[3] = {r[0], r[64], rope ? r[128] : make_uint2(0u, 0u)};
#pragma unroll
      for (int c = 0; c < 3; ++c) {
        const Bf16x4 f = bf16x4_to_f32(w[c]);
#pragma unroll
        for (int x = 0; x < 4; ++x) acc[c][x] += f.v[x];
      }
    }
  }
  float4* d = reinterpret_cast<float4*>(dkv + s * kDqk) + lane;
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    if (c == 2 && !rope) break;
    float4 o = d[64 * c];
    o.x += acc[c][0];
    o.y += acc[c][1];
    o.z += acc[c][2];
    o.w += acc[c][3];
    d[64 * c] = o;
  }
}

__global__ void zero_f32_kernel(float* __restrict__ x, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t j = i; j < n; j += stride) x[j] = 0.f;
}

}  // namespace

int32_t mla_bwd_padded_heads(int32_t H) { return (H + 31) / 32 * 32; }
int32_t mla_bwd_slot_heads(int32_t H) { return (H + 63) / 64 * 64; }

hipError_t launch_zero_f32(float* x, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(zero_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, st, x, n);
  return hipGetLastError();
}

hipError_t launch_sparse_mla_bwd(const MlaBwdArgs& a, int stage, hipStream_t st) {
  if (a.T <= 0) return hipSuccess;
  if (stage == 2) {  // inverted index of the tile's entries, then the per-row sums
    const int64_t n_ent = a.T * (int64_t)a.k;
    hipError_t e = launch_zero_f32((float*)a.row_count, a.N, st);  // int32 zeros
    if (e != hipSuccess) return e;
    int64_t g = (n_ent + 255) / 256;
    g = g > 16384 ? 16384 : g;
    hipLaunchKernelGGL(csr_count_kernel, dim3((unsigned)g), dim3(256), 0, st, a.idx, n_ent, a.N, a.row_count);
    hipLaunchKernelGGL(csr_scan_kernel, dim3(1), dim3(1024), 0, st, a.row_count, a.row_offsets, a.N);
    hipLaunchKernelGGL(csr_fill_kernel, dim3((unsigned)g), dim3(256), 0, st, a.idx, n_ent, a.N, a.row_count,
                       a.row_list);
    hipLaunchKernelGGL(dkv_reduce_kernel, dim3((unsigned)((a.N + 3) / 4)), dim3(256), 0, st, a.row_offsets,
                       a.row_list, a.addend, a.dkv, a.N);
    return hipGetLastError();
  }
  BwdParams p;
  p.q = a.q;
  p.kv = a.kv;
  p.idx = a.idx;
  p.out = a.out;
  p.lse = a.lse;
  p.dout = a.dout;
  p.T = a.T;
  p.N = a.N;
  p.H = a.H;
  p.Hp = mla_bwd_padded_heads(a.H);
  p.Hs = mla_bwd_slot_heads(a.H);
  p.k = a.k;
  p.kp = (a.k + kBlk - 1) / kBlk * kBlk;
  p.kv_bytes = a.N * (int64_t)kDqk * 2 < ((int64_t)1 << 32) ? (uint32_t)(a.N * (int64_t)kDqk * 2) : 0u;
  p.scale = a.scale;
  p.scale_log2 = a.scale * 1.4426950408889634f;
  p.dq = a.dq;
  p.pbuf = a.pbuf;
  p.dsbuf = a.dsbuf;
  p.addend = a.addend;
  if (stage == 0) {
    const int n_half = (p.Hp + 63) / 64;
    const int64_t grid = n_half == 2 ? (a.T + 7) / 8 * 16 : a.T;
    if (p.kv_bytes)
      hipLaunchKernelGGL(mla_bwd_dq_kernel<true>, dim3((unsigned)grid), dim3(kThreads), 0, st, p);
    else
      hipLaunchKernelGGL(mla_bwd_dq_kernel<false>, dim3((unsigned)grid), dim3(kThreads), 0, st, p);
  } else {
    hipLaunchKernelGGL(mla_bwd_dkv_kernel, dim3((unsigned)a.T), dim3(kKvThreads), 0, st, p);
  }
  return hipGetLastError();
}

}  // namespace dsa
