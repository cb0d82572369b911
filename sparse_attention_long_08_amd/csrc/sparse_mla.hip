// Sparse MLA attention in MQA mode on gfx950 bf16 matrix cores.
//
// DeepSeek Sparse Attention attends only over the top-k selected latent KV
// rows of each query ("DeepSeek-V3.2" report walk-through, §2.1.2 attention
// equation), and in MLA's MQA mode every latent row is shared by all query
// heads of the token (§2.2).  Per query t and head h:
//   z_s = scale * q[t,h,:576] . kv[s,:576],  s in S_t
//   out[t,h] = sum_s softmax(z)_s * kv[s,:512],  lse[t,h] = ln sum_s exp(z_s)
//
// Mapping.  One workgroup of 4 waves owns one query (or one split of its
// entries); wave w owns heads 32w .. 32w+31 as two 16-head MFMA tiles, keeps
// their query rows in registers (the B operand of the logit product) and
// their fp32 output accumulators O^T (512 x 32) in accumulation registers.
// Every operand read from LDS feeds both head tiles, so the LDS bytes per
// flop are those of a 32-head tile.
//
// Data movement.  Selected latent rows are gathered 32 at a time straight
// from HBM into LDS with the global->LDS DMA (16 bytes per lane, no staging
// registers) into a ring of three stages.  A stage is "band-major": band b
// (4 KB) holds 16-byte chunks 8b .. 8b+7 of all 32 rows, 128 bytes per row,
// with an XOR swizzle of the chunk slot by row.  One DMA instruction then
// moves one band of eight rows, so a wave gathers its eight rows with one
// row lookup, one address and nine DMAs.  The logits S^T = K Q^T read rows
// of a stage; the value product O^T = V^T P^T reads the same bytes
// transposed with ds_read_b64_tr_b16, so one copy serves both.
//
// Schedule.  Keys sit on the MFMA rows, so each lane owns single heads and
// the softmax statistics are per-lane scalars.  The loop is software
// pipelined by one block: step b issues the value MFMAs of block b and the
// logit MFMAs of block b+1 interleaved (operand reads a few slots ahead),
// then the softmax of block b+1.  Probabilities are taken against a fixed
// reference max per head (the max of its first block with a valid key), so
// O is never rescaled inside the loop; if a later block max exceeds the
// reference by more than 2^64 the query is recomputed with the true max,
// which the first pass tracked.  The gather uses the buffer-addressed form of
// the DMA when the latent cache spans less than 4 GiB.
//
// Small batches (decode) split each query's k entries over several
// workgroups; partial (out, lse) pairs are merged exactly by combine_kernel:
// lse = ln sum_i e^{lse_i}, out = sum_i e^{lse_i - lse} out_i.
#include "common.h"
#include "launch.h"

namespace dsa {

constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kBlk = 32;                     // selected rows per block
constexpr int kBufBytes = kBlk * kDqk * 2;   // 36864 bytes per stage
constexpr int kBand = 4096;                  // bytes per 8-chunk band of a stage
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kHeadsPerWave = 32;            // two 16-head MFMA tiles
constexpr int kDmaPerWave = 9;               // one DMA per band, eight rows per wave
constexpr int kQReg = 16;                    // query k-steps held in registers (the 512 latent dims)
constexpr int kQTail = 18 - kQReg;           // query k-steps parked in LDS (the 64 rope dims)
constexpr int kMaxK = 4096;                  // entries per query the row table holds
constexpr int kPfS = 1;                      // logit operand reads issued this many slots ahead
constexpr int kPfP = 3;                      // value operand reads issued this many slots ahead

typedef short v4s __attribute__((ext_vector_type(4)));
typedef float v8f __attribute__((ext_vector_type(8)));
typedef short v8s_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4s* lds_v4s_ptr;
typedef __attribute__((address_space(3))) void* lds_ptr;
typedef __attribute__((address_space(3))) uint8_t* lds_u8_ptr;

// XOR swizzle of the chunk slot within a 128-byte band row: the rows read
// together by an operand load land on distinct banks.
__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 2)) & 7; }

struct MlaParams {
  const uint16_t* q;
  const uint16_t* kv;
  uint32_t kv_bytes;  // extent of the latent cache when it is below 4 GiB (buffer DMA), else 0
  const int32_t* idx;
  const int32_t* ctx_len;
  int64_t seq_len;
  int32_t seq_per_query;
  int64_t T;
  int32_t H;
  int32_t k;
  float scale_log2;  // scale * log2(e)
  int32_t n_split;
  int32_t per_split;
  float* out;
  float* lse;
  float* part_o;
  float* part_lse;
};

// Drives the pipeline over the three stage buffers.  They arrive as
// restrict-qualified parameters: after inlining, every access through them
// carries alias-scope metadata, which lets the compiler see that the stages
// being read are not the stage a DMA is still writing.
template <class Step>
__device__ __forceinline__ void run_ring(uint8_t* __restrict__ kb0, uint8_t* __restrict__ kb1,
                                         uint8_t* __restrict__ kb2, int nb, Step& step) {
  for (int blk = 0; blk < nb; blk += 3) {
    step(kb0, kb1, kb2, blk);
    if (blk + 1 < nb) step(kb1, kb2, kb0, blk + 1);
    if (blk + 2 < nb) step(kb2, kb0, kb1, blk + 2);
  }
}

template <class Addr, bool kBufDma>
__global__ __launch_bounds__(kThreads, 1) void sparse_mla_kernel(MlaParams p, Addr addr) {
  __shared__ __attribute__((aligned(16))) uint8_t kb0[kBufBytes];
  __shared__ __attribute__((aligned(16))) uint8_t kb1[kBufBytes];
  __shared__ __attribute__((aligned(16))) uint8_t kb2[kBufBytes];
  __shared__ v8bf qtail[kQTail * 2 * kWaves * 64];  // query steps kQReg..17 of every head tile
  __shared__ int32_t rows[kMaxK];                      // latent row of every entry (-1: skipped)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = lane >> 4, hl = lane & 15;
  const int64_t t = blockIdx.x / p.n_split;
  const int sp = blockIdx.x % p.n_split;
  const int j0 = sp * p.per_split;
  const int j1 = min(j0 + p.per_split, p.k);
  const int64_t b = p.seq_per_query ? t : 0;
  int64_t n_b = p.ctx_len ? (int64_t)p.ctx_len[b] : p.seq_len;
  if (n_b > p.seq_len) n_b = p.seq_len;
  const bool active = kHeadsPerWave * wave < p.H;
  const int32_t* idx_row = p.idx + t * (int64_t)p.k;
  const int n_ent = j1 > j0 ? j1 - j0 : 0;
  const int nb = (n_ent + kBlk - 1) / kBlk;

  // ---- resolve every entry to a latent row once (index and page-table
  // loads happen here only, so the block loop issues no other memory reads)
  for (int e = tid; e < nb * kBlk; e += kThreads) {
    int32_t row = -1;
    if (e < n_ent) {
      const int32_t s = idx_row[j0 + e];
      if (s >= 0 && s < n_b) row = (int32_t)addr.row(b, s);
    }
    rows[e] = row;
  }

  // ---- query rows of this wave's head tiles: step st covers dims
  // 32*st + 8*g4 .. +7.  Lanes past the last head read head H-1 and zero it.
  v8bf qf[2][kQReg];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int head = kHeadsPerWave * wave + 16 * nt + hl;
    const bool hv = head < p.H;
    const uint16_t* qrow = p.q + (t * p.H + (hv ? head : p.H - 1)) * (int64_t)kDqk + 8 * g4;
#pragma unroll
    for (int st = 0; st < kQReg; ++st) {
      const v8bf v = *(const v8bf*)(qrow + 32 * st);
      qf[nt][st] = hv ? v : (v8bf){};
    }
#pragma unroll
    for (int st = kQReg; st < 18; ++st) {
      const v8bf v = *(const v8bf*)(qrow + 32 * st);
      qtail[(((st - kQReg) * 2 + nt) * kWaves + wave) * 64 + lane] = hv ? v : (v8bf){};
    }
  }
  __syncthreads();

  // Gather block `blk` into stage `base`: this wave moves rows 8w .. 8w+7,
  // one DMA per band; lane L carries row 8w + L/8, chunk slot L%8 of the band.
  const int g_row = 8 * wave + (lane >> 3);
  const int g_chunk = (lane & 7) ^ swz(g_row);
  // Buffer-addressed DMA when the latent cache spans less than 4 GiB (the
  // host checks): unlike the FLAT form it leaves the compiler's LDS wait
  // counting exact, so operand prefetches are not flushed by every gather.
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

  // ---- per-lane LDS byte offsets of the operand reads (the rest are
  // compile-time immediates).  Logits: M-tile mt reads key row 16*mt + hl,
  // chunk 4*st + g4, i.e. band st/2, band slot 4*(st%2) + g4.
  uint32_t s_addr[2][2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int r = 16 * mt + hl;
#pragma unroll
    for (int par = 0; par < 2; ++par) s_addr[mt][par] = (uint32_t)(r * 128 + (((4 * par + g4) ^ swz(r)) << 4));
  }
  // Values: for c'-tile ct, lane (g4, 4*rq + qq) supplies columns
  // 16*ct + 4*qq .. +3 of key rows 4*g4 + rq (k-slots 0..3) and
  // 16 + 4*g4 + rq (k-slots 4..7): chunk 2*ct + qq/2 = band ct/4, slot
  // 2*(ct%4) + qq/2, byte 8*(qq%2) within the chunk.
  uint32_t v_addr[2][4];
  {
    const int rq = hl >> 2, qq = hl & 3;
#pragma unroll
    for (int hv = 0; hv < 2; ++hv) {
      const int r = 16 * hv + 4 * g4 + rq;
#pragma unroll
      for (int m4 = 0; m4 < 4; ++m4)
        v_addr[hv][m4] = (uint32_t)(r * 128 + (((2 * m4 + (qq >> 1)) ^ swz(r)) << 4) + 8 * (qq & 1));
    }
  }

  v4f o[2][32];
  float m_ref[2] = {-INFINITY, -INFINITY};  // reference max of each head (log2 units)
  float m_max[2] = {-INFINITY, -INFINITY};  // largest block max seen
  float l_run[2];
  bool over = false;                         // a logit exceeded its reference by more than 2^64
  v8bf pb[2];                                // probabilities of the block whose value product is next
  v4f sacc[2][2];

  auto read_a = [&](const lds_u8_ptr base, int st, int mt) {
    return *(const __attribute__((address_space(3))) v8bf*)(base + s_addr[mt][st & 1] + kBand * (st >> 1));
  };
  auto read_q = [&](int st, int nt) {
    return st < kQReg ? qf[nt][st < kQReg ? st : 0]
                      : qtail[(((st < kQReg ? 0 : st - kQReg) * 2 + nt) * kWaves + wave) * 64 + lane];
  };
  auto read_v = [&](const lds_u8_ptr base, int ct) {
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(base + v_addr[0][ct & 3] + kBand * (ct >> 2)));
    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(base + v_addr[1][ct & 3] + kBand * (ct >> 2)));
    return __builtin_bit_cast(v8bf, (v8s_t){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
  };

  // Logits of one block alone (first block of the pipeline).
  auto logits = [&](const lds_u8_ptr base) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) sacc[mt][nt] = (v4f){0.f, 0.f, 0.f, 0.f};
    v8bf abuf[kPfS + 1][2];
#pragma unroll
    for (int st = 0; st < kPfS; ++st)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) abuf[st][mt] = read_a(base, st, mt);
#pragma unroll
    for (int st = 0; st < 18; ++st) {
      if (st + kPfS < 18)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) abuf[(st + kPfS) % (kPfS + 1)][mt] = read_a(base, st + kPfS, mt);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          sacc[mt][nt] = mfma_bf16_16x16x32(abuf[st % (kPfS + 1)][mt], read_q(st, nt), sacc[mt][nt]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Softmax of the block in sacc (validity bits in `valid`), against a fixed
  // reference max per head: p = 2^(z*log2e - m_ref), so O is never rescaled.
  // m_ref is the max of the head's first block with a valid key (until then
  // nothing has been accumulated, so setting it changes nothing).  A later
  // block max more than 64 above m_ref flags the query; it is then redone with
  // m_ref = the true max, which keeps every p <= 1.  lane: heads (nt, hl);
  // sacc[mt][nt][i] is key 16*mt + 4*g4 + i of the block.
  auto softmax = [&](uint32_t valid) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      float mloc = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = 16 * mt + 4 * g4 + i;
          sacc[mt][nt][i] = ((valid >> key) & 1) ? sacc[mt][nt][i] : -INFINITY;
          mloc = fmaxf(mloc, sacc[mt][nt][i]);
        }
      mloc = fmaxf(mloc, shfl_xor_f(mloc, 16));
      mloc = fmaxf(mloc, shfl_xor_f(mloc, 32));
      mloc *= p.scale_log2;  // scale > 0 keeps the order
      m_max[nt] = fmaxf(m_max[nt], mloc);
      if (m_ref[nt] == -INFINITY) m_ref[nt] = mloc;
      over |= mloc > m_ref[nt] + 64.0f;
      // masked keys: fma(-inf, s, -m) = -inf -> 2^-inf = 0; while m_ref is
      // -inf every logit is -inf, so the bias is 0
      const float mneg = (m_ref[nt] == -INFINITY) ? 0.f : -m_ref[nt];
      v8f pf;
      float lsum = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float pv = __builtin_amdgcn_exp2f(fmaf(sacc[i >> 2][nt][i & 3], p.scale_log2, mneg));
        lsum += pv;
        pf[i] = pv;
      }
      l_run[nt] += lsum;
      // B operand of the value MFMA: k-slot 8*g4 + j <-> key 4*g4 + j (j < 4),
      // 16 + 4*g4 + (j - 4) (j >= 4): exactly this lane's probabilities
      pb[nt] = __builtin_convertvector(pf, v8bf);
    }
  };

  auto block_valid = [&](int blk) {
    return (uint32_t)(__ballot(rows[blk * kBlk + (lane & 31)] >= 0) & 0xFFFFFFFFull);
  };

  // One pipeline step: wait for this wave's DMA of block blk+1, barrier
  // (every wave's DMA of blk+1 landed and stage (blk+2)%3 -- last read by
  // the value product of blk-1 -- is free), launch the DMA of blk+2 into it,
  // then value product of blk interleaved with the logits of blk+1, and the
  // softmax of blk+1.  s_barrier is used bare: a fenced __syncthreads()
  // would also wait for the DMA just issued.
  auto step = [&](uint8_t* cur, uint8_t* nxt, uint8_t* nx2, int blk) {
    const bool more = blk + 1 < nb;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    if (blk + 2 < nb) gather(nx2, blk + 2);
    const uint32_t valid_next = block_valid(more ? blk + 1 : blk);
    const lds_u8_ptr vb = (lds_u8_ptr)cur;
    const lds_u8_ptr kb = (lds_u8_ptr)nxt;
    // 36 slots: slot i issues the logit MFMAs of one (k-step, M-tile) pair
    // of block blk+1 and, for i < 32, the value MFMAs of c'-tile i of block
    // blk.  The logit k-steps run in the order 16, 17, 0, 1, .., 15 so the
    // two query steps parked in LDS are read with the initial prefetch.  Each
    // slot first issues the LDS reads of slot i + PF, then its four MFMAs.
    // On the last block the logits read a stale stage and are discarded.
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) sacc[mt][nt] = (v4f){0.f, 0.f, 0.f, 0.f};
    auto slot_st = [](int i) { return (i >> 1) < kQTail ? kQReg + (i >> 1) : (i >> 1) - kQTail; };
    v8bf qt[kQTail][2];
#pragma unroll
    for (int j = 0; j < kQTail; ++j)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) qt[j][nt] = read_q(kQReg + j, nt);
    v8bf abuf[kPfS + 1];
    v8bf vbuf[kPfP + 1];
#pragma unroll
    for (int i = 0; i < kPfS; ++i) abuf[i] = read_a(kb, slot_st(i), i & 1);
#pragma unroll
    for (int i = 0; i < kPfP; ++i) vbuf[i] = read_v(vb, i);
#pragma unroll
    for (int i = 0; i < 36; ++i) {
      int nreads = 0;
      if (i + kPfS < 36) {
        abuf[(i + kPfS) % (kPfS + 1)] = read_a(kb, slot_st(i + kPfS), (i + kPfS) & 1);
        nreads += 1;
      }
      if (i + kPfP < 32) {
        vbuf[(i + kPfP) % (kPfP + 1)] = read_v(vb, i + kPfP);
        nreads += 2;
      }
      const int st = slot_st(i), mt = i & 1;
      int nmfma = 0;
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const v8bf qb = st < kQReg ? qf[nt][st < kQReg ? st : 0] : qt[st < kQReg ? 0 : st - kQReg][nt];
        sacc[mt][nt] = mfma_bf16_16x16x32(abuf[i % (kPfS + 1)], qb, sacc[mt][nt]);
        nmfma += 1;
      }
      if (i < 32) {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) o[nt][i] = mfma_bf16_16x16x32(vbuf[i % (kPfP + 1)], pb[nt], o[nt][i]);
        nmfma += 2;
      }
      // pin the slot's order: its LDS reads, then its MFMAs
      if (nreads == 3) __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
      if (nreads == 2) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      if (nreads == 1) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      if (nmfma == 4) __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      if (nmfma == 2) __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (more) softmax(valid_next);
  };

  for (int pass = 0;; ++pass) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      l_run[nt] = 0.f;
#pragma unroll
      for (int i = 0; i < 32; ++i) o[nt][i] = (v4f){0.f, 0.f, 0.f, 0.f};
    }
    // ---- prologue: blocks 0 and 1 in flight, logits and softmax of block 0
    if (nb > 0) gather(kb0, 0);
    if (nb > 1) gather(kb1, 1);
    if (nb > 1)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kDmaPerWave) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    if (nb > 0) {
      logits((lds_u8_ptr)kb0);
      softmax(block_valid(0));
    }
    run_ring(kb0, kb1, kb2, nb, step);
    // every wave is past its last read of the stages here, and no DMA is outstanding
    if (pass > 0 || !__syncthreads_or(over ? 1 : 0)) break;
    m_ref[0] = m_max[0];
    m_ref[1] = m_max[1];
    over = false;
  }

  if (!active) return;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int head = kHeadsPerWave * wave + 16 * nt + hl;
    float l_tot = l_run[nt] + shfl_xor_f(l_run[nt], 16);
    l_tot += shfl_xor_f(l_tot, 32);
    if (head >= p.H) continue;
    const bool empty = !(l_tot > 0.f);
    const float inv = empty ? 0.f : 1.f / l_tot;
    const float lse_v = empty ? -INFINITY : (m_ref[nt] + log2f(l_tot)) * 0.69314718055994530942f;
    float* orow;
    float* lrow;
    if (p.n_split == 1) {
      orow = p.out + (t * p.H + head) * (int64_t)kDv;
      lrow = p.lse + t * p.H + head;
    } else {
      orow = p.part_o + ((t * p.n_split + sp) * p.H + head) * (int64_t)kDv;
      lrow = p.part_lse + (t * p.n_split + sp) * p.H + head;
    }
    // O^T layout: lane (g4, head hl) holds c' = 16*ct + 4*g4 + i
#pragma unroll
    for (int ct = 0; ct < 32; ++ct) *(v4f*)(orow + 16 * ct + 4 * g4) = o[nt][ct] * inv;
    if (g4 == 0) *lrow = lse_v;
  }
}

// Exact merge of split partials; one workgroup of 128 threads per (t, head).
__global__ __launch_bounds__(128) void combine_kernel(const float* __restrict__ part_o,
                                                      const float* __restrict__ part_lse, int64_t T, int32_t H,
                                                      int32_t n_split, float* __restrict__ out,
                                                      float* __restrict__ lse) {
  const int64_t th = blockIdx.x;  // t * H + h
  const int64_t t = th / H;
  const int h = (int)(th % H);
  float mx = -INFINITY;
  for (int i = 0; i < n_split; ++i) mx = fmaxf(mx, part_lse[(t * n_split + i) * H + h]);
  float wsum = 0.f;
  for (int i = 0; i < n_split; ++i) {
    const float li = part_lse[(t * n_split + i) * H + h];
    wsum += (li == -INFINITY) ? 0.f : expf(li - mx);
  }
  const bool empty = !(wsum > 0.f);
  const float lse_tot = empty ? -INFINITY : mx + logf(wsum);
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < n_split; ++i) {
    const float li = part_lse[(t * n_split + i) * H + h];
    if (li == -INFINITY) continue;
    const float wgt = expf(li - lse_tot);
    const v4f v = *(const v4f*)(part_o + ((t * n_split + i) * H + h) * (int64_t)kDv + 4 * threadIdx.x);
    acc += wgt * v;
  }
  *(v4f*)(out + th * (int64_t)kDv + 4 * threadIdx.x) = acc;
  if (threadIdx.x == 0) lse[th] = lse_tot;
}

int32_t sparse_mla_splits(int64_t T, int32_t /*H*/, int32_t k) {
  if (T >= 256) return 1;
  int64_t s = (256 + T - 1) / T;
  const int64_t max_s = (k + kBlk - 1) / kBlk;
  if (s > max_s) s = max_s;
  if (s > 16) s = 16;
  return (int32_t)(s < 1 ? 1 : s);
}

namespace {
template <class Addr>
hipError_t launch_mla(const MlaParams& p, Addr addr, hipStream_t st) {
  const int64_t blocks = p.T * p.n_split;
  if (p.kv_bytes != 0)
    hipLaunchKernelGGL((sparse_mla_kernel<Addr, true>), dim3((unsigned)blocks), dim3(kThreads), 0, st, p, addr);
  else
    hipLaunchKernelGGL((sparse_mla_kernel<Addr, false>), dim3((unsigned)blocks), dim3(kThreads), 0, st, p, addr);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_sparse_mla(const MlaArgs& a, hipStream_t st) {
  if (a.T <= 0) return hipSuccess;
  MlaParams p;
  p.q = a.q;
  p.kv = a.kv;
  // rows the addressing can reach: the page pool, or the contiguous cache
  const int64_t kv_rows = a.paged ? a.paged->n_pages * (int64_t)a.paged->page_size
                                  : (a.seq_per_query ? a.T : 1) * (a.stride > a.seq_len ? a.stride : a.seq_len);
  const uint64_t extent = (uint64_t)kv_rows * kDqk * 2;
  p.kv_bytes = extent < 0xFFFFFFFFull ? (uint32_t)extent : 0u;
  p.idx = a.idx;
  p.ctx_len = a.ctx_len;
  p.seq_len = a.seq_len;
  p.seq_per_query = a.seq_per_query ? 1 : 0;
  p.T = a.T;
  p.H = a.H;
  p.k = a.k;
  p.scale_log2 = a.scale * 1.44269504088896340736f;
  p.n_split = a.n_split < 1 ? 1 : a.n_split;
  const int per = (a.k + p.n_split - 1) / p.n_split;
  p.per_split = ((per + kBlk - 1) / kBlk) * kBlk;
  p.out = a.out;
  p.lse = a.lse;
  p.part_o = a.part_o;
  p.part_lse = a.part_lse;
  hipError_t e;
  if (a.paged) {
    AddrPaged ad{a.paged->page_table, a.paged->max_pages, __builtin_ctz((unsigned)a.paged->page_size),
                 a.paged->n_pages};
    e = launch_mla(p, ad, st);
  } else {
    AddrBatched ad{a.stride};
    e = launch_mla(p, ad, st);
  }
  if (e != hipSuccess || p.n_split == 1) return e;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)(a.T * a.H)), dim3(128), 0, st, a.part_o, a.part_lse, a.T,
                     a.H, p.n_split, a.out, a.lse);
  return hipGetLastError();
}

}  // namespace dsa
