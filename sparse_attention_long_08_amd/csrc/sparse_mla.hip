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
// entries); wave w owns heads 32w .. 32w+31 as the N side of 32x32x16 MFMAs.
// It keeps the query rows of its heads in registers (the B operand of the
// logit product S^T = K Q^T, 32 keys x 32 heads per block) and the fp32
// output O^T (512 x 32, sixteen 32x32 tiles) in the accumulation registers.
//
// Data movement.  Selected latent rows are gathered 32 at a time straight
// from HBM into LDS with the global->LDS DMA (16 bytes per lane, no staging
// registers) into a ring of three stages.  A stage is "band-major": band b
// (4 KB) holds 16-byte chunks 8b .. 8b+7 of all 32 rows, 128 bytes per row,
// with an XOR swizzle of the chunk slot by row.  One DMA instruction then
// moves one band of eight rows, so a wave gathers its eight rows with one
// row lookup, one address and nine DMAs.  The logit product reads rows of a
// stage; the value product O^T = V^T P^T reads the same bytes transposed
// with ds_read_b64_tr_b16, so one copy serves both.
//
// Schedule.  Keys sit on the MFMA rows, so each lane owns one head and the
// softmax statistics are per-lane scalars.  The loop is software pipelined
// by one block: step b runs the logit MFMAs of block b+1 with the softmax of
// block b spread between them, then the value MFMAs of block b.  Operand
// tiles are read from LDS a fixed number of tiles ahead of their MFMA.
// Probabilities are taken against a fixed reference max per head (the max
// of its first block with a valid key), so O is never rescaled inside the
// loop; if a later block max exceeds the reference by more than 2^64 the
// query is recomputed with the true max, which the first pass tracked.  The
// gather uses the buffer-addressed form of the DMA when the latent cache
// spans less than 4 GiB.  A query's blocks end at its last entry with a
// latent row.  The output goes through LDS on its way out, so that every
// store instruction writes 1 KB of one head row.
//
// Small batches (decode) split each query's k entries over several
// workgroups; the partial (out, lse) pairs, out stored in f16 with a
// power-of-two scale per row, are merged by combine_kernel:
// lse = ln sum_i e^{lse_i}, out = sum_i e^{lse_i - lse} out_i.
#include <type_traits>

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
constexpr int kHeadsPerWave = 32;            // the N side of a 32x32x16 MFMA
constexpr int kDmaPerWave = 9;               // one DMA per band, eight rows per wave
constexpr int kKSteps = kDqk / 16;           // 36 k-steps of the logit product
constexpr int kQReg = 28;                    // query k-steps held in registers
constexpr int kQTail = kKSteps - kQReg;      // query k-steps parked in LDS
constexpr int kCt = kDv / 32;                // 16 output tiles of 32 latent dims
constexpr int kMaxK = 4096;                  // entries per query the row table holds
constexpr int kAhead = 6;                    // operand tiles in flight ahead of the one consumed

// ---- the operand stream of one pipeline step.  Slots 0..35 are the logit
// product of the next block (slot i: k-step s_slot_ks(i)), slots 36..67 the
// value product of the current block (slot 36+j: output tile j/2, key half
// j%2).  A slot consumes one "unit" of four registers read from LDS: a key
// tile (one 16-byte read per lane) or a value tile (two 8-byte transposed
// reads); a slot on a query k-step parked in LDS also consumes that query
// tile.  Unit k is read kAhead units before it is consumed.
constexpr int kSSlots = kKSteps;
constexpr int kSlots = kSSlots + 2 * kCt;
constexpr int s_slot_ks(int i) { return i < kQTail ? kQReg + i : i - kQTail; }
constexpr bool slot_loads_q(int i) { return i < kQTail; }
constexpr int slot_units(int i) { return slot_loads_q(i) ? 2 : 1; }
constexpr int slot_first_unit(int i) {
  int u = 0;
  for (int s = 0; s < i; ++s) u += slot_units(s);
  return u;
}
constexpr int kUnits = slot_first_unit(kSlots);
struct UnitDesc {
  int kind;  // 0: key tile of k-step a; 1: query tile of k-step a; 2: value tile (ct a, key half b)
  int a, b;
};
constexpr UnitDesc unit_desc(int k) {
  for (int s = 0; s < kSlots; ++s) {
    const int f = slot_first_unit(s);
    if (k < f || k >= f + slot_units(s)) continue;
    if (s >= kSSlots) return {2, (s - kSSlots) >> 1, (s - kSSlots) & 1};
    if (slot_loads_q(s) && k == f) return {1, s_slot_ks(s), 0};
    return {0, s_slot_ks(s), 0};
  }
  return {-1, 0, 0};
}
constexpr int unit_reads(int k) { return unit_desc(k).kind == 2 ? 2 : 1; }
constexpr int reads_in(int lo, int hi) {
  int n = 0;
  for (int k = lo; k < hi; ++k) n += unit_reads(k);
  return n;
}
constexpr int imin(int a, int b) { return a < b ? a : b; }
// units issued before slot 0, and in slot i (before its MFMAs)
constexpr int issue_lo(int i) { return i == 0 ? kAhead : imin(slot_first_unit(i) + kAhead, kUnits); }
constexpr int issue_hi(int i) { return imin(slot_first_unit(i + 1) + kAhead, kUnits); }
// every unit is read in an earlier slot than the one consuming it
static_assert(kAhead >= 2, "a slot consumes up to two units");

typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s_t __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v4s* lds_v4s_ptr;
typedef __attribute__((address_space(3))) void* lds_ptr;
typedef __attribute__((address_space(3))) uint8_t* lds_u8_ptr;

// Calls f(integral_constant<int, I>) for I = B .. E-1, each as its own
// straight-line code with I a compile-time constant.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// XOR swizzle of the chunk slot within a 128-byte band row, chosen by
// measuring LDS bank conflicts of both operand reads: the 16-byte key-tile
// reads (32 rows, one chunk each) and the transposed 8-byte value-tile reads
// (4 rows x 16 columns per 16-lane group) are conflict-free with it.  For a
// row 16a + 8b + r0 (r0 < 8) it equals swz(r0) ^ 4a ^ 2b.
__device__ __forceinline__ int swz(int r) { return ((r >> 2) ^ (2 * r)) & 7; }

// O^T tile += V^T tile * P^T with the accumulator pinned to the accumulation
// registers (the compiler would otherwise shuttle the 256 accumulators
// between register files around the VALU work of the loop).
__device__ __forceinline__ void mfma_acc_32x32x16(v16f& acc, v8bf a, v8bf b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

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
  uint16_t* part_o;  // f16
  float* part_lse;
  float* part_scale;
};

// Workgroups are handed to the eight XCDs in turn (workgroup b to XCD b % 8),
// and each XCD has an L2 of its own.  This numbering gives XCD x one
// contiguous run of the G logical workgroups, so that the splits of one query
// (every one of which loads the query's rows) and the merge of their partials
// run on one XCD.  It is a bijection of [0, G): XCD x receives the
// q + (x < r) workgroups b = x, x + 8, ... (G = 8q + r).
__device__ __forceinline__ int64_t xcd_major(int64_t b, int64_t G) {
  const int64_t x = b & 7, i = b >> 3, q = G >> 3, r = G & 7;
  return x * q + (x < r ? x : r) + i;
}

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
  __shared__ v8bf qtail[kQTail * kWaves * 64];  // query k-steps kQReg..35 of every wave
  __shared__ int32_t rows[kMaxK];                 // latent row of every entry (-1: skipped)
  __shared__ int32_t wave_last[kWaves];           // last entry with a latent row, per wave
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hn = lane & 31, hh = lane >> 5;  // MFMA column (head) and k-half of this lane
  // split queries: XCD-major numbering (one query's splits on one XCD)
  const int64_t wg = p.n_split > 1 ? xcd_major(blockIdx.x, gridDim.x) : (int64_t)blockIdx.x;
  const int64_t t = wg / p.n_split;
  const int sp = (int)(wg % p.n_split);
  const int j0 = sp * p.per_split;
  const int j1 = min(j0 + p.per_split, p.k);
  const int64_t b = p.seq_per_query ? t : 0;
  int64_t n_b = p.ctx_len ? (int64_t)p.ctx_len[b] : p.seq_len;
  if (n_b > p.seq_len) n_b = p.seq_len;
  const bool active = kHeadsPerWave * wave < p.H;
  const int32_t* idx_row = p.idx + t * (int64_t)p.k;
  const int n_ent = j1 > j0 ? j1 - j0 : 0;
  const int nb_all = (n_ent + kBlk - 1) / kBlk;

  // ---- query rows of this wave's heads in the B layout of the logit
  // MFMA: k-step ks of lane (head hn, half hh) is dims 16*ks + 8*hh .. +7.
  // Lanes past the last head read head H-1 and zero it.  Issued first, so
  // that they are in flight while the entries resolve.
  v8bf qf[kQReg];
  v8bf qt[kQTail];
  const bool q_hv = kHeadsPerWave * wave + hn < p.H;
  {
    const uint16_t* qrow =
        p.q + (t * p.H + (q_hv ? kHeadsPerWave * wave + hn : p.H - 1)) * (int64_t)kDqk + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
      const v8bf v = *(const v8bf*)(qrow + 16 * ks);
      if (ks < kQReg)
        qf[ks < kQReg ? ks : 0] = v;
      else
        qt[ks < kQReg ? 0 : ks - kQReg] = v;
    }
  }

  // ---- resolve every entry to a latent row once (index and page-table
  // loads happen here only, so the block loop issues no other memory
  // reads).  Four entries per thread at a time: their index loads, then
  // their page-table loads, each issued together.
  constexpr int kResolve = 4;
  int32_t last = -1;
  for (int e0 = 0; e0 < nb_all * kBlk; e0 += kResolve * kThreads) {
    int32_t sv[kResolve], pe[kResolve];
#pragma unroll
    for (int u = 0; u < kResolve; ++u) sv[u] = idx_row[j0 + min(e0 + u * kThreads + tid, n_ent - 1)];
#pragma unroll
    for (int u = 0; u < kResolve; ++u) {
      const int e = e0 + u * kThreads + tid;
      sv[u] = (e < n_ent && sv[u] >= 0 && sv[u] < n_b) ? sv[u] : -1;
      pe[u] = addr.lookup(b, sv[u]);
    }
#pragma unroll
    for (int u = 0; u < kResolve; ++u) {
      const int e = e0 + u * kThreads + tid;
      if (e < nb_all * kBlk) {
        const int32_t rv = sv[u] < 0 ? -1 : (int32_t)addr.row_of(b, sv[u], pe[u]);
        rows[e] = rv;
        if (rv >= 0) last = e;  // e grows with u and e0
      }
    }
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) last = max(last, __shfl_xor(last, d, 64));
  if (lane == 0) wave_last[wave] = last;
#pragma unroll
  for (int ks = 0; ks < kQReg; ++ks) qf[ks] = q_hv ? qf[ks] : (v8bf){};
#pragma unroll
  for (int ks = 0; ks < kQTail; ++ks) qtail[(ks * kWaves + wave) * 64 + lane] = q_hv ? qt[ks] : (v8bf){};
  __syncthreads();
  // Blocks up to the last entry with a latent row: the blocks after it hold
  // only skipped entries, which add exact zeros (a selection padded with -1
  // at its end, as for rows with fewer than k candidates, stops early).
  const int nb = (max(max(wave_last[0], wave_last[1]), max(wave_last[2], wave_last[3])) + kBlk) / kBlk;

  // Gather one block into stage `base`: this wave moves rows 8w .. 8w+7, one
  // DMA per band; lane L carries row 8w + L/8, chunk slot L%8 of the band.
  const int g_row = 8 * wave + (lane >> 3);
  const int g_chunk = (lane & 7) ^ swz(g_row);
  // Buffer-addressed DMA when the latent cache spans less than 4 GiB (the
  // host checks): unlike the FLAT form it leaves the compiler's LDS wait
  // counting exact, so operand prefetches are not flushed by every gather.
  const __amdgpu_buffer_rsrc_t kv_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.kv, (short)0, (int)p.kv_bytes, 0x00020000);
  auto gather = [&](uint8_t* base, int32_t row) {
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
  // compile-time immediates).  Key tile of k-step ks: lane (row hn, half hh)
  // reads chunk 2*ks + hh of its row = band ks/4, slot 2*(ks%4) + hh.
  uint32_t k_addr[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) k_addr[q] = (uint32_t)(hn * 128 + (((2 * q + hh) ^ swz(hn)) << 4));
  // Value tile (ct, kt), read hr: the A operand of lane (column c' = 32*ct +
  // hn, half hh) holds keys 16*kt + 8*hr + 4*hh + 0..3.  ds_read_b64_tr_b16
  // hands lane i of a 16-lane group column i of the 4 x 16 block whose rows
  // lane 4*rho + q addresses at columns 4*q .. 4*q+3: lane (group G, rho, q)
  // reads row 16*kt + 8*hr + 4*(G/2) + rho, columns 32*ct + 16*(G%2) + 4*q,
  // i.e. band ct/2, chunk slot 4*(ct%2) + 2*(G%2) + q/2, byte 8*(q%2).  The
  // swizzle of that row is swz(4*(G/2) + rho) ^ 4*kt ^ 2*hr, so the slot is
  // a per-lane base XOR a compile-time mask m = 4*((ct%2)^kt) + 2*hr.
  uint32_t v_addr[4];
  {
    const int grp = lane >> 4, rho = (lane >> 2) & 3, q = lane & 3;
    const int r0 = 4 * (grp >> 1) + rho;
    const int s0 = (2 * (grp & 1) + (q >> 1)) ^ swz(r0);
#pragma unroll
    for (int m = 0; m < 4; ++m) v_addr[m] = (uint32_t)(r0 * 128 + ((s0 ^ (2 * m)) << 4) + 8 * (q & 1));
  }

  v16f o[kCt];
  float m_ref = -INFINITY;  // reference max of this lane's head (log2 units)
  float m_max = -INFINITY;  // largest block max seen
  float l_run;
  bool over = false;        // a logit exceeded its reference by more than 2^64
  uint32_t pbw[2][4];       // bf16 probabilities of the block whose value product is next
  v16f sacc;                // logits of the block whose softmax is next

  auto read_k = [&](const lds_u8_ptr base, int ks) {
    return *(const __attribute__((address_space(3))) v8bf*)(base + k_addr[ks & 3] + kBand * (ks >> 2));
  };
  auto read_q = [&](int ks) {
    return ks < kQReg ? qf[ks < kQReg ? ks : 0] : qtail[((ks < kQReg ? 0 : ks - kQReg) * kWaves + wave) * 64 + lane];
  };
  auto read_v = [&](const lds_u8_ptr base, int ct, int kt) {
    const uint32_t off = kBand * (ct >> 1) + 2048 * kt;
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(base + v_addr[2 * ((ct & 1) ^ kt)] + off));
    const v4s hi =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(base + v_addr[2 * ((ct & 1) ^ kt) + 1] + off + 1024));
    return __builtin_bit_cast(v8bf, (v8s_t){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
  };

  // Logits of one block alone (first block of the pipeline).
  auto logits = [&](const lds_u8_ptr base) {
    constexpr int kPf = 3;  // key-tile reads in flight
    v16f acc = {};
    v8bf abuf[kPf + 1];
#pragma unroll
    for (int ks = 0; ks < kPf; ++ks) abuf[ks] = read_k(base, ks);
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
      if (ks + kPf < kKSteps) abuf[(ks + kPf) % (kPf + 1)] = read_k(base, ks + kPf);
      acc = mfma_bf16_32x32x16(abuf[ks % (kPf + 1)], read_q(ks), acc);
      __builtin_amdgcn_sched_barrier(0);
    }
    sacc = acc;
  };

  // Softmax of the block in sacc (validity bits in `valid`), against a fixed
  // reference max per head: p = 2^(z*log2e - m_ref), so O is never rescaled.
  // m_ref is the max of the head's first block with a valid key (until then
  // nothing has been accumulated, so setting it changes nothing).  A later
  // block max more than 64 above m_ref flags the query; it is then redone with
  // m_ref = the true max, which keeps every p <= 1.  Lane (head hn, half hh)
  // holds keys 8*(r/4) + 4*hh + r%4 of the block in sacc[r].
  //
  // The work is cut into pieces issued one per logit MFMA of the next block,
  // so the VALU and the matrix cores overlap: piece c runs after slot c.
  // Probabilities overwrite sacc; their sum is taken after pb is formed.
  float sm_m = 0.f, sm_neg = 0.f;
  auto sm_piece = [&](auto cc, uint32_t valid) {
    constexpr int c = decltype(cc)::value;
    if constexpr (c == 0) {
      if (valid != 0xFFFFFFFFu) {  // uniform: only partial blocks pay for the mask
        const uint32_t lv = valid >> (4 * hh);
#pragma unroll
        for (int r = 0; r < 16; ++r)
          sacc[r] = ((lv >> (8 * (r >> 2) + (r & 3))) & 1) ? sacc[r] : -INFINITY;
      }
    } else if constexpr (c == 1) {
      float m = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) m = fmaxf(m, sacc[r]);
      sm_m = m;
    } else if constexpr (c == 2) {
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(sm_m), __float_as_uint(sm_m), false, false);
      sm_m = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    } else if constexpr (c == 3) {
      const float mloc = sm_m * p.scale_log2;  // scale > 0 keeps the order
      m_max = fmaxf(m_max, mloc);
      if (m_ref == -INFINITY) m_ref = mloc;
      over |= mloc > m_ref + 64.0f;
      // masked keys: fma(-inf, s, -m) = -inf -> 2^-inf = 0; while m_ref is
      // -inf every logit is -inf, so the bias is 0
      sm_neg = (m_ref == -INFINITY) ? 0.f : -m_ref;
    } else if constexpr (c >= 4 && c < 20) {
      sacc[c - 4] = __builtin_amdgcn_exp2f(fmaf(sacc[c - 4], p.scale_log2, sm_neg));
    } else if constexpr (c >= 20 && c < 24) {
      // B operand of the value MFMA for key half kt: k-slot 8*hh + j is key
      // 16*kt + 8*(j/4) + 4*hh + j%4, i.e. this lane's sacc[8*kt + j]
#pragma unroll
      for (int w = 2 * (c - 20); w < 2 * (c - 20) + 2; ++w)
        pbw[w >> 2][w & 3] = __builtin_bit_cast(
            uint32_t, __builtin_convertvector((v2f){sacc[2 * w], sacc[2 * w + 1]}, v2bf));
    } else if constexpr (c >= 24 && c < 32) {
      l_run += sacc[2 * (c - 24)] + sacc[2 * (c - 24) + 1];
    }
  };

  auto block_valid = [&](int blk) {
    return (uint32_t)(__ballot(rows[blk * kBlk + (lane & 31)] >= 0) & 0xFFFFFFFFull);
  };

  // Row-table values the next step needs, read one step early so that no
  // LDS wait sits between a barrier and the first operand reads: the row
  // this lane gathers for block blk+2, and the entry behind the validity bit
  // of block blk+1 (indexes clamped into the table; values past the last
  // block are never used).
  int32_t g_next = 0, v_next = 0;
  auto read_meta = [&](int blk) {
    g_next = rows[imin((blk + 2) * kBlk + g_row, kMaxK - 1)];
    v_next = rows[imin((blk + 1) * kBlk + (lane & 31), kMaxK - 1)];
  };

  // One pipeline step: wait for this wave's DMA of block blk+1, barrier
  // (every wave's DMA of blk+1 landed and stage (blk+2)%3 -- last read by
  // the value product of blk-1 -- is free), launch the DMA of blk+2 into it,
  // then 68 MFMA slots: 36 of the logit product of blk+1 with the softmax of
  // blk (whose logits the previous step left in sacc) spread over them, then
  // 32 of the value product of blk.  s_barrier is used bare: a fenced
  // __syncthreads() would also wait for the DMA just issued.
  uint32_t valid_cur = 0;
  auto step = [&](uint8_t* cur, uint8_t* nxt, uint8_t* nx2, int blk) {
    const bool more = blk + 1 < nb;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    const lds_u8_ptr vb = (lds_u8_ptr)cur;
    const lds_u8_ptr kb = (lds_u8_ptr)nxt;
    v8bf u[kUnits];
    auto issue = [&](auto kc) {
      constexpr int k = decltype(kc)::value;
      constexpr UnitDesc d = unit_desc(k);
      if constexpr (d.kind == 0)
        u[k] = read_k(kb, d.a);
      else if constexpr (d.kind == 1)
        u[k] = read_q(d.a);
      else
        u[k] = read_v(vb, d.a, d.b);
    };
    static_for<0, kAhead>(issue);
    const int32_t grow = g_next;
    const uint32_t valid_now = valid_cur;
    valid_cur = more ? (uint32_t)(__ballot(v_next >= 0) & 0xFFFFFFFFull) : 0u;
    read_meta(blk + 1);
    if (blk + 2 < nb) gather(nx2, grow);
    v16f snx = {};
    // Each slot first issues the LDS reads of later units, then its MFMA,
    // then its softmax piece.  On the last block the logits read a stale
    // stage and are discarded.
    static_for<0, kSlots>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      constexpr int f = slot_first_unit(i);
      static_for<issue_lo(i), issue_hi(i)>(issue);
      if constexpr (i < kSSlots) {
        constexpr int ks = s_slot_ks(i);
        const v8bf qb = ks < kQReg ? qf[ks < kQReg ? ks : 0] : u[f];
        snx = mfma_bf16_32x32x16(u[slot_loads_q(i) ? f + 1 : f], qb, snx);
      } else {
        constexpr int j = i - kSSlots;
        mfma_acc_32x32x16(o[j >> 1], u[f], __builtin_bit_cast(v8bf, pbw[j & 1]));
      }
      // pin the slot's order: its LDS reads, then its MFMA, then the VALU piece
      constexpr int nreads = reads_in(issue_lo(i), issue_hi(i));
      if constexpr (nreads > 0) __builtin_amdgcn_sched_group_barrier(0x100, nreads, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      sm_piece(ic, valid_now);
      __builtin_amdgcn_sched_barrier(0);
    });
    sacc = snx;
  };

  for (int pass = 0;; ++pass) {
    l_run = 0.f;
#pragma unroll
    for (int ct = 0; ct < kCt; ++ct) o[ct] = (v16f){};
    // ---- prologue: blocks 0 and 1 in flight, logits of block 0
    if (nb > 0) gather(kb0, rows[g_row]);
    if (nb > 1) gather(kb1, rows[kBlk + g_row]);
    read_meta(0);
    if (nb > 1)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kDmaPerWave) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    if (nb > 0) {
      logits((lds_u8_ptr)kb0);
      valid_cur = block_valid(0);
    }
    run_ring(kb0, kb1, kb2, nb, step);
    // the value MFMAs are inline asm, so the compiler does not know that
    // their accumulators are written late: cover the MFMA-write to
    // VALU-read/write distance before O is read or cleared
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    // every wave is past its last read of the stages here, and no DMA is outstanding
    if (pass > 0 || !__syncthreads_or(over ? 1 : 0)) break;
    m_ref = m_max;
    over = false;
  }

  // every wave is past its last read of the stages and of qtail: the
  // epilogue stages the output through them
  __syncthreads();
  if (!active) return;
  const int head = kHeadsPerWave * wave + hn;
  const bool head_ok = head < p.H;
  const int n_heads = min(kHeadsPerWave, p.H - kHeadsPerWave * wave);  // heads of this wave (>= 1)
  const auto lr = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
  const float l_tot = __uint_as_float(lr[0]) + __uint_as_float(lr[1]);
  const bool empty = !(l_tot > 0.f);
  const float inv = empty ? 0.f : 1.f / l_tot;
  const float lse_v = empty ? -INFINITY : (m_ref + log2f(l_tot)) * 0.69314718055994530942f;
  // O^T tile ct: lane (head hn, half hh) holds c' = 32*ct + 8*(r/4) + 4*hh + r%4
  auto o4 = [&](int ct, int r4) {
    return (v4f){o[ct][4 * r4], o[ct][4 * r4 + 1], o[ct][4 * r4 + 2], o[ct][4 * r4 + 3]};
  };
  // The wave's output goes through 32 KB of LDS of its own (a stage, or the
  // query tail for wave 3): 32 head rows of 1 KB whose 16-byte chunks are
  // XOR-swizzled by head, so that the writes from the MFMA layout spread over
  // the banks and each row reads back conflict-free; every global store then
  // writes 1 KB of one head row.
  uint8_t* stage = wave == 0 ? kb0 : (wave == 1 ? kb1 : (wave == 2 ? kb2 : reinterpret_cast<uint8_t*>(qtail)));
  auto chunk = [&](int j, int c) -> uint8_t* { return stage + 1024 * j + 16 * (c ^ (j & 31)); };
  auto wave_sync = [] {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  if (p.n_split == 1) {
    float* obase = p.out + (t * p.H + kHeadsPerWave * wave) * (int64_t)kDv;
#pragma unroll
    for (int half = 0; half < 2; ++half) {  // dims 256 half .. +255, 4 per chunk
#pragma unroll
      for (int ct = 0; ct < kCt / 2; ++ct)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          *(v4f*)chunk(hn, 8 * ct + 2 * r4 + hh) = o4(kCt / 2 * half + ct, r4) * inv;
      wave_sync();
      for (int j = 0; j < n_heads; ++j)
        *(v4f*)(obase + j * (int64_t)kDv + 256 * half + 4 * lane) = *(const v4f*)chunk(j, lane);
      wave_sync();
    }
    if (hh == 0 && head_ok) p.lse[t * p.H + head] = lse_v;
    return;
  }
  // A split's partial: the normalised output in f16, times 2^-e with e >= 0
  // the smallest that brings the head's largest |value| to at most 2^15
  // (2^e kept beside its lse; e = 0 unless the latent values are that large).
  float amax = 0.f;
#pragma unroll
  for (int ct = 0; ct < kCt; ++ct)
#pragma unroll
    for (int r = 0; r < 16; ++r) amax = fmaxf(amax, __builtin_fabsf(o[ct][r]));
  amax *= inv;
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(amax), __float_as_uint(amax), false, false);
    amax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));  // both halves of the head
  }
  const int e = (amax > 32768.f && amax < INFINITY) ? ilogbf(amax) - 14 : 0;
  const float sc = inv * ldexpf(1.f, -e);
  const int64_t prow0 = (t * p.n_split + sp) * p.H + kHeadsPerWave * wave;
  // dims 8 c .. 8 c + 7 of a head row form chunk c; lane (hn, hh) fills half hh
#pragma unroll
  for (int ct = 0; ct < kCt; ++ct)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
      *(v4h*)(chunk(hn, 4 * ct + r4) + 8 * hh) = __builtin_convertvector(o4(ct, r4) * sc, v4h);
  wave_sync();
  _Float16* pbase = reinterpret_cast<_Float16*>(p.part_o) + prow0 * (int64_t)kDv;
  for (int j = 0; j < n_heads; ++j)
    *(v8h*)(pbase + j * (int64_t)kDv + 8 * lane) = *(const v8h*)chunk(j, lane);
  if (hh == 0 && head_ok) {
    p.part_lse[prow0 + hn] = lse_v;
    p.part_scale[prow0 + hn] = ldexpf(1.f, e);
  }
}

// Merge of split partials; one wave per (t, head), four per workgroup, each
// lane merging 8 consecutive dims.  Every split's lse, scale and partial
// slice are loaded before any is used (one memory round trip per wave), then
// merged in split order.
constexpr int kMaxSplits = 16;

__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ part_o,
                                                      const float* __restrict__ part_lse,
                                                      const float* __restrict__ part_scale, int64_t T, int32_t H,
                                                      int32_t n_split, float* __restrict__ out,
                                                      float* __restrict__ lse) {
  // XCD-major like the split attention: a query's merge runs on the XCD that wrote its partials
  const int64_t th = xcd_major(blockIdx.x, gridDim.x) * 4 + (threadIdx.x >> 6);  // t * H + h
  if (th >= T * H) return;
  const int ln = threadIdx.x & 63;
  const int64_t t = th / H;
  const int h = (int)(th % H);
  float li[kMaxSplits], scl[kMaxSplits];
  v8h v[kMaxSplits];
#pragma unroll
  for (int i = 0; i < kMaxSplits; ++i) {
    if (i < n_split) {
      const int64_t prow = (t * n_split + i) * H + h;
      li[i] = part_lse[prow];
      scl[i] = part_scale[prow];
      v[i] = *(const v8h*)(reinterpret_cast<const _Float16*>(part_o) + prow * (int64_t)kDv + 8 * ln);
    }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < kMaxSplits; ++i)
    if (i < n_split) mx = fmaxf(mx, li[i]);
  float wsum = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxSplits; ++i)
    if (i < n_split) wsum += (li[i] == -INFINITY) ? 0.f : expf(li[i] - mx);
  const bool empty = !(wsum > 0.f);
  const float lse_tot = empty ? -INFINITY : mx + logf(wsum);
  v4f acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
#pragma unroll
  for (int i = 0; i < kMaxSplits; ++i) {
    if (i < n_split && li[i] != -INFINITY) {
      const float wgt = expf(li[i] - lse_tot) * scl[i];
      acc0 += wgt * __builtin_convertvector(v[i].lo, v4f);
      acc1 += wgt * __builtin_convertvector(v[i].hi, v4f);
    }
  }
  *(v4f*)(out + th * (int64_t)kDv + 8 * ln) = acc0;
  *(v4f*)(out + th * (int64_t)kDv + 8 * ln + 4) = acc1;
  if (ln == 0) lse[th] = lse_tot;
}

// Each split keeps at least kMinSplitKeys entries: a split's fixed cost (query
// load, entry resolution, partial write and merge) outweighs further
// parallelism below that.  Measured on MI355X, 32 queries x 2048 entries:
// attention + combine 50.3 us with 8 splits against 51.6 us with 4 (with the
// output staged through LDS and f16 partials; 62 against 58 us before them).
constexpr int kMinSplitKeys = 256;

int32_t sparse_mla_splits(int64_t T, int32_t /*H*/, int32_t k) {
  if (T >= 256) return 1;
  int64_t s = (256 + T - 1) / T;
  const int64_t max_s = k / kMinSplitKeys;
  if (s > max_s) s = max_s;
  if (s > kMaxSplits) s = kMaxSplits;
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
  p.part_scale = a.part_scale;
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
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((a.T * a.H + 3) / 4)), dim3(256), 0, st, a.part_o, a.part_lse,
                     a.part_scale, a.T, a.H, p.n_split, a.out, a.lse);
  return hipGetLastError();
}

}  // namespace dsa
