// Sparse MLA attention in MQA mode on gfx950 bf16 matrix cores.
//
// DeepSeek Sparse Attention attends only over the top-k selected latent KV
// rows of each query ("DeepSeek-V3.2" report walk-through, §2.1.2 attention
// equation), and in MLA's MQA mode every latent row is shared by all query
// heads of the token (§2.2).  Per query t and head h:
//   z_s = scale * q[t,h,:576] . kv[s,:576],  s in S_t
//   out[t,h] = sum_s softmax(z)_s * kv[s,:512],  lse[t,h] = ln sum_s exp(z_s)
//
// Mapping: one workgroup (4 waves) owns one query and all its heads; wave w
// owns heads 32w..32w+31, keeps their query rows in VGPRs (the MFMA B operand
// of the logit product) and their fp32 output accumulators (512 x 32) in
// accumulation registers.  Selected latent rows are gathered 32 at a time
// straight from HBM into LDS with the gfx950 global->LDS DMA (16 bytes per
// lane, no staging registers), double buffered so the next block streams in
// while the current one is consumed.  The LDS copy is row-major in 16-byte
// chunks with an XOR swizzle; the logits S^T = K Q^T read it as rows, and
// the value product O^T = V^T P^T reads the same bytes transposed with
// ds_read_b64_tr_b16, so one copy serves both.  Putting keys on the MFMA
// rows makes each lane own a single head: softmax statistics are per-lane
// scalars, the probabilities feed the value MFMA's B operand directly from
// the logit accumulator layout (a key permutation mirrored in the transposed
// V reads), and a rescale is one multiply per accumulator.  The running max
// only moves when it grows by more than 2^8 (exact: the final normalisation
// uses the same max), so rescales are rare.
// Small batches (decode) split each query's k entries over several
// workgroups; partial (out, lse) pairs are merged exactly by combine_kernel:
// lse = ln sum_i e^{lse_i}, out = sum_i e^{lse_i - lse} out_i.
#include "common.h"
#include "launch.h"

namespace dsa {

constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kBlk = 32;                     // selected rows per block
constexpr int kChunks = kDqk / 8;            // 16-byte chunks per latent row (72)
constexpr int kBufBytes = kBlk * kDqk * 2;   // 36864 bytes per buffer
constexpr int kHeadsPerWave = 16;               // 8 waves x 16 heads
constexpr int kStages = 3;                      // LDS pipeline depth
constexpr int kDmaPerWave = 5;                  // ceil(36 DMA instructions / 8 waves)
constexpr int kMaxK = 4096;                     // entries per query the row table holds

typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef float v8f __attribute__((ext_vector_type(8)));
typedef short v8s_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4s* lds_v4s_ptr;
typedef __attribute__((address_space(3))) void* lds_ptr;
typedef __attribute__((address_space(3))) uint8_t* lds_u8_ptr;

// 16-byte chunk slot of (row r, chunk c); the XOR swizzle spreads the eight
// rows read together by an MFMA operand load over all LDS banks.
__device__ __forceinline__ int kslot(int r, int c) { return r * kChunks + (c ^ ((r ^ (r >> 2)) & 7)); }
__device__ __forceinline__ void kslot_inv(int slot, int& r, int& c) {
  r = slot / kChunks;
  c = (slot - r * kChunks) ^ ((r ^ (r >> 2)) & 7);
}

struct MlaParams {
  const uint16_t* q;
  const uint16_t* kv;
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

// Drives the 3-stage pipeline over the three LDS stage buffers.  The buffers
// arrive as restrict-qualified parameters: after inlining, every access
// through them carries alias-scope metadata, which lets the compiler see that
// the stage being read is not the stage a DMA is still writing (otherwise it
// waits for every outstanding DMA before the first LDS read).
template <class Gather, class Step>
__device__ __forceinline__ void run_pipeline(uint8_t* __restrict__ kb0, uint8_t* __restrict__ kb1,
                                             uint8_t* __restrict__ kb2, int nb, Gather& gather, Step& step) {
  if (nb > 0) gather(kb0, 0);
  if (nb > 1) gather(kb1, 1);
  for (int blk = 0; blk < nb; blk += 3) {
    step(kb0, kb2, blk);
    if (blk + 1 < nb) step(kb1, kb0, blk + 1);
    if (blk + 2 < nb) step(kb2, kb1, blk + 2);
  }
}

template <class Addr>
__global__ __launch_bounds__(512, 1) void sparse_mla_kernel(MlaParams p, Addr addr) {
  // three separate stage buffers, so the compiler can tell the stage being
  // read from the stages the DMA is still writing
  __shared__ __attribute__((aligned(16))) uint8_t kb0[kBufBytes];
  __shared__ __attribute__((aligned(16))) uint8_t kb1[kBufBytes];
  __shared__ __attribute__((aligned(16))) uint8_t kb2[kBufBytes];
  __shared__ v8bf qtail[4 * 8 * 64];   // 32 KiB: query steps 14..17 of all waves
  __shared__ int32_t rows[kMaxK];      // latent row of every entry of this split (-1: skipped)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = lane >> 4, hl = lane & 15;
  const int64_t t = blockIdx.x / p.n_split;
  const int sp = blockIdx.x % p.n_split;
  const int j0 = sp * p.per_split;
  const int j1 = min(j0 + p.per_split, p.k);
  const int64_t b = p.seq_per_query ? t : 0;
  int64_t n_b = p.ctx_len ? (int64_t)p.ctx_len[b] : p.seq_len;
  if (n_b > p.seq_len) n_b = p.seq_len;
  const int head = kHeadsPerWave * wave + hl;
  const bool active = kHeadsPerWave * wave < p.H;
  const int32_t* idx_row = p.idx + t * (int64_t)p.k;
  const int n_ent = j1 > j0 ? j1 - j0 : 0;
  const int nb = (n_ent + kBlk - 1) / kBlk;

  // ---- resolve every entry to a latent row once (index and page-table
  // loads happen here only, so the block loop issues no other memory reads)
  for (int e = tid; e < nb * kBlk; e += 512) {
    int32_t row = -1;
    if (e < n_ent) {
      const int32_t s = idx_row[j0 + e];
      if (s >= 0 && s < n_b) row = (int32_t)addr.row(b, s);
    }
    rows[e] = row;
  }

  // ---- query rows of this wave's 16 heads: B operand of the logit MFMA,
  // step st covers dims 32*st + 8*g4 .. +7.  Steps 0..13 stay in VGPRs; steps
  // 14..17 (dims 448..575) are parked in LDS in the same lane order and read
  // back per block.  Lanes past the last head read head H-1 and zero it.
  constexpr int kQReg = 14;
  v8bf qf[kQReg];
  {
    const bool hv = head < p.H;
    const uint16_t* qrow = p.q + (t * p.H + (hv ? head : p.H - 1)) * (int64_t)kDqk + 8 * g4;
#pragma unroll
    for (int st = 0; st < kQReg; ++st) {
      const v8bf v = *(const v8bf*)(qrow + 32 * st);
      qf[st] = hv ? v : (v8bf){};
    }
#pragma unroll
    for (int st = kQReg; st < 18; ++st) {
      const v8bf v = *(const v8bf*)(qrow + 32 * st);
      qtail[((st - kQReg) * 8 + wave) * 64 + lane] = hv ? v : (v8bf){};
    }
  }
  __syncthreads();

  // Gather the 32 rows of block `blk` into LDS stage `bi`: 36 DMA
  // instructions of 64 x 16 bytes; every wave issues exactly kDmaPerWave
  // (waves 4..7 repeat their first one, an identical rewrite) so the
  // outstanding-load count is the same on every wave.  Skipped entries read
  // row 0 (their logits are masked, so the bytes only have to be finite).
  auto gather = [&](uint8_t* base, int blk) {
    // slot indices are recomputed per call (cheap) rather than kept live
    int zero;
    asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
#pragma unroll
    for (int i = 0; i < kDmaPerWave; ++i) {
      int ins = wave + 8 * i;
      if (ins >= kBlk * kChunks / 64) ins = wave;
      const int slot0 = 64 * ins;
      int r, c;
      kslot_inv(slot0 + lane + zero, r, c);
      int32_t row = rows[blk * kBlk + r];
      row = row < 0 ? 0 : row;
      const uint16_t* src = p.kv + ((uint64_t)(uint32_t)row * kDqk + 8 * c);
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_ptr)(base + slot0 * 16), 16, 0, 0);
    }
  };

  // ---- per-lane LDS byte offsets of the operand reads (everything else is
  // a compile-time immediate).  Logits: M-tile mt reads key 16*mt + hl, chunk
  // 4*st + g4 = 8*(st/2) + (4*(st%2) + g4).
  uint32_t s_addr[2][2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int r = 16 * mt + hl;
    const int f = (r ^ (r >> 2)) & 7;
#pragma unroll
    for (int par = 0; par < 2; ++par) s_addr[mt][par] = (uint32_t)(r * kChunks + ((4 * par + g4) ^ f)) * 16u;
  }
  // Values: for c'-tile ct, lane (g4, 4*rq + qq) supplies columns 16*ct + 4*qq ..
  // of key rows 4*g4 + rq (k-slots 0..3) and 16 + 4*g4 + rq (k-slots 4..7);
  // chunk 2*ct + qq/2 = 8*(ct/4) + (2*(ct%4) + qq/2), byte 8*(qq%2) within it.
  uint32_t v_addr[2][4];
  {
    const int rq = hl >> 2, qq = hl & 3;
#pragma unroll
    for (int hv = 0; hv < 2; ++hv) {
      const int r = 16 * hv + 4 * g4 + rq;
      const int f = (r ^ (r >> 2)) & 7;
#pragma unroll
      for (int m4 = 0; m4 < 4; ++m4)
        v_addr[hv][m4] = (uint32_t)(r * kChunks + ((2 * m4 + (qq >> 1)) ^ f)) * 16u + 8u * (qq & 1);
    }
  }

  v4f o[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) o[i] = (v4f){0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // 3-stage pipeline: blocks blk+1 and blk+2 stream in while blk is consumed
  // One pipeline step: wait for this wave's DMA of block blk (block blk+1 may
  // stay in flight), barrier (every wave's DMA of blk landed and block blk-1
  // is fully consumed), launch the DMA of blk+2 into the freed stage, then
  // consume stage `cur`.  s_barrier is used bare: a fenced __syncthreads()
  // would also wait for the DMA still in flight.
  auto step = [&](const uint8_t* cur, uint8_t* next2, int blk) {
    if (blk + 1 < nb)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kDmaPerWave) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    if (blk + 2 < nb) gather(next2, blk + 2);
    const uint64_t valid = __ballot(rows[blk * kBlk + (lane & 31)] >= 0) & 0xFFFFFFFFull;
    if (active) {
      const lds_u8_ptr base = (lds_u8_ptr)cur;
      // logits S^T[key, head]: two 16-key M-tiles x 18 k-steps
      v4f sacc[2] = {(v4f){0.f, 0.f, 0.f, 0.f}, (v4f){0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int st = 0; st < 18; ++st) {
        const v8bf qb = st < kQReg ? qf[st < kQReg ? st : 0] : qtail[((st - kQReg) * 8 + wave) * 64 + lane];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const v8bf a =
              *(const __attribute__((address_space(3))) v8bf*)(base + s_addr[mt][st & 1] + 128 * (st >> 1));
          sacc[mt] = mfma_bf16_16x16x32(a, qb, sacc[mt]);
        }
        if ((st % 2) == 1) __builtin_amdgcn_sched_barrier(0);
      }
      // lane: head hl; sacc[mt][i] is key 16*mt + 4*g4 + i of the block (raw
      // logit; masked keys set to -inf).  The running max m_run is kept in
      // log2 units: p = 2^(logit * scale*log2e - m_run).
      float mloc = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = 16 * mt + 4 * g4 + i;
          sacc[mt][i] = ((valid >> key) & 1) ? sacc[mt][i] : -INFINITY;
          mloc = fmaxf(mloc, sacc[mt][i]);
        }
      }
      mloc = fmaxf(mloc, shfl_xor_f(mloc, 16));
      mloc = fmaxf(mloc, shfl_xor_f(mloc, 32));
      mloc *= p.scale_log2;  // scale > 0 keeps the order
      const bool need = mloc > m_run + 8.0f;
      if (__any(need)) {
        const float m_new = need ? mloc : m_run;
        const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int ct = 0; ct < 32; ++ct) o[ct] *= alpha;
      }
      // masked keys: fma(-inf, s, -m) = -inf -> 2^-inf = 0; before the first
      // valid key m_run is -inf and every logit is -inf, so the bias is 0
      const float mneg = (m_run == -INFINITY) ? 0.f : -m_run;
      v8f pf;
      float lsum = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float pv = __builtin_amdgcn_exp2f(fmaf(sacc[i >> 2][i & 3], p.scale_log2, mneg));
        lsum += pv;
        pf[i] = pv;
      }
      l_run += lsum;
      // B operand of the value MFMA: k-slot 8*g4 + j <-> key 4*g4 + j (j < 4),
      // 16 + 4*g4 + (j - 4) (j >= 4): exactly this lane's probabilities
      const v8bf pb = __builtin_convertvector(pf, v8bf);
      // O^T[c', head] += V^T[c', keys] P^T[keys, head], 32 c'-tiles of 16
#pragma unroll
      for (int ct = 0; ct < 32; ++ct) {
        const v4s lo =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(base + v_addr[0][ct & 3] + 128 * (ct >> 2)));
        const v4s hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(base + v_addr[1][ct & 3] + 128 * (ct >> 2)));
        const v8bf va = __builtin_bit_cast(v8bf, (v8s_t){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
        o[ct] = mfma_bf16_16x16x32(va, pb, o[ct]);
        // bound how far the scheduler hoists operand reads (register budget)
        if ((ct & 3) == 3) __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  run_pipeline(kb0, kb1, kb2, nb, gather, step);

  if (!active || head >= p.H) return;
  float l_tot = l_run + shfl_xor_f(l_run, 16);
  l_tot += shfl_xor_f(l_tot, 32);
  const bool empty = !(l_tot > 0.f);
  const float inv = empty ? 0.f : 1.f / l_tot;
  const float lse_v = empty ? -INFINITY : (m_run + log2f(l_tot)) * 0.69314718055994530942f;
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
  for (int ct = 0; ct < 32; ++ct) *(v4f*)(orow + 16 * ct + 4 * g4) = o[ct] * inv;
  if (g4 == 0) *lrow = lse_v;
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
  hipLaunchKernelGGL((sparse_mla_kernel<Addr>), dim3((unsigned)blocks), dim3(512), 0, st, p, addr);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_sparse_mla(const MlaArgs& a, hipStream_t st) {
  if (a.T <= 0) return hipSuccess;
  MlaParams p;
  p.q = a.q;
  p.kv = a.kv;
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
