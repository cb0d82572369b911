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
// owns heads 32w..32w+31 and keeps their query rows in VGPRs (as the MFMA B
// operand) and their fp32 output accumulators (512 x 32 per wave) in
// registers.  Selected latent rows are gathered 32 at a time into LDS (double
// buffered, next block prefetched into registers while the current one is
// consumed) in two layouts: row-major (swizzled 16-byte chunks) for the
// logits S^T = K Q^T, and transposed for the value product O^T = V^T P^T.
// Writing the logits transposed (keys on MFMA rows, heads on columns) makes
// each lane own a single head: the softmax statistics are per-lane scalars,
// the fp32 probabilities feed the value MFMA's B operand straight from the
// logit accumulator layout (only a key permutation, mirrored in the V^T
// reads), and the output rescale is one multiply per accumulator.  The
// running max is only moved when it grows by more than 2^8 (exact: the
// final normalisation uses the same max), so rescales are rare.
// Small batches (decode) split each query's k entries over several
// workgroups; partial (out, lse) pairs are merged exactly by
// combine_kernel: lse = ln sum_i e^{lse_i}, out = sum_i e^{lse_i - lse} out_i.
#include "common.h"
#include "launch.h"

namespace dsa {

constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kBlk = 32;                  // selected rows per block
constexpr int kChunks = kDqk / 8;         // 16-byte chunks per latent row (72)
constexpr int kVtStride = 36;             // V^T row stride in bf16 (32 keys + 4 pad)
constexpr int kKBytes = kBlk * kDqk * 2;  // 36864
constexpr int kVtBytes = kDv * kVtStride * 2;  // 36864
constexpr int kBufBytes = kKBytes + kVtBytes + 128;
constexpr int kMlaLds = kBufBytes;
constexpr int kUnits = kChunks * (kBlk / 4);  // (chunk, row-quad) staging units per block: 576

typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
typedef float v8f __attribute__((ext_vector_type(8)));

// 16-byte chunk slot of (row r, chunk c) in the K layout; XOR swizzle keeps
// both the row-quad staging writes and the MFMA operand reads conflict-free.
__device__ __forceinline__ int kslot(int r, int c) { return r * kChunks + (c ^ ((r ^ (r >> 2)) & 7)); }

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

template <class Addr>
__global__ __launch_bounds__(256, 1) void sparse_mla_kernel(MlaParams p, Addr addr) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, hl = lane & 31;
  const int64_t t = blockIdx.x / p.n_split;
  const int sp = blockIdx.x % p.n_split;
  const int j0 = sp * p.per_split;
  const int j1 = min(j0 + p.per_split, p.k);
  const int64_t b = p.seq_per_query ? t : 0;
  int64_t n_b = p.ctx_len ? (int64_t)p.ctx_len[b] : p.seq_len;
  if (n_b > p.seq_len) n_b = p.seq_len;
  const int head = 32 * wave + hl;
  const bool active = 32 * wave < p.H;
  const int32_t* idx_row = p.idx + t * (int64_t)p.k;

  // ---- query rows of this wave's heads (MFMA B operand of the logit product)
  v8bf qf[36];
#pragma unroll
  for (int st = 0; st < 36; ++st) {
    if (head < p.H) {
      qf[st] = *(const v8bf*)(p.q + ((t * p.H + head) * (int64_t)kDqk + 16 * st + 8 * g));
    } else {
      qf[st] = (v8bf){};
    }
  }

  // ---- staging: unit u = c*8 + qd moves chunk c of rows 4qd..4qd+3
  v4i stg[3][4];
  int32_t stg_ok[3];
  auto stage_load = [&](int jb) {
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int u = tid + 256 * i;
      stg_ok[i] = 0;
      if (u < kUnits) {
        const int c = u >> 3, qd = u & 7;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int j = jb + 4 * qd + rr;
          int64_t row = -1;
          if (j < j1) {
            const int32_t s = idx_row[j];
            if (s >= 0 && s < n_b) row = addr.row(b, s);
          }
          if (row >= 0) {
            stg[i][rr] = *(const v4i*)(p.kv + row * kDqk + 8 * c);
            stg_ok[i] |= 1 << rr;
          } else {
            stg[i][rr] = (v4i){0, 0, 0, 0};
          }
        }
      }
    }
  };
  auto stage_store = [&](int buf) {
    uint8_t* base = smem + buf * kBufBytes;
    uint16_t* vt = (uint16_t*)(base + kKBytes);
    int32_t* valid = (int32_t*)(base + kKBytes + kVtBytes);
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int u = tid + 256 * i;
      if (u < kUnits) {
        const int c = u >> 3, qd = u & 7;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) ((v4i*)base)[kslot(4 * qd + rr, c)] = stg[i][rr];
        if (c < kDv / 8) {
          // transpose 4 rows x 8 columns: column e -> 4 keys at V^T[8c + e][4qd .. 4qd+3]
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            // dword e2 of each row holds columns 2*e2 (low half) and 2*e2+1 (high half)
            const uint32_t r0 = (uint32_t)stg[i][0][e2], r1 = (uint32_t)stg[i][1][e2];
            const uint32_t r2 = (uint32_t)stg[i][2][e2], r3 = (uint32_t)stg[i][3][e2];
            v2i lo, hi;
            lo.x = (int)__builtin_amdgcn_perm(r1, r0, 0x05040100u);  // (r0.lo, r1.lo)
            lo.y = (int)__builtin_amdgcn_perm(r3, r2, 0x05040100u);
            hi.x = (int)__builtin_amdgcn_perm(r1, r0, 0x07060302u);  // (r0.hi, r1.hi)
            hi.y = (int)__builtin_amdgcn_perm(r3, r2, 0x07060302u);
            *(v2i*)(vt + (8 * c + 2 * e2) * kVtStride + 4 * qd) = lo;
            *(v2i*)(vt + (8 * c + 2 * e2 + 1) * kVtStride + 4 * qd) = hi;
          }
        }
        if (c == 0) {
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) valid[4 * qd + rr] = (stg_ok[i] >> rr) & 1;
        }
      }
    }
  };

  v16f o[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) o[i] = (v16f){};
  float m_run = -INFINITY, l_run = 0.f;

  for (int jb = j0; jb < j1; jb += kBlk) {
    stage_load(jb);
    stage_store(0);
    __syncthreads();
    if (active) {
      const uint8_t* base = smem;
      const uint16_t* vt = (const uint16_t*)(base + kKBytes);
      const int32_t* valid = (const int32_t*)(base + kKBytes + kVtBytes);
      // logits S^T[key, head] over the 576 latent dims
      v16f sacc = (v16f){};
#pragma unroll
      for (int st = 0; st < 36; ++st) {
        const v8bf a = ((const v8bf*)base)[kslot(hl, 2 * st + g)];
        sacc = mfma_bf16_32x32x16(a, qf[st], sacc);
      }
      // lane: head hl; register i: key 8*(i/4) + 4*g + (i%4) of the block
      float z[16];
      float mloc = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = 8 * (i >> 2) + 4 * g + (i & 3);
        z[i] = valid[key] ? sacc[i] * p.scale_log2 : -INFINITY;
        mloc = fmaxf(mloc, z[i]);
      }
      mloc = fmaxf(mloc, shfl_xor_f(mloc, 32));
      const bool need = mloc > m_run + 8.0f;
      if (__any(need)) {
        const float m_new = need ? mloc : m_run;
        const float alpha = (m_run == -INFINITY) ? 0.f : exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int ti = 0; ti < 16; ++ti) o[ti] *= alpha;
      }
      v8f pf0, pf1;
      float lsum = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = (m_run == -INFINITY) ? 0.f : exp2f(z[i] - m_run);
        lsum += pv;
        if (i < 8)
          pf0[i] = pv;
        else
          pf1[i - 8] = pv;
      }
      l_run += lsum;
      const v8bf pb0 = __builtin_convertvector(pf0, v8bf);
      const v8bf pb1 = __builtin_convertvector(pf1, v8bf);
      // O^T[c', head] += V^T[c', keys] P^T[keys, head]
#pragma unroll
      for (int ti = 0; ti < 16; ++ti) {
        const uint16_t* vrow = vt + (32 * ti + hl) * kVtStride;
        const v4bf a0 = *(const v4bf*)(vrow + 4 * g);
        const v4bf a1 = *(const v4bf*)(vrow + 8 + 4 * g);
        const v4bf a2 = *(const v4bf*)(vrow + 16 + 4 * g);
        const v4bf a3 = *(const v4bf*)(vrow + 24 + 4 * g);
        const v8bf va = (v8bf){a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
        const v8bf vb = (v8bf){a2[0], a2[1], a2[2], a2[3], a3[0], a3[1], a3[2], a3[3]};
        o[ti] = mfma_bf16_32x32x16(va, pb0, o[ti]);
        o[ti] = mfma_bf16_32x32x16(vb, pb1, o[ti]);
      }
    }
    __syncthreads();
  }

  if (!active || head >= p.H) return;
  const float l_tot = l_run + shfl_xor_f(l_run, 32);
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
#pragma unroll
  for (int ti = 0; ti < 16; ++ti) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      v4f v = {o[ti][4 * q4] * inv, o[ti][4 * q4 + 1] * inv, o[ti][4 * q4 + 2] * inv, o[ti][4 * q4 + 3] * inv};
      *(v4f*)(orow + 32 * ti + 8 * q4 + 4 * g) = v;
    }
  }
  if (g == 0) *lrow = lse_v;
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
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)sparse_mla_kernel<Addr>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kMlaLds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int64_t blocks = p.T * p.n_split;
  hipLaunchKernelGGL((sparse_mla_kernel<Addr>), dim3((unsigned)blocks), dim3(256), kMlaLds, st, p, addr);
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
