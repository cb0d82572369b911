// Per-row top-k selection (fine-grained token selection of DeepSeek Sparse
// Attention, "DeepSeek-V3.2" report walk-through §2.1.2): for each query row
// keep the k candidates with the largest index scores, ties to the lower
// position, emitted in ascending position order and padded with -1.
//
// One workgroup per row; scores become order-preserving uint32 keys.
//
// Sampled path (long rows): 1/16 of the row, in 256-byte chunks spread over
// the whole row, is read into LDS and its exact r-th largest key is found by
// radix selection, with r chosen so that about 1.37k keys of the full row are
// expected at or above it.  One pass over the row then gathers every key at
// or above that estimate into an LDS list; if the list holds at least k and at
// most its capacity, the exact k-th largest key (theta) and the selection come
// from the list alone -- about 1.06 row reads in all.  Otherwise the row takes
// the exact path.
//
// Exact path: theta by radix refinement -- a 12-bit histogram over the whole
// row (one pass), then the keys of the threshold bin (~1% of a row) are
// gathered into the LDS list (second pass) and refined there (12 + 8 more
// bits).  Rows whose threshold bin overflows the list (heavy ties) refine
// with further passes over the row.
//
// Either way the selection is recorded in two LDS bitmaps over the row,
// "key > theta" and "key == theta"; one block scan over the bitmaps gives each
// selected position its output slot (the lowest-position ties are the first r
// "== theta" bits), so the output is ascending with no sort.
#include "common.h"
#include "launch.h"

namespace dsa {

constexpr int kTopkThreads = 512;
constexpr int kTopkWaves = kTopkThreads / kWave;
constexpr int kTopkCap = 3584;  // LDS candidate list capacity (two workgroups fit a CU)
constexpr int kSampleStride = 16;   // the sample reads one 64-key chunk in 16
constexpr int kSampleMinN = 8192;   // shorter rows take the exact path

struct TopkShared {
  uint32_t hist[4096];
  uint32_t list_key[kTopkCap];
  int32_t list_idx[kTopkCap];
  uint32_t wave_a[kTopkWaves];
  uint32_t wave_b[kTopkWaves];
  uint32_t sel_bin;
  uint32_t sel_above;
  uint32_t list_n;
  uint32_t pad;
};

// Inclusive block scan of two counters (one workgroup).  Returns inclusive
// prefixes in *a, *b and the block totals in *ta, *tb.
__device__ __forceinline__ void block_scan2(TopkShared& sh, uint32_t* a, uint32_t* b, uint32_t* ta,
                                            uint32_t* tb) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = *a, y = *b;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    uint32_t xs = __shfl_up(x, d, 64), ys = __shfl_up(y, d, 64);
    if (lane >= d) {
      x += xs;
      y += ys;
    }
  }
  if (lane == 63) {
    sh.wave_a[wave] = x;
    sh.wave_b[wave] = y;
  }
  __syncthreads();
  uint32_t pa = 0, pb = 0, sa = 0, sb = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    const uint32_t wa = sh.wave_a[w], wb = sh.wave_b[w];
    if (w < wave) {
      pa += wa;
      pb += wb;
    }
    sa += wa;
    sb += wb;
  }
  __syncthreads();
  *a = x + pa;
  *b = y + pb;
  *ta = sa;
  *tb = sb;
}

// Given histogram counts over `nbins` bins (bins are ordered by key), the
// number `above` of keys greater than every bin and the rank k, find the
// bin holding the k-th largest key.  Publishes sh.sel_bin and sh.sel_above
// (= keys greater than that bin).
__device__ __forceinline__ void find_bin(TopkShared& sh, int nbins, uint32_t above, uint32_t k) {
  constexpr int BPT = 4096 / kTopkThreads;  // bins per thread at the widest level
  const int tid = threadIdx.x;
  // thread tid owns bins nbins-1-BPT*tid .. nbins-BPT-BPT*tid (top-down order)
  uint32_t c = 0;
  const int top = nbins - 1 - BPT * tid;
#pragma unroll
  for (int i = 0; i < BPT; ++i)
    if (top - i >= 0) c += sh.hist[top - i];
  uint32_t inc = c, dummy = 0, tot, tot2;
  block_scan2(sh, &inc, &dummy, &tot, &tot2);
  uint32_t run = above + inc - c;  // keys in bins above this thread's bins
  if (top >= 0 && run < k && run + c >= k) {
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      const int bin = top - i;
      if (bin < 0) break;
      const uint32_t h = sh.hist[bin];
      if (run < k && run + h >= k) {
        sh.sel_bin = (uint32_t)bin;
        sh.sel_above = run;
        break;
      }
      run += h;
    }
  }
  __syncthreads();
}

// Calls fn(s, key) for every candidate s < n of the row (any order: the
// callers only count, mark or gather).  On a 16-byte aligned row each thread
// issues four 16-byte loads before using any of them, so enough reads are in
// flight to cover the memory latency.
template <class Fn>
__device__ __forceinline__ void scan_row(const float* __restrict__ row, int64_t n, bool vec, Fn&& fn) {
  const int tid = threadIdx.x;
  if (vec) {
    constexpr int kU = 4;
    constexpr int64_t kStep = 4 * kTopkThreads;  // keys per unrolled sub-step
    const int64_t n16 = n / (kU * kStep) * (kU * kStep);
    for (int64_t s0 = 4 * (int64_t)tid; s0 < n16; s0 += kU * kStep) {
      v4f v[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) v[u] = *(const v4f*)(row + s0 + u * kStep);
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t s = s0 + u * kStep;
        fn(s, order_key(v[u][0]));
        fn(s + 1, order_key(v[u][1]));
        fn(s + 2, order_key(v[u][2]));
        fn(s + 3, order_key(v[u][3]));
      }
    }
    const int64_t n4 = n & ~(int64_t)3;
    for (int64_t s = n16 + 4 * (int64_t)tid; s < n4; s += kStep) {
      const v4f v = *(const v4f*)(row + s);
      fn(s, order_key(v[0]));
      fn(s + 1, order_key(v[1]));
      fn(s + 2, order_key(v[2]));
      fn(s + 3, order_key(v[3]));
    }
    for (int64_t s = n4 + tid; s < n; s += kTopkThreads) fn(s, order_key(row[s]));
  } else {
    for (int64_t s = tid; s < n; s += kTopkThreads) fn(s, order_key(row[s]));
  }
}

// Radix levels: 0 -> key bits 31..20, 1 -> bits 19..8, 2 -> bits 7..0.
__device__ __forceinline__ int level_shift(int level) { return level == 0 ? 20 : (level == 1 ? 8 : 0); }
__device__ __forceinline__ int level_bits(int level) { return level == 2 ? 8 : 12; }

// Ordered emit: positions whose gt bit is set, plus the lowest-position
// (k - #gt) positions whose eq bit is set, in ascending order.
__device__ __forceinline__ void emit_selection(TopkShared& sh, const uint32_t* gt_bits, const uint32_t* eq_bits,
                                               int n_words, uint32_t k, int32_t* __restrict__ out) {
  const int tid = threadIdx.x;
  // Thread tid owns words [wpt*tid, wpt*tid + wpt) i.e. a contiguous range of positions.
  const int wpt = (n_words + kTopkThreads - 1) / kTopkThreads;
  const int w0 = tid * wpt;
  uint32_t cg = 0, ce = 0;
  for (int i = 0; i < wpt; ++i) {
    const int wi = w0 + i;
    if (wi < n_words) {
      cg += __popc(gt_bits[wi]);
      ce += __popc(eq_bits[wi]);
    }
  }
  uint32_t ig = cg, ie = ce, tg, te;
  block_scan2(sh, &ig, &ie, &tg, &te);
  const uint32_t r = k - tg;  // ties to take, lowest positions first
  uint32_t eq_before = ie - ce;
  uint32_t sel_words[16];
  uint32_t cs = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int wi = w0 + i;
    uint32_t g = 0, e = 0;
    if (i < wpt && wi < n_words) {
      g = gt_bits[wi];
      e = eq_bits[wi];
    }
    uint32_t keep = 0;
    while (e && eq_before < r) {
      const uint32_t lowbit = e & (~e + 1u);
      keep |= lowbit;
      e &= e - 1u;
      ++eq_before;
    }
    sel_words[i] = g | keep;
    cs += __popc(sel_words[i]);
  }
  uint32_t is = cs, dummy = 0, ts, td;
  block_scan2(sh, &is, &dummy, &ts, &td);
  uint32_t pos = is - cs;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    uint32_t m = sel_words[i];
    const int base = (w0 + i) * 32;
    while (m) {
      const int b = __ffs(m) - 1;
      out[pos++] = base + b;
      m &= m - 1u;
    }
  }
}

// Exact radix selection of the k-th largest of the `nl` keys in sh.list_key
// whose value lies in [lo, hi] (`above` list keys are larger than hi), from
// radix level `level` on; leaves lo == hi == that key.
__device__ __forceinline__ void refine_list(TopkShared& sh, int nl, uint32_t& lo, uint32_t& hi, uint32_t above,
                                            int level, uint32_t k, const uint32_t* keys) {
  const int tid = threadIdx.x;
  for (; level < 3; ++level) {
    const int sh_ = level_shift(level), nb = 1 << level_bits(level);
    for (int i = tid; i < nb; i += kTopkThreads) sh.hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < nl; i += kTopkThreads) {
      const uint32_t key = keys[i];
      if (key >= lo && key <= hi) atomicAdd(&sh.hist[(key >> sh_) & (nb - 1)], 1u);
    }
    __syncthreads();
    find_bin(sh, nb, above, k);
    const uint32_t bin = sh.sel_bin;
    above = sh.sel_above;
    const uint32_t span = (sh_ == 0) ? 0u : ((1u << sh_) - 1u);
    lo = (lo & ~(((uint32_t)(nb - 1)) << sh_)) | (bin << sh_);
    hi = lo | span;
    __syncthreads();
  }
}

// Smallest and largest of the nl keys in LDS (block-wide; every thread gets
// both).
__device__ __forceinline__ void block_minmax(TopkShared& sh, int nl, const uint32_t* keys, uint32_t* mn,
                                             uint32_t* mx) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t a = 0xFFFFFFFFu, b = 0u;
  for (int i = tid; i < nl; i += kTopkThreads) {
    const uint32_t key = keys[i];
    a = min(a, key);
    b = max(b, key);
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    a = min(a, (uint32_t)__shfl_xor((int)a, d, 64));
    b = max(b, (uint32_t)__shfl_xor((int)b, d, 64));
  }
  if (lane == 0) {
    sh.wave_a[wave] = a;
    sh.wave_b[wave] = b;
  }
  __syncthreads();
  a = sh.wave_a[0];
  b = sh.wave_b[0];
#pragma unroll
  for (int w = 1; w < kTopkWaves; ++w) {
    a = min(a, sh.wave_a[w]);
    b = max(b, sh.wave_b[w]);
  }
  *mn = a;
  *mx = b;
  __syncthreads();
}

// Radix selection of the k-th largest of the nl keys in LDS (k <= nl) over
// the bits in which the keys differ: the bits above the highest bit where the
// smallest and largest key differ are common to all, and each level
// histograms the next (up to) 12 bits below them, so the bins spread over the
// keys' actual range.  After `levels` levels (or when every bit is resolved)
// returns the lowest key of the window holding the k-th largest: at least k
// keys are >= it, and it is the k-th largest exactly when the window is a
// single key, which takes at most three levels.
__device__ __forceinline__ uint32_t select_in_list(TopkShared& sh, int nl, const uint32_t* keys, uint32_t k,
                                                   int levels) {
  const int tid = threadIdx.x;
  uint32_t mn, mx;
  block_minmax(sh, nl, keys, &mn, &mx);
  int top = mn == mx ? 0 : 32 - __clz(mn ^ mx);  // low bits in which keys differ
  const uint32_t low_mask = top == 32 ? 0xFFFFFFFFu : ((1u << top) - 1u);
  uint32_t lo = mn & ~low_mask, hi = lo | low_mask, above = 0u;
  for (int level = 0; level < levels && top > 0; ++level) {
    const int shift = top > 12 ? top - 12 : 0, nb = 1 << (top - shift);
    for (int i = tid; i < nb; i += kTopkThreads) sh.hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < nl; i += kTopkThreads) {
      const uint32_t key = keys[i];
      if (key >= lo && key <= hi) atomicAdd(&sh.hist[(key >> shift) & (nb - 1)], 1u);
    }
    __syncthreads();
    find_bin(sh, nb, above, k);
    above = sh.sel_above;
    lo |= sh.sel_bin << shift;
    hi = lo | (shift == 0 ? 0u : ((1u << shift) - 1u));
    top = shift;
    __syncthreads();
  }
  return lo;
}

// Sampled path (see the file comment).  Returns false, having written
// nothing, when the gathered list misses [k, capacity]; the caller then takes
// the exact path.  Needs a 16-byte aligned row with n >= kSampleMinN; the
// bitmap area (n_words * 8 bytes >= n / 4 bytes) doubles as the sample buffer.
// The sampled threshold estimate: 1/16 of the row (64-key chunks spread
// over the whole row) is read into `sample` (at least n/4 + 240 bytes of
// LDS) and its exact r-th largest key returned, with r chosen so that about
// 1.37k keys of the full row are expected at or above it.  Needs a 16-byte
// aligned row with n >= kSampleMinN.
__device__ __forceinline__ uint32_t sample_estimate(TopkShared& sh, const float* __restrict__ row, int64_t n,
                                                    int32_t k, uint32_t* sample) {
  const int tid = threadIdx.x;
  // sampled chunk j: keys 64*(16*j + (5*j % 16)) .. +63, whole chunks inside the row
  const int64_t n_chunks = n / 64;
  const int m_chunks = (int)((n_chunks + kSampleStride - 1) / kSampleStride);
  int m = 0;  // sampled keys (a multiple of 64, counted by every thread alike)
  for (int j = 0; j < m_chunks; ++j)
    if ((int64_t)kSampleStride * j + (5 * j) % kSampleStride < n_chunks) m += 64;
  for (int f = tid; f < m_chunks * 16; f += kTopkThreads) {
    const int j = f >> 4;
    const int64_t chunk = (int64_t)kSampleStride * j + (5 * j) % kSampleStride;
    if (chunk < n_chunks) {
      const v4f v = *(const v4f*)(row + 64 * chunk + 4 * (f & 15));
      // compact slot: chunks are skipped only at the very end, so j-th kept chunk = j
      uint32_t* dst = sample + 64 * j + 4 * (f & 15);
      dst[0] = order_key(v[0]);
      dst[1] = order_key(v[1]);
      dst[2] = order_key(v[2]);
      dst[3] = order_key(v[3]);
    }
  }
  __syncthreads();
  // rank of the estimate within the sample: about 1.37k of the row lie above it
  const int64_t target = (int64_t)k + (int64_t)k * 3 / 8;
  int64_t rs = (target * m + n - 1) / n;
  if (rs < 1) rs = 1;
  if (rs > m) rs = m;
  return select_in_list(sh, m, sample, (uint32_t)rs, 2);
}

__device__ __forceinline__ bool topk_sampled(TopkShared& sh, const float* __restrict__ row, int64_t n, int32_t k,
                                             uint32_t* gt_bits, uint32_t* eq_bits, int n_words,
                                             int32_t* __restrict__ out) {
  const int tid = threadIdx.x;
  const uint32_t t_est = sample_estimate(sh, row, n, k, gt_bits);

  if (tid == 0) sh.list_n = 0;
  __syncthreads();
  scan_row(row, n, true, [&](int64_t s, uint32_t key) {
    if (key >= t_est) {
      const uint32_t slot = atomicAdd(&sh.list_n, 1u);
      if (slot < (uint32_t)kTopkCap) {
        sh.list_key[slot] = key;
        sh.list_idx[slot] = (int32_t)s;
      }
    }
  });
  __syncthreads();
  const uint32_t c = sh.list_n;
  if (c < (uint32_t)k || c > (uint32_t)kTopkCap) return false;  // uniform across the workgroup

  const uint32_t hi = select_in_list(sh, (int)c, sh.list_key, (uint32_t)k, 3);  // theta, the k-th largest
  const int rw = (int)((n + 31) / 32);  // bitmap words of this row
  for (int i = tid; i < rw; i += kTopkThreads) {
    gt_bits[i] = 0;
    eq_bits[i] = 0;
  }
  __syncthreads();
  for (int i = tid; i < (int)c; i += kTopkThreads) {
    const uint32_t key = sh.list_key[i];
    const int32_t s = sh.list_idx[i];
    if (key > hi)
      atomicOr(&gt_bits[s >> 5], 1u << (s & 31));
    else if (key == hi)
      atomicOr(&eq_bits[s >> 5], 1u << (s & 31));
  }
  __syncthreads();
  emit_selection(sh, gt_bits, eq_bits, rw, (uint32_t)k, out);
  return true;
}

// Exact path of one row (see the file comment): radix refinement over the
// row in global memory, then the LDS list, then the ordered emit.
__device__ __forceinline__ void topk_exact_row(TopkShared& sh, const float* __restrict__ row, int64_t n, bool vec,
                                               int32_t k, uint32_t* gt_bits, uint32_t* eq_bits, int n_words,
                                               int32_t* __restrict__ out) {
  const int tid = threadIdx.x;
  // Current candidate key range [lo, hi]; `above` keys are > hi.
  uint32_t lo = 0u, hi = 0xFFFFFFFFu, above = 0u, in_range = (uint32_t)n;
  int level = 0;  // 0: bits 31..20, 1: bits 19..8, 2: bits 7..0
  for (; level < 3; ++level) {
    if (level > 0 && in_range <= (uint32_t)kTopkCap) break;
    const int sh_ = level_shift(level), nb = 1 << level_bits(level);
    for (int i = tid; i < nb; i += kTopkThreads) sh.hist[i] = 0;
    __syncthreads();
    scan_row(row, n, vec, [&](int64_t, uint32_t key) {
      if (key >= lo && key <= hi) atomicAdd(&sh.hist[(key >> sh_) & (nb - 1)], 1u);
    });
    __syncthreads();
    find_bin(sh, nb, above, (uint32_t)k);
    const uint32_t bin = sh.sel_bin;
    above = sh.sel_above;
    in_range = sh.hist[bin];
    const uint32_t span = (sh_ == 0) ? 0u : ((1u << sh_) - 1u);
    lo = (lo & ~(((uint32_t)(nb - 1)) << sh_)) | (bin << sh_);
    hi = lo | span;
    __syncthreads();
  }

  // ------------------------------------------------------------ collect pass
  const int rw = (int)((n + 31) / 32);  // bitmap words of this row
  for (int i = tid; i < rw; i += kTopkThreads) {
    gt_bits[i] = 0;
    eq_bits[i] = 0;
  }
  if (tid == 0) sh.list_n = 0;
  __syncthreads();
  const bool exact = (lo == hi);
  scan_row(row, n, vec, [&](int64_t s, uint32_t key) {
    if (key > hi) {
      atomicOr(&gt_bits[s >> 5], 1u << (s & 31));
    } else if (key >= lo) {
      if (exact) {
        atomicOr(&eq_bits[s >> 5], 1u << (s & 31));
      } else {
        const uint32_t slot = atomicAdd(&sh.list_n, 1u);
        sh.list_key[slot] = key;
        sh.list_idx[slot] = (int32_t)s;
      }
    }
  });
  __syncthreads();

  // ------------------------------------------------------------ LDS refinement
  if (!exact) {
    const int nl = (int)sh.list_n;
    refine_list(sh, nl, lo, hi, above, level, (uint32_t)k, sh.list_key);
    // lo == hi == theta: mark list entries
    for (int i = tid; i < nl; i += kTopkThreads) {
      const uint32_t key = sh.list_key[i];
      const int32_t s = sh.list_idx[i];
      if (key > hi)
        atomicOr(&gt_bits[s >> 5], 1u << (s & 31));
      else if (key == hi)
        atomicOr(&eq_bits[s >> 5], 1u << (s & 31));
    }
    __syncthreads();
  }

  emit_selection(sh, gt_bits, eq_bits, rw, (uint32_t)k, out);
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const float* __restrict__ scores, int64_t ld,
                                                             int64_t T, int64_t N, int64_t q_pos0,
                                                             const int32_t* __restrict__ n_valid, int32_t k,
                                                             int32_t* __restrict__ idx, int32_t n_words) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  TopkShared& sh = *reinterpret_cast<TopkShared*>(smem);
  uint32_t* gt_bits = reinterpret_cast<uint32_t*>(smem + sizeof(TopkShared));
  uint32_t* eq_bits = gt_bits + n_words;

  const int tid = threadIdx.x;
  const int64_t t = blockIdx.x;
  int64_t n = n_valid ? (int64_t)n_valid[t] : q_pos0 + t + 1;
  n = n < 0 ? 0 : (n > N ? N : n);
  int32_t* out = idx + t * (int64_t)k;
  if (n <= k) {
    for (int i = tid; i < k; i += kTopkThreads) out[i] = i < n ? i : -1;
    return;
  }
  const float* row = scores + t * ld;
  const bool vec = ((reinterpret_cast<uintptr_t>(row) & 15) == 0);
  if (vec && n >= kSampleMinN && topk_sampled(sh, row, n, k, gt_bits, eq_bits, n_words, out)) return;
  topk_exact_row(sh, row, n, vec, k, gt_bits, eq_bits, n_words, out);
}

hipError_t launch_topk(const float* scores, int64_t ld, int64_t T, int64_t N, int64_t q_pos0,
                       const int32_t* n_valid, int32_t k, int32_t* idx, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  const int32_t n_words = (int32_t)((N + 31) / 32);
  // bitmaps (2 x n_words words) + 256 bytes: the sampled path's key sample
  // (at most n/4 + 240 bytes) reuses the bitmap area
  const size_t lds = sizeof(TopkShared) + sizeof(uint32_t) * 2 * (size_t)n_words + 256;
  static bool attr_set = false;
  if (!attr_set) {
    // rows up to 262144 keys: fixed state + 64 KiB of bitmaps
    hipError_t e = hipFuncSetAttribute((const void*)topk_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)(sizeof(TopkShared) + sizeof(uint32_t) * 2 * 8192 + 256));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)T), dim3(kTopkThreads), lds, st, scores, ld, T, N, q_pos0,
                     n_valid, k, idx, n_words);
  return hipGetLastError();
}


// ------------------------------------------------------------ few long rows
// Decode has a handful of rows, each up to 2^18 keys long: one workgroup per
// row would stream each row through one CU and leave most CUs idle.  Here the
// full-row pass is split over 4096-key chunks:
//   estimate: per row, the sampled threshold estimate t_est of topk_sampled
//             (1/16 of the row);
//   collect:  every chunk appends its keys >= t_est to the row's candidate
//             list (about 1.37k keys per row);
//   finish:   per row, theta = the k-th largest candidate, "> theta" and
//             "== theta" marked in LDS bitmaps and emitted in ascending
//             position order -- the selection rule of topk_kernel.  A row
//             whose list missed [k, capacity], or too short to sample, takes
//             topk_kernel's exact path.
constexpr int kRowChunk = 4096;

struct RowsMeta {
  uint32_t t_est;   // sampled threshold estimate (0: row takes the exact path)
  uint32_t n_cand;  // keys >= t_est appended so far
};

__device__ __forceinline__ int64_t row_len(const int32_t* n_valid, int64_t t, int64_t N) {
  int64_t n = n_valid[t];
  return n < 0 ? 0 : (n > N ? N : n);
}

__device__ __forceinline__ bool row_sampled(const float* row, int64_t n, int32_t k) {
  return n > k && n >= kSampleMinN && (reinterpret_cast<uintptr_t>(row) & 15) == 0;
}

__global__ __launch_bounds__(kTopkThreads) void topk_rows_estimate_kernel(const float* __restrict__ scores,
                                                                          int64_t ld, int64_t N,
                                                                          const int32_t* __restrict__ n_valid,
                                                                          int32_t k, RowsMeta* __restrict__ meta) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  TopkShared& sh = *reinterpret_cast<TopkShared*>(smem);
  uint32_t* sample = reinterpret_cast<uint32_t*>(smem + sizeof(TopkShared));
  const int64_t t = blockIdx.x;
  const int64_t n = row_len(n_valid, t, N);
  const float* row = scores + t * ld;
  uint32_t t_est = 0u;
  if (row_sampled(row, n, k)) t_est = sample_estimate(sh, row, n, k, sample);
  if (threadIdx.x == 0) meta[t] = RowsMeta{t_est, 0u};
}

__global__ __launch_bounds__(256) void topk_rows_collect_kernel(const float* __restrict__ scores, int64_t ld,
                                                                 int64_t N, const int32_t* __restrict__ n_valid,
                                                                 int32_t k, RowsMeta* __restrict__ meta,
                                                                 uint32_t* __restrict__ cand_key,
                                                                 int32_t* __restrict__ cand_idx) {
  __shared__ uint32_t lkey[kRowChunk];
  __shared__ int32_t lidx[kRowChunk];
  __shared__ uint32_t ln, base;
  const int64_t t = blockIdx.y, c = blockIdx.x;
  const int64_t n = row_len(n_valid, t, N);
  const int64_t s0 = c * kRowChunk;
  const float* row = scores + t * ld;
  if (s0 >= n || !row_sampled(row, n, k)) return;
  const uint32_t t_est = meta[t].t_est;
  if (threadIdx.x == 0) ln = 0;
  __syncthreads();
  const int64_t s1 = min(s0 + kRowChunk, n);
  auto visit = [&](int64_t s, float f) {
    const uint32_t key = order_key(f);
    if (key >= t_est) {
      const uint32_t slot = atomicAdd(&ln, 1u);
      lkey[slot] = key;
      lidx[slot] = (int32_t)s;
    }
  };
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t s = s0 + 4 * (threadIdx.x + 256 * u);
    if (s + 3 < s1) {
      const v4f v = *(const v4f*)(row + s);
#pragma unroll
      for (int j = 0; j < 4; ++j) visit(s + j, v[j]);
    } else {
      for (int j = 0; j < 4; ++j)
        if (s + j < s1) visit(s + j, row[s + j]);
    }
  }
  __syncthreads();
  if (ln == 0) return;
  if (threadIdx.x == 0) base = atomicAdd(&meta[t].n_cand, ln);
  __syncthreads();
  for (uint32_t i = threadIdx.x; i < ln; i += 256) {
    const uint32_t slot = base + i;
    if (slot < (uint32_t)kTopkCap) {
      cand_key[t * kTopkCap + slot] = lkey[i];
      cand_idx[t * kTopkCap + slot] = lidx[i];
    }
  }
}

__global__ __launch_bounds__(kTopkThreads) void topk_rows_finish_kernel(
    const float* __restrict__ scores, int64_t ld, int64_t N, const int32_t* __restrict__ n_valid, int32_t k,
    const RowsMeta* __restrict__ meta, const uint32_t* __restrict__ cand_key, const int32_t* __restrict__ cand_idx,
    int32_t* __restrict__ idx, int32_t n_words_max) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  TopkShared& sh = *reinterpret_cast<TopkShared*>(smem);
  uint32_t* gt_bits = reinterpret_cast<uint32_t*>(smem + sizeof(TopkShared));
  uint32_t* eq_bits = gt_bits + n_words_max;
  const int tid = threadIdx.x;
  const int64_t t = blockIdx.x;
  const int64_t n = row_len(n_valid, t, N);
  int32_t* out = idx + t * (int64_t)k;
  if (n <= k) {
    for (int i = tid; i < k; i += kTopkThreads) out[i] = i < n ? i : -1;
    return;
  }
  const float* row = scores + t * ld;
  const bool vec = (reinterpret_cast<uintptr_t>(row) & 15) == 0;
  const uint32_t c = row_sampled(row, n, k) ? meta[t].n_cand : 0u;
  if (c < (uint32_t)k || c > (uint32_t)kTopkCap) {  // uniform: the exact path over the row
    topk_exact_row(sh, row, n, vec, k, gt_bits, eq_bits, n_words_max, out);
    return;
  }
  const int n_words = (int)((n + 31) / 32);  // bitmap words of this row
  for (int i = tid; i < n_words; i += kTopkThreads) {
    gt_bits[i] = 0u;
    eq_bits[i] = 0u;
  }
  for (int i = tid; i < (int)c; i += kTopkThreads) {
    sh.list_key[i] = cand_key[t * kTopkCap + i];
    sh.list_idx[i] = cand_idx[t * kTopkCap + i];
  }
  __syncthreads();
  const uint32_t hi = select_in_list(sh, (int)c, sh.list_key, (uint32_t)k, 3);  // theta, the k-th largest
  for (int i = tid; i < (int)c; i += kTopkThreads) {
    const uint32_t key = sh.list_key[i];
    const int32_t s = sh.list_idx[i];
    if (key > hi)
      atomicOr(&gt_bits[s >> 5], 1u << (s & 31));
    else if (key == hi)
      atomicOr(&eq_bits[s >> 5], 1u << (s & 31));
  }
  __syncthreads();
  emit_selection(sh, gt_bits, eq_bits, n_words, (uint32_t)k, out);
}

size_t topk_rows_scratch_bytes(int64_t T, int64_t /*N*/) {
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  return al(sizeof(RowsMeta) * (size_t)T) + al(sizeof(uint32_t) * (size_t)T * kTopkCap) +
         al(sizeof(int32_t) * (size_t)T * kTopkCap);
}

// measured on MI355X: the split pays for rows of 64K keys and more (a 127K
// row: 48 us against 61 us in one workgroup); at 32K the two are even
bool topk_rows_preferred(int64_t T, int64_t N) { return T <= 1024 && N >= 65536; }

hipError_t launch_topk_rows(const float* scores, int64_t ld, int64_t T, int64_t N, const int32_t* n_valid,
                            int32_t k, int32_t* idx, void* scratch, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  const int64_t n_chunks = (N + kRowChunk - 1) / kRowChunk;
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  char* p = (char*)scratch;
  RowsMeta* meta = (RowsMeta*)p;
  p += al(sizeof(RowsMeta) * (size_t)T);
  uint32_t* cand_key = (uint32_t*)p;
  p += al(sizeof(uint32_t) * (size_t)T * kTopkCap);
  int32_t* cand_idx = (int32_t*)p;
  const int32_t n_words = (int32_t)((N + 31) / 32);
  // the estimate's sample (at most n/4 + 240 bytes) and the finish's bitmaps
  // (2 x n_words words) both fit the same dynamic LDS as topk_kernel
  const size_t lds = sizeof(TopkShared) + sizeof(uint32_t) * 2 * (size_t)n_words + 256;
  static bool attr_set = false;
  if (!attr_set) {
    const int cap = (int)(sizeof(TopkShared) + sizeof(uint32_t) * 2 * 8192 + 256);
    hipError_t e = hipFuncSetAttribute((const void*)topk_rows_finish_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, cap);
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void*)topk_rows_estimate_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                              cap);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(topk_rows_estimate_kernel, dim3((unsigned)T), dim3(kTopkThreads), lds, st, scores, ld, N,
                     n_valid, k, meta);
  hipLaunchKernelGGL(topk_rows_collect_kernel, dim3((unsigned)n_chunks, (unsigned)T), dim3(256), 0, st, scores, ld,
                     N, n_valid, k, meta, cand_key, cand_idx);
  hipLaunchKernelGGL(topk_rows_finish_kernel, dim3((unsigned)T), dim3(kTopkThreads), lds, st, scores, ld, N,
                     n_valid, k, meta, cand_key, cand_idx, idx, n_words);
  return hipGetLastError();
}

}  // namespace dsa
