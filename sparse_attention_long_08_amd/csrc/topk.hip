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
#include <atomic>

#include "common.h"
#include "indexer_exact.h"
#include "launch.h"

namespace dsa {

constexpr int kTopkThreads = 512;     // workgroup of the plain, multi-workgroup and band kernels
constexpr int kTopkWideThreads = 1024;  // topk_kernel on few rows (decode): a workgroup alone on its CU
constexpr int kTopkMaxWaves = kTopkWideThreads / kWave;
constexpr int64_t kTopkWideMaxRows = 256;  // launches of at most this many rows take kTopkWideThreads
constexpr int kTopkCap = 3584;  // LDS candidate list capacity (two workgroups fit a CU)
// The sampled estimate reads one 64-key chunk in kSampleStride of the fp32
// rows (the plain and the multi-workgroup top-k) and one in kSampleStrideH of
// the fused prefill's f16 rows.  Measured on MI355X: a 1-in-32 sample took the
// decode top-k from 29.6 to 28.2 us (64 rows of 32K) and from 44.2 to 38.3 us
// (32 rows of 4K..128K), while the band top-k of the 128K prefill took 19.5
// against 18.6 ms with it, so the f16 rows keep 1 in 16.
constexpr int kSampleStride = 32;
constexpr int kSampleStrideH = 16;
constexpr int kSampleMinN = 8192;   // shorter rows take the exact path
// Radix levels of the sampled estimate.  The estimate only has to be a lower
// bound near the sample's r-th key: one 12-bit level over the keys' narrowed
// range returns the low edge of the bin holding that key, at most 1/4096 of
// the sample's key range below it, and the candidate list absorbs the extra
// keys that lets in (a row whose list overflows takes the exact path, so the
// selection never depends on it).  A second level costs a histogram pass and
// four barriers per row.  Measured on MI355X with one level against two:
// decode top-k 26.2 -> 24.5 us (64 x 32K) and 39.1 -> 36.6 us
// (32 x 4K..128K), band top-k 18.6 -> 18.0 ms per 128K step.
constexpr int kSampleLevels = 1;

struct TopkShared {
  uint32_t hist[4096];
  uint32_t list_key[kTopkCap];
  int32_t list_idx[kTopkCap];
  uint32_t wave_a[kTopkMaxWaves];
  uint32_t wave_b[kTopkMaxWaves];
  uint32_t sel_bin;
  uint32_t sel_above;
  uint32_t list_n;
  uint32_t n_sure;  // band selection: keys selected on their approximate score alone
  uint32_t fin_n;    // keys gathered for the direct ranking that ends a selection
  uint32_t sel_key;  // the key that ranking selects
};

// The fused prefill's score tile holds f16 approximate scores, each the row's
// score times 2^-s (the row's scale is 2^s, so every score fits f16's range);
// a key is that of the fp32 value f16 * 2^s, which is exact.
__device__ __forceinline__ uint32_t h_key(_Float16 h, float scale) { return order_key((float)h * scale); }

// Keys sampled from a row of n_chunks whole 64-key chunks when chunk
// S * j + (5 j mod S) is read for every j < ceil(n_chunks / S) that lies in
// the row: all but the last such j give chunks below S * (ceil(n_chunks / S) - 1),
// which is at most n_chunks - 1, so only the last needs the test.  (Counted
// chunk by chunk, ceil(n_chunks / S) serial steps ran ahead of the sample's
// loads: measured on MI355X, band top-k 16.6 -> 15.5 ms per 128K prefill
// step, decode top-k 24.3 -> 23.0 us on 64 x 32K and 36.7 -> 33.9 us paged.)
__device__ __forceinline__ int sampled_keys(int64_t n_chunks, int S) {
  const int64_t mc = (n_chunks + S - 1) / S;
  if (mc == 0) return 0;
  const int64_t j = mc - 1;
  return 64 * (int)(j + (S * j + (5 * j) % S < n_chunks ? 1 : 0));
}

// Radix levels: 0 -> key bits 31..20, 1 -> bits 19..8, 2 -> bits 7..0.
__device__ __forceinline__ int level_shift(int level) { return level == 0 ? 20 : (level == 1 ? 8 : 0); }
__device__ __forceinline__ int level_bits(int level) { return level == 2 ? 8 : 12; }

// Appends the B keys of this thread's batch whose bits are set in m, with
// their positions pos(j), to a list in LDS (keys[], idxs[], its length in
// *count; slots from cap on are counted but not written), at slots from one
// LDS atomic per wave: the wave's exclusive prefix of the per-thread counts
// comes from six ballots (counts < 64).  Every lane of the wave must call it.
template <int B, class Pos>
__device__ __forceinline__ void append_marked(uint32_t* count, uint32_t* keys, int32_t* idxs, uint32_t cap,
                                              const uint32_t (&key)[B], uint32_t m, Pos&& pos) {
  static_assert(B <= 32, "one 32-bit mark word per batch");
  const int lane = threadIdx.x & (kWave - 1);
  const uint32_t cnt = __popc(m);
  uint32_t pre = 0u, tot = 0u;  // marks of the lower lanes, and of the wave
#pragma unroll
  for (int b = 0; b < 6; ++b) {
    const uint64_t bal = __ballot((cnt >> b) & 1u);
    pre += __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u)) << b;
    tot += (uint32_t)__popcll(bal) << b;
  }
  if (tot == 0u) return;  // uniform across the wave
  uint32_t base = 0u;
  if (lane == 0) base = atomicAdd(count, tot);
  uint32_t slot = __builtin_amdgcn_readfirstlane(base) + pre;
#pragma unroll
  for (int j = 0; j < B; ++j) {
    if (m & (1u << j)) {
      if (slot < cap) {
        keys[slot] = key[j];
        idxs[slot] = (int32_t)pos(j);
      }
      ++slot;
    }
  }
}

// The per-row selection steps, for a workgroup of NTH threads (every thread
// of the workgroup calls them together).
template <int NTH>
struct TopkOps {
  static constexpr int kW = NTH / kWave;
  static_assert(NTH % kWave == 0 && kW <= kTopkMaxWaves && 4096 % NTH == 0, "workgroup of whole waves");

// Inclusive block scan of two counters (one workgroup).  Returns inclusive
// prefixes in *a, *b and the block totals in *ta, *tb.
static __device__ __forceinline__ void block_scan2(TopkShared& sh, uint32_t* a, uint32_t* b, uint32_t* ta,
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
  for (int w = 0; w < kW; ++w) {
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
static __device__ __forceinline__ void find_bin(TopkShared& sh, int nbins, uint32_t above, uint32_t k) {
  constexpr int BPT = 4096 / NTH;  // bins per thread at the widest level
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
static __device__ __forceinline__ void scan_row(const float* __restrict__ row, int64_t n, bool vec, Fn&& fn) {
  const int tid = threadIdx.x;
  if (vec) {
    constexpr int kU = 4;
    constexpr int64_t kStep = 4 * NTH;  // keys per unrolled sub-step
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
    for (int64_t s = n4 + tid; s < n; s += NTH) fn(s, order_key(row[s]));
  } else {
    for (int64_t s = tid; s < n; s += NTH) fn(s, order_key(row[s]));
  }
}


// scan_row over such a row (16-byte aligned): eight keys per 16-byte load,
// four loads in flight per thread.
template <class Fn>
static __device__ __forceinline__ void scan_row_h(const _Float16* __restrict__ row, float scale, int64_t n, Fn&& fn) {
  const int tid = threadIdx.x;
  constexpr int kU = 4;
  constexpr int64_t kStep = 8 * NTH;  // keys per unrolled sub-step
  const int64_t nU = n / (kU * kStep) * (kU * kStep);
  for (int64_t s0 = 8 * (int64_t)tid; s0 < nU; s0 += kU * kStep) {
    v8h v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) v[u] = *(const v8h*)(row + s0 + u * kStep);
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int j = 0; j < 8; ++j) fn(s0 + u * kStep + j, h_key(v[u][j], scale));
  }
  const int64_t n8 = n & ~(int64_t)7;
  for (int64_t s = nU + 8 * (int64_t)tid; s < n8; s += kStep) {
    const v8h v = *(const v8h*)(row + s);
#pragma unroll
    for (int j = 0; j < 8; ++j) fn(s + j, h_key(v[j], scale));
  }
  for (int64_t s = n8 + tid; s < n; s += NTH) fn(s, h_key(row[s], scale));
}

// The same append for a 16-byte aligned fp32 row: batches of 16 keys per
// thread (four 16-byte loads in flight), the tail key by key.  Measured on
// MI355X: decode top-k 23.0 -> 22.7 us on 64 x 32K.
// With use_first, first holds the thread's first batch (first_batch_f,
// taken when the row has at least 16 NTH keys).
static __device__ __forceinline__ void first_batch_f(const float* __restrict__ row, v4f (&v)[4]) {
  const int64_t s0 = 4 * (int64_t)threadIdx.x;
#pragma unroll
  for (int u = 0; u < 4; ++u) v[u] = *(const v4f*)(row + s0 + u * (4 * NTH));
}

static __device__ __forceinline__ void gather_ge_f(TopkShared& sh, const float* __restrict__ row, int64_t n,
                                                   uint32_t cut, bool use_first, const v4f (&first)[4]) {
  const int tid = threadIdx.x;
  constexpr int kU = 4;
  constexpr int64_t kStep = 4 * NTH;
  const int64_t nU = n / (kU * kStep) * (kU * kStep);
  // every thread runs the same number of these iterations (whole waves active)
  for (int64_t s0 = 4 * (int64_t)tid; s0 < nU; s0 += kU * kStep) {
    v4f v[kU];
    if (use_first && s0 == 4 * (int64_t)tid) {
#pragma unroll
      for (int u = 0; u < kU; ++u) v[u] = first[u];
    } else {
#pragma unroll
      for (int u = 0; u < kU; ++u) v[u] = *(const v4f*)(row + s0 + u * kStep);
    }
    uint32_t key[kU * 4], m = 0u;
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        key[u * 4 + j] = order_key(v[u][j]);
        m |= (key[u * 4 + j] >= cut ? 1u : 0u) << (u * 4 + j);
      }
    append_marked<kU * 4>(&sh.list_n, sh.list_key, sh.list_idx, (uint32_t)kTopkCap, key, m,
                          [&](int j) { return s0 + (j >> 2) * kStep + (j & 3); });
  }
  auto one = [&](int64_t s, uint32_t k1) {
    if (k1 >= cut) {
      const uint32_t slot = atomicAdd(&sh.list_n, 1u);
      if (slot < (uint32_t)kTopkCap) {
        sh.list_key[slot] = k1;
        sh.list_idx[slot] = (int32_t)s;
      }
    }
  };
  const int64_t n4 = n & ~(int64_t)3;
  for (int64_t s = nU + 4 * (int64_t)tid; s < n4; s += kStep) {
    const v4f v = *(const v4f*)(row + s);
#pragma unroll
    for (int j = 0; j < 4; ++j) one(s + j, order_key(v[j]));
  }
  for (int64_t s = n4 + tid; s < n; s += NTH) one(s, order_key(row[s]));
}

// Keys of one 32-key batch (four 16-byte loads at s0 + u * 8 NTH) appended
// when >= cut, through append_marked.
static __device__ __forceinline__ void gather_batch_h(TopkShared& sh, int64_t s0, const v8h (&v)[4], float scale,
                                                      uint32_t cut) {
  constexpr int64_t kStep = 8 * NTH;
  uint32_t key[32], m = 0u;
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      key[u * 8 + j] = h_key(v[u][j], scale);
      m |= (key[u * 8 + j] >= cut ? 1u : 0u) << (u * 8 + j);
    }
  append_marked<32>(&sh.list_n, sh.list_key, sh.list_idx, (uint32_t)kTopkCap, key, m,
                    [&](int j) { return s0 + (j >> 3) * kStep + (j & 7); });
}

// The loads of a thread's first batch of gather_ge_h (rows of at least
// 32 NTH keys), issued ahead of the work that finds the cut.
static __device__ __forceinline__ void first_batch_h(const _Float16* __restrict__ row, v8h (&v)[4]) {
  const int64_t s0 = 8 * (int64_t)threadIdx.x;
#pragma unroll
  for (int u = 0; u < 4; ++u) v[u] = *(const v8h*)(row + s0 + u * (8 * NTH));
}

// Appends to the LDS list every key >= cut of such a row, with its position
// (slots from kTopkCap on are counted in list_n but not written), as the
// candidate passes do.  In the unrolled part each thread keeps the keys of
// its 32-key batch in registers and marks those to append; one wave prefix
// count of the marks (six ballots) and one LDS atomic per wave and batch then
// give every thread its slots, where an append per key position would wait
// for an LDS atomic at nearly every position (some lane of 64 usually holds
// a key above the cut).  Measured on MI355X: band top-k 17.4 -> 16.8 ms per
// 128K prefill step, 5.23 -> 5.14 ms per chunked paged prefill call.
// With use_first (first holding the first_batch_h loads, taken when the
// row has at least 32 NTH keys) the first batch comes from those registers.
// Expects list_n set and a barrier before the call.
static __device__ __forceinline__ void gather_ge_h(TopkShared& sh, const _Float16* __restrict__ row, float scale,
                                                   int64_t n, uint32_t cut, bool use_first, const v8h (&first)[4]) {
  const int tid = threadIdx.x;
  constexpr int kU = 4;
  constexpr int64_t kStep = 8 * NTH;
  const int64_t nU = n / (kU * kStep) * (kU * kStep);
  // every thread runs the same number of these iterations (whole waves active)
  int64_t s0 = 8 * (int64_t)tid;
  if (use_first && s0 < nU) {
    gather_batch_h(sh, s0, first, scale, cut);
    s0 += kU * kStep;
  }
  for (; s0 < nU; s0 += kU * kStep) {
    v8h v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) v[u] = *(const v8h*)(row + s0 + u * kStep);
    gather_batch_h(sh, s0, v, scale, cut);
  }
  auto one = [&](int64_t s, uint32_t k1) {
    if (k1 >= cut) {
      const uint32_t slot = atomicAdd(&sh.list_n, 1u);
      if (slot < (uint32_t)kTopkCap) {
        sh.list_key[slot] = k1;
        sh.list_idx[slot] = (int32_t)s;
      }
    }
  };
  const int64_t n8 = n & ~(int64_t)7;
  for (int64_t s = nU + 8 * (int64_t)tid; s < n8; s += kStep) {
    const v8h v = *(const v8h*)(row + s);
#pragma unroll
    for (int j = 0; j < 8; ++j) one(s + j, h_key(v[j], scale));
  }
  for (int64_t s = n8 + tid; s < n; s += NTH) one(s, h_key(row[s], scale));
}


// Ordered emit: positions whose gt bit is set, plus the lowest-position
// (k - #gt) positions whose eq bit is set, in ascending order.
static __device__ __forceinline__ void emit_selection(TopkShared& sh, const uint32_t* gt_bits, const uint32_t* eq_bits,
                                               int n_words, uint32_t k, int32_t* __restrict__ out) {
  const int tid = threadIdx.x;
  // Thread tid owns words [wpt*tid, wpt*tid + wpt) i.e. a contiguous range of positions.
  const int wpt = (n_words + NTH - 1) / NTH;
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
  }
  // output slot of this thread's first selected position: the selection is
  // every gt position and the first r eq positions, so min(eq prefix, r) of
  // those eq positions lie in the words before this thread's (no second
  // block scan; measured on MI355X: decode top-k 22.3 -> 21.8 us on 64 x 32K,
  // 31.3 -> 30.8 us paged, band top-k 15.65 -> 15.53 ms per 128K step)
  uint32_t pos = (ig - cg) + min(ie - ce, r);
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
static __device__ __forceinline__ void refine_list(TopkShared& sh, int nl, uint32_t& lo, uint32_t& hi, uint32_t above,
                                            int level, uint32_t k, const uint32_t* keys) {
  const int tid = threadIdx.x;
  for (; level < 3; ++level) {
    const int sh_ = level_shift(level), nb = 1 << level_bits(level);
    for (int i = tid; i < nb; i += NTH) sh.hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < nl; i += NTH) {
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
static __device__ __forceinline__ void block_minmax(TopkShared& sh, int nl, const uint32_t* keys, uint32_t* mn,
                                             uint32_t* mx) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t a = 0xFFFFFFFFu, b = 0u;
  for (int i = tid; i < nl; i += NTH) {
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
  for (int w = 1; w < kW; ++w) {
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
// single key, which takes at most three levels.  When a level leaves at most
// kFinishMax keys in the window and more levels are allowed, those keys are
// ranked directly instead, which gives the same exact key (the k-th largest)
// with one pass over the list instead of up to two more levels (measured on
// MI355X: band top-k 17.9 -> 17.3 ms per 128K prefill step, decode top-k
// 24.4 -> 24.2 us on 64 x 32K).
static constexpr uint32_t kFinishMax = kWave;

// The kk-th largest (1 <= kk <= n) of the n <= kFinishMax keys of the list
// that lie in [lo, hi]: the keys are gathered into hist[0, n) and the first
// wave counts, for each, the keys greater than and not less than it.  Expects
// sh.fin_n = 0 and a barrier since hist was last read.
static __device__ __forceinline__ uint32_t rank_in_window(TopkShared& sh, int nl, const uint32_t* keys, uint32_t lo,
                                                   uint32_t hi, uint32_t kk, uint32_t n) {
  const int tid = threadIdx.x;
  for (int i = tid; i < nl; i += NTH) {
    const uint32_t key = keys[i];
    if (key >= lo && key <= hi) {
      const uint32_t slot = atomicAdd(&sh.fin_n, 1u);
      if (slot < kFinishMax) sh.hist[slot] = key;
    }
  }
  __syncthreads();
  if (tid < kWave) {
    const uint32_t v = (uint32_t)tid < n ? sh.hist[tid] : 0u;
    uint32_t gt = 0, ge = 0;
    for (uint32_t j = 0; j < n; ++j) {
      const uint32_t w = sh.hist[j];
      gt += w > v ? 1u : 0u;
      ge += w >= v ? 1u : 0u;
    }
    if ((uint32_t)tid < n && gt < kk && ge >= kk) sh.sel_key = v;  // lanes holding equal keys write one value
  }
  __syncthreads();
  return sh.sel_key;
}

static __device__ __forceinline__ uint32_t select_in_list(TopkShared& sh, int nl, const uint32_t* keys, uint32_t k,
                                                   int levels) {
  const int tid = threadIdx.x;
  uint32_t mn, mx;
  block_minmax(sh, nl, keys, &mn, &mx);
  int top = mn == mx ? 0 : 32 - __clz(mn ^ mx);  // low bits in which keys differ
  const uint32_t low_mask = top == 32 ? 0xFFFFFFFFu : ((1u << top) - 1u);
  uint32_t lo = mn & ~low_mask, hi = lo | low_mask, above = 0u;
  for (int level = 0; level < levels && top > 0; ++level) {
    const int shift = top > 12 ? top - 12 : 0, nb = 1 << (top - shift);
    for (int i = tid; i < nb; i += NTH) sh.hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < nl; i += NTH) {
      const uint32_t key = keys[i];
      if (key >= lo && key <= hi) atomicAdd(&sh.hist[(key >> shift) & (nb - 1)], 1u);
    }
    __syncthreads();
    find_bin(sh, nb, above, k);
    above = sh.sel_above;
    const uint32_t in_bin = sh.hist[sh.sel_bin];
    lo |= sh.sel_bin << shift;
    hi = lo | (shift == 0 ? 0u : ((1u << shift) - 1u));
    top = shift;
    const bool finish = top > 0 && level + 1 < levels && in_bin <= kFinishMax;  // uniform
    if (finish && tid == 0) sh.fin_n = 0;
    __syncthreads();
    if (finish) return rank_in_window(sh, nl, keys, lo, hi, k - above, in_bin);
  }
  return lo;
}

// Sampled path (see the file comment).  Returns false, having written
// nothing, when the gathered list misses [k, capacity]; the caller then takes
// the exact path.  Needs a 16-byte aligned row with n >= kSampleMinN; the
// bitmap area (n_words * 8 bytes >= n / 4 bytes) doubles as the sample buffer.
// The sampled threshold estimate: one 64-key chunk in kSampleStride of the
// row (chunks spread over the whole row) is read into `sample` (at most n/4
// + 240 bytes of LDS, for the f16 rows' 1 in 16) and its exact r-th largest
// key returned, with r chosen so that about
// target_eighths / 8 of k keys of the full row are expected at or above it.
// Needs a 16-byte aligned row with n >= kSampleMinN.
// The estimate from the m sampled keys of a row of n: the key of sample rank
// ceil(target * m / n), target = target_eighths / 8 of k (1.375 k unless the
// caller asks for more), so that about `target` keys of the row lie above it.
static __device__ __forceinline__ uint32_t sample_select(TopkShared& sh, int m, int64_t n, int32_t k, uint32_t* sample,
                                                  int32_t target_eighths) {
  const int64_t target = (int64_t)k * target_eighths / 8;
  int64_t rs = (target * m + n - 1) / n;
  if (rs < 1) rs = 1;
  if (rs > m) rs = m;
  return select_in_list(sh, m, sample, (uint32_t)rs, kSampleLevels);
}

static __device__ __forceinline__ uint32_t sample_estimate(TopkShared& sh, const float* __restrict__ row, int64_t n,
                                                    int32_t k, uint32_t* sample, int32_t target_eighths = 11) {
  const int tid = threadIdx.x;
  // sampled chunk j: keys 64*(S*j + (5*j % S)) .. +63 with S = kSampleStride, whole chunks inside the row
  const int64_t n_chunks = n / 64;
  const int m_chunks = (int)((n_chunks + kSampleStride - 1) / kSampleStride);
  const int m = sampled_keys(n_chunks, kSampleStride);  // a multiple of 64
  for (int f = tid; f < m_chunks * 16; f += NTH) {
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
  return sample_select(sh, m, n, k, sample, target_eighths);
}

// sample_estimate over an f16 tile row (16-byte aligned), one chunk in kSampleStrideH.
static __device__ __forceinline__ uint32_t sample_estimate_h(TopkShared& sh, const _Float16* __restrict__ row, float scale,
                                                      int64_t n, int32_t k, uint32_t* sample, int32_t target_eighths) {
  const int tid = threadIdx.x;
  const int64_t n_chunks = n / 64;
  const int m_chunks = (int)((n_chunks + kSampleStrideH - 1) / kSampleStrideH);
  const int m = sampled_keys(n_chunks, kSampleStrideH);
  for (int f = tid; f < m_chunks * 8; f += NTH) {
    const int j = f >> 3;
    const int64_t chunk = (int64_t)kSampleStrideH * j + (5 * j) % kSampleStrideH;
    if (chunk < n_chunks) {
      const v8h v = *(const v8h*)(row + 64 * chunk + 8 * (f & 7));
      uint32_t* dst = sample + 64 * j + 8 * (f & 7);
#pragma unroll
      for (int i = 0; i < 8; ++i) dst[i] = h_key(v[i], scale);
    }
  }
  __syncthreads();
  return sample_select(sh, m, n, k, sample, target_eighths);
}

static __device__ __forceinline__ bool topk_sampled(TopkShared& sh, const float* __restrict__ row, int64_t n, int32_t k,
                                             uint32_t* gt_bits, uint32_t* eq_bits, int n_words,
                                             int32_t* __restrict__ out) {
  const int tid = threadIdx.x;
  // the candidate pass's first loads go out with the sample's (measured on
  // MI355X: decode top-k 23.1 -> 22.5 us on 64 x 32K)
  v4f first[4];
  const bool pre = n >= 16 * NTH;  // uniform
  if (pre) first_batch_f(row, first);
  const uint32_t t_est = sample_estimate(sh, row, n, k, gt_bits);

  if (tid == 0) sh.list_n = 0;
  __syncthreads();
  gather_ge_f(sh, row, n, t_est, pre, first);
  __syncthreads();
  const uint32_t c = sh.list_n;
  if (c < (uint32_t)k || c > (uint32_t)kTopkCap) return false;  // uniform across the workgroup

  const uint32_t hi = select_in_list(sh, (int)c, sh.list_key, (uint32_t)k, 3);  // theta, the k-th largest
  const int rw = (int)((n + 31) / 32);  // bitmap words of this row
  for (int i = tid; i < rw; i += NTH) {
    gt_bits[i] = 0;
    eq_bits[i] = 0;
  }
  __syncthreads();
  for (int i = tid; i < (int)c; i += NTH) {
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
static __device__ __forceinline__ void topk_exact_row(TopkShared& sh, const float* __restrict__ row, int64_t n, bool vec,
                                               int32_t k, uint32_t* gt_bits, uint32_t* eq_bits, int n_words,
                                               int32_t* __restrict__ out) {
  const int tid = threadIdx.x;
  // Current candidate key range [lo, hi]; `above` keys are > hi.
  uint32_t lo = 0u, hi = 0xFFFFFFFFu, above = 0u, in_range = (uint32_t)n;
  int level = 0;  // 0: bits 31..20, 1: bits 19..8, 2: bits 7..0
  for (; level < 3; ++level) {
    if (level > 0 && in_range <= (uint32_t)kTopkCap) break;
    const int sh_ = level_shift(level), nb = 1 << level_bits(level);
    for (int i = tid; i < nb; i += NTH) sh.hist[i] = 0;
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
  for (int i = tid; i < rw; i += NTH) {
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
    for (int i = tid; i < nl; i += NTH) {
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

};

template <int NTH>
__global__ __launch_bounds__(NTH) void topk_kernel(const float* __restrict__ scores, int64_t ld, int64_t T,
                                                   int64_t N, int64_t q_pos0, const int32_t* __restrict__ n_valid,
                                                   int32_t k, int32_t* __restrict__ idx, int32_t n_words) {
  using Ops = TopkOps<NTH>;
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
    for (int i = tid; i < k; i += NTH) out[i] = i < n ? i : -1;
    return;
  }
  const float* row = scores + t * ld;
  const bool vec = ((reinterpret_cast<uintptr_t>(row) & 15) == 0);
  if (vec && n >= kSampleMinN && Ops::topk_sampled(sh, row, n, k, gt_bits, eq_bits, n_words, out)) return;
  Ops::topk_exact_row(sh, row, n, vec, k, gt_bits, eq_bits, n_words, out);
}

// Every kernel here takes up to kTopkLdsCap bytes of dynamic LDS: the fixed
// state and the two bitmaps of a 262144-key row.
constexpr int kTopkLdsCap = (int)(sizeof(TopkShared) + sizeof(uint32_t) * 2 * 8192 + 256);

// Raises the dynamic-LDS limit of the given kernels to kTopkLdsCap on the
// current device, once per device (the limit is a per-device attribute): the
// device's bit in `done` records it, so concurrent callers at worst set it
// twice.  Devices past the 64th set it on every call.
inline hipError_t lds_limit_once(std::atomic<uint64_t>& done, std::initializer_list<const void*> kernels) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = (dev >= 0 && dev < 64) ? (1ull << dev) : 0ull;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  for (const void* fn : kernels) {
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kTopkLdsCap);
    if (e != hipSuccess) return e;
  }
  if (bit) done.fetch_or(bit, std::memory_order_release);
  return hipSuccess;
}

hipError_t launch_topk(const float* scores, int64_t ld, int64_t T, int64_t N, int64_t q_pos0,
                       const int32_t* n_valid, int32_t k, int32_t* idx, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  const int32_t n_words = (int32_t)((N + 31) / 32);
  // bitmaps (2 x n_words words) + 256 bytes: the sampled path's key sample
  // (at most n/4 + 240 bytes) reuses the bitmap area
  const size_t lds = sizeof(TopkShared) + sizeof(uint32_t) * 2 * (size_t)n_words + 256;
  static std::atomic<uint64_t> lds_set{0};
  if (hipError_t e = lds_limit_once(lds_set, {(const void*)topk_kernel<kTopkThreads>,
                                              (const void*)topk_kernel<kTopkWideThreads>}))
    return e;
  // Few rows (decode) leave most compute units idle: each row's workgroup is
  // alone on its compute unit, so it takes twice the threads (measured on
  // MI355X: 64 rows of 32K keys 28.7 -> 26.8 us).
  if (T <= kTopkWideMaxRows)
    hipLaunchKernelGGL(topk_kernel<kTopkWideThreads>, dim3((unsigned)T), dim3(kTopkWideThreads), lds, st, scores,
                       ld, T, N, q_pos0, n_valid, k, idx, n_words);
  else
    hipLaunchKernelGGL(topk_kernel<kTopkThreads>, dim3((unsigned)T), dim3(kTopkThreads), lds, st, scores, ld, T,
                       N, q_pos0, n_valid, k, idx, n_words);
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

// The estimate and finish kernels run one workgroup of NTH threads per row
// (kTopkWideThreads for launches of few rows, as topk_kernel).  Measured on
// MI355X, 32 rows of 4K..128K: the collect kernel's batched append took the
// three kernels from 33.7 to 32.4 us, the wide workgroups to 32.0 us.
template <int NTH>
__global__ __launch_bounds__(NTH) void topk_rows_estimate_kernel(const float* __restrict__ scores, int64_t ld,
                                                                 int64_t N, const int32_t* __restrict__ n_valid,
                                                                 int32_t k, RowsMeta* __restrict__ meta) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  TopkShared& sh = *reinterpret_cast<TopkShared*>(smem);
  uint32_t* sample = reinterpret_cast<uint32_t*>(smem + sizeof(TopkShared));
  const int64_t t = blockIdx.x;
  const int64_t n = row_len(n_valid, t, N);
  const float* row = scores + t * ld;
  uint32_t t_est = 0u;
  if (row_sampled(row, n, k)) t_est = TopkOps<NTH>::sample_estimate(sh, row, n, k, sample);
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
  // the chunk's 16 keys of this thread, marked when inside the row and >= t_est
  uint32_t key[16], m = 0u;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t s = s0 + 4 * (threadIdx.x + 256 * u);
    v4f v = {0.f, 0.f, 0.f, 0.f};
    if (s + 3 < s1) {
      v = *(const v4f*)(row + s);
    } else {
      for (int j = 0; j < 4; ++j)
        if (s + j < s1) v[j] = row[s + j];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      key[4 * u + j] = order_key(v[j]);
      m |= (s + j < s1 && key[4 * u + j] >= t_est ? 1u : 0u) << (4 * u + j);
    }
  }
  append_marked<16>(&ln, lkey, lidx, (uint32_t)kRowChunk, key, m,
                    [&](int j) { return s0 + 4 * (threadIdx.x + 256 * (j >> 2)) + (j & 3); });
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

template <int NTH>
__global__ __launch_bounds__(NTH) void topk_rows_finish_kernel(
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
    for (int i = tid; i < k; i += NTH) out[i] = i < n ? i : -1;
    return;
  }
  const float* row = scores + t * ld;
  const bool vec = (reinterpret_cast<uintptr_t>(row) & 15) == 0;
  const uint32_t c = row_sampled(row, n, k) ? meta[t].n_cand : 0u;
  if (c < (uint32_t)k || c > (uint32_t)kTopkCap) {  // uniform: the exact path over the row
    TopkOps<NTH>::topk_exact_row(sh, row, n, vec, k, gt_bits, eq_bits, n_words_max, out);
    return;
  }
  const int n_words = (int)((n + 31) / 32);  // bitmap words of this row
  for (int i = tid; i < n_words; i += NTH) {
    gt_bits[i] = 0u;
    eq_bits[i] = 0u;
  }
  for (int i = tid; i < (int)c; i += NTH) {
    sh.list_key[i] = cand_key[t * kTopkCap + i];
    sh.list_idx[i] = cand_idx[t * kTopkCap + i];
  }
  __syncthreads();
  // theta, the k-th largest
  const uint32_t hi = TopkOps<NTH>::select_in_list(sh, (int)c, sh.list_key, (uint32_t)k, 3);
  for (int i = tid; i < (int)c; i += NTH) {
    const uint32_t key = sh.list_key[i];
    const int32_t s = sh.list_idx[i];
    if (key > hi)
      atomicOr(&gt_bits[s >> 5], 1u << (s & 31));
    else if (key == hi)
      atomicOr(&eq_bits[s >> 5], 1u << (s & 31));
  }
  __syncthreads();
  TopkOps<NTH>::emit_selection(sh, gt_bits, eq_bits, n_words, (uint32_t)k, out);
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
  static std::atomic<uint64_t> lds_set{0};
  if (hipError_t e = lds_limit_once(lds_set, {(const void*)topk_rows_finish_kernel<kTopkThreads>,
                                              (const void*)topk_rows_estimate_kernel<kTopkThreads>,
                                              (const void*)topk_rows_finish_kernel<kTopkWideThreads>,
                                              (const void*)topk_rows_estimate_kernel<kTopkWideThreads>}))
    return e;
  const bool wide = T <= kTopkWideMaxRows;
  const dim3 block(wide ? kTopkWideThreads : kTopkThreads);
  if (wide)
    hipLaunchKernelGGL(topk_rows_estimate_kernel<kTopkWideThreads>, dim3((unsigned)T), block, lds, st, scores, ld, N,
                       n_valid, k, meta);
  else
    hipLaunchKernelGGL(topk_rows_estimate_kernel<kTopkThreads>, dim3((unsigned)T), block, lds, st, scores, ld, N,
                       n_valid, k, meta);
  hipLaunchKernelGGL(topk_rows_collect_kernel, dim3((unsigned)n_chunks, (unsigned)T), dim3(256), 0, st, scores, ld,
                     N, n_valid, k, meta, cand_key, cand_idx);
  if (wide)
    hipLaunchKernelGGL(topk_rows_finish_kernel<kTopkWideThreads>, dim3((unsigned)T), block, lds, st, scores, ld, N,
                       n_valid, k, meta, cand_key, cand_idx, idx, n_words);
  else
    hipLaunchKernelGGL(topk_rows_finish_kernel<kTopkThreads>, dim3((unsigned)T), block, lds, st, scores, ld, N,
                       n_valid, k, meta, cand_key, cand_idx, idx, n_words);
  return hipGetLastError();
}

// ------------------------------------------------------------ fused prefill: band selection
// The fused prefill scores every causal pair with the FP8 scoring pass
// (indexer.hip) and selects on those approximate scores I~ as follows, which
// gives exactly the selection the exact scores I (those of
// dsa_indexer_scores, bit for bit) give.  With |I~[s] - I[s]| <= E[s] =
// fac S[s] + r I~[s] + eps (the bound of the scoring pass, r = 1.0625 2^-9;
// I~ >= 0 on rows that are not flagged) and theta~ the k-th largest I~ of the
// row, the k-th largest exact score theta lies in [L, U] = theta~ -+ H with
// H = fac max(S) + r theta~ + eps.  A key with I~ - E > U is above theta,
// so it is selected whatever the ties; one with I~ + E < L is below theta and
// is not.  Every other key (the band, a few hundred per row) is rescored with
// the exact arithmetic, and the band's (k - #sure) largest exact scores, ties
// to the lower position, complete the selection: every key whose exact score
// equals theta is in the band, so the tie rule sees all of them.  Rows that
// are flagged, or whose candidate list would overflow, are rescored whole and
// take the plain selection.
struct BandArgs {
  const uint8_t* q_idx;     // the tile's query rows [T, H_I, 128]
  const float* w;           // [T, H_I]
  const uint8_t* k_idx;     // keys: rows 0..N-1, or a page pool through page_table
  const int32_t* page_table;  // nullptr: contiguous keys; else the sequence's page-table row
  int32_t max_pages;
  int32_t page_shift;
  int64_t n_pages;
  int32_t H_I;
  const float* key_s;       // [N] S of each key
  const uint32_t* glob;     // [0]: largest S (float bits)
  const float* row_fac;     // [T]
  const float* row_eps;     // [T]
  const int32_t* row_flag;  // [T] nonzero: exact route
  const float* row_scale;   // [T] 2^s: the tile holds each row's scores times 2^-s, in f16
};

// Row of k_idx holding key s (-1: no backing row, a zero key).  A template
// parameter, so that the contiguous kernel carries none of the paged lookup.
template <bool kPaged>
__device__ __forceinline__ int64_t band_key_row(const BandArgs& ba, int64_t s) {
  if constexpr (!kPaged) return s;
  return AddrPaged{ba.page_table, ba.max_pages, ba.page_shift, ba.n_pages}.row(0, s);
}

// inverse of order_key
__device__ __forceinline__ float key_float(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// The k-th largest key of a row (theta) by radix refinement over the row,
// then over the threshold bin gathered into the LDS list; scan(fn) calls
// fn(s, key) for every candidate of the row.
template <class Scan>
__device__ __forceinline__ uint32_t row_theta_exact(TopkShared& sh, int64_t n, int32_t k, Scan&& scan) {
  const int tid = threadIdx.x;
  uint32_t lo = 0u, hi = 0xFFFFFFFFu, above = 0u, in_range = (uint32_t)n;
  int level = 0;
  for (; level < 3; ++level) {
    if (level > 0 && in_range <= (uint32_t)kTopkCap) break;
    const int sh_ = level_shift(level), nb = 1 << level_bits(level);
    for (int i = tid; i < nb; i += kTopkThreads) sh.hist[i] = 0;
    __syncthreads();
    scan([&](int64_t, uint32_t key) {
      if (key >= lo && key <= hi) atomicAdd(&sh.hist[(key >> sh_) & (nb - 1)], 1u);
    });
    __syncthreads();
    TopkOps<kTopkThreads>::find_bin(sh, nb, above, (uint32_t)k);
    const uint32_t bin = sh.sel_bin;
    above = sh.sel_above;
    in_range = sh.hist[bin];
    const uint32_t span = (sh_ == 0) ? 0u : ((1u << sh_) - 1u);
    lo = (lo & ~(((uint32_t)(nb - 1)) << sh_)) | (bin << sh_);
    hi = lo | span;
    __syncthreads();
  }
  if (lo == hi) return lo;
  if (tid == 0) sh.list_n = 0;
  __syncthreads();
  scan([&](int64_t s, uint32_t key) {
    if (key >= lo && key <= hi) {
      const uint32_t slot = atomicAdd(&sh.list_n, 1u);
      sh.list_key[slot] = key;
      sh.list_idx[slot] = (int32_t)s;
    }
  });
  __syncthreads();
  TopkOps<kTopkThreads>::refine_list(sh, (int)sh.list_n, lo, hi, above, level, (uint32_t)k, sh.list_key);
  return lo;
}

// Exact scores of nk keys of one query row, each wave taking 64 keys at a
// time through the score kernels' own arithmetic (indexer_exact.h): entry e
// is the key in row key_row(e) of k_idx (with kZeroKeys, -1 is a zero key);
// out(e, score) runs on the lane that holds entry e.
template <int NT, bool kZeroKeys, class RowFn, class OutFn>
__device__ __forceinline__ void rescore_exact(const uint8_t* __restrict__ q_row, const float* __restrict__ w_row,
                                              int32_t H_I, const uint8_t* __restrict__ k_idx, int nk,
                                              RowFn key_row, OutFn out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int n_chunks = (nk + 63) / 64;
  if (wave >= n_chunks) return;
  Frag a[NT];
  float wr[NT][4];
  load_query<NT>(q_row, w_row, 0, true, H_I, col, grp, a, wr);
  for (int ch = wave; ch < n_chunks; ch += kTopkThreads / kWave) {
    float part[4];
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
      const int e = min(64 * ch + 16 * blk + col, nk - 1);
      const int64_t r = key_row(e);
      if constexpr (kZeroKeys) {  // a zero key scores +0 exactly, whatever row 0 holds
        const v4i* p = (const v4i*)(k_idx + (r < 0 ? 0 : r) * kIdxD + 32 * grp);
        const float h = head_sum<NT>(a, wr, widen32(p[0], p[1]));
        part[blk] = r < 0 ? 0.f : h;
      } else {
        const v4i* p = (const v4i*)(k_idx + r * kIdxD + 32 * grp);
        part[blk] = head_sum<NT>(a, wr, widen32(p[0], p[1]));
      }
    }
    const float v = group_transpose_reduce(part[0], part[1], part[2], part[3], grp);
    const int e = 64 * ch + lane;
    if (e < nk) out(e, v);
  }
}

// Relative part of the bound E (the f16 roundings of the scoring pass and of
// the stored score).
constexpr float kRelErr = 0x1.1p-9f;

// The band selection of one row (see above).  Returns false, having written
// no output, when the row must take the exact route instead.
template <int NT, bool kPaged>
__device__ __forceinline__ bool band_select(TopkShared& sh, const _Float16* __restrict__ row, int64_t n, int32_t k,
                                            int64_t t, const BandArgs& ba, uint32_t* gt_bits, uint32_t* eq_bits,
                                            int32_t* __restrict__ out) {
  constexpr int kPer = (kTopkCap + kTopkThreads - 1) / kTopkThreads;  // list entries per thread
  const int tid = threadIdx.x;
  // theta~: from the sampled candidate list when it brackets rank k, else by
  // radix refinement over the row
  const float scale = ba.row_scale[t];
  auto scan = [&](auto&& fn) { TopkOps<kTopkThreads>::scan_row_h(row, scale, n, fn); };
  uint32_t th_key = 0u, t_low = 0xFFFFFFFFu;
  bool have_list = false;
  if (n >= kSampleMinN) {
    // 1.5 k keys expected above the estimate: the band reaches about 1.2 k
    // to 1.3 k below the top on these workloads, so the list gathered here
    // usually holds every band key and no second pass over the row is needed
    // the candidate pass's first loads go out with the sample's, one memory
    // round trip for both (measured on MI355X: 5.00 -> 4.95 ms of top-k per
    // chunked paged prefill call; the 128K prefill's 15.7 ms unchanged)
    v8h first[4];
    const bool pre = n >= 32 * kTopkThreads;  // uniform
    if (pre) TopkOps<kTopkThreads>::first_batch_h(row, first);
    const uint32_t t_est = TopkOps<kTopkThreads>::sample_estimate_h(sh, row, scale, n, k, gt_bits, 12);
    if (tid == 0) sh.list_n = 0;
    __syncthreads();
    TopkOps<kTopkThreads>::gather_ge_h(sh, row, scale, n, t_est, pre, first);
    __syncthreads();
    const uint32_t c = sh.list_n;
    if (c >= (uint32_t)k && c <= (uint32_t)kTopkCap) {
      th_key = TopkOps<kTopkThreads>::select_in_list(sh, (int)c, sh.list_key, (uint32_t)k, 3);
      have_list = true;
      t_low = t_est;
    }
  }
  if (!have_list) th_key = row_theta_exact(sh, n, k, scan);

  // the bracket [L, U] of theta and the lowest approximate score a band key
  // can have; the 2^-18 terms cover the fp32 rounding of these sums
  const float theta = key_float(th_key);
  const float fac = ba.row_fac[t], eps = ba.row_eps[t];
  const float base = fmaf(fac, __uint_as_float(ba.glob[0]), eps);
  float H = fmaf(kRelErr, fabsf(theta), base);
  H += 0x1p-18f * (fabsf(theta) + H);
  const float U = theta + H, L = theta - H;
  const float lcut = L - base - 2.f * kRelErr * fabsf(L) - 0x1p-18f * (fabsf(L) + base);
  const uint32_t key_lcut = order_key(lcut);

  // candidate list: every key with I~ >= lcut (the sampled list already holds
  // them when its threshold is at or below lcut; its other entries classify
  // as out below)
  if (!(have_list && key_lcut >= t_low)) {
    if (tid == 0) sh.list_n = 0;
    __syncthreads();
    v8h none[4];  // not read
    TopkOps<kTopkThreads>::gather_ge_h(sh, row, scale, n, key_lcut, false, none);
    __syncthreads();
    if (sh.list_n > (uint32_t)kTopkCap) return false;  // uniform across the workgroup
  }

  // classify the list: sure keys into the "> theta" bitmap, band keys
  // compacted into the front of the list (positions only), the rest out
  const int nl = (int)sh.list_n;
  const int rw = (int)((n + 31) / 32);  // bitmap words of this row
  for (int i = tid; i < rw; i += kTopkThreads) {
    gt_bits[i] = 0u;
    eq_bits[i] = 0u;
  }
  int32_t pos[kPer];
  int cls[kPer];  // 0 out, 1 sure, 2 band
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = tid + kTopkThreads * j;
    cls[j] = 0;
    pos[j] = 0;
    if (i < nl) {
      const float x = key_float(sh.list_key[i]);
      pos[j] = sh.list_idx[i];
      float E = fmaf(fac, ba.key_s[pos[j]], fmaf(kRelErr, fabsf(x), eps));
      E += 0x1p-18f * (fabsf(x) + E);
      cls[j] = (x - E > U) ? 1 : ((x + E >= L) ? 2 : 0);
    }
  }
  __syncthreads();
  if (tid == 0) {
    sh.list_n = 0;
    sh.n_sure = 0;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    if (cls[j] == 1) {
      atomicOr(&gt_bits[pos[j] >> 5], 1u << (pos[j] & 31));
      atomicAdd(&sh.n_sure, 1u);
    } else if (cls[j] == 2) {
      sh.list_idx[atomicAdd(&sh.list_n, 1u)] = pos[j];
    }
  }
  __syncthreads();
  const int nb = (int)sh.list_n;
  const uint32_t n_sure = sh.n_sure;
  // the bound guarantees n_sure < k <= n_sure + nb; were it ever violated the
  // row takes the exact route (uniform)
  if (n_sure >= (uint32_t)k || (uint32_t)nb < (uint32_t)k - n_sure) return false;

  // exact scores of the band keys, as order keys in the list
  rescore_exact<NT, kPaged>(ba.q_idx + t * ba.H_I * kIdxD, ba.w + t * ba.H_I, ba.H_I, ba.k_idx, nb,
                    [&](int e) { return band_key_row<kPaged>(ba, sh.list_idx[e]); },
                    [&](int e, float v) { sh.list_key[e] = order_key(v); });
  __syncthreads();
  // theta itself
  const uint32_t hi = TopkOps<kTopkThreads>::select_in_list(sh, nb, sh.list_key, (uint32_t)k - n_sure, 3);
  for (int i = tid; i < nb; i += kTopkThreads) {
    const uint32_t key = sh.list_key[i];
    const int32_t s = sh.list_idx[i];
    if (key > hi)
      atomicOr(&gt_bits[s >> 5], 1u << (s & 31));
    else if (key == hi)
      atomicOr(&eq_bits[s >> 5], 1u << (s & 31));
  }
  __syncthreads();
  TopkOps<kTopkThreads>::emit_selection(sh, gt_bits, eq_bits, rw, (uint32_t)k, out);
  return true;
}

// One workgroup per row of the fused prefill's score tile (approximate
// scores of the candidates, f16 scaled per row).  Rows without a band
// selection are rescored in place with the exact arithmetic (as fp32, over
// the row's full fp32 stride) and take the plain selection.
template <int NT, bool kPaged>
__global__ __launch_bounds__(kTopkThreads) void topk_band_kernel(float* __restrict__ scores, int64_t ld, int64_t T,
                                                                  int64_t N, int64_t q_pos0, int32_t k,
                                                                  int32_t* __restrict__ idx, int32_t n_words,
                                                                  BandArgs ba) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  TopkShared& sh = *reinterpret_cast<TopkShared*>(smem);
  uint32_t* gt_bits = reinterpret_cast<uint32_t*>(smem + sizeof(TopkShared));
  uint32_t* eq_bits = gt_bits + n_words;
  const int tid = threadIdx.x;
  const int64_t t = blockIdx.x;
  int64_t n = q_pos0 + t + 1;
  n = n > N ? N : n;
  int32_t* out = idx + t * (int64_t)k;
  if (n <= k) {
    for (int i = tid; i < k; i += kTopkThreads) out[i] = i < n ? i : -1;
    return;
  }
  float* row = scores + t * ld;  // 16-byte aligned (ld is a multiple of 64)
  if (ba.row_flag[t] == 0 && band_select<NT, kPaged>(sh, reinterpret_cast<const _Float16*>(row), n, k, t, ba, gt_bits,
                                             eq_bits, out))
    return;
  // exact route: the whole row rescored in place as fp32, then the plain selection
  rescore_exact<NT, kPaged>(ba.q_idx + t * ba.H_I * kIdxD, ba.w + t * ba.H_I, ba.H_I, ba.k_idx, (int)n,
                    [&](int e) { return band_key_row<kPaged>(ba, e); }, [&](int e, float v) { row[e] = v; });
  __threadfence();
  __syncthreads();
  if (n >= kSampleMinN && TopkOps<kTopkThreads>::topk_sampled(sh, row, n, k, gt_bits, eq_bits, n_words, out))
    return;
  TopkOps<kTopkThreads>::topk_exact_row(sh, row, n, true, k, gt_bits, eq_bits, n_words, out);
}

namespace {
template <int NT, bool kPaged>
hipError_t topk_band_nt(float* scores, int64_t ld, int64_t T, int64_t N, int64_t q_pos0, int32_t k, int32_t* idx,
                        const BandArgs& ba, hipStream_t st) {
  const int32_t n_words = (int32_t)((N + 31) / 32);
  const size_t lds = sizeof(TopkShared) + sizeof(uint32_t) * 2 * (size_t)n_words + 256;
  static std::atomic<uint64_t> lds_set{0};
  if (hipError_t e = lds_limit_once(lds_set, {(const void*)topk_band_kernel<NT, kPaged>})) return e;
  hipLaunchKernelGGL((topk_band_kernel<NT, kPaged>), dim3((unsigned)T), dim3(kTopkThreads), lds, st, scores, ld, T, N, q_pos0,
                     k, idx, n_words, ba);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_topk_band(float* scores, int64_t ld, int64_t T, int64_t N, int64_t q_pos0, int32_t k,
                            int32_t* idx, const uint8_t* q_idx, const float* w, const uint8_t* k_idx, int32_t H_I,
                            const float* key_s, const uint32_t* glob, const float* row_fac, const float* row_eps,
                            const int32_t* row_flag, const float* row_scale, const PagedArgs* paged,
                            hipStream_t st) {
  if (T <= 0) return hipSuccess;
  const BandArgs ba{q_idx,
                    w,
                    k_idx,
                    paged ? paged->page_table : nullptr,
                    paged ? paged->max_pages : 0,
                    paged ? __builtin_ctz((unsigned)paged->page_size) : 0,
                    paged ? paged->n_pages : 0,
                    H_I,
                    key_s,
                    glob,
                    row_fac,
                    row_eps,
                    row_flag,
                    row_scale};
  switch ((H_I + 15) / 16) {
    case 1: return paged ? topk_band_nt<1, true>(scores, ld, T, N, q_pos0, k, idx, ba, st)
                         : topk_band_nt<1, false>(scores, ld, T, N, q_pos0, k, idx, ba, st);
    case 2: return paged ? topk_band_nt<2, true>(scores, ld, T, N, q_pos0, k, idx, ba, st)
                         : topk_band_nt<2, false>(scores, ld, T, N, q_pos0, k, idx, ba, st);
    case 3: return paged ? topk_band_nt<3, true>(scores, ld, T, N, q_pos0, k, idx, ba, st)
                         : topk_band_nt<3, false>(scores, ld, T, N, q_pos0, k, idx, ba, st);
    default: return paged ? topk_band_nt<4, true>(scores, ld, T, N, q_pos0, k, idx, ba, st)
                          : topk_band_nt<4, false>(scores, ld, T, N, q_pos0, k, idx, ba, st);
  }
}

}  // namespace dsa
