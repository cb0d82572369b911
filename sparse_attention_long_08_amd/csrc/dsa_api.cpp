// C ABI of the DSA forward library: host-side validation, workspace sizing
// and kernel dispatch.  Every check runs before any launch, so a rejected
// call touches no output.  See include/dsa.h for the contract of each call.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <vector>

#include "../../include/dsa.h"
#include "launch.h"

namespace {

thread_local char g_err[512] = "";

dsa_status fail(dsa_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

dsa_status ok() {
  g_err[0] = '\0';
  return DSA_OK;
}

dsa_status hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// ---- launch timing (dsa_timing_begin / dsa_timing_end): per host thread
struct TimedLaunch {
  int32_t kind;
  hipEvent_t start, stop;
};
thread_local bool g_timing = false;
thread_local std::vector<TimedLaunch> g_timed;

// Runs `launch` (which enqueues one stage's kernels on st); while timing is
// on, brackets it with two events recorded on st.
template <class F>
hipError_t timed(int32_t kind, hipStream_t st, F&& launch) {
  if (!g_timing) return launch();
  TimedLaunch t{kind, nullptr, nullptr};
  hipError_t e = hipEventCreate(&t.start);
  if (e != hipSuccess) return e;
  e = hipEventCreate(&t.stop);
  if (e == hipSuccess) e = hipEventRecord(t.start, st);
  if (e == hipSuccess) e = launch();
  if (e == hipSuccess) e = hipEventRecord(t.stop, st);
  if (e != hipSuccess) {
    (void)hipEventDestroy(t.start);
    if (t.stop) (void)hipEventDestroy(t.stop);
    return e;
  }
  g_timed.push_back(t);
  return hipSuccess;
}

void drop_timed() {
  for (const TimedLaunch& t : g_timed) {
    (void)hipEventDestroy(t.start);
    (void)hipEventDestroy(t.stop);
  }
  g_timed.clear();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int64_t kMaxCtx = 262144;  // longest row the top-k bitmaps cover
constexpr int32_t kMaxK = 4096;
constexpr size_t kAlign = 256;

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

#define REQUIRE(cond, status, ...) \
  do {                             \
    if (!(cond)) return fail(status, __VA_ARGS__); \
  } while (0)

#define REQUIRE_PTR(p) REQUIRE((p) != nullptr, DSA_ERR_INVALID_ARG, "%s is NULL", #p)
#define REQUIRE_AL(p) REQUIRE(aligned16(p), DSA_ERR_INVALID_ARG, "%s is not 16-byte aligned", #p)

dsa_status check_indexer_shape(int32_t H_I, int32_t d_I) {
  REQUIRE(d_I == 128, DSA_ERR_UNSUPPORTED, "d_I must be 128 (got %d)", d_I);
  REQUIRE(H_I >= 1 && H_I <= 64, DSA_ERR_UNSUPPORTED, "H_I must be in [1, 64] (got %d)", H_I);
  return DSA_OK;
}

dsa_status check_mla_shape(int32_t H, int32_t D_qk, int32_t D_v, int32_t k) {
  REQUIRE(D_qk == 576, DSA_ERR_UNSUPPORTED, "D_qk must be 576 (got %d)", D_qk);
  REQUIRE(D_v == 512, DSA_ERR_UNSUPPORTED, "D_v must be 512 (got %d)", D_v);
  REQUIRE(H >= 1 && H <= 128, DSA_ERR_UNSUPPORTED, "H must be in [1, 128] (got %d)", H);
  REQUIRE(k >= 1 && k <= kMaxK, DSA_ERR_UNSUPPORTED, "k must be in [1, %d] (got %d)", kMaxK, k);
  return DSA_OK;
}

dsa_status check_paged(const void* pool, int64_t n_pages, const int32_t* page_table, int32_t max_pages,
                       const int32_t* ctx_len, int32_t page_size, int64_t max_ctx) {
  REQUIRE_PTR(pool);
  REQUIRE_PTR(page_table);
  REQUIRE_PTR(ctx_len);
  REQUIRE_AL(pool);
  REQUIRE(page_size == 64, DSA_ERR_UNSUPPORTED, "page_size must be 64 (got %d)", page_size);
  REQUIRE(n_pages >= 1 && max_pages >= 1, DSA_ERR_INVALID_ARG, "n_pages and max_pages must be >= 1");
  REQUIRE(max_ctx >= 1 && max_ctx <= (int64_t)max_pages * page_size, DSA_ERR_INVALID_ARG,
          "max_ctx (%lld) must be in [1, max_pages*page_size]", (long long)max_ctx);
  return DSA_OK;
}

// workspace pieces
size_t mla_ws(int64_t T, int32_t H, int32_t k) {
  const int32_t s = dsa::sparse_mla_splits(T, H, k);
  if (s <= 1) return 0;
  // f16 partial outputs, fp32 lse and scale per (query, split, head)
  return round_up(sizeof(uint16_t) * (size_t)T * s * H * 512) + 2 * round_up(sizeof(float) * (size_t)T * s * H);
}

int64_t prefill_tile_rows(int64_t T, int64_t N) {
  // score scratch of about 2 GiB (fp32 stride): enough rows that the top-k's
  // last round of workgroups is a small part of a launch, bounded memory
  int64_t rows = (int64_t)(((int64_t)1 << 29) / std::max<int64_t>(N, 1));
  rows = std::max<int64_t>(rows, 256);
  rows = (rows + 7) / 8 * 8;
  return std::min<int64_t>(rows, std::max<int64_t>(T, 1));
}

int64_t score_ld(int64_t N) { return (N + 63) / 64 * 64; }

}  // namespace

extern "C" {

int32_t dsa_abi_version(void) { return 2; }

const char* dsa_status_string(int32_t status) {
  switch (status) {
    case DSA_OK: return "ok";
    case DSA_ERR_INVALID_ARG: return "invalid argument";
    case DSA_ERR_UNSUPPORTED: return "unsupported shape";
    case DSA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case DSA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* dsa_last_error_message(void) { return g_err; }

dsa_status dsa_timing_begin(void) {
  drop_timed();
  g_timing = true;
  return ok();
}

dsa_status dsa_timing_end(double* ms, int64_t* launches, int32_t n_kinds) {
  g_timing = false;
  REQUIRE(n_kinds >= 0 && n_kinds <= DSA_KERNEL_KINDS, DSA_ERR_INVALID_ARG, "n_kinds must be in [0, %d]",
          DSA_KERNEL_KINDS);
  if (n_kinds > 0) {
    if (!ms || !launches) {
      drop_timed();
      return fail(DSA_ERR_INVALID_ARG, "ms and launches must not be NULL");
    }
    for (int32_t i = 0; i < n_kinds; ++i) {
      ms[i] = 0.0;
      launches[i] = 0;
    }
  }
  hipError_t err = hipSuccess;
  for (const TimedLaunch& t : g_timed) {
    float f = 0.f;
    hipError_t e = hipEventSynchronize(t.stop);
    if (e == hipSuccess) e = hipEventElapsedTime(&f, t.start, t.stop);
    if (e != hipSuccess) {
      if (err == hipSuccess) err = e;
      continue;
    }
    if (t.kind < n_kinds) {
      ms[t.kind] += f;
      launches[t.kind] += 1;
    }
  }
  drop_timed();
  return hip_check(err, "timing events");
}

dsa_status dsa_indexer_scores(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, int64_t T, int64_t N,
                              int32_t H_I, int32_t d_I, int64_t q_pos0, float* scores, int64_t ld,
                              dsa_stream_t stream) {
  REQUIRE(T >= 0 && N >= 1, DSA_ERR_INVALID_ARG, "T must be >= 0 and N >= 1");
  REQUIRE(q_pos0 >= 0, DSA_ERR_INVALID_ARG, "q_pos0 must be >= 0");
  REQUIRE(ld >= N, DSA_ERR_INVALID_ARG, "ld (%lld) must be >= N (%lld)", (long long)ld, (long long)N);
  if (dsa_status s = check_indexer_shape(H_I, d_I)) return s;
  if (T == 0) return ok();
  REQUIRE_PTR(q_idx); REQUIRE_PTR(w); REQUIRE_PTR(k_idx); REQUIRE_PTR(scores);
  REQUIRE_AL(q_idx); REQUIRE_AL(k_idx); REQUIRE_AL(w); REQUIRE_AL(scores);
  hipStream_t st = (hipStream_t)stream;
  return hip_check(timed(DSA_KERNEL_INDEXER, st,
                         [&] {
                           return dsa::launch_indexer_prefill(q_idx, w, k_idx, T, N, H_I, q_pos0, scores, ld, true,
                                                              nullptr, st);
                         }),
                   "indexer launch");
}

dsa_status dsa_indexer_scores_paged(const uint8_t* q_idx, const float* w, const uint8_t* k_pool, int64_t n_pages,
                                    const int32_t* page_table, int32_t max_pages, const int32_t* ctx_len,
                                    int32_t page_size, int64_t B, int32_t H_I, int32_t d_I, int64_t max_ctx,
                                    float* scores, int64_t ld, dsa_stream_t stream) {
  REQUIRE(B >= 0, DSA_ERR_INVALID_ARG, "B must be >= 0");
  if (dsa_status s = check_indexer_shape(H_I, d_I)) return s;
  if (dsa_status s = check_paged(k_pool, n_pages, page_table, max_pages, ctx_len, page_size, max_ctx)) return s;
  REQUIRE(ld >= max_ctx, DSA_ERR_INVALID_ARG, "ld must be >= max_ctx");
  if (B == 0) return ok();
  REQUIRE_PTR(q_idx); REQUIRE_PTR(w); REQUIRE_PTR(scores);
  REQUIRE_AL(q_idx); REQUIRE_AL(w); REQUIRE_AL(scores);
  dsa::PagedArgs pa{page_table, max_pages, page_size, n_pages};
  hipStream_t st = (hipStream_t)stream;
  return hip_check(timed(DSA_KERNEL_INDEXER, st,
                         [&] {
                           return dsa::launch_indexer_decode(q_idx, w, k_pool, 0, &pa, ctx_len, B, max_ctx, H_I,
                                                             scores, ld, st);
                         }),
                   "paged indexer launch");
}

dsa_status dsa_topk(const float* scores, int64_t ld, int64_t T, int64_t N, int64_t q_pos0, const int32_t* n_valid,
                    int32_t k, int32_t* idx, dsa_stream_t stream) {
  REQUIRE(T >= 0 && N >= 1, DSA_ERR_INVALID_ARG, "T must be >= 0 and N >= 1");
  REQUIRE(N <= kMaxCtx, DSA_ERR_UNSUPPORTED, "N must be <= %lld", (long long)kMaxCtx);
  REQUIRE(ld >= N, DSA_ERR_INVALID_ARG, "ld must be >= N");
  REQUIRE(q_pos0 >= 0, DSA_ERR_INVALID_ARG, "q_pos0 must be >= 0");
  REQUIRE(k >= 1 && k <= kMaxK, DSA_ERR_UNSUPPORTED, "k must be in [1, %d]", kMaxK);
  if (T == 0) return ok();
  REQUIRE_PTR(scores); REQUIRE_PTR(idx);
  REQUIRE_AL(scores); REQUIRE_AL(idx);
  hipStream_t st = (hipStream_t)stream;
  return hip_check(
      timed(DSA_KERNEL_TOPK, st, [&] { return dsa::launch_topk(scores, ld, T, N, q_pos0, n_valid, k, idx, st); }),
      "top-k launch");
}

size_t dsa_sparse_mla_fwd_workspace_bytes(int64_t T, int32_t H, int32_t /*D_v*/, int32_t k) {
  return mla_ws(T, H, k);
}

static dsa_status run_mla(const uint16_t* q, const uint16_t* kv, const int32_t* idx, int64_t T, int32_t H,
                          int32_t k, float scale, float* out, float* lse, void* ws, size_t ws_bytes,
                          bool seq_per_query, int64_t stride, int64_t seq_len, const int32_t* ctx_len,
                          const dsa::PagedArgs* paged, hipStream_t st) {
  const size_t need = mla_ws(T, H, k);
  REQUIRE(ws_bytes >= need, DSA_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes (got %zu)", need, ws_bytes);
  REQUIRE(need == 0 || ws != nullptr, DSA_ERR_INVALID_ARG, "ws is NULL");
  dsa::MlaArgs a{};
  a.q = q;
  a.kv = kv;
  a.idx = idx;
  a.T = T;
  a.H = H;
  a.k = k;
  a.scale = scale;
  a.out = out;
  a.lse = lse;
  a.seq_per_query = seq_per_query;
  a.stride = stride;
  a.seq_len = seq_len;
  a.ctx_len = ctx_len;
  a.paged = paged;
  a.n_split = dsa::sparse_mla_splits(T, H, k);
  if (a.n_split > 1) {
    char* w = (char*)ws;
    a.part_o = (uint16_t*)w;
    w += round_up(sizeof(uint16_t) * (size_t)T * a.n_split * H * 512);
    a.part_lse = (float*)w;
    w += round_up(sizeof(float) * (size_t)T * a.n_split * H);
    a.part_scale = (float*)w;
  }
  return hip_check(timed(DSA_KERNEL_ATTENTION, st, [&] { return dsa::launch_sparse_mla(a, st); }),
                   "sparse attention launch");
}

dsa_status dsa_sparse_mla_fwd(const uint16_t* q, const uint16_t* kv, const int32_t* idx, int64_t T, int64_t N,
                              int32_t H, int32_t D_qk, int32_t D_v, int32_t k, float scale, float* out,
                              float* lse, void* ws, size_t ws_bytes, dsa_stream_t stream) {
  REQUIRE(T >= 0 && N >= 1, DSA_ERR_INVALID_ARG, "T must be >= 0 and N >= 1");
  if (dsa_status s = check_mla_shape(H, D_qk, D_v, k)) return s;
  REQUIRE(scale > 0.f && scale < 1e30f, DSA_ERR_INVALID_ARG, "scale must be positive and finite");
  if (T == 0) return ok();
  REQUIRE_PTR(q); REQUIRE_PTR(kv); REQUIRE_PTR(idx); REQUIRE_PTR(out); REQUIRE_PTR(lse);
  REQUIRE_AL(q); REQUIRE_AL(kv); REQUIRE_AL(idx); REQUIRE_AL(out); REQUIRE_AL(lse);
  return run_mla(q, kv, idx, T, H, k, scale, out, lse, ws, ws_bytes, false, N, N, nullptr, nullptr,
                 (hipStream_t)stream);
}

// Queries per tile of the attention backward.  A tile's workspace holds P
// and dS (bf16 [tile, k rounded up to 32, H rounded up to 64]), the bf16 addend rows [tile, k, 576] (4.8 GB at
// k = 2048) and the inverted index of its entries.
constexpr int64_t kBwdTile = 2048;

namespace {
struct BwdWs {
  size_t p, ds, addend, count, offsets, list, total;
};
size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }
BwdWs bwd_ws(int64_t T, int64_t N, int32_t H, int32_t k) {
  const int64_t tile = T < kBwdTile ? T : kBwdTile;
  const size_t ent = (size_t)tile * (size_t)k;
  const size_t ent_p = (size_t)tile * (size_t)((k + 31) / 32 * 32);
  BwdWs w;
  size_t o = 0;
  w.p = o;
  o += al256(ent_p * dsa::mla_bwd_slot_heads(H) * 2);
  w.ds = o;
  o += al256(ent_p * dsa::mla_bwd_slot_heads(H) * 2);
  w.addend = o;
  o += al256(ent * 576 * 2);
  w.count = o;
  o += al256((size_t)N * 4);
  w.offsets = o;
  o += al256((size_t)(N + 1) * 4);
  w.list = o;
  o += al256(ent * 4);
  w.total = o;
  return w;
}
}  // namespace

size_t dsa_sparse_mla_bwd_workspace_bytes(int64_t T, int64_t N, int32_t H, int32_t k) {
  if (T <= 0 || N < 1 || H < 1 || k < 1) return 0;
  return bwd_ws(T, N, H, k).total;
}

dsa_status dsa_sparse_mla_bwd(const uint16_t* q, const uint16_t* kv, const int32_t* idx, const float* out,
                              const float* lse, const uint16_t* dout, int64_t T, int64_t N, int32_t H,
                              int32_t D_qk, int32_t D_v, int32_t k, float scale, float* dq, float* dkv,
                              void* ws, size_t ws_bytes, dsa_stream_t stream) {
  REQUIRE(T >= 0 && N >= 1, DSA_ERR_INVALID_ARG, "T must be >= 0 and N >= 1");
  REQUIRE(N <= (int64_t)1 << 30, DSA_ERR_UNSUPPORTED, "N must be <= 2^30 (got %lld)", (long long)N);
  if (dsa_status s = check_mla_shape(H, D_qk, D_v, k)) return s;
  REQUIRE(scale > 0.f && scale < 1e30f, DSA_ERR_INVALID_ARG, "scale must be positive and finite");
  REQUIRE_PTR(dkv);
  REQUIRE_AL(dkv);
  if (T > 0) {
    REQUIRE_PTR(q); REQUIRE_PTR(kv); REQUIRE_PTR(idx); REQUIRE_PTR(out); REQUIRE_PTR(lse); REQUIRE_PTR(dout);
    REQUIRE_PTR(dq); REQUIRE_PTR(ws);
    REQUIRE_AL(q); REQUIRE_AL(kv); REQUIRE_AL(idx); REQUIRE_AL(out); REQUIRE_AL(lse); REQUIRE_AL(dout);
    REQUIRE_AL(dq); REQUIRE_AL(ws);
    const size_t need = dsa_sparse_mla_bwd_workspace_bytes(T, N, H, k);
    REQUIRE(ws_bytes >= need, DSA_ERR_WORKSPACE_TOO_SMALL, "ws_bytes (%zu) below %zu", ws_bytes, need);
  }
  hipStream_t st = (hipStream_t)stream;
  if (hipError_t e = dsa::launch_zero_f32(dkv, N * (int64_t)D_qk, st)) return hip_check(e, "dkv clear");
  const BwdWs w = bwd_ws(T, N, H, k);
  uint8_t* const base = (uint8_t*)ws;
  for (int64_t t0 = 0; t0 < T; t0 += kBwdTile) {
    const int64_t tn = T - t0 < kBwdTile ? T - t0 : kBwdTile;
    dsa::MlaBwdArgs a;
    a.q = q + t0 * H * (int64_t)D_qk;
    a.kv = kv;
    a.idx = idx + t0 * (int64_t)k;
    a.out = out + t0 * H * (int64_t)D_v;
    a.lse = lse + t0 * H;
    a.dout = dout + t0 * H * (int64_t)D_v;
    a.T = tn;
    a.N = N;
    a.H = H;
    a.k = k;
    a.scale = scale;
    a.dq = dq + t0 * H * (int64_t)D_qk;
    a.pbuf = (uint16_t*)(base + w.p);
    a.dsbuf = (uint16_t*)(base + w.ds);
    a.addend = (uint16_t*)(base + w.addend);
    a.row_count = (int32_t*)(base + w.count);
    a.row_offsets = (int32_t*)(base + w.offsets);
    a.row_list = (int32_t*)(base + w.list);
    a.dkv = dkv;
    hipError_t e = timed(DSA_KERNEL_MLA_BWD_DQ, st, [&] { return dsa::launch_sparse_mla_bwd(a, 0, st); });
    if (e != hipSuccess) return hip_check(e, "attention backward (dq) launch");
    e = timed(DSA_KERNEL_MLA_BWD_DKV, st, [&] { return dsa::launch_sparse_mla_bwd(a, 1, st); });
    if (e != hipSuccess) return hip_check(e, "attention backward (dkv) launch");
    e = timed(DSA_KERNEL_MLA_BWD_REDUCE, st, [&] { return dsa::launch_sparse_mla_bwd(a, 2, st); });
    if (e != hipSuccess) return hip_check(e, "attention backward (row sums) launch");
  }
  return ok();
}

dsa_status dsa_indexer_kl_fwd(const uint16_t* q, const uint16_t* kv, const int32_t* idx, const float* lse,
                              const float* scores, int64_t ld, int64_t T, int64_t N, int32_t H, int32_t D_qk,
                              int32_t k, float scale, float* kl, dsa_stream_t stream) {
  REQUIRE(T >= 0 && N >= 1, DSA_ERR_INVALID_ARG, "T must be >= 0 and N >= 1");
  if (dsa_status s = check_mla_shape(H, D_qk, 512, k)) return s;
  REQUIRE(ld >= N, DSA_ERR_INVALID_ARG, "ld (%lld) must be >= N (%lld)", (long long)ld, (long long)N);
  REQUIRE(scale > 0.f && scale < 1e30f, DSA_ERR_INVALID_ARG, "scale must be positive and finite");
  if (T == 0) return ok();
  REQUIRE_PTR(q); REQUIRE_PTR(kv); REQUIRE_PTR(idx); REQUIRE_PTR(lse); REQUIRE_PTR(scores); REQUIRE_PTR(kl);
  REQUIRE_AL(q); REQUIRE_AL(kv); REQUIRE_AL(idx);
  hipStream_t st = (hipStream_t)stream;
  return hip_check(timed(DSA_KERNEL_INDEXER_KL, st,
                         [&] { return dsa::launch_indexer_kl(q, kv, N, idx, lse, scores, ld, T, H, k, scale, kl, st); }),
                   "indexer KL launch");
}

dsa_status dsa_indexer_dense_kl_fwd(const uint16_t* q, const uint16_t* kv, const float* scores, int64_t ld,
                                    int64_t T, int64_t N, int64_t q_pos0, int32_t H, int32_t D_qk, float scale,
                                    float* kl, float* lse, dsa_stream_t stream) {
  REQUIRE(T >= 0 && N >= 1, DSA_ERR_INVALID_ARG, "T must be >= 0 and N >= 1");
  REQUIRE(q_pos0 >= 0, DSA_ERR_INVALID_ARG, "q_pos0 must be >= 0");
  if (dsa_status s = check_mla_shape(H, D_qk, 512, 1)) return s;
  REQUIRE(ld >= N, DSA_ERR_INVALID_ARG, "ld (%lld) must be >= N (%lld)", (long long)ld, (long long)N);
  REQUIRE(scale > 0.f && scale < 1e30f, DSA_ERR_INVALID_ARG, "scale must be positive and finite");
  if (T == 0) return ok();
  REQUIRE_PTR(q); REQUIRE_PTR(kv); REQUIRE_PTR(scores); REQUIRE_PTR(kl);
  REQUIRE_AL(q); REQUIRE_AL(kv);
  hipStream_t st = (hipStream_t)stream;
  return hip_check(timed(DSA_KERNEL_DENSE_KL, st,
                         [&] {
                           return dsa::launch_indexer_dense_kl(q, kv, N, scores, ld, T, q_pos0, H, scale, kl, lse, st);
                         }),
                   "dense KL launch");
}

size_t dsa_sparse_mla_fwd_paged_workspace_bytes(int64_t B, int32_t H, int32_t /*D_v*/, int32_t k) {
  return mla_ws(B, H, k);
}

dsa_status dsa_sparse_mla_fwd_paged(const uint16_t* q, const uint16_t* kv_pool, int64_t n_pages,
                                    const int32_t* page_table, int32_t max_pages, const int32_t* ctx_len,
                                    int32_t page_size, const int32_t* idx, int64_t B, int32_t H, int32_t D_qk,
                                    int32_t D_v, int32_t k, float scale, float* out, float* lse, void* ws,
                                    size_t ws_bytes, dsa_stream_t stream) {
  REQUIRE(B >= 0, DSA_ERR_INVALID_ARG, "B must be >= 0");
  if (dsa_status s = check_mla_shape(H, D_qk, D_v, k)) return s;
  const int64_t cap = (int64_t)max_pages * page_size;
  if (dsa_status s = check_paged(kv_pool, n_pages, page_table, max_pages, ctx_len, page_size,
                                 cap > 0 ? cap : 1))
    return s;
  REQUIRE(scale > 0.f && scale < 1e30f, DSA_ERR_INVALID_ARG, "scale must be positive and finite");
  if (B == 0) return ok();
  REQUIRE_PTR(q); REQUIRE_PTR(idx); REQUIRE_PTR(out); REQUIRE_PTR(lse);
  REQUIRE_AL(q); REQUIRE_AL(idx); REQUIRE_AL(out); REQUIRE_AL(lse);
  dsa::PagedArgs pa{page_table, max_pages, page_size, n_pages};
  return run_mla(q, kv_pool, idx, B, H, k, scale, out, lse, ws, ws_bytes, true, 0, cap, ctx_len, &pa,
                 (hipStream_t)stream);
}

// ------------------------------------------------------------------ fused prefill
// Workspace of the fused prefill: the score tile, the selection (when the
// caller passes no idx), the FP8 scoring pass's bound inputs (per key, two
// globals, per row) and the attention's split partials.
namespace {
struct PrefillWs {
  size_t scores, idx, key_s, glob, row_fac, row_eps, row_flag, row_scale, mla, total;
};
PrefillWs prefill_ws(int64_t T, int64_t N, int32_t H, int32_t k) {
  PrefillWs w{};
  size_t o = 0;
  w.scores = o;
  o += round_up(sizeof(float) * (size_t)prefill_tile_rows(T, N) * score_ld(N));
  w.idx = o;
  o += round_up(sizeof(int32_t) * (size_t)T * k);
  w.key_s = o;
  o += round_up(sizeof(float) * (size_t)N);
  w.glob = o;
  o += round_up(2 * sizeof(uint32_t));
  w.row_fac = o;
  o += round_up(sizeof(float) * (size_t)T);
  w.row_eps = o;
  o += round_up(sizeof(float) * (size_t)T);
  w.row_flag = o;
  o += round_up(sizeof(int32_t) * (size_t)T);
  w.row_scale = o;
  o += round_up(sizeof(float) * (size_t)T);
  w.mla = o;
  o += mla_ws(T, H, k);
  w.total = o;
  return w;
}
}  // namespace

size_t dsa_forward_prefill_workspace_bytes(int64_t T, int64_t N, int32_t H, int32_t /*D_v*/, int32_t k) {
  if (T <= 0 || N <= 0 || k <= 0) return 0;
  return prefill_ws(T, N, H, k).total;
}

dsa_status dsa_forward_prefill_plan(int64_t T, int64_t N, int64_t* tile_rows, int64_t* score_ld_out) {
  REQUIRE(T >= 1 && N >= 1, DSA_ERR_INVALID_ARG, "T and N must be >= 1");
  REQUIRE_PTR(tile_rows);
  REQUIRE_PTR(score_ld_out);
  *tile_rows = prefill_tile_rows(T, N);
  *score_ld_out = score_ld(N);
  return ok();
}

dsa_status dsa_forward_prefill(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, const uint16_t* q,
                               const uint16_t* kv, int64_t T, int64_t N, int32_t H_I, int32_t d_I, int32_t H,
                               int32_t D_qk, int32_t D_v, int32_t k, int64_t q_pos0, float scale, int32_t* idx,
                               float* out, float* lse, void* ws, size_t ws_bytes, dsa_stream_t stream) {
  REQUIRE(T >= 0 && N >= 1, DSA_ERR_INVALID_ARG, "T must be >= 0 and N >= 1");
  REQUIRE(N <= kMaxCtx, DSA_ERR_UNSUPPORTED, "N must be <= %lld", (long long)kMaxCtx);
  REQUIRE(q_pos0 >= 0, DSA_ERR_INVALID_ARG, "q_pos0 must be >= 0");
  if (dsa_status s = check_indexer_shape(H_I, d_I)) return s;
  if (dsa_status s = check_mla_shape(H, D_qk, D_v, k)) return s;
  REQUIRE(scale > 0.f && scale < 1e30f, DSA_ERR_INVALID_ARG, "scale must be positive and finite");
  if (T == 0) return ok();
  REQUIRE_PTR(q_idx); REQUIRE_PTR(w); REQUIRE_PTR(k_idx); REQUIRE_PTR(q); REQUIRE_PTR(kv);
  REQUIRE_PTR(out); REQUIRE_PTR(lse);
  REQUIRE_AL(q_idx); REQUIRE_AL(w); REQUIRE_AL(k_idx); REQUIRE_AL(q); REQUIRE_AL(kv); REQUIRE_AL(out);
  REQUIRE_AL(lse);
  if (idx) REQUIRE_AL(idx);
  const size_t need = dsa_forward_prefill_workspace_bytes(T, N, H, D_v, k);
  REQUIRE(ws_bytes >= need, DSA_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes (got %zu)", need, ws_bytes);
  REQUIRE(ws != nullptr, DSA_ERR_INVALID_ARG, "ws is NULL");
  REQUIRE_AL(ws);
  hipStream_t st = (hipStream_t)stream;
  const int64_t rows = prefill_tile_rows(T, N);
  const int64_t ld = score_ld(N);
  const PrefillWs wl = prefill_ws(T, N, H, k);
  char* base = (char*)ws;
  float* scores = (float*)(base + wl.scores);
  int32_t* sel = idx ? idx : (int32_t*)(base + wl.idx);
  float* key_s = (float*)(base + wl.key_s);
  uint32_t* glob = (uint32_t*)(base + wl.glob);
  float* row_fac = (float*)(base + wl.row_fac);
  float* row_eps = (float*)(base + wl.row_eps);
  int32_t* row_flag = (int32_t*)(base + wl.row_flag);
  float* row_scale = (float*)(base + wl.row_scale);
  // Per row tile: the FP8 scoring pass, then the band top-k, which rescores
  // the keys near each row's threshold exactly (the selection is that of the
  // exact scores).  The bound inputs are computed once, with the first tile.
  for (int64_t r0 = 0; r0 < T; r0 += rows) {
    const int64_t tr = std::min(rows, T - r0);
    if (dsa_status s = hip_check(timed(DSA_KERNEL_INDEXER, st,
                                       [&] {
                                         if (r0 == 0) {
                                           hipError_t e = dsa::launch_fp8_bounds(q_idx, w, k_idx, T, N, H_I, key_s,
                                                                                 glob, row_fac, row_eps, row_flag,
                                                                                 row_scale, nullptr, st);
                                           if (e != hipSuccess) return e;
                                         }
                                         return dsa::launch_indexer_fp8_prefill(q_idx + r0 * H_I * 128, w + r0 * H_I,
                                                                                k_idx, tr, N, H_I, q_pos0 + r0,
                                                                                row_scale + r0, scores, ld, nullptr,
                                                                                st);
                                       }),
                                 "indexer launch"))
      return s;
    if (dsa_status s = hip_check(timed(DSA_KERNEL_TOPK, st,
                                       [&] {
                                         return dsa::launch_topk_band(scores, ld, tr, N, q_pos0 + r0, k, sel + r0 * k,
                                                                      q_idx + r0 * H_I * 128, w + r0 * H_I, k_idx, H_I,
                                                                      key_s, glob, row_fac + r0, row_eps + r0,
                                                                      row_flag + r0, row_scale + r0, nullptr, st);
                                       }),
                                 "top-k launch"))
      return s;
  }
  return run_mla(q, kv, sel, T, H, k, scale, out, lse, base + wl.mla, ws_bytes - wl.mla, false, N, N, nullptr,
                 nullptr, st);
}

// ------------------------------------------------------------------ dense warm-up loss
size_t dsa_dense_warmup_loss_workspace_bytes(int64_t T, int64_t N) {
  if (T <= 0 || N <= 0) return 0;
  return round_up(sizeof(float) * (size_t)prefill_tile_rows(T, N) * score_ld(N));
}

dsa_status dsa_dense_warmup_loss(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, const uint16_t* q,
                                 const uint16_t* kv, int64_t T, int64_t N, int32_t H_I, int32_t d_I, int32_t H,
                                 int32_t D_qk, int64_t q_pos0, float scale, float* kl, float* lse, void* ws,
                                 size_t ws_bytes, dsa_stream_t stream) {
  REQUIRE(T >= 0 && N >= 1, DSA_ERR_INVALID_ARG, "T must be >= 0 and N >= 1");
  REQUIRE(N <= kMaxCtx, DSA_ERR_UNSUPPORTED, "N must be <= %lld", (long long)kMaxCtx);
  REQUIRE(q_pos0 >= 0, DSA_ERR_INVALID_ARG, "q_pos0 must be >= 0");
  if (dsa_status s = check_indexer_shape(H_I, d_I)) return s;
  if (dsa_status s = check_mla_shape(H, D_qk, 512, 1)) return s;
  REQUIRE(scale > 0.f && scale < 1e30f, DSA_ERR_INVALID_ARG, "scale must be positive and finite");
  if (T == 0) return ok();
  REQUIRE_PTR(q_idx); REQUIRE_PTR(w); REQUIRE_PTR(k_idx); REQUIRE_PTR(q); REQUIRE_PTR(kv); REQUIRE_PTR(kl);
  REQUIRE_AL(q_idx); REQUIRE_AL(w); REQUIRE_AL(k_idx); REQUIRE_AL(q); REQUIRE_AL(kv);
  const size_t need = dsa_dense_warmup_loss_workspace_bytes(T, N);
  REQUIRE(ws_bytes >= need, DSA_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes (got %zu)", need, ws_bytes);
  REQUIRE(ws != nullptr, DSA_ERR_INVALID_ARG, "ws is NULL");
  REQUIRE_AL(ws);
  hipStream_t st = (hipStream_t)stream;
  const int64_t rows = prefill_tile_rows(T, N);
  const int64_t ld = score_ld(N);
  float* scores = (float*)ws;
  for (int64_t r0 = 0; r0 < T; r0 += rows) {
    const int64_t tr = std::min(rows, T - r0);
    if (dsa_status s = hip_check(timed(DSA_KERNEL_INDEXER, st,
                                       [&] {
                                         return dsa::launch_indexer_prefill(q_idx + r0 * H_I * 128, w + r0 * H_I,
                                                                            k_idx, tr, N, H_I, q_pos0 + r0, scores,
                                                                            ld, false, nullptr, st);
                                       }),
                                 "indexer launch"))
      return s;
    if (dsa_status s = hip_check(timed(DSA_KERNEL_DENSE_KL, st,
                                       [&] {
                                         return dsa::launch_indexer_dense_kl(q + r0 * H * 576, kv, N, scores, ld, tr,
                                                                             q_pos0 + r0, H, scale, kl + r0,
                                                                             lse ? lse + r0 * H : nullptr, st);
                                       }),
                                 "dense KL launch"))
      return s;
  }
  return ok();
}

// ------------------------------------------------------------------ ragged paged prefill
// Largest split-attention workspace of one sequence's chunk of at most
// total_q rows (only chunks of fewer than 256 rows are split).
static size_t chunk_mla_ws(int64_t total_q, int32_t H, int32_t k) {
  size_t m = 0;
  for (int64_t t = 1; t <= std::min<int64_t>(total_q, 256); ++t) m = std::max(m, mla_ws(t, H, k));
  return m;
}

// The fused prefill's layout over all chunks' rows: one score tile, the
// selection, the FP8 pass's bound inputs (keys of the longest context, the
// rows of every chunk), then the attention's split partials of one chunk.
static PrefillWs paged_prefill_ws(int64_t total_q, int64_t max_ctx, int32_t H, int32_t k) {
  PrefillWs w = prefill_ws(total_q, max_ctx, H, k);
  w.total = w.mla + chunk_mla_ws(total_q, H, k);
  return w;
}

size_t dsa_forward_prefill_paged_workspace_bytes(int64_t total_q, int64_t max_ctx, int32_t H, int32_t /*D_v*/,
                                                 int32_t k) {
  if (total_q <= 0 || max_ctx <= 0 || k <= 0) return 0;
  return paged_prefill_ws(total_q, max_ctx, H, k).total;
}

dsa_status dsa_forward_prefill_paged(const uint8_t* q_idx, const float* w, const uint8_t* k_pool,
                                     const uint16_t* q, const uint16_t* kv_pool, int64_t n_pages,
                                     const int32_t* page_table, int32_t max_pages, int32_t page_size,
                                     const int64_t* q_start, const int64_t* ctx_len, int64_t B, int32_t H_I,
                                     int32_t d_I, int32_t H, int32_t D_qk, int32_t D_v, int32_t k, float scale,
                                     int32_t* idx, float* out, float* lse, void* ws, size_t ws_bytes,
                                     dsa_stream_t stream) {
  REQUIRE(B >= 0, DSA_ERR_INVALID_ARG, "B must be >= 0");
  if (dsa_status s = check_indexer_shape(H_I, d_I)) return s;
  if (dsa_status s = check_mla_shape(H, D_qk, D_v, k)) return s;
  REQUIRE(scale > 0.f && scale < 1e30f, DSA_ERR_INVALID_ARG, "scale must be positive and finite");
  if (B == 0) return ok();
  REQUIRE_PTR(q_start);
  REQUIRE_PTR(ctx_len);
  REQUIRE(page_size == 64, DSA_ERR_UNSUPPORTED, "page_size must be 64 (got %d)", page_size);
  REQUIRE(n_pages >= 1 && max_pages >= 1, DSA_ERR_INVALID_ARG, "n_pages and max_pages must be >= 1");
  REQUIRE(q_start[0] == 0, DSA_ERR_INVALID_ARG, "q_start[0] must be 0 (got %lld)", (long long)q_start[0]);
  int64_t max_ctx = 1;
  for (int64_t b = 0; b < B; ++b) {
    const int64_t nq = q_start[b + 1] - q_start[b], n = ctx_len[b];
    REQUIRE(nq >= 0, DSA_ERR_INVALID_ARG, "q_start must be non-decreasing (sequence %lld)", (long long)b);
    REQUIRE(n >= nq && n <= (int64_t)max_pages * page_size && n <= kMaxCtx, DSA_ERR_INVALID_ARG,
            "ctx_len[%lld] = %lld must be in [new rows (%lld), min(max_pages*page_size, %lld)]", (long long)b,
            (long long)n, (long long)nq, (long long)kMaxCtx);
    max_ctx = std::max(max_ctx, n);
  }
  const int64_t total_q = q_start[B];
  if (total_q == 0) return ok();
  REQUIRE_PTR(q_idx); REQUIRE_PTR(w); REQUIRE_PTR(k_pool); REQUIRE_PTR(q); REQUIRE_PTR(kv_pool);
  REQUIRE_PTR(page_table); REQUIRE_PTR(out); REQUIRE_PTR(lse);
  REQUIRE_AL(q_idx); REQUIRE_AL(w); REQUIRE_AL(k_pool); REQUIRE_AL(q); REQUIRE_AL(kv_pool); REQUIRE_AL(out);
  REQUIRE_AL(lse);
  if (idx) REQUIRE_AL(idx);
  const size_t need = dsa_forward_prefill_paged_workspace_bytes(total_q, max_ctx, H, D_v, k);
  REQUIRE(ws_bytes >= need, DSA_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes (got %zu)", need, ws_bytes);
  REQUIRE(ws != nullptr, DSA_ERR_INVALID_ARG, "ws is NULL");
  REQUIRE_AL(ws);
  hipStream_t st = (hipStream_t)stream;
  const int64_t rows = prefill_tile_rows(total_q, max_ctx);
  const int64_t ld = score_ld(max_ctx);
  const PrefillWs wl = paged_prefill_ws(total_q, max_ctx, H, k);
  char* base = (char*)ws;
  float* scores = (float*)(base + wl.scores);
  int32_t* sel = idx ? idx : (int32_t*)(base + wl.idx);
  float* key_s = (float*)(base + wl.key_s);
  uint32_t* glob = (uint32_t*)(base + wl.glob);
  float* row_fac = (float*)(base + wl.row_fac);
  float* row_eps = (float*)(base + wl.row_eps);
  int32_t* row_flag = (int32_t*)(base + wl.row_flag);
  float* row_scale = (float*)(base + wl.row_scale);
  char* mla = base + wl.mla;
  // Per sequence: the bound inputs of its keys and chunk rows, then per row
  // tile the FP8 scoring pass and the band top-k, as in the contiguous fused
  // prefill, with the keys addressed through the sequence's page-table row.
  for (int64_t b = 0; b < B; ++b) {
    const int64_t q0 = q_start[b], nq = q_start[b + 1] - q0, n = ctx_len[b];
    if (nq == 0) continue;
    // the sequence's page-table row as row 0 of a one-sequence table
    const dsa::PagedArgs pa{page_table + b * (int64_t)max_pages, max_pages, page_size, n_pages};
    const int64_t pos0 = n - nq;  // position of the chunk's first query
    for (int64_t r0 = 0; r0 < nq; r0 += rows) {
      const int64_t tr = std::min(rows, nq - r0);
      const int64_t g = q0 + r0;  // first global query row of the tile
      if (dsa_status s = hip_check(
              timed(DSA_KERNEL_INDEXER, st,
                    [&] {
                      if (r0 == 0) {
                        hipError_t e = dsa::launch_fp8_bounds(q_idx + q0 * H_I * 128, w + q0 * H_I, k_pool, nq, n,
                                                              H_I, key_s, glob, row_fac + q0, row_eps + q0,
                                                              row_flag + q0, row_scale + q0, &pa, st);
                        if (e != hipSuccess) return e;
                      }
                      return dsa::launch_indexer_fp8_prefill(q_idx + g * H_I * 128, w + g * H_I, k_pool, tr, n, H_I,
                                                             pos0 + r0, row_scale + g, scores, ld, &pa, st);
                    }),
              "indexer launch"))
        return s;
      if (dsa_status s = hip_check(timed(DSA_KERNEL_TOPK, st,
                                         [&] {
                                           return dsa::launch_topk_band(scores, ld, tr, n, pos0 + r0, k, sel + g * k,
                                                                        q_idx + g * H_I * 128, w + g * H_I, k_pool,
                                                                        H_I, key_s, glob, row_fac + g, row_eps + g,
                                                                        row_flag + g, row_scale + g, &pa, st);
                                         }),
                                   "top-k launch"))
        return s;
    }
    if (dsa_status s = run_mla(q + q0 * H * 576, kv_pool, sel + q0 * k, nq, H, k, scale, out + q0 * H * 512,
                               lse + q0 * H, mla, ws_bytes - wl.mla, false, 0, n, nullptr, &pa, st))
      return s;
  }
  return ok();
}

// ------------------------------------------------------------------ fused decode
// scratch of the multi-workgroup top-k (few long rows), 0 when it is not used
static size_t decode_topk_ws(int64_t B, int64_t max_ctx) {
  return dsa::topk_rows_preferred(B, max_ctx) ? round_up(dsa::topk_rows_scratch_bytes(B, max_ctx)) : 0;
}

static size_t decode_ws(int64_t B, int64_t max_ctx, int32_t H, int32_t k) {
  if (B <= 0 || max_ctx <= 0 || k <= 0) return 0;
  return round_up(sizeof(float) * (size_t)B * score_ld(max_ctx)) + round_up(sizeof(int32_t) * (size_t)B * k) +
         decode_topk_ws(B, max_ctx) + mla_ws(B, H, k);
}

size_t dsa_forward_decode_workspace_bytes(int64_t B, int64_t N, int32_t H, int32_t /*D_v*/, int32_t k) {
  return decode_ws(B, N, H, k);
}

size_t dsa_forward_decode_paged_workspace_bytes(int64_t B, int64_t max_ctx, int32_t H, int32_t /*D_v*/,
                                                int32_t k) {
  return decode_ws(B, max_ctx, H, k);
}

static dsa_status run_decode(const uint8_t* q_idx, const float* w, const uint8_t* keys, const uint16_t* q,
                             const uint16_t* kv, const int32_t* ctx_len, int64_t B, int64_t max_ctx, int32_t H_I,
                             int32_t H, int32_t k, float scale, int32_t* idx, float* out, float* lse, void* ws,
                             size_t ws_bytes, int64_t stride, const dsa::PagedArgs* paged, hipStream_t st) {
  const size_t need = decode_ws(B, max_ctx, H, k);
  REQUIRE(ws_bytes >= need, DSA_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes (got %zu)", need, ws_bytes);
  REQUIRE(ws != nullptr, DSA_ERR_INVALID_ARG, "ws is NULL");
  REQUIRE_AL(ws);
  const int64_t ld = score_ld(max_ctx);
  char* p = (char*)ws;
  float* scores = (float*)p;
  p += round_up(sizeof(float) * (size_t)B * ld);
  int32_t* idx_ws = (int32_t*)p;
  p += round_up(sizeof(int32_t) * (size_t)B * k);
  int32_t* sel = idx ? idx : idx_ws;
  void* topk_scratch = p;
  const size_t topk_bytes = decode_topk_ws(B, max_ctx);
  p += topk_bytes;
  if (dsa_status s = hip_check(timed(DSA_KERNEL_INDEXER, st,
                                     [&] {
                                       return dsa::launch_indexer_decode(q_idx, w, keys, stride, paged, ctx_len, B,
                                                                         max_ctx, H_I, scores, ld, st);
                                     }),
                               "decode indexer launch"))
    return s;
  const hipError_t te = timed(DSA_KERNEL_TOPK, st, [&] {
    return topk_bytes ? dsa::launch_topk_rows(scores, ld, B, max_ctx, ctx_len, k, sel, topk_scratch, st)
                      : dsa::launch_topk(scores, ld, B, max_ctx, 0, ctx_len, k, sel, st);
  });
  if (dsa_status s = hip_check(te, "top-k launch")) return s;
  const int64_t seq_len = paged ? (int64_t)paged->max_pages * paged->page_size : stride;
  return run_mla(q, kv, sel, B, H, k, scale, out, lse, p, ws_bytes - (size_t)(p - (char*)ws), true, stride,
                 seq_len, ctx_len, paged, st);
}

dsa_status dsa_forward_decode(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, const uint16_t* q,
                              const uint16_t* kv, const int32_t* ctx_len, int64_t B, int64_t N, int32_t H_I,
                              int32_t d_I, int32_t H, int32_t D_qk, int32_t D_v, int32_t k, float scale,
                              int32_t* idx, float* out, float* lse, void* ws, size_t ws_bytes,
                              dsa_stream_t stream) {
  REQUIRE(B >= 0 && N >= 1, DSA_ERR_INVALID_ARG, "B must be >= 0 and N >= 1");
  REQUIRE(N <= kMaxCtx, DSA_ERR_UNSUPPORTED, "N must be <= %lld", (long long)kMaxCtx);
  if (dsa_status s = check_indexer_shape(H_I, d_I)) return s;
  if (dsa_status s = check_mla_shape(H, D_qk, D_v, k)) return s;
  REQUIRE(scale > 0.f && scale < 1e30f, DSA_ERR_INVALID_ARG, "scale must be positive and finite");
  if (B == 0) return ok();
  REQUIRE_PTR(q_idx); REQUIRE_PTR(w); REQUIRE_PTR(k_idx); REQUIRE_PTR(q); REQUIRE_PTR(kv);
  REQUIRE_PTR(ctx_len); REQUIRE_PTR(out); REQUIRE_PTR(lse);
  REQUIRE_AL(q_idx); REQUIRE_AL(w); REQUIRE_AL(k_idx); REQUIRE_AL(q); REQUIRE_AL(kv); REQUIRE_AL(out);
  REQUIRE_AL(lse);
  if (idx) REQUIRE_AL(idx);
  return run_decode(q_idx, w, k_idx, q, kv, ctx_len, B, N, H_I, H, k, scale, idx, out, lse, ws, ws_bytes, N,
                    nullptr, (hipStream_t)stream);
}

// Validation shared by the two paged decode entry points.
static dsa_status check_decode_paged(const uint8_t* q_idx, const float* w, const uint8_t* k_pool, const uint16_t* q,
                                     const uint16_t* kv_pool, int64_t n_pages, const int32_t* page_table,
                                     int32_t max_pages, const int32_t* ctx_len, int32_t page_size, int64_t B,
                                     int64_t max_ctx, int32_t H_I, int32_t d_I, int32_t H, int32_t D_qk, int32_t D_v,
                                     int32_t k, float scale, int32_t* idx, float* out, float* lse) {
  REQUIRE(B >= 0, DSA_ERR_INVALID_ARG, "B must be >= 0");
  REQUIRE(max_ctx <= kMaxCtx, DSA_ERR_UNSUPPORTED, "max_ctx must be <= %lld", (long long)kMaxCtx);
  if (dsa_status s = check_indexer_shape(H_I, d_I)) return s;
  if (dsa_status s = check_mla_shape(H, D_qk, D_v, k)) return s;
  if (dsa_status s = check_paged(k_pool, n_pages, page_table, max_pages, ctx_len, page_size, max_ctx)) return s;
  REQUIRE_PTR(kv_pool);
  REQUIRE_AL(kv_pool);
  REQUIRE(scale > 0.f && scale < 1e30f, DSA_ERR_INVALID_ARG, "scale must be positive and finite");
  if (B == 0) return DSA_OK;
  REQUIRE_PTR(q_idx); REQUIRE_PTR(w); REQUIRE_PTR(q); REQUIRE_PTR(out); REQUIRE_PTR(lse);
  REQUIRE_AL(q_idx); REQUIRE_AL(w); REQUIRE_AL(q); REQUIRE_AL(out); REQUIRE_AL(lse);
  if (idx) REQUIRE_AL(idx);
  return DSA_OK;
}

dsa_status dsa_forward_decode_paged(const uint8_t* q_idx, const float* w, const uint8_t* k_pool, const uint16_t* q,
                                    const uint16_t* kv_pool, int64_t n_pages, const int32_t* page_table,
                                    int32_t max_pages, const int32_t* ctx_len, int32_t page_size, int64_t B,
                                    int64_t max_ctx, int32_t H_I, int32_t d_I, int32_t H, int32_t D_qk, int32_t D_v,
                                    int32_t k, float scale, int32_t* idx, float* out, float* lse, void* ws,
                                    size_t ws_bytes, dsa_stream_t stream) {
  if (dsa_status s = check_decode_paged(q_idx, w, k_pool, q, kv_pool, n_pages, page_table, max_pages, ctx_len,
                                        page_size, B, max_ctx, H_I, d_I, H, D_qk, D_v, k, scale, idx, out, lse))
    return s;
  if (B == 0) return ok();
  dsa::PagedArgs pa{page_table, max_pages, page_size, n_pages};
  return run_decode(q_idx, w, k_pool, q, kv_pool, ctx_len, B, max_ctx, H_I, H, k, scale, idx, out, lse, ws,
                    ws_bytes, 0, &pa, (hipStream_t)stream);
}

}  // extern "C"

// ------------------------------------------------------------------ allocation-free paged decode
// Scratch of dsa_forward_decode_paged_noalloc: one array per GPU, part of the
// library's code object (so held by each GPU the library runs on until the
// process ends) and shared by every call on that GPU.  In host code the
// array's name is only a stand-in; kernels get its device address, looked up
// once per device.
constexpr size_t kNoallocScratchBytes = (size_t)96 << 20;
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

namespace {
hipError_t scratch_ptr(void** out) {
  static std::mutex m;
  static std::map<int, void*> by_dev;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(m);
  const auto it = by_dev.find(dev);
  if (it != by_dev.end()) {
    *out = it->second;
    return hipSuccess;
  }
  void* ptr = nullptr;
  e = hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  by_dev[dev] = ptr;
  *out = ptr;
  return hipSuccess;
}
}  // namespace

extern "C" dsa_status dsa_forward_decode_paged_noalloc(
    const uint8_t* q_idx, const float* w, const uint8_t* k_pool, const uint16_t* q, const uint16_t* kv_pool,
    int64_t n_pages, const int32_t* page_table, int32_t max_pages, const int32_t* ctx_len, int32_t page_size,
    int64_t B, int64_t max_ctx, int32_t H_I, int32_t d_I, int32_t H, int32_t D_qk, int32_t D_v, int32_t k,
    float scale, int32_t* idx, float* out, float* lse, dsa_stream_t stream) {
  if (dsa_status s = check_decode_paged(q_idx, w, k_pool, q, kv_pool, n_pages, page_table, max_pages, ctx_len,
                                        page_size, B, max_ctx, H_I, d_I, H, D_qk, D_v, k, scale, idx, out, lse))
    return s;
  if (B == 0) return ok();
  // the kernels write every scratch byte they later read (score rows, the
  // selection, the top-k candidate lists with their counters, the split
  // partials), so nothing has to be cleared between calls
  const size_t need = decode_ws(B, max_ctx, H, k);
  REQUIRE(need <= kNoallocScratchBytes, DSA_ERR_UNSUPPORTED,
          "this decode needs %zu bytes of scratch, above the %zu-byte maximum of the allocation-free call", need,
          kNoallocScratchBytes);
  void* ptr = nullptr;
  if (dsa_status s = hip_check(scratch_ptr(&ptr), "scratch address")) return s;
  dsa::PagedArgs pa{page_table, max_pages, page_size, n_pages};
  return run_decode(q_idx, w, k_pool, q, kv_pool, ctx_len, B, max_ctx, H_I, H, k, scale, idx, out, lse, ptr,
                    kNoallocScratchBytes, 0, &pa, (hipStream_t)stream);
}
