// Internal kernel launchers (host side).  Shapes are validated by the C-ABI
// layer before any of these is called; each returns the launch status.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

struct PagedArgs {
  const int32_t* page_table;
  int32_t max_pages;
  int32_t page_size;
  int64_t n_pages;
};

// Lightning-indexer scores for T query rows of one sequence (rows at
// positions q_pos0 + t) over keys 0..N-1.  fill_masked: also write -inf to
// the non-candidate keys s < N; otherwise only candidates are written.
// Keys are rows 0..N-1 of k_idx, or (paged != nullptr) pool rows through
// page-table row 0 of `paged`.
hipError_t launch_indexer_prefill(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, int64_t T,
                                  int64_t N, int32_t H_I, int64_t q_pos0, float* scores, int64_t ld,
                                  bool fill_masked, const PagedArgs* paged, hipStream_t st);

// Fused prefill's FP8 scoring pass (indexer.hip): error-bound inputs, then the
// approximate scores of the causal pairs (candidates only, f16 I~ * 2^-s in
// the first half of each fp32 tile row).  key_s [N], glob [2] (cleared here:
// largest key_s, largest |k_I|, as float bits), row_fac / row_eps / row_flag /
// row_scale (2^s) [T].  Keys are rows 0..N-1 of k_idx, or (paged != nullptr)
// pool rows through page-table row 0 of `paged`.
hipError_t launch_fp8_bounds(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, int64_t T, int64_t N,
                             int32_t H_I, float* key_s, uint32_t* glob, float* row_fac, float* row_eps,
                             int32_t* row_flag, float* row_scale, const PagedArgs* paged, hipStream_t st);
hipError_t launch_indexer_fp8_prefill(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, int64_t T,
                                      int64_t N, int32_t H_I, int64_t q_pos0, const float* row_scale, float* scores,
                                      int64_t ld, const PagedArgs* paged, hipStream_t st);

// Indexer scores for B decode queries; keys of sequence b are either rows
// b*stride + s of k_idx (paged == nullptr) or pool rows via the page table.
// Writes scores[b*ld + s] for s < max_ctx (-inf past ctx_len[b]).
hipError_t launch_indexer_decode(const uint8_t* q_idx, const float* w, const uint8_t* keys, int64_t stride,
                                 const PagedArgs* paged, const int32_t* ctx_len, int64_t B, int64_t max_ctx,
                                 int32_t H_I, float* scores, int64_t ld, hipStream_t st);

// Top-k per row: n_t = min(n_valid ? n_valid[t] : q_pos0 + t + 1, N).
hipError_t launch_topk(const float* scores, int64_t ld, int64_t T, int64_t N, int64_t q_pos0,
                       const int32_t* n_valid, int32_t k, int32_t* idx, hipStream_t st);

// The fused prefill's top-k over the FP8 scoring pass's approximate scores
// (topk.hip): the selection of the exact scores, from the band of keys near
// each row's threshold rescored exactly.  scores (the tile) is also written:
// rows that take the exact route are rescored in place.  q_idx, w, row_fac,
// row_eps, row_flag and row_scale are the tile's rows; key_s and glob as
// filled by launch_fp8_bounds; keys addressed as there.
hipError_t launch_topk_band(float* scores, int64_t ld, int64_t T, int64_t N, int64_t q_pos0, int32_t k,
                            int32_t* idx, const uint8_t* q_idx, const float* w, const uint8_t* k_idx, int32_t H_I,
                            const float* key_s, const uint32_t* glob, const float* row_fac, const float* row_eps,
                            const int32_t* row_flag, const float* row_scale, const PagedArgs* paged,
                            hipStream_t st);

// Top-k for a few long rows (decode): the full-row passes run over
// 4096-key chunks in parallel; needs topk_rows_scratch_bytes(T, N) of device
// scratch and n_valid.  Same selection as launch_topk.
bool topk_rows_preferred(int64_t T, int64_t N);
size_t topk_rows_scratch_bytes(int64_t T, int64_t N);
hipError_t launch_topk_rows(const float* scores, int64_t ld, int64_t T, int64_t N, const int32_t* n_valid,
                            int32_t k, int32_t* idx, void* scratch, hipStream_t st);

// Sparse MLA-MQA attention.  Query t reads latent rows of sequence
// (seq_per_query ? t : 0) through the given addressing: contiguous rows
// (kv + row*D_qk with row = b*stride + s, s < seq_len) or paged.
// n_split > 1 splits each query's k entries over n_split workgroups and
// merges the partials (part_o [T, n_split, H, D_v] f16 scaled by 1/part_scale,
// part_lse and part_scale [T, n_split, H] fp32).
struct MlaArgs {
  const uint16_t* q;
  const uint16_t* kv;
  const int32_t* idx;
  int64_t T;
  int32_t H;
  int32_t k;
  float scale;
  float* out;
  float* lse;
  // addressing
  bool seq_per_query;
  int64_t stride;            // contiguous: row = b*stride + s
  int64_t seq_len;           // contiguous: valid s < seq_len
  const int32_t* ctx_len;    // optional per-sequence valid length (decode)
  const PagedArgs* paged;    // non-null: paged addressing
  // split-key partials
  int32_t n_split;
  uint16_t* part_o;
  float* part_lse;
  float* part_scale;
};
hipError_t launch_sparse_mla(const MlaArgs& a, hipStream_t st);

// Indexer KL loss per query over its selected entries (one workgroup per
// query; lse from the attention of the same q, kv and idx).
hipError_t launch_indexer_kl(const uint16_t* q, const uint16_t* kv, int64_t N, const int32_t* idx,
                             const float* lse, const float* scores, int64_t ld, int64_t T, int32_t H, int32_t k,
                             float scale, float* kl, hipStream_t st);

// Dense warm-up indexer loss per query (one workgroup per query): KL over
// all keys s < min(q_pos0 + t + 1, N) of the head-averaged dense attention and
// the softmax of score row t; optionally the dense lse [T, H].
hipError_t launch_indexer_dense_kl(const uint16_t* q, const uint16_t* kv, int64_t N, const float* scores, int64_t ld,
                                   int64_t T, int64_t q_pos0, int32_t H, float scale, float* kl, float* lse,
                                   hipStream_t st);

// Sparse MLA-MQA backward over one tile of T queries.  Stage 0 (dq kernel):
// dq, and P / dS of every entry into pbuf / dsbuf ([T, kp, Hs] bf16, kp = k
// rounded up to 32, Hs = mla_bwd_slot_heads(H)); stage 1 (dkv kernel): each entry's contribution
// to its cache row into addend ([T, k, 576] bf16); stage 2: groups the
// entries by cache row (row_count [N], row_offsets [N+1], row_list [T*k]
// int32) and adds each row's sum to dkv (dkv cleared beforehand).
struct MlaBwdArgs {
  const uint16_t* q;
  const uint16_t* kv;
  const int32_t* idx;
  const float* out;
  const float* lse;
  const uint16_t* dout;
  int64_t T;
  int64_t N;
  int32_t H;
  int32_t k;
  float scale;
  float* dq;
  uint16_t* pbuf;
  uint16_t* dsbuf;
  uint16_t* addend;
  int32_t* row_count;
  int32_t* row_offsets;
  int32_t* row_list;
  float* dkv;
};
int32_t mla_bwd_padded_heads(int32_t H);
int32_t mla_bwd_slot_heads(int32_t H);
hipError_t launch_sparse_mla_bwd(const MlaBwdArgs& a, int stage, hipStream_t st);
hipError_t launch_zero_f32(float* x, int64_t n, hipStream_t st);

// Number of key splits used for T queries of H heads with k entries each.
int32_t sparse_mla_splits(int64_t T, int32_t H, int32_t k);

}  // namespace dsa
