/*
 * CPU oracle for DeepSeek Sparse Attention (DSA) forward: lightning-indexer
 * scores, per-query top-k selection and sparse MLA attention in MQA mode.
 *
 * TEST INFRASTRUCTURE ONLY.  Plain, slow, single-threaded C in double
 * precision, written from the method's definitions so that a reader can
 * check each function against the pages by eye.  It shares no code with the
 * GPU library; only the test suite, the smoke check and the bench's
 * CPU-baseline leg may call it.
 *
 * Sources (page titles; sections and equations on them):
 *  [P1] "DeepSeek-V3.2" release thread with a walk-through of the technical
 *       report (freezhihu.org question 1978819912970555965):
 *       §2.1.1 "Lightning Indexer" (index-score equation and its symbols),
 *       §2.1.2 "Fine-grained token selection" (top-k and the attention
 *       equation u_t = Attn(h_t, {c_s | I_{t,s} in Top-k(I_{t,:})})),
 *       §2.2 "DSA instantiated in MLA" (MQA mode: each latent KV entry is
 *       shared by all query heads of a token).
 *       §2.3.2 "Sparse training stage" (the indexer's KL loss over the
 *       selected set S_t, with the target built as in §2.3.1: attention
 *       scores summed over heads, L1-normalised along the sequence).
 *  [P2] "DeepSeek v3.2" analysis article (2048ai.net), §1.2: indexer keys are
 *       one 128-dim vector per token and run in FP8.
 *
 * Readings where the pages are silent (all stated in the design notes):
 *  - a query at position p has candidates s = 0..p (itself included);
 *  - equal scores are broken toward the lower token index; the selected set
 *    is returned in ascending token order, padded with -1 when fewer than k
 *    candidates exist (then all candidates are taken);
 *  - FP8 is OCP E4M3FN with unit scale; the attention is softmax(scale*q.k)
 *    over the first D_qk latent dims, values are the first D_v dims, natural
 *    exp/log, no bias or sink.
 *
 * Parity status: every function below is pinned by tests against values fixed
 * by hand or by independent routines (see tests/test_oracle_pins.py).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------ storage formats */

/* OCP FP8 E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no
 * infinities; S.1111.111 is NaN; largest finite value 448. */
double oracle_e4m3_to_double(uint8_t b) {
  int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);          /* subnormal: m * 2^-6 * 2^-3 */
  else
    v = ldexp((double)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */
  return s ? -v : v;
}

/* bfloat16: the upper half of an IEEE binary32. */
double oracle_bf16_to_double(uint16_t u) {
  uint32_t bits = (uint32_t)u << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* ------------------------------------------------------------ lightning indexer */

/* [P1] §2.1.1, index-score equation:
 *   I_{t,s} = sum_{j=1..H^I} w^I_{t,j} * ReLU(q^I_{t,j} . k^I_s)
 * for the one query row t given by q_row [H_I][d] and w_row [H_I], over the
 * n key rows k [n][d] (token s = 0..n-1).  out[s] = I_{t,s}.
 * Every FP8 product is exact in double and a d = 128 term sum of them needs
 * fewer than 53 significant bits, so the dot products are exact. */
void oracle_indexer_row(const uint8_t* q_row, const float* w_row, const uint8_t* k, int64_t n,
                        int32_t H_I, int32_t d, double* out) {
  double lut[256];
  for (int b = 0; b < 256; ++b) lut[b] = oracle_e4m3_to_double((uint8_t)b);
  double* qd = (double*)malloc(sizeof(double) * (size_t)H_I * (size_t)d);
  double* kd = (double*)malloc(sizeof(double) * (size_t)d);
  for (int64_t i = 0; i < (int64_t)H_I * d; ++i) qd[i] = lut[q_row[i]];
  for (int64_t s = 0; s < n; ++s) {
    for (int i = 0; i < d; ++i) kd[i] = lut[k[s * d + i]];
    double score = 0.0;
    for (int j = 0; j < H_I; ++j) {
      double dot = 0.0;
      for (int i = 0; i < d; ++i) dot += qd[(int64_t)j * d + i] * kd[i];
      double relu = dot > 0.0 ? dot : 0.0;
      score += (double)w_row[j] * relu;
    }
    out[s] = score;
  }
  free(kd);
  free(qd);
}

/* ------------------------------------------------------------ top-k selection */

typedef struct {
  double v;
  int64_t s;
} scored_t;

/* Larger score first; equal scores (+0 and -0 compare equal) by lower index. */
static int by_score_desc(const void* a, const void* b) {
  const scored_t* x = (const scored_t*)a;
  const scored_t* y = (const scored_t*)b;
  if (x->v > y->v) return -1;
  if (x->v < y->v) return 1;
  return (x->s < y->s) ? -1 : (x->s > y->s);
}

static int by_index_asc(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

/* [P1] §2.1.2: for query t keep the k candidates with the highest index
 * scores, S_t = {s | I_{t,s} in Top-k(I_{t,:})}.  Candidates are s = 0..n-1.
 * Writes out[0..k-1]: the selected token indices in ascending order, then -1
 * padding.  Returns the number selected, min(k, n). */
int32_t oracle_topk_row(const double* scores, int64_t n, int32_t k, int32_t* out) {
  int32_t m = (n < (int64_t)k) ? (int32_t)n : k;
  if (n <= (int64_t)k) {
    for (int32_t i = 0; i < m; ++i) out[i] = i;
  } else {
    scored_t* all = (scored_t*)malloc(sizeof(scored_t) * (size_t)n);
    for (int64_t s = 0; s < n; ++s) {
      all[s].v = scores[s];
      all[s].s = s;
    }
    qsort(all, (size_t)n, sizeof(scored_t), by_score_desc);
    for (int32_t i = 0; i < m; ++i) out[i] = (int32_t)all[i].s;
    free(all);
    qsort(out, (size_t)m, sizeof(int32_t), by_index_asc);
  }
  for (int32_t i = m; i < k; ++i) out[i] = -1;
  return m;
}

/* ------------------------------------------------------------ sparse attention */

/* [P1] §2.1.2 attention equation with §2.2's MQA mode: every head h of the
 * query attends over the same m selected latent rows kv_rows [m][D_qk]:
 *   z_s   = scale * sum_{c<D_qk} q[h,c] * kv[s,c]
 *   o[h]  = sum_s softmax(z)_s * kv[s, 0:D_v]
 *   lse[h]= ln sum_s exp(z_s)
 * q is [H][D_qk] bf16 bits.  With m == 0 the output is 0 and lse is -inf. */
void oracle_sparse_mla_row(const uint16_t* q, const uint16_t* kv_rows, int64_t m, int32_t H, int32_t D_qk,
                           int32_t D_v, double scale, double* out, double* lse) {
  if (m == 0) {
    for (int64_t i = 0; i < (int64_t)H * D_v; ++i) out[i] = 0.0;
    for (int h = 0; h < H; ++h) lse[h] = -INFINITY;
    return;
  }
  double* kvd = (double*)malloc(sizeof(double) * (size_t)m * (size_t)D_qk);
  double* z = (double*)malloc(sizeof(double) * (size_t)m);
  double* qd = (double*)malloc(sizeof(double) * (size_t)D_qk);
  for (int64_t i = 0; i < m * D_qk; ++i) kvd[i] = oracle_bf16_to_double(kv_rows[i]);
  for (int h = 0; h < H; ++h) {
    for (int c = 0; c < D_qk; ++c) qd[c] = oracle_bf16_to_double(q[(int64_t)h * D_qk + c]);
    double zmax = -INFINITY;
    for (int64_t s = 0; s < m; ++s) {
      double dot = 0.0;
      for (int c = 0; c < D_qk; ++c) dot += qd[c] * kvd[s * D_qk + c];
      z[s] = scale * dot;
      if (z[s] > zmax) zmax = z[s];
    }
    double denom = 0.0;
    for (int64_t s = 0; s < m; ++s) denom += exp(z[s] - zmax);
    double* o = out + (int64_t)h * D_v;
    for (int c = 0; c < D_v; ++c) o[c] = 0.0;
    for (int64_t s = 0; s < m; ++s) {
      double p = exp(z[s] - zmax) / denom;
      for (int c = 0; c < D_v; ++c) o[c] += p * kvd[s * D_qk + c];
    }
    lse[h] = zmax + log(denom);
  }
  free(qd);
  free(z);
  free(kvd);
}

/* Dense causal MLA-MQA for one query, used only to check the sparse routine:
 * a full row of N logits with positions s >= n masked to -inf, then an
 * ordinary softmax over the row (no index list involved). */
void oracle_dense_mla_row(const uint16_t* q, const uint16_t* kv, int64_t N, int64_t n, int32_t H,
                          int32_t D_qk, int32_t D_v, double scale, double* out, double* lse) {
  double* logits = (double*)malloc(sizeof(double) * (size_t)N);
  for (int h = 0; h < H; ++h) {
    for (int64_t s = 0; s < N; ++s) {
      if (s >= n) {
        logits[s] = -INFINITY;
        continue;
      }
      double dot = 0.0;
      for (int c = 0; c < D_qk; ++c)
        dot += oracle_bf16_to_double(q[(int64_t)h * D_qk + c]) * oracle_bf16_to_double(kv[s * D_qk + c]);
      logits[s] = dot * scale;
    }
    double mx = -INFINITY;
    for (int64_t s = 0; s < N; ++s) mx = logits[s] > mx ? logits[s] : mx;
    double sum = 0.0;
    for (int64_t s = 0; s < N; ++s) sum += (logits[s] == -INFINITY) ? 0.0 : exp(logits[s] - mx);
    for (int c = 0; c < D_v; ++c) {
      double acc = 0.0;
      for (int64_t s = 0; s < n; ++s) acc += exp(logits[s] - mx) * oracle_bf16_to_double(kv[s * D_qk + c]);
      out[(int64_t)h * D_v + c] = acc / sum;
    }
    lse[h] = mx + log(sum);
  }
  free(logits);
}

/* Indexer KL loss of one query over its selected set ([P1] §2.3.2, with the
 * target of §2.3.1 restricted to S_t).  The m selected latent rows are
 * kv_rows[m][D_qk] (bf16 bits); iscore[s] is the indexer score I_{t,s} of
 * selected entry s.
 *   P_h(s) = softmax over S_t of scale * q[h] . kv[s]   (head h's attention)
 *   p(s)   = sum_h P_h(s) / sum_{s'} sum_h P_h(s')      (heads summed, L1-normalised)
 *   r(s)   = softmax over S_t of I_{t,s}
 *   KL     = sum_s p(s) * (ln p(s) - ln r(s)),  with 0 * ln 0 = 0.
 * m == 0 gives 0. */
double oracle_indexer_kl_row(const uint16_t* q, const uint16_t* kv_rows, int64_t m, int32_t H, int32_t D_qk,
                             double scale, const double* iscore) {
  if (m == 0) return 0.0;
  double* kvd = (double*)malloc(sizeof(double) * (size_t)m * (size_t)D_qk);
  double* z = (double*)malloc(sizeof(double) * (size_t)m);
  double* agg = (double*)calloc((size_t)m, sizeof(double));
  double* qd = (double*)malloc(sizeof(double) * (size_t)D_qk);
  for (int64_t i = 0; i < m * D_qk; ++i) kvd[i] = oracle_bf16_to_double(kv_rows[i]);
  for (int h = 0; h < H; ++h) {
    for (int c = 0; c < D_qk; ++c) qd[c] = oracle_bf16_to_double(q[(int64_t)h * D_qk + c]);
    double zmax = -INFINITY;
    for (int64_t s = 0; s < m; ++s) {
      double dot = 0.0;
      for (int c = 0; c < D_qk; ++c) dot += qd[c] * kvd[s * D_qk + c];
      z[s] = scale * dot;
      if (z[s] > zmax) zmax = z[s];
    }
    double denom = 0.0;
    for (int64_t s = 0; s < m; ++s) denom += exp(z[s] - zmax);
    for (int64_t s = 0; s < m; ++s) agg[s] += exp(z[s] - zmax) / denom;
  }
  double total = 0.0;
  for (int64_t s = 0; s < m; ++s) total += agg[s];
  double imax = -INFINITY;
  for (int64_t s = 0; s < m; ++s) imax = iscore[s] > imax ? iscore[s] : imax;
  double isum = 0.0;
  for (int64_t s = 0; s < m; ++s) isum += exp(iscore[s] - imax);
  const double log_norm = imax + log(isum); /* ln sum_s e^{I_s} */
  double kl = 0.0;
  for (int64_t s = 0; s < m; ++s) {
    const double ps = agg[s] / total;
    if (ps > 0.0) kl += ps * (log(ps) - (iscore[s] - log_norm));
  }
  free(qd);
  free(agg);
  free(z);
  free(kvd);
  return kl;
}

/* Gradient of the sparse MLA-MQA attention of one query (the attention
 * equation of [P1] §2.1.2 in the MQA form of §2.2), as the sparse training
 * stage of [P1] §2.3.2 needs it to train the main model through the sparse
 * attention.  For a loss L with upstream gradient dO[h][D_v] = dL/du_t[h]:
 *   z_h(s)  = scale * q[h] . kv[s]            (first D_qk dims)
 *   P_h(s)  = softmax over the m entries of z_h
 *   dP_h(s) = dO[h] . kv[s][0..D_v)           (dL/dP_h(s), since u = sum_s P V)
 *   dZ_h(s) = P_h(s) * (dP_h(s) - sum_s' P_h(s') dP_h(s'))   (softmax Jacobian)
 *   dq[h]   = scale * sum_s dZ_h(s) kv[s]
 *   dkv[s]  = scale * sum_h dZ_h(s) q[h]  +  sum_h P_h(s) dO[h]  (the second
 *             term on the first D_v dims only: the values are those dims)
 * dq is [H][D_qk]; dkv_rows is [m][D_qk], one row per gathered entry (the
 * caller adds them into the cache rows the entries came from).
 * mag_dq / mag_dkv (optional, same shapes) receive the same sums taken over
 * absolute values, with |dP - D| replaced by A(s) + sum_s' P(s') A(s'), where
 * A(s) = sum_c |dO[h][c]| |kv[s][c]|: the scale against which rounding of the
 * terms is measured (P, dP and D each carry a relative error of at most a few
 * units of the format they were formed in, and A bounds |dP| and D's
 * sensitivity to P).
 * m == 0 gives zeros. */
void oracle_sparse_mla_bwd_row(const uint16_t* q, const uint16_t* kv_rows, const uint16_t* dO, int64_t m,
                               int32_t H, int32_t D_qk, int32_t D_v, double scale, double* dq, double* dkv_rows,
                               double* mag_dq, double* mag_dkv) {
  for (int64_t i = 0; i < (int64_t)H * D_qk; ++i) {
    dq[i] = 0.0;
    if (mag_dq) mag_dq[i] = 0.0;
  }
  for (int64_t i = 0; i < m * D_qk; ++i) {
    dkv_rows[i] = 0.0;
    if (mag_dkv) mag_dkv[i] = 0.0;
  }
  if (m == 0) return;
  double* kvd = (double*)malloc(sizeof(double) * (size_t)m * (size_t)D_qk);
  double* z = (double*)malloc(sizeof(double) * (size_t)m);
  double* dp = (double*)malloc(sizeof(double) * (size_t)m);
  double* adp = (double*)malloc(sizeof(double) * (size_t)m);
  double* qd = (double*)malloc(sizeof(double) * (size_t)D_qk);
  double* gd = (double*)malloc(sizeof(double) * (size_t)D_v);
  for (int64_t i = 0; i < m * D_qk; ++i) kvd[i] = oracle_bf16_to_double(kv_rows[i]);
  for (int h = 0; h < H; ++h) {
    for (int c = 0; c < D_qk; ++c) qd[c] = oracle_bf16_to_double(q[(int64_t)h * D_qk + c]);
    for (int c = 0; c < D_v; ++c) gd[c] = oracle_bf16_to_double(dO[(int64_t)h * D_v + c]);
    double zmax = -INFINITY;
    for (int64_t s = 0; s < m; ++s) {
      double dot = 0.0;
      for (int c = 0; c < D_qk; ++c) dot += qd[c] * kvd[s * D_qk + c];
      z[s] = scale * dot;
      if (z[s] > zmax) zmax = z[s];
    }
    double denom = 0.0;
    for (int64_t s = 0; s < m; ++s) denom += exp(z[s] - zmax);
    double dsum = 0.0, dmag = 0.0; /* sum_s P(s) dP(s), sum_s P(s) A(s) */
    for (int64_t s = 0; s < m; ++s) {
      z[s] = exp(z[s] - zmax) / denom; /* z now holds P */
      double dot = 0.0, adot = 0.0;
      for (int c = 0; c < D_v; ++c) {
        dot += gd[c] * kvd[s * D_qk + c];
        adot += fabs(gd[c]) * fabs(kvd[s * D_qk + c]);
      }
      dp[s] = dot;
      adp[s] = adot;
      dsum += z[s] * dot;
      dmag += z[s] * adot;
    }
    for (int64_t s = 0; s < m; ++s) {
      const double p = z[s];
      const double dz = p * (dp[s] - dsum);
      const double dz_mag = p * (adp[s] + dmag);
      for (int c = 0; c < D_qk; ++c) {
        dq[(int64_t)h * D_qk + c] += scale * dz * kvd[s * D_qk + c];
        dkv_rows[s * D_qk + c] += scale * dz * qd[c];
        if (mag_dq) mag_dq[(int64_t)h * D_qk + c] += scale * dz_mag * fabs(kvd[s * D_qk + c]);
        if (mag_dkv) mag_dkv[s * D_qk + c] += scale * dz_mag * fabs(qd[c]);
      }
      for (int c = 0; c < D_v; ++c) {
        dkv_rows[s * D_qk + c] += p * gd[c];
        if (mag_dkv) mag_dkv[s * D_qk + c] += p * fabs(gd[c]);
      }
    }
  }
  free(gd);
  free(qd);
  free(adp);
  free(dp);
  free(z);
  free(kvd);
}
