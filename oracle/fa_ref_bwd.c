/*
 * CPU oracle for the exact attention backward — TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the package smoke check and the benchmark's CPU-baseline leg may load this
 * library. The GPU product path never links, loads or calls it, and it shares no code, header or
 * constant with the GPU library.
 *
 * What it computes: the gradients of O = softmax(scale * Q K^T, mask) V with respect to Q, K and V
 * for an output gradient dO, by recomputing the probabilities from Q and K. The pages say this much
 * of the backward: the forward keeps only the per-row statistics (the logsumexp) and the backward
 * recomputes S and P block by block instead of storing the T x T matrix
 * (learn-llm.fim.ai "手写 FlashAttention：拆开 SDPA 这个黑盒", STEP 4, the note on training;
 * ijyty.com FlashAttention article, section 2.2, recomputation and per-block gradient
 * accumulation). The gradient itself is the derivative of that definition, written out:
 *
 *   P_ij   = exp(s_ij - m_i) / l_i,  s_ij = scale * q_i . k_j  over the visible keys j
 *   dV_j   = sum_i P_ij dO_i
 *   dP_ij  = dO_i . v_j
 *   D_i    = sum_j P_ij dP_ij = dO_i . O_i           (returned as delta)
 *   dS_ij  = P_ij (dP_ij - D_i)                      (derivative of the row softmax)
 *   dQ_i   = scale * sum_j dS_ij k_j
 *   dK_j   = scale * sum_i dS_ij q_i
 *
 * Everything is double precision; heads are independent and are spread over OpenMP threads; within
 * a head rows i ascend and, in each row, keys j and channels c ascend. A forward on double inputs
 * with exactly the operation order of fa_ref.c is included so that the gradients can be checked
 * against finite differences of the forward.
 *
 * Layouts: all tensors contiguous [B, H, T, d] (delta and lse [B, H, T]); bf16 inputs are bit
 * patterns, everything else double.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

#include "fa_ref.h"

static double bwd_bf16_to_double(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static int bwd_check(const void* a, const void* b, const void* c, const void* e, int64_t B, int64_t H,
                     int64_t T, int64_t d, double scale) {
  if (!a || !b || !c || !e) return FA_REF_EINVAL;
  if (B < 0 || H < 0 || T < 0 || d <= 0) return FA_REF_EINVAL;
  if (!isfinite(scale)) return FA_REF_EINVAL;
  return FA_REF_OK;
}

/* Forward of one head on doubles, in the order of fa_ref.c: scores, max, exp-sum, o / l, m + log l. */
static void fwd_head_f64(const double* q, const double* k, const double* v, int64_t T, int64_t d,
                         int causal, double scale, double* o, double* lse, double* s) {
  for (int64_t i = 0; i < T; ++i) {
    const int64_t n_keys = causal ? i + 1 : T;
    for (int64_t j = 0; j < n_keys; ++j) {
      double dot = 0.0;
      for (int64_t c = 0; c < d; ++c) dot += q[i * d + c] * k[j * d + c];
      s[j] = scale * dot;
    }
    double m = -INFINITY;
    for (int64_t j = 0; j < n_keys; ++j)
      if (s[j] > m) m = s[j];
    double l = 0.0;
    double* o_row = o + i * d;
    for (int64_t c = 0; c < d; ++c) o_row[c] = 0.0;
    for (int64_t j = 0; j < n_keys; ++j) {
      const double e = exp(s[j] - m);
      l += e;
      for (int64_t c = 0; c < d; ++c) o_row[c] += e * v[j * d + c];
    }
    for (int64_t c = 0; c < d; ++c) o_row[c] /= l;
    lse[i] = m + log(l);
  }
}

/*
 * Backward of one head. p (T doubles) and o_row (d doubles) are scratch. dk and dv are accumulated
 * over the rows, so they are cleared first.
 */
static void bwd_head_f64(const double* q, const double* k, const double* v, const double* dout,
                         int64_t T, int64_t d, int causal, double scale, double* dq, double* dk,
                         double* dv, double* delta, double* p, double* o_row) {
  for (int64_t x = 0; x < T * d; ++x) {
    dk[x] = 0.0;
    dv[x] = 0.0;
  }
  for (int64_t i = 0; i < T; ++i) {
    const int64_t n_keys = causal ? i + 1 : T;
    const double* qi = q + i * d;
    const double* doi = dout + i * d;
    /* the row's probabilities, by the two-pass softmax of the scaled scores */
    for (int64_t j = 0; j < n_keys; ++j) {
      double dot = 0.0;
      for (int64_t c = 0; c < d; ++c) dot += qi[c] * k[j * d + c];
      p[j] = scale * dot;
    }
    double m = -INFINITY;
    for (int64_t j = 0; j < n_keys; ++j)
      if (p[j] > m) m = p[j];
    double l = 0.0;
    for (int64_t j = 0; j < n_keys; ++j) {
      p[j] = exp(p[j] - m);
      l += p[j];
    }
    for (int64_t j = 0; j < n_keys; ++j) p[j] /= l;
    /* O_i and D_i = dO_i . O_i */
    for (int64_t c = 0; c < d; ++c) o_row[c] = 0.0;
    for (int64_t j = 0; j < n_keys; ++j)
      for (int64_t c = 0; c < d; ++c) o_row[c] += p[j] * v[j * d + c];
    double D = 0.0;
    for (int64_t c = 0; c < d; ++c) D += doi[c] * o_row[c];
    delta[i] = D;
    /* dS_ij = P_ij (dO_i . v_j - D_i); accumulate dQ_i, dK_j, dV_j */
    double* dqi = dq + i * d;
    for (int64_t c = 0; c < d; ++c) dqi[c] = 0.0;
    for (int64_t j = 0; j < n_keys; ++j) {
      double dp = 0.0;
      for (int64_t c = 0; c < d; ++c) dp += doi[c] * v[j * d + c];
      const double ds = p[j] * (dp - D);
      for (int64_t c = 0; c < d; ++c) {
        dqi[c] += ds * k[j * d + c];
        dk[j * d + c] += ds * qi[c];
        dv[j * d + c] += p[j] * doi[c];
      }
    }
    for (int64_t c = 0; c < d; ++c) dqi[c] *= scale;
  }
  for (int64_t x = 0; x < T * d; ++x) dk[x] *= scale;
}

/* Forward on double inputs (o [B,H,T,d], lse [B,H,T]); the order of operations is fa_ref_fwd's. */
int fa_ref_fwd_f64(const double* q, const double* k, const double* v, double* o, double* lse,
                   int64_t B, int64_t H, int64_t T, int64_t d, int causal, double scale,
                   int num_threads) {
  int rc = bwd_check(q, k, v, o, B, H, T, d, scale);
  if (rc) return rc;
  if (!lse) return FA_REF_EINVAL;
  const int64_t n_heads = B * H;
  if (n_heads == 0 || T == 0) return FA_REF_OK;
  int failed = 0;
  const int nt = num_threads > 0 ? num_threads : omp_get_max_threads();
#pragma omp parallel num_threads(nt)
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)T);
    if (!s) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t h = 0; h < n_heads; ++h) {
      if (!s) continue;
      const int64_t off = h * T * d;
      fwd_head_f64(q + off, k + off, v + off, T, d, causal, scale, o + off, lse + h * T, s);
    }
    free(s);
  }
  return failed ? FA_REF_ENOMEM : FA_REF_OK;
}

/* Backward on double inputs: dq, dk, dv [B,H,T,d] and delta [B,H,T]. */
int fa_ref_bwd_f64(const double* q, const double* k, const double* v, const double* dout, double* dq,
                   double* dk, double* dv, double* delta, int64_t B, int64_t H, int64_t T, int64_t d,
                   int causal, double scale, int num_threads) {
  int rc = bwd_check(q, k, v, dout, B, H, T, d, scale);
  if (rc) return rc;
  if (!dq || !dk || !dv || !delta) return FA_REF_EINVAL;
  const int64_t n_heads = B * H;
  if (n_heads == 0 || T == 0) return FA_REF_OK;
  int failed = 0;
  const int nt = num_threads > 0 ? num_threads : omp_get_max_threads();
#pragma omp parallel num_threads(nt)
  {
    double* p = (double*)malloc(sizeof(double) * (size_t)T);
    double* o_row = (double*)malloc(sizeof(double) * (size_t)d);
    if (!p || !o_row) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t h = 0; h < n_heads; ++h) {
      if (!p || !o_row) continue;
      const int64_t off = h * T * d;
      bwd_head_f64(q + off, k + off, v + off, dout + off, T, d, causal, scale, dq + off, dk + off,
                   dv + off, delta + h * T, p, o_row);
    }
    free(p);
    free(o_row);
  }
  return failed ? FA_REF_ENOMEM : FA_REF_OK;
}

/* Backward on bf16 inputs (bit patterns): widens every input to double, then fa_ref_bwd_f64. */
int fa_ref_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dout,
               double* dq, double* dk, double* dv, double* delta, int64_t B, int64_t H, int64_t T,
               int64_t d, int causal, double scale, int num_threads) {
  int rc = bwd_check(q, k, v, dout, B, H, T, d, scale);
  if (rc) return rc;
  if (!dq || !dk || !dv || !delta) return FA_REF_EINVAL;
  const int64_t n = B * H * T * d;
  if (n == 0) return FA_REF_OK;
  double* buf = (double*)malloc(sizeof(double) * (size_t)n * 4);
  if (!buf) return FA_REF_ENOMEM;
  const uint16_t* src[4] = {q, k, v, dout};
  for (int t = 0; t < 4; ++t)
    for (int64_t x = 0; x < n; ++x) buf[t * n + x] = bwd_bf16_to_double(src[t][x]);
  rc = fa_ref_bwd_f64(buf, buf + n, buf + 2 * n, buf + 3 * n, dq, dk, dv, delta, B, H, T, d, causal,
                      scale, num_threads);
  free(buf);
  return rc;
}
