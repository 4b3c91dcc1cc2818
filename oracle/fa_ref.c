/*
 * CPU oracle for exact attention forward — TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the package smoke check and the benchmark's CPU-baseline leg may load this
 * library. The GPU product path never links, loads or calls it, and it shares no code, header or
 * constant with the GPU library.
 *
 * What it computes is the plain definition of attention, written out naively in double precision
 * on the bf16 inputs (every bf16 value is exactly representable as a double):
 *
 *   S = scale * Q K^T, then a row softmax, then P V
 *       (learn-llm.fim.ai, "手写 FlashAttention：拆开 SDPA 这个黑盒", STEP 1: the naive form
 *        that materialises the T x T score matrix per head)
 *
 *   the softmax subtracts the row maximum before exponentiating, which leaves the result unchanged
 *       (same page, STEP 2, the note on why the maximum is subtracted: numerator and denominator
 *        are both multiplied by exp(-m), so every exponent is <= 1)
 *
 *   causal masking keeps key j for query i only when j <= i: the upper-right part of the T x T grid
 *   is masked (same page, STEP 3, the block-grid legend)
 *
 *   the per-row logsumexp (natural log, over the scaled scores of the visible keys) is returned as
 *   well; it is what the forward pass saves for the backward (same page, STEP 4, the note on whether
 *   the kernel can be used for training)
 *
 * The softmax is two-pass (max, then exp-sum), not the online recurrence the GPU kernel uses, so the
 * two implementations share neither code nor algorithm. Rows are independent and are spread over
 * OpenMP threads; within a row the key loop and the channel loop run in ascending order.
 *
 * Layouts: q, k, v are bf16 bit patterns, contiguous [B, H, T, d]. o is double [B, H, T, d]; lse is
 * double [B, H, T].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

#include "fa_ref.h"

/* A bf16 value is the top half of an IEEE binary32; widening it to double is exact. */
static double bf16_bits_to_double(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/*
 * One query row i of one head. qh/kh/vh point at the head's [T, d] slices. scores is caller-owned
 * scratch of at least T doubles. Writes d outputs to o_row and the row's logsumexp to *lse_out.
 */
static void attend_one_row(const uint16_t* qh, const uint16_t* kh, const uint16_t* vh, int64_t T,
                           int64_t d, int causal, double scale, int64_t i, double* scores,
                           double* o_row, double* lse_out) {
  const int64_t n_keys = causal ? i + 1 : T; /* visible keys are 0 .. n_keys-1 */
  const uint16_t* q_row = qh + i * d;

  /* scores s_j = scale * sum_c q[i,c] k[j,c] */
  for (int64_t j = 0; j < n_keys; ++j) {
    const uint16_t* k_row = kh + j * d;
    double dot = 0.0;
    for (int64_t c = 0; c < d; ++c) dot += bf16_bits_to_double(q_row[c]) * bf16_bits_to_double(k_row[c]);
    scores[j] = scale * dot;
  }

  /* pass 1: row maximum */
  double m = -INFINITY;
  for (int64_t j = 0; j < n_keys; ++j)
    if (scores[j] > m) m = scores[j];

  /* pass 2: e_j = exp(s_j - m), l = sum e_j, o = sum e_j v_j / l */
  double l = 0.0;
  for (int64_t c = 0; c < d; ++c) o_row[c] = 0.0;
  for (int64_t j = 0; j < n_keys; ++j) {
    const double e = exp(scores[j] - m);
    l += e;
    const uint16_t* v_row = vh + j * d;
    for (int64_t c = 0; c < d; ++c) o_row[c] += e * bf16_bits_to_double(v_row[c]);
  }
  for (int64_t c = 0; c < d; ++c) o_row[c] /= l;
  *lse_out = m + log(l);
}

static int check_args(const void* q, const void* k, const void* v, int64_t B, int64_t H, int64_t T,
                      int64_t d, double scale) {
  if (!q || !k || !v) return FA_REF_EINVAL;
  if (B < 0 || H < 0 || T < 0 || d <= 0) return FA_REF_EINVAL;
  if (!isfinite(scale)) return FA_REF_EINVAL;
  return FA_REF_OK;
}

/* Number of threads an OpenMP team gets when num_threads are requested (<= 0: the default). */
int fa_ref_threads_used(int num_threads) {
  int used = 1;
  if (num_threads > 0) {
#pragma omp parallel num_threads(num_threads)
    {
#pragma omp single
      used = omp_get_num_threads();
    }
  } else {
#pragma omp parallel
    {
#pragma omp single
      used = omp_get_num_threads();
    }
  }
  return used;
}

/*
 * Full forward: every row of every head. Returns 0, or a negative code for bad arguments or a
 * failed scratch allocation.
 */
int fa_ref_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, double* o, double* lse,
               int64_t B, int64_t H, int64_t T, int64_t d, int causal, double scale, int num_threads) {
  int rc = check_args(q, k, v, B, H, T, d, scale);
  if (rc) return rc;
  if (!o || !lse) return FA_REF_EINVAL;
  const int64_t n_rows = B * H * T;
  if (n_rows == 0) return FA_REF_OK;
  int failed = 0;
  const int nt = num_threads > 0 ? num_threads : omp_get_max_threads();
#pragma omp parallel num_threads(nt)
  {
    double* scores = (double*)malloc(sizeof(double) * (size_t)T);
    if (!scores) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 16)
    for (int64_t r = 0; r < n_rows; ++r) {
      if (!scores) continue;
      const int64_t head = r / T, i = r % T;
      const int64_t off = head * T * d;
      attend_one_row(q + off, k + off, v + off, T, d, causal, scale, i, scores, o + r * d, lse + r);
    }
    free(scores);
  }
  return failed ? FA_REF_ENOMEM : FA_REF_OK;
}

/*
 * Selected rows only. rows[n] is a flat row index (b*H + h)*T + i in [0, B*H*T). Output n goes to
 * o[n*d .. n*d+d) and lse[n]. Used where the full problem is too large to evaluate on the host.
 */
int fa_ref_fwd_rows(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t B, int64_t H,
                    int64_t T, int64_t d, int causal, double scale, const int64_t* rows, int64_t n_sel,
                    double* o, double* lse, int num_threads) {
  int rc = check_args(q, k, v, B, H, T, d, scale);
  if (rc) return rc;
  if (n_sel < 0 || (n_sel > 0 && (!rows || !o || !lse))) return FA_REF_EINVAL;
  const int64_t n_rows = B * H * T;
  for (int64_t n = 0; n < n_sel; ++n)
    if (rows[n] < 0 || rows[n] >= n_rows) return FA_REF_EINVAL;
  if (n_sel == 0) return FA_REF_OK;
  int failed = 0;
  const int nt = num_threads > 0 ? num_threads : omp_get_max_threads();
#pragma omp parallel num_threads(nt)
  {
    double* scores = (double*)malloc(sizeof(double) * (size_t)T);
    if (!scores) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 4)
    for (int64_t n = 0; n < n_sel; ++n) {
      if (!scores) continue;
      const int64_t r = rows[n];
      const int64_t head = r / T, i = r % T;
      const int64_t off = head * T * d;
      attend_one_row(q + off, k + off, v + off, T, d, causal, scale, i, scores, o + n * d, lse + n);
    }
    free(scores);
  }
  return failed ? FA_REF_ENOMEM : FA_REF_OK;
}
