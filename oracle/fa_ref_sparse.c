/*
 * CPU oracle for the block-sparse attention forward — TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the package smoke check and the benchmark's CPU-baseline leg may load this
 * library. The GPU product path never links, loads or calls it.
 *
 * A block mask marks, per (query block, key block), whether the block takes part at all; a block
 * whose mask is zero is skipped as a whole, the way the causal mask skips the blocks above the
 * diagonal (cnblogs "内核案例研究：Flash Attention", section "块稀疏注意力 V2 和 V3"). Written
 * out as the plain definition: key j is visible to query i iff
 *
 *     mask[h][i / block_m][j / block_n] != 0   and, with the causal mask, j <= i,
 *
 * and the row is the exact softmax over its visible keys (two passes: max, then exp-sum, as in
 * fa_ref.c). A row with no visible key has no softmax; it is given O = 0 and LSE = -inf.
 *
 * Layouts: q, k, v bf16 bit patterns [B, H, T, d]; o double [B, H, T, d]; lse double [B, H, T];
 * mask uint8 [mask_heads, ceil(T / block_m), ceil(T / block_n)], mask_heads 1 (one mask for every
 * batch and head) or B*H (head b*H + h uses mask b*H + h).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

#include "fa_ref.h"

static double sp_bf16_to_double(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

int fa_ref_fwd_blockmask(const uint16_t* q, const uint16_t* k, const uint16_t* v, double* o,
                         double* lse, int64_t B, int64_t H, int64_t T, int64_t d, int causal,
                         double scale, const uint8_t* mask, int64_t mask_heads, int64_t block_m,
                         int64_t block_n, int num_threads) {
  if (!q || !k || !v || !o || !lse || !mask) return FA_REF_EINVAL;
  if (B < 0 || H < 0 || T < 0 || d <= 0 || block_m <= 0 || block_n <= 0) return FA_REF_EINVAL;
  if (!isfinite(scale)) return FA_REF_EINVAL;
  if (mask_heads != 1 && mask_heads != B * H) return FA_REF_EINVAL;
  const int64_t n_rows = B * H * T;
  if (n_rows == 0) return FA_REF_OK;
  const int64_t nqb = (T + block_m - 1) / block_m, nkb = (T + block_n - 1) / block_n;
  int failed = 0;
  const int nt = num_threads > 0 ? num_threads : omp_get_max_threads();
#pragma omp parallel num_threads(nt)
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)T);
    char* vis = (char*)malloc((size_t)T);
    if (!s || !vis) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 16)
    for (int64_t r = 0; r < n_rows; ++r) {
      if (!s || !vis) continue;
      const int64_t head = r / T, i = r % T;
      const int64_t off = head * T * d;
      const uint8_t* mrow = mask + (mask_heads == 1 ? 0 : head) * nqb * nkb + (i / block_m) * nkb;
      const uint16_t* qr = q + off + i * d;
      double* orow = o + r * d;
      /* visible keys and their scores */
      int64_t n_vis = 0;
      for (int64_t j = 0; j < T; ++j) {
        vis[j] = mrow[j / block_n] != 0 && (!causal || j <= i);
        if (!vis[j]) continue;
        ++n_vis;
        double dot = 0.0;
        for (int64_t c = 0; c < d; ++c) dot += sp_bf16_to_double(qr[c]) * sp_bf16_to_double(k[off + j * d + c]);
        s[j] = scale * dot;
      }
      for (int64_t c = 0; c < d; ++c) orow[c] = 0.0;
      if (n_vis == 0) {
        lse[r] = -INFINITY;
        continue;
      }
      double m = -INFINITY;
      for (int64_t j = 0; j < T; ++j)
        if (vis[j] && s[j] > m) m = s[j];
      double l = 0.0;
      for (int64_t j = 0; j < T; ++j) {
        if (!vis[j]) continue;
        const double e = exp(s[j] - m);
        l += e;
        for (int64_t c = 0; c < d; ++c) orow[c] += e * sp_bf16_to_double(v[off + j * d + c]);
      }
      for (int64_t c = 0; c < d; ++c) orow[c] /= l;
      lse[r] = m + log(l);
    }
    free(s);
    free(vis);
  }
  return failed ? FA_REF_ENOMEM : FA_REF_OK;
}
