/*
 * fa_ref.h — C entry points of the CPU oracle (liboracle.so) — TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the package smoke check and the benchmark's CPU-baseline leg load this
 * library (through ctypes, oracle/__init__.py, or a test's own C driver). The GPU library never
 * includes this header, links or calls the oracle, and this header shares nothing with include/fa.h.
 *
 * What each function computes is stated at its definition (fa_ref.c, fa_ref_bwd.c,
 * fa_ref_sparse.c): the plain two-pass definition of attention in double precision on bf16 inputs
 * (learn-llm.fim.ai "手写 FlashAttention：拆开 SDPA 这个黑盒", STEP 1-4), its gradients, and the
 * block-mask variant (cnblogs "内核案例研究：Flash Attention", section "块稀疏注意力 V2 和 V3").
 *
 * Conventions:
 *   - Sizes are int64_t: the oracle is called from Python with shapes that may exceed a C int in
 *     products (B*H*T*d), and it indexes with 64-bit integers throughout. (The GPU library's own
 *     entry points take int sizes, as its contract fixes.)
 *   - q, k, v, dout are bf16 bit patterns (uint16_t), contiguous [B, H, T, d], on the host; outputs
 *     are double, host, written in full. The caller owns every buffer.
 *   - num_threads: OpenMP threads for the call; 0 takes the OpenMP default.
 *   - Return FA_REF_OK, FA_REF_EINVAL (a NULL pointer, a negative size, d <= 0, a non-finite scale)
 *     or FA_REF_ENOMEM (a per-thread scratch row could not be allocated). Nothing is guaranteed
 *     about the outputs after an error.
 */
#ifndef FA_REF_H_
#define FA_REF_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_REF_OK 0
#define FA_REF_EINVAL (-1)
#define FA_REF_ENOMEM (-2)

/* Threads an OpenMP team of the oracle gets for num_threads (0: the default). */
int fa_ref_threads_used(int num_threads);

/* Forward, every row: o [B,H,T,d], lse [B,H,T] (natural log over the visible scaled scores). */
int fa_ref_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, double* o, double* lse,
               int64_t B, int64_t H, int64_t T, int64_t d, int causal, double scale, int num_threads);

/* Forward of selected rows: rows[n] = (b*H + h)*T + i; output n goes to o[n*d ..] and lse[n]. */
int fa_ref_fwd_rows(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t B, int64_t H,
                    int64_t T, int64_t d, int causal, double scale, const int64_t* rows, int64_t n_sel,
                    double* o, double* lse, int num_threads);

/* Forward on double inputs, with fa_ref_fwd's order of operations (for finite differences). */
int fa_ref_fwd_f64(const double* q, const double* k, const double* v, double* o, double* lse,
                   int64_t B, int64_t H, int64_t T, int64_t d, int causal, double scale,
                   int num_threads);

/* Backward on double inputs: dq, dk, dv [B,H,T,d] and delta [B,H,T] (D_i = dO_i . O_i). */
int fa_ref_bwd_f64(const double* q, const double* k, const double* v, const double* dout, double* dq,
                   double* dk, double* dv, double* delta, int64_t B, int64_t H, int64_t T, int64_t d,
                   int causal, double scale, int num_threads);

/* Backward on bf16 inputs (widened exactly to double, then fa_ref_bwd_f64). */
int fa_ref_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dout,
               double* dq, double* dk, double* dv, double* delta, int64_t B, int64_t H, int64_t T,
               int64_t d, int causal, double scale, int num_threads);

/* Forward under a block mask [mask_heads, ceil(T/block_m), ceil(T/block_n)] (nonzero = visible);
 * a row with no visible key gets O = 0 and LSE = -inf. mask_heads is 1 or B*H. */
int fa_ref_fwd_blockmask(const uint16_t* q, const uint16_t* k, const uint16_t* v, double* o,
                         double* lse, int64_t B, int64_t H, int64_t T, int64_t d, int causal,
                         double scale, const uint8_t* mask, int64_t mask_heads, int64_t block_m,
                         int64_t block_n, int num_threads);

#ifdef __cplusplus
}
#endif

#endif /* FA_REF_H_ */
