/*
 * fa.h — C-ABI of the MI355X (gfx950) exact tiled attention library (libfa.so).
 *
 * The main operation is the fused, tiled, exact attention forward
 *
 *     O[b,h,i,:] = sum_j P[i,j] V[b,h,j,:],   P[i,:] = softmax_j( scale * Q[b,h,i,:] . K[b,h,j,:] )
 *     LSE[b,h,i] = ln sum_j exp( scale * Q[b,h,i,:] . K[b,h,j,:] )
 *
 * over the visible keys j (all j < T, or j <= i with the causal mask), computed block by block with
 * the online softmax so that the T x T score matrix never reaches HBM:
 *   - the naive definition and why the T x T matrix is the problem: learn-llm.fim.ai
 *     "手写 FlashAttention：拆开 SDPA 这个黑盒", STEP 1;
 *   - the online max / sum recurrence and the deferred division by l: same page, STEP 2;
 *   - one program per Q block walking the K/V blocks, causal blocks above the diagonal skipped:
 *     same page, STEP 3;
 *   - exp2 with log2(e) folded into the scale, and the per-row logsumexp kept for a backward pass:
 *     same page, STEP 4;
 *   - the Q-block-parallel ordering that keeps m and l on chip: cnblogs
 *     "内核案例研究：Flash Attention", section "块稀疏注意力 V2 和 V3".
 * Its gradients (fa_bwd) are computed from the saved logsumexp by recomputation.
 *
 * Conventions shared by every entry point:
 *   - Tensors are row-major and contiguous. q, k, v and o are bf16 [B, H, T, d] (the innermost
 *     dimension is d); lse is fp32 [B, H, T]. All of them are device pointers.
 *   - The caller owns every buffer. The library never allocates, frees or keeps a pointer after the
 *     call returns. o and lse must not overlap q, k, v or each other.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL is the default stream). They return
 *     after enqueueing the kernel and never synchronise. Apart from the address of
 *     fa_fwd_splitkv_noalloc's fixed buffer, looked up once per device and kept in an atomic, the
 *     library keeps no mutable global state; every entry point is safe to call from several host
 *     threads at once (fa_fwd_splitkv_noalloc's calls that overlap on one GPU share its buffer).
 *   - A call enqueues kernel launches only (no allocation, memset, copy or synchronisation), so it
 *     may be captured into a HIP graph on a capturing stream and replayed.
 *   - Arguments are checked before anything is launched; on any error nothing is written.
 *   - B*H*T == 0 is a valid empty problem: FA_OK, nothing launched, nothing written.
 *   - Inputs must be finite. NaN or Inf inputs give unspecified outputs (no error is raised), and so
 *     do scaled scores (scale * q.k) beyond fp32's range, which no check can see before launching.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_status {
  FA_OK = 0,
  FA_ERR_NULL = -1,           /* a required pointer is NULL */
  FA_ERR_INVALID_ARG = -2,    /* negative size, size too large, scale not finite and > 0 (or
                                 scale * log2 e not finite), overlap */
  FA_ERR_UNSUPPORTED_D = -3,  /* head dim d is not 64 or 128 */
  FA_ERR_ALIGNMENT = -4,      /* q, k, v or o not 16-byte aligned, or lse not 4-byte aligned */
  FA_ERR_HIP = -5,            /* the kernel launch itself failed (its own status, not an earlier
                                 error still pending in hipGetLastError) */
  FA_ERR_TILE = -6,           /* fa_fwd_ex / fa_fwd_plan: tile shape not in the supported table */
  FA_ERR_SCRATCH = -7         /* fa_fwd_splitkv_noalloc: the problem needs more scratch than the
                                 library's fixed buffer holds (FA_NOALLOC_SCRATCH_BYTES) */
} fa_status;

/* Largest accepted sequence length and largest accepted B*H (checked by every entry point). */
#define FA_MAX_T (1 << 22)
#define FA_MAX_BH (1 << 24)

/*
 * fa_fwd — exact attention forward.
 *   q, k, v  [in]  bf16 [B, H, T, d], device, 16-byte aligned
 *   o        [out] bf16 [B, H, T, d], device, 16-byte aligned; rounded to nearest even
 *   lse      [out] fp32 [B, H, T], device, 4-byte aligned; natural-log logsumexp of each row's
 *                  scaled scores over its visible keys
 *   B, H, T  batch, heads, sequence length (queries and keys both have length T); >= 0,
 *            T <= FA_MAX_T, B*H <= FA_MAX_BH
 *   d        head dimension: 64 or 128
 *   causal   nonzero: query i sees keys 0..i (the causal mask); zero: it sees all T keys
 *   scale    finite and > 0, and scale * log2(e) finite in fp32 (scale below about 2.36e38); the
 *            scores are scale * q.k (1/sqrt(d) for standard attention)
 *   stream   hipStream_t to launch on (NULL: default stream)
 * The launch depends on the sizes (fa_fwd_plan reports it): 128 queries x 64 keys per workgroup and
 * tile, or, at d = 64 for short sequences, one of two others. With nq = ceil(T/128) query blocks
 * per head and grid = nq*B*H:
 *   - the key split (two waves per 32-query block each take every other K/V tile and merge their
 *     partial results in log space; ijyty.com FlashAttention article, section 2.1) when causal,
 *     nq >= 8, grid <= 384 and (nq >= 16 or grid <= 288), or non-causal and grid <= 256;
 *   - else 128-key tiles when nq >= 5 and (nq <= 8 or grid <= 768).
 * At d = 128, non-causal launches with T >= 2048 take 256 queries (8 waves) per workgroup. Every
 * launch gives the exact result up to rounding order; a fixed problem always takes the same launch,
 * so repeated calls are bit-identical.
 * Returns FA_OK or a negative fa_status.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int T,
           int d, int causal, float scale, void* stream);

/*
 * fa_fwd_ex — fa_fwd with the tile shape forced, for the tile-shape study. The block size is bounded
 * by what one program's Q, K, V, score and accumulator blocks can keep on chip, and real kernels pick
 * it by measuring a few candidates (learn-llm.fim.ai "手写 FlashAttention：拆开 SDPA 这个黑盒",
 * STEP 3, the note on choosing the block size); the extra arguments name the candidate.
 *   block_m  query rows per workgroup: 32 * waves (one 32-query block per wave), 64 * waves (two per
 *            wave) or 16 * waves (the key split, two waves per block: fa_fwd_ex(..., 64, 64, 4))
 *   block_n  keys per K/V tile staged in LDS
 *   waves    64-lane wavefronts per workgroup
 * The supported (d, block_m, block_n, waves) combinations are those fa_fwd_plan accepts; any other
 * returns FA_ERR_TILE. Otherwise identical to fa_fwd (same arguments, errors and results).
 */
int fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int T,
              int d, int causal, float scale, void* stream, int block_m, int block_n, int waves);

/* Launch plan of one call: what fa_fwd (or fa_fwd_ex) would launch. Host-only; no HIP call. */
typedef struct fa_plan_info {
  int block_m;     /* query rows per workgroup */
  int block_n;     /* keys per K/V tile */
  int waves;       /* wavefronts per workgroup */
  int q_blocks;    /* ceil(T / block_m) */
  long long grid;  /* workgroups: q_blocks * B * H (one per (Q block, batch*head)); a grid of more
                      than (2^32 - 1) / (64 * waves) workgroups is launched folded into two grid
                      dimensions, with fewer than 8 spare workgroups per fold that exit at once */
  int lds_bytes;   /* LDS per workgroup: double-buffered K and V tiles */
  long long kv_tiles; /* K/V tiles processed by all workgroups (fully masked ones skipped) */
  int key_split;   /* 1, or 2: two waves share each 32-query block, each taking every other K/V tile,
                      and merge their partial results in log space (a default at d = 64 for
                      the short sequences described at fa_fwd) */
  int head_group;  /* when B*H is a multiple of 8 each of the 8 XCDs takes B*H/8 heads, and streams
                      their K/V head_group heads at a time: the largest divisor of B*H/8 whose K and
                      V fit in 16 MB (causal) or 2 MB (non-causal); 1 otherwise */
} fa_plan_info;

/*
 * fa_fwd_plan — fill *out with the launch plan for these sizes.
 *   block_m, block_n, waves: all 0 for the default table entry, or all > 0 to ask about a forced
 *   shape (as fa_fwd_ex would use it).
 * Returns FA_OK, FA_ERR_NULL (out NULL), FA_ERR_INVALID_ARG (bad sizes), FA_ERR_UNSUPPORTED_D or
 * FA_ERR_TILE. Sizes may be zero (then grid and kv_tiles are 0).
 */
int fa_fwd_plan(int B, int H, int T, int d, int causal, int block_m, int block_n, int waves,
                fa_plan_info* out);

/*
 * fa_fwd_sparse — exact attention forward under a block mask (block-sparse attention).
 *
 * The keys are split into blocks per (query block, key block), and a block whose mask is zero is
 * skipped as a whole, computing nothing, the way the causal mask skips the blocks above the
 * diagonal (cnblogs "内核案例研究：Flash Attention", section "块稀疏注意力 V2 和 V3"). Key j is
 * visible to query i iff
 *     block_mask[m][i / FA_SPARSE_BLOCK_M][j / FA_SPARSE_BLOCK_N] != 0   (and j <= i if causal),
 * with m = 0 when mask_heads == 1 and m = b*H + h when mask_heads == B*H. O and LSE are the exact
 * softmax over the visible keys, as for fa_fwd; a row with no visible key gets O = 0 and
 * LSE = -inf.
 *   block_mask [in] uint8 [mask_heads, ceil(T / FA_SPARSE_BLOCK_M), ceil(T / FA_SPARSE_BLOCK_N)],
 *                   device; nonzero = the block is computed
 *   mask_heads      1 (one mask for every batch and head) or B*H (one per head)
 *   T               <= FA_SPARSE_MAX_T
 *   other arguments, layouts, ownership and errors as for fa_fwd (d = 64 or 128); o and lse must
 *   not overlap the mask either. FA_ERR_INVALID_ARG for a bad mask_heads or T.
 */
#define FA_SPARSE_BLOCK_M 128
#define FA_SPARSE_BLOCK_N 64
#define FA_SPARSE_MAX_T 65536
int fa_fwd_sparse(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                  int T, int d, int causal, float scale, const unsigned char* block_mask,
                  int mask_heads, void* stream);

/*
 * fa_fwd_partial — exact attention forward of T queries restricted to the keys [k_begin, k_end) of
 * a sequence of Tk keys: the partial result of one key range, for a split of the keys across
 * launches (split-KV) or devices (the keys of a sequence shard).
 *   q        [in]  bf16 [B, H, T, d], device, 16-byte aligned
 *   k, v     [in]  bf16 [B, H, Tk, d], device, 16-byte aligned (Tk = T for self-attention)
 *   o_part   [out] fp32 [B, H, T, d], 16-byte aligned: softmax over the range's visible keys times V
 *   lse_part [out] fp32 [B, H, T], 4-byte aligned: logsumexp over the range's visible keys
 *   k_begin, k_end  0 <= k_begin <= k_end <= Tk; k_begin a multiple of FA_PARTIAL_KEY_ALIGN, k_end
 *                   a multiple of it or Tk
 *   causal   the queries are the last T positions of the Tk-key sequence: query i sees key j iff
 *            j <= i + Tk - T (with Tk = T, the usual j <= i; with T > Tk, the first T - Tk queries
 *            see no key)
 *   other arguments as for fa_fwd (d = 64 or 128; 0 <= Tk <= FA_MAX_T)
 * A row with no visible key in the range gets o_part = 0 and lse_part = -inf. Merging the partial
 * results of disjoint ranges that cover [0, Tk) with fa_merge gives the full attention.
 */
#define FA_PARTIAL_KEY_ALIGN 64
int fa_fwd_partial(const void* q, const void* k, const void* v, float* o_part, float* lse_part,
                   int B, int H, int T, int Tk, int d, int causal, float scale, int k_begin, int k_end,
                   void* stream);

/*
 * fa_merge — combine partial results over disjoint key ranges in log space (ijyty.com
 * FlashAttention article, section 2.1: per-block logsumexp accumulated in log space, the output
 * divided by exp(lse) at the end):
 *     LSE = log sum_s exp(LSE_s),   O = sum_s exp(LSE_s - LSE) O_s
 *   o_parts   [in]  fp32 [n_parts, B, H, T, d], 16-byte aligned (e.g. fa_fwd_partial outputs)
 *   lse_parts [in]  fp32 [n_parts, B, H, T], 4-byte aligned
 *   n_parts         1 .. FA_MERGE_MAX_PARTS
 *   o         [out] bf16 [B, H, T, d], 16-byte aligned; lse [out] fp32 [B, H, T], 4-byte aligned
 *   B, H, T, d, stream as for fa_fwd. Rows whose parts are all -inf get O = 0 and LSE = -inf.
 * Outputs must not overlap the inputs or each other. Returns FA_OK or a negative fa_status.
 */
#define FA_MERGE_MAX_PARTS 4096
int fa_merge(const float* o_parts, const float* lse_parts, int n_parts, void* o, float* lse, int B,
             int H, int T, int d, void* stream);

/*
 * fa_fwd_splitkv — exact attention of T queries over Tk keys with the keys split into equal ranges
 * that run side by side, then merged in log space (the two steps above in one call): for shapes
 * with few queries and many keys (T << Tk, e.g. decoding against a long prefix), where one
 * workgroup per query block would leave most of the GPU idle.
 *   q, k, v, causal, scale  as for fa_fwd_partial; o bf16 [B, H, T, d] and lse fp32 [B, H, T] as
 *                           for fa_fwd
 *   n_splits   1 .. FA_MERGE_MAX_PARTS: the keys are cut into ranges of ceil(ceil(Tk/64)/n_splits)
 *              tiles of 64 keys; ranges past Tk are not launched
 *   workspace  device memory of at least fa_splitkv_workspace_bytes(B, H, T, d, n_splits) bytes,
 *              16-byte aligned, owned by the caller: the fp32 partial results (O, then LSE);
 *              overwritten
 *   workspace_bytes  its size; FA_ERR_INVALID_ARG if below that figure, or if the figure is 0 for a
 *              non-empty problem (sizes or n_splits out of range)
 * Two kernels run in order on `stream`. No allocation. Returns FA_OK or a negative fa_status.
 */
/* Workspace bytes fa_fwd_splitkv needs: n_splits * B*H*T * (d + 1) * 4 (fp32 O and LSE per range).
 * 0 for an empty problem, or when fa_fwd_splitkv would reject the sizes (B, H, T or d out of range,
 * n_splits outside 1 .. FA_MERGE_MAX_PARTS) or the product does not fit in size_t. Host-only. */
size_t fa_splitkv_workspace_bytes(int B, int H, int T, int d, int n_splits);
/* A split count for these sizes that fills the GPU: enough key ranges for about 512 workgroups, each
 * range at least 8 tiles of 64 keys, at most 256 ranges. 1 for empty or out-of-range sizes.
 * Host-only. */
int fa_splitkv_splits(int B, int H, int T, int Tk, int d);
int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                   int T, int Tk, int d, int causal, float scale, int n_splits, void* workspace,
                   size_t workspace_bytes, void* stream);

/*
 * fa_fwd_splitkv_noalloc — fa_fwd_splitkv without a workspace argument and without any allocation,
 * for callers that cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). The fp32 partial results go through a fixed buffer that the
 * library holds in device memory, FA_NOALLOC_SCRATCH_BYTES per GPU, from the first call on that GPU
 * until the process ends.
 *   q, k, v, o, lse, B, H, T, Tk, d, causal, scale, n_splits, stream  as for fa_fwd_splitkv; the
 *            scratch used is that of the calling thread's current device, so `stream` must belong
 *            to that device
 * Needs fa_splitkv_workspace_bytes(B, H, T, d, n_splits) <= FA_NOALLOC_SCRATCH_BYTES, else returns
 * FA_ERR_SCRATCH before anything is launched (a smaller n_splits needs less). The first call on a
 * device looks up the buffer's device address (FA_ERR_HIP if that fails); no call allocates, frees,
 * copies or clears memory: every partial result the merge reads is written first by the same call.
 * All calls on one GPU share its buffer, so calls that overlap in time on one GPU (two streams, or
 * two host threads) race and give undefined results; calls ordered on one stream are safe.
 * Results are bit-identical to fa_fwd_splitkv with the same n_splits.
 */
#define FA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                           int H, int T, int Tk, int d, int causal, float scale, int n_splits,
                           void* stream);

/*
 * fa_fwd_fp8 — the attention forward on FP8 inputs: q, k and v are OCP FP8 E4M3 codes ("e4m3fn":
 * bias 7, no infinities, largest magnitude 448) that stand for code * descale, one descale factor per
 * tensor. Both matrix products run on the FP8 matrix unit (the low-precision mode that doubles matrix
 * throughput: cnblogs "内核案例研究：Flash Attention", the closing section on its third version).
 *   q, k, v  [in]  uint8 E4M3 codes [B, H, T, d], device, 16-byte aligned
 *   o        [out] bf16 [B, H, T, d], device, 16-byte aligned
 *   lse      [out] fp32 [B, H, T], device, 4-byte aligned: natural-log logsumexp of the scaled scores
 *   scale, q_descale, k_descale, v_descale  finite and > 0: the scores are
 *            scale * (q_descale * q) . (k_descale * k), and V is v_descale * v; the factor the
 *            kernel applies to the raw products, scale * q_descale * k_descale * log2(e), must lie
 *            between 1e-37 and 3e38 (a normal fp32 number), else FA_ERR_INVALID_ARG
 *   B, H, T, d, causal, stream  as for fa_fwd (d = 64 or 128)
 * Numerics: fp32 accumulation and softmax; the probabilities are rounded to E4M3 (round to nearest
 * even, after scaling the largest weight of each row to 2^8) before the second product, which bounds
 * the relative error of each term of O by 2^-4. O is rounded once to bf16.
 * Returns FA_OK or a negative fa_status (checked before anything is launched).
 */
int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int T,
               int d, int causal, float scale, float q_descale, float k_descale, float v_descale,
               void* stream);

/*
 * fa_bwd — exact attention backward (gradients of fa_fwd), by recomputation from the saved LSE.
 *
 *     dV = P^T dO,  dP = dO V^T,  D_i = dO_i . O_i,  dS = P o (dP - D),
 *     dQ = scale dS K,  dK = scale dS^T Q,   with P = exp(scale Q K^T - LSE) over the visible keys
 *
 * The forward keeps only O and the per-row logsumexp; the backward recomputes the scores and the
 * probabilities block by block instead of storing the T x T matrix (learn-llm.fim.ai
 * "手写 FlashAttention：拆开 SDPA 这个黑盒", STEP 4, the note on training; ijyty.com
 * FlashAttention article, section 2.2: recomputation, and gradients accumulated per block).
 *   q, k, v  [in]  bf16 [B, H, T, d], device, 16-byte aligned: the forward's inputs
 *   o        [in]  bf16 [B, H, T, d], device, 16-byte aligned: the forward's output
 *   lse      [in]  fp32 [B, H, T], device, 4-byte aligned: the forward's logsumexp
 *   dout     [in]  bf16 [B, H, T, d], device, 16-byte aligned: the gradient of the loss wrt o
 *   dq, dk, dv [out] bf16 [B, H, T, d], device, 16-byte aligned; rounded to nearest even
 *   delta    [out] fp32 [B, H, T], device, 4-byte aligned: D_i = dO_i . O_i (written, then read by
 *                  the second kernel; its content after the call is that value)
 *   B, H, T, causal, scale, stream: as for fa_fwd (o and lse must come from fa_fwd with the same
 *   q, k, causal and scale)
 *   d        head dimension: 64 or 128
 * The outputs dq, dk, dv and delta must not overlap each other or any input. The kernels run in
 * order on `stream`: dQ and D, then dK and dV (at d = 128 one pass for dV and one for dK); no
 * atomics, no allocation.
 * Returns FA_OK or a negative fa_status (checked before anything is launched).
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dout, void* dq, void* dk, void* dv, float* delta, int B, int H, int T, int d,
           int causal, float scale, void* stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* fa_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
