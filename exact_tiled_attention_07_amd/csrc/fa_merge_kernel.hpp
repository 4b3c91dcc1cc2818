// Log-space merge of partial attention results over disjoint key ranges (the split-KV combine).
//
// For a row with partial results (O_s, LSE_s) over disjoint key ranges s, the attention over the
// union is LSE = log sum_s exp(LSE_s) and O = sum_s exp(LSE_s - LSE) O_s: the logsumexp combine of
// partial blocks in log space (ijyty.com FlashAttention article, section 2.1, the per-block lse
// accumulation and the final division by exp(lse)). A part with LSE_s = -inf (no visible key)
// contributes nothing; a row whose parts are all -inf gets O = 0 and LSE = -inf.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// One thread per 4 channels of a row: D/4 threads per row, 256 / (D/4) rows per workgroup. The
// kernel is bound by HBM traffic (every part's O row is read once) or, for few rows, by the latency
// of its loads: each chunk of up to U parts is loaded with all its loads in flight together, and the
// chunks are combined with a running maximum (what earlier chunks accumulated is rescaled by
// exp(m_old - m_new) when a later chunk raises it). With at most U parts there is a single chunk
// and the result is that of the two-pass form: the weights exp(LSE_s - max_s LSE_s) summed in part
// order.
template <int D>
__global__ __launch_bounds__(256) void fa_merge_kernel(const float* __restrict__ o_parts,
                                                       const float* __restrict__ lse_parts,
                                                       int n_parts, __bf16* __restrict__ o,
                                                       float* __restrict__ lse, int64_t rows) {
  constexpr int TPR = D / 4;
  constexpr int RPB = 256 / TPR;
  constexpr int U = 16;  // parts per chunk of loads
  // a long grid is folded into x and z (32-bit work-item counts per dimension)
  const int64_t row = ((int64_t)blockIdx.z * gridDim.x + blockIdx.x) * RPB + threadIdx.x / TPR;
  const int c4 = threadIdx.x % TPR;
  if (row >= rows) return;
  const float* lp = lse_parts + row;
  const float* op = o_parts + row * D + 4 * c4;
  const int64_t lstride = rows, ostride = rows * D;
  float m = -__builtin_inff();  // largest part LSE so far
  float l = 0.0f;               // sum of exp(LSE_s - m) so far
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int s = 0; s < n_parts; s += U) {
    float ls[U];
    float4 xs[U];
#pragma unroll
    for (int e = 0; e < U; ++e) {
      if (s + e < n_parts) {  // n_parts is the same for every lane: a uniform branch
        ls[e] = lp[(s + e) * lstride];
        xs[e] = *reinterpret_cast<const float4*>(op + (s + e) * ostride);
      } else {
        ls[e] = -__builtin_inff();
        xs[e] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      }
    }
    float mc = m;
#pragma unroll
    for (int e = 0; e < U; ++e) mc = fmaxf(mc, ls[e]);
    if (mc > -__builtin_inff()) {
      const float r = expf(m - mc);  // 0 while nothing was seen (m = -inf), 1 if m is unchanged
      l *= r;
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] *= r;
#pragma unroll
      for (int e = 0; e < U; ++e) {
        const float wgt = expf(ls[e] - mc);  // 0 for an empty part (LSE_s = -inf)
        l += wgt;
        acc[0] += wgt * xs[e].x;
        acc[1] += wgt * xs[e].y;
        acc[2] += wgt * xs[e].z;
        acc[3] += wgt * xs[e].w;
      }
      m = mc;
    }
  }
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  bf16x4 out;
#pragma unroll
  for (int e = 0; e < 4; ++e) out[e] = (__bf16)(acc[e] * inv);  // round to nearest even
  *reinterpret_cast<bf16x4*>(o + row * D + 4 * c4) = out;
  if (c4 == 0) lse[row] = l > 0.0f ? m + logf(l) : -__builtin_inff();
}

}  // namespace fa
