// Test infrastructure: measures the accuracy of the bf16 matrix instruction that the forward uses
// (v_mfma_f32_32x32x16_bf16, chained over k in one fp32 accumulator as the kernel chains it over
// the head dimension for the scores and over the keys for P V), so that the bf16 forward's derived
// error bound can rest on a measurement that runs with the tests.
//
//   bf16_mfma_probe(a, b, c, n, k, stream): for g < n, c[g] = A[g] B[g]^T with A[g], B[g] 32 x k bf16
//   (row-major, k a multiple of 16 in [16, 16384]) and c[g] 32 x 32 fp32 (row-major, c[g][i][j] =
//   sum_k A[g][i][k] B[g][j][k]), accumulated by k / 16 MFMAs in order of k. Device pointers, 16-byte
//   aligned; a and b hold n * 32 * k bf16 each, c n * 1024 floats. One 64-lane workgroup per g.
//   Returns 0, -1 for a bad argument (nothing launched) or -5 for a failed launch.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(64) void bf16_mfma_probe_kernel(const __bf16* __restrict__ a,
                                                             const __bf16* __restrict__ b,
                                                             float* __restrict__ c, int n, int k) {
  const int g = blockIdx.x;
  if (g >= n) return;
  const int lane = threadIdx.x;
  // lane l: row (of A) / column (of C, i.e. row of B) l % 32; k-values 16 t + 8 (l / 32) .. + 7
  const int row = lane & 31, half = lane >> 5;
  const __bf16* ar = a + ((int64_t)g * 32 + row) * k + 8 * half;
  const __bf16* br = b + ((int64_t)g * 32 + row) * k + 8 * half;
  f32x16 acc = {};
  for (int t = 0; t < k / 16; ++t) {
    const bf16x8 fa = *reinterpret_cast<const bf16x8*>(ar + 16 * t);
    const bf16x8 fb = *reinterpret_cast<const bf16x8*>(br + 16 * t);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fb, acc, 0, 0, 0);
  }
  float* cg = c + (int64_t)g * 1024;
#pragma unroll
  for (int r = 0; r < 16; ++r) cg[(8 * (r / 4) + 4 * half + r % 4) * 32 + row] = acc[r];
}

}  // namespace

extern "C" int bf16_mfma_probe(const void* a, const void* b, float* c, int n, int k, void* stream) {
  if (!a || !b || !c || n < 1 || n > (1 << 20) || k < 16 || k > 16384 || k % 16 != 0) return -1;
  if (((uintptr_t)a | (uintptr_t)b | (uintptr_t)c) & 15u) return -1;
  hipLaunchKernelGGL(bf16_mfma_probe_kernel, dim3(n), dim3(64), 0, (hipStream_t)stream,
                     (const __bf16*)a, (const __bf16*)b, c, n, k);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}
