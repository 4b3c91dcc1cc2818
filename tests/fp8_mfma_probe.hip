// Test infrastructure: measures the accuracy of the FP8 matrix instruction that fa_fwd_fp8 uses
// (v_mfma_f32_32x32x64_f8f6f4 on OCP E4M3 operands, through the kernel's own mfma_e4m3), so the
// FP8 forward's tolerance can rest on a measurement that runs with the tests.
//
//   fp8_mfma_probe(a, b, c, n, stream): for g < n, c[g] = A[g] B[g]^T with A[g], B[g] 32 x 64 E4M3
//   codes (row-major, 64 bytes per row) and c[g] 32 x 32 fp32 (row-major, c[g][i][j] = sum_k
//   A[g][i][k] B[g][j][k]). Device pointers; a and b n * 2048 bytes, c n * 4096 bytes, 16-byte
//   aligned. One 64-lane workgroup per g. Returns 0, -1 for a bad argument (nothing launched) or -5
//   for a failed launch.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_fp8_kernel.hpp"

namespace {

__global__ __launch_bounds__(64) void fp8_mfma_probe_kernel(const uint8_t* __restrict__ a,
                                                            const uint8_t* __restrict__ b,
                                                            float* __restrict__ c, int n) {
  const int g = blockIdx.x;
  if (g >= n) return;
  const int lane = threadIdx.x;
  // lane l: row (of A) / column (of C, i.e. row of B) l % 32, k-values 32 * (l / 32) .. +31
  const int row = lane & 31, half = lane >> 5;
  const fa::i32x8 fa_ = *reinterpret_cast<const fa::i32x8*>(a + (int64_t)g * 2048 + row * 64 + 32 * half);
  const fa::i32x8 fb = *reinterpret_cast<const fa::i32x8*>(b + (int64_t)g * 2048 + row * 64 + 32 * half);
  // S^T layout of the kernel: the first operand gives the output row, the second its column
  const fa::f32x16 acc = fa::mfma_e4m3(fa_, fb, fa::f32x16{});
  float* cg = c + (int64_t)g * 1024;
#pragma unroll
  for (int r = 0; r < 16; ++r) cg[(8 * (r / 4) + 4 * half + r % 4) * 32 + row] = acc[r];
}

}  // namespace

extern "C" int fp8_mfma_probe(const void* a, const void* b, float* c, int n, void* stream) {
  if (!a || !b || !c || n < 1 || n > (1 << 20)) return -1;
  if (((uintptr_t)a | (uintptr_t)b | (uintptr_t)c) & 15u) return -1;
  hipLaunchKernelGGL(fp8_mfma_probe_kernel, dim3(n), dim3(64), 0, (hipStream_t)stream,
                     (const uint8_t*)a, (const uint8_t*)b, c, n);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}
