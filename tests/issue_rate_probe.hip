// Test infrastructure: issue rates of the instructions the forward kernel's inner loop is made of,
// measured on the device, for the per-tile cycle budget of the d = 64 forward.
//
//   issue_rate_probe(mode, waves_per_simd, iters, out_cycles): launches one workgroup of
//   64 * 4 * waves_per_simd threads on each of 256 compute units; every wave runs `iters` iterations
//   of the mode's instruction mix between two reads of the shader cycle counter. *out_cycles gets the
//   mean over workgroups of the slowest wave's elapsed cycles (the SIMD's time: waves of one SIMD
//   do not finish together, since the matrix unit serves the oldest waiting wave first).
//   Returns 0, -1 for a bad argument (nothing launched), -5 for a HIP error.
// Modes (per iteration of one wave):
//   0: 16 v_fma_f32         1: 16 v_exp_f32        2: 16 v_add_f32        3: 16 v_max3_f32
//   4: 16 v_cvt_pk_bf16_f32 5: 4 MFMA 32x32x16 bf16
//   6: 4 MFMA + the softmax mix of the forward for 4 MFMAs at d = 64 (37 VALU: 8.25 exp, 8 fma,
//      8 add, 4 max3, 4 cvt_pk, the rest multiplies)
//   7: mode 6 plus 6 LDS 16-byte reads feeding the MFMAs (the forward's 1.5 fragment reads per MFMA)
//   8: mode 6 plus 3 LDS reads, each fragment feeding two MFMAs (64 queries per wave)
//   9: half the waves only the 4 MFMAs, half only the 37 VALU (a two-role split of the same work)
//  10: the 37 VALU of mode 6 alone
//  11: 16 v_cvt_pk_fp8_f32 (the FP8 forward's conversion of the weights)
//  12: mode 6's 128 MFMA cycles as 2 MFMA 32x32x64 f8f6f4 (half the instructions) + the 37 VALU
//  13: mode 6's flops as 8 MFMA 16x16x32 bf16 (twice the instructions) + the 37 VALU
//  14: mode 6 with the matrix accumulators in AGPRs (the other modes keep them in VGPRs)
//  15: 2 MFMA 32x32x64 f8f6f4
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Register-to-register ALU instructions only (no memory access, no scalar stores).
#define P_FMA(r) asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(r) : "v"(x1), "v"(x2))
#define P_EXP(r) asm volatile("v_exp_f32 %0, %0" : "+v"(r))
#define P_MAX3(r) asm volatile("v_max3_f32 %0, %0, %1, %2" : "+v"(r) : "v"(x1), "v"(x2))
#define P_CVT(r) asm volatile("v_cvt_pk_bf16_f32 %0, %0, %1" : "+v"(r) : "v"(x1))
#define P_ADD(r) asm volatile("v_add_f32 %0, %0, %1" : "+v"(r) : "v"(x1))
#define P_MUL(r) asm volatile("v_mul_f32 %0, %0, %1" : "+v"(r) : "v"(x3))
#define P_MIX_A P_EXP(a0); P_FMA(a1); P_ADD(a2); P_EXP(a3); P_FMA(a4); P_ADD(a5); P_MAX3(a6); P_CVT(a7); P_FMA(a0); P_MUL(a1)
#define P_MIX_B P_EXP(a6); P_FMA(a7); P_ADD(a0); P_EXP(a1); P_FMA(a2); P_ADD(a3); P_MAX3(a4); P_CVT(a5); P_ADD(a6)
#define P_MIX_C P_EXP(a4); P_FMA(a5); P_ADD(a6); P_EXP(a7); P_FMA(a0); P_ADD(a1); P_MAX3(a2); P_CVT(a3); P_FMA(a4); P_MUL(a5)
#define P_MIX_D P_EXP(a2); P_FMA(a3); P_ADD(a4); P_EXP(a5); P_FMA(a6); P_ADD(a7); P_MAX3(a0); P_CVT(a1); P_MUL(a2)
#define P_MFMA(c, a, b) c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0)
#define P_MFMA16(c) c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, c, 0, 0, 0)
#define P_MFMA8(c) c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(I8, I8, c, 0, 0, 0, 0, 0, 0)
#define P_CVT8(r) asm volatile("v_cvt_pk_fp8_f32 %0, %0, %1" : "+v"(r) : "v"(x1))

template <int MODE>
__global__ __launch_bounds__(1024) void issue_rate_kernel(uint64_t* out, int iters, float seed) {
  float a0 = seed, a1 = seed + 1, a2 = seed + 2, a3 = seed + 3, a4 = seed + 4, a5 = seed + 5,
        a6 = seed + 6, a7 = seed + 7;
  float x1 = 0.999f, x2 = 1e-7f, x3 = 1.0001f;
  // An (empty) use of an AGPR makes the compiler keep this instance's MFMA accumulators in AGPRs.
  if constexpr (MODE == 14) asm volatile("" ::: "a0");
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  f32x4 d0 = {}, d1 = {}, d2 = {}, d3 = {}, d4 = {}, d5 = {}, d6 = {}, d7 = {};
  bf16x8 A, B;
  i32x8 I8;  // E4M3 codes 0x38..0x3f (1.0 .. 1.875)
  for (int i = 0; i < 8; ++i) I8[i] = 0x38383838 + 0x01010101 * i;
  for (int i = 0; i < 8; ++i) {
    A[i] = (__bf16)(seed * i);
    B[i] = (__bf16)(seed + i);
  }
  __shared__ bf16x8 lds[512];  // 8 KiB; every index below is taken modulo 512
  for (int i = threadIdx.x; i < 512; i += blockDim.x) {
    bf16x8 t;
    for (int e = 0; e < 8; ++e) t[e] = (__bf16)(0.001f * (i + e));
    lds[i] = t;
  }
  const int lane = threadIdx.x & 63;
  const bool mfma_role = ((threadIdx.x >> 6) / 4) % 2 == 1;  // mode 9: waves 4..7, 12..15 of the group
  __syncthreads();
  const uint64_t t0 = __builtin_readcyclecounter();
  for (int it = 0; it < iters; ++it) {
    if constexpr (MODE == 0) {
      P_FMA(a0); P_FMA(a1); P_FMA(a2); P_FMA(a3); P_FMA(a4); P_FMA(a5); P_FMA(a6); P_FMA(a7);
      P_FMA(a0); P_FMA(a1); P_FMA(a2); P_FMA(a3); P_FMA(a4); P_FMA(a5); P_FMA(a6); P_FMA(a7);
    } else if constexpr (MODE == 1) {
      P_EXP(a0); P_EXP(a1); P_EXP(a2); P_EXP(a3); P_EXP(a4); P_EXP(a5); P_EXP(a6); P_EXP(a7);
      P_EXP(a0); P_EXP(a1); P_EXP(a2); P_EXP(a3); P_EXP(a4); P_EXP(a5); P_EXP(a6); P_EXP(a7);
    } else if constexpr (MODE == 2) {
      P_ADD(a0); P_ADD(a1); P_ADD(a2); P_ADD(a3); P_ADD(a4); P_ADD(a5); P_ADD(a6); P_ADD(a7);
      P_ADD(a0); P_ADD(a1); P_ADD(a2); P_ADD(a3); P_ADD(a4); P_ADD(a5); P_ADD(a6); P_ADD(a7);
    } else if constexpr (MODE == 3) {
      P_MAX3(a0); P_MAX3(a1); P_MAX3(a2); P_MAX3(a3); P_MAX3(a4); P_MAX3(a5); P_MAX3(a6); P_MAX3(a7);
      P_MAX3(a0); P_MAX3(a1); P_MAX3(a2); P_MAX3(a3); P_MAX3(a4); P_MAX3(a5); P_MAX3(a6); P_MAX3(a7);
    } else if constexpr (MODE == 4) {
      P_CVT(a0); P_CVT(a1); P_CVT(a2); P_CVT(a3); P_CVT(a4); P_CVT(a5); P_CVT(a6); P_CVT(a7);
      P_CVT(a0); P_CVT(a1); P_CVT(a2); P_CVT(a3); P_CVT(a4); P_CVT(a5); P_CVT(a6); P_CVT(a7);
    } else if constexpr (MODE == 5) {
      P_MFMA(c0, A, B); P_MFMA(c1, A, B); P_MFMA(c2, A, B); P_MFMA(c3, A, B);
    } else if constexpr (MODE == 6 || MODE == 7 || MODE == 14) {
      bf16x8 A0 = A, A1 = A, A2 = A, A3 = A;
      if constexpr (MODE == 7) {
        const int base = (it * 6 + lane) & 511;
        A0 = lds[base]; A1 = lds[(base + 64) & 511]; A2 = lds[(base + 128) & 511];
        A3 = lds[(base + 192) & 511];
        const bf16x8 e0 = lds[(base + 256) & 511], e1 = lds[(base + 320) & 511];
        A0[0] = A0[0] + e0[1];
        A1[0] = A1[0] + e1[1];
      }
      P_MFMA(c0, A0, B); P_MIX_A;
      P_MFMA(c1, A1, B); P_MIX_B;
      P_MFMA(c2, A2, B); P_MIX_C;
      P_MFMA(c3, A3, B); P_MIX_D;
    } else if constexpr (MODE == 8) {
      const int base = (it * 3 + lane) & 511;
      bf16x8 A0 = lds[base], A1 = lds[(base + 64) & 511];
      const bf16x8 e0 = lds[(base + 256) & 511];
      A0[0] = A0[0] + e0[1];
      P_MFMA(c0, A0, B); P_MIX_A;
      P_MFMA(c1, A0, A); P_MIX_B;
      P_MFMA(c2, A1, B); P_MIX_C;
      P_MFMA(c3, A1, A); P_MIX_D;
    } else if constexpr (MODE == 9) {
      if (mfma_role) {
        P_MFMA(c0, A, B); P_MFMA(c1, A, B); P_MFMA(c2, A, B); P_MFMA(c3, A, B);
      } else {
        P_MIX_A; P_MIX_B; P_MIX_C; P_MIX_D;
      }
    } else if constexpr (MODE == 10) {
      P_MIX_A; P_MIX_B; P_MIX_C; P_MIX_D;
    } else if constexpr (MODE == 11) {
      P_CVT8(a0); P_CVT8(a1); P_CVT8(a2); P_CVT8(a3); P_CVT8(a4); P_CVT8(a5); P_CVT8(a6); P_CVT8(a7);
      P_CVT8(a0); P_CVT8(a1); P_CVT8(a2); P_CVT8(a3); P_CVT8(a4); P_CVT8(a5); P_CVT8(a6); P_CVT8(a7);
    } else if constexpr (MODE == 12) {
      P_MFMA8(c0); P_MIX_A; P_MIX_B;
      P_MFMA8(c1); P_MIX_C; P_MIX_D;
    } else if constexpr (MODE == 13) {
      P_MFMA16(d0); P_MIX_A; P_MFMA16(d1);
      P_MFMA16(d2); P_MIX_B; P_MFMA16(d3);
      P_MFMA16(d4); P_MIX_C; P_MFMA16(d5);
      P_MFMA16(d6); P_MIX_D; P_MFMA16(d7);
    } else if constexpr (MODE == 15) {
      P_MFMA8(c0); P_MFMA8(c1);
    }
  }
  const uint64_t t1 = __builtin_readcyclecounter();
  float s = a0 + a1 + a2 + a3 + a4 + a5 + a6 + a7;
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  for (int i = 0; i < 4; ++i) s += d0[i] + d1[i] + d2[i] + d3[i] + d4[i] + d5[i] + d6[i] + d7[i];
  const int wave = threadIdx.x >> 6;  // < 16
  if (lane == 0) out[blockIdx.x * 16 + wave] = (t1 - t0) + (s == 12345.0f ? 1 : 0);
}

using ProbeFn = void (*)(uint64_t*, int, float);
const ProbeFn kModes[] = {issue_rate_kernel<0>, issue_rate_kernel<1>, issue_rate_kernel<2>,
                          issue_rate_kernel<3>, issue_rate_kernel<4>, issue_rate_kernel<5>,
                          issue_rate_kernel<6>, issue_rate_kernel<7>, issue_rate_kernel<8>,
                          issue_rate_kernel<9>,  issue_rate_kernel<10>, issue_rate_kernel<11>,
                          issue_rate_kernel<12>, issue_rate_kernel<13>, issue_rate_kernel<14>,
                          issue_rate_kernel<15>};

}  // namespace

extern "C" int issue_rate_probe(int mode, int waves_per_simd, int iters, double* out_cycles) {
  if (mode < 0 || mode > 15 || waves_per_simd < 1 || waves_per_simd > 4 || iters < 1 ||
      iters > (1 << 20) || !out_cycles)
    return -1;
  if (mode == 9 && waves_per_simd % 2 != 0) return -1;
  uint64_t* d = nullptr;
  const size_t n = 256 * 16;
  if (hipMalloc(&d, n * sizeof(uint64_t)) != hipSuccess) return -5;
  hipLaunchKernelGGL(kModes[mode], dim3(256), dim3(256 * waves_per_simd), 0, 0, d, iters, 0.5f);
  uint64_t h[256 * 16];
  hipError_t e = hipMemcpy(h, d, sizeof(h), hipMemcpyDeviceToHost);  // waits for the kernel
  if (hipFree(d) != hipSuccess || e != hipSuccess) return -5;
  double sum = 0.0;
  for (int b = 0; b < 256; ++b) {
    uint64_t mx = 0;
    for (int w = 0; w < 4 * waves_per_simd; ++w) mx = h[b * 16 + w] > mx ? h[b * 16 + w] : mx;
    sum += (double)mx;
  }
  *out_cycles = sum / 256.0;
  return 0;
}
