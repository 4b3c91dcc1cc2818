// Exact attention forward on FP8 inputs for gfx950: Q, K, V as OCP FP8 E4M3 codes with per-tensor
// descale factors, both matrix products on the FP8 MFMA, online softmax in fp32, bf16 output and
// fp32 logsumexp.
//
// Method: the same tiled forward as fa_kernel.hpp (one workgroup per Q block of a head walking the
// K/V tiles, running max and sum in base 2, one division at the end, causal tiles above the
// diagonal never loaded, learn-llm.fim.ai "手写 FlashAttention：拆开 SDPA 这个黑盒", STEP 2-4), with
// the matrix work in the low-precision mode that doubles the matrix throughput (cnblogs
// "内核案例研究：Flash Attention", the closing section on its third version: FP8 on newer GPUs).
//   - scores: S^T = K Q^T on v_mfma_f32_32x32x64_f8f6f4 (E4M3 x E4M3, fp32 accumulation), then
//     multiplied by scale * q_descale * k_descale * log2(e) inside the exp2 argument;
//   - probabilities: p = exp2(s - m + 8) in fp32, so the largest weight of a row is exactly 2^8 and
//     the small ones stay clear of the E4M3 subnormal range; l sums the fp32 p; P is rounded to
//     E4M3 (round to nearest even) for the second product, the one rounding this path adds;
//   - output: O^T += V^T P^T on the same MFMA; at the end O = acc * v_descale / l, rounded once to
//     bf16, and LSE = ln 2 * (m + log2 l - 8).
//   - one score set per wave (the scores, softmax and P.V of a tile in turn): the kernel is bound by
//     the softmax's VALU work, so it keeps registers low (116 VGPRs at d = 64: four waves per SIMD,
//     164 at d = 128: three) and lets the resident waves overlap each other, rather than holding a
//     second score set to overlap the next tile's scores inside a wave (182 VGPRs, two waves).
//
// gfx950 mapping (measured on the device with one-off probes):
//   - v_mfma_f32_32x32x64_f8f6f4 (OCP E4M3 when both format fields are 0): lane l holds 32 bytes of
//     A row l%32 and 32 bytes of B column l%32; A byte i of lane l and B byte i of lane l' meet in
//     the same product term whenever l/32 = l'/32, so a consistent assignment of the 64 k-values to
//     (half, byte) pairs on both sides is all the layout needs. C is laid out as for the bf16 MFMA:
//     column l%32, rows 8*(r/4) + 4*(l/32) + r%4 for register r.
//   - ds_read_b64_tr_b8: within each group of 16 lanes, output lane i byte e is byte i%8 of the
//     8 bytes that source lane 2e + i/8 addresses, an 8 x 8 byte transpose per half group.
//   - v_cvt_pk_fp8_f32 rounds to nearest even (OCP E4M3); the first operand lands in byte 0.
#pragma once

#include "fa_kernel.hpp"

namespace fa {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

template <int D_, bool CAUSAL_>
struct Fp8Cfg {
  static constexpr int D = D_;
  static constexpr bool CAUSAL = CAUSAL_;
  static constexpr int NW = 4;                      // waves per workgroup, 32 queries each
  static constexpr int BM = 32 * NW;                // queries per workgroup
  static constexpr int BN = 64;                     // keys per K/V tile
  static constexpr int THREADS = 64 * NW;
  static constexpr int NSTAGE = 2;                  // buffers per ring (K ring, V ring)
  static constexpr int ROW_BYTES = D;               // one E4M3 row of K or V
  static constexpr int CHUNKS = D / 16;             // 16-byte chunks per row
  static constexpr int TILE_BYTES = BN * ROW_BYTES;
  static constexpr int VRING = NSTAGE * TILE_BYTES;
  static constexpr int LDS_BYTES = 2 * VRING;
  static constexpr int LOADS = TILE_BYTES / (16 * THREADS);  // 16-byte copies per lane per tile
  static constexpr int KSTEPS = D / 64;             // k-steps of the score MFMA
  static constexpr int KB = BN / 32;                // 32-key blocks per tile
  static constexpr int CB = D / 32;                 // 32-channel blocks of the output
  static_assert(D == 64 || D == 128, "head dim");
  static_assert(LOADS >= 1 && LOADS * 16 * THREADS == TILE_BYTES, "tile load split");
};

constexpr float kFp8PShift = 8.0f;  // P = exp2(s - m + 8): the largest weight of a row is 2^8

// Physical 16-byte chunk of logical chunk c in LDS row r (an XOR involution). Chosen with a CPU
// model of the 64 banks so that the K reads (16 consecutive rows at one chunk per 16-lane pass) and
// the transposing V reads (8 rows x 2 chunks per 32-lane pass) hit distinct banks.
template <int D>
__device__ __forceinline__ int swz8(int r, int c) {
  if constexpr (D == 64) {
    return c ^ ((r >> 2) & 3);
  } else {
    const int x = (r >> 1) & 7;
    return c ^ (((x & 1) << 1) | ((x >> 1) & 1) | (x & 4));
  }
}

__device__ __forceinline__ f32x16 mfma_e4m3(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

template <class C>
__global__ __launch_bounds__(C::THREADS) void fa_fwd_fp8_kernel(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ k, const uint8_t* __restrict__ v,
    __bf16* __restrict__ o, float* __restrict__ lse, int T, int nq, int BH, float scale_log2,
    float v_descale, int head_group) {
  constexpr int D = C::D, NW = C::NW, BN = C::BN, BM = C::BM, RB = C::ROW_BYTES;
  constexpr int KB = C::KB, CB = C::CB, KS = C::KSTEPS;
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31;   // query column of this lane (scores), or A row (fragments)
  const int hf = lane >> 5;  // half of the wave

  const int bid = block_index((int64_t)nq * BH);
  if (bid < 0) return;
  int qblk, bh;
  map_block<C::CAUSAL>(bid, nq, BH, head_group, qblk, bh);
  const int q0 = qblk * BM;
  const int64_t head_off = (int64_t)bh * T * D;  // elements (= bytes of the E4M3 tensors)
  const char* kg = reinterpret_cast<const char*>(k + head_off);
  const char* vg = reinterpret_cast<const char*>(v + head_off);
  const int qw0 = q0 + 32 * w;

  const int kv_end = C::CAUSAL ? min(q0 + BM, T) : T;
  const int n_tiles = (kv_end + BN - 1) / BN;  // at least 1: q0 < T
  const int last_tile = n_tiles - 1;
  const bool tail_ragged = (last_tile + 1) * BN > T;

  // ---- HBM -> LDS copies: lane `lane` of copy i fills 16 bytes of the 1 KiB LDS region
  // (i*NW + w) and fetches the logical chunk the swizzle puts there; rows past T are clamped.
  int dma_row[C::LOADS], dma_col[C::LOADS];
  uint32_t dma_off[C::LOADS];
#pragma unroll
  for (int i = 0; i < C::LOADS; ++i) {
    const int lofs = (i * NW + w) * 1024 + lane * 16;
    dma_row[i] = lofs / RB;
    dma_col[i] = swz8<D>(dma_row[i], (lofs % RB) >> 4) * 16;
    dma_off[i] = (uint32_t)(dma_row[i] * RB + dma_col[i]);
  }
  auto dma = [&](const char* g, int tile, int buf_off) {
    const int kt0 = tile * BN;
    if (kt0 + BN <= T) {
      const char* gt = g + (size_t)kt0 * RB;
#pragma unroll
      for (int i = 0; i < C::LOADS; ++i) lds_copy16(gt, dma_off[i], lds0 + buf_off + (i * NW + w) * 1024);
    } else {
      int first = kt0, last = T - 1;
      asm volatile("" : "+s"(first), "+s"(last));
#pragma unroll
      for (int i = 0; i < C::LOADS; ++i) {
        const uint32_t gofs = (uint32_t)(min(first + dma_row[i], last) * RB + dma_col[i]);
        lds_copy16(g + gofs, lds0 + buf_off + (i * NW + w) * 1024);
      }
    }
  };
  // V rows at or past T of a ragged last tile are zeroed (their weights are 0 already).
  auto zero_v_tail = [&](int buf_off) {
    const int first = T - last_tile * BN;
    char* vl = smem + buf_off;
    for (int idx = tid; idx < (BN - first) * C::CHUNKS; idx += C::THREADS) {
      const int r = first + idx / C::CHUNKS;
      *reinterpret_cast<u32x4*>(vl + r * RB + (idx % C::CHUNKS) * 16) = u32x4{0u, 0u, 0u, 0u};
    }
  };

  dma(kg, 0, 0);
  dma(vg, 0, C::VRING);

  // ---- Q fragments (B operand of S^T = K Q^T): lane (n, hf) holds query qw0 + n, channels
  // 64*s + 32*hf .. +31 of k-step s.
  i32x8 qf[KS];
  {
    const int row = min(qw0 + n, T - 1);
    const i32x4* src = reinterpret_cast<const i32x4*>(q + head_off + (int64_t)row * D);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const i32x4 a = src[4 * s + 2 * hf], b = src[4 * s + 2 * hf + 1];
      qf[s] = i32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    }
  }
  // ---- fragment addresses. K (A of S^T): lane (n, hf) of key block kb reads row 32*kb + n,
  // channels 64*s + 32*hf .. +31 (two chunks). V^T (A of O^T): the lane supplies output channel
  // 32*cb + 16*(g%2) + i for g = lane/16, i = lane%16, at the 32 keys of the P^T bytes of its
  // half hf: byte 8*rd + e is key 16*rd + 8*(e/4) + 4*hf + e%4 (P^T byte b of lane (n, hf) is score
  // register b%16 of key block b/16). Each of the four transposing reads rd takes as source
  // address row 16*rd + 8*(e/4) + 4*(g/2) + e%4, chunk 2*cb + g%2, byte 8*(i%2), e = i/2.
  int k_off[KS][2];
#pragma unroll
  for (int s = 0; s < KS; ++s)
#pragma unroll
    for (int x = 0; x < 2; ++x) k_off[s][x] = n * RB + swz8<D>(n, 4 * s + 2 * hf + x) * 16;
  int v_off[CB];
  {
    const int g = lane >> 4, si = lane & 15;
    const int e = si >> 1, b = si & 1;
    const int row0 = 8 * (e >> 2) + 4 * (g >> 1) + (e & 3);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) v_off[cb] = row0 * RB + swz8<D>(row0, 2 * cb + (g & 1)) * 16 + 8 * b;
  }
  auto read_k = [&](int buf_off, int kb, int s) {
    const char* p = smem + buf_off + kb * 32 * RB;
    const i32x4 a = *reinterpret_cast<const i32x4*>(p + k_off[s][0]);
    const i32x4 b = *reinterpret_cast<const i32x4*>(p + k_off[s][1]);
    return i32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  };
  auto read_v = [&](int buf_off, int cb) {
    i32x2 r[4];
#pragma unroll
    for (int rd = 0; rd < 4; ++rd)
      r[rd] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(smem + buf_off + rd * 16 * RB + v_off[cb]));
    return i32x8{r[0][0], r[0][1], r[1][0], r[1][1], r[2][0], r[2][1], r[3][0], r[3][1]};
  };

  f32x16 acc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) acc[cb] = f32x16{};
  float m_run = kSparseMaxFloor, l_run = 0.0f;


  auto scores = [&](int KR, f32x16 (&s_out)[KB]) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int s = 0; s < KS; ++s) s_out[kb] = mfma_e4m3(read_k(KR, kb, s), qf[s], s == 0 ? f32x16{} : s_out[kb]);
  };
  // key of score register r of key block kb: kt0 + 32*kb + 8*(r/4) + 4*hf + r%4
  auto mask_tile = [&](f32x16 (&s)[KB], int tile) {
    const int kt0 = tile * BN;
    const int qi = qw0 + n;
    const int last = C::CAUSAL ? min(qi, T - 1) : T - 1;
    const int bound = last - kt0 - 4 * hf;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int off = 32 * kb + 8 * (r >> 2) + (r & 3);
        s[kb][r] = off <= bound ? s[kb][r] : -__builtin_inff();
      }
  };
  auto needs_mask = [&](int tile) {
    const int kt0 = tile * BN;
    return (C::CAUSAL && kt0 + BN - 1 > qw0) || (kt0 + BN > T);
  };
  auto row_max = [&](f32x16 (&s)[KB]) {
    float mx = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    return wave_max_halves(mx) * scale_log2;
  };
  // softmax of one tile into E4M3 P^T (byte 16*kb + r is register r of key block kb) and its sum
  auto softmax_pack = [&](f32x16 (&s)[KB], i32x8& pf) {
    const float neg_m = kFp8PShift - m_run;
    float lsum = 0.0f;
#pragma unroll
    for (int wd = 0; wd < 8; ++wd) {
      const int kb = wd >> 2, r = 4 * (wd & 3);
      float p[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        p[x] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r + x], scale_log2, neg_m));
        lsum += p[x];
      }
      int word = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
      word = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], word, true);
      pf[wd] = word;
    }
    return lsum;
  };
  auto pv = [&](int VR, const i32x8& pf) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[cb] = mfma_e4m3(read_v(VR, cb), pf, acc[cb]);
  };

  // ---- one K/V tile per step: its scores, the online softmax and P.V. One score set only, so
  // that more waves fit on a SIMD; the copies of tile j+1 run during step j.
  vmem_wait<0>();
  __syncthreads();
  if (tail_ragged && n_tiles == 1) {
    zero_v_tail(C::VRING);
    __syncthreads();
  }
  for (int j = 0; j < n_tiles; ++j) {
    const int buf = j & 1;
    if (j + 1 < n_tiles) {
      dma(kg, j + 1, (buf ^ 1) * C::TILE_BYTES);
      dma(vg, j + 1, C::VRING + (buf ^ 1) * C::TILE_BYTES);
    }
    f32x16 s[KB];
    scores(buf * C::TILE_BYTES, s);
    if (needs_mask(j)) mask_tile(s, j);
    const float m_new = max_f32(m_run, row_max(s));
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    i32x8 pf;
    l_run = l_run * alpha + softmax_pack(s, pf);
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) acc[cb] *= alpha;
    }
    pv(C::VRING + buf * C::TILE_BYTES, pf);
    vmem_wait<0>();
    __syncthreads();
    if (tail_ragged && j + 2 == n_tiles) {  // V(n-1) just landed
      zero_v_tail(C::VRING + ((j + 1) & 1) * C::TILE_BYTES);
      __syncthreads();
    }
  }

  // ---- epilogue: O = acc * v_descale / l (the 2^8 of P cancels against l), rounded to bf16;
  // LSE = ln 2 * (m + log2 l - 8). Lane (n, hf) holds channels 32*cb + 8*a + 4*hf + 0..3 in
  // registers 4*a .. 4*a+3.
  const int row = qw0 + n;
  const float l_tot = wave_sum_halves(l_run);
  const float f = v_descale / l_tot;
  if (row < T) {
    char* orow = reinterpret_cast<char*>(o + head_off + (int64_t)row * D);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        u32x2 out;
        out[0] = pack_bf16x2(acc[cb][4 * a] * f, acc[cb][4 * a + 1] * f);
        out[1] = pack_bf16x2(acc[cb][4 * a + 2] * f, acc[cb][4 * a + 3] * f);
        *reinterpret_cast<u32x2*>(orow + (32 * cb + 8 * a + 4 * hf) * 2) = out;
      }
    if (hf == 0) lse[(int64_t)bh * T + row] = (m_run + __log2f(l_tot) - kFp8PShift) * kLn2;
  }
}

}  // namespace fa
