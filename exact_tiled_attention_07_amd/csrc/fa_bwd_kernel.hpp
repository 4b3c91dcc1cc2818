// Exact attention backward for gfx950 (CDNA4), d = 64 and 128: dQ, dK and dV of O = softmax(scale Q K^T) V
// from the saved per-row logsumexp, by recomputing the probabilities block by block.
//
// Method (what is computed and in which order):
//   - the forward kept only O and the row logsumexp; the backward recomputes the scores and the
//     probabilities P = exp(scale q.k - LSE) per block instead of storing the T x T matrix
//     (learn-llm.fim.ai "手写 FlashAttention：拆开 SDPA 这个黑盒", STEP 4, the note on training;
//     ijyty.com FlashAttention article, section 2.2, the recomputation strategy);
//   - the gradient of the row softmax: dP = dO V^T, D_i = dO_i . O_i, dS = P (dP - D), then
//     dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO;
//   - gradients are accumulated per block (same article, section 2.2); instead of atomic adds into
//     a global dQ, two kernels each own the rows they write: fa_bwd_dq_kernel owns a block of
//     queries and walks the K/V tiles (it also writes D), fa_bwd_dkdv_kernel owns a block of keys
//     and walks the Q/dO tiles. S and dP are computed in both. At d = 128 the second kernel runs as
//     a dV pass and a dK pass (fewer registers, two waves per SIMD), each recomputing S.
//
// gfx950 mapping: the operand layouts, the LDS swizzle, the HBM -> LDS copies and the transposing
// LDS reads are those of the forward kernel (fa_kernel.hpp):
//   - fa_bwd_dq_kernel: lane = query. S^T = K Q^T and dP^T = V dO^T (K and V rows read from LDS as
//     the A operand, Q and dO in registers as B), then dQ^T += K^T dS^T with K^T from transposing
//     reads of the K tile and dS^T packed from the S^T accumulator layout (the forward's P^T path).
//   - fa_bwd_dkdv_kernel: lane = key. S = Q K^T and dP = dO V^T (Q and dO rows from LDS, K and V in
//     registers), then dV^T += dO^T P and dK^T += Q^T dS with transposing reads of the dO and Q
//     tiles. The row statistics (LSE, D) of a Q tile are copied into LDS next to it and read as
//     broadcasts (each half-wave needs the same 16 rows).
#pragma once

#include "fa_kernel.hpp"

namespace fa {

template <int D_, bool CAUSAL_>
struct BwdCfg {
  static constexpr int D = D_;
  static constexpr int NW = 4;                       // waves per workgroup
  static constexpr int THREADS = 64 * NW;
  static constexpr int BM = 32 * NW;                 // rows a workgroup owns (queries or keys)
  static constexpr int BN = 64;                      // rows of a streamed tile
  static constexpr bool CAUSAL = CAUSAL_;
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int TILE_BYTES = BN * ROW_BYTES;  // one streamed tile
  static constexpr int LOADS = TILE_BYTES / (16 * THREADS);
  static constexpr int KSTEPS = D / 16;              // k-steps over channels
  static constexpr int CB = D / 32;                  // 32-channel blocks of an output
  static constexpr int KB = BN / 32;                 // 32-row blocks of a streamed tile
  static constexpr int PT = BN / 16;                 // k-steps over a streamed tile's rows
  static constexpr int STATS_BYTES = 2 * BN * 4;     // LSE and D of a Q tile (dK/dV kernel)
  static constexpr int LDS_BYTES = 4 * TILE_BYTES + 2 * STATS_BYTES;
  static_assert(D == 64 || D == 128, "backward: head dim");
  static_assert(LOADS >= 1 && LOADS * 16 * THREADS == TILE_BYTES, "tile load split");
};

// HBM -> LDS copy of one 4-byte word per lane: LDS [lds_addr + 4*lane] <- global [addr].
__device__ __forceinline__ void lds_copy4(const void* addr, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dword %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_addr), "v"(addr)
      : "memory");
}

// Per-lane placement of the HBM -> LDS copies of one [BN, D] tile (as in the forward): lane `lane`
// of load i fills 16 bytes of the 1 KiB LDS region (i*NW + w) with the logical chunk that the
// swizzle puts there. Rows past T are clamped to row T-1.
template <class C>
struct TileCopier {
  int row[C::LOADS], col[C::LOADS];
  uint32_t off[C::LOADS];
  int w;
  __device__ __forceinline__ void init(int wave, int lane) {
    w = wave;
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int lofs = (i * C::NW + w) * 1024 + lane * 16;
      row[i] = lofs / C::ROW_BYTES;
      col[i] = swz<C::D>(row[i], (lofs % C::ROW_BYTES) >> 4) * 16;
      off[i] = (uint32_t)(row[i] * C::ROW_BYTES + col[i]);
    }
  }
  // rows [t0, t0 + BN) of the [T, D] slab g into the LDS tile at byte address lds_tile
  __device__ __forceinline__ void copy(const char* g, int t0, int T, uint32_t lds_tile) const {
    if (t0 + C::BN <= T) {
      const char* gt = g + (size_t)t0 * C::ROW_BYTES;
#pragma unroll
      for (int i = 0; i < C::LOADS; ++i) lds_copy16(gt, off[i], lds_tile + (i * C::NW + w) * 1024);
    } else {
      int first = t0, last = T - 1;  // through an empty asm: keep the clamping in this branch
      asm volatile("" : "+s"(first), "+s"(last));
#pragma unroll
      for (int i = 0; i < C::LOADS; ++i) {
        const uint32_t gofs = (uint32_t)(min(first + row[i], last) * C::ROW_BYTES + col[i]);
        lds_copy16(g + gofs, lds_tile + (i * C::NW + w) * 1024);
      }
    }
  }
};

// LDS byte offsets of the MFMA fragments of a [BN, D] tile, the same for every tile:
//   row_off[s]: A-operand row fragment (row n of a 32-row block, channels 16*s + 8*hf .. +7);
//   tr_off[cb][rr]: the two transposing reads that give lane l the 8 tile rows of its k-step slots
//   for channel row (cb, l%32) of a transposed operand (the forward's V^T fragment).
template <class C>
struct FragOffsets {
  int row_off[C::KSTEPS];
  int tr_off[C::CB][2];
  __device__ __forceinline__ void init(int lane) {
    constexpr int D = C::D, RB = C::ROW_BYTES;
    const int n = lane & 31, hf = lane >> 5;
#pragma unroll
    for (int s = 0; s < C::KSTEPS; ++s) row_off[s] = n * RB + swz<D>(n, 2 * s + hf) * 16;
    const int grp = lane >> 4, gi = lane & 15;
    const int ga = grp & 1, gh = grp >> 1;
    const int e_src = gi >> 2, q_src = gi & 3;
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb) {
      const int col = (D / 2) * (q_src & 1) + 16 * cb + 4 * (2 * ga + (q_src >> 1));
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        const int r = 4 * gh + e_src + 8 * rr;
        tr_off[cb][rr] = r * RB + swz<D>(r, col >> 3) * 16 + (col & 7) * 2;
      }
    }
  }
};

// Fragments of one global row (this lane's query or key) in the B-operand layout: channels
// 16*s + 8*hf .. +7 for k-step s.
template <int KSTEPS>
__device__ __forceinline__ void load_row_frags(const __bf16* row_ptr, int hf, bf16x8 (&f)[KSTEPS]) {
  const bf16x8* src = reinterpret_cast<const bf16x8*>(row_ptr);
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) f[s] = src[2 * s + hf];
}

// Store a transposed [D, 32] accumulator (rows = channels, column = this lane's row) as bf16 row
// `row` of a [T, D] output, multiplied by mul: lane (n, hf) holds channels (D/2)*hf + 16*cb + r.
template <int CB, int D>
__device__ __forceinline__ void store_rows(__bf16* out_row, const f32x16 (&acc)[CB], int hf, float mul) {
  char* orow = reinterpret_cast<char*>(out_row);
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      u32x4 out;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        out[e] = pack_bf16x2(acc[cb][8 * half + 2 * e] * mul, acc[cb][8 * half + 2 * e + 1] * mul);
      *reinterpret_cast<u32x4*>(orow + ((D / 2) * hf + 16 * cb + 8 * half) * 2) = out;
    }
}

// ---- dQ (and D): one workgroup per (block of BM queries, batch*head); lane = query.
template <class C>
__global__ __launch_bounds__(C::THREADS) void fa_bwd_dq_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ o, const float* __restrict__ lse, const __bf16* __restrict__ dout,
    __bf16* __restrict__ dq, float* __restrict__ delta, int T, int nq, int BH, float scale,
    float scale_log2, int head_group) {
  constexpr int D = C::D, BN = C::BN, BM = C::BM, KB = C::KB, CB = C::CB, PT = C::PT;
  constexpr int KSTEPS = C::KSTEPS, RB = C::ROW_BYTES, TB = C::TILE_BYTES;
  __shared__ __attribute__((aligned(1024))) char smem[4 * TB];  // K ring (2 tiles), V ring (2 tiles)
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, hf = lane >> 5;
  const int bid = block_index((int64_t)nq * BH);
  if (bid < 0) return;
  int qblk, bh;
  map_block<C::CAUSAL>(bid, nq, BH, head_group, qblk, bh);
  const int q0 = qblk * BM;
  const int64_t head_off = (int64_t)bh * T * D;
  const char* kg = reinterpret_cast<const char*>(k + head_off);
  const char* vg = reinterpret_cast<const char*>(v + head_off);
  const int qi = q0 + 32 * w + n;  // this lane's query
  const int row = min(qi, T - 1);
  const int kv_end = C::CAUSAL ? min(q0 + BM, T) : T;
  const int n_tiles = (kv_end + BN - 1) / BN;

  TileCopier<C> cp;
  cp.init(w, lane);
  FragOffsets<C> fo;
  fo.init(lane);
  cp.copy(kg, 0, T, lds0);
  cp.copy(vg, 0, T, lds0 + 2 * TB);

  // Q, dO, O of this lane's query (B-operand layout); D = dO . O (fp32, both wave halves).
  bf16x8 qf[KSTEPS], dof[KSTEPS], of[KSTEPS];
  load_row_frags<KSTEPS>(q + head_off + (int64_t)row * D, hf, qf);
  load_row_frags<KSTEPS>(dout + head_off + (int64_t)row * D, hf, dof);
  load_row_frags<KSTEPS>(o + head_off + (int64_t)row * D, hf, of);
  float dpart = 0.0f;
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) dpart = __builtin_fmaf((float)dof[s][e], (float)of[s][e], dpart);
  const float Drow = wave_sum_halves(dpart);
  if (hf == 0 && qi < T) delta[(int64_t)bh * T + qi] = Drow;
  const float neg_lse2 = -lse[(int64_t)bh * T + row] * kLog2e;

  f32x16 acc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) acc[cb] = f32x16{};

  vmem_wait<0>();
  __syncthreads();

  for (int j = 0; j < n_tiles; ++j) {
    const int buf = j & 1;
    const int KR = buf * TB, VR = (2 + buf) * TB;
    if (j + 1 < n_tiles) {  // the other buffers were last read in step j-1 (closed by its barrier)
      cp.copy(kg, (j + 1) * BN, T, lds0 + (buf ^ 1) * TB);
      cp.copy(vg, (j + 1) * BN, T, lds0 + (2 + (buf ^ 1)) * TB);
    }
    // S^T = K Q^T and dP^T = V dO^T for the tile's two 32-key blocks
    f32x16 s[KB], dp[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      s[kb] = f32x16{};
      dp[kb] = f32x16{};
#pragma unroll
      for (int st = 0; st < KSTEPS; ++st) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(smem + KR + kb * 32 * RB + fo.row_off[st]);
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(smem + VR + kb * 32 * RB + fo.row_off[st]);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[st], s[kb], 0, 0, 0);
        dp[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, dof[st], dp[kb], 0, 0, 0);
      }
    }
    // diagonal or ragged tile: keys past min(query, T-1) get P = 0
    const int kt0 = j * BN;
    if ((C::CAUSAL && kt0 + BN - 1 > q0 + 32 * w) || kt0 + BN > T) {
      const int last = C::CAUSAL ? min(qi, T - 1) : T - 1;
      const int bound = last - kt0 - 4 * hf;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = 32 * kb + 8 * (r >> 2) + (r & 3);
          s[kb][r] = off <= bound ? s[kb][r] : -__builtin_inff();
        }
    }
    // P = exp2(s * scale*log2e - LSE*log2e); dS = P (dP - D), packed to bf16 in the B-operand
    // layout of the k-steps over the tile's keys
    u32x4 dsf[PT];
#pragma unroll
    for (int p = 0; p < KB * 8; ++p) {
      const int kb = p >> 3, r = (p & 7) * 2;
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], scale_log2, neg_lse2));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r + 1], scale_log2, neg_lse2));
      dsf[p >> 2][p & 3] = pack_bf16x2(p0 * (dp[kb][r] - Drow), p1 * (dp[kb][r + 1] - Drow));
    }
    // dQ^T += K^T dS^T
#pragma unroll
    for (int t = 0; t < PT; ++t)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(smem + KR + t * 16 * RB + fo.tr_off[cb][0]));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(smem + KR + t * 16 * RB + fo.tr_off[cb][1]));
        const bf16x8 kt = __builtin_bit_cast(
            bf16x8, s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
        acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt, __builtin_bit_cast(bf16x8, dsf[t]),
                                                          acc[cb], 0, 0, 0);
      }
    // the next tile's copies have landed; the barrier publishes them and closes this tile's reads
    vmem_wait<0>();
    __syncthreads();
  }

  if (qi < T) store_rows<CB, D>(dq + head_off + (int64_t)qi * D, acc, hf, scale);
}

// ---- dK, dV: one workgroup per (block of BM keys, batch*head); lane = key. Requires D from
// fa_bwd_dq_kernel (same stream, launched before). PART selects the outputs: kDV, kDK or both. A pass
// that computes one of them holds one accumulator and the fragments it needs only (dV: K; dK: K
// and V), so more waves fit on a SIMD; the two passes recompute S = Q K^T each.
constexpr int kDV = 1, kDK = 2;
template <class C, int PART = kDV | kDK>
__global__ __launch_bounds__(C::THREADS) void fa_bwd_dkdv_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const float* __restrict__ lse, const __bf16* __restrict__ dout, const float* __restrict__ delta,
    __bf16* __restrict__ dk, __bf16* __restrict__ dv, int T, int nk, int BH, float scale,
    float scale_log2, int head_group) {
  constexpr int D = C::D, BN = C::BN, BM = C::BM, KB = C::KB, CB = C::CB;
  constexpr int KSTEPS = C::KSTEPS, RB = C::ROW_BYTES, TB = C::TILE_BYTES, SB = C::STATS_BYTES;
  // Q ring (2 tiles), dO ring (2 tiles), statistics ring (2 x [LSE | D] of a Q tile)
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem;
  constexpr int STATS = 4 * TB;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, hf = lane >> 5;
  const int bid = block_index((int64_t)nk * BH);
  if (bid < 0) return;
  int kblk, bh;
  map_block<false>(bid, nk, BH, head_group, kblk, bh);  // in rank order: the earliest key blocks (most Q tiles) first
  const int k0 = kblk * BM;
  const int64_t head_off = (int64_t)bh * T * D;
  const char* qg = reinterpret_cast<const char*>(q + head_off);
  const char* dog = reinterpret_cast<const char*>(dout + head_off);
  const float* lse_h = lse + (int64_t)bh * T;
  const float* delta_h = delta + (int64_t)bh * T;
  const int kw0 = k0 + 32 * w;
  const int key = kw0 + n;  // this lane's key
  const int krow = min(key, T - 1);
  const int n_qt = (T + BN - 1) / BN;
  const int i0 = C::CAUSAL ? k0 / BN : 0;  // first Q tile holding a query >= the block's first key

  TileCopier<C> cp;
  cp.init(w, lane);
  FragOffsets<C> fo;
  fo.init(lane);
  // one Q tile's rows, dO rows and statistics (waves 0 and 1 copy LSE and D, one word per lane)
  auto copy_tile = [&](int i, int buf) {
    cp.copy(qg, i * BN, T, lds0 + buf * TB);
    cp.copy(dog, i * BN, T, lds0 + (2 + buf) * TB);
    const int r = min(i * BN + lane, T - 1);
    if (w == 0) lds_copy4(lse_h + r, lds0 + STATS + buf * SB);
    if (w == 1) lds_copy4(delta_h + r, lds0 + STATS + buf * SB + BN * 4);
  };
  copy_tile(i0, 0);

  constexpr bool DO_DV = (PART & kDV) != 0, DO_DK = (PART & kDK) != 0;
  bf16x8 kf[KSTEPS], vf[DO_DK ? KSTEPS : 1];
  load_row_frags<KSTEPS>(k + head_off + (int64_t)krow * D, hf, kf);
  if constexpr (DO_DK) load_row_frags<KSTEPS>(v + head_off + (int64_t)krow * D, hf, vf);
  f32x16 acc_dk[DO_DK ? CB : 1], acc_dv[DO_DV ? CB : 1];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    if constexpr (DO_DK) acc_dk[cb] = f32x16{};
    if constexpr (DO_DV) acc_dv[cb] = f32x16{};
  }

  vmem_wait<0>();
  __syncthreads();

  for (int i = i0; i < n_qt; ++i) {
    const int buf = (i - i0) & 1;
    const int QR = buf * TB, DR = (2 + buf) * TB, SR = STATS + buf * SB;
    if (i + 1 < n_qt) copy_tile(i + 1, buf ^ 1);
    const int qt0 = i * BN;
#pragma unroll
    for (int qb = 0; qb < KB; ++qb) {
      const int qs = qt0 + 32 * qb;  // first query of this 32-row block
      // (a block whose queries all precede this wave's keys is computed and masked whole: a branch
      // around it raised the kernel from 196 to 252 VGPRs and measured 8-12% slower overall)
      // S = Q K^T and dP = dO V^T: rows = queries 8*(r/4) + 4*hf + r%4 of the block, column = key
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int st = 0; st < KSTEPS; ++st) {
        const bf16x8 qa = *reinterpret_cast<const bf16x8*>(smem + QR + qb * 32 * RB + fo.row_off[st]);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[st], s, 0, 0, 0);
        if constexpr (DO_DK) {
          const bf16x8 da = *reinterpret_cast<const bf16x8*>(smem + DR + qb * 32 * RB + fo.row_off[st]);
          dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, vf[st], dp, 0, 0, 0);
        }
      }
      // the block's row statistics: registers 4g .. 4g+3 are rows 8g + 4*hf + 0..3
      float lse4[16], d4[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int rofs = (32 * qb + 8 * g + 4 * hf) * 4;
        const f32x4 a = *reinterpret_cast<const f32x4*>(smem + SR + rofs);
        const f32x4 b = *reinterpret_cast<const f32x4*>(smem + SR + BN * 4 + rofs);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lse4[4 * g + e] = -a[e] * kLog2e;
          d4[4 * g + e] = b[e];
        }
      }
      // visible iff key <= query < T: off = 8*(r/4) + r%4 in [key - qs - 4*hf, T-1 - qs - 4*hf]
      if ((C::CAUSAL && qs < kw0 + 32) || qs + 32 > T) {
        const int lo = C::CAUSAL ? key - qs - 4 * hf : -1;
        const int hi = T - 1 - qs - 4 * hf;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = 8 * (r >> 2) + (r & 3);
          s[r] = (off >= lo && off <= hi) ? s[r] : -__builtin_inff();
        }
      }
      // P and dS, packed in the B-operand layout of the two 16-query k-steps of this block
      u32x4 pf[2], dsf[2];
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const int r = 2 * p;
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], scale_log2, lse4[r]));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r + 1], scale_log2, lse4[r + 1]));
        if constexpr (DO_DV) pf[p >> 2][p & 3] = pack_bf16x2(p0, p1);
        if constexpr (DO_DK) dsf[p >> 2][p & 3] = pack_bf16x2(p0 * (dp[r] - d4[r]), p1 * (dp[r + 1] - d4[r + 1]));
      }
      // dV^T += dO^T P and dK^T += Q^T dS over the block's two k-steps
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int t = 2 * qb + tt;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          if constexpr (DO_DV) {
            const s16x4 dlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4*)(smem + DR + t * 16 * RB + fo.tr_off[cb][0]));
            const s16x4 dhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4*)(smem + DR + t * 16 * RB + fo.tr_off[cb][1]));
            const bf16x8 dot = __builtin_bit_cast(
                bf16x8, s16x8{dlo[0], dlo[1], dlo[2], dlo[3], dhi[0], dhi[1], dhi[2], dhi[3]});
            acc_dv[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dot, __builtin_bit_cast(bf16x8, pf[tt]),
                                                                 acc_dv[cb], 0, 0, 0);
          }
          if constexpr (DO_DK) {
            const s16x4 qlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4*)(smem + QR + t * 16 * RB + fo.tr_off[cb][0]));
            const s16x4 qhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4*)(smem + QR + t * 16 * RB + fo.tr_off[cb][1]));
            const bf16x8 qtr = __builtin_bit_cast(
                bf16x8, s16x8{qlo[0], qlo[1], qlo[2], qlo[3], qhi[0], qhi[1], qhi[2], qhi[3]});
            acc_dk[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qtr, __builtin_bit_cast(bf16x8, dsf[tt]),
                                                                 acc_dk[cb], 0, 0, 0);
          }
        }
      }
    }
    vmem_wait<0>();
    __syncthreads();
  }

  if (key < T) {
    if constexpr (DO_DK) store_rows<CB, D>(dk + head_off + (int64_t)key * D, acc_dk, hf, scale);
    if constexpr (DO_DV) store_rows<CB, D>(dv + head_off + (int64_t)key * D, acc_dv, hf, 1.0f);
  }
}

}  // namespace fa
