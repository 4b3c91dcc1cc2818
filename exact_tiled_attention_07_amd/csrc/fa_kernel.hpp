// Fused, tiled, exact attention forward for gfx950 (CDNA4): bf16 MFMA, LDS-staged K/V, online
// softmax in base 2, causal block skipping, per-row logsumexp.
//
// Method (what is computed and in which order):
//   - one workgroup owns one Q block of one (batch, head) and walks the K/V blocks; Q blocks never
//     communicate (learn-llm.fim.ai "手写 FlashAttention：拆开 SDPA 这个黑盒", STEP 3);
//   - per K/V block: scores on chip, running row max m and l = sum exp(x - m), and the output
//     accumulator rescaled by alpha = exp(m_old - m_new) when the max grows (same page, STEP 2);
//   - the division by l happens once, after the last block (same page, STEP 2, the note on
//     FlashAttention-2 moving the divide to the end; cnblogs "内核案例研究：Flash Attention",
//     section "块稀疏注意力 V2 和 V3", item 3);
//   - exp2 with log2(e) folded into the softmax scale, so m and l live in base 2 and the base
//     cancels in acc / l (learn-llm page, STEP 4, note on exp2 and 1.4427);
//   - causal blocks that lie wholly above the diagonal are skipped, and only blocks that touch the
//     diagonal (or the ragged end of the sequence) are masked element by element (STEP 3 legend;
//     STEP 5 note contrasting per-block masking with separate diagonal handling);
//   - the per-row logsumexp is written for a backward pass (STEP 4, note on training).
//
// gfx950 mapping (measured on the device, not taken from the pages):
//   - v_mfma_f32_32x32x16_bf16 (32 cycles, 1024 flop/clk/SIMD). Lane l holds A row l%32 and
//     B column l%32 with k = 8*(l/32) .. +7; C column l%32, rows 8*(r/4) + 4*(l/32) + r%4 for
//     register r.
//   - Scores are computed transposed, S^T = K Q^T, so a lane owns one query and its row statistics
//     need one cross-half exchange (v_permlane32_swap) instead of a 32-lane reduction.
//   - The output is computed transposed too, O^T = V^T P^T: the P^T operand is exactly the S^T
//     accumulator layout (after exp and bf16 rounding), and the rescale factor is per lane.
//   - V^T comes from the row-major V tile through ds_read_b64_tr_b16 (a transposing LDS read).
//   - K/V tiles go HBM -> LDS with global_load_lds_dwordx4 (no register staging), double
//     buffered, 16-byte chunks XOR-swizzled per row against LDS bank conflicts.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// The running max may lag the true max by up to this much (base-2 units) before the accumulator is
// rescaled. Any stabiliser gives the same exact result because it cancels in acc / l; this bound
// keeps every exp2 argument <= 8, so p <= 256 and l <= 256 * T stays far from fp32 overflow.
constexpr float kRescaleSlack = 8.0f;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int D_, int QB_, int NW_, int BN_, bool CAUSAL_>
struct Cfg {
  static constexpr int D = D_;        // head dim
  static constexpr int QB = QB_;      // 32-query column blocks per wave
  static constexpr int NW = NW_;      // waves per workgroup
  static constexpr int BN = BN_;      // keys per K/V tile
  static constexpr bool CAUSAL = CAUSAL_;
  static constexpr int BM = 32 * QB * NW;           // queries per workgroup
  static constexpr int THREADS = 64 * NW;
  static constexpr int ROW_BYTES = D * 2;           // one bf16 row of K or V
  static constexpr int CHUNKS = D / 8;              // 16-byte chunks per row
  static constexpr int TILE_BYTES = BN * ROW_BYTES; // one K (or V) tile
  static constexpr int LDS_BYTES = 4 * TILE_BYTES;  // K and V, two buffers each
  static constexpr int LOADS = TILE_BYTES / (16 * THREADS);  // 16-byte loads per lane per tile
  static constexpr int KSTEPS = D / 16;             // k-steps of the score MFMA
  static constexpr int KB = BN / 32;                // 32-key blocks per tile
  static constexpr int CB = D / 32;                 // 32-channel blocks of the output
  static constexpr int PT = BN / 16;                // k-steps of the P.V MFMA
  static_assert(D == 64 || D == 128, "head dim");
  static_assert(BN % 32 == 0 && BN >= 32, "tile keys");
  static_assert(LOADS >= 1 && LOADS * 16 * THREADS == TILE_BYTES, "tile load split");
};

// Physical 16-byte chunk of logical chunk c in LDS row r. An involution (XOR), so the same
// function maps physical back to logical. With 128-byte rows (d=64) two consecutive rows share a
// bank half, so the key is r/2; with 256-byte rows (d=128) every row starts on bank 0, so it is r.
template <int D>
__device__ __forceinline__ int swz(int r, int c) {
  return D == 64 ? (c ^ ((r >> 1) & 7)) : (c ^ (r & 15));
}

__device__ __forceinline__ float wave_max_halves(float x) {
  // v_permlane32_swap(x, x) returns (x of lanes 0-31 twice, x of lanes 32-63 twice).
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float wave_sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum of the two bf16 halves of a packed pair, added to acc in fp32 (v_dot2c_f32_bf16 with 1, 1).
__device__ __forceinline__ float add_bf16_pair(uint32_t pair, float acc) {
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), ones, acc, false);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 f = {a, b};
  bf16x2 h = __builtin_convertvector(f, bf16x2);  // v_cvt_pk_bf16_f32, round to nearest even
  return __builtin_bit_cast(uint32_t, h);
}

// Map the flat workgroup id to (Q block, batch*head). Workgroups are handed to the 8 XCDs round
// robin, so when B*H is a multiple of 8 each XCD gets its own set of heads (their K/V stay in that
// XCD's L2), and within an XCD the Q blocks with the most K/V tiles start first.
template <bool CAUSAL>
__device__ __forceinline__ void map_block(int bid, int nq, int BH, int& qblk, int& bh) {
  int rank;
  if ((BH & 7) == 0) {
    const int xcd = bid & 7, slot = bid >> 3, per = BH >> 3;
    rank = slot / per;
    bh = (slot - rank * per) * 8 + xcd;
  } else {
    rank = bid / BH;
    bh = bid - rank * BH;
  }
  qblk = CAUSAL ? (nq - 1 - rank) : rank;
}

template <class C>
__global__ __launch_bounds__(C::THREADS) void fa_fwd_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    __bf16* __restrict__ o, float* __restrict__ lse, int T, int nq, int BH, float scale_log2) {
  constexpr int D = C::D, QB = C::QB, NW = C::NW, BN = C::BN, BM = C::BM;
  constexpr int KB = C::KB, CB = C::CB, PT = C::PT, KSTEPS = C::KSTEPS;
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform per wave
  const int n = lane & 31;    // query column of this lane within a 32-query block
  const int hf = lane >> 5;   // which half of the wave (0/1)

  int qblk, bh;
  map_block<C::CAUSAL>(blockIdx.x, nq, BH, qblk, bh);
  const int q0 = qblk * BM;
  const int64_t head_off = (int64_t)bh * T * D;
  const char* kg = reinterpret_cast<const char*>(k + head_off);
  const char* vg = reinterpret_cast<const char*>(v + head_off);

  // Number of K/V tiles this workgroup needs: up to the diagonal when causal.
  const int kv_end = C::CAUSAL ? min(q0 + BM, T) : T;
  const int ntiles = (kv_end + BN - 1) / BN;

  // ---- K/V tile loads, HBM -> LDS directly. Rows past T are clamped to row T-1 (always in
  // bounds); their scores are masked and their V rows are zeroed before use.
  auto issue_tile = [&](int j, int buf) {
    const int kt0 = j * BN;
    char* kl = smem + buf * 2 * C::TILE_BYTES;
    char* vl = kl + C::TILE_BYTES;
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int region = i * NW + w;                 // 1 KiB of LDS per wave instruction
      const int lofs = region * 1024 + lane * 16;    // byte offset inside the tile
      const int r = lofs / C::ROW_BYTES;
      const int pc = (lofs % C::ROW_BYTES) >> 4;
      const int lc = swz<D>(r, pc);
      const int grow = min(kt0 + r, T - 1);
      const int64_t gofs = (int64_t)grow * C::ROW_BYTES + lc * 16;
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(kg + gofs),
          (__attribute__((address_space(3))) void*)(kl + region * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(vg + gofs),
          (__attribute__((address_space(3))) void*)(vl + region * 1024), 16, 0, 0);
    }
  };
  // Zero the V rows at or past T of a ragged last tile, so a clamped copy of row T-1 can never
  // reach the output (0 * p stays 0 even for non-finite p; p is 0 there anyway).
  auto zero_v_tail = [&](int j, int buf) {
    const int kt0 = j * BN;
    const int first = T - kt0;  // first row to clear, 0 < first < BN
    char* vl = smem + buf * 2 * C::TILE_BYTES + C::TILE_BYTES;
    for (int idx = tid; idx < (BN - first) * C::CHUNKS; idx += C::THREADS) {
      const int r = first + idx / C::CHUNKS;
      const int c = idx % C::CHUNKS;
      *reinterpret_cast<u32x4*>(vl + r * C::ROW_BYTES + c * 16) = u32x4{0u, 0u, 0u, 0u};
    }
  };
  // The last tile reaches past T only for a ragged sequence end.
  const bool tail_ragged = ntiles * BN > T;

  issue_tile(0, 0);

  // ---- Q fragments straight into registers: B operand of S^T = K Q^T. Lane (n, hf) holds
  // query row q0 + 32*(QB*w + qb) + n, channels 16*s + 8*hf .. +7.
  bf16x8 qf[QB][KSTEPS];
  const int qw0 = q0 + 32 * QB * w;  // first query of this wave
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = min(qw0 + 32 * qb + n, T - 1);
    const bf16x8* src = reinterpret_cast<const bf16x8*>(q + head_off + (int64_t)row * D);
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) qf[qb][s] = src[2 * s + hf];
  }

  // Per query row (this lane's half of the keys): running max m (base 2, scaled), the fp32 sum
  // l of the exponentials (for the logsumexp) and the sum w of the same weights after rounding to
  // bf16, i.e. of exactly the weights that enter P.V. O is normalised by w, so the rounding of a
  // dominant weight cancels between numerator and denominator instead of scaling its V row.
  f32x16 acc[CB][QB];
  float m_run[QB], l_run[QB], w_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -__builtin_inff();
    l_run[qb] = 0.0f;
    w_run[qb] = 0.0f;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[cb][qb] = f32x16{};
  }

  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tail_ragged && ntiles == 1) {
    zero_v_tail(0, 0);
    __syncthreads();
  }

  for (int j = 0; j < ntiles; ++j) {
    const int buf = j & 1;
    if (j + 1 < ntiles) issue_tile(j + 1, buf ^ 1);

    const int kt0 = j * BN;
    const bool active = !C::CAUSAL || kt0 <= qw0 + 32 * QB - 1;
    if (active) {
      const char* kl = smem + buf * 2 * C::TILE_BYTES;
      const char* vl = kl + C::TILE_BYTES;

      // ---- S^T = K Q^T: lane (n, hf) gets query column n; register r of block kb is key
      // kt0 + 32*kb + 8*(r/4) + 4*hf + r%4.
      f32x16 st[KB][QB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) st[kb][qb] = f32x16{};
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const int r = 32 * kb + n;
          const bf16x8 kfrag =
              *reinterpret_cast<const bf16x8*>(kl + r * C::ROW_BYTES + swz<D>(r, 2 * s + hf) * 16);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            st[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfrag, qf[qb][s], st[kb][qb], 0, 0, 0);
        }
      }

      // ---- mask: only tiles that reach past this wave's first query (causal) or past T.
      const bool need_mask = (C::CAUSAL && kt0 + BN - 1 > qw0) || (kt0 + BN > T);
      if (need_mask) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const int qi = qw0 + 32 * qb + n;
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = kt0 + 32 * kb + 8 * (r >> 2) + 4 * hf + (r & 3);
              const bool visible = (key < T) && (!C::CAUSAL || key <= qi);
              st[kb][qb][r] = visible ? st[kb][qb][r] : -__builtin_inff();
            }
        }
      }

      // ---- online softmax (base 2) and P in bf16, laid out as the B operand of O^T += V^T P^T.
      bf16x8 pf[QB][PT];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float mx = -__builtin_inff();
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[kb][qb][r]);
        mx = wave_max_halves(mx) * scale_log2;  // scale_log2 > 0, so scaling keeps the max
        // Rescale only when some row's max rose by more than the slack; otherwise the previous
        // max keeps serving as the stabiliser (exact: it cancels in acc / l).
        const bool grow = mx > m_run[qb] + kRescaleSlack;
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
          const float m_new = fmaxf(m_run[qb], mx);
          const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - m_new);
          l_run[qb] *= alpha;
          w_run[qb] *= alpha;
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) acc[cb][qb] *= alpha;
          m_run[qb] = m_new;
        }
        const float neg_m = -m_run[qb];
        float lsum0 = 0.0f, lsum1 = 0.0f, wsum = 0.0f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            uint32_t pk[4];
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
              const int r = 8 * half + e;
              const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(st[kb][qb][r], scale_log2, neg_m));
              const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(st[kb][qb][r + 1], scale_log2, neg_m));
              lsum0 += p0;
              lsum1 += p1;
              pk[e >> 1] = pack_bf16x2(p0, p1);
              wsum = add_bf16_pair(pk[e >> 1], wsum);
            }
            u32x4 pv = {pk[0], pk[1], pk[2], pk[3]};
            pf[qb][2 * kb + half] = __builtin_bit_cast(bf16x8, pv);
          }
        }
        l_run[qb] += lsum0 + lsum1;
        w_run[qb] += wsum;
      }

      // ---- O^T += V^T P^T. A operand: lane l (group g = l/16, i = l%16) must hold V^T row
      // c(cb, l%32) at the 8 keys of its P^T slots. Two transposing reads, 4 keys each: source lane
      // i of a group reads V row (key base + i/4), 4 channels starting at the column below.
      const int grp = lane >> 4, gi = lane & 15;
      const int ga = grp & 1, gh = grp >> 1;
      const int e_src = gi >> 2, q_src = gi & 3;
#pragma unroll
      for (int t = 0; t < PT; ++t) {
        const int kb = t >> 1, u = t & 1;
        const int r1 = 32 * kb + 16 * u + 4 * gh + e_src;  // key row of the first read
        const int r2 = r1 + 8;                              // and of the second
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          const int col = (D / 2) * (q_src & 1) + 16 * cb + 4 * (2 * ga + (q_src >> 1));
          const int chunk = col >> 3, within = (col & 7) * 2;
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4*)(vl + r1 * C::ROW_BYTES + swz<D>(r1, chunk) * 16 + within));
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4*)(vl + r2 * C::ROW_BYTES + swz<D>(r2, chunk) * 16 + within));
          typedef short s16x8 __attribute__((ext_vector_type(8)));
          const s16x8 both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          const bf16x8 vfrag = __builtin_bit_cast(bf16x8, both);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            acc[cb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfrag, pf[qb][t], acc[cb][qb], 0, 0, 0);
        }
      }
    }

    // Tile j+1 has landed in LDS for this wave; the barrier makes it (and the end of every wave's
    // reads of tile j) visible to all waves.
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tail_ragged && j + 2 == ntiles) {
      zero_v_tail(j + 1, buf ^ 1);
      __syncthreads();
    }
  }

  // ---- epilogue: O = acc / w, rounded once to bf16; LSE = ln2 * (m + log2 l).
  // Lane (n, hf) of channel block cb holds channels (D/2)*hf + 16*cb + r, r = 0..15, in order.
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = qw0 + 32 * qb + n;
    const float l_tot = wave_sum_halves(l_run[qb]);
    const float inv = 1.0f / wave_sum_halves(w_run[qb]);
    if (row < T) {
      char* orow = reinterpret_cast<char*>(o + head_off + (int64_t)row * D);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          u32x4 out;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            out[e] = pack_bf16x2(acc[cb][qb][8 * half + 2 * e] * inv, acc[cb][qb][8 * half + 2 * e + 1] * inv);
          *reinterpret_cast<u32x4*>(orow + ((D / 2) * hf + 16 * cb + 8 * half) * 2) = out;
        }
      }
      if (hf == 0) lse[(int64_t)bh * T + row] = (m_run[qb] + __log2f(l_tot)) * kLn2;
    }
  }
}

}  // namespace fa
