// Fused, tiled, exact attention forward for gfx950 (CDNA4): bf16 MFMA, LDS-staged K/V, online
// softmax in base 2, causal block skipping, per-row logsumexp.
//
// Method (what is computed and in which order):
//   - one workgroup owns one Q block of one (batch, head) and walks the K/V blocks; Q blocks never
//     communicate (learn-llm.fim.ai "手写 FlashAttention：拆开 SDPA 这个黑盒", STEP 3);
//   - per K/V block: scores on chip, running row max m and l = sum exp(x - m), and the output
//     accumulator rescaled by alpha = exp(m_old - m_new) (same page, STEP 2); alpha is exactly 1
//     when a row's max did not grow, and a wave skips the multiplications when that holds for all
//     of its rows;
//   - the division by l happens once, after the last block (same page, STEP 2, the note on
//     FlashAttention-2 moving the divide to the end; cnblogs "内核案例研究：Flash Attention",
//     section "块稀疏注意力 V2 和 V3", item 3);
//   - exp2 with log2(e) folded into the softmax scale, so m and l live in base 2 and the base
//     cancels in acc / l (learn-llm page, STEP 4, note on exp2 and 1.4427);
//   - causal blocks that lie wholly above the diagonal are never loaded, and only blocks that touch
//     the diagonal (or the ragged end of the sequence) are masked element by element (STEP 3
//     legend; STEP 5 note contrasting per-block masking with separate diagonal handling);
//   - the softmax of one block runs while the matrix unit computes the next block's scores, the
//     overlap of non-matrix work with matrix work that the cnblogs page describes for its third
//     version (the closing section, on V3);
//   - the per-row logsumexp is written for a backward pass (STEP 4, note on training);
//   - for short sequences (few Q blocks) two waves may share one block of queries, each walking
//     every other K/V block, and combine their (m, l, O) at the end with the log-space merge of
//     partial results over disjoint key sets (ijyty.com FlashAttention article, section 2.1).
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
//   - K/V tiles go HBM -> LDS with global_load_lds_dwordx4 (no register staging) into two rings of
//     NSTAGE buffers; K is fetched NSTAGE tiles ahead and V NSTAGE-1 tiles ahead, so each copy has
//     NSTAGE-1 steps to land. 16-byte chunks are XOR-swizzled per row against LDS bank conflicts.
//   - Each wave is software-pipelined: in step j its MFMA "slots" first compute S(j+1) = K(j+1) Q^T
//     and then O += V(j)^T P(j)^T, while the VALU work of the softmax of tile j (and the row max
//     of S(j+1)) is spread over those slots. LDS fragments are read a few slots ahead.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kSparseMaxFloor = -1.0e30f;  // running-max floor of the block-sparse path

template <int D_, int QB_, int NW_, int BN_, bool CAUSAL_, int NSTAGE_, bool SPARSE_ = false,
          bool RANGE_ = false, bool FEWQ_ = false, int KSPLIT_ = 1>
struct Cfg {
  static constexpr int D = D_;        // head dim
  static constexpr int QB = QB_;      // 32-query column blocks per wave
  static constexpr int NW = NW_;      // waves per workgroup
  static constexpr int BN = BN_;      // keys per K/V tile
  static constexpr bool CAUSAL = CAUSAL_;
  static constexpr int NSTAGE = NSTAGE_;            // LDS buffers per ring (K ring and V ring)
  // block-sparse: a per-(Q block, K/V tile) mask selects the tiles a workgroup visits; their
  // indices are compacted into an LDS list (at most MAX_LIST tiles, i.e. T <= MAX_LIST * BN)
  static constexpr bool SPARSE = SPARSE_;
  static constexpr int MAX_LIST = SPARSE_ ? 1024 : 0;
  // key range: only the tiles of keys [k_begin, k_end) are visited and the outputs are the partial
  // O (fp32, normalised over the range) and LSE of that range, for a later log-space merge
  static constexpr bool RANGE = RANGE_;
  static constexpr bool LISTED = SPARSE_ || RANGE_;  // rows may see no key
  static_assert(!(SPARSE_ && RANGE_), "one tile selection at a time");
  // fewer queries than a workgroup holds (T < BM): waves without a query row skip the arithmetic
  static constexpr bool FEWQ = FEWQ_;
  // key split: KSPLIT waves share one block of queries; wave (block b, part p) visits the K/V tiles
  // p, p + KSPLIT, ... of the block's range, and the parts are merged in log space at the end
  static constexpr int KSPLIT = KSPLIT_;
  static constexpr bool FLOORED = SPARSE_ || RANGE_ || KSPLIT_ > 1;  // a wave's row may see no key
  static_assert(KSPLIT == 1 || (KSPLIT == 2 && QB == 1 && NW % 2 == 0 && !SPARSE_ && !RANGE_ && !FEWQ_),
                "key split: two waves per 32-query block, dense forward only");
  static constexpr int BM = 32 * QB * NW / KSPLIT;  // queries per workgroup
  static constexpr int THREADS = 64 * NW;
  static constexpr int ROW_BYTES = D * 2;           // one bf16 row of K or V
  static constexpr int CHUNKS = D / 8;              // 16-byte chunks per row
  static constexpr int TILE_BYTES = BN * ROW_BYTES; // one K (or V) tile
  static constexpr int SLOT_BYTES = KSPLIT * TILE_BYTES;     // one ring buffer: the tiles of a step
  static constexpr int LDS_BYTES = 2 * NSTAGE * SLOT_BYTES;  // K ring, then V ring
  static constexpr int LOADS = TILE_BYTES / (16 * THREADS);  // 16-byte loads per lane per tile
  static constexpr int KSTEPS = D / 16;             // k-steps of the score MFMA
  static constexpr int KB = BN / 32;                // 32-key blocks per tile
  static constexpr int CB = D / 32;                 // 32-channel blocks of the output
  static constexpr int PT = BN / 16;                // k-steps of the P.V MFMA
  static constexpr int NS_QK = KSTEPS * KB;         // score MFMA slots per tile (QB MFMAs each)
  static constexpr int NS_PV = PT * CB;             // P.V MFMA slots per tile (QB MFMAs each)
  static constexpr int NS = NS_QK + NS_PV;
  static constexpr int NPAIRS = KB * 8;             // score pairs per lane per 32-query block
  static constexpr int PD = 3;                      // LDS fragment prefetch distance, in slots
  // exp pairs are spread over slots [0, EXP_WINDOW); pair p must be done before the P.V slots of
  // its k-step p/4 start.
  static constexpr int EXP_WINDOW = NS_QK + (PT - 1) * CB;
  // the row max of the next tile is spread over slots [MAX_FIRST, MAX_LAST]; slots NS-2 and NS-1
  // combine the two wave halves and form the new max and alpha
  static constexpr int MAX_FIRST = NS_QK + 2;
  static constexpr int MAX_LAST = NS - 3;
  static_assert(MAX_LAST >= MAX_FIRST, "slots for the row max");
  static constexpr int VRING = NSTAGE * SLOT_BYTES; // offset of the V ring
  static_assert(D == 64 || D == 128, "head dim");
  static_assert(BN % 32 == 0 && BN >= 32, "tile keys");
  static_assert(LOADS >= 1 && LOADS * 16 * THREADS == TILE_BYTES, "tile load split");
  static_assert(NSTAGE >= 2 && NSTAGE <= 4, "ring depth");
  static_assert(LDS_BYTES <= 65536, "static LDS of one workgroup");
  // the merge of a key split exchanges acc (16*CB floats per lane), m and l of one wave per block
  static_assert(KSPLIT == 1 || 256 * (16 * CB + 2) * (NW / KSPLIT) <= LDS_BYTES, "merge area");
};

template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// Physical 16-byte chunk of logical chunk c in LDS row r: c XOR a per-row key (an involution, so
// the same function maps physical back to logical). The key is a bit permutation of r/2 (128-byte
// rows, d=64: two consecutive rows fill the two bank halves) or of r (256-byte rows, d=128). It is
// chosen so that (a) the 16 lanes of a K read (16 consecutive rows, one chunk) hit distinct banks,
// and (b) the four rows of each 16-lane group of a transposing V read, each read at the chunk set
// {c, c^1, c^4, c^5} (d=64) or {c, c^1, c^8, c^9} (d=128), land in disjoint banks: the low bits of
// the row pick key bits that those chunk sets do not cover. Adding a multiple of 16 to r leaves the
// key unchanged.
template <int D>
__device__ __forceinline__ int swz(int r, int c) {
  if constexpr (D == 64) {
    const int g = (r >> 1) & 7;
    return c ^ (((g & 1) << 1) | ((g >> 1) & 1) | (g & 4));
  } else {
    const int x = r & 15;
    return c ^ (((x & 3) << 1) | ((x >> 2) & 1) | (x & 8));
  }
}

// max of two floats as one v_max_f32. The row statistics never hold a signalling NaN, so the
// quieting maxes the compiler puts in front of fmaxf for operands it cannot prove canonical (the
// cross-lane swap below, values carried around the loop) are not needed.
__device__ __forceinline__ float max_f32(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

__device__ __forceinline__ float wave_max_halves(float x) {
  // v_permlane32_swap(x, x) returns (x of lanes 0-31 twice, x of lanes 32-63 twice).
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max_f32(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float wave_sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 f = {a, b};
  bf16x2 h = __builtin_convertvector(f, bf16x2);  // v_cvt_pk_bf16_f32, round to nearest even
  return __builtin_bit_cast(uint32_t, h);
}

// HBM -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4) as inline asm: LDS bytes
// [lds_addr + 16*lane, +16) <- global bytes [base + voff, +16). If the compiler saw these copies it
// would, not knowing which LDS bytes they fill, wait for all of them before every transposing LDS
// read, serialising the prefetch with the compute. Completion is waited for explicitly
// (s_waitcnt vmcnt(0) before the barrier that publishes a tile). M0 is saved and restored because
// the compiler owns it.
__device__ __forceinline__ void lds_copy16(const char* base, uint32_t voff, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_addr), "v"(voff), "s"(base)
      : "memory");
}
__device__ __forceinline__ void lds_copy16(const char* addr, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_addr), "v"(addr)
      : "memory");
}
template <int N>
__device__ __forceinline__ void vmem_wait() {  // all but the newest N vector-memory ops complete
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Flat index of this workgroup among n. The dispatch counts work-items per grid dimension in 32
// bits, so a launch of more workgroups than one dimension holds folds them into x (a multiple of
// 8, which keeps the XCD round robin of the flat index) and z; workgroups past n get -1 and exit.
__device__ __forceinline__ int block_index(int64_t n) {
  const int64_t b = (int64_t)blockIdx.z * gridDim.x + blockIdx.x;
  return b < n ? (int)b : -1;
}

// Map the flat workgroup id to (Q block, batch*head). Workgroups are handed to the 8 XCDs round
// robin, so when B*H is a multiple of 8 each XCD gets its own set of heads (their K/V stay in that
// XCD's L2). Within an XCD the heads run in groups of hg (hg divides B*H/8): a group's Q blocks,
// interleaved over its heads and the ones with the most K/V tiles first, are dispatched before the
// next group's, so that only the K/V of hg heads compete for the XCD's L2 at a time. hg = B*H/8
// interleaves all of the XCD's heads.
template <bool CAUSAL>
__device__ __forceinline__ void map_block(int bid, int nq, int BH, int hg, int& qblk, int& bh) {
  int rank;
  if ((BH & 7) == 0) {
    const int xcd = bid & 7, slot = bid >> 3;
    const int span = hg * nq, g = slot / span, s = slot - g * span;
    rank = s / hg;
    bh = (g * hg + (s - rank * hg)) * 8 + xcd;
  } else {
    rank = bid / BH;
    bh = bid - rank * BH;
  }
  qblk = CAUSAL ? (nq - 1 - rank) : rank;
}

template <class C>
__global__ __launch_bounds__(C::THREADS) void fa_fwd_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    __bf16* __restrict__ o, float* __restrict__ lse, int T, int nq, int BH, float scale_log2,
    const uint8_t* __restrict__ bmask, int mask_heads, int k_begin, int k_end, int t_keys,
    int k_chunk, int head_group) {
  constexpr int D = C::D, QB = C::QB, NW = C::NW, BN = C::BN, BM = C::BM;
  constexpr int KB = C::KB, CB = C::CB, PT = C::PT, KSTEPS = C::KSTEPS, RB = C::ROW_BYTES;
  constexpr int NS_QK = C::NS_QK, NS = C::NS, PD = C::PD;
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform per wave
  const int n = lane & 31;    // query column of this lane within a 32-query block
  const int hf = lane >> 5;   // which half of the wave (0/1)
  (void)bmask;
  (void)mask_heads;
  (void)k_begin;
  (void)k_end;
  (void)t_keys;
  (void)k_chunk;

  const int bid = block_index((int64_t)nq * BH);
  if (bid < 0) return;
  int qblk, bh;
  map_block<C::CAUSAL>(bid, nq, BH, head_group, qblk, bh);
  const int q0 = qblk * BM;
  // T is the number of queries. A key range may come from a longer sequence of Tk keys (queries
  // then sit at its end: query i is at key position i + coff, the causal diagonal shifted by coff),
  // and blockIdx.y picks one of several equal key ranges, each with its own partial output.
  const int Tk = C::RANGE ? t_keys : T;
  const int coff = C::RANGE ? Tk - T : 0;
  if constexpr (C::RANGE) {
    const int split = blockIdx.y;
    k_begin += split * k_chunk;
    k_end = min(k_begin + k_chunk, k_end);
    o = reinterpret_cast<__bf16*>(reinterpret_cast<float*>(o) + (int64_t)split * BH * T * D);
    lse += (int64_t)split * BH * T;
  }
  const int64_t head_off = (int64_t)bh * T * D;    // q and o rows of this head
  const int64_t head_off_k = (int64_t)bh * Tk * D;  // k and v rows of this head
  const char* kg = reinterpret_cast<const char*>(k + head_off_k);
  const char* vg = reinterpret_cast<const char*>(v + head_off_k);
  // with a key split, wave w holds query block w / KSPLIT and visits every KSPLIT-th tile from
  // tile w % KSPLIT (both uniform per wave)
  const int wq = C::KSPLIT == 1 ? w : w / C::KSPLIT;
  const int part = C::KSPLIT == 1 ? 0 : w % C::KSPLIT;
  const int qw0 = q0 + 32 * QB * wq;  // first query of this wave
  // With few queries (a key range for a handful of new queries) whole waves hold no query row:
  // they still copy their share of every tile and meet every barrier, but skip the MFMA and the
  // softmax (a wave-uniform branch; the barriers stay outside it).
  const bool wave_active = !C::FEWQ || qw0 < T;

  // K/V tiles this workgroup needs: up to the diagonal when causal (tiles above it are never
  // touched), all of them otherwise. The last one reaches past T only for a ragged end.
  const int kv_end = C::CAUSAL ? max(0, min(q0 + BM + coff, Tk)) : Tk;
  const int n_cand = (kv_end + BN - 1) / BN;  // candidate tiles 0 .. n_cand-1
  // Block-sparse: keep the candidates whose mask byte is nonzero, in ascending order, as a list in
  // LDS; tile_at(x) is the x-th tile visited (the identity when dense).
  __shared__ uint16_t tlist[C::SPARSE ? C::MAX_LIST : 1];
  __shared__ int wcount[C::SPARSE ? NW : 1];
  int n_tiles = n_cand;
  if constexpr (C::SPARSE) {
    const uint8_t* mrow = bmask + ((int64_t)(mask_heads == 1 ? 0 : bh) * nq + qblk) * ((T + BN - 1) / BN);
    int count = 0;
    for (int base = 0; base < n_cand; base += C::THREADS) {
      const int t = base + tid;
      const bool on = t < n_cand && mrow[t] != 0;
      const uint64_t bal = __builtin_amdgcn_ballot_w64(on);
      if (lane == 0) wcount[w] = __builtin_popcountll(bal);
      __syncthreads();
      int before = 0, total = 0;
#pragma unroll
      for (int x = 0; x < NW; ++x) {
        const int c = wcount[x];
        before += x < w ? c : 0;
        total += c;
      }
      const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
      if (on) tlist[count + before + below] = (uint16_t)t;
      count += total;
      __syncthreads();
    }
    n_tiles = __builtin_amdgcn_readfirstlane(count);
  }
  const int t_begin = C::RANGE ? k_begin / BN : 0;  // first tile of the key range
  if constexpr (C::RANGE) n_tiles = max(0, min((k_end + BN - 1) / BN, n_cand) - t_begin);
  // key split: n_tiles counts steps; step x copies tiles KSPLIT*x .. +KSPLIT-1 (clamped to the last
  // one, a harmless re-copy) and this wave computes tile KSPLIT*x + part, which past n_cand-1 is a
  // wholly masked tile (its keys are past the sequence: the ragged-end mask removes them all)
  if constexpr (C::KSPLIT > 1) n_tiles = (n_cand + C::KSPLIT - 1) / C::KSPLIT;
  // (k_begin, k_end and t_begin are uniform; n_tiles stays a scalar)
  auto tile_at = [&](int x) -> int {
    if constexpr (C::SPARSE) return __builtin_amdgcn_readfirstlane((int)tlist[x]);
    else if constexpr (C::KSPLIT > 1) return C::KSPLIT * x + part;
    else return t_begin + x;
  };
  // the tile copied into sub-buffer sub of step x's ring buffer
  auto copy_tile = [&](int x, int sub) -> int {
    if constexpr (C::KSPLIT > 1) return min(C::KSPLIT * x + sub, n_cand - 1);
    else return tile_at(x);
  };
  if constexpr (C::LISTED) {
    if (n_tiles == 0) {  // no key visible to any row of the block: O = 0, LSE = -inf
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int row = qw0 + 32 * qb + n;
        if (row < T) {
          u32x4* orow = reinterpret_cast<u32x4*>(
              C::RANGE ? static_cast<void*>(reinterpret_cast<float*>(o) + head_off + (int64_t)row * D)
                       : static_cast<void*>(o + head_off + (int64_t)row * D));
          constexpr int CHUNKS16 = C::RANGE ? D / 4 : D / 8;  // 16-byte chunks of one output row
#pragma unroll
          for (int c = 0; c < CHUNKS16 / 2; ++c) orow[2 * c + hf] = u32x4{0u, 0u, 0u, 0u};
          if (hf == 0) lse[(int64_t)bh * T + row] = -__builtin_inff();
        }
      }
      return;
    }
  }
  // the last tile holding keys (uniform over the workgroup) and its sub-buffer
  const int last_tile = C::KSPLIT > 1 ? n_cand - 1 : tile_at(n_tiles - 1);
  const int last_sub = C::KSPLIT > 1 ? last_tile % C::KSPLIT : 0;
  const bool tail_ragged = (last_tile + 1) * BN > Tk;

  // ---- HBM -> LDS copies of one K or V tile. Lane `lane` of load i fills 16 bytes of the 1 KiB
  // LDS region (i*NW + w); it fetches the logical chunk that the swizzle puts there. Rows past Tk
  // are clamped to row Tk-1 (always in bounds); their scores are masked and their V rows zeroed.
  int dma_row[C::LOADS], dma_col[C::LOADS];
  uint32_t dma_off[C::LOADS];
#pragma unroll
  for (int i = 0; i < C::LOADS; ++i) {
    const int lofs = (i * NW + w) * 1024 + lane * 16;
    dma_row[i] = lofs / RB;
    dma_col[i] = swz<D>(dma_row[i], (lofs % RB) >> 4) * 16;
    dma_off[i] = (uint32_t)(dma_row[i] * RB + dma_col[i]);
  }
  auto dma = [&](const char* g, int tile, int buf_off) {
    const int kt0 = tile * BN;
    if (kt0 + BN <= Tk) {  // whole tile inside the sequence: scalar base + per-lane constant
      const char* gt = g + (size_t)kt0 * RB;
#pragma unroll
      for (int i = 0; i < C::LOADS; ++i) lds_copy16(gt, dma_off[i], lds0 + buf_off + (i * NW + w) * 1024);
    } else {
      // the tile's first and the sequence's last row pass through an empty asm so that the
      // per-lane clamping below stays in this (rare) branch instead of being hoisted into every step
      int first = kt0, last = Tk - 1;
      asm volatile("" : "+s"(first), "+s"(last));
#pragma unroll
      for (int i = 0; i < C::LOADS; ++i) {
        const uint32_t gofs = (uint32_t)(min(first + dma_row[i], last) * RB + dma_col[i]);
        lds_copy16(g + gofs, lds0 + buf_off + (i * NW + w) * 1024);
      }
    }
  };
  // the tiles of step x into the ring buffer at buf_off (one tile unless the keys are split)
  auto dma_step = [&](const char* g, int x, int buf_off) {
#pragma unroll
    for (int sub = 0; sub < C::KSPLIT; ++sub) dma(g, copy_tile(x, sub), buf_off + sub * C::TILE_BYTES);
  };
  // Zero the V rows at or past Tk of a ragged last tile, so a clamped copy of row Tk-1 can never
  // reach the output (their weights are 0; a non-finite input row would still give 0 * inf).
  auto zero_v_tail = [&](int buf_off) {
    const int first = Tk - last_tile * BN;  // first row to clear, 0 < first < BN
    char* vl = smem + buf_off;
    for (int idx = tid; idx < (BN - first) * C::CHUNKS; idx += C::THREADS) {
      const int r = first + idx / C::CHUNKS;
      *reinterpret_cast<u32x4*>(vl + r * RB + (idx % C::CHUNKS) * 16) = u32x4{0u, 0u, 0u, 0u};
    }
  };

  // Tile t's K and V live in buffer (t + ring0) % NSTAGE of their rings. With two buffers per
  // ring, ring0 is the parity of the number of pipelined steps, so that the steps taken in pairs
  // (the main loop below) always start at buffer 0 and every LDS offset in the loop is an
  // immediate; with more buffers ring0 is 0.
  const int ring0 = C::NSTAGE == 2 ? ((n_tiles - 1) & 1) : 0;
  auto buf_of = [&](int t) {
    const int r = t % C::NSTAGE + ring0;
    return r >= C::NSTAGE ? r - C::NSTAGE : r;
  };

  // Prologue copies: K(0 .. NSTAGE-1) and V(0 .. NSTAGE-2) (clamped to the last tile).
#pragma unroll
  for (int t = 0; t < C::NSTAGE; ++t) {
    if (t < n_tiles) dma_step(kg, t, buf_of(t) * C::SLOT_BYTES);
    if (t < C::NSTAGE - 1 && t < n_tiles) dma_step(vg, t, C::VRING + buf_of(t) * C::SLOT_BYTES);
  }

  // ---- Q fragments straight into registers: B operand of S^T = K Q^T. Lane (n, hf) holds
  // query row qw0 + 32*qb + n, channels 16*s + 8*hf .. +7.
  bf16x8 qf[QB][KSTEPS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = min(qw0 + 32 * qb + n, T - 1);
    const bf16x8* src = reinterpret_cast<const bf16x8*>(q + head_off + (int64_t)row * D);
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) qf[qb][s] = src[2 * s + hf];
  }

  // ---- per-lane LDS byte addresses of the MFMA fragments (the buffer and the k-step / key block
  // parts are compile-time immediates).
  // K fragment (kb, s): row 32*kb + n, channels 16*s + 8*hf .. +7.
  // (with a key split the wave's sub-buffer is folded in here)
  int k_off[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) k_off[s] = part * C::TILE_BYTES + n * RB + swz<D>(n, 2 * s + hf) * 16;
  // V^T fragment (t, cb): lane l (group g = l/16, i = l%16) holds V^T row c(cb, l%32) at the 8
  // keys of its P^T slots, via two transposing reads of 4 keys each. Source lane i of a group
  // reads V row (16*t + 4*(g/2) + i/4 [+ 8]) at 4 channels starting at the column below.
  int v_off[CB][2];
  {
    const int grp = lane >> 4, gi = lane & 15;
    const int ga = grp & 1, gh = grp >> 1;
    const int e_src = gi >> 2, q_src = gi & 3;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int col = (D / 2) * (q_src & 1) + 16 * cb + 4 * (2 * ga + (q_src >> 1));
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        const int r = 4 * gh + e_src + 8 * rr;
        v_off[cb][rr] = part * C::TILE_BYTES + r * RB + swz<D>(r, col >> 3) * 16 + (col & 7) * 2;
      }
    }
  }

  // Per query row: the exact running max m (base 2, scaled; the same in both halves of the wave),
  // the fp32 sum l of this lane's half of the exponentials, and the factor alpha = exp2(m_old -
  // m_new) still to be applied to acc and l before the next block is added. Because m is the
  // exact max, the largest weight of a row rounds to exactly 1 in bf16 (in fp32 it is exp2 of the
  // rounding residual of m, which the FMA s * c - m keeps: within 2^-23 of 1).
  f32x16 acc[CB][QB];
  float m_run[QB], l_run[QB], alpha[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    l_run[qb] = 0.0f;
    alpha[qb] = 1.0f;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[cb][qb] = f32x16{};
  }
  f32x16 sa[KB][QB], sb[KB][QB];  // scores of the current and the next tile (ping-pong)
  u32x4 pf[QB][PT];               // bf16 P of the current tile, B operand layout of P.V

  // ---- score-tile helpers -----------------------------------------------------------------
  // Mask tile `tile` of scores in place: key > query + coff (causal) or key >= Tk become -inf.
  // Register r of key block kb holds key kt0 + 4*hf + off with off = 32*kb + 8*(r/4) + r%4, a
  // compile-time constant. The key is visible iff key <= last, last = min(query + coff, Tk-1)
  // (causal) or Tk-1, so each score needs one compare of the constant against a per-lane bound.
  auto mask_tile = [&](f32x16 (&s)[KB][QB], int tile) {
    const int kt0 = tile * BN;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int qi = qw0 + 32 * qb + n;
      const int last = C::CAUSAL ? min(qi + coff, Tk - 1) : Tk - 1;
      const int bound = last - kt0 - 4 * hf;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = 32 * kb + 8 * (r >> 2) + (r & 3);
          s[kb][qb][r] = off <= bound ? s[kb][qb][r] : -__builtin_inff();
        }
    }
  };
  auto needs_mask = [&](int tile) {
    const int kt0 = tile * BN;
    return (C::CAUSAL && kt0 + BN - 1 > qw0 + coff) || (kt0 + BN > Tk);
  };
  // One pair of scores -> exp2, fp32 row sum, packed bf16 P. Pair p covers registers 2*(p%8), +1
  // of key block p/8, i.e. element p%4 of P^T k-step p/4.
  auto exp_pair = [&](f32x16 (&s)[KB][QB], int qb, int p, float neg_m, float& lsum) {
    const int kb = p >> 3, r = (p & 7) * 2;
    const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][qb][r], scale_log2, neg_m));
    const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][qb][r + 1], scale_log2, neg_m));
    lsum = p == 0 ? p0 + p1 : lsum + (p0 + p1);  // the first pair starts the sum
    uint32_t pk = pack_bf16x2(p0, p1);
    // keep this pair's work in the slot it was placed in (the optimizer would otherwise sink it
    // towards its P.V use, past the slots whose MFMAs it is meant to overlap)
    asm volatile("" : "+v"(pk), "+v"(lsum));
    pf[qb][p >> 2][p & 3] = pk;
  };
  // Apply the pending rescale to registers [r0, r1) of every output block of query block qb.
  auto rescale_chunk = [&](int qb, int r0, int r1) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int r = r0; r < r1; ++r) acc[cb][qb][r] *= alpha[qb];
  };
  // Row max (raw scores) over registers [r0, r1) of every key block.
  auto max_chunk = [&](f32x16 (&s)[KB][QB], int qb, int r0, int r1, float& mx) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = r0; r < r1; ++r) mx = fmaxf(mx, s[kb][qb][r]);
  };
  // Online-softmax max update from the row max mx (raw scores, this lane's half) of the next tile:
  // the new max (scaled, base 2); the factor alpha = exp2(m_old - m_new) for acc and l is applied
  // while that tile is processed. A fully masked row chunk has mx = -inf and leaves m unchanged.
  auto new_max = [&](float mx, float m_old) {
    return max_f32(m_old, wave_max_halves(mx) * scale_log2);  // scale_log2 > 0 keeps the max
  };
  auto read_k = [&](int buf_off, int kb, int s) {
    return *reinterpret_cast<const bf16x8*>(smem + buf_off + kb * 32 * RB + k_off[s]);
  };
  auto read_v = [&](int buf_off, int t, int cb, int rr) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)(smem + buf_off + t * 16 * RB + v_off[cb][rr]));
  };
  auto pv_mfma = [&](int cb, int t, s16x4 lo, s16x4 hi) {
    const bf16x8 vfrag =
        __builtin_bit_cast(bf16x8, s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
      acc[cb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfrag, __builtin_bit_cast(bf16x8, pf[qb][t]),
                                                           acc[cb][qb], 0, 0, 0);
  };

  // ---- prologue: tiles 0 (K, V) and 1 (K) in LDS; S(0) = K(0) Q^T; first row max.
  vmem_wait<0>();
  __syncthreads();
  if (tail_ragged && n_tiles - 1 <= C::NSTAGE - 2) {  // the last V tile came with the prologue
    zero_v_tail(C::VRING + buf_of(n_tiles - 1) * C::SLOT_BYTES + last_sub * C::TILE_BYTES);
    __syncthreads();
  }
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) sa[kb][qb] = f32x16{};
  if (wave_active) {
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const bf16x8 kf = read_k(buf_of(0) * C::SLOT_BYTES, kb, s);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          sa[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qb][s], sa[kb][qb], 0, 0, 0);
      }
  }
  __syncthreads();  // every wave has read K(0) before K(2) is copied into its buffer
  if (wave_active && needs_mask(tile_at(0))) mask_tile(sa, tile_at(0));
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    float mx = -__builtin_inff();
    max_chunk(sa, qb, 0, 16, mx);
    m_run[qb] = wave_max_halves(mx) * scale_log2;  // dense: key 0 is visible to every row: finite
    // block-sparse, key ranges, key split: a row may see no key of its first tile (or of any); a
    // finite floor keeps exp2(s - m) at 0 for masked scores instead of NaN, and the floor is left
    // behind (with alpha = 0) as soon as the row sees a key
    if constexpr (C::FLOORED) m_run[qb] = max_f32(m_run[qb], kSparseMaxFloor);
  }

  // ---- one pipelined step: softmax + P.V of tile j (scores in s_cur, V at LDS offset VR) while
  // the scores of tile j+1 (K at KR) go into s_nxt. Copies K(j+NSTAGE) -> KW and
  // V(j+NSTAGE-1) -> VW (both buffers were consumed in the previous step).
  auto step = [&](int j, int KR, int VR, int KW, int VW, f32x16 (&s_cur)[KB][QB],
                  f32x16 (&s_nxt)[KB][QB]) {
    // past the end: harmless re-copies of the last tile into a buffer nobody reads any more
    dma_step(kg, min(j + C::NSTAGE, n_tiles - 1), KW);
    dma_step(vg, min(j + C::NSTAGE - 1, n_tiles - 1), VW);

    if (wave_active) {
      float neg_m[QB], lsum[QB], mx[QB], m_spec[QB], a_spec[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        neg_m[qb] = -m_run[qb];
        l_run[qb] *= alpha[qb];
        lsum[qb] = 0.0f;
        mx[qb] = -__builtin_inff();
      }
      const int tile_next = tile_at(j + 1);
      const bool mask_next = needs_mask(tile_next);
      bool any_alpha = false;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) any_alpha |= alpha[qb] != 1.0f;
      const bool need_rescale = __builtin_amdgcn_ballot_w64(any_alpha) != 0;

      // LDS fragment of slot b: one K read (score slots) or two transposing V reads (P.V slots).
      bf16x8 kfr[NS_QK];
      s16x4 vfr[C::NS_PV][2];
      auto issue = [&](auto b_) {
        constexpr int b = decltype(b_)::value;
        if constexpr (b < NS_QK) {
          kfr[b] = read_k(KR, b % KB, b / KB);
        } else {
          constexpr int t = (b - NS_QK) / CB, cb = (b - NS_QK) % CB;
          vfr[b - NS_QK][0] = read_v(VR, t, cb, 0);
          vfr[b - NS_QK][1] = read_v(VR, t, cb, 1);
        }
      };
      static_for<0, PD>([&](auto b_) { issue(b_); });

      static_for<0, NS>([&](auto b_) {
        constexpr int b = decltype(b_)::value;
        // prefetch the fragments of slot b+PD (the compiler waits for slot b's before its MFMA)
        if constexpr (b + PD < NS) issue(std::integral_constant<int, b + PD>{});
        if constexpr (b < NS_QK) {
          constexpr int s = b / KB, kb = b % KB;
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            s_nxt[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                kfr[b], qf[qb][s], s == 0 ? f32x16{} : s_nxt[kb][qb], 0, 0, 0);
        } else {
          constexpr int t = (b - NS_QK) / CB, cb = (b - NS_QK) % CB;
          pv_mfma(cb, t, vfr[b - NS_QK][0], vfr[b - NS_QK][1]);
        }
        // VALU work of this slot: the exp pairs assigned to it ...
        if constexpr (b < C::EXP_WINDOW) {
          constexpr int p_lo = (b * C::NPAIRS + C::EXP_WINDOW - 1) / C::EXP_WINDOW;
          constexpr int p_hi = ((b + 1) * C::NPAIRS + C::EXP_WINDOW - 1) / C::EXP_WINDOW;
          static_for<p_lo, (p_hi < C::NPAIRS ? p_hi : C::NPAIRS)>([&](auto p_) {
            constexpr int p = decltype(p_)::value;
            static_assert(NS_QK + (p / 4) * CB > b, "exp pair scheduled after its P.V slot");
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) exp_pair(s_cur, qb, p, neg_m[qb], lsum[qb]);
          });
        }
        // ... the pending rescale of acc, in the first slot and skipped when no row of the wave has
        // a new max (alpha is then exactly 1 in every lane: a wave-uniform branch) ...
        if constexpr (b == 0) {
          if (need_rescale) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) rescale_chunk(qb, 0, 16);
          }
        }
        // ... and, once the next scores are complete, a chunk of their row max, then the new max and
        // alpha (assuming the tile needs no mask; masked tiles redo this after the slots).
        if constexpr (b >= C::MAX_FIRST && b <= C::MAX_LAST) {
          constexpr int nmax = C::MAX_LAST - C::MAX_FIRST + 1;
          constexpr int r0 = (b - C::MAX_FIRST) * 16 / nmax, r1 = (b - C::MAX_FIRST + 1) * 16 / nmax;
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            max_chunk(s_nxt, qb, r0, r1, mx[qb]);
            // keep the chunk in this slot (otherwise it sinks past the edge-tile branch below)
            asm volatile("" : "+v"(mx[qb]));
          }
        }
        if constexpr (b == NS - 2) {
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            m_spec[qb] = new_max(mx[qb], m_run[qb]);
            asm volatile("" : "+v"(m_spec[qb]));
          }
        }
        if constexpr (b == NS - 1) {
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            a_spec[qb] = __builtin_amdgcn_exp2f(m_run[qb] - m_spec[qb]);
            asm volatile("" : "+v"(a_spec[qb]));
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      });

#pragma unroll
      for (int qb = 0; qb < QB; ++qb) l_run[qb] += lsum[qb];
      if (mask_next) {  // diagonal or ragged tile: mask, then take the row max again
        mask_tile(s_nxt, tile_next);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          float m = -__builtin_inff();
          max_chunk(s_nxt, qb, 0, 16, m);
          m_spec[qb] = new_max(m, m_run[qb]);
          a_spec[qb] = __builtin_amdgcn_exp2f(m_run[qb] - m_spec[qb]);
        }
      }
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        m_run[qb] = m_spec[qb];
        alpha[qb] = a_spec[qb];
      }
    }  // wave_active
    // the copies of the previous step (K(j+NSTAGE-1), V(j+NSTAGE-2)) have landed; this step's may
    // still be in flight. The barrier publishes them and closes every wave's reads of K(j+1), V(j).
    vmem_wait<2 * C::LOADS * (C::NSTAGE - 2)>();
    __syncthreads();
    if (tail_ragged && j + 2 == n_tiles && n_tiles - 1 > C::NSTAGE - 2) {  // V(n-1) just landed
      zero_v_tail(C::VRING + buf_of(n_tiles - 1) * C::SLOT_BYTES + last_sub * C::TILE_BYTES);
      __syncthreads();
    }
  };

  // ---- last tile: softmax and P.V only.
  auto last_step = [&](int VR, f32x16 (&s_cur)[KB][QB]) {
    if (!wave_active) return;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float lsum = 0.0f;
      const float neg_m = -m_run[qb];
      rescale_chunk(qb, 0, 16);
#pragma unroll
      for (int p = 0; p < C::NPAIRS; ++p) exp_pair(s_cur, qb, p, neg_m, lsum);
      l_run[qb] = l_run[qb] * alpha[qb] + lsum;
    }
#pragma unroll
    for (int t = 0; t < PT; ++t)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) pv_mfma(cb, t, read_v(VR, t, cb, 0), read_v(VR, t, cb, 1));
  };

  // The loop is unrolled by two so the score ping-pong needs no register copies, and it has a
  // single exit with the last scores in sa: two exits (one per parity) would keep both register
  // sets of the output accumulator and of the scores live through the whole loop. An odd number
  // of steps runs its first step before the loop and moves its scores into sa once.
  int ring_j = ring0;  // buffer of tile j
  auto nxt = [](int r) { return r + 1 == C::NSTAGE ? 0 : r + 1; };
  auto run_step = [&](int j, f32x16 (&s_cur)[KB][QB], f32x16 (&s_nxt)[KB][QB]) {
    const int r1 = nxt(ring_j);                       // (j+1) % NSTAGE
    const int rv = C::NSTAGE == 2 ? r1 : nxt(r1);     // (j+NSTAGE-1) % NSTAGE
    step(j, r1 * C::SLOT_BYTES, C::VRING + ring_j * C::SLOT_BYTES, ring_j * C::SLOT_BYTES,
         C::VRING + rv * C::SLOT_BYTES, s_cur, s_nxt);
    ring_j = r1;
  };
  const int n_steps = n_tiles - 1;  // pipelined steps; the last tile is finished by last_step
  int j0 = 0;
  if (n_steps & 1) {
    run_step(0, sa, sb);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) sa[kb][qb] = sb[kb][qb];
    j0 = 1;
  }
  if (C::NSTAGE == 2) ring_j = 0;  // tile j0 sits in buffer 0 (see ring0)
  for (int j = j0; j < n_steps; j += 2) {
    run_step(j, sa, sb);
    run_step(j + 1, sb, sa);
  }
  last_step(C::VRING + ring_j * C::SLOT_BYTES, sa);
  // Copies issued by the last steps may still be in flight (re-copies past the end); they must land
  // before this workgroup's LDS can be handed to another one.
  vmem_wait<0>();
  if (!wave_active) return;  // no query row to store
  float l_tot[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) l_tot[qb] = wave_sum_halves(l_run[qb]);

  // ---- key split: the two waves of a query block saw disjoint sets of keys; the second hands its
  // (acc, m, l) to the first through LDS (the rings are free once every wave is past its last
  // tile), which merges them in log space: m = max(m0, m1), acc = acc0 2^(m0-m) + acc1 2^(m1-m),
  // l likewise. Lane (n, hf) of both waves holds the same query and channels.
  if constexpr (C::KSPLIT > 1) {
    constexpr int NX = 16 * CB + 2;  // floats per lane: acc, m, l
    float* xch = reinterpret_cast<float*>(smem) + wq * NX * 64 + lane;
    __syncthreads();
    if (part != 0) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) xch[(16 * cb + r) * 64] = acc[cb][0][r];
      xch[(16 * CB) * 64] = m_run[0];
      xch[(16 * CB + 1) * 64] = l_tot[0];
    }
    __syncthreads();
    if (part != 0) return;
    const float m1 = xch[(16 * CB) * 64], l1 = xch[(16 * CB + 1) * 64];
    const float m = max_f32(m_run[0], m1);
    const float a0 = __builtin_amdgcn_exp2f(m_run[0] - m), a1 = __builtin_amdgcn_exp2f(m1 - m);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[cb][0][r] = acc[cb][0][r] * a0 + xch[(16 * cb + r) * 64] * a1;
    l_tot[0] = l_tot[0] * a0 + l1 * a1;
    m_run[0] = m;
  }

  // ---- epilogue: O = acc / l, rounded once to bf16; LSE = ln2 * (m + log2 l).
  // Lane (n, hf) of channel block cb holds channels (D/2)*hf + 16*cb + r, r = 0..15, in order.
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = qw0 + 32 * qb + n;
    float inv = 1.0f / l_tot[qb];
    if constexpr (C::LISTED) inv = l_tot[qb] > 0.0f ? inv : 0.0f;  // a row that saw no key: O = 0
    if (row < T) {
      if constexpr (C::RANGE) {  // partial output of a key range: fp32
        float* orow = reinterpret_cast<float*>(o) + head_off + (int64_t)row * D;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
          for (int c4 = 0; c4 < 4; ++c4) {
            f32x4 out;
#pragma unroll
            for (int e = 0; e < 4; ++e) out[e] = acc[cb][qb][4 * c4 + e] * inv;
            *reinterpret_cast<f32x4*>(orow + (D / 2) * hf + 16 * cb + 4 * c4) = out;
          }
      } else {
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
      }
      float lse_row = (m_run[qb] + __log2f(l_tot[qb])) * kLn2;
      if constexpr (C::LISTED) lse_row = l_tot[qb] > 0.0f ? lse_row : -__builtin_inff();
      if (hf == 0) lse[(int64_t)bh * T + row] = lse_row;
    }
  }
}

}  // namespace fa
