// Host side of libfa.so: argument checks, the tile table, the launch plan and the kernel launches.
// Declarations and the contract of every entry point are in include/fa.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <mutex>
#include <tuple>

#include "fa.h"
#include "fa_bwd_kernel.hpp"
#include "fa_fp8_kernel.hpp"
#include "fa_kernel.hpp"
#include "fa_merge_kernel.hpp"

// Fixed device buffer of fa_fwd_splitkv_noalloc: the fp32 partial results of the key ranges, for
// callers that cannot allocate. Every GPU the library runs on holds its own copy until the process
// ends. In host code `scratch` names a host-side stand-in, not device memory: its device address on
// the current GPU comes from hipGetSymbolAddress, looked up once per device (scratch_address below).
static __device__ __align__(256) char scratch[FA_NOALLOC_SCRATCH_BYTES];

namespace {

// Launches `fn` on `stream` with the given arguments (each converted to the kernel's parameter type)
// and returns the status of this launch itself, not whatever error an earlier, unrelated HIP call
// may have left for hipGetLastError.
template <typename... P, typename... A>
int launch_kernel(void (*fn)(P...), dim3 grid, dim3 block, void* stream, A... a) {
  static_assert(sizeof...(P) == sizeof...(A), "one argument per kernel parameter");
  std::tuple<P...> vals(static_cast<P>(a)...);
  void* ptrs[sizeof...(P)];
  std::apply([&ptrs](P&... x) {
    int i = 0;
    ((ptrs[i++] = static_cast<void*>(&x)), ...);
  }, vals);
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(fn), grid, block, ptrs, 0,
                                       static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

// Grid of n workgroups of `threads` work-items (times `splits` in y). The dispatch counts
// work-items per dimension in 32 bits, so above (2^32 - 1) / threads workgroups the 1-D grid is
// folded into x (a multiple of 8) and z; the kernels recover the flat index and let the workgroups
// past n exit. FA_ERR_INVALID_ARG when even the folded grid does not fit (n >= 2^31, or z > 65535).
int fold_grid(int64_t n, int threads, int splits, dim3* grid) {
  const int64_t max_x = (int64_t)UINT32_MAX / threads;
  if (n <= 0 || n > INT32_MAX || splits < 1 || splits > 65535) return FA_ERR_INVALID_ARG;
  if (n <= max_x) {
    *grid = dim3((unsigned)n, (unsigned)splits, 1u);
    return FA_OK;
  }
  const int64_t max_x8 = max_x & ~(int64_t)7;
  const int64_t z = (n + max_x8 - 1) / max_x8;
  const int64_t x = ((n + z - 1) / z + 7) & ~(int64_t)7;  // <= max_x8; fewer than 8 * z spare
  if (z > 65535) return FA_ERR_INVALID_ARG;
  *grid = dim3((unsigned)x, (unsigned)splits, (unsigned)z);
  return FA_OK;
}

using KernelFn = void (*)(const __bf16*, const __bf16*, const __bf16*, __bf16*, float*, int, int, int,
                          float, const uint8_t*, int, int, int, int, int, int);

// Heads per group within an XCD (see map_block): the largest divisor of B*H/8 whose K and V fit in
// a byte budget, so that the XCD's workgroups stream the K/V of that many heads at a time. Used only
// when B*H is a multiple of 8.
// - Non-causal, where every workgroup has the same work: half of the XCD's 4 MB L2, so that a
//   group's Q blocks share its K/V tiles in L2 (B4 H16 T8192 d128: 1105-1108 against 1076-1103
//   TFLOP/s on two boxes; non-causal d64 shapes 0.2-0.4% faster).
// - Causal: 16 MB. The heads of a group are interleaved so that the Q blocks with the most tiles
//   start first and the short ones fill the end, and grouping fewer heads than the budget allows
//   leaves XCDs idle at the end of each group (B4 H12 T4096 d64, 1 MB of K/V per head: 652-737
//   against 796 TFLOP/s). Beyond the budget (the K/V that eight XCDs stream at once no longer fit
//   in half of the 256 MB last-level cache, a reading consistent with these measurements) larger
//   groups lose time: with all heads interleaved, B4 H16 T32768 d64 (8 MB per head) ran
//   at 881-917 TFLOP/s against 941-948 in groups of 2 or 4, B4 H16 T16384 d128 at 984-995 against
//   1065-1081, B1 H32 T65536 d64 (16 MB) at 933-959 against 953-965 in groups of 1 or 2; at
//   B4 H12 T16384 d64 (4 MB) groups of 3 and all 6 heads are level (909-920), and at T8192 d64
//   (2 MB) all 6 heads are fastest (875-878 against 871-876 for 3, 834-840 for 2).
// The backward kernels take the same groups, and so does the FP8 forward with its one-byte K and V
// (elem_bytes = 1; non-causal B4 H16 T8192 d128: 1801-1811 against 1784-1785), and the block-sparse
// forward (causal, 25% of the blocks: B4 H12 T16384 d64 0.517-0.518 against 0.531 ms with all heads
// interleaved, B4 H16 T32768 d64 2.59-2.61 against 2.91 ms).
constexpr int64_t kHeadGroupBytes = int64_t{2} << 20;
constexpr int64_t kCausalHeadGroupBytes = int64_t{16} << 20;

int head_group(int64_t BH, int64_t Tk, int d, bool causal, int elem_bytes = 2) {
  if (BH <= 0 || BH % 8 != 0) return 1;  // (an empty problem launches nothing)
  const int per = (int)(BH / 8);
  const int64_t kv = std::max<int64_t>(Tk * d * elem_bytes * 2, 1);
  const int64_t gmax = std::max<int64_t>(1, (causal ? kCausalHeadGroupBytes : kHeadGroupBytes) / kv);
  int g = per;
  while (g > 1 && (g > gmax || per % g != 0)) --g;
  return g;
}

struct TileEntry {
  int d, block_m, block_n, waves;
  KernelFn causal_fn, full_fn;
  int lds_bytes;
  int key_split;  // waves sharing one 32-query block, each on every key_split-th K/V tile
};

template <int D, int QB, int NW, int BN, int NSTAGE = 2, int KSPLIT = 1>
constexpr TileEntry entry() {
  using Cc = fa::Cfg<D, QB, NW, BN, true, NSTAGE, false, false, false, KSPLIT>;
  using Cf = fa::Cfg<D, QB, NW, BN, false, NSTAGE, false, false, false, KSPLIT>;
  return TileEntry{D, Cc::BM, BN, NW, &fa::fa_fwd_kernel<Cc>, &fa::fa_fwd_kernel<Cf>, Cc::LDS_BYTES,
                   KSPLIT};
}

// Supported tile shapes. The first entry for each d is the default (see default_tile()).
const TileEntry kTiles[] = {
    entry<64, 1, 4, 64>(),   // d=64: 128 queries (4 waves x 32), 64-key tiles
    entry<64, 1, 4, 128>(),  // d=64: 128 queries (4 waves x 32), 128-key tiles
    entry<64, 1, 2, 64>(),   // d=64: 64 x 64, the tile shape of the tutorial page
    entry<64, 2, 2, 64>(),   // d=64: 128 queries (2 waves x 64)
    entry<64, 2, 4, 64>(),   // d=64: 256 queries (4 waves x 64)
    entry<64, 1, 8, 64>(),   // d=64: 256 queries (8 waves x 32)
    entry<64, 1, 4, 64, 2, 2>(),  // d=64: 64 queries, two waves per 32 queries splitting the keys
    entry<128, 1, 4, 64>(),  // d=128: 128 queries (4 waves x 32), 64-key tiles
    entry<128, 1, 2, 64>(),  // d=128: 64 x 64
    entry<128, 1, 8, 64>(),  // d=128: 256 queries (8 waves x 32), 64-key tiles
};

const TileEntry* find_tile(int d, int block_m, int block_n, int waves) {
  for (const TileEntry& t : kTiles)
    if (t.d == d && t.block_m == block_m && t.block_n == block_n && t.waves == waves) return &t;
  return nullptr;
}

// The d = 64 default depends on the grid of the 128 x 64 launch (nq = ceil(T/128) Q blocks per head,
// grid = nq * B * H workgroups). Measured on one box (time relative to 128 x 64 x 4):
// - the key split (two waves per 32-query block, each on every other K/V tile; 64 queries and 64 KB
//   of LDS per workgroup, two per compute unit) halves the path of a head's last Q block at the cost
//   of twice the workgroups. Causal: 0.73-0.75 at nq 8 up to grid 288, 0.77-0.83 at nq 16-32 and
//   grid 384, but 0.96 at nq 8 and grid 384 and 0.93-0.94 at grid 512. Non-causal: 0.77 at grid 96,
//   0.91-0.95 at grid 384.
// - 128-key tiles (230 VGPRs, two workgroups per compute unit, half the barriers and loop steps per
//   key) win on short heads: causal 0.89-0.92 at grid 96-512, 0.96-0.98 at nq 8 up to grid 1536 and
//   at nq 16 and grid 768; non-causal 0.89-0.93 at grid 384; but 1.01-1.07 at nq 4, at nq 16 and grid
//   1536 and at nq 32 and grid 1536.
// The rules below take the faster of the three in each measured region.
bool take_key_split(int64_t nq, int64_t grid, bool causal) {
  if (causal) return nq >= 8 && grid <= 384 && (nq >= 16 || grid <= 288);
  return grid <= 256;
}

bool take_wide_key_tiles(int64_t nq, int64_t grid) {
  return nq >= 5 && (nq <= 8 || grid <= 768);
}

// d = 128, non-causal, T >= 2048: 256 queries in 8 waves per workgroup share each K/V tile copied to
// LDS (half the copies per query; 222 VGPRs, one workgroup of 8 waves per CU). Measured against
// 128 x 64 x 4: 0.964-0.977 non-causal (B1-B4 H16, T = 4096 and 8192), 0.991-1.002 causal (kept).
const TileEntry* default_tile(int d, int T, int64_t BH, bool causal) {
  if (d == 128 && !causal && T >= 2048) {
    const TileEntry* t = find_tile(128, 256, 64, 8);
    if (t) return t;
  }
  if (d == 64) {
    const int64_t nq = (T + 127) / 128, grid = nq * BH;
    const TileEntry* t = nullptr;
    if (take_key_split(nq, grid, causal)) t = find_tile(64, 64, 64, 4);
    else if (take_wide_key_tiles(nq, grid)) t = find_tile(64, 128, 128, 4);
    if (t) return t;
  }
  for (const TileEntry& t : kTiles)
    if (t.d == d) return &t;
  return nullptr;
}

int check_sizes(int B, int H, int T, int d) {
  if (B < 0 || H < 0 || T < 0) return FA_ERR_INVALID_ARG;
  if (T > FA_MAX_T) return FA_ERR_INVALID_ARG;
  if ((int64_t)B * H > FA_MAX_BH) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED_D;
  return FA_OK;
}

int resolve_tile(int d, int T, int64_t BH, bool causal, int block_m, int block_n, int waves,
                 const TileEntry** out) {
  if (block_m == 0 && block_n == 0 && waves == 0) {
    *out = default_tile(d, T, BH, causal);
  } else {
    if (block_m <= 0 || block_n <= 0 || waves <= 0) return FA_ERR_TILE;
    *out = find_tile(d, block_m, block_n, waves);
  }
  return *out ? FA_OK : FA_ERR_TILE;
}

// The kernels take the scores into exp2 as s * (scale * log2 e) in fp32, so that factor must be a
// finite positive fp32 number too (scale below about 2.36e38), not only scale itself.
bool scale_ok(float scale) {
  return std::isfinite(scale) && scale > 0.0f && std::isfinite(scale * fa::kLog2e);
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return na && nb && x < y + nb && y < x + na;
}

int launch(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int T, int d,
           int causal, float scale, void* stream, int block_m, int block_n, int waves) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  int rc = check_sizes(B, H, T, d);
  if (rc != FA_OK) return rc;
  if (!scale_ok(scale)) return FA_ERR_INVALID_ARG;
  const TileEntry* tile = nullptr;
  rc = resolve_tile(d, T, (int64_t)B * H, causal != 0, block_m, block_n, waves, &tile);
  if (rc != FA_OK) return rc;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15u) return FA_ERR_ALIGNMENT;
  if ((uintptr_t)lse & 3u) return FA_ERR_ALIGNMENT;
  const size_t n_elem = (size_t)B * H * T * d;
  const size_t bytes = n_elem * 2, lse_bytes = (size_t)B * H * T * 4;
  if (overlaps(o, bytes, q, bytes) || overlaps(o, bytes, k, bytes) || overlaps(o, bytes, v, bytes) ||
      overlaps(lse, lse_bytes, q, bytes) || overlaps(lse, lse_bytes, k, bytes) ||
      overlaps(lse, lse_bytes, v, bytes) || overlaps(lse, lse_bytes, o, bytes))
    return FA_ERR_INVALID_ARG;
  if (n_elem == 0) return FA_OK;

  const int nq = (T + tile->block_m - 1) / tile->block_m;
  const int BH = B * H;
  dim3 grid;
  if (fold_grid((int64_t)nq * BH, 64 * tile->waves, 1, &grid) != FA_OK) return FA_ERR_INVALID_ARG;
  const float scale_log2 = scale * fa::kLog2e;
  KernelFn fn = causal ? tile->causal_fn : tile->full_fn;
  return launch_kernel(fn, grid, dim3(64 * tile->waves), stream,
                       (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (__bf16*)o, lse, T, nq, BH,
                       scale_log2, (const uint8_t*)nullptr, 0, 0, 0, 0, 0, head_group(BH, T, d, causal != 0));
}

// Block-sparse forward: the default tile shape (128 queries x 64 keys per tile, 4 waves) with the
// tile list built from the caller's mask.
template <int D>
struct SparseFns {
  using Cc = fa::Cfg<D, 1, 4, 64, true, 2, true>;
  using Cf = fa::Cfg<D, 1, 4, 64, false, 2, true>;
  static_assert(Cc::BM == FA_SPARSE_BLOCK_M && Cc::BN == FA_SPARSE_BLOCK_N, "mask blocks = tiles");
  static_assert(Cc::MAX_LIST * Cc::BN >= FA_SPARSE_MAX_T, "tile list capacity");
};

int launch_sparse(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                  int T, int d, int causal, float scale, const unsigned char* block_mask,
                  int mask_heads, void* stream) {
  if (!q || !k || !v || !o || !lse || !block_mask) return FA_ERR_NULL;
  int rc = check_sizes(B, H, T, d);
  if (rc != FA_OK) return rc;
  if (T > FA_SPARSE_MAX_T) return FA_ERR_INVALID_ARG;
  if (mask_heads != 1 && (int64_t)mask_heads != (int64_t)B * H) return FA_ERR_INVALID_ARG;
  if (!scale_ok(scale)) return FA_ERR_INVALID_ARG;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15u) return FA_ERR_ALIGNMENT;
  if ((uintptr_t)lse & 3u) return FA_ERR_ALIGNMENT;
  const size_t n_elem = (size_t)B * H * T * d;
  const size_t bytes = n_elem * 2, lse_bytes = (size_t)B * H * T * 4;
  const int nq = (T + FA_SPARSE_BLOCK_M - 1) / FA_SPARSE_BLOCK_M;
  const int nk = (T + FA_SPARSE_BLOCK_N - 1) / FA_SPARSE_BLOCK_N;
  const size_t mask_bytes = (size_t)mask_heads * nq * nk;
  const void* ins[4] = {q, k, v, block_mask};
  const size_t in_bytes[4] = {bytes, bytes, bytes, mask_bytes};
  for (int a = 0; a < 4; ++a)
    if (overlaps(o, bytes, ins[a], in_bytes[a]) || overlaps(lse, lse_bytes, ins[a], in_bytes[a]))
      return FA_ERR_INVALID_ARG;
  if (overlaps(o, bytes, lse, lse_bytes)) return FA_ERR_INVALID_ARG;
  if (n_elem == 0) return FA_OK;
  const int BH = B * H;
  dim3 grid;
  if (fold_grid((int64_t)nq * BH, 256, 1, &grid) != FA_OK) return FA_ERR_INVALID_ARG;
  KernelFn fn;
  if (d == 64) fn = causal ? &fa::fa_fwd_kernel<SparseFns<64>::Cc> : &fa::fa_fwd_kernel<SparseFns<64>::Cf>;
  else fn = causal ? &fa::fa_fwd_kernel<SparseFns<128>::Cc> : &fa::fa_fwd_kernel<SparseFns<128>::Cf>;
  return launch_kernel(fn, grid, dim3(256), stream, (const __bf16*)q,
                       (const __bf16*)k, (const __bf16*)v, (__bf16*)o, lse, T, nq, BH,
                       scale * fa::kLog2e, (const uint8_t*)block_mask, mask_heads, 0, 0, 0, 0,
                       head_group(BH, T, d, causal != 0));
}

// Partial forward over a key range: the default tile with the range selection and fp32 output.
template <int D>
struct RangeFns {
  using Cc = fa::Cfg<D, 1, 4, 64, true, 2, false, true>;
  using Cf = fa::Cfg<D, 1, 4, 64, false, 2, false, true>;
  // fewer queries than one workgroup's 128: the idle waves skip the arithmetic
  using CcFew = fa::Cfg<D, 1, 4, 64, true, 2, false, true, true>;
  using CfFew = fa::Cfg<D, 1, 4, 64, false, 2, false, true, true>;
  static_assert(Cc::BN == FA_PARTIAL_KEY_ALIGN, "key ranges start on tile boundaries");
  static_assert(CcFew::BM == Cc::BM, "same workgroup shape");
};

// Checks shared by the key-range entry points: sizes, the query/key lengths and the alignment of q,
// k, v and the fp32 partial outputs. `parts` partial results of B*H*T rows are written.
int check_partial_args(const void* q, const void* k, const void* v, const float* o_part,
                       const float* lse_part, int B, int H, int T, int Tk, int d, float scale,
                       int64_t parts) {
  if (!q || !k || !v || !o_part || !lse_part) return FA_ERR_NULL;
  int rc = check_sizes(B, H, T, d);
  if (rc != FA_OK) return rc;
  if (Tk < 0 || Tk > FA_MAX_T) return FA_ERR_INVALID_ARG;
  if (!scale_ok(scale)) return FA_ERR_INVALID_ARG;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o_part) & 15u) return FA_ERR_ALIGNMENT;
  if ((uintptr_t)lse_part & 3u) return FA_ERR_ALIGNMENT;
  const size_t rows = (size_t)B * H * T, krows = (size_t)B * H * Tk;
  const size_t qbytes = rows * d * 2, kbytes = krows * d * 2;
  const size_t obytes = (size_t)parts * rows * d * 4, lse_bytes = (size_t)parts * rows * 4;
  const void* ins[3] = {q, k, v};
  const size_t in_bytes[3] = {qbytes, kbytes, kbytes};
  for (int a = 0; a < 3; ++a)
    if (overlaps(o_part, obytes, ins[a], in_bytes[a]) || overlaps(lse_part, lse_bytes, ins[a], in_bytes[a]))
      return FA_ERR_INVALID_ARG;
  if (overlaps(o_part, obytes, lse_part, lse_bytes)) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

// One launch of the key-range kernel: grid x = (Q block, head), grid y = n_splits key ranges of
// k_chunk keys from k_begin (the last one ends at k_end); range s writes partial result s.
int launch_ranges(const void* q, const void* k, const void* v, float* o_part, float* lse_part, int B,
                  int H, int T, int Tk, int d, int causal, float scale, int k_begin, int k_end,
                  int k_chunk, int n_splits, void* stream) {
  const int nq = (T + 127) / 128;
  const int BH = B * H;
  dim3 grid;
  if (fold_grid((int64_t)nq * BH, 256, n_splits, &grid) != FA_OK) return FA_ERR_INVALID_ARG;
  const bool few = T < RangeFns<64>::Cc::BM;
  KernelFn fn;
  if (d == 64)
    fn = few ? (causal ? &fa::fa_fwd_kernel<RangeFns<64>::CcFew> : &fa::fa_fwd_kernel<RangeFns<64>::CfFew>)
             : (causal ? &fa::fa_fwd_kernel<RangeFns<64>::Cc> : &fa::fa_fwd_kernel<RangeFns<64>::Cf>);
  else
    fn = few ? (causal ? &fa::fa_fwd_kernel<RangeFns<128>::CcFew> : &fa::fa_fwd_kernel<RangeFns<128>::CfFew>)
             : (causal ? &fa::fa_fwd_kernel<RangeFns<128>::Cc> : &fa::fa_fwd_kernel<RangeFns<128>::Cf>);
  return launch_kernel(fn, grid, dim3(256), stream,
                       (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (__bf16*)o_part,
                       lse_part, T, nq, BH, scale * fa::kLog2e, (const uint8_t*)nullptr, 0, k_begin,
                       k_end, Tk, k_chunk, BH / 8);
}

int launch_partial(const void* q, const void* k, const void* v, float* o_part, float* lse_part, int B,
                   int H, int T, int Tk, int d, int causal, float scale, int k_begin, int k_end,
                   void* stream) {
  int rc = check_partial_args(q, k, v, o_part, lse_part, B, H, T, Tk, d, scale, 1);
  if (rc != FA_OK) return rc;
  if (k_begin < 0 || k_end < k_begin || k_end > Tk || k_begin % FA_PARTIAL_KEY_ALIGN != 0 ||
      (k_end % FA_PARTIAL_KEY_ALIGN != 0 && k_end != Tk))
    return FA_ERR_INVALID_ARG;
  if ((size_t)B * H * T == 0) return FA_OK;
  return launch_ranges(q, k, v, o_part, lse_part, B, H, T, Tk, d, causal, scale, k_begin, k_end,
                       std::max(k_end - k_begin, 1), 1, stream);
}

// Keys per range when Tk keys are split n_splits ways: equal ranges of whole 64-key tiles.
int split_chunk(int Tk, int n_splits) {
  const int tiles = (Tk + FA_PARTIAL_KEY_ALIGN - 1) / FA_PARTIAL_KEY_ALIGN;
  const int per = std::max(1, (tiles + n_splits - 1) / n_splits);
  return per * FA_PARTIAL_KEY_ALIGN;
}

int splits_used(int Tk, int n_splits) {
  const int chunk = split_chunk(Tk, n_splits);
  return std::max(1, (Tk + chunk - 1) / chunk);
}

int launch_merge_kernel(const float* o_parts, const float* lse_parts, int n_parts, void* o, float* lse,
                        int64_t rows, int d, void* stream);

int launch_merge(const float* o_parts, const float* lse_parts, int n_parts, void* o, float* lse,
                 int B, int H, int T, int d, void* stream) {
  if (!o_parts || !lse_parts || !o || !lse) return FA_ERR_NULL;
  int rc = check_sizes(B, H, T, d);
  if (rc != FA_OK) return rc;
  if (n_parts < 1 || n_parts > FA_MERGE_MAX_PARTS) return FA_ERR_INVALID_ARG;
  if ((((uintptr_t)o_parts | (uintptr_t)o) & 15u) || ((uintptr_t)lse_parts | (uintptr_t)lse) & 3u)
    return FA_ERR_ALIGNMENT;
  const int64_t rows = (int64_t)B * H * T;
  const size_t pbytes = (size_t)n_parts * rows * d * 4, plbytes = (size_t)n_parts * rows * 4;
  const size_t obytes = (size_t)rows * d * 2, lbytes = (size_t)rows * 4;
  if (overlaps(o, obytes, o_parts, pbytes) || overlaps(o, obytes, lse_parts, plbytes) ||
      overlaps(lse, lbytes, o_parts, pbytes) || overlaps(lse, lbytes, lse_parts, plbytes) ||
      overlaps(o, obytes, lse, lbytes))
    return FA_ERR_INVALID_ARG;
  if (rows == 0) return FA_OK;
  return launch_merge_kernel(o_parts, lse_parts, n_parts, o, lse, rows, d, stream);
}

int launch_merge_kernel(const float* o_parts, const float* lse_parts, int n_parts, void* o, float* lse,
                        int64_t rows, int d, void* stream) {
  const int rpb = 256 / (d / 4);
  dim3 grid;
  if (fold_grid((rows + rpb - 1) / rpb, 256, 1, &grid) != FA_OK) return FA_ERR_INVALID_ARG;
  auto fn = d == 64 ? &fa::fa_merge_kernel<64> : &fa::fa_merge_kernel<128>;
  return launch_kernel(fn, grid, dim3(256), stream, o_parts, lse_parts,
                       n_parts, (__bf16*)o, lse, rows);
}

int launch_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                   int T, int Tk, int d, int causal, float scale, int n_splits, void* workspace,
                   size_t workspace_bytes, void* stream) {
  if (!o || !lse || !workspace) return FA_ERR_NULL;
  if (n_splits < 1 || n_splits > FA_MERGE_MAX_PARTS) return FA_ERR_INVALID_ARG;
  int rc = check_sizes(B, H, T, d);
  if (rc != FA_OK) return rc;
  const size_t need = fa_splitkv_workspace_bytes(B, H, T, d, n_splits);
  if (workspace_bytes < need || (need == 0 && (size_t)B * H * T != 0)) return FA_ERR_INVALID_ARG;
  const int64_t rows = (int64_t)B * H * T;
  float* o_parts = static_cast<float*>(workspace);
  float* lse_parts = o_parts + (size_t)n_splits * rows * d;
  rc = check_partial_args(q, k, v, o_parts, lse_parts, B, H, T, Tk, d, scale, n_splits);
  if (rc != FA_OK) return rc;
  if (((uintptr_t)o & 15u) || ((uintptr_t)lse & 3u)) return FA_ERR_ALIGNMENT;
  const size_t obytes = (size_t)rows * d * 2, lbytes = (size_t)rows * 4;
  const void* ins[4] = {q, k, v, workspace};
  const size_t in_bytes[4] = {(size_t)rows * d * 2, (size_t)B * H * Tk * d * 2, (size_t)B * H * Tk * d * 2,
                              need};
  for (int a = 0; a < 4; ++a)
    if (overlaps(o, obytes, ins[a], in_bytes[a]) || overlaps(lse, lbytes, ins[a], in_bytes[a]))
      return FA_ERR_INVALID_ARG;
  if (overlaps(o, obytes, lse, lbytes)) return FA_ERR_INVALID_ARG;
  if (rows == 0) return FA_OK;
  const int used = splits_used(Tk, n_splits);
  rc = launch_ranges(q, k, v, o_parts, lse_parts, B, H, T, Tk, d, causal, scale, 0, Tk,
                     split_chunk(Tk, n_splits), used, stream);
  if (rc != FA_OK) return rc;
  return launch_merge_kernel(o_parts, lse_parts, used, o, lse, rows, d, stream);
}

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];  // per device; null until looked up
std::mutex g_scratch_mu;

// Device address of `scratch` on the calling thread's current device.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_HIP;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return FA_ERR_HIP;
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return FA_OK;
}

int launch_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                           int H, int T, int Tk, int d, int causal, float scale, int n_splits,
                           void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (n_splits < 1 || n_splits > FA_MERGE_MAX_PARTS) return FA_ERR_INVALID_ARG;
  int rc = check_sizes(B, H, T, d);
  if (rc != FA_OK) return rc;
  if (Tk < 0 || Tk > FA_MAX_T) return FA_ERR_INVALID_ARG;
  if (!scale_ok(scale)) return FA_ERR_INVALID_ARG;
  if ((((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15u) || ((uintptr_t)lse & 3u))
    return FA_ERR_ALIGNMENT;
  if ((size_t)B * H * T == 0) return FA_OK;  // an empty problem: nothing launched, no scratch used
  const size_t need = fa_splitkv_workspace_bytes(B, H, T, d, n_splits);
  if (need == 0 || need > FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_SCRATCH;
  void* ws = nullptr;
  rc = scratch_address(&ws);
  if (rc != FA_OK) return rc;
  return launch_splitkv(q, k, v, o, lse, B, H, T, Tk, d, causal, scale, n_splits, ws,
                        FA_NOALLOC_SCRATCH_BYTES, stream);
}

// FP8 forward: E4M3 inputs with per-tensor descale factors, 128 queries x 64 keys per tile.
int launch_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int T,
               int d, int causal, float scale, float q_descale, float k_descale, float v_descale,
               void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  int rc = check_sizes(B, H, T, d);
  if (rc != FA_OK) return rc;
  const float fs[4] = {scale, q_descale, k_descale, v_descale};
  for (float x : fs)
    if (!std::isfinite(x) || !(x > 0.0f)) return FA_ERR_INVALID_ARG;
  const double sl2 = (double)scale * q_descale * k_descale * 1.4426950408889634;
  if (!(sl2 < 3.0e38) || !(sl2 > 1.0e-37)) return FA_ERR_INVALID_ARG;  // fp32 range of the factor
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15u) return FA_ERR_ALIGNMENT;
  if ((uintptr_t)lse & 3u) return FA_ERR_ALIGNMENT;
  const size_t n_elem = (size_t)B * H * T * d;
  const size_t in_bytes = n_elem, o_bytes = n_elem * 2, lse_bytes = (size_t)B * H * T * 4;
  const void* ins[3] = {q, k, v};
  for (int a = 0; a < 3; ++a)
    if (overlaps(o, o_bytes, ins[a], in_bytes) || overlaps(lse, lse_bytes, ins[a], in_bytes))
      return FA_ERR_INVALID_ARG;
  if (overlaps(o, o_bytes, lse, lse_bytes)) return FA_ERR_INVALID_ARG;
  if (n_elem == 0) return FA_OK;
  const int nq = (T + 127) / 128;
  const int BH = B * H;
  dim3 grid;
  if (fold_grid((int64_t)nq * BH, 256, 1, &grid) != FA_OK) return FA_ERR_INVALID_ARG;
  using Fn8 = void (*)(const uint8_t*, const uint8_t*, const uint8_t*, __bf16*, float*, int, int, int,
                       float, float, int);
  Fn8 fn;
  if (d == 64)
    fn = causal ? &fa::fa_fwd_fp8_kernel<fa::Fp8Cfg<64, true>> : &fa::fa_fwd_fp8_kernel<fa::Fp8Cfg<64, false>>;
  else
    fn = causal ? &fa::fa_fwd_fp8_kernel<fa::Fp8Cfg<128, true>> : &fa::fa_fwd_fp8_kernel<fa::Fp8Cfg<128, false>>;
  static_assert(fa::Fp8Cfg<64, true>::BM == 128 && fa::Fp8Cfg<128, true>::BM == 128, "Q block");
  return launch_kernel(fn, grid, dim3(256), stream, (const uint8_t*)q,
                       (const uint8_t*)k, (const uint8_t*)v, (__bf16*)o, lse, T, nq, BH, (float)sl2,
                       v_descale, head_group(BH, T, d, causal != 0, 1));
}

template <int D>
int launch_bwd_kernels(const void* q, const void* k, const void* v, const void* o, const float* lse,
                       const void* dout, void* dq, void* dk, void* dv, float* delta, int B, int H,
                       int T, int causal, float scale, void* stream);

int launch_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
               const void* dout, void* dq, void* dk, void* dv, float* delta, int B, int H, int T,
               int d, int causal, float scale, void* stream) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !delta) return FA_ERR_NULL;
  int rc = check_sizes(B, H, T, d);
  if (rc != FA_OK) return rc;
  if (!scale_ok(scale)) return FA_ERR_INVALID_ARG;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)dout |
       (uintptr_t)dq | (uintptr_t)dk | (uintptr_t)dv) & 15u)
    return FA_ERR_ALIGNMENT;
  if (((uintptr_t)lse | (uintptr_t)delta) & 3u) return FA_ERR_ALIGNMENT;
  const size_t n_elem = (size_t)B * H * T * d;
  const size_t bytes = n_elem * 2, sbytes = (size_t)B * H * T * 4;
  const void* ins[6] = {q, k, v, o, dout, lse};
  const size_t in_bytes[6] = {bytes, bytes, bytes, bytes, bytes, sbytes};
  const void* outs[4] = {dq, dk, dv, delta};
  const size_t out_bytes[4] = {bytes, bytes, bytes, sbytes};
  for (int a = 0; a < 4; ++a) {
    for (int b = 0; b < 6; ++b)
      if (overlaps(outs[a], out_bytes[a], ins[b], in_bytes[b])) return FA_ERR_INVALID_ARG;
    for (int b = a + 1; b < 4; ++b)
      if (overlaps(outs[a], out_bytes[a], outs[b], out_bytes[b])) return FA_ERR_INVALID_ARG;
  }
  if (n_elem == 0) return FA_OK;

  return d == 64 ? launch_bwd_kernels<64>(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, T, causal,
                                           scale, stream)
                 : launch_bwd_kernels<128>(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, T, causal,
                                           scale, stream);
}

// The two backward kernels for head dim D: dQ and D first, then dK and dV (which read D).
template <int D>
int launch_bwd_kernels(const void* q, const void* k, const void* v, const void* o, const float* lse,
                       const void* dout, void* dq, void* dk, void* dv, float* delta, int B, int H,
                       int T, int causal, float scale, void* stream) {
  using Cc = fa::BwdCfg<D, true>;
  using Cf = fa::BwdCfg<D, false>;
  const int nb = (T + Cc::BM - 1) / Cc::BM;  // query blocks (dQ kernel) = key blocks (dK/dV kernel)
  const int BH = B * H;
  dim3 grid;
  if (fold_grid((int64_t)nb * BH, Cc::THREADS, 1, &grid) != FA_OK) return FA_ERR_INVALID_ARG;
  const float scale_log2 = scale * fa::kLog2e;
  // heads per group within an XCD, as for the forward: the dQ kernel streams a head's K and V, the
  // dK/dV kernel its Q and dO (as many bytes)
  const int hg = head_group(BH, T, D, causal != 0);
  auto dq_fn = causal ? &fa::fa_bwd_dq_kernel<Cc> : &fa::fa_bwd_dq_kernel<Cf>;
  int rc = launch_kernel(dq_fn, grid, dim3(Cc::THREADS), stream, (const __bf16*)q,
                         (const __bf16*)k, (const __bf16*)v, (const __bf16*)o, lse,
                         (const __bf16*)dout, (__bf16*)dq, delta, T, nb, BH, scale, scale_log2, hg);
  if (rc != FA_OK) return rc;
  auto dkdv = [&](auto fn) {
    return launch_kernel(fn, grid, dim3(Cc::THREADS), stream, (const __bf16*)q, (const __bf16*)k,
                         (const __bf16*)v, lse, (const __bf16*)dout, (const float*)delta, (__bf16*)dk,
                         (__bf16*)dv, T, nb, BH, scale, scale_log2, hg);
  };
  if constexpr (D == 64) {
    // dK and dV in one pass (196 registers, two waves per SIMD). The two passes of d = 128 would
    // fit in 112 and 164 registers here, but their second computation of S and second reads of Q
    // and dO cost more than the extra waves return: 16% slower at causal B4 H12 T4096.
    return dkdv(causal ? &fa::fa_bwd_dkdv_kernel<Cc> : &fa::fa_bwd_dkdv_kernel<Cf>);
  } else {
    // d = 128: one pass for dV, then one for dK. Holding both accumulators and both fragment sets
    // took 319 registers (one wave per SIMD); each single-output pass holds half as much.
    rc = dkdv(causal ? &fa::fa_bwd_dkdv_kernel<Cc, fa::kDV> : &fa::fa_bwd_dkdv_kernel<Cf, fa::kDV>);
    if (rc != FA_OK) return rc;
    return dkdv(causal ? &fa::fa_bwd_dkdv_kernel<Cc, fa::kDK> : &fa::fa_bwd_dkdv_kernel<Cf, fa::kDK>);
  }
}

}  // namespace

extern "C" {

int fa_fwd_sparse(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                  int T, int d, int causal, float scale, const unsigned char* block_mask,
                  int mask_heads, void* stream) {
  return launch_sparse(q, k, v, o, lse, B, H, T, d, causal, scale, block_mask, mask_heads, stream);
}

int fa_fwd_partial(const void* q, const void* k, const void* v, float* o_part, float* lse_part,
                   int B, int H, int T, int Tk, int d, int causal, float scale, int k_begin, int k_end,
                   void* stream) {
  return launch_partial(q, k, v, o_part, lse_part, B, H, T, Tk, d, causal, scale, k_begin, k_end,
                        stream);
}

size_t fa_splitkv_workspace_bytes(int B, int H, int T, int d, int n_splits) {
  if (check_sizes(B, H, T, d) != FA_OK || n_splits < 1 || n_splits > FA_MERGE_MAX_PARTS) return 0;
  // B*H*T <= 2^46 and d + 1 <= 129: one part is below 2^56 bytes
  const size_t per_part = (size_t)B * H * T * ((size_t)d + 1) * 4;
  if (per_part > SIZE_MAX / (size_t)n_splits) return 0;
  return (size_t)n_splits * per_part;
}

int fa_splitkv_splits(int B, int H, int T, int Tk, int d) {
  if (B <= 0 || H <= 0 || T <= 0 || Tk <= 0 || check_sizes(B, H, T, d) != FA_OK || Tk > FA_MAX_T)
    return 1;
  // as many workgroups as two per compute unit hold at once (not more: a second round would wait
  // for the first), with at least 8 key tiles (512 keys) per range and at most 256 ranges: the
  // merge loads a row's parts 16 at a time, so for few rows many parts cost more latency than the
  // finer split saves (one head, 2^20 keys: 85 us with 256 ranges, 92 us with 512, 121 with 128)
  const int64_t base = (int64_t)((T + 127) / 128) * B * H;
  const int64_t want = 512 / base;
  const int64_t most = std::max(1, ((Tk + FA_PARTIAL_KEY_ALIGN - 1) / FA_PARTIAL_KEY_ALIGN) / 8);
  return (int)std::max<int64_t>(1, std::min<int64_t>({want, most, int64_t{256}}));
}

int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                   int T, int Tk, int d, int causal, float scale, int n_splits, void* workspace,
                   size_t workspace_bytes, void* stream) {
  return launch_splitkv(q, k, v, o, lse, B, H, T, Tk, d, causal, scale, n_splits, workspace,
                        workspace_bytes, stream);
}

int fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                           int H, int T, int Tk, int d, int causal, float scale, int n_splits,
                           void* stream) {
  return launch_splitkv_noalloc(q, k, v, o, lse, B, H, T, Tk, d, causal, scale, n_splits, stream);
}

int fa_merge(const float* o_parts, const float* lse_parts, int n_parts, void* o, float* lse, int B,
             int H, int T, int d, void* stream) {
  return launch_merge(o_parts, lse_parts, n_parts, o, lse, B, H, T, d, stream);
}

int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int T,
               int d, int causal, float scale, float q_descale, float k_descale, float v_descale,
               void* stream) {
  return launch_fp8(q, k, v, o, lse, B, H, T, d, causal, scale, q_descale, k_descale, v_descale,
                    stream);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dout, void* dq, void* dk, void* dv, float* delta, int B, int H, int T, int d,
           int causal, float scale, void* stream) {
  return launch_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, T, d, causal, scale, stream);
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int T, int d,
           int causal, float scale, void* stream) {
  return launch(q, k, v, o, lse, B, H, T, d, causal, scale, stream, 0, 0, 0);
}

int fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int T,
              int d, int causal, float scale, void* stream, int block_m, int block_n, int waves) {
  if (block_m == 0 && block_n == 0 && waves == 0) return FA_ERR_TILE;
  return launch(q, k, v, o, lse, B, H, T, d, causal, scale, stream, block_m, block_n, waves);
}

int fa_fwd_plan(int B, int H, int T, int d, int causal, int block_m, int block_n, int waves,
                fa_plan_info* out) {
  if (!out) return FA_ERR_NULL;
  int rc = check_sizes(B, H, T, d);
  if (rc != FA_OK) return rc;
  const TileEntry* tile = nullptr;
  rc = resolve_tile(d, T, (int64_t)B * H, causal != 0, block_m, block_n, waves, &tile);
  if (rc != FA_OK) return rc;
  fa_plan_info p;
  p.block_m = tile->block_m;
  p.block_n = tile->block_n;
  p.waves = tile->waves;
  p.q_blocks = (T + tile->block_m - 1) / tile->block_m;
  p.grid = (long long)p.q_blocks * B * H;
  p.lds_bytes = tile->lds_bytes;
  p.key_split = tile->key_split;
  p.head_group = head_group((int64_t)B * H, T, d, causal != 0);
  // K/V tiles per Q block: up to the diagonal when causal, all of them otherwise.
  long long tiles_per_head = 0;
  for (int qb = 0; qb < p.q_blocks; ++qb) {
    const int kv_end = causal ? std::min((qb + 1) * tile->block_m, T) : T;
    tiles_per_head += (kv_end + tile->block_n - 1) / tile->block_n;
  }
  p.kv_tiles = tiles_per_head * B * H;
  *out = p;
  return FA_OK;
}

const char* fa_strerror(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_INVALID_ARG: return "invalid argument (size out of range, scale not finite and > 0, or overlapping buffers)";
    case FA_ERR_UNSUPPORTED_D: return "unsupported head dimension (d must be 64 or 128)";
    case FA_ERR_ALIGNMENT: return "misaligned pointer (bf16 tensors need 16 bytes; lse and delta need 4)";
    case FA_ERR_HIP: return "HIP runtime error at kernel launch";
    case FA_ERR_TILE: return "tile shape not in the supported table";
    case FA_ERR_SCRATCH: return "problem needs more scratch than the fixed no-allocation buffer holds (FA_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

}  // extern "C"
