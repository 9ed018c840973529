// Shrink: v[p, j] = sum_k x[perm[p], k] * A_a[j, k] for the rows of each
// adapter segment ("LoRazor" 3.1.1 Eq. 1; "LoRAForge" 5, rank-aware shrink:
// directions beyond the adapter's retained rank exit before reading operands).
//
// bf16 pools: one work item is (row tile of <= 16 rows of one segment, or
// one half of it in the one-launch build + shrink, NB consecutive blocks of
// db = 16, 8 or 4 rank directions), each block computed
// as a 16 x 16 tile of MFMA v_mfma_f32_16x16x32_bf16 products that share the
// item's x fragments.  Small batches use narrow blocks and one block per
// item, so that enough workgroups share the A rows to keep the chip's CUs
// streaming; batches with more row tiles than that need take several blocks
// per item, so that a tile's x rows and its chain of metadata loads serve
// all of its rank directions (blocks past the adapter's rank do no work).
// Operand fragments come straight from global memory: lane l reads 16
// contiguous bytes of a token row and 16 of a direction row, at k offset
// 8 * (l / 16) inside each 32-wide k chunk, so both operands stream in
// 128-bit loads and A_a is read once per row tile.  Row slot l mod 16 is a
// token row / direction for a full item; an item of few rows and directions
// folds the k range instead: with P = 4, 8 or 16 >= max(rows, directions),
// slot s + P q reads row / direction s over the q-th of 16 / P k slices, so
// no two lanes load the same bytes, and the slices' partial sums (the
// diagonal P x P blocks of the product) are added in slice order.  The 16
// waves of the workgroup (8 for bf16 items of four rank blocks, two
// workgroups per CU) take interleaved k chunks (so that for decode widths
// every load of a wave is in flight at once) and their partial tiles are
// summed through LDS in a fixed order: no atomics, bitwise reproducible.
//
// fp32 pools use the same tiling with v_mfma_f32_16x16x4f32 (four MFMAs per
// 16-byte load, one per element).
#include "build_small.h"
#include "shrink_core.h"
#include "tiles.h"

#include <algorithm>
#include <type_traits>

namespace lora {
namespace {

template <typename TI, int NB, int WAVES = kWaves>
__global__ __launch_bounds__(64 * WAVES) void shrink_mfma_kernel(ShrinkArgs a) {
  __shared__ f32x4_t red[WAVES][64];
  shrink_items<TI, NB, WAVES>(a, seg_ptrs(a.seg, a.T), red);
}

// Small batches (T <= 256 rows, pools of at most 1024 slots): the segment
// build and the shrink in one launch.  Every workgroup groups the batch
// itself, into its own LDS copy of the segment buffer (a few microseconds of
// LDS work, no dependent global round trips), and takes its shrink items
// from that copy; workgroup 0 also writes the copy out as the segment buffer
// that later launches read.  This removes a launch and, per item, the chain
// of segment-buffer loads from global memory.  The segment buffer equals the
// device builder's bit for bit; v equals the persistent shrink's up to fp32
// rounding (four waves add the k chunks in another fixed order).
template <typename TI, int NB>
__global__ __launch_bounds__(kSmallRows) void build_shrink_kernel(const int32_t* __restrict__ ids,
                                                                  const uint8_t* __restrict__ active, int N,
                                                                  int order, ShrinkArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint64_t tbl[];   // small_build_lds_bytes(N)
  __shared__ BuildLds sh;
  __shared__ __attribute__((aligned(16))) int32_t lseg[kSegHeader + 8 * kSmallRows + 1];
  __shared__ f32x4_t red[kSmallRows / 64][64];
  __shared__ int32_t lrank[1024];
  // every slot's rank, loaded beside the ids and kept in LDS: the items then
  // read their rank with no global round trip
  int rk[1024 / kSmallRows];
#pragma unroll
  for (int q = 0; q < 1024 / kSmallRows; ++q) {
    const int i = q * kSmallRows + (int)threadIdx.x;
    rk[q] = i < N ? a.slot_rank[i] : 0;
  }
  const SegPtrs L = seg_ptrs(lseg, a.T);
  const bool ok = small_build(ids, active, a.T, N, order, L, tbl, sh);
#pragma unroll
  for (int q = 0; q < 1024 / kSmallRows; ++q) lrank[q * kSmallRows + threadIdx.x] = rk[q];
  lds_sync();
  if (blockIdx.x == 0) {
    const int words = (int)seg_words(a.T);
    for (int i = threadIdx.x; i < words; i += kSmallRows) a.seg[i] = lseg[i];
  }
  if (!ok) return;
  ShrinkArgs b = a;
  b.slot_rank = lrank;
  shrink_items<TI, NB, kSmallRows / 64>(b, L, red);
}

}  // namespace

namespace {
// Item shape of a shrink launch: rank-block width, blocks per item, items per
// row tile, and the grid (PERSISTENT: the tile bound; else the mode's count).
struct ShrinkShape {
  int nb, grid;
};

ShrinkShape shrink_shape(const lora_pool_t& pool, int T, const LaunchShape& ls, ShrinkArgs& a, int max_grid,
                         int rsub = 1) {
  a.A = pool.A;
  a.slot_rank = pool.slot_rank;
  a.r_cap = pool.r_cap;
  a.d_in = pool.d_in;
  a.T = T;
  a.mode = ls.mode;
  a.rtiles = host_row_tiles(ls, T, LORA_TILE_SMALL);
  a.slots = ls.slots;
  // The rank-block width (and with it each item's k folding) follows from
  // the batch shape alone, through the bound sum_a ceil(m_a / 16) <= T / 16 +
  // min(T, n_slots) of the row tiles, so v is the same in every launch mode.
  const long bound = (long)T / LORA_TILE_SMALL + std::min(T, pool.n_slots);
  a.db = 16;
  while (a.db > 4 && bound * ((pool.r_cap + a.db - 1) / a.db) < kMinItems) a.db >>= 1;
  const int nblocks = (pool.r_cap + a.db - 1) / a.db;
  // blocks per item: one, unless the row tiles are mostly full (at least 8
  // rows on average by the bound), so that sharing a tile's x rows across
  // blocks saves real traffic; then as many as still leave about kMinItems
  // items.  (Batches of one- or two-row tiles keep one block per item: their
  // bytes are the A rows, which must spread over every CU.)
  int nb = 1;
  if ((long)T >= 8 * bound)
    while (nb < 8 && nb < nblocks && bound * ((nblocks + 2 * nb - 1) / (2 * nb)) >= kMinItems) nb *= 2;
  a.nrb = (nblocks + nb - 1) / nb;
  a.rsub = rsub;
  // row tiles: the bound for PERSISTENT, else the mode's host count
  const long tiles = ls.mode == LORA_LAUNCH_PERSISTENT ? bound : (long)host_tile_items(ls, T, LORA_TILE_SMALL);
  ShrinkShape sh;
  sh.nb = nb;
  if (ls.mode == LORA_LAUNCH_PERSISTENT) {
    a.n_items = 0;
    sh.grid = (int)std::min<long>(tiles * a.nrb * a.rsub, max_grid);
  } else {
    a.n_items = (int)(tiles * a.nrb * a.rsub);
    // (at least one workgroup, which finds the device's own count)
    sh.grid = std::max(a.n_items, 1);
  }
  return sh;
}

template <typename F>
void with_nb(int nb, F&& f) {
  switch (nb) {
    case 1: f(std::integral_constant<int, 1>{}); break;
    case 2: f(std::integral_constant<int, 2>{}); break;
    case 4: f(std::integral_constant<int, 4>{}); break;
    default: f(std::integral_constant<int, 8>{}); break;
  }
}
}  // namespace

hipError_t launch_shrink(const lora_pool_t& pool, int32_t* seg, int T, const LaunchShape& ls, const void* x,
                         int ld_x, float* v, int ld_v, hipStream_t st) {
  ShrinkArgs a;
  a.x = x;
  a.seg = seg;
  a.v = v;
  a.ld_x = ld_x;
  a.ld_v = ld_v;
  const ShrinkShape sh = shrink_shape(pool, T, ls, a, 1024);
  if (sh.grid <= 0 || T == 0) return hipSuccess;
  with_nb(sh.nb, [&](auto nb_c) {
    constexpr int NB = decltype(nb_c)::value;
    // bf16 items of four rank blocks (long batches of mostly full row
    // tiles) run in 8-wave workgroups, two per CU: an item is bound by its
    // latency, and the second workgroup's items overlap it (prefill batch
    // 42.9 -> 36.8 us in the bench; narrower items keep 16 waves, which
    // measured faster for them)
    if (pool.dtype == LORA_BF16 && NB == 4)
      hipLaunchKernelGGL((shrink_mfma_kernel<uint16_t, NB, kWaves / 2>), dim3(sh.grid), dim3(kThreads / 2), 0, st, a);
    else if (pool.dtype == LORA_BF16)
      hipLaunchKernelGGL((shrink_mfma_kernel<uint16_t, NB>), dim3(sh.grid), dim3(kThreads), 0, st, a);
    else
      hipLaunchKernelGGL((shrink_mfma_kernel<float, NB>), dim3(sh.grid), dim3(kThreads), 0, st, a);
  });
  return hipGetLastError();
}

void shrink_item_geometry(const lora_pool_t& pool, int T, int* db, int* nrb) {
  const long bound = (long)T / LORA_TILE_SMALL + std::min(T, pool.n_slots);
  int w = 16;
  while (w > 4 && bound * ((pool.r_cap + w - 1) / w) < kMinItems) w >>= 1;
  *db = w;
  *nrb = (pool.r_cap + w - 1) / w;
}

bool build_shrink_fits(int T, int n_slots) { return T >= 1 && T <= kSmallRows && n_slots >= 1 && n_slots <= 1024; }

hipError_t launch_build_shrink(const int32_t* ids, const uint8_t* active, int T, int order, const lora_pool_t& pool,
                               int32_t* seg, const void* x, int ld_x, float* v, int ld_v, hipStream_t st) {
  ShrinkArgs a;
  a.x = x;
  a.seg = seg;
  a.v = v;
  a.ld_x = ld_x;
  a.ld_v = ld_v;
  LaunchShape ls{LORA_LAUNCH_PERSISTENT, 0, 0, std::min(T, pool.n_slots)};
  // every workgroup builds the segments, so the grid is the item bound (at
  // least one workgroup, which writes the segment buffer).  Every row tile
  // is split into two items of up to 8 rows: the few full tiles of a batch of
  // mostly one-row tiles (a Zipf head adapter) then stream half the x bytes
  // each, which is where this launch waits longest (measured: the decode
  // batch 11.3 -> 10.3 us; four parts slower, and in the separate shrink of
  // 1024-thread workgroups the doubled item count costs more than it saves)
  const ShrinkShape sh = shrink_shape(pool, T, ls, a, 1 << 20, 2);
  const int grid = std::max(sh.grid, 1);
  const size_t lds = small_build_lds_bytes(pool.n_slots);
  with_nb(sh.nb, [&](auto nb_c) {
    constexpr int NB = decltype(nb_c)::value;
    if (pool.dtype == LORA_BF16)
      hipLaunchKernelGGL((build_shrink_kernel<uint16_t, NB>), dim3(grid), dim3(kSmallRows), lds, st, ids, active,
                         pool.n_slots, order, a);
    else
      hipLaunchKernelGGL((build_shrink_kernel<float, NB>), dim3(grid), dim3(kSmallRows), lds, st, ids, active,
                         pool.n_slots, order, a);
  });
  return hipGetLastError();
}

}  // namespace lora
