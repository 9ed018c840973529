// Shrink: v[p, j] = sum_k x[perm[p], k] * A_a[j, k] for the rows of each
// adapter segment ("LoRazor" 3.1.1 Eq. 1; "LoRAForge" 5, rank-aware shrink:
// directions beyond the adapter's retained rank exit before reading operands).
//
// bf16 pools: one work item is (row tile of <= 16 rows of one segment, NB
// consecutive blocks of db = 16, 8 or 4 rank directions), each block computed
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
// waves of the workgroup take interleaved k chunks (so that for decode
// widths every load of a wave is in flight at once) and their partial tiles
// are summed through LDS in a fixed order: no atomics, bitwise reproducible.
//
// fp32 pools use the same tiling with v_mfma_f32_16x16x4f32 (four MFMAs per
// 16-byte load, one per element).
#include "build_small.h"
#include "tiles.h"

#include <algorithm>
#include <type_traits>

namespace lora {
namespace {

constexpr int kThreads = 1024;        // 16 waves: for d_in <= 4096 a wave's loads all go out at once
constexpr int kWaves = kThreads / 64;
struct ShrinkArgs {
  const void* x;
  const void* A;
  const int32_t* slot_rank;
  int32_t* seg;
  float* v;
  int ld_x, r_cap, d_in, T, ld_v;
  int mode, db, nrb, rtiles, n_items;  // nrb: items per row tile; n_items: host item count (FULL_BATCH)
  int slots;                           // L = min(T, n_slots) adapter slots (BUCKETED)
};

constexpr int kUnroll = 8;        // k chunks in flight per wave
constexpr int kMinItems = 256;    // narrow the rank blocks until about this many items exist

// One k chunk of the 16 x 16 tile: bf16 takes one 16x16x32 MFMA; fp32 takes
// four 16x16x4 MFMAs, MFMA e using element e of every lane's 4 values, so
// that the four lane groups x four elements cover the chunk's 16 k.
template <typename TI>
__device__ __forceinline__ f32x4_t mfma_chunk(const u32x4_t& xv, const u32x4_t& av, f32x4_t acc) {
  if constexpr (sizeof(TI) == 2) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xv), __builtin_bit_cast(bf16x8_t, av),
                                                   acc, 0, 0, 0);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(xv[e]), __uint_as_float(av[e]), acc, 0, 0, 0);
    return acc;
  }
}

// The shrink items of a launch, by a workgroup of WAVES waves, from the
// segment buffer P (global memory, or the workgroup's own LDS copy); red is
// LDS of WAVES x 64 x 16 bytes.
template <typename TI, int NB, int WAVES>
__device__ __forceinline__ void shrink_items(const ShrinkArgs& a, const SegPtrs& P, f32x4_t (*red)[64]) {
  constexpr int VEC = 16 / sizeof(TI);      // elements per 16-byte load
  constexpr int KC = 4 * VEC;               // k per chunk (4 lane groups)
  constexpr int UNR = kUnroll / NB > 0 ? kUnroll / NB : 1;   // k chunks in flight per wave
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int frow = lane & 15, fk = lane >> 4;
  const TI* __restrict__ X = static_cast<const TI*>(a.x);
  const TI* __restrict__ Ab = static_cast<const TI*>(a.A);
  const bool listed = a.mode == LORA_LAUNCH_EXACT || a.mode == LORA_LAUNCH_PERSISTENT;
  // The metadata of an item is a chain of dependent loads (tile record ->
  // segment -> adapter -> rank -> operands); each level is a full memory
  // latency, so independent loads of a level go out together: the summary
  // words with the first item's tile record, the segment's end and adapter
  // with the permutation entries of all 16 rows the tile may hold.
  // (all five loads before any branch; the tile index is clamped into the
  // list's T entries, T >= 1 for every launch)
  const int first_tile = min((int)(blockIdx.x / a.nrb), a.T - 1);
  int rec_p0 = P.tiles_small[2 * first_tile];
  int rec_seg = P.tiles_small[2 * first_tile + 1];
  const int n_tiles = P.sum[kNTilesSmall];
  const int s_err = P.sum[kError], s_rows = P.sum[kRows];
  // an invalid buffer has no live rows (a listed tile record is never
  // negative; testing it here also keeps its load ahead of the branch)
  const bool bad_rec = listed & (first_tile < n_tiles) & ((rec_p0 | rec_seg) < 0);
  if ((s_err != 0) | (s_rows != a.T) | bad_rec) return;
  // The work comes from the device summary in every mode; the host summary
  // (EXACT, BUCKETED) only sizes the grid, which strides over the items, so
  // a summary of another batch costs time, never rows.
  int n_items = a.n_items, rtiles = a.rtiles;
  if (listed) {
    n_items = n_tiles * a.nrb;
  } else if (a.mode == LORA_LAUNCH_BUCKETED) {
    rtiles = (P.sum[kRowBound] + LORA_TILE_SMALL - 1) / LORA_TILE_SMALL;
    n_items = a.slots * rtiles * a.nrb;
  }
  const int nchunk = (a.d_in + KC - 1) / KC;

  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int tile_item = item / a.nrb;
    const int rb = item - tile_item * a.nrb;
    TileWork w;
    if (listed) {
      if (tile_item >= n_tiles) continue;   // a host count that disagrees with the device buffer
      if (item != (int)blockIdx.x) {
        rec_p0 = P.tiles_small[2 * tile_item];
        rec_seg = P.tiles_small[2 * tile_item + 1];
      }
      w.p0 = rec_p0;
      w.seg = rec_seg;
    } else if (!decode_tile<LORA_TILE_SMALL>(P, a.mode, tile_item, P.tiles_small, rtiles, w)) {
      continue;
    }
    // segment end, adapter and the tile's 16 permutation entries (row frow,
    // or a later valid row past the tile) as one round of loads
    const int seg_end = P.seg_start[w.seg + 1];
    const int adapter = P.seg_adapter[w.seg];
    const int my_perm = P.perm[min(w.p0 + frow, a.T - 1)];
    // an empty use of all three keeps the compiler from sinking the segment
    // end and the permutation loads past the rank test below
    asm volatile("" ::"v"(seg_end), "v"(adapter), "v"(my_perm));
    w.rows = min(LORA_TILE_SMALL, seg_end - w.p0);
    const int r = a.slot_rank[adapter];
    const int j0 = rb * NB * a.db;
    if (j0 >= r) continue;                      // directions beyond the retained rank
    const int jn = min(a.db, r - j0);           // directions of the item's first block
    const int nbl = min(NB, (r - j0 + a.db - 1) / a.db);   // blocks with directions below the rank
    const int span = max(w.rows, jn);
    const int Pw = span <= 4 ? 4 : (span <= 8 ? 8 : 16);   // row slots per k slice
    const int sl = frow % Pw, ks = frow / Pw;                // this lane's slot and k slice
    const int nchq = (nchunk * Pw + 15) / 16;                // k chunks per slice
    // slots past the tile's rows / the block's directions repeat a valid one;
    // their products are never stored
    const int xrow = __shfl(my_perm, (lane & ~15) | min(sl, w.rows - 1), 64);
    const TI* xr = X + (size_t)xrow * a.ld_x + fk * VEC;
    const TI* ar[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int jb = min(a.db, r - j0 - b * a.db);   // directions of block b (<= 0: no work)
      ar[b] = Ab + ((size_t)adapter * a.r_cap + j0 + b * a.db + min(sl, max(jb, 1) - 1)) * a.d_in + fk * VEC;
    }

    f32x4_t acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int c0 = wave; c0 < nchq; c0 += WAVES * UNR) {
      u32x4_t xv[UNR], av[UNR][NB];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int c = c0 + WAVES * u;
        const int g = ks * nchq + c;            // this lane's chunk
        // d_in % 8 == 0: a lane's group is all in or all out
        const bool in = c < nchq && g * KC + fk * VEC < a.d_in;
        xv[u] = in ? ld128(xr + (size_t)g * KC) : u32x4_t{0, 0, 0, 0};
#pragma unroll
        for (int b = 0; b < NB; ++b) av[u][b] = (in && b < nbl) ? ld128(ar[b] + (size_t)g * KC) : u32x4_t{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[b] = mfma_chunk<TI>(xv[u], av[u][b], acc[b]);
    }
    // acc[b][e] = partial product[row = 4 * (lane / 16) + e][col = lane % 16]
    // of block b; v[s, c] is the sum over slices q of product[s + Pw q][c + Pw q]
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (b >= nbl) break;
      red[wave][lane] = acc[b];
      lds_sync();
      if (threadIdx.x < 256) {
        const int t = threadIdx.x;              // one output each, slices and waves summed in order
        const int row = t >> 4, col = t & 15;
        const int jb = min(a.db, r - j0 - b * a.db);
        float s = 0.f;
        if (row < Pw && col < Pw) {
          for (int q = 0; q < 16 / Pw; ++q) {
            const int i = row + Pw * q, j = col + Pw * q;
            const int src = (i >> 2) * 16 + j, e = i & 3;
#pragma unroll
            for (int wv = 0; wv < WAVES; ++wv) s += red[wv][src][e];
          }
        }
        if (row < w.rows && col < jb) a.v[(size_t)(w.p0 + row) * a.ld_v + j0 + b * a.db + col] = s;
      }
      lds_sync();
    }
  }
}

template <typename TI, int NB>
__global__ __launch_bounds__(kThreads) void shrink_mfma_kernel(ShrinkArgs a) {
  __shared__ f32x4_t red[kWaves][64];
  shrink_items<TI, NB, kWaves>(a, seg_ptrs(a.seg, a.T), red);
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

ShrinkShape shrink_shape(const lora_pool_t& pool, int T, const LaunchShape& ls, ShrinkArgs& a, int max_grid) {
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
  // row tiles: the bound for PERSISTENT, else the mode's host count
  const long tiles = ls.mode == LORA_LAUNCH_PERSISTENT ? bound : (long)host_tile_items(ls, T, LORA_TILE_SMALL);
  ShrinkShape sh;
  sh.nb = nb;
  if (ls.mode == LORA_LAUNCH_PERSISTENT) {
    a.n_items = 0;
    sh.grid = (int)std::min<long>(tiles * a.nrb, max_grid);
  } else {
    a.n_items = (int)(tiles * a.nrb);
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
    if (pool.dtype == LORA_BF16)
      hipLaunchKernelGGL((shrink_mfma_kernel<uint16_t, NB>), dim3(sh.grid), dim3(kThreads), 0, st, a);
    else
      hipLaunchKernelGGL((shrink_mfma_kernel<float, NB>), dim3(sh.grid), dim3(kThreads), 0, st, a);
  });
  return hipGetLastError();
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
  // least one workgroup, which writes the segment buffer)
  const ShrinkShape sh = shrink_shape(pool, T, ls, a, 1 << 20);
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
