// Shrink: v[p, j] = sum_k x[perm[p], k] * A_a[j, k] for the rows of each
// adapter segment ("LoRazor" 3.1.1 Eq. 1; "LoRAForge" 5, rank-aware shrink:
// directions beyond the adapter's retained rank exit before reading operands).
//
// Decode-sized work is a gather of A rows and is bound by HBM: each work
// item is (row tile of <= 16 rows of one segment, block of 4 rank directions).
// The 4 waves of the workgroup split d_in; every lane streams 16-byte chunks
// of the 4 A rows and of the tile's x rows, so each A row is read from HBM
// once per row tile (once per segment for segments of <= 16 rows) and x rows
// come from L2.  Partial dot products are combined with a transposed
// butterfly inside the wave (each shuffle step halves the values per lane)
// and then across the 4 waves through LDS in a fixed order: no atomics, so
// results are bitwise reproducible.
#include "common.h"
#include "tiles.h"

namespace lora {
namespace {

constexpr int kThreads = 256;
constexpr int kJB = 4;            // rank directions per workgroup

struct ShrinkArgs {
  const void* x;
  const void* A;
  const int32_t* slot_rank;
  int32_t* seg;
  float* v;
  int ld_x, r_cap, d_in, T, ld_v;
  int mode, nrb, rtiles, n_items;  // n_items: host item count (EXACT/BUCKETED/FULL)
};

template <typename TI>
__device__ __forceinline__ float dot16(const u32x4_t& a, const u32x4_t& b, float acc);

template <>
__device__ __forceinline__ float dot16<uint16_t>(const u32x4_t& a, const u32x4_t& b, float acc) {
  // exact widening of both bf16 halves, fp32 FMA
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    acc = fmaf(bf16lo(a[q]), bf16lo(b[q]), acc);
    acc = fmaf(bf16hi(a[q]), bf16hi(b[q]), acc);
  }
  return acc;
}

template <>
__device__ __forceinline__ float dot16<float>(const u32x4_t& a, const u32x4_t& b, float acc) {
#pragma unroll
  for (int q = 0; q < 4; ++q) acc = fmaf(__uint_as_float(a[q]), __uint_as_float(b[q]), acc);
  return acc;
}

// Sum NV per-lane values over the 64 lanes.  Afterwards lane l holds the
// total of value index l >> (6 - log2 NV).
template <int NV>
__device__ __forceinline__ float wave_reduce_transpose(float (&v)[NV], int lane) {
  constexpr int LOG2 = NV == 1 ? 0 : NV == 2 ? 1 : NV == 4 ? 2 : NV == 8 ? 3 : NV == 16 ? 4 : NV == 32 ? 5 : 6;
  static_assert((1 << LOG2) == NV, "NV must be a power of two <= 64");
#pragma unroll
  for (int step = 0; step < LOG2; ++step) {
    const int o = 32 >> step;
    const int half = NV >> (step + 1);
    const bool upper = (lane & o) != 0;
#pragma unroll
    for (int i = 0; i < half; ++i) {
      const float send = upper ? v[i] : v[i + half];
      const float keep = upper ? v[i + half] : v[i];
      v[i] = keep + __shfl_xor(send, o, 64);
    }
  }
  float r = v[0];
#pragma unroll
  for (int o = 32 >> LOG2; o >= 1; o >>= 1) r += __shfl_xor(r, o, 64);
  return r;
}

template <typename TI, int MR>
__device__ __forceinline__ void shrink_tile(const ShrinkArgs& a, const SegPtrs& P, const TileWork& w, int adapter,
                                            int j0, int jn, float (*red)[64]) {
  constexpr int VEC = 16 / sizeof(TI);
  constexpr int NV = MR * kJB;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const TI* __restrict__ X = static_cast<const TI*>(a.x);
  const TI* __restrict__ Ab = static_cast<const TI*>(a.A);

  const TI* xr[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) xr[m] = X + (size_t)P.perm[w.p0 + min(m, w.rows - 1)] * a.ld_x;
  const TI* ar[kJB];
#pragma unroll
  for (int jj = 0; jj < kJB; ++jj) ar[jj] = Ab + ((size_t)adapter * a.r_cap + j0 + min(jj, jn - 1)) * a.d_in;

  float acc[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) acc[i] = 0.f;

  const int stride = 4 * 64 * VEC;
#pragma unroll 2
  for (int k = (wave * 64 + lane) * VEC; k < a.d_in; k += stride) {
    u32x4_t av[kJB];
#pragma unroll
    for (int jj = 0; jj < kJB; ++jj) av[jj] = jj < jn ? ld128(ar[jj] + k) : u32x4_t{0, 0, 0, 0};
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      if (m < w.rows) {
        const u32x4_t xv = ld128(xr[m] + k);
#pragma unroll
        for (int jj = 0; jj < kJB; ++jj) acc[m * kJB + jj] = dot16<TI>(xv, av[jj], acc[m * kJB + jj]);
      }
    }
  }

  const float r = wave_reduce_transpose<NV>(acc, lane);
  constexpr int GROUP = 64 / NV;
  if ((lane & (GROUP - 1)) == 0) red[wave][lane / GROUP] = r;
  __syncthreads();
  if (threadIdx.x < NV) {
    const int t = threadIdx.x;
    const float s = red[0][t] + red[1][t] + red[2][t] + red[3][t];
    const int m = t / kJB, jj = t - m * kJB;
    if (m < w.rows && jj < jn) a.v[(size_t)(w.p0 + m) * a.ld_v + j0 + jj] = s;
  }
  __syncthreads();
}

template <typename TI>
__global__ __launch_bounds__(kThreads) void shrink_gather_kernel(ShrinkArgs a) {
  __shared__ float red[4][64];
  const SegPtrs P = seg_ptrs(a.seg, a.T);
  if (!seg_valid(P, a.T)) return;
  int n_items = a.n_items;
  if (a.mode == LORA_LAUNCH_PERSISTENT) n_items = device_tile_count<LORA_TILE_SMALL>(P) * a.nrb;
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int tile_item = item / a.nrb;
    const int rb = item - tile_item * a.nrb;
    TileWork w;
    if (!decode_tile<LORA_TILE_SMALL>(P, a.mode, tile_item, P.tiles_small, a.rtiles, w)) continue;
    const int adapter = P.seg_adapter[w.seg];
    const int r = a.slot_rank[adapter];
    const int j0 = rb * kJB;
    if (j0 >= r) continue;                      // directions beyond the retained rank
    const int jn = min(kJB, r - j0);
    if (w.rows <= 1)      shrink_tile<TI, 1>(a, P, w, adapter, j0, jn, red);
    else if (w.rows <= 2) shrink_tile<TI, 2>(a, P, w, adapter, j0, jn, red);
    else if (w.rows <= 4) shrink_tile<TI, 4>(a, P, w, adapter, j0, jn, red);
    else if (w.rows <= 8) shrink_tile<TI, 8>(a, P, w, adapter, j0, jn, red);
    else                  shrink_tile<TI, 16>(a, P, w, adapter, j0, jn, red);
  }
}

}  // namespace

hipError_t launch_shrink(const lora_pool_t& pool, int32_t* seg, int T, const LaunchShape& ls, const void* x,
                         int ld_x, float* v, int ld_v, hipStream_t st) {
  ShrinkArgs a;
  a.x = x;
  a.A = pool.A;
  a.slot_rank = pool.slot_rank;
  a.seg = seg;
  a.v = v;
  a.ld_x = ld_x;
  a.r_cap = pool.r_cap;
  a.d_in = pool.d_in;
  a.T = T;
  a.ld_v = ld_v;
  a.mode = ls.mode;
  a.nrb = (pool.r_cap + kJB - 1) / kJB;
  a.rtiles = host_row_tiles(ls, T, LORA_TILE_SMALL);
  int grid;
  if (ls.mode == LORA_LAUNCH_PERSISTENT) {
    a.n_items = 0;
    grid = 2048;
  } else {
    a.n_items = host_tile_items(ls, T, LORA_TILE_SMALL) * a.nrb;
    grid = a.n_items;
  }
  if (grid <= 0 || T == 0) return hipSuccess;
  if (pool.dtype == LORA_BF16)
    hipLaunchKernelGGL(shrink_gather_kernel<uint16_t>, dim3(grid), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL(shrink_gather_kernel<float>, dim3(grid), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace lora
