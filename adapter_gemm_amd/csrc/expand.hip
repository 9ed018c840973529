// Expand: y[perm[p], n] += s_a * sum_{j < r_a} v[p, j] * B_a[n, j]
// ("LoRazor" 3.1.1 Eq. 2; "LoRAForge" 5, RowExpand).
//
// Work item = (row tile of <= 16 rows of one segment, block of output
// columns).  Each thread owns NPT consecutive output channels: it loads their
// B rows (rank-contiguous, so a wave reads one contiguous span of B) into
// registers once and reuses them for every row of the tile.  The tile's v rows
// sit in LDS and are read as broadcasts.  The rank reduction is local to the
// thread (no cross-lane traffic); the scaled update is added to y in place
// with one rounding.  NPT is chosen so that NPT * RC = 128 registers of B.
#include "common.h"
#include "tiles.h"

#include <algorithm>

namespace lora {
namespace {

struct ExpandArgs {
  const void* B;
  const int32_t* slot_rank;
  const float* slot_scale;
  int32_t* seg;
  const float* v;
  void* y;
  int r_cap, d_out, T, ld_v, ld_y;
  int mode, ncb, rtiles, n_items;
  int slots;                      // L = min(T, n_slots) adapter slots (BUCKETED)
};

template <typename TY, int NPT>
__device__ __forceinline__ void ld_vals(const TY* p, float (&o)[NPT]) {
  if constexpr (sizeof(TY) == 2) {
    if constexpr (NPT == 8) {
      const u32x4_t u = ld128(p);
#pragma unroll
      for (int q = 0; q < 4; ++q) { o[2 * q] = bf16lo(u[q]); o[2 * q + 1] = bf16hi(u[q]); }
    } else if constexpr (NPT == 4) {
      const uint2 u = *reinterpret_cast<const uint2*>(p);
      o[0] = bf16lo(u.x); o[1] = bf16hi(u.x); o[2] = bf16lo(u.y); o[3] = bf16hi(u.y);
    } else if constexpr (NPT == 2) {
      const uint32_t u = *reinterpret_cast<const uint32_t*>(p);
      o[0] = bf16lo(u); o[1] = bf16hi(u);
    } else {
      o[0] = bf16_to_f32(*reinterpret_cast<const uint16_t*>(p));
    }
  } else {
#pragma unroll
    for (int c = 0; c < NPT; ++c) o[c] = reinterpret_cast<const float*>(p)[c];
  }
}

template <typename TY, int NPT>
__device__ __forceinline__ void st_vals(TY* p, const float (&o)[NPT]) {
  if constexpr (sizeof(TY) == 2) {
    if constexpr (NPT == 8) {
      u32x4_t u;
#pragma unroll
      for (int q = 0; q < 4; ++q) u[q] = pack_bf16x2(o[2 * q], o[2 * q + 1]);
      st128(p, u);
    } else if constexpr (NPT == 4) {
      uint2 u;
      u.x = pack_bf16x2(o[0], o[1]);
      u.y = pack_bf16x2(o[2], o[3]);
      *reinterpret_cast<uint2*>(p) = u;
    } else if constexpr (NPT == 2) {
      *reinterpret_cast<uint32_t*>(p) = pack_bf16x2(o[0], o[1]);
    } else {
      *reinterpret_cast<uint16_t*>(p) = f32_to_bf16(o[0]);
    }
  } else {
#pragma unroll
    for (int c = 0; c < NPT; ++c) reinterpret_cast<float*>(p)[c] = o[c];
  }
}

// B row of one channel: RC values starting at p (rank-contiguous), entries
// j >= r are replaced by zero so that padding never reaches the sum.
template <typename TB, int RC>
__device__ __forceinline__ void ld_brow(const TB* p, int r, float (&o)[RC]) {
  if constexpr (sizeof(TB) == 2) {
    static_assert(RC % 8 == 0, "bf16 rank bucket must be a multiple of 8");
#pragma unroll
    for (int q = 0; q < RC / 8; ++q) {
      u32x4_t u = {0, 0, 0, 0};
      if (8 * q < r) u = ld128(p + 8 * q);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[8 * q + 2 * e] = bf16lo(u[e]);
        o[8 * q + 2 * e + 1] = bf16hi(u[e]);
      }
    }
  } else {
    static_assert(RC % 4 == 0, "fp32 rank bucket must be a multiple of 4");
#pragma unroll
    for (int q = 0; q < RC / 4; ++q) {
      u32x4_t u = {0, 0, 0, 0};
      if (4 * q < r) u = ld128(p + 4 * q);
#pragma unroll
      for (int e = 0; e < 4; ++e) o[4 * q + e] = __uint_as_float(u[e]);
    }
  }
#pragma unroll
  for (int j = 0; j < RC; ++j)
    if (j >= r) o[j] = 0.f;
}

template <typename TB, typename TY, int RC, int NPT, int THREADS>
__global__ __launch_bounds__(THREADS) void expand_kernel(ExpandArgs a) {
  __shared__ float vt[LORA_TILE_SMALL][RC];
  const SegPtrs P = seg_ptrs(a.seg, a.T);
  if (!seg_valid(P, a.T)) return;
  const TB* __restrict__ Bp = static_cast<const TB*>(a.B);
  TY* __restrict__ Y = static_cast<TY*>(a.y);
  // The work comes from the device summary in every mode; the host summary
  // (EXACT, BUCKETED) only sizes the grid, which strides over the items, so
  // a summary of another batch costs time, never rows.
  int n_items = a.n_items, rtiles = a.rtiles;
  if (a.mode == LORA_LAUNCH_PERSISTENT || a.mode == LORA_LAUNCH_EXACT) {
    n_items = device_tile_count<LORA_TILE_SMALL>(P) * a.ncb;
  } else if (a.mode == LORA_LAUNCH_BUCKETED) {
    rtiles = (P.sum[kRowBound] + LORA_TILE_SMALL - 1) / LORA_TILE_SMALL;
    n_items = a.slots * rtiles * a.ncb;
  }

  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int tile_item = item / a.ncb;
    const int cb = item - tile_item * a.ncb;
    TileWork w;
    if (!decode_tile<LORA_TILE_SMALL>(P, a.mode, tile_item, P.tiles_small, rtiles, w)) continue;
    const int adapter = P.seg_adapter[w.seg];
    const int r = a.slot_rank[adapter];
    if (r <= 0) continue;
    const float sc = a.slot_scale[adapter];

    // v tile -> LDS (zeros beyond the rank and the tile's rows)
    for (int e = threadIdx.x; e < LORA_TILE_SMALL * RC; e += THREADS) {
      const int m = e / RC, j = e - m * RC;
      vt[m][j] = (m < w.rows && j < r) ? a.v[(size_t)(w.p0 + m) * a.ld_v + j] : 0.f;
    }
    __syncthreads();

    const int n = (cb * THREADS + threadIdx.x) * NPT;
    if (n < a.d_out) {
      float b[NPT][RC];
#pragma unroll
      for (int c = 0; c < NPT; ++c) ld_brow<TB, RC>(Bp + ((size_t)adapter * a.d_out + n + c) * a.r_cap, r, b[c]);
      for (int m = 0; m < w.rows; ++m) {
        float acc[NPT];
#pragma unroll
        for (int c = 0; c < NPT; ++c) acc[c] = 0.f;
#pragma unroll
        for (int j = 0; j < RC; ++j) {
          const float vj = vt[m][j];
#pragma unroll
          for (int c = 0; c < NPT; ++c) acc[c] = fmaf(vj, b[c][j], acc[c]);
        }
        TY* yp = Y + (size_t)P.perm[w.p0 + m] * a.ld_y + n;
        float yv[NPT];
        ld_vals<TY, NPT>(yp, yv);
#pragma unroll
        for (int c = 0; c < NPT; ++c) yv[c] = fmaf(sc, acc[c], yv[c]);
        st_vals<TY, NPT>(yp, yv);
      }
    }
    __syncthreads();
  }
}

template <typename TB, typename TY, int RC>
hipError_t launch_rc(ExpandArgs a, const LaunchShape& ls, int T, hipStream_t st) {
  constexpr int NPT = 128 / RC > 8 ? 8 : 128 / RC;
  // narrow column blocks for small batches so that the grid still spans the chip
  const bool small = (ls.mode == LORA_LAUNCH_EXACT && ls.n_tiles < 256);
  const int threads = small ? 64 : 256;
  a.ncb = (a.d_out + threads * NPT - 1) / (threads * NPT);
  a.rtiles = host_row_tiles(ls, T, LORA_TILE_SMALL);
  int grid;
  if (ls.mode == LORA_LAUNCH_PERSISTENT) {
    a.n_items = 0;
    grid = 2048;
  } else {
    a.n_items = host_tile_items(ls, T, LORA_TILE_SMALL) * a.ncb;
    grid = std::max(a.n_items, 1);   // (at least one workgroup, which finds the device's own count)
  }
  if (grid <= 0) return hipSuccess;
  if (small)
    hipLaunchKernelGGL((expand_kernel<TB, TY, RC, NPT, 64>), dim3(grid), dim3(64), 0, st, a);
  else
    hipLaunchKernelGGL((expand_kernel<TB, TY, RC, NPT, 256>), dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <typename TB, typename TY>
hipError_t launch_typed(const ExpandArgs& a, const LaunchShape& ls, int T, hipStream_t st) {
  const int rc = a.r_cap;
  if (rc <= 8 && sizeof(TB) == 2) return launch_rc<TB, TY, 8>(a, ls, T, st);
  if (rc <= 8) return launch_rc<TB, TY, 8>(a, ls, T, st);
  if (rc <= 16) return launch_rc<TB, TY, 16>(a, ls, T, st);
  if (rc <= 32) return launch_rc<TB, TY, 32>(a, ls, T, st);
  if (rc <= 64) return launch_rc<TB, TY, 64>(a, ls, T, st);
  return launch_rc<TB, TY, 128>(a, ls, T, st);
}

}  // namespace

hipError_t launch_expand(const lora_pool_t& pool, int32_t* seg, int T, const LaunchShape& ls, const float* v,
                         int ld_v, void* y, int y_dtype, int ld_y, hipStream_t st) {
  if (T == 0) return hipSuccess;
  ExpandArgs a;
  a.B = pool.B;
  a.slot_rank = pool.slot_rank;
  a.slot_scale = pool.slot_scale;
  a.seg = seg;
  a.v = v;
  a.y = y;
  a.r_cap = pool.r_cap;
  a.d_out = pool.d_out;
  a.T = T;
  a.ld_v = ld_v;
  a.ld_y = ld_y;
  a.mode = ls.mode;
  a.slots = ls.slots;
  if (pool.dtype == LORA_BF16) {
    if (y_dtype == LORA_BF16) return launch_typed<uint16_t, uint16_t>(a, ls, T, st);
    return launch_typed<uint16_t, float>(a, ls, T, st);
  }
  if (y_dtype == LORA_BF16) return launch_typed<float, uint16_t>(a, ls, T, st);
  return launch_typed<float, float>(a, ls, T, st);
}

}  // namespace lora
