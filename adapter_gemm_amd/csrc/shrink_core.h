// Shrink work items shared by the shrink kernels and the fused kernel's
// in-launch shrink: v[p, j] = sum_k x[perm[p], k] * A_a[j, k] for one row tile
// of one segment and one or more blocks of rank directions ("LoRazor" 3.1.1
// Eq. 1; "LoRAForge" 5, rank-aware shrink).  The tiling is described at the
// top of shrink.hip.
#pragma once

#include "common.h"
#include "tiles.h"

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
  int rsub = 1;                        // items per row tile and rank block (row halves: 2)
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

// One item: row tile w (first grouped position and segment), its sub-th part
// of LORA_TILE_SMALL / a.rsub rows (empty parts return at once) and its rb-th
// group of NB rank blocks, by a workgroup of WAVES waves; red is LDS of
// WAVES x 64 x 16 bytes.  COH: v is stored device-coherently (scope sc1:
// never left dirty in, nor read stale from, one XCD's L2), for a consumer in
// the same launch that reads it after a counter says it is complete.
template <typename TI, int NB, int WAVES, bool COH = false>
__device__ __forceinline__ void shrink_item_body(const ShrinkArgs& a, const SegPtrs& P, TileWork w, int rb,
                                                 f32x4_t (*red)[64], int sub = 0) {
  constexpr int VEC = 16 / sizeof(TI);      // elements per 16-byte load
  constexpr int KC = 4 * VEC;               // k per chunk (4 lane groups)
  constexpr int UNR = kUnroll / NB > 0 ? kUnroll / NB : 1;   // k chunks in flight per wave
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int frow = lane & 15, fk = lane >> 4;
  const TI* __restrict__ X = static_cast<const TI*>(a.x);
  const TI* __restrict__ Ab = static_cast<const TI*>(a.A);
  const int nchunk = (a.d_in + KC - 1) / KC;
  {
    // (the item is the workgroup's: its tile record is wave-uniform, and so
    // are the segment's end, adapter and rank read from it, which steer
    // branches around barriers)
    const int sub_rows = LORA_TILE_SMALL / a.rsub;
    w.p0 = __builtin_amdgcn_readfirstlane(w.p0) + sub * sub_rows;
    w.seg = __builtin_amdgcn_readfirstlane(w.seg);
    // segment end, adapter and the tile's 16 permutation entries (row frow,
    // or a later valid row past the tile) as one round of loads
    const int seg_end = __builtin_amdgcn_readfirstlane(P.seg_start[w.seg + 1]);
    const int adapter = __builtin_amdgcn_readfirstlane(P.seg_adapter[w.seg]);
    const int my_perm = P.perm[min(w.p0 + frow, a.T - 1)];
    // an empty use of all three keeps the compiler from sinking the segment
    // end and the permutation loads past the rank test below
    asm volatile("" ::"v"(seg_end), "v"(adapter), "v"(my_perm));
    w.rows = min(sub_rows, seg_end - w.p0);
    if (w.rows <= 0) return;                 // a part past the segment's rows
    const int r = __builtin_amdgcn_readfirstlane(a.slot_rank[adapter]);
    const int j0 = rb * NB * a.db;
    if (j0 >= r) return;                     // directions beyond the retained rank
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
        if (row < w.rows && col < jb) {
          float* dst = a.v + (size_t)(w.p0 + row) * a.ld_v + j0 + b * a.db + col;
          if constexpr (COH) __hip_atomic_store(dst, s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          else *dst = s;
        }
      }
      lds_sync();
    }
  }
}

// The shrink items of a launch, by a workgroup of WAVES waves, from the
// segment buffer P (global memory, or the workgroup's own LDS copy); red is
// LDS of WAVES x 64 x 16 bytes.
template <typename TI, int NB, int WAVES>
__device__ __forceinline__ void shrink_items(const ShrinkArgs& a, const SegPtrs& P, f32x4_t (*red)[64]) {
  const bool listed = a.mode == LORA_LAUNCH_EXACT || a.mode == LORA_LAUNCH_PERSISTENT;
  // The metadata of an item is a chain of dependent loads (tile record ->
  // segment -> adapter -> rank -> operands); each level is a full memory
  // latency, so independent loads of a level go out together: the summary
  // words with the first item's tile record, the segment's end and adapter
  // with the permutation entries of all 16 rows the tile may hold.
  // (all five loads before any branch; the tile index is clamped into the
  // list's T entries, T >= 1 for every launch)
  const int ipt = a.nrb * a.rsub;       // items per row tile
  const int first_tile = min((int)(blockIdx.x / ipt), a.T - 1);
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
    n_items = n_tiles * ipt;
  } else if (a.mode == LORA_LAUNCH_BUCKETED) {
    rtiles = (P.sum[kRowBound] + LORA_TILE_SMALL - 1) / LORA_TILE_SMALL;
    n_items = a.slots * rtiles * ipt;
  }

  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int tile_item = item / ipt;
    const int in_tile = item - tile_item * ipt, sub = in_tile / a.nrb;
    const int rb = in_tile - sub * a.nrb;
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
    shrink_item_body<TI, NB, WAVES>(a, P, w, rb, red, sub);
  }
}


}  // namespace
}  // namespace lora
