// Work-item decoding shared by the row-tiled shrink and expand kernels.
//
// A work item is one row tile of one adapter segment (at most `TILE` rows of
// the grouped order) times one column block.  How blocks map to items
// depends on the launch-sizing mode ("LoRazor" 3.1.1-3.1.4):
//   EXACT / PERSISTENT  item = (tile list entry, column block); the tile list
//                       holds only tiles with live rows
//   BUCKETED / FULL     item = (slot s < L, row tile t < ceil(R/TILE) or
//                       ceil(T/TILE), column block); items whose slot or row
//                       tile holds no rows exit before touching any operand
#pragma once
#include "common.h"

namespace lora {

struct TileWork {
  int seg;     // segment index
  int p0;      // first grouped position of the tile
  int rows;    // 1 .. TILE
};

// Returns false when the item holds no rows.
template <int TILE>
__device__ __forceinline__ bool decode_tile(const SegPtrs& P, int mode, int tile_item, const int32_t* tiles,
                                            int rtiles, TileWork& w) {
  if (mode == LORA_LAUNCH_EXACT || mode == LORA_LAUNCH_PERSISTENT) {
    // a host count that disagrees with the device buffer never reads past it
    if (tile_item >= (TILE == LORA_TILE_SMALL ? P.sum[kNTilesSmall] : P.sum[kNTilesLarge])) return false;
    w.p0 = tiles[2 * tile_item];
    w.seg = tiles[2 * tile_item + 1];
    const int end = P.seg_start[w.seg + 1];
    w.rows = min(TILE, end - w.p0);
    return true;
  }
  const int s = tile_item / rtiles;
  const int t = tile_item - s * rtiles;
  if (s >= P.sum[kNSegments]) return false;
  const int begin = P.seg_start[s];
  const int end = P.seg_start[s + 1];
  w.p0 = begin + t * TILE;
  if (w.p0 >= end) return false;
  w.seg = s;
  w.rows = min(TILE, end - w.p0);
  return true;
}

// Number of tile items for the persistent mode, read on the device.
template <int TILE>
__device__ __forceinline__ int device_tile_count(const SegPtrs& P) {
  return TILE == LORA_TILE_SMALL ? P.sum[kNTilesSmall] : P.sum[kNTilesLarge];
}

// Host: grid size in tile items (before multiplying by column blocks).
inline int host_tile_items(const LaunchShape& ls, int T, int tile) {
  switch (ls.mode) {
    case LORA_LAUNCH_EXACT: return ls.n_tiles;
    case LORA_LAUNCH_BUCKETED: return ls.slots * ((ls.row_bound + tile - 1) / tile);
    case LORA_LAUNCH_FULL_BATCH: return ls.slots * ((T + tile - 1) / tile);
    default: return 0;
  }
}
inline int host_row_tiles(const LaunchShape& ls, int T, int tile) {
  if (ls.mode == LORA_LAUNCH_BUCKETED) return (ls.row_bound + tile - 1) / tile;
  return (T + tile - 1) / tile;
}

}  // namespace lora
