// One-workgroup grouping of token rows by adapter, shared by the segment
// builder kernels and the fused build-and-shrink kernel of small batches.
//
// "LLM-stack book 7.14", 7.14.2 (The data layout): the batch is sorted by
// adapter and described by seg_start / seg_adapter.  "LoRazor" 3.1.1: kernels
// gather inputs and scatter results through the adapter-grouped row-index
// array I_a (here `perm`), with m_a = |I_a|; 3.1.4 Eqs. 7-8: the row bound R.
#pragma once

#include "common.h"

namespace lora {
namespace {

struct BuildLds {
  int wave_sums[17];
  int4 wave_sums4[16];
  int err, nseg, nact, mmax, dead_run;
  int wave_dead[16];
  int run_base[16][64];     // per wave: base position of the run led by each lane
};

// Inclusive prefix sum over the 64 lanes of a wave: DPP shifts inside rows
// of 16 lanes, then row broadcasts (lane 15 into rows 1 and 3, lane 31 into
// rows 2 and 3).  Lanes whose DPP source is disabled add 0.
__device__ __forceinline__ int wave_incl_sum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);   // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);   // row_bcast:31
  return v;
}

// Maximum over the 64 lanes of a wave of values >= 0, in lane 63 (the same
// shifts as the sum; a disabled DPP source reads as 0).  Every lane of the
// wave must take part.
__device__ __forceinline__ int wave_max_nonneg(int v) {
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false));
  return v;
}

// Exclusive prefix sum of one value per thread over the workgroup; the total
// is written to *total for every thread.
template <int THREADS>
__device__ int block_exclusive_scan(int v, int* wave_sums, int* total) {
  constexpr int kWaves = THREADS / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_incl_sum(v);
  if (lane == 63) wave_sums[wave] = incl;
  lds_sync();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int t = wave_sums[w];
    if (w < wave) before += t;
    all += t;
  }
  *total = all;
  lds_sync();
  return before + incl - v;
}

// Exclusive prefix sums of four values per thread over the workgroup, with
// their totals (all threads).
template <int THREADS>
__device__ int4 block_exclusive_scan4(int4 v, int4* wave_sums, int4* total) {
  constexpr int kWaves = THREADS / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int4 incl = make_int4(wave_incl_sum(v.x), wave_incl_sum(v.y), wave_incl_sum(v.z), wave_incl_sum(v.w));
  if (lane == 63) wave_sums[wave] = incl;
  lds_sync();
  int4 before = make_int4(0, 0, 0, 0), all = make_int4(0, 0, 0, 0);
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int4 t = wave_sums[w];
    if (w < wave) { before.x += t.x; before.y += t.y; before.z += t.z; before.w += t.w; }
    all.x += t.x; all.y += t.y; all.z += t.z; all.w += t.w;
  }
  *total = all;
  lds_sync();
  return make_int4(before.x + incl.x - v.x, before.y + incl.y - v.y, before.z + incl.z - v.z,
                   before.w + incl.w - v.w);
}

// Runs of equal live ids inside one wave.  Returns the lane's rank among the
// live lanes of its id (lower lanes first); `leader` = lowest lane of the id,
// `run` = number of lanes of the id (valid in the leader lane).
__device__ __forceinline__ int wave_runs(bool live, int id, int lane, int& leader, int& run) {
  uint64_t remaining = __ballot(live);
  int rank = 0;
  leader = -1;
  run = 0;
  while (remaining) {
    const int l = __ffsll((unsigned long long)remaining) - 1;
    const int key = __builtin_amdgcn_readlane(id, l);   // l is wave-uniform: a VALU lane read, no LDS trip
    const uint64_t m = __ballot(live && id == key);
    if (live && id == key) {
      rank = __popcll(m & lanemask_lt());
      leader = l;
    }
    if (lane == l) run = __popcll(m);
    remaining &= ~m;
  }
  return rank;
}

// First-appearance order: segment lengths in segment order, then segment
// starts, row tiles and the placement cursors (cnt[a] = start of a's
// segment).  sh.nseg holds the segment count.
template <int THREADS>
__device__ void build_order1_segments(int N, int* cnt, const int* sidx, int* sst, const SegPtrs& P, BuildLds& sh) {
  const int tid = threadIdx.x;
  const int S = sh.nseg;
  int mx = 0;
  for (int base = 0; base < N; base += THREADS) {
    const int a = base + tid;
    const int c = a < N ? cnt[a] : 0;
    if (c > 0) {
      sst[sidx[a]] = c;
      P.seg_adapter[sidx[a]] = a;
    }
    mx = max(mx, c);
  }
  mx = wave_max_nonneg(mx);
  if ((tid & 63) == 63 && mx > 0) atomicMax(&sh.mmax, mx);
  lds_sync();

  // segment starts and row tiles
  {
    int run = 0, run_s = 0, run_l = 0;
    for (int base = 0; base < S; base += THREADS) {
      const int s = base + tid;
      const int len = s < S ? sst[s] : 0;
      const int ns = (len + LORA_TILE_SMALL - 1) / LORA_TILE_SMALL;
      const int nl = (len + LORA_TILE_LARGE - 1) / LORA_TILE_LARGE;
      int tot, tot_s, tot_l;
      const int st = block_exclusive_scan<THREADS>(len, sh.wave_sums, &tot) + run;
      const int os = block_exclusive_scan<THREADS>(ns, sh.wave_sums, &tot_s) + run_s;
      const int ol = block_exclusive_scan<THREADS>(nl, sh.wave_sums, &tot_l) + run_l;
      if (s < S) {
        P.seg_start[s] = st;
        for (int t = 0; t < ns; ++t) {
          P.tiles_small[2 * (os + t)] = st + t * LORA_TILE_SMALL;
          P.tiles_small[2 * (os + t) + 1] = s;
        }
        for (int t = 0; t < nl; ++t) {
          P.tiles_large[2 * (ol + t)] = st + t * LORA_TILE_LARGE;
          P.tiles_large[2 * (ol + t) + 1] = s;
        }
        sst[s] = st;
      }
      run += tot;
      run_s += tot_s;
      run_l += tot_l;
    }
    if (tid == 0) {
      P.seg_start[S] = run;
      sh.nact = run;
      P.sum[kNTilesSmall] = run_s;
      P.sum[kNTilesLarge] = run_l;
    }
  }
  lds_sync();

  // placement cursor per adapter = start of its segment
  for (int a = tid; a < N; a += THREADS)
    if (cnt[a] > 0) cnt[a] = sst[sidx[a]];
}

// Canonical order (ascending adapter id): segment index, start and row-tile
// offsets of every present adapter are one four-field prefix sum over the
// adapters; cnt[a] (rows of a) becomes a's placement cursor.  Sets sh.nseg,
// sh.nact, sh.mmax and the tile counts of the summary.
template <int THREADS>
__device__ void canonical_segments(int N, int* cnt, int* sidx, const SegPtrs& P, BuildLds& sh) {
  const int tid = threadIdx.x;
  int4 run = make_int4(0, 0, 0, 0);
  int mx = 0;
  for (int base = 0; base < N; base += THREADS) {
    const int a = base + tid;
    const int len = a < N ? cnt[a] : 0;
    const int ns = (len + LORA_TILE_SMALL - 1) / LORA_TILE_SMALL;
    const int nl = (len + LORA_TILE_LARGE - 1) / LORA_TILE_LARGE;
    int4 tot;
    const int4 ex = block_exclusive_scan4<THREADS>(make_int4(len > 0, len, ns, nl), sh.wave_sums4, &tot);
    if (len > 0) {
      const int sg = run.x + ex.x, st = run.y + ex.y, os = run.z + ex.z, ol = run.w + ex.w;
      sidx[a] = sg;
      P.seg_adapter[sg] = a;
      P.seg_start[sg] = st;
      for (int t = 0; t < ns; ++t) {
        P.tiles_small[2 * (os + t)] = st + t * LORA_TILE_SMALL;
        P.tiles_small[2 * (os + t) + 1] = sg;
      }
      for (int t = 0; t < nl; ++t) {
        P.tiles_large[2 * (ol + t)] = st + t * LORA_TILE_LARGE;
        P.tiles_large[2 * (ol + t) + 1] = sg;
      }
      cnt[a] = st;
    }
    mx = max(mx, len);
    run.x += tot.x; run.y += tot.y; run.z += tot.z; run.w += tot.w;
  }
  // m_max: one wave maximum and one LDS atomic per wave (a per-lane atomic on
  // one address becomes a serial loop over the lanes)
  mx = wave_max_nonneg(mx);
  if ((tid & 63) == 63 && mx > 0) atomicMax(&sh.mmax, mx);
  if (tid == 0) {
    sh.nseg = run.x;
    sh.nact = run.y;
    P.seg_start[run.x] = run.y;
    P.sum[kNTilesSmall] = run.z;
    P.sum[kNTilesLarge] = run.w;
  }
}

// Batches of at most 256 rows and pools of at most kSmallMaxSlots adapters:
// per-wave lane masks instead of a loop over distinct ids.  Each live lane
// sets its bit in tbl[wave][id] (a 64-bit LDS OR) and reads the word back:
// its rank among the wave's rows of that id is the popcount of the lower
// lanes, the lowest set lane leads the run.  A row's place in its segment is
// the segment start plus the rows of its id in earlier waves (their words)
// plus its rank, so rows stay in batch order inside every segment.
constexpr int kSmallRows = 256;
constexpr int kSmallMaxSlots = 1024;   // 4 waves x N x 8 bytes of masks

// The whole build by one workgroup of kSmallRows threads, into the segment
// buffer P (global memory, or a workgroup's LDS copy); tbl is LDS scratch of
// small_build_lds_bytes(N).  Returns false (summary error set) for an id
// out of range.  Every thread of the workgroup must call it.
__device__ __forceinline__ bool small_build(const int32_t* __restrict__ ids, const uint8_t* __restrict__ active, int T,
                                            int N, int order, const SegPtrs& P, uint64_t* tbl, BuildLds& sh) {
  constexpr int kWaves = kSmallRows / 64;
  int* cnt = reinterpret_cast<int*>(tbl + kWaves * N);              // [N] rows, then placement cursor
  int* sidx = cnt + N;                                              // [N] segment index per adapter
  int* sst = sidx + N;                                              // [N] first appearance: lengths/starts

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;

  int id = -1, on = 1;
  if (tid < T) {
    id = ids[tid];
    if (active != nullptr) on = active[tid];
  }
  for (int a = tid; a < N; a += kSmallRows) {
    cnt[a] = 0;
    sidx[a] = (order == 1) ? 0x7fffffff : 0;
  }
  for (int q = tid; q < kWaves * N; q += kSmallRows) tbl[q] = 0ull;
  if (tid == 0) { sh.err = 0; sh.mmax = 0; }
  lds_sync();

  // 1. masks, histogram, validation, first appearance
  bool live = false;
  if (tid < T) {
    if (id < -1 || id >= N) sh.err = 1;
    else live = id >= 0 && on != 0;
  }
  uint64_t* mine = tbl + wave * N;
  if (live) atomicOr(reinterpret_cast<unsigned long long*>(&mine[id]), 1ull << lane);
  lds_sync();
  const uint64_t m = live ? mine[id] : 0ull;
  if (live && lane == __ffsll((unsigned long long)m) - 1) {
    atomicAdd(&cnt[id], __popcll(m));
    if (order == 1) atomicMin(&sidx[id], tid);
  }
  lds_sync();
  if (sh.err) {
    if (tid == 0) {
      for (int w = 0; w < kSegHeader; ++w) P.sum[w] = 0;
      P.sum[kRows] = T;
      P.sum[kError] = LORA_E_ID;
    }
    return false;
  }

  // 2. segments
  if (order == 0) {
    canonical_segments<kSmallRows>(N, cnt, sidx, P, sh);
  } else {
    // rows that are the first appearance of their adapter, in batch order
    int tot;
    const int first = (live && sidx[id] == tid) ? 1 : 0;
    const int ex = block_exclusive_scan<kSmallRows>(first, sh.wave_sums, &tot);
    if (first) sidx[id] = ex;
    if (tid == 0) sh.nseg = tot;
    lds_sync();
    build_order1_segments<kSmallRows>(N, cnt, sidx, sst, P, sh);
  }
  lds_sync();

  // 3. scatter: live rows at their segment place, the others after all live
  // rows in batch order
  const int n_active = sh.nact;
  const uint64_t dead_mask = __ballot(tid < T && !live);
  if (lane == 0) sh.wave_dead[wave] = __popcll(dead_mask);
  lds_sync();
  if (tid < T) {
    int pos;
    if (live) {
      pos = cnt[id] + __popcll(m & lanemask_lt());
      for (int w = 0; w < wave; ++w) pos += __popcll(tbl[w * N + id]);
    } else {
      pos = n_active + __popcll(dead_mask & lanemask_lt());
      for (int w = 0; w < wave; ++w) pos += sh.wave_dead[w];
    }
    P.perm[pos] = tid;
    P.pos_seg[pos] = live ? sidx[id] : -1;
  }

  // 4. summary; R = min{r in {16*2^k < T} U {T} : r >= m_max}
  if (tid == 0) {
    const int mmax = sh.mmax;
    int R = 0;
    if (n_active > 0) {
      R = T;
      for (int r = 16; r < T; r <<= 1)
        if (r >= mmax) { R = r; break; }
    }
    P.sum[kNActive] = n_active;
    P.sum[kNSegments] = sh.nseg;
    P.sum[kMMax] = mmax;
    P.sum[kRowBound] = R;
    P.sum[kRows] = T;
    P.sum[kError] = 0;
    for (int w = 8; w < kSegHeader; ++w) P.sum[w] = 0;
  }
  return true;
}

__host__ __device__ inline size_t small_build_lds_bytes(int N) {
  return (size_t)(kSmallRows / 64) * N * sizeof(uint64_t) + 3 * (size_t)N * sizeof(int);
}


}  // namespace
}  // namespace lora
