// Device-side grouping of token rows by adapter.
//
// "LLM-stack book 7.14", 7.14.2 (The data layout): the batch is sorted by
// adapter and described by seg_start / seg_adapter.  "LoRazor" 3.1.1: kernels
// gather inputs and scatter results through the adapter-grouped row-index
// array I_a (here `perm`), with m_a = |I_a|; 3.1.4 Eqs. 7-8: the row bound R.
//
// One workgroup of 1024 threads does the whole build (decode/prefill batches
// are a few thousand rows; the build is a handful of microseconds):
//   1. histogram of live ids in LDS (and first appearance for order = 1),
//   2. segment index per adapter (exclusive scan of "present", or of first
//      appearances over the rows), segment lengths and starts,
//   3. stable scatter: rows are visited in batch order, 1024 at a time; the
//      16 waves of a chunk take turns, each placing its 64 rows with ballots
//      (rows of equal id inside a wave get consecutive slots in lane order),
//      so the grouping is deterministic and stable without a sort,
//   4. per-segment row tiles of 16 and 64 rows, m_max, R and the summary.
#include "common.h"

namespace lora {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

// exclusive scan of one value per thread over the workgroup; returns the
// prefix and writes the total to *total (valid for all threads after return)
__device__ int block_exclusive_scan(int v, int* wave_sums, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) wave_sums[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    int s = lane < kWaves ? wave_sums[lane] : 0;
    int si = s;
#pragma unroll
    for (int o = 1; o < kWaves; o <<= 1) {
      int t = __shfl_up(si, o, 64);
      if (lane >= o) si += t;
    }
    if (lane < kWaves) wave_sums[lane] = si - s;      // exclusive wave offsets
    if (lane == kWaves - 1) wave_sums[kWaves] = si;   // total
  }
  __syncthreads();
  int res = wave_sums[wave] + incl - v;
  *total = wave_sums[kWaves];
  __syncthreads();                                     // wave_sums reusable
  return res;
}

__global__ __launch_bounds__(kThreads) void build_segments_kernel(const int32_t* __restrict__ ids,
                                                                  const uint8_t* __restrict__ active, int T,
                                                                  int N, int order, int32_t* __restrict__ seg) {
  extern __shared__ int lds[];
  int* cnt = lds;           // [N] live rows per adapter, later the placement cursor
  int* sidx = lds + N;      // [N] segment index per adapter (order 1: first row first)
  int* slen = lds + 2 * N;  // [N] segment lengths in segment order
  __shared__ int wave_sums[kWaves + 1];
  __shared__ int s_err, s_nseg, s_nact, s_mmax, s_inact, s_run;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  SegPtrs P = seg_ptrs(seg, T);

  for (int a = tid; a < N; a += kThreads) {
    cnt[a] = 0;
    sidx[a] = (order == 1) ? 0x7fffffff : 0;
    slen[a] = 0;
  }
  if (tid == 0) { s_err = 0; s_mmax = 0; s_inact = 0; s_run = 0; }
  __syncthreads();

  // 1. histogram, validation, first appearance
  for (int i = tid; i < T; i += kThreads) {
    int id = ids[i];
    if (id < -1 || id >= N) {
      s_err = 1;
    } else if (id >= 0 && (active == nullptr || active[i] != 0)) {
      atomicAdd(&cnt[id], 1);
      if (order == 1) atomicMin(&sidx[id], i);
    }
  }
  __syncthreads();
  if (s_err) {
    if (tid == 0) {
      for (int w = 0; w < kSegHeader; ++w) P.sum[w] = 0;
      P.sum[kRows] = T;
      P.sum[kError] = LORA_E_ID;
    }
    return;
  }

  // 2. segment index of each present adapter
  if (order == 0) {
    int run = 0;
    for (int base = 0; base < N; base += kThreads) {
      int a = base + tid;
      int present = (a < N && cnt[a] > 0) ? 1 : 0;
      int tot;
      int ex = block_exclusive_scan(present, wave_sums, &tot);
      if (present) sidx[a] = run + ex;
      run += tot;
    }
    if (tid == 0) s_nseg = run;
  } else {
    // rows that are the first appearance of their adapter, in batch order;
    // assigned indices are stored negated so that a later row never matches
    int run = 0;
    for (int base = 0; base < T; base += kThreads) {
      int i = base + tid;
      int id = -1, first = 0;
      if (i < T) {
        id = ids[i];
        bool live = id >= 0 && (active == nullptr || active[i] != 0);
        first = (live && sidx[id] == i) ? 1 : 0;
      }
      int tot;
      int ex = block_exclusive_scan(first, wave_sums, &tot);   // contains barriers
      if (first) sidx[id] = -(run + ex) - 1;
      run += tot;
      __syncthreads();
    }
    for (int a = tid; a < N; a += kThreads)
      if (cnt[a] > 0) sidx[a] = -sidx[a] - 1;
    if (tid == 0) s_nseg = run;
  }
  __syncthreads();
  const int S = s_nseg;

  // segment lengths and adapters in segment order
  for (int a = tid; a < N; a += kThreads) {
    if (cnt[a] > 0) {
      slen[sidx[a]] = cnt[a];
      P.seg_adapter[sidx[a]] = a;
      atomicMax(&s_mmax, cnt[a]);
    }
  }
  __syncthreads();

  // segment starts; tiles
  {
    int run = 0, run_s = 0, run_l = 0;
    for (int base = 0; base < S; base += kThreads) {
      int s = base + tid;
      int len = s < S ? slen[s] : 0;
      int ns = (len + LORA_TILE_SMALL - 1) / LORA_TILE_SMALL;
      int nl = (len + LORA_TILE_LARGE - 1) / LORA_TILE_LARGE;
      int tot, tot_s, tot_l;
      int st = block_exclusive_scan(len, wave_sums, &tot) + run;
      int os = block_exclusive_scan(ns, wave_sums, &tot_s) + run_s;
      int ol = block_exclusive_scan(nl, wave_sums, &tot_l) + run_l;
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
        slen[s] = st;               // slen now holds the start of segment s
      }
      run += tot;
      run_s += tot_s;
      run_l += tot_l;
    }
    if (tid == 0) {
      P.seg_start[S] = run;
      s_nact = run;
      P.sum[kNTilesSmall] = run_s;
      P.sum[kNTilesLarge] = run_l;
    }
  }
  __syncthreads();

  // placement cursor per adapter = start of its segment
  for (int a = tid; a < N; a += kThreads)
    if (cnt[a] > 0) cnt[a] = slen[sidx[a]];
  __syncthreads();

  // 3. stable scatter, chunk by chunk; waves take turns within a chunk
  const int n_active = s_nact;
  for (int base = 0; base < T; base += kThreads) {
    const int i = base + tid;
    int id = -1;
    bool live = false;
    if (i < T) {
      id = ids[i];
      live = id >= 0 && (active == nullptr || active[i] != 0);
    }
    for (int w = 0; w < kWaves; ++w) {
      if (wave == w) {
        const uint64_t live_mask = __ballot(live);
        const uint64_t dead_mask = __ballot(i < T && !live);
        uint64_t remaining = live_mask;
        int pos = -1;
        while (remaining) {
          const int leader = __ffsll((unsigned long long)remaining) - 1;
          const int key = __shfl(id, leader, 64);
          const uint64_t m = __ballot(live && id == key);
          int b = 0;
          if (lane == leader) {
            b = cnt[key];
            cnt[key] = b + __popcll(m);
          }
          b = __shfl(b, leader, 64);
          if (live && id == key) pos = b + __popcll(m & lanemask_lt());
          remaining &= ~m;
        }
        const int dead_base = s_inact;
        if (i < T && !live) pos = n_active + dead_base + __popcll(dead_mask & lanemask_lt());
        if (i < T) {
          P.perm[pos] = i;
          P.pos_seg[pos] = live ? sidx[id] : -1;
        }
        if (lane == 0) s_inact = dead_base + __popcll(dead_mask);
      }
      __syncthreads();
    }
  }

  // 4. summary; R = min{r in {16*2^k < T} U {T} : r >= m_max}
  if (tid == 0) {
    const int mmax = s_mmax;
    int R = 0;
    if (n_active > 0) {
      R = T;
      for (int r = 16; r < T; r <<= 1)
        if (r >= mmax) { R = r; break; }
    }
    P.sum[kNActive] = n_active;
    P.sum[kNSegments] = S;
    P.sum[kMMax] = mmax;
    P.sum[kRowBound] = R;
    P.sum[kRows] = T;
    P.sum[kError] = 0;
    for (int w = 8; w < kSegHeader; ++w) P.sum[w] = 0;
  }
}

}  // namespace

hipError_t launch_build_segments(const int32_t* ids, const uint8_t* active, int T, int n_slots, int order,
                                 int32_t* seg, hipStream_t st) {
  size_t lds = 3 * (size_t)n_slots * sizeof(int);
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(build_segments_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(build_segments_kernel, dim3(1), dim3(kThreads), lds, st, ids, active, T, n_slots, order,
                     seg);
  return hipGetLastError();
}

}  // namespace lora
