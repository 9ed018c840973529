// Device-side grouping of token rows by adapter.
//
// "LLM-stack book 7.14", 7.14.2 (The data layout): the batch is sorted by
// adapter and described by seg_start / seg_adapter.  "LoRazor" 3.1.1: kernels
// gather inputs and scatter results through the adapter-grouped row-index
// array I_a (here `perm`), with m_a = |I_a|; 3.1.4 Eqs. 7-8: the row bound R.
//
// One workgroup does the whole build (256 threads for batches of at most 256
// rows, else 1024); rows are taken in chunks of one row per thread (a batch
// that fits one chunk keeps its rows in registers from step 1 to step 3):
//   1. per wave, a ballot loop splits the wave's live rows into runs of equal
//      id: every lane learns its rank among equal ids inside the wave, and one
//      leader lane per distinct id adds the run length to an LDS histogram
//      (for order = 1 it also records the first row of the id);
//   2. segment index per adapter, segment starts, row tiles of 16 and 64
//      rows, m_max and R.  Canonical order: one scan over the adapters of
//      (present, rows, 16-row tiles, 64-row tiles) gives all of them and the
//      placement cursors at once.  First-appearance order: a scan of first
//      appearances over the rows, then a scan over the segments;
//   3. the chunk's waves visit a per-adapter cursor in wave order: each
//      leader takes its run's base position and advances the cursor, so rows
//      land in batch order inside every segment (stable, deterministic) while
//      the ballot work itself runs in all waves at once.
#include "build_small.h"

namespace lora {
namespace {

template <int THREADS>
__global__ __launch_bounds__(THREADS) void build_segments_kernel(const int32_t* __restrict__ ids,
                                                                 const uint8_t* __restrict__ active, int T, int N,
                                                                 int order, int32_t* __restrict__ seg) {
  constexpr int kWaves = THREADS / 64;
  extern __shared__ int lds[];
  int* cnt = lds;           // [N] live rows per adapter, later the placement cursor
  int* sidx = lds + N;      // [N] segment index per adapter (order 1: first row first)
  int* sst = lds + 2 * N;   // [N] segment lengths, then segment starts, in segment order
  __shared__ BuildLds sh;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  SegPtrs P = seg_ptrs(seg, T);

  // the first chunk's ids and flags are loaded together, before the LDS set-up
  int id0 = -1, on0 = 1;
  if (tid < T) {
    id0 = ids[tid];
    if (active != nullptr) on0 = active[tid];
  }
  for (int a = tid; a < N; a += THREADS) {
    cnt[a] = 0;
    sidx[a] = (order == 1) ? 0x7fffffff : 0;
  }
  if (tid == 0) { sh.err = 0; sh.mmax = 0; sh.dead_run = 0; }
  lds_sync();

  // 1. histogram by runs, validation, first appearance.  A batch of at most
  // THREADS rows is one chunk: its ids, live flags and runs stay in registers
  // for the scatter.
  const bool single = T <= THREADS;
  int r_id = -1, r_rank = 0, r_leader = -1, r_run = 0;
  bool r_live = false;
  for (int base = 0; base < T; base += THREADS) {
    const int i = base + tid;
    int id = -1;
    bool live = false;
    if (i < T) {
      bool on = on0 != 0;
      id = id0;
      if (base > 0) {
        id = ids[i];
        on = active == nullptr || active[i] != 0;   // both loads in flight together
      }
      if (id < -1 || id >= N) sh.err = 1;
      else live = id >= 0 && on;
    }
    if (base + wave * 64 < T) {
      int leader, run;
      const int rank = wave_runs(live, id, lane, leader, run);
      if (run > 0) {
        atomicAdd(&cnt[id], run);
        if (order == 1) atomicMin(&sidx[id], i);
      }
      if (single) { r_id = id; r_live = live; r_rank = rank; r_leader = leader; r_run = run; }
    }
  }
  lds_sync();
  if (sh.err) {
    if (tid == 0) {
      for (int w = 0; w < kSegHeader; ++w) P.sum[w] = 0;
      P.sum[kRows] = T;
      P.sum[kError] = LORA_E_ID;
    }
    return;
  }

  // 2. segments
  if (order == 0) {
    canonical_segments<THREADS>(N, cnt, sidx, P, sh);
  } else {
    // rows that are the first appearance of their adapter, in batch order;
    // indices are stored negated so that a later row never matches
    int run = 0;
    for (int base = 0; base < T; base += THREADS) {
      const int i = base + tid;
      int id = -1, first = 0;
      if (i < T) {
        id = ids[i];
        const bool on = active == nullptr || active[i] != 0;
        const bool live = id >= 0 && on;
        first = (live && sidx[id] == i) ? 1 : 0;
      }
      int tot;
      const int ex = block_exclusive_scan<THREADS>(first, sh.wave_sums, &tot);
      if (first) sidx[id] = -(run + ex) - 1;
      run += tot;
    }
    lds_sync();
    for (int a = tid; a < N; a += THREADS)
      if (cnt[a] > 0) sidx[a] = -sidx[a] - 1;
    if (tid == 0) sh.nseg = run;
    lds_sync();
    build_order1_segments<THREADS>(N, cnt, sidx, sst, P, sh);
  }
  lds_sync();
  const int S = sh.nseg;


  // 3. stable scatter, chunk by chunk
  const int n_active = sh.nact;
  for (int base = 0; base < T; base += THREADS) {
    const int i = base + tid;
    int id = r_id, leader = r_leader, run = r_run, rank = r_rank;
    bool live = r_live;
    if (!single) {
      id = -1;
      live = false;
      if (i < T) {
        id = ids[i];
        const bool on = active == nullptr || active[i] != 0;
        live = id >= 0 && on;
      }
      leader = -1;
      run = 0;
      rank = 0;
      if (base + wave * 64 < T) rank = wave_runs(live, id, lane, leader, run);
    }
    const uint64_t dead_mask = __ballot(i < T && !live);
    if (lane == 0) sh.wave_dead[wave] = __popcll(dead_mask);
    // waves take their cursor positions in wave order
    const int chunk_waves = min(kWaves, (T - base + 63) / 64);
    for (int w = 0; w < chunk_waves; ++w) {
      if (wave == w && run > 0) {
        const int b = cnt[id];
        cnt[id] = b + run;
        sh.run_base[wave][lane] = b;
      }
      lds_sync();
    }
    int dead_before = sh.dead_run;
    for (int w = 0; w < wave; ++w) dead_before += sh.wave_dead[w];
    if (i < T) {
      int pos;
      if (live) pos = sh.run_base[wave][leader] + rank;
      else pos = n_active + dead_before + __popcll(dead_mask & lanemask_lt());
      P.perm[pos] = i;
      P.pos_seg[pos] = live ? sidx[id] : -1;
    }
    lds_sync();
    if (tid == 0) {
      int d = 0;
      for (int w = 0; w < kWaves; ++w) d += sh.wave_dead[w];
      sh.dead_run += d;
    }
    lds_sync();
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
    P.sum[kNSegments] = S;
    P.sum[kMMax] = mmax;
    P.sum[kRowBound] = R;
    P.sum[kRows] = T;
    P.sum[kError] = 0;
    for (int w = 8; w < kSegHeader; ++w) P.sum[w] = 0;
  }
}

__global__ __launch_bounds__(kSmallRows) void build_segments_small_kernel(const int32_t* __restrict__ ids,
                                                                          const uint8_t* __restrict__ active, int T,
                                                                          int N, int order,
                                                                          int32_t* __restrict__ seg) {
  extern __shared__ __attribute__((aligned(16))) uint64_t tbl[];   // small_build_lds_bytes(N)
  __shared__ BuildLds sh;
  small_build(ids, active, T, N, order, seg_ptrs(seg, T), tbl, sh);
}

template <int THREADS>
hipError_t launch_threads(const int32_t* ids, const uint8_t* active, int T, int n_slots, int order, int32_t* seg,
                          hipStream_t st) {
  const size_t lds = 3 * (size_t)(n_slots > 0 ? n_slots : 1) * sizeof(int);
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(build_segments_kernel<THREADS>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(build_segments_kernel<THREADS>, dim3(1), dim3(THREADS), lds, st, ids, active, T, n_slots,
                     order, seg);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_build_segments(const int32_t* ids, const uint8_t* active, int T, int n_slots, int order,
                                 int32_t* seg, hipStream_t st) {
  if (T <= kSmallRows && n_slots >= 1 && n_slots <= kSmallMaxSlots) {
    const size_t lds = small_build_lds_bytes(n_slots);
    hipLaunchKernelGGL(build_segments_small_kernel, dim3(1), dim3(kSmallRows), lds, st, ids, active, T, n_slots,
                       order, seg);
    return hipGetLastError();
  }
  if (T <= 256) return launch_threads<256>(ids, active, T, n_slots, order, seg, st);
  return launch_threads<1024>(ids, active, T, n_slots, order, seg, st);
}

}  // namespace lora
