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

// Batches of 2049 .. kWaveRowsMax * 1024 rows over at most kWaveMaxSlots
// adapters: each of the 16 waves owns one contiguous range of rows (a
// multiple of 64), so the placement needs no barrier per chunk.  Every wave
// counts its rows per adapter in its own LDS row wc[wave][a] (step 1); after
// the segments are laid out, one pass per adapter turns the 16 counts into
// per-wave cursors (segment start plus the rows of earlier waves); each wave
// then places its rows in order, advancing only its own cursors.  Rows land
// in batch order inside every segment, as in the chunked build.
constexpr int kWaveRowsMax = 16;      // 64-row sub-chunks per wave (T <= 16384)
constexpr int kWaveMaxSlots = 1024;   // 16 x N counts in LDS

__global__ __launch_bounds__(1024) void build_segments_waves_kernel(const int32_t* __restrict__ ids,
                                                                   const uint8_t* __restrict__ active, int T,
                                                                   int N, int order, int32_t* __restrict__ seg) {
  constexpr int THREADS = 1024, kW = THREADS / 64;
  extern __shared__ int lds[];
  int* cnt = lds;           // [N] live rows per adapter, later the segment start
  int* sidx = lds + N;      // [N] segment index per adapter (order 1: first row first)
  int* sst = lds + 2 * N;   // [N] (order 1) segment lengths, then starts
  int* wc = lds + 3 * N;    // [kW][N] rows of each adapter per wave, then the wave's cursors
  __shared__ BuildLds sh;
  __shared__ int wave_first[kW];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  SegPtrs P = seg_ptrs(seg, T);
  const int rpw = (T + kW * 64 - 1) / (kW * 64) * 64;   // rows per wave
  const int r0 = wave * rpw;
  const int nsub = r0 < T ? (min(T, r0 + rpw) - r0 + 63) / 64 : 0;

  // every id and flag of this wave's rows in flight at once
  int idv[kWaveRowsMax];
  int onv[kWaveRowsMax];
#pragma unroll
  for (int q = 0; q < kWaveRowsMax; ++q) {
    const int i = r0 + q * 64 + lane;
    idv[q] = -1;
    onv[q] = 1;
    if (q < nsub && i < T) {
      idv[q] = ids[i];
      if (active != nullptr) onv[q] = active[i];
    }
  }
  for (int a = tid; a < N; a += THREADS) {
    cnt[a] = 0;
    sidx[a] = (order == 1) ? 0x7fffffff : 0;
  }
  for (int q = tid; q < kW * N; q += THREADS) wc[q] = 0;
  if (tid == 0) { sh.err = 0; sh.mmax = 0; }
  lds_sync();

  // 1. per-wave counts, validation, first appearance; idv keeps the live id
  // of each row (-1: not live)
  bool bad = false;
  int ndead = 0;
#pragma unroll
  for (int q = 0; q < kWaveRowsMax; ++q) {
    if (q < nsub) {
      const int i = r0 + q * 64 + lane;
      const int id = idv[q];
      const bool in = i < T;
      bad |= in && (id < -1 || id >= N);
      const bool live = in && id >= 0 && id < N && onv[q] != 0;
      int leader, run;
      wave_runs(live, id, lane, leader, run);
      if (run > 0) {
        wc[wave * N + id] += run;                 // this wave's row of counts: no other writer
        if (order == 1) atomicMin(&sidx[id], i);
      }
      ndead += __popcll(__ballot(in && !live));
      idv[q] = live ? id : -1;
    }
  }
  if (bad) sh.err = 1;
  if (lane == 0) sh.wave_dead[wave] = ndead;
  lds_sync();
  if (sh.err) {
    if (tid == 0) {
      for (int w = 0; w < kSegHeader; ++w) P.sum[w] = 0;
      P.sum[kRows] = T;
      P.sum[kError] = LORA_E_ID;
    }
    return;
  }
  for (int a = tid; a < N; a += THREADS) {
    int c = 0;
    for (int w = 0; w < kW; ++w) c += wc[w * N + a];
    cnt[a] = c;
  }
  lds_sync();

  // 2. segments
  if (order == 0) {
    canonical_segments<THREADS>(N, cnt, sidx, P, sh);
  } else {
    // rows that are the first appearance of their adapter, numbered in batch
    // order: per wave in its row order, the waves in order
    uint64_t fm[kWaveRowsMax];
    int nf = 0;
#pragma unroll
    for (int q = 0; q < kWaveRowsMax; ++q) {
      fm[q] = 0;
      if (q < nsub) {
        const int i = r0 + q * 64 + lane;
        const int id = idv[q];
        fm[q] = __ballot(id >= 0 && sidx[id] == i);
        nf += __popcll(fm[q]);
      }
    }
    if (lane == 0) wave_first[wave] = nf;
    lds_sync();
    int run = 0;
    for (int w = 0; w < wave; ++w) run += wave_first[w];
#pragma unroll
    for (int q = 0; q < kWaveRowsMax; ++q) {
      if (q < nsub) {
        const int id = idv[q];
        if ((fm[q] >> lane) & 1) sidx[id] = run + __popcll(fm[q] & lanemask_lt());
        run += __popcll(fm[q]);
      }
    }
    if (tid == 0) {
      int tot = 0;
      for (int w = 0; w < kW; ++w) tot += wave_first[w];
      sh.nseg = tot;
    }
    lds_sync();
    build_order1_segments<THREADS>(N, cnt, sidx, sst, P, sh);
  }
  lds_sync();
  const int S = sh.nseg;
  const int n_active = sh.nact;

  // 3. per-wave cursors (cnt[a] now holds a's segment start) and the place
  // of each wave's first non-live row (after all live rows, batch order)
  for (int a = tid; a < N; a += THREADS) {
    int run = cnt[a];
    for (int w = 0; w < kW; ++w) {
      const int c = wc[w * N + a];
      wc[w * N + a] = run;
      run += c;
    }
  }
  int dcur = n_active;
  for (int w = 0; w < wave; ++w) dcur += sh.wave_dead[w];
  lds_sync();

  // 4. placement, each wave in its own row order
#pragma unroll
  for (int q = 0; q < kWaveRowsMax; ++q) {
    if (q < nsub) {
      const int i = r0 + q * 64 + lane;
      const int id = idv[q];
      const bool live = id >= 0;
      int leader, run;
      const int rank = wave_runs(live, id, lane, leader, run);
      int pos = 0;
      if (live) {
        const int b = wc[wave * N + id];
        pos = b + rank;
        if (run > 0) wc[wave * N + id] = b + run;   // after every lane of the id has read it
      }
      const uint64_t dm = __ballot(i < T && !live);
      if (i < T && !live) pos = dcur + __popcll(dm & lanemask_lt());
      dcur += __popcll(dm);
      if (i < T) {
        P.perm[pos] = i;
        P.pos_seg[pos] = live ? sidx[id] : -1;
      }
    }
  }

  // 5. summary; R = min{r in {16*2^k < T} U {T} : r >= m_max}
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
  // (at most two chunks: the chunked build is as fast, without the 16 x N
  // table passes; measured on MI355X at T = 512 and 2048)
  if (T > 2048 && T <= kWaveRowsMax * 1024 && n_slots >= 1 && n_slots <= kWaveMaxSlots) {
    const size_t lds = (3 + 16) * (size_t)n_slots * sizeof(int);
    if (lds > 65536) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(build_segments_waves_kernel),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(build_segments_waves_kernel, dim3(1), dim3(1024), lds, st, ids, active, T, n_slots, order,
                       seg);
    return hipGetLastError();
  }
  return launch_threads<1024>(ids, active, T, n_slots, order, seg, st);
}

}  // namespace lora
