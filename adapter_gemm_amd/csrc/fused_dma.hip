// Fused linear, pipelined form for gfx950:
//   y[i, n] = epi( sum_k x[i, k] W0[n, k] ) + [live_i] s_a sum_j v[p(i), j] B_a[n, j]
// ("EpiLoRA" 3.1 and Fig. 10, kernel K2: a GEMM over adapter-sorted rows
// whose epilogue adds, per adapter group in the output tile, h_l B_l^T over
// the tile's slice of B_l, then writes rows back in token order).
//
// Main loop.  A workgroup (4 or 8 waves in a WGM x WGN grid) owns a BM x BN
// output tile.  Every
// k-step stages a BM x 128-byte slab of x rows (gathered through the grouped
// order) and a BN x 128-byte (bf16, W8A8) or BN x 64-byte (fp8 codes, W8A16)
// slab of W0 rows in one slot of an LDS ring of STAGES slots.  The slabs are
// moved by buffer_load_dwordx4 ... lds (each lane chooses its own 16-byte
// source, so the XOR swizzle of the LDS layout is applied on the source
// side), with STAGES - 1 k-steps in flight; waits use explicit vmcnt counts
// and a plain s_barrier, so no fence or compiler-inserted wait drains the
// ring.  Rows past T and
// channels past d_out use a buffer offset beyond the descriptor's range,
// which the hardware turns into zeros.  MFMA: v_mfma_f32_16x16x32_bf16
// (bf16, and W8A16 with codes widened to bf16 as fragments leave LDS) or
// v_mfma_scale_f32_16x16x128_f8f6f4 (W8A8).
//
// Adapter phase.  The tile's adapter groups (segments that meet its rows)
// become extra pipelined steps: step (group g, rank chunk c) stages
// B_g[n0 : n0 + BN, 64c : 64c + 64] through the same ring, rank entries at or
// beyond the adapter's rank read as zeros, and multiplies it by s_g v of the
// group's rows, held as a bf16 tile in LDS with rows of other groups masked
// to zero.  The products land on the same accumulators as the base GEMM.
//
// Output slices.  One launch can cover several projections of the same x
// (q / k / v, gate / up: "LoRAForge" 4, S slices per layer), each with its
// own W0 rows, adapter pool, v and y: the tile grid's columns are the slices'
// column tiles laid end to end, and a workgroup takes the slice of its column
// tile (slices start at tile boundaries; a slice's last tile may be ragged).
//
// Split K.  When the output has too few tiles to fill the chip (decode
// batches), the k range is split over `splits` workgroups per tile and one
// more workgroup per tile runs the adapter phase alone.  Each writes its
// scaled partial tile to the workspace; the last to arrive (an integer
// counter per tile) adds the partials in split order, so the result does not
// depend on which workgroup finished last, writes y and re-arms the counter.
#include "common.h"
#include "shrink_core.h"

#include <algorithm>

namespace lora {
namespace {

enum DmaMode { kBF16 = 0, kW8A16 = 1, kW8A8 = 2 };
constexpr uint32_t kOOB = 0x80000000u;   // offset past every descriptor's range: loads return zeros
constexpr int kLoraNBMax = 4;            // adapter-phase ring slots (at most)
constexpr int kPersistMinTiles = 256;    // persistent launches above this many tiles (MI355X CUs)
constexpr int kPersistCounters = 16;     // per-XCD claim counters (8 used), 64 bytes of workspace
constexpr int kBufferWord3 = 0x00020000; // raw 32-bit buffer, gfx9-family descriptor word 3

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

constexpr int kMaxSlices = 4;

// One output slice of a launch (everything that differs between slices).
struct SliceArgs {
  const void* W;
  const float* w_scale;
  const void* B;
  const int32_t* slot_rank;
  const float* slot_scale;
  const float* v;
  void* y;
  uint32_t w_bytes, b_bytes, v_bytes;
  int ld_w, d_out, r_cap, ld_v, ld_y;
  int b_ch, b_n0;         // B pool channels per slot, and the slice's first channel in it
  int tn0;                // first column tile of the slice
};

struct DmaArgs {
  const void* x;
  const void* W;
  const float* w_scale;
  const float* s_x;
  const void* B;
  const int32_t* slot_rank;
  const float* slot_scale;
  const int32_t* seg;
  const float* v;
  void* y;
  float* part;
  int32_t* counters;
  uint32_t x_bytes, w_bytes, v_bytes, b_bytes;   // descriptor ranges (b: the whole B pool)
  int r_cap, ld_v, ld_y, ld_x, ld_w, T, d_in, d_out;
  int b_ch, b_n0;         // B pool channels per slot, and the first channel of these outputs
  int tiles_m, tiles_n, group_m, nk, splits, lora_split;
  int lpt_cols;           // (persistent) columns per XCD of the row-tile-weight claim order, else 0
  int n_work;             // work items: tiles x (splits + lora_split)
  int n_slices;           // > 1: the per-slice fields above come from sl[]
  SliceArgs sl[kMaxSlices];
  // in-launch shrink (n_prod > 0): the first n_prod workgroups take shrink
  // items from a claim counter; tiles help with any left when their main loop
  // ends and wait until all are done before they read v
  int n_prod;
  int32_t* ovc;           // {claimed, done, error}, cleared before the launch
  ShrinkArgs sh;
  // packed adapter steps (bf16 tiles of 128+ rows): one record of apk_rec
  // bytes per (slice, row tile), written by pack_adapter_kernel; NULL: none
  const uint8_t* apk;
  size_t apk_rec;
};

// Record of one (slice, row tile) in the packed adapter area:
//   [0, 64)     int32 n: adapter steps of 64 packed ranks (0: no live row;
//               -1: more than kApChunks chunks, the tile takes the
//               unpacked adapter phase)
//   [64, 320)   kApChunks x {uint32 B byte offset of the chunk's 8 ranks of
//               channel 0 (0xffffffff: none), uint32 ranks of the chunk
//               below the adapter's rank (1..8)}
//   [320, ...)  BM rows x kApCap bf16: packed s_g v of the row's group at its
//               chunks, zeros elsewhere
constexpr int kApChunks = 32;               // packed chunks of 8 ranks per tile, at most
constexpr int kApCap = kApChunks * 8;       // packed ranks per row
constexpr int kApHdr = 320;
inline size_t apk_rec_bytes(int bm) { return ((size_t)kApHdr + (size_t)bm * kApCap * 2 + 255) / 256 * 256; }

constexpr int kSc1 = 16;                    // cache-policy bits of a device-coherent (sc1) buffer access
constexpr long kOvlSpinLimit = 1L << 22;    // bound of a tile's wait for the in-launch shrink (seconds)

typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));

// Raw buffer descriptor (base, stride 0, range in bytes).
__device__ __forceinline__ i32x4_t rsrc(const void* p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  i32x4_t r;
  r[0] = (int32_t)(uint32_t)a;
  r[1] = (int32_t)((uint32_t)(a >> 32) & 0xffffu);
  r[2] = (int32_t)bytes;
  r[3] = kBufferWord3;
  return r;
}

// 16 bytes per lane from rs + voff + soff into lds + 16 * lane.  Issued as
// inline assembly: the compiler, which sees an LDS write it cannot bound,
// would otherwise drain every load in flight (vmcnt(0)) before each LDS
// read of the ring; the waits are placed by hand instead (vm_barrier).
// Waits the compiler inserts for its own loads stay correct: vector memory
// operations complete in issue order, so extra younger operations only make
// a count-based wait stricter.
__device__ __forceinline__ void dma16(const i32x4_t& rs, void* lds, uint32_t voff, uint32_t soff) {
  // the destination is wave-uniform; make that visible to the compiler
  const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(LDS_PTR(lds)));
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               ::"s"(m), "v"(voff), "s"(rs), "s"(soff)
               : "memory", "m0");
}

// Wait until at most N vector-memory operations of this wave are
// outstanding and all its LDS operations are done, then meet the other waves.
template <int N>
__device__ __forceinline__ void vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Wait for the ring slot of the current step: `ahead` (0 .. MAXA) later
// steps of L operations each may stay in flight.
// EXTRA: later operations of another kind (issued after this step's slab)
// that may stay in flight as well.
template <int L, int MAXA, int EXTRA = 0>
__device__ __forceinline__ void wait_step(int ahead) {
  static_assert(MAXA * L + EXTRA <= 63, "vmcnt counts at most 63 operations");
  if constexpr (MAXA >= 1) {
    if (ahead >= MAXA) { vm_barrier<MAXA * L + EXTRA>(); return; }
    wait_step<L, MAXA - 1, EXTRA>(ahead);
  } else {
    vm_barrier<EXTRA>();
  }
}

// Drain this wave's vector memory operations with a wait the compiler sees:
// afterwards it knows that none of its own loads is pending, so it places no
// conservative vmcnt(0) of its own inside the pipelined loops that follow
// (such a wait would also drain the hand-issued DMAs it does not see).
__device__ __forceinline__ void vm_drain() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0)

// Meet the other waves once this wave's LDS operations are done; vector
// memory operations may stay in flight.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Exclusive prefix sum over the NW waves of the workgroup; *total gets the sum.
template <int NW>
__device__ __forceinline__ int block_exclusive_sum(int v, int* sums, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) sums[wave] = incl;
  lds_barrier();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    if (w < wave) before += sums[w];
    all += sums[w];
  }
  *total = all;
  lds_barrier();
  return before + incl - v;
}

__device__ __forceinline__ int sw128(int row, int c) { return row * 128 + ((c ^ (row & 7)) << 4); }
__device__ __forceinline__ int sw64(int row, int c) { return row * 64 + ((c ^ ((row >> 2) & 3)) << 4); }
// 16-byte chunk c of an LDS row of RB bytes (128 or 64), XOR-swizzled so that
// the 16 rows of a fragment read spread over the LDS banks
template <int RB>
__device__ __forceinline__ int swz(int row, int c) {
  if constexpr (RB == 128) return sw128(row, c);
  else return sw64(row, c);
}
// inverse of the swizzle for the DMA: the chunk whose data lands at physical
// chunk position cl of row `row`
template <int RB>
__device__ __forceinline__ int swz_src(int row, int cl) {
  if constexpr (RB == 128) return cl ^ (row & 7);
  else return cl ^ ((row >> 2) & 3);
}

// 8 e4m3 codes -> 8 bf16, exact (e4m3 values have 4 significant bits)
__device__ __forceinline__ bf16x8_t e4m3x8_to_bf16(uint2 c) {
  const u32x4_t o = {e4m3x2_to_bf16x2<false>(c.x), e4m3x2_to_bf16x2<true>(c.x), e4m3x2_to_bf16x2<false>(c.y),
                     e4m3x2_to_bf16x2<true>(c.y)};
  return __builtin_bit_cast(bf16x8_t, o);
}

template <int BM, int BN, int MODE, int STAGES, int WGM, int WGN, bool PERSIST, int XROW = 128, bool OVL = false>
__global__ __launch_bounds__(64 * WGM * WGN) void fused_dma_kernel(DmaArgs a) {
  constexpr int NW = WGM * WGN, NT = 64 * NW;          // waves (WGM x WGN grid) and threads
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int TM = WM / 16, TN = WN / 16;
  // x bytes per row per k-step (XROW: 128, or 64 for the bf16 ring of
  // shorter, more numerous steps) and W bytes (fp8 codes: half as many)
  static_assert(XROW == 128 || (XROW == 64 && MODE == kBF16), "64-byte k-steps: bf16 only");
  constexpr int WROW = MODE == kW8A16 ? 64 : XROW;
  constexpr int KK = XROW / 64;                        // 32-wide k chunks per step (bf16, W8A16)
  constexpr int XS = BM * XROW, WSB = BN * WROW, STAGE = XS + WSB;
  constexpr int LX = XS / (1024 * NW), LW = WSB / (1024 * NW), L = LX + LW;   // DMA ops per wave per step
  constexpr int RING = STAGES * STAGE;
  constexpr int BSLICE = BN * 128;                     // one adapter step: BN channels x 64 packed ranks
  constexpr int LB = BSLICE / (1024 * NW);
  constexpr int XE = MODE == kW8A8 ? 1 : 2;            // x element bytes
  constexpr int WE = MODE == kBF16 ? 2 : 1;            // W element bytes
  static_assert(XS % (1024 * NW) == 0 && WSB % (1024 * NW) == 0 && BSLICE % (1024 * NW) == 0,
                "slabs must be whole 1 KB DMA rows per wave");
  static_assert(NT >= BM && WM % 16 == 0 && WN % 16 == 0, "one thread per tile row; 16 x 16 fragments");
  static_assert(STAGES >= 2, "the ring needs two slots");

  __shared__ __attribute__((aligned(1024))) uint8_t ring[RING];
  __shared__ int g_row0[BM], g_row1[BM], g_rank[BM], t_rowseg[BM];
  __shared__ int t_perm[BM == 64 ? 1 : BM];   // token row of each tile row (-1 past T)
  __shared__ float g_scale[BM];
  __shared__ int s_flag, s_claim, s_sums[NW];
  __shared__ int s_order[8];                  // row tiles, most adapter groups first
  __shared__ int s_lpt;                       // the weights differ: claim in that order
  __shared__ uint32_t a_boff[kApChunks];      // packed adapter steps: B offset and rank limit per chunk
  __shared__ int a_lim[kApChunks];
  // (decode tiles) fp32 v rows of the tile for the per-output adapter epilogue
  constexpr bool kRowEpi = BM == 64 && MODE == kBF16;
  __shared__ __attribute__((aligned(16))) float v_rows[kRowEpi ? BM * 16 : 4];

  // with several row fragments per wave the wave index is read into a scalar
  // register, so that the adapter phase's per-fragment tests branch on SCC
  // (measured: faster there, slower for one fragment per wave)
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = TM > 1 ? __builtin_amdgcn_readfirstlane(tid >> 6) : tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int frow = lane & 15, fk = lane >> 4;

  // ---- work items: (tile, split) -----------------------------------------
  // Item i of XCD x (x = workgroup index mod 8, the XCD the hardware gives
  // it) is x * (n / 8) + i, so that consecutive items, which share W0
  // columns, meet in one L2.  One-shot launches take item blockIdx / 8 of
  // their XCD.  Persistent launches (more tiles than CUs) run a workgroup per
  // CU that claims the next item of its XCD from a counter until none is
  // left: a CU that finishes early takes more items, where the hardware would
  // otherwise hold a ready CU idle behind a busy one.
  // In-launch shrink ("EpiLoRA" 3.1, the decode path: the down-projection
  // runs while the GEMM streams its weights, and the epilogue needs its
  // result only at the end).  Items are claimed from ovc[0]; the workgroup
  // that claims one runs it, stores v device-coherently, and counts it done
  // in ovc[1].  Every claimed item is run by a workgroup that is already
  // running, so the count reaches the total whatever the hardware schedules.
  auto ovl_items = [&](bool wait) {
    const SegPtrs SP = seg_ptrs(const_cast<int32_t*>(a.seg), a.T);
    const bool valid = SP.sum[kError] == 0 && SP.sum[kRows] == a.T;
    // every value that steers the loop below is made wave-uniform for the
    // compiler: a branch it takes for divergent would put the loop's
    // barriers under divergent control flow
    const int n_items = __builtin_amdgcn_readfirstlane(valid ? SP.sum[kNTilesSmall] * a.sh.nrb : 0);
    f32x4_t (*red)[64] = reinterpret_cast<f32x4_t (*)[64]>(ring);
    lds_barrier();                              // the ring is free (every wave is past its LDS reads)
    // one lane-0 region per iteration, at its top: count the item the
    // workgroup finished last (its v stores drained by the barrier below
    // it), then claim the next
    int counted = 1;
    for (;;) {
      if (threadIdx.x == 0) {
        if (!counted) __hip_atomic_fetch_add(&a.ovc[1], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_claim = __hip_atomic_fetch_add(&a.ovc[0], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      lds_barrier();
      const int k = __builtin_amdgcn_readfirstlane(s_claim);
      lds_barrier();
      if (k >= n_items) break;
      const int ti = k / a.sh.nrb, rb = k - ti * a.sh.nrb;
      TileWork w;
      w.p0 = __builtin_amdgcn_readfirstlane(SP.tiles_small[2 * ti]);
      w.seg = __builtin_amdgcn_readfirstlane(SP.tiles_small[2 * ti + 1]);
      w.rows = 0;
      shrink_item_body<uint16_t, 1, NW, true>(a.sh, SP, w, rb, red);
      vm_barrier<0>();                          // every wave's v stores have completed
      counted = 0;
    }
    if (wait) {
      if (threadIdx.x == 0) {
        long spins = 0;
        while (__hip_atomic_load(&a.ovc[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < n_items) {
          __builtin_amdgcn_s_sleep(1);
          if (++spins > kOvlSpinLimit) {        // never expected: report instead of hanging
            __hip_atomic_store(&a.ovc[2], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
          }
        }
      }
      lds_barrier();
    }
  };
  int bid = (int)blockIdx.x;
  if constexpr (OVL) {
    if (bid < a.n_prod) {
      ovl_items(false);
      return;
    }
    bid -= a.n_prod;                            // (n_prod is a multiple of 8: bid & 7 is still the XCD)
  }

  const int S_total = a.splits + a.lora_split;
  const int full = (a.n_work / 8) * 8, per_xcd = full / 8, xcd = blockIdx.x & 7;
  // (more tiles than CUs, at most 8 row tiles, each XCD's items whole
  // columns) every XCD takes the row tiles with the most adapter groups
  // first (persistent claims, or the one-shot grid's dispatch order): a
  // tile's adapter phase grows with its groups, and a heavy tile taken last
  // is the launch's tail.  The weight of a row tile is the number of segments
  // meeting its live rows (0 without a valid segment buffer); ties keep the
  // row order, so every workgroup computes the same permutation.  Equal
  // weights keep the column-major order below (consecutive items share W0
  // columns).
  {
    if (a.lpt_cols > 0 && tid < 64) {
      int wgt = -1;
      if (tid < a.tiles_m) {
        wgt = 0;
        if (a.seg != nullptr && a.B != nullptr) {
          const SegPtrs SP = seg_ptrs(const_cast<int32_t*>(a.seg), a.T);
          const int na = SP.sum[kError] == 0 && SP.sum[kRows] == a.T ? SP.sum[kNActive] : 0;
          const int first = tid * BM, last = min(first + BM, na) - 1;
          if (first <= last) wgt = SP.pos_seg[last] - SP.pos_seg[first] + 1;
        }
      }
      int rank = 0, differ = 0;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int wr = __shfl(wgt, r, 64);
        if (r < a.tiles_m && tid < a.tiles_m && (wr > wgt || (wr == wgt && r < tid))) ++rank;
        if (r < a.tiles_m && wr != __shfl(wgt, 0, 64)) differ = 1;
      }
      if (tid < a.tiles_m) s_order[rank] = tid;
      if (tid == 0) s_lpt = differ;
    }
    if (a.lpt_cols > 0) lds_barrier();        // the order is every wave's before any maps an item
  }
  // (persistent) a workgroup claims its next item only once it is free:
  // claiming earlier would hold an item while the adapter phase, whose
  // length varies from tile to tile, still runs
  for (int round = 0;; ++round) {
  int pid;
  if constexpr (PERSIST) {
    if (round > 0) lds_barrier();               // every wave is past the last tile's LDS reads
    if (tid == 0) s_claim = __hip_atomic_fetch_add(&a.counters[xcd], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    lds_barrier();
    const int k = __builtin_amdgcn_readfirstlane(s_claim);   // wave-uniform: the loop holds barriers
    if (k < per_xcd) pid = xcd * per_xcd + k;
    else if (k == per_xcd && full + xcd < a.n_work) pid = full + xcd;
    else break;
  } else {
    if (round > 0) break;
    pid = bid;
    if (pid < full) pid = (pid & 7) * per_xcd + (pid >> 3);
  }
  const int tile = pid / S_total, split = pid - tile * S_total;
  int tm, tn;
  if (a.lpt_cols > 0 && pid < full && s_lpt) {
    // XCD x's items are columns [x C, x C + C) of every row tile (C =
    // lpt_cols), the same set as below, claimed row tile by row tile
    const int x = pid / per_xcd, k = pid - x * per_xcd;
    tm = s_order[k / a.lpt_cols];
    tn = x * a.lpt_cols + k % a.lpt_cols;
  } else {
    const int per_group = a.group_m * a.tiles_n;
    const int g = tile / per_group, first_m = g * a.group_m;
    const int gm = min(a.tiles_m - first_m, a.group_m);
    const int in = tile - g * per_group;
    tm = first_m + in % gm;
    tn = in / gm;
  }
  int n0 = tn * BN;
  int slice_idx = 0;
  if (a.n_slices > 1) {
    // constant indices keep the slice fields in scalar registers
    SliceArgs q = a.sl[0];
#pragma unroll
    for (int s = 1; s < kMaxSlices; ++s)
      if (s < a.n_slices && tn >= a.sl[s].tn0) {
        q = a.sl[s];
        slice_idx = s;
      }
    a.W = q.W;
    a.w_scale = q.w_scale;
    a.B = q.B;
    a.slot_rank = q.slot_rank;
    a.slot_scale = q.slot_scale;
    a.v = q.v;
    a.y = q.y;
    a.w_bytes = q.w_bytes;
    a.b_bytes = q.b_bytes;
    a.b_ch = q.b_ch;
    a.b_n0 = q.b_n0;
    a.v_bytes = q.v_bytes;
    a.ld_w = q.ld_w;
    a.d_out = q.d_out;
    a.r_cap = q.r_cap;
    a.ld_v = q.ld_v;
    a.ld_y = q.ld_y;
    n0 = (tn - q.tn0) * BN;
  }
  const int m0 = tm * BM;

  // The segment buffer's summary words, the permutation entries of the
  // tile's rows and their segment ids go out as one round of loads (the
  // entries below T are readable whether or not the buffer proves valid, and
  // are used only if it does); the first slabs can move one memory latency
  // after the start instead of after a chain of dependent rounds.
  SegPtrs P;
  const bool seg_given = a.seg != nullptr;
  int s_err = 0, s_rows = 0, s_nact = 0, rowseg_ld = -1;
  // (bf16 tiles of 128+ rows) the adapter term as extra k-steps of the main
  // pipeline, from the packed record of this tile: the s v slab through the
  // x slot, B slices through the W slot
  constexpr bool kAPipe = MODE == kBF16 && BM >= 128;
  const uint8_t* arec = nullptr;
  int ap_n = 0;
  uint32_t ap_boff = 0xffffffffu, ap_lim = 0;
  int perm_q[LX];
  int oseg[kRowEpi ? TM * 4 : 1];             // (decode tiles) segment of each output row of this lane
#pragma unroll
  for (int q = 0; q < (kRowEpi ? TM * 4 : 1); ++q) oseg[q] = -1;
#pragma unroll
  for (int q = 0; q < LX; ++q) perm_q[q] = 0;
  if (seg_given) {
    P = seg_ptrs(const_cast<int32_t*>(a.seg), a.T);
    s_err = P.sum[kError];
    s_rows = P.sum[kRows];
    s_nact = P.sum[kNActive];
#pragma unroll
    for (int q = 0; q < LX; ++q) {
      const int pos = m0 + ((wave * LX + q) * 64 + lane) / 8;
      perm_q[q] = P.perm[min(pos, a.T - 1)];
    }
    if (tid < BM) rowseg_ld = P.pos_seg[min(m0 + tid, a.T - 1)];
    if constexpr (kRowEpi) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          oseg[i * 4 + e] = P.pos_seg[min(m0 + wm * WM + i * 16 + (lane >> 4) * 4 + e, a.T - 1)];
#pragma unroll
      for (int q = 0; q < TM * 4; ++q) asm volatile("" ::"v"(oseg[q]));
    }
    if constexpr (kAPipe) {
      // the packed adapter record's step count and chunk table, in the same round
      if (a.apk != nullptr) {
        arec = a.apk + (size_t)(slice_idx * a.tiles_m + tm) * a.apk_rec;
        ap_n = *reinterpret_cast<const int32_t*>(arec);
        if (tid < kApChunks) {
          ap_boff = reinterpret_cast<const uint32_t*>(arec + 64)[2 * tid];
          ap_lim = reinterpret_cast<const uint32_t*>(arec + 64)[2 * tid + 1];
        }
        asm volatile("" ::"v"(ap_boff), "v"(ap_lim));
      }
    }
#pragma unroll
    for (int q = 0; q < LX; ++q) asm volatile("" ::"v"(perm_q[q]));   // keep the round together
    asm volatile("" ::"v"(rowseg_ld), "s"(s_err), "s"(s_rows), "s"(s_nact));
  }
  const bool has_seg = seg_given && s_err == 0 && s_rows == a.T;

  // ---- base k range of this split ----------------------------------------
  int kbeg = 0, kend = 0;
  if (split < a.splits) {
    kbeg = (int)((long)split * a.nk / a.splits);
    kend = (int)((long)(split + 1) * a.nk / a.splits);
  }
  const int nsteps = kend - kbeg;

  // the adapter phase's row -> segment ids, fetched now and used after the
  // main loop
  const bool do_lora = has_seg && a.B != nullptr && (a.lora_split ? split == a.splits : true);
  // packed adapter steps of this tile (n_as > 0), or the unpacked phase after
  // the main loop (old_phase)
  int n_as = 0;
  bool old_phase = do_lora;
  if constexpr (kAPipe) {
    if (do_lora && arec != nullptr) {
      const int n = __builtin_amdgcn_readfirstlane(ap_n);
      if (n >= 0) {
        n_as = n;
        old_phase = false;
      }
    }
  }
  int n_active = 0, my_rowseg = -1;
  if (do_lora) {
    n_active = s_nact;
    if (tid < BM && m0 + tid < n_active) my_rowseg = rowseg_ld;
  }

  // (decode tiles, ranks <= 16) the per-output adapter epilogue's operands:
  // the tile's fp32 v rows go into LDS now; each output row's adapter, then
  // its rank, scale and the B rank rows of this lane's outputs are loaded
  // right after the first slabs' DMA (load_row_epi below), so that their
  // dependent round trips run beside the slabs' and land while the main loop
  // runs.  The waits of the first STAGES - 1 steps allow for them.
  bool row_epi = false;
  int ad_o[kRowEpi ? TM * 4 : 1], rk_o[kRowEpi ? TM * 4 : 1];
  float sc_o[kRowEpi ? TM * 4 : 1];
  u32x4_t bq[kRowEpi ? TM * 4 : 1][kRowEpi ? TN : 1][2];
  // vector loads load_row_epi issues (every one unconditional)
  constexpr int kEpiLoads = kRowEpi ? TM * 4 * (3 + 2 * TN) : 0;
  if constexpr (kRowEpi) {
    row_epi = do_lora && a.r_cap <= 16;
    if (row_epi && m0 < min(m0 + BM, n_active) && !OVL) {
      // raw fp32 v rows [m0, min(m0 + BM, n_active)) x r_cap (rows past it: zeros)
      const int pe = min(m0 + BM, n_active);
      const int rq = a.r_cap / 4;
      const i32x4_t vrs = rsrc(a.v, a.v_bytes);
      for (int c0 = wave * 64; c0 < BM * rq; c0 += NT) {
        const int c = c0 + lane;
        const int row = c / rq, c4 = c - row * rq;
        const uint32_t o = (m0 + row < pe) ? (uint32_t)(((m0 + row) * a.ld_v + c4 * 4) * 4) : kOOB;
        dma16(vrs, reinterpret_cast<uint8_t*>(v_rows) + c0 * 16, o, 0u);
      }
    }
  }
  auto load_row_epi = [&]() {
    // every load below is unconditional (kEpiLoads of them), from an address
    // clamped into its buffer (adapter 0, channel 0 where there is nothing
    // to read) or from an empty range, which returns zeros without touching
    // memory; what it returns is masked only where it is used
    const __amdgpu_buffer_rsrc_t adr = __builtin_amdgcn_make_buffer_rsrc(
        has_seg ? static_cast<void*>(P.seg_adapter) : nullptr, 0, has_seg ? a.T * 4 : 0, kBufferWord3);
#pragma unroll
    for (int q = 0; q < TM * 4; ++q) {
      const int r = wm * WM + (q >> 2) * 16 + (lane >> 4) * 4 + (q & 3);
      const bool live = row_epi && m0 + r < n_active && oseg[q] >= 0;
      const int ad = (int)__builtin_amdgcn_raw_buffer_load_b32(adr, max(oseg[q], 0) * 4, 0, 0);
      ad_o[q] = live ? ad : -1;
    }
    // without a pool (row_epi false) the ranges are empty
    const __amdgpu_buffer_rsrc_t rkr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int32_t*>(a.slot_rank), 0, row_epi ? 0x7fffffff : 0, kBufferWord3);
    const __amdgpu_buffer_rsrc_t scr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(a.slot_scale), 0, row_epi ? 0x7fffffff : 0, kBufferWord3);
    const __amdgpu_buffer_rsrc_t bqr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(a.B), 0, row_epi ? (int)a.b_bytes : 0, kBufferWord3);
#pragma unroll
    for (int q = 0; q < TM * 4; ++q) {
      const int ad = max(ad_o[q], 0);
      rk_o[q] = (int)__builtin_amdgcn_raw_buffer_load_b32(rkr, ad * 4, 0, 0);
      sc_o[q] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(scr, ad * 4, 0, 0));
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = n0 + wn * WN + j * 16 + (lane & 15);
        const uint32_t o = (uint32_t)(((size_t)ad * a.b_ch + a.b_n0 + (n < a.d_out ? n : 0)) * a.r_cap * 2);
        // (capacity 8: the second chunk reads the next row, or zeros past
        // the pool, and is never used)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          bq[q][j][h] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(bqr, (int)o, h * 16, 0));
      }
    }
  };

  // per-lane DMA source offsets (k-step offsets go into soffset)
  uint32_t xoff[LX], woff[LW];
#pragma unroll
  for (int q = 0; q < LX; ++q) {
    const int s = (wave * LX + q) * 64 + lane;
    const int row = s / (XROW / 16), c = swz_src<XROW>(row, s % (XROW / 16));
    const int pos = m0 + row;
    uint32_t o = kOOB;
    if (pos < a.T) o = (uint32_t)((has_seg ? perm_q[q] : pos) * a.ld_x * XE + c * 16);
    xoff[q] = o;
  }
#pragma unroll
  for (int q = 0; q < LW; ++q) {
    const int s = (wave * LW + q) * 64 + lane;
    int row, c;
    row = s / (WROW / 16);
    c = swz_src<WROW>(row, s % (WROW / 16));
    const int n = n0 + row;
    woff[q] = n < a.d_out ? (uint32_t)(n * a.ld_w * WE + c * 16) : kOOB;
  }
  // the tile's token rows for the output stage, one lane per row
  if constexpr (BM != 64) {
#pragma unroll
    for (int q = 0; q < LX; ++q) {
      const int s = (wave * LX + q) * 64 + lane;
      if (s % (XROW / 16) == 0) {
        const int row = s / (XROW / 16), pos = m0 + row;
        t_perm[row] = pos < a.T ? (has_seg ? perm_q[q] : pos) : -1;
      }
    }
  }
  const i32x4_t xrs = rsrc(a.x, a.x_bytes);
  const i32x4_t wrs = rsrc(a.W, a.w_bytes);

  // DMA operation q (0 .. L-1) of step kt into ring slot `slot`
  auto issue_part = [&](int kt, int slot, int q) {
    uint8_t* st = ring + slot * STAGE;
    if (q < LX) dma16(xrs, st + (wave * LX + q) * 1024, xoff[q], (uint32_t)kt * XROW);
    else dma16(wrs, st + XS + (wave * LW + (q - LX)) * 1024, woff[q - LX], (uint32_t)kt * WROW);
  };
  auto issue = [&](int kt, int slot) {
#pragma unroll
    for (int q = 0; q < L; ++q) issue_part(kt, slot, q);
  };
  // DMA operation q of packed adapter step p (64 packed ranks): the x slot
  // takes the record's s v columns [64p, 64p + 64) of the tile's rows, the W
  // slot the matching B ranks of the tile's channels (chunk table in LDS)
  const i32x4_t aprs = rsrc(arec, kAPipe && arec ? (uint32_t)a.apk_rec : 0u);
  const i32x4_t bprs = rsrc(a.B, kAPipe ? a.b_bytes : 0u);
  auto issue_apart = [&](int p, int slot, int q) {
    uint8_t* st = ring + slot * STAGE;
    if (q < LX) {
      const int s = (wave * LX + q) * 64 + lane;
      const int row = s / (XROW / 16), c = swz_src<XROW>(row, s % (XROW / 16));
      dma16(aprs, st + (wave * LX + q) * 1024, (uint32_t)(kApHdr + row * (kApCap * 2) + p * 128 + c * 16), 0u);
    } else {
      const int qq = q - LX;
      const int s = (wave * LW + qq) * 64 + lane;
      const int row = s / (WROW / 16), c = swz_src<WROW>(row, s % (WROW / 16));
      const uint32_t bo = a_boff[p * 8 + c];
      const int n = n0 + row;
      const uint32_t o = (bo != 0xffffffffu && n < a.d_out) ? bo + (uint32_t)n * (uint32_t)a.r_cap * 2u : kOOB;
      dma16(bprs, st + XS + (wave * LW + qq) * 1024, o, 0u);
    }
  };

  f32x4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // bf16: the next step's DMA operations go out one per row fragment between
  // the MFMA blocks (kt_next < 0: none), so that a wave never stalls on a
  // burst of vector-memory issues while its matrix core could be busy
  // DMA operations per fragment block: a 2-slot ring gives the next step's
  // loads one step to land, so they all go out before its first MFMAs
  // (measured: spreading them over the first half of the step is slower)
  constexpr int DPB = STAGES == 2 ? L : 1;
  auto compute = [&](int slot, int kt_next, int slot_next) {
    const uint8_t* As = ring + slot * STAGE;
    const uint8_t* Ws = As + XS;
    if constexpr (MODE == kW8A8) {
      i32x8_t fa[TM], fb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int row = wm * WM + i * 16 + frow;
        const u32x4_t c0 = *reinterpret_cast<const u32x4_t*>(As + sw128(row, 2 * fk));
        const u32x4_t c1 = *reinterpret_cast<const u32x4_t*>(As + sw128(row, 2 * fk + 1));
        fa[i] = i32x8_t{(int)c0[0], (int)c0[1], (int)c0[2], (int)c0[3], (int)c1[0], (int)c1[1], (int)c1[2], (int)c1[3]};
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int row = wn * WN + j * 16 + frow;
        const u32x4_t c0 = *reinterpret_cast<const u32x4_t*>(Ws + sw128(row, 2 * fk));
        const u32x4_t c1 = *reinterpret_cast<const u32x4_t*>(Ws + sw128(row, 2 * fk + 1));
        fb[j] = i32x8_t{(int)c0[0], (int)c0[1], (int)c0[2], (int)c0[3], (int)c1[0], (int)c1[1], (int)c1[2], (int)c1[3]};
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa[i], fb[j], acc[i][j], 0, 0, 0, 127, 0, 127);
    } else if constexpr (MODE == kW8A16) {
      // every LDS read of the step (both 32-wide k halves) goes out before
      // the first MFMA; without the scheduling barrier the compiler reuses
      // one A-fragment register set and waits for each read in turn
      bf16x8_t fa[2][TM];
      uint2 c8[2][TN];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const int row = wm * WM + i * 16 + frow;
          fa[kk][i] = *reinterpret_cast<const bf16x8_t*>(As + sw128(row, kk * 4 + fk));
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int row = wn * WN + j * 16 + frow;
          // 8 codes at byte kk * 32 + fk * 8 of the 64-byte row
          c8[kk][j] = *reinterpret_cast<const uint2*>(Ws + sw64(row, kk * 2 + (fk >> 1)) + (fk & 1) * 8);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        bf16x8_t fb[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j) fb[j] = e4m3x8_to_bf16(c8[kk][j]);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[kk][i], fb[j], acc[i][j], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        bf16x8_t fa[TM], fb[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const int row = wm * WM + i * 16 + frow;
          fa[i] = *reinterpret_cast<const bf16x8_t*>(As + swz<XROW>(row, kk * 4 + fk));
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int row = wn * WN + j * 16 + frow;
          fb[j] = *reinterpret_cast<const bf16x8_t*>(Ws + swz<XROW>(row, kk * 4 + fk));
        }

#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
          for (int u = 0; u < DPB; ++u) {
            const int q = (kk * TM + i) * DPB + u;
            if (kt_next >= 0 && q < L) issue_part(kt_next, slot_next, q);
          }
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
      }
#pragma unroll
      for (int q = KK * TM * DPB; q < L; ++q)
        if (kt_next >= 0) issue_part(kt_next, slot_next, q);
    }
  };

  // ---- main loop -----------------------------------------------------------
  if constexpr (kAPipe) {
    if (n_as > 0) {
      // the chunk table into LDS for the adapter steps' B offsets and masks
      if (tid < kApChunks) {
        a_boff[tid] = ap_boff;
        a_lim[tid] = (int)ap_lim;
      }
      lds_barrier();
    }
  }
#pragma unroll
  for (int p = 0; p < STAGES - 1; ++p)
    if (p < nsteps) issue(kbeg + p, p);
  // (the adapter steps continue the same slot sequence: step nsteps + p of
  // the tile is adapter step p, and the last base steps already issue the
  // first adapter steps' loads)
  const int total = nsteps + n_as;
  if constexpr (kAPipe) {
    if (n_as > 0) {
#pragma unroll
      for (int p = 0; p < STAGES - 1; ++p)
        if (p >= nsteps && p < total) {
#pragma unroll
          for (int q = 0; q < L; ++q) issue_apart(p - nsteps, p, q);
        }
    }
  }
  if constexpr (kRowEpi) load_row_epi();
  for (int t = 0; t < nsteps; ++t) {
    // (the first STAGES - 1 slabs are older than the epilogue's loads)
    if (kEpiLoads > 0 && t < STAGES - 1) wait_step<L, STAGES - 2, kEpiLoads>(min(STAGES - 2, total - 1 - t));
    else wait_step<L, STAGES - 2>(min(STAGES - 2, total - 1 - t));
    const bool more = t + STAGES - 1 < nsteps;
    if constexpr (kAPipe) {
      const int nxt = t + STAGES - 1;
      if (nxt >= nsteps && nxt < total) {
#pragma unroll
        for (int q = 0; q < L; ++q) issue_apart(nxt - nsteps, nxt % STAGES, q);
      }
    }
    if constexpr (MODE == kBF16) {
      compute(t % STAGES, more ? kbeg + t + STAGES - 1 : -1, (t + STAGES - 1) % STAGES);
    } else {
      if (more) issue(kbeg + t + STAGES - 1, (t + STAGES - 1) % STAGES);
      compute(t % STAGES, -1, 0);
    }
  }

  // ---- adapter steps (bf16 tiles of 128+ rows with a packed record) ---------
  // Their own short pipeline through the same ring, after the base steps:
  // step p multiplies the record's s v columns [64p, 64p + 64) by the matching
  // B ranks of the tile's channels on the same accumulators.  (A separate loop
  // keeps the base steps' code free of the rank masks.)
  if constexpr (kAPipe) {
    if (n_as > 0) {
      for (int p = 0; p < n_as; ++p) {
        const int t = nsteps + p;               // the tile's step (and slot) sequence continues
        wait_step<L, STAGES - 2>(min(STAGES - 2, total - 1 - t));
        if (t + STAGES - 1 < total) {
#pragma unroll
          for (int q = 0; q < L; ++q) issue_apart(p + STAGES - 1, (t + STAGES - 1) % STAGES, q);
        }
        const uint8_t* As = ring + (t % STAGES) * STAGE;
        const uint8_t* Ws = As + XS;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          bf16x8_t fa[TM], fb[TN];
#pragma unroll
          for (int i = 0; i < TM; ++i)
            fa[i] = *reinterpret_cast<const bf16x8_t*>(As + swz<XROW>(wm * WM + i * 16 + frow, kk * 4 + fk));
          // ranks of a chunk at or past its adapter's rank (pool padding)
          // never enter the product
          const int lim = a_lim[p * 8 + kk * 4 + fk];
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            u32x4_t u = *reinterpret_cast<const u32x4_t*>(Ws + swz<XROW>(wn * WN + j * 16 + frow, kk * 4 + fk));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t keep = 2 * e >= lim ? 0u : (2 * e + 1 >= lim ? 0xffffu : 0xffffffffu);
              u[e] &= keep;
            }
            fb[j] = __builtin_bit_cast(bf16x8_t, u);
          }
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
      }
    }
  }

  const int row_base = m0 + wm * WM;   // first grouped position of this wave's rows
  const int col_base = n0 + wn * WN;
  const int ocol = lane & 15, orow = (lane >> 4) * 4;

  // base scales (fp8): w_scale[n] [* s_x[row]]
  if constexpr (MODE != kBF16) {
    if (nsteps > 0) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = col_base + j * 16 + ocol;
        const float sw = n < a.d_out ? a.w_scale[n] : 0.f;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float s = sw;
            if constexpr (MODE == kW8A8) {
              const int pos = row_base + i * 16 + orow + e;
              if (pos < a.T) s *= a.s_x[has_seg ? P.perm[pos] : pos];
            }
            acc[i][j][e] *= s;
          }
        }
      }
    }
  }

  // in-launch shrink: help with the items still unclaimed, then wait for all
  // of them before any read of v
  if constexpr (OVL)
    if (do_lora) ovl_items(true);

  // ---- adapter phase, per output (decode tiles, ranks <= 16) ------------------
  // Each lane adds, to every output it holds, s_a sum_j v[row, j] B_a[n, j]
  // of its row's adapter in fp32 ("LoRAForge" 5, RowExpand: a channel's rank
  // row read whole, the rank-r dot in registers), from the operands loaded
  // before the main loop; the packed-rank MFMA steps below would take one
  // barrier-separated step per four adapter groups, and a 64-row decode tile
  // holds up to ~25 groups of rank 16.
  if constexpr (kRowEpi) {
    if (row_epi && m0 < min(m0 + BM, n_active)) {
      const int rq = a.r_cap / 4;
      if constexpr (OVL) {
        // v of this launch: device-coherent loads (the raw v rows, rows past
        // the live ones as zeros), then into LDS
        const int pe = min(m0 + BM, n_active);
        const __amdgpu_buffer_rsrc_t vr =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(a.v), 0, (int)a.v_bytes, kBufferWord3);
        for (int c = tid; c < BM * rq; c += NT) {
          const int row = c / rq, c4 = c - row * rq;
          u32x4_t val = {0, 0, 0, 0};
          if (m0 + row < pe)
            val = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                  vr, ((m0 + row) * a.ld_v + c4 * 4) * 4, 0, kSc1));
          *reinterpret_cast<u32x4_t*>(reinterpret_cast<uint8_t*>(v_rows) + c * 16) = val;
        }
      }
      vm_barrier<0>();                          // every wave's v rows and B rows have landed
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int q = i * 4 + e;
          const int r = wm * WM + i * 16 + (lane >> 4) * 4 + e;
          const int rk = ad_o[q] >= 0 ? rk_o[q] : 0;    // rows without a live adapter add nothing
          float vv[16];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            // rank padding of v and B is never read into the sum
            const f32x4_t t = c < rq ? *reinterpret_cast<const f32x4_t*>(v_rows + r * a.r_cap + 4 * c)
                                     : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < 4; ++u) vv[4 * c + u] = t[u];
          }
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            float dot = 0.f;
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
              for (int u = 0; u < 4; ++u) {
                const int k0 = 8 * h + 2 * u;
                const uint32_t b2 = bq[q][j][h][u];
                if (k0 < rk) dot = fmaf(vv[k0], bf16lo(b2), dot);
                if (k0 + 1 < rk) dot = fmaf(vv[k0 + 1], bf16hi(b2), dot);
              }
            if (rk > 0) acc[i][j][e] = fmaf(sc_o[q], dot, acc[i][j][e]);
          }
        }
    }
  }

  // ---- adapter phase -------------------------------------------------------
  // The tile's groups are laid end to end along one packed rank axis: group
  // g occupies chunks [off_g, off_g + ceil(r_g / 8)) of 8 ranks.  Packed
  // A[row, k] is s_g v[row, j] when the row belongs to the group owning chunk
  // k / 8 (j its rank index inside the group), else 0; packed B[n, k] is
  // B_g[n, j].  A x B^T over the packed axis is exactly the sum of the
  // groups' s_g v B_g^T, run as dense 64-wide MFMA steps.
  if (do_lora && !row_epi && old_phase) {
    const int pe = min(m0 + BM, n_active);
    if (m0 < pe) {
      vm_barrier<0>();                          // ring free: every wave is past its last main step
      // LDS layout of the phase: [v16: bf16 s_g v, BM x c16 chunks][chunk
      // records][half-step row ranges] | slot region: raw fp32 v during the
      // set-up, then nb B slices of BSLICE bytes
      const int c16 = a.r_cap / 8;              // 16-byte bf16 chunks per v row
      const int cap_chunks = BM * c16;          // packed chunks at most (ng <= BM, ranks <= r_cap)
      uint8_t* v16 = ring;
      uint2* crec = reinterpret_cast<uint2*>(ring + BM * a.r_cap * 2);
      uint32_t* hrange = reinterpret_cast<uint32_t*>(crec + cap_chunks);
      const int slot_off = (BM * a.r_cap * 2 + cap_chunks * 8 + (cap_chunks / 4 + 1) * 4 + 1023) & ~1023;
      uint8_t* bsl = ring + slot_off;
      const int nb = min(kLoraNBMax, (RING - slot_off) / BSLICE);   // >= 2 by the host plan

      // raw fp32 v rows [m0, pe) x r_cap -> slot region; rows at or past pe
      // read as zeros.  Logical 16-byte chunk c4 of row r sits at chunk
      // (c4 + r / vd) mod rq of the row, so that a pass over one column of 16
      // rows touches distinct LDS banks.
      const int rq = a.r_cap / 4;
      const int vd = rq >= 16 ? 1 : 16 / rq;
      const int vchunks = BM * rq;              // a multiple of 128
      const i32x4_t vrs = rsrc(a.v, a.v_bytes);
      for (int c0 = wave * 64; c0 < vchunks; c0 += NT) {
        const int c = c0 + lane;
        const int row = c / rq, phys = c - row * rq;
        const int c4 = (phys + rq - (row / vd) % rq) % rq;
        const uint32_t o = (m0 + row < pe) ? (uint32_t)(((m0 + row) * a.ld_v + c4 * 4) * 4) : kOOB;
        if constexpr (!OVL) {
          dma16(vrs, bsl + c0 * 16, o, 0u);
        } else {
          // v of this launch: a device-coherent load into registers, then LDS
          const __amdgpu_buffer_rsrc_t vr =
              __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(a.v), 0, (int)a.v_bytes, kBufferWord3);
          u32x4_t val = {0, 0, 0, 0};
          if (o != kOOB) val = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(vr, (int)o, 0, kSc1));
          *reinterpret_cast<u32x4_t*>(bsl + c * 16) = val;
        }
      }
      // group table (segments meeting the tile's live rows)
      if (tid < BM) t_rowseg[tid] = my_rowseg;
      lds_barrier();
      const int s_first = t_rowseg[0];
      const int ng = t_rowseg[pe - 1 - m0] - s_first + 1;
      int gad = 0, grk = 0, gr0 = 0, gr1 = 0;
      float gsc = 0.f;
      if (tid < ng) {
        gad = P.seg_adapter[s_first + tid];
        gr0 = max(P.seg_start[s_first + tid], m0) - m0;         // the group's rows, tile-local
        gr1 = min(P.seg_start[s_first + tid + 1], pe) - m0;
        grk = a.slot_rank[gad];
        gsc = a.slot_scale[gad];
      }
      int n_chunks;
      const int w8 = (grk + 7) / 8;
      const int off = block_exclusive_sum<NW>(w8, s_sums, &n_chunks);
      // per packed chunk: x = group | j8 << 8 | lim << 12 (lim = ranks of the
      // chunk below the group's rank, 1..8), y = byte offset of the chunk's 8
      // ranks of channel 0 of B_g; per group its rank and scale for the v tile
      if (tid < ng) {
        g_row0[tid] = gr0;
        g_row1[tid] = gr1;
        g_rank[tid] = grk;
        g_scale[tid] = gsc;
        for (int j = 0; j < w8; ++j) {
          const uint32_t lim = (uint32_t)min(8, grk - 8 * j);
          crec[off + j] = make_uint2((uint32_t)tid | ((uint32_t)j << 8) | (lim << 12),
                                     (uint32_t)(((size_t)gad * a.b_ch + a.b_n0) * a.r_cap * 2 + j * 16));
        }
      }
      vm_drain();                               // the raw v rows have landed
      lds_barrier();
      // v16[row] = bf16(s_g v[row, j]) for j < r_g of the row's group, else 0;
      // chunk j8 of row r at (j8 + r / vd16) mod c16
      const int vd16 = c16 >= 16 ? 1 : 16 / c16;
      const float* V32 = reinterpret_cast<const float*>(bsl);
      for (int u = tid; u < BM * c16; u += NT) {
        const int r = u / c16, j8 = u - r * c16;
        const int sg = t_rowseg[r];
        u32x4_t o = {0, 0, 0, 0};
        if (sg >= 0) {
          const int g = sg - s_first;
          const int lim = g_rank[g] - 8 * j8;
          if (lim > 0) {
            const float sc = g_scale[g];
            const int p0 = (2 * j8 + (r / vd) % rq) % rq, p1 = (2 * j8 + 1 + (r / vd) % rq) % rq;
            const f32x4_t a0 = *reinterpret_cast<const f32x4_t*>(V32 + r * a.r_cap + p0 * 4);
            const f32x4_t a1 = *reinterpret_cast<const f32x4_t*>(V32 + r * a.r_cap + p1 * 4);
            float w[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              w[e] = e < lim ? sc * a0[e] : 0.f;
              w[4 + e] = 4 + e < lim ? sc * a1[e] : 0.f;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(w[2 * e], w[2 * e + 1]);
          }
        }
        *reinterpret_cast<u32x4_t*>(v16 + (r * c16 + (j8 + r / vd16) % c16) * 16) = o;
      }
      const int nhalf = (n_chunks + 3) / 4;
      for (int h = tid; h < nhalf; h += NT) {
        const int lo = (int)(crec[4 * h].x & 0xff), hi = (int)(crec[min(4 * h + 3, n_chunks - 1)].x & 0xff);
        hrange[h] = (uint32_t)g_row0[lo] | ((uint32_t)g_row1[hi] << 16);
      }
      // this lane's rows: group, v16 row offset and chunk rotation, per fragment
      int rg[TM], vro[TM], vsh[TM];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = wm * WM + i * 16 + frow;
        const int sg = t_rowseg[r];
        rg[i] = sg < 0 ? -1 : sg - s_first;
        vro[i] = r * c16;
        vsh[i] = (r / vd16) % c16;
      }
      lds_barrier();                            // v16, ranges ready; the slot region is free
      const int nls = (n_chunks + 7) / 8;
      const i32x4_t brs = rsrc(a.B, a.b_bytes);
      const uint32_t nrow_bytes = (uint32_t)a.r_cap * 2;

      auto issue_b = [&](int t, int slot) {
        uint8_t* dst = bsl + slot * BSLICE;
#pragma unroll
        for (int q = 0; q < LB; ++q) {
          const int s = (wave * LB + q) * 64 + lane;
          const int n = s >> 3, c = (s & 7) ^ (n & 7);
          const int kc = t * 8 + c;
          uint32_t o = kOOB;
          if (kc < n_chunks && n0 + n < a.d_out) o = crec[kc].y + (uint32_t)(n0 + n) * nrow_bytes;
          dma16(brs, dst + (wave * LB + q) * 1024, o, 0u);
        }
      };

      int slot = 0, fill = 0;
      for (int t = 0; t < nb - 1 && t < nls; ++t) {
        issue_b(t, fill);
        fill = fill + 1 == nb ? 0 : fill + 1;
      }
      for (int t = 0; t < nls; ++t) {
        wait_step<LB, kLoraNBMax - 2>(min(nb - 2, nls - 1 - t));
        if (t + nb - 1 < nls) {
          issue_b(t + nb - 1, fill);
          fill = fill + 1 == nb ? 0 : fill + 1;
        }
        const uint8_t* Bs = bsl + slot * BSLICE;
        slot = slot + 1 == nb ? 0 : slot + 1;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const int h = 2 * t + kk;
          if (h >= nhalf) break;
          // the groups of this half step are consecutive, so their rows are
          // one range [r_lo, r_hi); fragments outside it multiply zeros
          // (wave-uniform: with several fragments per wave kept in a scalar
          // register, so that the fragment skips below are scalar branches)
          const uint32_t hr = TM > 1 ? __builtin_amdgcn_readfirstlane(hrange[h]) : hrange[h];
          const int r_lo = (int)(hr & 0xffff), r_hi = (int)(hr >> 16);
          // a wave of several fragments none of whose rows the half step's
          // groups cover has nothing to add: it skips the chunk records and B
          // fragments as well (one fragment per wave: the test below is the same)
          if constexpr (TM > 1)
            if (wm * WM + WM <= r_lo || wm * WM >= r_hi) continue;
          const int kc = 4 * h + fk;            // this lane's packed chunk
          const uint32_t rx = kc < n_chunks ? crec[kc].x : 0u;
          const int g = kc < n_chunks ? (int)(rx & 0xff) : -2;
          const int j8 = (int)((rx >> 8) & 15), lim = (int)((rx >> 12) & 15);
          bf16x8_t fb[TN];
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const int row = wn * WN + j * 16 + frow;
            u32x4_t u = *reinterpret_cast<const u32x4_t*>(Bs + sw128(row, kk * 4 + fk));
            if (lim < 8) {                      // rank padding inside the chunk, or no chunk
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                if (2 * e >= lim) u[e] = 0;
                else if (2 * e + 1 >= lim) u[e] &= 0xffffu;
              }
            }
            fb[j] = __builtin_bit_cast(bf16x8_t, u);
          }
#pragma unroll
          for (int i = 0; i < TM; ++i) {
            const int f0 = wm * WM + i * 16;
            if (f0 + 16 <= r_lo || f0 >= r_hi) continue;
            int cj = j8 + vsh[i];
            if (cj >= c16) cj -= c16;
            u32x4_t ua = *reinterpret_cast<const u32x4_t*>(v16 + (vro[i] + cj) * 16);
            if (rg[i] != g) ua = u32x4_t{0, 0, 0, 0};
            const bf16x8_t fa = __builtin_bit_cast(bf16x8_t, ua);
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fb[j], acc[i][j], 0, 0, 0);
          }
        }
      }
    }
  }

  // ---- output ----------------------------------------------------------------
  uint16_t* __restrict__ Y = static_cast<uint16_t*>(a.y);
  if (S_total > 1) {
    // Hand-off without L2-wide fences: partial tiles are written and read
    // 16 bytes per lane with device-coherent (sc1) buffer accesses, which
    // are never left dirty in or read stale from an XCD's L2; every wave
    // drains its stores (vmcnt(0)) before the barrier that precedes the
    // counter increment, and the reads are issued only after the increment
    // that found all other partials counted.
    const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(a.part, 0, 0x7fffffff, kBufferWord3);
    const uint32_t wave_off = (uint32_t)(wave * TM * TN * 256) * 4u;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        __builtin_amdgcn_raw_buffer_store_b128(
            acc[i][j], prs, wave_off + (uint32_t)(((i * TN + j) * 64 + lane) * 16),
            (int)(((uint32_t)(tile * S_total + split) * (BM * BN)) * 4u), kSc1);
    vm_barrier<0>();
    if (tid == 0)
      s_flag = __hip_atomic_fetch_add(&a.counters[tile], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == S_total - 1;
    vm_barrier<0>();
    if (!s_flag) return;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < S_total; ++s) {
      const int soff = (int)(((uint32_t)(tile * S_total + s) * (BM * BN)) * 4u);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] += __builtin_amdgcn_raw_buffer_load_b128(
              prs, wave_off + (uint32_t)(((i * TN + j) * 64 + lane) * 16), soff, kSc1);
    }
    if (tid == 0) __hip_atomic_store(&a.counters[tile], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // 128- and 256-row tiles go through LDS: each wave writes its bf16 outputs
  // into a private region of the ring (free now), then stores whole 16-byte
  // row chunks, 16 lanes per row of the wave's columns, instead of 2 bytes
  // per lane and instruction.  Chunk c of row r sits at c ^ (2 ((r >> 2) mod
  // 4)) (within the row), so that the 4 rows of one fragment write land on
  // distinct LDS banks.  (64-row decode tiles store directly: a handful of
  // stores per lane, and no barrier behind the slowest wave's epilogue.)
  if constexpr (BM == 64) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int pos = row_base + i * 16 + orow + e;
        if (pos >= a.T) continue;
        const int row = has_seg ? P.perm[pos] : pos;
        uint16_t* yr = Y + (size_t)row * a.ld_y;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int n = col_base + j * 16 + ocol;
          if (n < a.d_out) yr[n] = f32_to_bf16(acc[i][j][e]);
        }
      }
    }
  } else {
  static_assert(BM * BN * 2 <= RING, "the bf16 output tile fits the ring");
  lds_barrier();                                // every wave is past its last ring read
  {
    constexpr int RB = WN * 2, NCH = WN / 8;    // bytes and 16-byte chunks per row of the wave
    static_assert((WM * NCH) % 64 == 0, "whole store rounds per wave");
    uint8_t* ob = ring + wave * (WM * RB);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = i * 16 + orow + e;
        const int key = (2 * ((r >> 2) & 3)) & (NCH - 1);
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int c = j * 16 + ocol;
          *reinterpret_cast<uint16_t*>(ob + r * RB + (((c >> 3) ^ key) << 4) + (c & 7) * 2) =
              f32_to_bf16(acc[i][j][e]);
        }
      }
#pragma unroll
    for (int t = 0; t < WM * NCH / 64; ++t) {
      const int ch = t * 64 + lane;
      const int r = ch / NCH, c = ch % NCH;
      const int key = (2 * ((r >> 2) & 3)) & (NCH - 1);
      const u32x4_t val = *reinterpret_cast<const u32x4_t*>(ob + r * RB + ((c ^ key) << 4));
      const int trow = t_perm[wm * WM + r];
      const int n = col_base + c * 8;
      if (trow >= 0 && n < a.d_out) st128(Y + (size_t)trow * a.ld_y + n, val);
    }
  }
  }
  }  // work items
}

__global__ void zero_words_kernel(int32_t* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

// Packed adapter records for the pipelined adapter steps (workgroups of 256
// threads, 8 rows of a row tile each; see below).  The tile's adapter groups (the segments
// meeting its live rows) are laid end to end on one packed rank axis, each
// padded to whole chunks of 8 ranks; a row's packed s v holds s_g v[row, j]
// at chunk off_g + j / 8 of its own group and zeros elsewhere, so that the
// dense product of the packed s v tile and the packed B slices over that axis
// is exactly the sum over groups of s_g v_g B_g^T for the tile's rows.
struct PackSlice {
  const float* v;
  const int32_t* slot_rank;
  const float* slot_scale;
  int ld_v, r_cap, b_ch, b_n0;
};
struct PackArgs {
  const int32_t* seg;
  uint8_t* apk;
  size_t rec;
  int T, tiles_m;
  PackSlice sl[kMaxSlices];
};

constexpr int kPackRows = 256 / kApChunks;   // rows of a tile per pack workgroup (one thread per chunk)

// Workgroup (blockIdx.x, slice blockIdx.y) packs rows [r0, r0 + kPackRows) of
// row tile r0 / BM: every workgroup of a tile rebuilds the tile's group table
// (a few loads), the first one also writes the header and chunk table, and
// each thread then writes one 16-byte chunk of one row, so that all of a
// row's v loads and chunk stores are in flight at once.
__global__ __launch_bounds__(256) void pack_adapter_kernel(PackArgs a, int BM) {
  __shared__ int g_ad[kApChunks], g_rk[kApChunks], g_off[kApChunks], g_w8[kApChunks];
  __shared__ float g_sc[kApChunks];
  __shared__ int s_nchunks;
  const int si = blockIdx.y, tid = threadIdx.x;
  const int per_tile = BM / kPackRows;
  const int tm = blockIdx.x / per_tile, r0 = (blockIdx.x - tm * per_tile) * kPackRows;
  const PackSlice S = a.sl[si];
  uint8_t* rec = a.apk + (size_t)(si * a.tiles_m + tm) * a.rec;
  int32_t* hdr = reinterpret_cast<int32_t*>(rec);
  uint32_t* tab = reinterpret_cast<uint32_t*>(rec + 64);
  u32x4_t* vpk = reinterpret_cast<u32x4_t*>(rec + kApHdr);
  const SegPtrs P = seg_ptrs(const_cast<int32_t*>(a.seg), a.T);
  const bool valid = P.sum[kError] == 0 && P.sum[kRows] == a.T;
  const int n_active = valid ? P.sum[kNActive] : 0;
  const int m0 = tm * BM, pe = min(m0 + BM, n_active);
  const bool lead = r0 == 0;                    // this workgroup writes the header and table
  if (m0 >= pe) {                               // no live row in the tile
    if (lead && tid == 0) hdr[0] = 0;
    return;
  }
  const int s_first = P.pos_seg[m0], ng = P.pos_seg[pe - 1] - s_first + 1;
  if (ng > kApChunks) {                         // more groups than chunks: the unpacked phase
    if (lead && tid == 0) hdr[0] = -1;
    return;
  }
  if (tid < ng) {
    const int ad = P.seg_adapter[s_first + tid];
    const int rk = S.slot_rank[ad];
    g_ad[tid] = ad;
    g_rk[tid] = rk;
    g_sc[tid] = S.slot_scale[ad];
    g_w8[tid] = (rk + 7) / 8;
  }
  __syncthreads();
  if (tid == 0) {
    int off = 0;
    for (int g = 0; g < ng; ++g) {
      g_off[g] = off;
      off += g_w8[g];
    }
    s_nchunks = off;
  }
  __syncthreads();
  const int n_chunks = s_nchunks;
  if (n_chunks > kApChunks) {
    if (lead && tid == 0) hdr[0] = -1;
    return;
  }
  const int n_steps = (n_chunks + 7) / 8;
  if (lead) {
    if (tid == 0) hdr[0] = n_steps;
    if (tid < kApChunks) {
      uint32_t boff = 0xffffffffu, lim = 0;
      if (tid < n_chunks) {
        int g = 0;
        while (g + 1 < ng && g_off[g + 1] <= tid) ++g;
        const int j8 = tid - g_off[g];
        boff = (uint32_t)((((size_t)g_ad[g] * S.b_ch + S.b_n0) * S.r_cap + 8 * j8) * 2);
        lim = (uint32_t)min(8, g_rk[g] - 8 * j8);
      }
      tab[2 * tid] = boff;
      tab[2 * tid + 1] = lim;
    }
  }
  // chunk c of row r: the row's group's s v (fp32, scaled, rounded to bf16)
  // at its chunks, zeros elsewhere and for rows past the live ones
  const int r = r0 + tid / kApChunks, c = tid % kApChunks;
  if (c >= n_steps * 8) return;
  const int g = m0 + r < pe ? P.pos_seg[m0 + r] - s_first : -1;
  u32x4_t o = {0, 0, 0, 0};
  if (g >= 0 && c >= g_off[g] && c < g_off[g] + g_w8[g]) {
    const int j8 = c - g_off[g];
    const int lim = min(8, g_rk[g] - 8 * j8);
    const float sc = g_sc[g];
    const float* vr = S.v + (size_t)(m0 + r) * S.ld_v + 8 * j8;
    float w[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = e < lim ? sc * vr[e] : 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(w[2 * e], w[2 * e + 1]);
  }
  vpk[(size_t)r * (kApCap / 8) + c] = o;
}

// CUs of the current device, 256 if the
// query fails
int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n <= 0)
    return kPersistMinTiles;
  return n;
}

// Workgroups of a kernel that one CU holds at once (registers and LDS), 1
// if the query fails.
template <typename K>
int resident_per_cu(K kernel, int threads) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0) != hipSuccess || n <= 0) return 1;
  return n;
}

template <int BM, int BN, int MODE, int STAGES, int WGM, int WGN, bool PERSIST = false, int XROW = 128,
          bool OVL = false>
hipError_t launch_cfg(DmaArgs a, const FusedPlan& pl, hipStream_t st) {
  const int S_total = a.splits + a.lora_split;
  // counters (split hand-off or persistent claims), then the in-launch
  // shrink's, contiguous: one clearing kernel for all
  const int n_counters = (int)(pl.counter_bytes / sizeof(int32_t)) + (a.n_prod > 0 ? 4 : 0);
  if (n_counters > 0) {
    hipLaunchKernelGGL(zero_words_kernel, dim3(1), dim3(256), 0, st, a.counters, n_counters);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  auto kernel = fused_dma_kernel<BM, BN, MODE, STAGES, WGM, WGN, PERSIST, XROW, OVL>;
  int grid = a.n_work;
  if (PERSIST) {
    // as many persistent workgroups as the chip holds at once
    static const int per_cu = resident_per_cu(kernel, 64 * WGM * WGN);
    grid = std::min(a.n_work, device_cus() * per_cu);
  }
  if constexpr (OVL) grid += a.n_prod;         // shrink producers at the head of the grid
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(64 * WGM * WGN), 0, st, a);
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_mode(const DmaArgs& a, const FusedPlan& pl, hipStream_t st) {
  if constexpr (MODE == kBF16)
    if (pl.bm == 256 && pl.bn == 256)
      return pl.xrow == 64 ? launch_cfg<256, 256, MODE, 4, 4, 2, false, 64>(a, pl, st)
                           : launch_cfg<256, 256, MODE, 2, 4, 2>(a, pl, st);
  if constexpr (MODE != kW8A16)
    if (pl.bm == 256) return launch_cfg<256, 128, MODE, 3, 4, 2>(a, pl, st);
  // 8 waves (two per SIMD) hide LDS and barrier latency; the wave grids are
  // the measured best per tile (the 64 x 64 W8A16 slab is too small for 8).
  // W8A16 128 x 128 runs 4 waves and a 3-slot ring instead, so that two
  // workgroups share a CU: their barriers are independent, and one's LDS
  // reads and code widening overlap the other's MFMAs (measured: fp8
  // 8192 -> 28672, 512 rows, 500 -> 418 us against one 8-wave workgroup).
  // (64- and 128-row tiles: persistent above one tile per CU)
  // (the in-launch shrink: 64- and 128-row tiles of bf16 and W8A16 only)
  if constexpr (MODE == kW8A16) {
    if (pl.bm == 128) {
      if (a.n_prod > 0)
        return pl.persist ? launch_cfg<128, 128, MODE, 3, 2, 2, true, 128, true>(a, pl, st)
                          : launch_cfg<128, 128, MODE, 3, 2, 2, false, 128, true>(a, pl, st);
      return pl.persist ? launch_cfg<128, 128, MODE, 3, 2, 2, true>(a, pl, st)
                        : launch_cfg<128, 128, MODE, 3, 2, 2>(a, pl, st);
    }
    if (a.n_prod > 0)
      return pl.persist ? launch_cfg<64, 64, MODE, 4, 2, 2, true, 128, true>(a, pl, st)
                        : launch_cfg<64, 64, MODE, 4, 2, 2, false, 128, true>(a, pl, st);
    return pl.persist ? launch_cfg<64, 64, MODE, 4, 2, 2, true>(a, pl, st) : launch_cfg<64, 64, MODE, 4, 2, 2>(a, pl, st);
  } else {
    if (pl.bm == 128) {
      if constexpr (MODE == kBF16)
        if (a.n_prod > 0)
          return pl.persist ? launch_cfg<128, 128, MODE, 4, 4, 2, true, 128, true>(a, pl, st)
                            : launch_cfg<128, 128, MODE, 4, 4, 2, false, 128, true>(a, pl, st);
      return pl.persist ? launch_cfg<128, 128, MODE, 4, 4, 2, true>(a, pl, st)
                        : launch_cfg<128, 128, MODE, 4, 4, 2>(a, pl, st);
    }
    if constexpr (MODE == kBF16)
      if (a.n_prod > 0)
        return pl.persist ? launch_cfg<64, 64, MODE, 4, 4, 2, true, 128, true>(a, pl, st)
                          : launch_cfg<64, 64, MODE, 4, 4, 2, false, 128, true>(a, pl, st);
    return pl.persist ? launch_cfg<64, 64, MODE, 4, 4, 2, true>(a, pl, st) : launch_cfg<64, 64, MODE, 4, 4, 2>(a, pl, st);
  }
}

}  // namespace

namespace {
// LDS ring of one configuration, and whether the adapter phase (fp32 v rows,
// the packed chunk map and at least two B slices) fits in it.
int ring_bytes(int bm, int bn, bool w8a16, int stages, int xrow = 128) {
  return stages * (bm * xrow + bn * (w8a16 ? xrow / 2 : xrow));
}
bool lora_fits(int bm, int bn, bool w8a16, int stages, int r_cap, int xrow = 128) {
  if (r_cap <= 0) return true;
  const int cap_chunks = bm * r_cap / 8;
  const int used = (bm * r_cap * 2 + cap_chunks * 8 + (cap_chunks / 4 + 1) * 4 + 1023) & ~1023;
  const int avail = ring_bytes(bm, bn, w8a16, stages, xrow) - used;
  return avail >= 2 * bn * 128 && avail >= bm * r_cap * 4;   // two B slices; the raw v rows
}
}  // namespace

int fused_device_cus() { return device_cus(); }

size_t fused_apk_bound(int T, int n_slices) {
  size_t b = 0;
  for (int bm : {128, 256}) b = std::max(b, (size_t)n_slices * ((T + bm - 1) / bm) * apk_rec_bytes(bm));
  return b;
}

// [partials][counters][in-launch shrink counters][packed adapter records (256-byte aligned)]
size_t fused_dma_apk_offset(const FusedPlan& pl) {
  return (pl.part_bytes + pl.counter_bytes + pl.ovl_bytes + 255) / 256 * 256;
}
size_t fused_dma_ws_bytes(const FusedPlan& pl) {
  return pl.apk_bytes ? fused_dma_apk_offset(pl) + pl.apk_bytes : pl.part_bytes + pl.counter_bytes + pl.ovl_bytes;
}

bool fused_ovl_supported(const FusedPlan& pl, int base_dtype, int flags) {
  return (flags & LORA_FLAG_SHRINK_IN_LAUNCH) && pl.dma && pl.bm <= 128 && pl.splits == 1 && pl.lora_split == 0 &&
         (base_dtype == LORA_BF16 || (base_dtype == LORA_FP8_E4M3 && !(flags & LORA_FLAG_ACT_QUANT_E4M3)));
}

FusedPlan plan_fused(int T, int d_in, int d_out, int base_dtype, int flags, int r_cap) {
  FusedPlan pl{};
  pl.dma = false;
  if (T <= 0 || d_out <= 0 || d_in <= 0) return pl;
  if (base_dtype != LORA_BF16 && base_dtype != LORA_FP8_E4M3) return pl;
  const bool w8a8 = base_dtype == LORA_FP8_E4M3 && (flags & LORA_FLAG_ACT_QUANT_E4M3);
  const bool w8a16 = base_dtype == LORA_FP8_E4M3 && !w8a8;
  const int kb = w8a8 ? 128 : 64;
  if (d_in % kb) return pl;
  // the largest tile that still gives every CU a tile (>= 256 tiles), else
  // 64 x 64; 256-row tiles are not built for the widened-fp8 mode
  // (256 x 256 needs two full rounds of the chip to beat 256 x 128's balance)
  // (bf16 256 x 256: xrow = 64 would be a 4-slot ring of 64-byte k-steps)
  struct Cfg { int bm, bn, stages, min_tiles, xrow; };
  const Cfg cands[] = {{256, 256, 2, 512, 128}, {256, 128, 3, 256, 128}, {128, 128, 4, 256, 128},
                       {64, 64, 4, 0, 128}};
  auto tiles_of = [&](const Cfg& c) { return (long)((T + c.bm - 1) / c.bm) * ((d_out + c.bn - 1) / c.bn); };
  const Cfg* pick = nullptr;
  for (const Cfg& c : cands) {
    if (c.bm == 256 && w8a16) continue;
    // (W8A8 256 x 256 would need more than 256 registers per lane: the 256 x
    // 128 tile is its largest)
    if (c.bm == 256 && c.bn == 256 && w8a8) continue;
    // ring slots as launched (W8A16 128 x 128: 3, two workgroups per CU)
    const int stages = (w8a16 && c.bm == 128) ? 3 : c.stages;
    if (!lora_fits(c.bm, c.bn, w8a16, stages, r_cap, c.xrow)) continue;
    if (tiles_of(c) >= c.min_tiles) { pick = &c; break; }
  }
  // 256 x 128 against 256 x 256 when the output fills the chip with the
  // smaller tile: by rounds of one-shot tiles over the CUs, times the
  // measured cost of one tile (bf16, 4096-deep: 256 x 256 ~114 us, 256 x 128
  // ~72 us on MI355X), so that 1.5 rounds of the smaller tile do not beat a
  // part-filled round of the larger one
  if (pick && pick->bm == 256 && pick->bn == 128 && !w8a8 &&
      lora_fits(256, 256, w8a16, cands[0].stages, r_cap, cands[0].xrow)) {
    const long cus = device_cus();
    const long r256 = (tiles_of(cands[0]) + cus - 1) / cus, r128 = (tiles_of(*pick) + cus - 1) / cus;
    if (r256 * 114 < r128 * 72) pick = &cands[0];
  }
  if (!pick) return pl;
  pl.dma = true;
  pl.bm = pick->bm;
  pl.bn = pick->bn;
  pl.xrow = (w8a8 || w8a16) ? 128 : pick->xrow;
  pl.nk = d_in / (w8a8 ? kb : pl.xrow / 2);
  pl.tiles_m = (T + pl.bm - 1) / pl.bm;
  pl.tiles_n = (d_out + pl.bn - 1) / pl.bn;
  pl.tiles = pl.tiles_m * pl.tiles_n;
  // very small outputs: split k over up to 4 workgroups per tile (at least 8
  // k-steps each), plus one for the adapter phase
  pl.splits = 1;
  // (no k split with the in-launch shrink: its producers fill the chip)
  if (pl.tiles < 64 && !(flags & LORA_FLAG_SHRINK_IN_LAUNCH)) pl.splits = std::max(1, std::min(4, pl.nk / 8));
  pl.lora_split = (pl.splits > 1 && r_cap > 0) ? 1 : 0;
  const int S_total = pl.splits + pl.lora_split;
  // persistent: 64- and 128-row tiles with more tiles than CUs (measured:
  // 256-row tiles, of even cost, keep the one-shot grid)
  pl.persist = S_total == 1 && pl.bm < 256 && pl.tiles > kPersistMinTiles;
  pl.part_bytes = S_total > 1 ? (size_t)pl.tiles * S_total * pl.bm * pl.bn * sizeof(float) : 0;
  pl.counter_bytes = S_total > 1 ? (size_t)pl.tiles * sizeof(int32_t)
                                 : (pl.persist ? kPersistCounters * sizeof(int32_t) : 0);
  pl.ovl_bytes = fused_ovl_supported(pl, base_dtype, flags) && r_cap > 0 ? 64 : 0;
  // the adapter term as pipelined steps: bf16 tiles of 128+ rows, one
  // workgroup per tile, v given on entry (not computed in the launch)
  pl.apipe = r_cap > 0 && base_dtype == LORA_BF16 && pl.bm >= 128 && S_total == 1 &&
             !(flags & LORA_FLAG_SHRINK_IN_LAUNCH);
  pl.apk_bytes = pl.apipe ? (size_t)pl.tiles_m * apk_rec_bytes(pl.bm) : 0;
  return pl;
}

size_t fused_quant_bytes(int T, int d_in, int flags, int base_dtype) {
  if (!(flags & LORA_FLAG_ACT_QUANT_E4M3) || base_dtype != LORA_FP8_E4M3 || T <= 0 || d_in <= 0) return 0;
  const size_t ld_q = (size_t)(d_in + 15) / 16 * 16;
  return ((size_t)T * ld_q + (size_t)T * sizeof(float) + 255) / 256 * 256;
}

size_t fused_workspace_bytes(int T, int d_in, int d_out, int base_dtype, int flags, int r_cap) {
  const FusedPlan pl = plan_fused(T, d_in, d_out, base_dtype, flags, r_cap);
  return fused_quant_bytes(T, d_in, flags, base_dtype) + (pl.dma ? fused_dma_ws_bytes(pl) : 0);
}

bool fused_dma_fits(const FusedPlan& pl, int T, int ld_x, int d_out, int ld_w, int base_dtype, int flags,
                    const lora_pool_t* pool) {
  if (!pl.dma) return false;
  const bool w8a8 = base_dtype == LORA_FP8_E4M3 && (flags & LORA_FLAG_ACT_QUANT_E4M3);
  const long lim = 0x7fffffffL;
  const long xb = (long)T * ld_x * (w8a8 ? 1 : 2);
  const long wb = (long)d_out * ld_w * (base_dtype == LORA_BF16 ? 2 : 1);
  if (xb > lim || wb > lim) return false;
  if (pool && (long)pool->n_slots * pool->d_out * pool->r_cap * 2 > lim) return false;
  if (pool && pool->n_slots > 65535) return false;   // slot ids travel in 16 bits of the chunk records
  return true;
}

FusedPlan plan_fused_slices(int T, int d_in, const FusedSlice* sl, int n, int base_dtype, int flags) {
  int total = 0, r_cap = 0;
  for (int s = 0; s < n; ++s) {
    total += sl[s].d_out;
    if (sl[s].pool) r_cap = std::max(r_cap, sl[s].pool->r_cap);
  }
  FusedPlan pl = plan_fused(T, d_in, total, base_dtype, flags, r_cap);
  if (n > 1 && pl.dma) {
    // column tiles per slice; one launch only without a k split
    int tn = 0;
    for (int s = 0; s < n; ++s) tn += (sl[s].d_out + pl.bn - 1) / pl.bn;
    pl.tiles_n = tn;
    pl.tiles = pl.tiles_m * tn;
    if (pl.splits > 1 || n > kMaxSlices) pl.dma = false;
    pl.persist = pl.splits == 1 && pl.lora_split == 0 && pl.bm < 256 && pl.tiles > kPersistMinTiles;
    pl.counter_bytes = pl.persist ? kPersistCounters * sizeof(int32_t) : 0;
    pl.apk_bytes *= n;
  }
  return pl;
}

hipError_t launch_fused_dma_slices(const FusedPlan& pl, const FusedSlice* sl, int n, const int32_t* seg, int T,
                                   const void* x, int ld_x, const float* s_x, int d_in, int flags, void* part_ws,
                                   hipStream_t st, const OverlapShrink* ovl) {
  const lora_base_t& base = sl[0].base;
  const bool w8a8 = base.dtype == LORA_FP8_E4M3 && (flags & LORA_FLAG_ACT_QUANT_E4M3);
  const int wel = base.dtype == LORA_BF16 ? 2 : 1;
  auto fill = [&](SliceArgs& q, const FusedSlice& f) {
    // a slice that starts at column col0 of its projection: base rows, scales
    // and output columns from there, pool rows from channel col0 on
    q.W = static_cast<const uint8_t*>(f.base.W) + (size_t)f.col0 * f.base.ld_w * wel;
    q.w_scale = f.base.w_scale ? f.base.w_scale + f.col0 : nullptr;
    q.B = f.pool ? f.pool->B : nullptr;
    q.slot_rank = f.pool ? f.pool->slot_rank : nullptr;
    q.slot_scale = f.pool ? f.pool->slot_scale : nullptr;
    q.v = f.v;
    q.y = static_cast<uint16_t*>(f.y) + f.col0;
    q.b_ch = f.pool ? f.pool->d_out : 0;
    q.b_n0 = f.col0;
    q.w_bytes = (uint32_t)((long)f.d_out * f.base.ld_w * wel);
    q.b_bytes = f.pool ? (uint32_t)((long)f.pool->n_slots * f.pool->d_out * f.pool->r_cap * 2) : 0;
    q.v_bytes = f.pool ? (uint32_t)((long)T * f.ld_v * 4) : 0;
    q.ld_w = f.base.ld_w;
    q.d_out = f.d_out;
    q.r_cap = f.pool ? f.pool->r_cap : 0;
    q.ld_v = f.ld_v;
    q.ld_y = f.ld_y;
    q.tn0 = 0;
  };
  DmaArgs a;
  SliceArgs q0;
  fill(q0, sl[0]);
  a.x = x;
  a.W = q0.W;
  a.w_scale = q0.w_scale;
  a.s_x = s_x;
  a.B = q0.B;
  a.slot_rank = q0.slot_rank;
  a.slot_scale = q0.slot_scale;
  a.seg = seg;
  a.v = q0.v;
  a.y = q0.y;
  a.part = static_cast<float*>(part_ws);
  a.counters = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(part_ws) + pl.part_bytes);
  a.x_bytes = (uint32_t)((long)T * ld_x * (w8a8 ? 1 : 2));
  a.w_bytes = q0.w_bytes;
  a.b_bytes = q0.b_bytes;
  a.b_ch = q0.b_ch;
  a.b_n0 = q0.b_n0;
  a.v_bytes = q0.v_bytes;
  a.r_cap = q0.r_cap;
  a.ld_v = q0.ld_v;
  a.ld_y = q0.ld_y;
  a.ld_x = ld_x;
  a.ld_w = q0.ld_w;
  a.T = T;
  a.d_in = d_in;
  a.d_out = q0.d_out;
  a.tiles_m = pl.tiles_m;
  a.tiles_n = pl.tiles_n;
  a.group_m = std::min(pl.tiles_m, 8);
  a.nk = pl.nk;
  a.splits = pl.splits;
  a.lora_split = sl[0].pool ? pl.lora_split : 0;
  a.n_work = pl.tiles * (a.splits + a.lora_split);
  // heaviest row tiles first (launches of more tiles than CUs whose XCD
  // ranges are whole columns of one row-tile group: at most 8 row tiles,
  // per-XCD item count a multiple of them)
  a.lpt_cols = 0;
  if (a.splits + a.lora_split == 1 && a.n_work > fused_device_cus() && pl.tiles_m <= 8 && a.n_work % 8 == 0 &&
      (a.n_work / 8) % pl.tiles_m == 0)
    a.lpt_cols = a.n_work / 8 / pl.tiles_m;
  a.n_slices = n > 1 ? n : 1;
  a.apk = nullptr;
  a.apk_rec = 0;
  // Packed adapter steps pay for their pack launch when tiles hold few groups:
  // batches of at least 32 rows per usable slot on average (prefill); batches
  // of mostly one- or two-row groups (decode, mixed layers) keep the unpacked
  // phase, whose waves skip the fragments a group does not meet.
  if (pl.apipe && sl[0].pool && (long)T >= 32L * std::min(T, sl[0].pool->n_slots)) {
    PackArgs pk;
    pk.seg = seg;
    pk.apk = static_cast<uint8_t*>(part_ws) + fused_dma_apk_offset(pl);
    pk.rec = apk_rec_bytes(pl.bm);
    pk.T = T;
    pk.tiles_m = pl.tiles_m;
    for (int s = 0; s < n; ++s) {
      const lora_pool_t& pool = *sl[s].pool;
      pk.sl[s] = PackSlice{sl[s].v, pool.slot_rank, pool.slot_scale, sl[s].ld_v, pool.r_cap, pool.d_out, sl[s].col0};
    }
    hipLaunchKernelGGL(pack_adapter_kernel, dim3(pl.tiles_m * (pl.bm / kPackRows), n), dim3(256), 0, st, pk, pl.bm);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    a.apk = pk.apk;
    a.apk_rec = pk.rec;
  }
  a.n_prod = 0;
  a.ovc = a.counters + pl.counter_bytes / sizeof(int32_t);
  if (ovl && sl[0].pool && n == 1 && fused_ovl_supported(pl, base.dtype, flags)) {
    // the in-launch shrink over the pool of the (single) slice
    const lora_pool_t& pool = *sl[0].pool;
    ShrinkArgs& sh = a.sh;
    sh.x = ovl->x;
    sh.A = pool.A;
    sh.slot_rank = pool.slot_rank;
    sh.seg = const_cast<int32_t*>(seg);
    sh.v = const_cast<float*>(sl[0].v);
    sh.ld_x = ovl->ld_x;
    sh.r_cap = pool.r_cap;
    sh.d_in = pool.d_in;
    sh.T = T;
    sh.ld_v = sl[0].ld_v;
    sh.mode = LORA_LAUNCH_PERSISTENT;
    shrink_item_geometry(pool, T, &sh.db, &sh.nrb);
    sh.rtiles = 0;
    sh.n_items = 0;
    sh.slots = std::min(T, pool.n_slots);
    // producers: about one workgroup per 4 items of the bound, at most 64, a
    // multiple of 8 (a tile's workgroup index keeps its XCD)
    const long bound = ((long)T / LORA_TILE_SMALL + sh.slots) * sh.nrb;
    a.n_prod = (int)std::min<long>(64, std::max<long>(8, (bound / 4 + 7) / 8 * 8));
  }
  if (n > 1) {
    int tn0 = 0;
    for (int s = 0; s < n; ++s) {
      fill(a.sl[s], sl[s]);
      a.sl[s].tn0 = tn0;
      tn0 += (sl[s].d_out + pl.bn - 1) / pl.bn;
    }
  }
  if (base.dtype == LORA_BF16) return launch_mode<kBF16>(a, pl, st);
  if (w8a8) return launch_mode<kW8A8>(a, pl, st);
  return launch_mode<kW8A16>(a, pl, st);
}

hipError_t launch_fused_dma(const FusedPlan& pl, const lora_base_t& base, const lora_pool_t* pool,
                            const int32_t* seg, int T, const void* x, int ld_x, const float* s_x, const float* v,
                            int ld_v, void* y, int ld_y, int d_in, int d_out, int flags, void* part_ws,
                            hipStream_t st, const OverlapShrink* ovl) {
  const FusedSlice one{base, pool, v, ld_v, y, ld_y, d_out};
  return launch_fused_dma_slices(pl, &one, 1, seg, T, x, ld_x, s_x, d_in, flags, part_ws, st, ovl);
}

}  // namespace lora
