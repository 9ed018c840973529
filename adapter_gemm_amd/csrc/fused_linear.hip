// Fused linear: y[i, n] = epi( sum_k x[i, k] W0[n, k] ) with the adapter
// up-projection added in the epilogue ("EpiLoRA" 3.1 and Fig. 10, kernel K2:
// a GEMM over adapter-sorted rows whose epilogue, for each adapter group in
// the output tile, adds h_l B_l^T reading only the tile's slice of B_l, then
// writes the rows back in token order).
//
// gfx950 design
//  * Rows are taken in the grouped order (perm), so an output tile meets only
//    a few contiguous adapter groups; x rows are gathered through perm while
//    they are staged, and results are scattered back through perm.
//  * Main loop: 256 threads = 4 waves in a 2 x 2 grid; each k-step stages a
//    BM x 128-byte slab of x and a BN x 128-byte slab of W0 in LDS (double
//    buffered, 16-byte chunks XOR-swizzled by row), and each wave issues
//    v_mfma_f32_16x16x32_bf16 (bf16 base, or fp8 codes widened to bf16 while
//    staging: W8A16) or v_mfma_scale_f32_16x16x128_f8f6f4 (fp8 x fp8: W8A8).
//  * Epilogue: base scales (fp8: w_scale[n], W8A8 also s_x[i]); then, per
//    adapter group intersecting the wave's rows, the rank-r product
//    (s_a v) B_a^T runs on the same MFMA accumulators, with v rows of other
//    groups masked to zero.  Operand fragments come straight from global
//    memory: a lane's 8 rank values of one channel are 16 contiguous bytes of
//    B ([d_out, r_cap] per adapter), and of one row of v.
//  * Workgroups are remapped so that consecutive tiles land on the same XCD
//    (the hardware deals workgroups round-robin over the 8 XCDs), and tiles
//    are visited in groups of M tiles so each XCD's L2 holds the W0 panels it
//    streams.
#include "common.h"

#include <algorithm>
#include <vector>

namespace lora {
namespace {

constexpr int kThreads = 256;

enum FusedMode { kBF16 = 0, kW8A16 = 1, kW8A8 = 2 };

struct FusedArgs {
  const void* x;          // bf16 [T, ld_x] (kBF16, kW8A16) or e4m3 codes [T, ld_x] (kW8A8)
  const void* W;          // bf16 [d_out, ld_w] or e4m3 codes
  const float* w_scale;   // fp8 only
  const float* s_x;       // kW8A8 only, per original row
  const void* B;          // adapter pool B (bf16), or null
  const int32_t* slot_rank;
  const float* slot_scale;
  int32_t* seg;           // may be null (rows in batch order, no adapters)
  const float* v;
  void* y;
  int r_cap, ld_v, ld_y, ld_x, ld_w, T, d_in, d_out;
  int tiles_m, tiles_n, group_m;
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * 64 + ((chunk ^ (row & 7)) << 3); }

// XCD-aware, M-grouped tile order.  pid -> (tm, tn), a bijection.
__device__ __forceinline__ void tile_of(int pid, int nblk, int tiles_m, int tiles_n, int group_m, int& tm,
                                        int& tn) {
  const int full = (nblk / 8) * 8;
  int l = pid;
  if (pid < full) l = (pid & 7) * (full / 8) + (pid >> 3);
  const int per_group = group_m * tiles_n;
  const int g = l / per_group;
  const int first_m = g * group_m;
  const int gm = min(tiles_m - first_m, group_m);
  const int in = l - g * per_group;
  tm = first_m + in % gm;
  tn = in / gm;
}

// fp8 e4m3 x16 (one 16-byte chunk) -> bf16 x16 (two 16-byte chunks), exact.
__device__ __forceinline__ void e4m3x16_to_bf16(const u32x4_t& c, u32x4_t& lo, u32x4_t& hi) {
  lo = u32x4_t{e4m3x2_to_bf16x2<false>(c[0]), e4m3x2_to_bf16x2<true>(c[0]), e4m3x2_to_bf16x2<false>(c[1]),
               e4m3x2_to_bf16x2<true>(c[1])};
  hi = u32x4_t{e4m3x2_to_bf16x2<false>(c[2]), e4m3x2_to_bf16x2<true>(c[2]), e4m3x2_to_bf16x2<false>(c[3]),
               e4m3x2_to_bf16x2<true>(c[3])};
}

template <int BM, int BN, int MODE>
__global__ __launch_bounds__(kThreads) void fused_gemm_kernel(FusedArgs a) {
  constexpr int WM = BM / 2, WN = BN / 2;         // wave tile
  constexpr int TM = WM / 16, TN = WN / 16;       // 16x16 MFMA tiles per wave
  constexpr int KB = MODE == kW8A8 ? 128 : 64;    // k elements per 128-byte row slab
  constexpr int AR = BM / 32;                      // x rows staged per thread
  constexpr int WR = MODE == kW8A16 ? BN / 64 : BN / 32;   // W rows staged per thread

  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * 64];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * 64];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  int tm, tn;
  tile_of(blockIdx.x, gridDim.x, a.tiles_m, a.tiles_n, a.group_m, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  SegPtrs P;
  bool has_seg = a.seg != nullptr;
  if (has_seg) {
    P = seg_ptrs(a.seg, a.T);
    has_seg = seg_valid(P, a.T);       // unusable buffer: batch order, base only
  }

  // ---- staging assignment --------------------------------------------
  const uint8_t* arow[AR];
  {
    const int c = tid & 7, r = tid >> 3;
#pragma unroll
    for (int i = 0; i < AR; ++i) {
      const int pos = m0 + r + 32 * i;
      if (pos < a.T) {
        const int row = has_seg ? P.perm[pos] : pos;
        const size_t esz = MODE == kW8A8 ? 1 : 2;
        arow[i] = static_cast<const uint8_t*>(a.x) + ((size_t)row * a.ld_x) * esz + c * 16;
      } else {
        arow[i] = nullptr;
      }
    }
  }
  const uint8_t* wrow[WR];
  {
    if constexpr (MODE == kW8A16) {
      const int c = tid & 3, r = tid >> 2;
#pragma unroll
      for (int i = 0; i < WR; ++i) {
        const int n = n0 + r + 64 * i;
        wrow[i] = n < a.d_out ? static_cast<const uint8_t*>(a.W) + (size_t)n * a.ld_w + c * 16 : nullptr;
      }
    } else {
      const int c = tid & 7, r = tid >> 3;
      const size_t esz = MODE == kW8A8 ? 1 : 2;
#pragma unroll
      for (int i = 0; i < WR; ++i) {
        const int n = n0 + r + 32 * i;
        wrow[i] = n < a.d_out ? static_cast<const uint8_t*>(a.W) + ((size_t)n * a.ld_w) * esz + c * 16 : nullptr;
      }
    }
  }

  u32x4_t ra[AR];
  u32x4_t rw[WR];
  const u32x4_t zero4 = {0, 0, 0, 0};
  // bytes of one row per k-step: 64 bf16, 128 fp8 codes (W8A8), or 64 fp8
  // codes widened to bf16 while staging (W8A16)
  const size_t kstep_bytes_x = 128;
  const size_t kstep_bytes_w = MODE == kW8A16 ? 64 : 128;
  // element offset of this thread's chunk inside a k-step, for the d_in bound
  const int a_kofs = (tid & 7) * (MODE == kW8A8 ? 16 : 8);
  const int w_kofs = MODE == kW8A16 ? (tid & 3) * 16 : (tid & 7) * (MODE == kW8A8 ? 16 : 8);

  auto gload = [&](int kt) {
    const int k0 = kt * KB;
#pragma unroll
    for (int i = 0; i < AR; ++i)
      ra[i] = (arow[i] && k0 + a_kofs < a.d_in) ? ld128(arow[i] + (size_t)kt * kstep_bytes_x) : zero4;
#pragma unroll
    for (int i = 0; i < WR; ++i)
      rw[i] = (wrow[i] && k0 + w_kofs < a.d_in) ? ld128(wrow[i] + (size_t)kt * kstep_bytes_w) : zero4;
  };
  auto lstore = [&](int buf) {
    {
      const int c = tid & 7, r = tid >> 3;
#pragma unroll
      for (int i = 0; i < AR; ++i) *reinterpret_cast<u32x4_t*>(&As[buf][swz(r + 32 * i, c)]) = ra[i];
    }
    if constexpr (MODE == kW8A16) {
      const int c = tid & 3, r = tid >> 2;
#pragma unroll
      for (int i = 0; i < WR; ++i) {
        u32x4_t lo, hi;
        e4m3x16_to_bf16(rw[i], lo, hi);
        *reinterpret_cast<u32x4_t*>(&Bs[buf][swz(r + 64 * i, 2 * c)]) = lo;
        *reinterpret_cast<u32x4_t*>(&Bs[buf][swz(r + 64 * i, 2 * c + 1)]) = hi;
      }
    } else {
      const int c = tid & 7, r = tid >> 3;
#pragma unroll
      for (int i = 0; i < WR; ++i) *reinterpret_cast<u32x4_t*>(&Bs[buf][swz(r + 32 * i, c)]) = rw[i];
    }
  };

  f32x4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nk = (a.d_in + KB - 1) / KB;
  gload(0);
  lstore(0);
  __syncthreads();

  const int frow = lane & 15, fk = lane >> 4;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    if constexpr (MODE == kW8A8) {
      // one K=128 MFMA per fragment pair; a lane's 32 codes are chunks 2*fk, 2*fk+1
      i32x8_t fa[TM], fb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int row = wm * WM + i * 16 + frow;
        const u32x4_t c0 = *reinterpret_cast<const u32x4_t*>(&As[buf][swz(row, 2 * fk)]);
        const u32x4_t c1 = *reinterpret_cast<const u32x4_t*>(&As[buf][swz(row, 2 * fk + 1)]);
        fa[i] = i32x8_t{(int)c0[0], (int)c0[1], (int)c0[2], (int)c0[3], (int)c1[0], (int)c1[1], (int)c1[2], (int)c1[3]};
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int row = wn * WN + j * 16 + frow;
        const u32x4_t c0 = *reinterpret_cast<const u32x4_t*>(&Bs[buf][swz(row, 2 * fk)]);
        const u32x4_t c1 = *reinterpret_cast<const u32x4_t*>(&Bs[buf][swz(row, 2 * fk + 1)]);
        fb[j] = i32x8_t{(int)c0[0], (int)c0[1], (int)c0[2], (int)c0[3], (int)c1[0], (int)c1[1], (int)c1[2], (int)c1[3]};
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa[i], fb[j], acc[i][j], 0, 0, 0, 127, 0, 127);
    } else {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        bf16x8_t fa[TM], fb[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const int row = wm * WM + i * 16 + frow;
          fa[i] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(&As[buf][swz(row, kk * 4 + fk)]));
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int row = wn * WN + j * 16 + frow;
          fb[j] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(&Bs[buf][swz(row, kk * 4 + fk)]));
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
      }
    }
    if (kt + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue ---------------------------------------------------------
  const int row_base = m0 + wm * WM;          // first grouped position of this wave
  const int col_base = n0 + wn * WN;
  const int ocol = lane & 15, orow = (lane >> 4) * 4;

  if constexpr (MODE != kBF16) {
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

  if (has_seg && a.B != nullptr) {
    const uint16_t* __restrict__ Bp = static_cast<const uint16_t*>(a.B);
    const int n_active = P.sum[kNActive];
    const int pend = min(row_base + WM, n_active);
    int p = row_base;
    while (p < pend) {
      const int s = P.pos_seg[p];
      const int ad = P.seg_adapter[s];
      const int gend = min(P.seg_start[s + 1], pend);
      const int r = a.slot_rank[ad];
      const float sc = a.slot_scale[ad];
      for (int kq = 0; kq * 32 < r; ++kq) {
        const int k = kq * 32 + fk * 8;
        bf16x8_t fb[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int n = col_base + j * 16 + frow;
          u32x4_t u = zero4;
          if (n < a.d_out && k < r) {
            u = ld128(Bp + ((size_t)ad * a.d_out + n) * a.r_cap + k);
            if (k + 8 > r) {
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                if (k + 2 * e >= r) u[e] = 0;
                else if (k + 2 * e + 1 >= r) u[e] &= 0xffffu;
              }
            }
          }
          fb[j] = __builtin_bit_cast(bf16x8_t, u);
        }
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const int f0 = row_base + i * 16;
          if (f0 + 16 <= p || f0 >= gend) continue;     // no row of this group here
          const int pos = f0 + frow;
          float vv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) vv[e] = 0.f;
          if (pos >= p && pos < gend) {
            const float* vr = a.v + (size_t)pos * a.ld_v + k;
            if (k < r) {
              const u32x4_t c0 = ld128(vr);
#pragma unroll
              for (int e = 0; e < 4; ++e) vv[e] = __uint_as_float(c0[e]);
            }
            if (k + 4 < r) {
              const u32x4_t c1 = ld128(vr + 4);
#pragma unroll
              for (int e = 0; e < 4; ++e) vv[4 + e] = __uint_as_float(c1[e]);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) vv[e] = (k + e < r) ? vv[e] * sc : 0.f;
          }
          u32x4_t ua;
#pragma unroll
          for (int e = 0; e < 4; ++e) ua[e] = pack_bf16x2(vv[2 * e], vv[2 * e + 1]);
          const bf16x8_t fa = __builtin_bit_cast(bf16x8_t, ua);
#pragma unroll
          for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fb[j], acc[i][j], 0, 0, 0);
        }
      }
      p = gend;
    }
  }

  uint16_t* __restrict__ Y = static_cast<uint16_t*>(a.y);
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
}

// ---------------------------------------------------------------------------
// fp32 path (fp32 base, pool, x and y): LDS-tiled FMA GEMM, 32 x 32 tiles
// (small fp32 problems: many workgroups), 64-wide k blocks whose loads for
// the next block are in flight while the current one is multiplied; each
// thread 2 x 2 outputs; the adapter term is a per-element rank-r dot.
// ---------------------------------------------------------------------------
struct F32Args {
  const float* x;
  const float* W;
  const float* B;
  const int32_t* slot_rank;
  const float* slot_scale;
  int32_t* seg;
  const float* v;
  float* y;
  int r_cap, ld_v, ld_y, ld_x, ld_w, T, d_in, d_out, tiles_n;
};

constexpr int kF32Tile = 32;
constexpr int kF32Pre = 8;    // k blocks of 64 whose loads are in flight at once

__global__ __launch_bounds__(256) void fused_f32_kernel(F32Args a) {
  // k goes in chunks of KC = kF32Pre x 64: all of a chunk's loads go out at
  // once (a 64-wide block's FMAs take far less than one memory round trip,
  // so loading one block ahead would leave each block waiting for its own
  // loads), then the chunk is staged in LDS and multiplied in one loop
  constexpr int BM = kF32Tile, BN = kF32Tile, BK = 64, KC = kF32Pre * BK;
  __shared__ float As[KC][BM + 1];
  __shared__ float Ws[KC][BN + 1];
  const int tid = threadIdx.x;
  const int tm = blockIdx.x / a.tiles_n, tn = blockIdx.x % a.tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;
  bool has_seg = a.seg != nullptr;
  SegPtrs P;
  if (has_seg) {
    P = seg_ptrs(a.seg, a.T);
    has_seg = seg_valid(P, a.T);
  }

  // staging: row lr of the tile, 8 consecutive k of each 64-wide block
  // (d_in, ld_x, ld_w are multiples of 8 and the rows 16-byte aligned: two
  // float4 loads, all in or all out of range).  Every load goes out
  // unconditionally, from row 0 or the row's last 8 values where the tile's
  // row or k is past the operand, and such values become zeros only when
  // staged: a load under a per-lane branch, or a select right after it,
  // would be waited for at once.
  const int lr = tid >> 3, lk = (tid & 7) * 8;
  const int apos = m0 + lr;
  const float* xrow = nullptr;
  if (apos < a.T) xrow = a.x + (size_t)(has_seg ? P.perm[apos] : apos) * a.ld_x;
  const float* wrow = (n0 + lr < a.d_out) ? a.W + (size_t)(n0 + lr) * a.ld_w : nullptr;
  const float* xsrc = xrow ? xrow : a.x;
  const float* wsrc = wrow ? wrow : a.W;
  f32x4_t xa[kF32Pre][2], wa[kF32Pre][2];

  const int ty = tid >> 4, tx = tid & 15;
  float acc[2][2] = {};
  for (int c0 = 0; c0 < a.d_in; c0 += KC) {
#pragma unroll
    for (int p = 0; p < kF32Pre; ++p) {
      const int k = c0 + p * BK + lk;
      const int kc = k < a.d_in ? k : a.d_in - 8;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        xa[p][h] = *reinterpret_cast<const f32x4_t*>(xsrc + kc + 4 * h);
        wa[p][h] = *reinterpret_cast<const f32x4_t*>(wsrc + kc + 4 * h);
      }
    }
    if (c0 > 0) __syncthreads();              // every wave is done with the previous chunk
#pragma unroll
    for (int p = 0; p < kF32Pre; ++p) {
      const bool in = c0 + p * BK + lk < a.d_in;
      const bool xin = xrow && in, win = wrow && in;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          As[p * BK + lk + 4 * h + e][lr] = xin ? xa[p][h][e] : 0.f;
          Ws[p * BK + lk + 4 * h + e][lr] = win ? wa[p][h][e] : 0.f;
        }
    }
    __syncthreads();
    const int kn = min(KC, a.d_in - c0);      // a multiple of 8
#pragma unroll 8
    for (int kk = 0; kk < kn; ++kk) {
      const float a0 = As[kk][ty * 2], a1 = As[kk][ty * 2 + 1];
      const float w0 = Ws[kk][tx * 2], w1 = Ws[kk][tx * 2 + 1];
      acc[0][0] = fmaf(a0, w0, acc[0][0]);
      acc[0][1] = fmaf(a0, w1, acc[0][1]);
      acc[1][0] = fmaf(a1, w0, acc[1][0]);
      acc[1][1] = fmaf(a1, w1, acc[1][1]);
    }
  }

  // Epilogue: y[row, n] = acc + s_a sum_j v[pos, j] B_a[n, j] for live rows.
  // The loads go out one round per link of the chain (permutation and
  // segment -> adapter -> rank and scale -> v and B), for both of the
  // thread's rows at once, from indices clamped into their arrays; values of
  // rows past T or not live are never used.
  const int n_active = (has_seg && a.B) ? P.sum[kNActive] : 0;
  int pos[2], row[2], ad[2] = {0, 0}, rk[2] = {0, 0};
  bool live[2];
  float sc[2] = {0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    pos[i] = m0 + ty * 2 + i;
    live[i] = pos[i] < n_active;                // (n_active <= T; 0 without a pool or segments)
  }
  if (has_seg) {
    int sg[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int pc = min(pos[i], a.T - 1);
      row[i] = P.perm[pc];
      sg[i] = P.pos_seg[pc];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) ad[i] = P.seg_adapter[min(max(sg[i], 0), a.T - 1)];
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i) row[i] = pos[i];
  }
  if (live[0] || live[1]) {
    // (a row that is not live takes the other row's adapter: a valid slot)
    const int s0 = live[0] ? ad[0] : ad[1], s1 = live[1] ? ad[1] : ad[0];
    const int r0 = a.slot_rank[s0], r1 = a.slot_rank[s1];
    const float c0 = a.slot_scale[s0], c1 = a.slot_scale[s1];
    ad[0] = s0;
    ad[1] = s1;
    rk[0] = live[0] ? min(r0, a.r_cap) : 0;
    rk[1] = live[1] ? min(r1, a.r_cap) : 0;
    sc[0] = c0;
    sc[1] = c1;
  }
  // ranks in batches of 16: every v and B load of a batch goes out before
  // its FMAs; ranks at or past a row's rank are dropped (v may hold anything
  // there)
  float dot[2][2] = {};
  const int nbat = (max(rk[0], rk[1]) + 15) / 16;
  for (int bt = 0; bt < nbat; ++bt) {
    const int j0 = bt * 16;
    f32x4_t vv[2][4], bb[2][2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const float* vr = a.v + (size_t)min(pos[i], a.T - 1) * a.ld_v;
#pragma unroll
      for (int q = 0; q < 4; ++q) vv[i][q] = *reinterpret_cast<const f32x4_t*>(vr + min(j0 + 4 * q, a.r_cap - 4));
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = min(n0 + tx * 2 + j, a.d_out - 1);
        const float* br = a.B + ((size_t)ad[i] * a.d_out + n) * a.r_cap;
#pragma unroll
        for (int q = 0; q < 4; ++q) bb[i][j][q] = *reinterpret_cast<const f32x4_t*>(br + min(j0 + 4 * q, a.r_cap - 4));
      }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (j0 + 4 * q + e < rk[i]) dot[i][j] = fmaf(vv[i][q][e], bb[i][j][q][e], dot[i][j]);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    if (pos[i] >= a.T) continue;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + tx * 2 + j;
      if (n >= a.d_out) continue;
      a.y[(size_t)row[i] * a.ld_y + n] = rk[i] > 0 ? fmaf(sc[i], dot[i][j], acc[i][j]) : acc[i][j];
    }
  }
}

template <int BM, int BN, int MODE>
hipError_t launch_cfg(FusedArgs a, hipStream_t st) {
  a.tiles_m = (a.T + BM - 1) / BM;
  a.tiles_n = (a.d_out + BN - 1) / BN;
  a.group_m = a.tiles_m < 8 ? a.tiles_m : 8;
  const int grid = a.tiles_m * a.tiles_n;
  hipLaunchKernelGGL((fused_gemm_kernel<BM, BN, MODE>), dim3(grid), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_mode(const FusedArgs& a, hipStream_t st) {
  const long big = (long)((a.T + 127) / 128) * ((a.d_out + 127) / 128);
  if (big >= 512) return launch_cfg<128, 128, MODE>(a, st);
  return launch_cfg<64, 64, MODE>(a, st);
}

}  // namespace

hipError_t launch_fused(const lora_base_t& base, const lora_pool_t* pool, int32_t* seg, int T, const void* x,
                        int ld_x, const float* v, int ld_v, void* y, int ld_y, int d_in, int d_out, int flags,
                        void* workspace, hipStream_t st) {
  if (T == 0 || d_out == 0) return hipSuccess;
  if (base.dtype == LORA_F32) {
    F32Args a;
    a.x = static_cast<const float*>(x);
    a.W = static_cast<const float*>(base.W);
    a.B = pool ? static_cast<const float*>(pool->B) : nullptr;
    a.slot_rank = pool ? pool->slot_rank : nullptr;
    a.slot_scale = pool ? pool->slot_scale : nullptr;
    a.seg = seg;
    a.v = v;
    a.y = static_cast<float*>(y);
    a.r_cap = pool ? pool->r_cap : 0;
    a.ld_v = ld_v;
    a.ld_y = ld_y;
    a.ld_x = ld_x;
    a.ld_w = base.ld_w;
    a.T = T;
    a.d_in = d_in;
    a.d_out = d_out;
    a.tiles_n = (d_out + kF32Tile - 1) / kF32Tile;
    const int grid = ((T + kF32Tile - 1) / kF32Tile) * a.tiles_n;
    hipLaunchKernelGGL(fused_f32_kernel, dim3(grid), dim3(256), 0, st, a);
    return hipGetLastError();
  }
  FusedArgs a;
  a.x = x;
  a.W = base.W;
  a.w_scale = base.w_scale;
  a.s_x = nullptr;
  a.B = pool ? pool->B : nullptr;
  a.slot_rank = pool ? pool->slot_rank : nullptr;
  a.slot_scale = pool ? pool->slot_scale : nullptr;
  a.seg = seg;
  a.v = v;
  a.y = y;
  a.r_cap = pool ? pool->r_cap : 0;
  a.ld_v = ld_v;
  a.ld_y = ld_y;
  a.ld_x = ld_x;
  a.ld_w = base.ld_w;
  a.T = T;
  a.d_in = d_in;
  a.d_out = d_out;
  const FusedPlan pl = plan_fused(T, d_in, d_out, base.dtype, flags, pool ? pool->r_cap : 0);
  const bool w8a8 = base.dtype == LORA_FP8_E4M3 && (flags & LORA_FLAG_ACT_QUANT_E4M3);
  const size_t qbytes = fused_quant_bytes(T, d_in, flags, base.dtype);
  const void* xin = x;
  int ld_in = ld_x;
  float* s_x = nullptr;
  if (w8a8) {
    // quantise x per token into the workspace, then the fp8 x fp8 product
    uint8_t* q = static_cast<uint8_t*>(workspace);
    const int ld_q = (d_in + 15) / 16 * 16;
    s_x = reinterpret_cast<float*>(q + (size_t)T * ld_q);
    hipError_t e = launch_quantize_e4m3(x, T, d_in, ld_x, q, ld_q, s_x, st);
    if (e != hipSuccess) return e;
    xin = q;
    ld_in = ld_q;
  }
  const bool in_launch = (flags & LORA_FLAG_SHRINK_IN_LAUNCH) && pool;
  const bool dma = fused_dma_fits(pl, T, ld_in, d_out, base.ld_w, base.dtype, flags, pool);
  if (dma && in_launch && fused_ovl_supported(pl, base.dtype, flags)) {
    const OverlapShrink ovl{x, ld_x};
    return launch_fused_dma(pl, base, pool, seg, T, xin, ld_in, s_x, v, ld_v, y, ld_y, d_in, d_out, flags,
                            static_cast<uint8_t*>(workspace) + qbytes, st, &ovl);
  }
  if (in_launch) {
    // shapes the pipelined kernel does not take: the shrink as its own launch first
    LaunchShape ls{LORA_LAUNCH_PERSISTENT, 0, 0, std::min(T, pool->n_slots)};
    hipError_t e = launch_shrink(*pool, seg, T, ls, x, ld_x, const_cast<float*>(v), ld_v, st);
    if (e != hipSuccess) return e;
  }
  if (dma)
    return launch_fused_dma(pl, base, pool, seg, T, xin, ld_in, s_x, v, ld_v, y, ld_y, d_in, d_out, flags,
                            static_cast<uint8_t*>(workspace) + qbytes, st);
  a.x = xin;
  a.ld_x = ld_in;
  a.s_x = s_x;
  if (base.dtype == LORA_BF16) return launch_mode<kBF16>(a, st);
  if (!w8a8) return launch_mode<kW8A16>(a, st);
  return launch_mode<kW8A8>(a, st);
}

size_t fused_slices_workspace_bytes(int T, int d_in, const int32_t* d_out, const int32_t* r_cap, int n,
                                    int base_dtype, int flags) {
  // a merged launch needs the W8A8 codes and, when persistent, 64 bytes of
  // claim counters after them; slices launched one by one use their own
  // plans' workspaces, one after another
  // (bf16 with pools: and after them, 256-byte aligned, the packed adapter
  // records of every slice)
  bool pools = false;
  for (int s = 0; s < n; ++s) pools = pools || r_cap[s] > 0;
  const size_t apk = pools && base_dtype == LORA_BF16 ? 256 + fused_apk_bound(T, n) : 0;
  size_t need = fused_quant_bytes(T, d_in, flags, base_dtype) + 64 + apk;
  for (int s = 0; s < n; ++s)
    need = std::max(need, fused_workspace_bytes(T, d_in, d_out[s], base_dtype, flags, r_cap[s]));
  return need;
}

namespace {
// A bf16 launch of 256 x 256 one-shot tiles whose last round would fill at
// most half the CUs: the full rounds keep those tiles and the remaining
// columns become a second launch, whose planner picks narrower tiles (the
// Llama gate/up pair, 2048 rows by 28672 columns: 3.5 rounds of 256 x 256
// become 3 rounds plus one round of 256 x 128).  Slices are cut at a
// 256-column boundary; a cut slice continues in the second list from column
// col0.  False when the launch does not qualify.
bool split_tail_round(const FusedPlan& pl, const FusedSlice* sl, int n, int T, int d_in, int flags,
                      std::vector<FusedSlice>& first, std::vector<FusedSlice>& rest, FusedPlan& pl_first,
                      FusedPlan& pl_rest) {
  if (sl[0].base.dtype != LORA_BF16 || pl.bm != 256 || pl.bn != 256 || pl.persist || pl.splits != 1 ||
      pl.lora_split != 0)
    return false;
  const long cus = fused_device_cus();
  const long rounds = pl.tiles / cus, rem = pl.tiles % cus;
  if (rounds < 1 || rem == 0 || 2 * rem > cus || (rounds * cus) % pl.tiles_m != 0) return false;
  long left = rounds * cus / pl.tiles_m;       // column tiles of the first launch
  for (int s = 0; s < n; ++s) {
    const FusedSlice& f = sl[s];
    const long nt = (f.d_out + 255) / 256;
    if (left >= nt) {
      first.push_back(f);
      left -= nt;
    } else if (left > 0) {
      FusedSlice a = f, b = f;
      a.d_out = (int)(left * 256);
      b.d_out = f.d_out - a.d_out;
      b.col0 = f.col0 + a.d_out;
      first.push_back(a);
      rest.push_back(b);
      left = 0;
    } else {
      rest.push_back(f);
    }
  }
  if (first.empty() || rest.empty()) return false;
  pl_first = plan_fused_slices(T, d_in, first.data(), (int)first.size(), LORA_BF16, flags);
  pl_rest = plan_fused_slices(T, d_in, rest.data(), (int)rest.size(), LORA_BF16, flags);
  // both must run as merged pipelined launches that need no workspace
  auto ok = [](const FusedPlan& q) { return q.dma && q.part_bytes == 0 && q.counter_bytes == 0; };
  return ok(pl_first) && ok(pl_rest);
}
}  // namespace

hipError_t launch_fused_slices(const FusedSlice* sl, int n, int32_t* seg, int T, const void* x, int ld_x, int d_in,
                               int flags, void* workspace, hipStream_t st) {
  if (T == 0 || n <= 0) return hipSuccess;
  const int bt = sl[0].base.dtype;
  const bool w8a8 = bt == LORA_FP8_E4M3 && (flags & LORA_FLAG_ACT_QUANT_E4M3);
  const int ld_q = (d_in + 15) / 16 * 16;
  FusedPlan pl{};
  bool merged = n > 1 && bt != LORA_F32;
  if (merged) {
    pl = plan_fused_slices(T, d_in, sl, n, bt, flags);
    merged = pl.dma;
    for (int s = 0; merged && s < n; ++s)
      merged = fused_dma_fits(pl, T, w8a8 ? ld_q : ld_x, sl[s].d_out, sl[s].base.ld_w, bt, flags, sl[s].pool);
  }
  if (!merged) {
    for (int s = 0; s < n; ++s) {
      if (sl[s].d_out == 0) continue;
      hipError_t e = launch_fused(sl[s].base, sl[s].pool, seg, T, x, ld_x, sl[s].v, sl[s].ld_v, sl[s].y, sl[s].ld_y,
                                  d_in, sl[s].d_out, flags, workspace, st);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  {
    std::vector<FusedSlice> first, rest;
    FusedPlan pf{}, pr{};
    if (split_tail_round(pl, sl, n, T, d_in, flags, first, rest, pf, pr)) {
      bool fits = true;
      for (const FusedSlice& f : first) fits = fits && fused_dma_fits(pf, T, ld_x, f.d_out, f.base.ld_w, bt, flags, f.pool);
      for (const FusedSlice& f : rest) fits = fits && fused_dma_fits(pr, T, ld_x, f.d_out, f.base.ld_w, bt, flags, f.pool);
      if (fits) {
        hipError_t e = launch_fused_dma_slices(pf, first.data(), (int)first.size(), seg, T, x, ld_x, nullptr, d_in,
                                               flags, workspace, st);
        if (e != hipSuccess) return e;
        return launch_fused_dma_slices(pr, rest.data(), (int)rest.size(), seg, T, x, ld_x, nullptr, d_in, flags,
                                       workspace, st);
      }
    }
  }
  const void* xin = x;
  int ld_in = ld_x;
  float* s_x = nullptr;
  if (w8a8) {
    uint8_t* q = static_cast<uint8_t*>(workspace);
    s_x = reinterpret_cast<float*>(q + (size_t)T * ld_q);
    hipError_t e = launch_quantize_e4m3(x, T, d_in, ld_x, q, ld_q, s_x, st);
    if (e != hipSuccess) return e;
    xin = q;
    ld_in = ld_q;
  }
  return launch_fused_dma_slices(pl, sl, n, seg, T, xin, ld_in, s_x, d_in, flags,
                                 static_cast<uint8_t*>(workspace) + fused_quant_bytes(T, d_in, flags, bt), st);
}

}  // namespace lora
