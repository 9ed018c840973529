// Internal definitions shared by the HIP kernels and the C-ABI layer of
// liblora (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lora.h"

namespace lora {

// ---------------------------------------------------------------------------
// segment buffer layout (documented in lora.h)
// ---------------------------------------------------------------------------
constexpr int kSegHeader = 16;
enum SummaryWord {
  kNActive = 0, kNSegments = 1, kMMax = 2, kRowBound = 3,
  kNTilesSmall = 4, kNTilesLarge = 5, kRows = 6, kError = 7
};

struct SegPtrs {
  int32_t* sum;
  int32_t* perm;
  int32_t* pos_seg;
  int32_t* seg_start;
  int32_t* seg_adapter;
  int32_t* tiles_small;
  int32_t* tiles_large;
};

__host__ __device__ inline SegPtrs seg_ptrs(int32_t* base, int T) {
  SegPtrs p;
  p.sum = base;
  p.perm = base + kSegHeader;
  p.pos_seg = p.perm + T;
  p.seg_start = p.pos_seg + T;
  p.seg_adapter = p.seg_start + (T + 1);
  p.tiles_small = p.seg_adapter + T;
  p.tiles_large = p.tiles_small + 2 * T;
  return p;
}

__host__ __device__ inline size_t seg_words(int T) { return (size_t)kSegHeader + 8 * (size_t)T + 1; }

// A segment buffer is usable only if its build succeeded and covered T rows;
// otherwise kernels treat the batch as having no live rows, in batch order.
__device__ __forceinline__ bool seg_valid(const SegPtrs& P, int T) {
  return P.sum[kError] == 0 && P.sum[kRows] == T;
}

// ---------------------------------------------------------------------------
// vector types
// ---------------------------------------------------------------------------
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));

// bf16 bits -> fp32 (exact)
__device__ __forceinline__ float bf16lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t u) { return __uint_as_float(((uint32_t)u) << 16); }

// fp32 -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}

// Two fp8 e4m3 codes (bytes 0-1 of w, or 2-3 with HI) -> two bf16, exact: an
// e4m3 value has at most 4 significant bits and an exponent well inside
// bf16's range.  One v_cvt_scalef32_pk_bf16_fp8 with a unit scale (gfx950).
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// Workgroup barrier for data exchanged through LDS: waits for this wave's
// LDS operations only, so global stores still in flight (which no thread of
// the workgroup reads back) do not hold the barrier as __syncthreads() does.
__device__ __forceinline__ void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// 128-bit global loads / stores
__device__ __forceinline__ u32x4_t ld128(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }
__device__ __forceinline__ void st128(void* p, u32x4_t v) { *reinterpret_cast<u32x4_t*>(p) = v; }

__device__ __forceinline__ uint64_t lanemask_lt() {
  return (threadIdx.x & 63) ? (~0ull >> (64 - (threadIdx.x & 63))) : 0ull;
}

// ---------------------------------------------------------------------------
// host-side argument bundles for the kernel launchers
// ---------------------------------------------------------------------------
struct LaunchShape {
  int mode;          // LORA_LAUNCH_*
  int n_tiles;       // host summary (EXACT), else unused
  int row_bound;     // host summary (BUCKETED)
  int slots;         // L for BUCKETED / FULL_BATCH = min(T, n_slots)
};

hipError_t launch_build_segments(const int32_t* ids, const uint8_t* active, int T, int n_slots, int order,
                                 int32_t* seg, hipStream_t st);

hipError_t launch_shrink(const lora_pool_t& pool, int32_t* seg, int T, const LaunchShape& ls,
                         const void* x, int ld_x, float* v, int ld_v, hipStream_t st);

// segment build and persistent shrink in one launch (small batches only)
bool build_shrink_fits(int T, int n_slots);
hipError_t launch_build_shrink(const int32_t* ids, const uint8_t* active, int T, int order, const lora_pool_t& pool,
                               int32_t* seg, const void* x, int ld_x, float* v, int ld_v, hipStream_t st);

hipError_t launch_expand(const lora_pool_t& pool, int32_t* seg, int T, const LaunchShape& ls,
                         const float* v, int ld_v, void* y, int y_dtype, int ld_y, hipStream_t st);

hipError_t launch_fused(const lora_base_t& base, const lora_pool_t* pool, int32_t* seg, int T,
                        const void* x, int ld_x, const float* v, int ld_v, void* y, int ld_y, int d_in,
                        int d_out, int flags, void* workspace, hipStream_t st);

// Schedule of the pipelined fused linear for one call shape.
struct FusedPlan {
  bool dma;            // the pipelined kernel applies (d_in a multiple of its k-step)
  int bm, bn, nk;      // tile and k-steps
  int tiles_m, tiles_n, tiles;
  int splits;          // k splits per tile (1 = none)
  int lora_split;      // 1: one extra workgroup per tile runs the adapter phase
  size_t part_bytes;   // fp32 partial tiles when splits + lora_split > 1
  size_t counter_bytes;  // split hand-off counters, or the persistent launch's claim counters
  bool persist;        // more tiles than CUs, no split: a workgroup per CU claims tiles
  int xrow = 128;      // x bytes per row per k-step (64: bf16 256 x 256 tiles with a 4-slot ring)
  size_t ovl_bytes = 0;  // in-launch shrink: its claim / done / error counters
  bool apipe = false;    // the adapter term as pipelined steps from packed per-tile records
  size_t apk_bytes = 0;  // those records (every slice of the launch)
};
// workspace bytes of the pipelined kernel's parts of a plan, and the offset of
// its packed adapter records within them
size_t fused_dma_ws_bytes(const FusedPlan& pl);
// packed adapter records of a bf16 launch of n slices over T rows, at most
size_t fused_apk_bound(int T, int n_slices);
size_t fused_dma_apk_offset(const FusedPlan& pl);

// The shrink run inside a fused launch (LORA_FLAG_SHRINK_IN_LAUNCH): its
// input x (the unquantised bf16 activations) and the rank-block geometry of
// its items.
struct OverlapShrink {
  const void* x;
  int ld_x;
};
// Rank-block width and blocks per row tile of single-block shrink items for
// this pool and batch (the standalone shrink's rule for the width).
void shrink_item_geometry(const lora_pool_t& pool, int T, int* db, int* nrb);

// r_cap: the adapter pool's rank capacity, 0 without a pool
FusedPlan plan_fused(int T, int d_in, int d_out, int base_dtype, int flags, int r_cap);

// One output slice of a fused launch (slices share x, the rows and seg).
struct FusedSlice {
  lora_base_t base;
  const lora_pool_t* pool;   // NULL: the base product alone
  const float* v;
  int ld_v;
  void* y;
  int ld_y;
  int d_out;                 // output columns of this slice
  int col0 = 0;              // its first column within the projection (base, y and pool rows)
};
// CUs of the current device (256 if the query fails)
int fused_device_cus();
// Whether this plan runs the shrink inside the fused launch (the flag set,
// 64- or 128-row tiles of bf16 or W8A16, no k split)
bool fused_ovl_supported(const FusedPlan& pl, int base_dtype, int flags);
// The plan of one launch over n slices (dma false: the slices go one by one).
FusedPlan plan_fused_slices(int T, int d_in, const FusedSlice* sl, int n, int base_dtype, int flags);
hipError_t launch_fused_dma_slices(const FusedPlan& pl, const FusedSlice* sl, int n, const int32_t* seg, int T,
                                   const void* x, int ld_x, const float* s_x, int d_in, int flags, void* part_ws,
                                   hipStream_t st, const OverlapShrink* ovl = nullptr);
hipError_t launch_fused_slices(const FusedSlice* sl, int n, int32_t* seg, int T, const void* x, int ld_x, int d_in,
                               int flags, void* workspace, hipStream_t st);
size_t fused_slices_workspace_bytes(int T, int d_in, const int32_t* d_out, const int32_t* r_cap, int n,
                                    int base_dtype, int flags);
bool fused_dma_fits(const FusedPlan& pl, int T, int ld_x, int d_out, int ld_w, int base_dtype, int flags,
                    const lora_pool_t* pool);
hipError_t launch_fused_dma(const FusedPlan& pl, const lora_base_t& base, const lora_pool_t* pool,
                            const int32_t* seg, int T, const void* x, int ld_x, const float* s_x, const float* v,
                            int ld_v, void* y, int ld_y, int d_in, int d_out, int flags, void* part_ws,
                            hipStream_t st, const OverlapShrink* ovl = nullptr);
// bytes of the workspace for one fused call: [W8A8 codes + scales][partials][counters]
size_t fused_quant_bytes(int T, int d_in, int flags, int base_dtype);
size_t fused_workspace_bytes(int T, int d_in, int d_out, int base_dtype, int flags, int r_cap);

hipError_t launch_pool_install(const lora_pool_t& pool, int slot, const void* A, const void* B, int rank,
                               float scale, hipStream_t st);
hipError_t launch_quantize_e4m3(const void* x, int T, int d, int ld_x, uint8_t* q, int ld_q, float* s_x,
                                hipStream_t st);

}  // namespace lora
