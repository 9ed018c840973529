// C-ABI entry points of liblora: argument validation, the host segment
// planner and dispatch to the HIP kernel launchers.  Every check runs before
// anything is enqueued; errors never modify an output.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "common.h"

namespace {

thread_local std::string g_last_error;

int hip_status(hipError_t e) {
  if (e == hipSuccess) return LORA_OK;
  g_last_error = hipGetErrorString(e);
  return LORA_E_HIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_size(int dtype) { return dtype == LORA_F32 ? 4 : dtype == LORA_BF16 ? 2 : 1; }

int check_pool(const lora_pool_t* pool) {
  if (!pool || !pool->A || !pool->B || !pool->slot_rank || !pool->slot_scale) return LORA_E_ARG;
  if (pool->dtype != LORA_F32 && pool->dtype != LORA_BF16) return LORA_E_DTYPE;
  if (pool->n_slots < 0 || pool->d_in < 0 || pool->d_out < 0) return LORA_E_ARG;
  if (pool->r_cap < 1 || pool->r_cap > LORA_MAX_RANK) return LORA_E_RANK;
  const int vec = 16 / elem_size(pool->dtype);
  if (pool->r_cap % vec) return LORA_E_ALIGN;
  if (pool->d_in % 8 || pool->d_out % 8) return LORA_E_ALIGN;
  if (!aligned16(pool->A) || !aligned16(pool->B)) return LORA_E_ALIGN;
  return LORA_OK;
}

// Host mirror of the summary words.
void fill_summary(const int32_t* words, lora_summary_t* s) {
  if (!s) return;
  s->n_active = words[lora::kNActive];
  s->n_segments = words[lora::kNSegments];
  s->m_max = words[lora::kMMax];
  s->row_bound = words[lora::kRowBound];
  s->n_tiles_small = words[lora::kNTilesSmall];
  s->n_tiles_large = words[lora::kNTilesLarge];
  s->T = words[lora::kRows];
  s->error = words[lora::kError];
}

int launch_shape(int launch, const lora_summary_t* summary, int T, int n_slots, lora::LaunchShape& ls) {
  ls.mode = launch;
  ls.n_tiles = 0;
  ls.row_bound = 0;
  ls.slots = std::min(T, n_slots);
  switch (launch) {
    case LORA_LAUNCH_EXACT:
      if (!summary) return LORA_E_ARG;
      if (summary->T != T) return LORA_E_ARG;
      ls.n_tiles = summary->n_tiles_small;
      return LORA_OK;
    case LORA_LAUNCH_BUCKETED:
      if (!summary) return LORA_E_ARG;
      if (summary->T != T) return LORA_E_ARG;
      ls.row_bound = summary->row_bound;
      return LORA_OK;
    case LORA_LAUNCH_PERSISTENT:
    case LORA_LAUNCH_FULL_BATCH:
      return LORA_OK;
    default:
      return LORA_E_ARG;
  }
}

}  // namespace

extern "C" {

size_t lora_segment_words(int32_t T) { return T < 0 ? 0 : lora::seg_words(T); }

int lora_plan_segments(const int32_t* ids, const uint8_t* active, int32_t T, int32_t n_slots, int32_t order,
                       int32_t* plan, lora_summary_t* summary) {
  if (T < 0 || n_slots < 0 || (T > 0 && !ids) || !plan || (order != 0 && order != 1)) return LORA_E_ARG;
  for (int i = 0; i < T; ++i)
    if (ids[i] < -1 || ids[i] >= n_slots) return LORA_E_ID;

  std::memset(plan, 0, lora::seg_words(T) * sizeof(int32_t));
  lora::SegPtrs P = lora::seg_ptrs(plan, T);

  // live rows per adapter, in batch order
  std::vector<int> count(n_slots, 0), first(n_slots, -1);
  std::vector<int> seg_of(n_slots, -1);
  std::vector<int> adapters;  // segment order
  for (int i = 0; i < T; ++i) {
    const int id = ids[i];
    if (id < 0 || (active && active[i] == 0)) continue;
    if (count[id]++ == 0) {
      first[id] = i;
      if (order == 1) adapters.push_back(id);
    }
  }
  if (order == 0)
    for (int a = 0; a < n_slots; ++a)
      if (count[a] > 0) adapters.push_back(a);
  const int S = static_cast<int>(adapters.size());

  int pos = 0, mmax = 0, ts = 0, tl = 0;
  std::vector<int> cursor(n_slots, 0);
  for (int s = 0; s < S; ++s) {
    const int a = adapters[s];
    seg_of[a] = s;
    P.seg_start[s] = pos;
    P.seg_adapter[s] = a;
    cursor[a] = pos;
    const int len = count[a];
    for (int t = 0; t < len; t += LORA_TILE_SMALL) {
      P.tiles_small[2 * ts] = pos + t;
      P.tiles_small[2 * ts + 1] = s;
      ++ts;
    }
    for (int t = 0; t < len; t += LORA_TILE_LARGE) {
      P.tiles_large[2 * tl] = pos + t;
      P.tiles_large[2 * tl + 1] = s;
      ++tl;
    }
    pos += len;
    mmax = std::max(mmax, len);
  }
  P.seg_start[S] = pos;
  const int n_active = pos;
  int dead = n_active;
  for (int i = 0; i < T; ++i) {
    const int id = ids[i];
    const bool live = id >= 0 && !(active && active[i] == 0);
    if (live) {
      const int p = cursor[id]++;
      P.perm[p] = i;
      P.pos_seg[p] = seg_of[id];
    } else {
      P.perm[dead] = i;
      P.pos_seg[dead] = -1;
      ++dead;
    }
  }
  int R = 0;
  if (n_active > 0) {
    R = T;
    for (int r = 16; r < T; r <<= 1)
      if (r >= mmax) { R = r; break; }
  }
  P.sum[lora::kNActive] = n_active;
  P.sum[lora::kNSegments] = S;
  P.sum[lora::kMMax] = mmax;
  P.sum[lora::kRowBound] = R;
  P.sum[lora::kNTilesSmall] = ts;
  P.sum[lora::kNTilesLarge] = tl;
  P.sum[lora::kRows] = T;
  P.sum[lora::kError] = 0;
  fill_summary(P.sum, summary);
  return LORA_OK;
}

int lora_build_segments(const int32_t* ids, const uint8_t* active, int32_t T, int32_t n_slots, int32_t order,
                        int32_t* staging, int32_t* seg, lora_summary_t* summary, void* stream) {
  if (!seg) return LORA_E_ARG;
  int st = lora_plan_segments(ids, active, T, n_slots, order, staging, summary);
  if (st != LORA_OK) return st;
  return hip_status(hipMemcpyAsync(seg, staging, lora::seg_words(T) * sizeof(int32_t), hipMemcpyHostToDevice,
                                   static_cast<hipStream_t>(stream)));
}

int lora_build_segments_dev(const int32_t* ids, const uint8_t* active, int32_t T, int32_t n_slots, int32_t order,
                            int32_t* seg, void* stream) {
  if (T < 0 || n_slots < 0 || (T > 0 && !ids) || !seg || (order != 0 && order != 1)) return LORA_E_ARG;
  if (n_slots > LORA_DEV_MAX_SLOTS) return LORA_E_SIZE;
  return hip_status(lora::launch_build_segments(ids, active, T, n_slots, order, seg,
                                                static_cast<hipStream_t>(stream)));
}

int lora_shrink(const lora_pool_t* pool, const int32_t* seg, int32_t T, const lora_summary_t* summary,
                const void* x, int32_t ld_x, float* v, int32_t ld_v, int32_t launch, void* stream) {
  int st = check_pool(pool);
  if (st != LORA_OK) return st;
  if (T < 0 || !seg || (T > 0 && (!x || !v))) return LORA_E_ARG;
  if (ld_x < pool->d_in || ld_v < pool->r_cap) return LORA_E_ARG;
  if (ld_x % 8 || ld_v % 4 || !aligned16(x) || !aligned16(v)) return LORA_E_ALIGN;
  lora::LaunchShape ls;
  st = launch_shape(launch, summary, T, pool->n_slots, ls);
  if (st != LORA_OK) return st;
  if (T == 0) return LORA_OK;
  return hip_status(lora::launch_shrink(*pool, const_cast<int32_t*>(seg), T, ls, x, ld_x, v, ld_v,
                                        static_cast<hipStream_t>(stream)));
}

int lora_build_shrink_dev(const int32_t* ids, const uint8_t* active, int32_t T, int32_t order,
                          const lora_pool_t* pool, int32_t* seg, const void* x, int32_t ld_x, float* v, int32_t ld_v,
                          void* stream) {
  int st = check_pool(pool);
  if (st != LORA_OK) return st;
  if (T < 0 || !seg || (T > 0 && (!ids || !x || !v)) || (order != 0 && order != 1)) return LORA_E_ARG;
  if (pool->n_slots > LORA_DEV_MAX_SLOTS) return LORA_E_SIZE;
  if (ld_x < pool->d_in || ld_v < pool->r_cap) return LORA_E_ARG;
  if (ld_x % 8 || ld_v % 4 || !aligned16(x) || !aligned16(v)) return LORA_E_ALIGN;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (lora::build_shrink_fits(T, pool->n_slots))
    return hip_status(lora::launch_build_shrink(ids, active, T, order, *pool, seg, x, ld_x, v, ld_v, s));
  st = hip_status(lora::launch_build_segments(ids, active, T, pool->n_slots, order, seg, s));
  if (st != LORA_OK || T == 0) return st;
  lora::LaunchShape ls;
  st = launch_shape(LORA_LAUNCH_PERSISTENT, nullptr, T, pool->n_slots, ls);
  if (st != LORA_OK) return st;
  return hip_status(lora::launch_shrink(*pool, seg, T, ls, x, ld_x, v, ld_v, s));
}

int lora_expand(const lora_pool_t* pool, const int32_t* seg, int32_t T, const lora_summary_t* summary,
                const float* v, int32_t ld_v, void* y, int32_t y_dtype, int32_t ld_y, int32_t launch, void* stream) {
  int st = check_pool(pool);
  if (st != LORA_OK) return st;
  if (T < 0 || !seg || (T > 0 && (!v || !y))) return LORA_E_ARG;
  if (y_dtype != LORA_F32 && y_dtype != LORA_BF16) return LORA_E_DTYPE;
  if (ld_y < pool->d_out || ld_v < pool->r_cap) return LORA_E_ARG;
  if (ld_y % 8 || ld_v % 4 || !aligned16(y) || !aligned16(v)) return LORA_E_ALIGN;
  lora::LaunchShape ls;
  st = launch_shape(launch, summary, T, pool->n_slots, ls);
  if (st != LORA_OK) return st;
  if (T == 0) return LORA_OK;
  return hip_status(lora::launch_expand(*pool, const_cast<int32_t*>(seg), T, ls, v, ld_v, y, y_dtype, ld_y,
                                        static_cast<hipStream_t>(stream)));
}

size_t lora_fused_workspace_bytes(int32_t T, int32_t d_in, int32_t d_out, int32_t base_dtype, int32_t flags) {
  if (T <= 0 || d_in <= 0 || d_out <= 0) return 0;
  if (base_dtype != LORA_F32 && base_dtype != LORA_BF16 && base_dtype != LORA_FP8_E4M3) return 0;
  // The schedule depends on the pool's rank capacity (larger capacities leave
  // less LDS for the larger tiles, whose launches may then need claim
  // counters), so the size returned covers every capacity, and no pool.
  size_t need = lora::fused_workspace_bytes(T, d_in, d_out, base_dtype, flags, 0);
  for (int rc = 4; rc <= LORA_MAX_RANK; rc += 4)
    need = std::max(need, lora::fused_workspace_bytes(T, d_in, d_out, base_dtype, flags, rc));
  return need;
}

size_t lora_fused_workspace_bytes_rcap(int32_t T, int32_t d_in, int32_t d_out, int32_t base_dtype, int32_t flags,
                                       int32_t r_cap) {
  if (T <= 0 || d_in <= 0 || d_out <= 0 || r_cap < 0 || r_cap > LORA_MAX_RANK) return 0;
  if (base_dtype != LORA_F32 && base_dtype != LORA_BF16 && base_dtype != LORA_FP8_E4M3) return 0;
  return lora::fused_workspace_bytes(T, d_in, d_out, base_dtype, flags, r_cap);
}

}  // extern "C"

namespace {
// Arguments of one fused product (everything but the workspace).
int check_fused(const lora_base_t* base, const lora_pool_t* pool, const int32_t* seg, int32_t T, const void* x,
                int32_t ld_x, const float* v, int32_t ld_v, const void* y, int32_t ld_y, int32_t d_in, int32_t d_out,
                int32_t flags) {
  if (!base || !base->W) return LORA_E_ARG;
  if (T < 0 || d_in < 0 || d_out < 0 || (T > 0 && (!x || !y))) return LORA_E_ARG;
  if (flags & ~(LORA_FLAG_ACT_QUANT_E4M3 | LORA_FLAG_SHRINK_IN_LAUNCH)) return LORA_E_ARG;
  const int bt = base->dtype;
  if (bt != LORA_F32 && bt != LORA_BF16 && bt != LORA_FP8_E4M3) return LORA_E_DTYPE;
  const int dt = bt == LORA_F32 ? LORA_F32 : LORA_BF16;   // x, pool and y type
  if (bt == LORA_FP8_E4M3 && !base->w_scale) return LORA_E_ARG;
  if ((flags & LORA_FLAG_ACT_QUANT_E4M3) && bt != LORA_FP8_E4M3) return LORA_E_DTYPE;
  if (flags & LORA_FLAG_SHRINK_IN_LAUNCH) {        // v is computed by the call from x
    if (!pool) return LORA_E_ARG;
    if (bt == LORA_F32) return LORA_E_DTYPE;
  }
  if (pool) {
    int st = check_pool(pool);
    if (st != LORA_OK) return st;
    if (pool->dtype != dt) return LORA_E_DTYPE;
    if (pool->d_in != d_in || pool->d_out != d_out) return LORA_E_ARG;
    if (!seg || !v) return LORA_E_ARG;
    if (ld_v < pool->r_cap) return LORA_E_ARG;
    if (ld_v % 4 || !aligned16(v)) return LORA_E_ALIGN;
  } else if (v) {
    return LORA_E_ARG;
  }
  if (ld_x < d_in || ld_y < d_out || base->ld_w < d_in) return LORA_E_ARG;
  if (d_in % 8 || d_out % 8 || ld_x % 8 || ld_y % 8) return LORA_E_ALIGN;
  if (bt == LORA_FP8_E4M3 && (d_in % 16 || base->ld_w % 16)) return LORA_E_ALIGN;
  if (bt != LORA_FP8_E4M3 && base->ld_w % 8) return LORA_E_ALIGN;
  if (!aligned16(x) || !aligned16(y) || !aligned16(base->W)) return LORA_E_ALIGN;
  if (x == y) return LORA_E_ARG;
  return LORA_OK;
}
}  // namespace

extern "C" {

int lora_fused_linear(const lora_base_t* base, const lora_pool_t* pool, const int32_t* seg, int32_t T,
                      const void* x, int32_t ld_x, const float* v, int32_t ld_v, void* y, int32_t ld_y,
                      int32_t d_in, int32_t d_out, int32_t flags, void* workspace, size_t workspace_bytes,
                      void* stream) {
  const int st = check_fused(base, pool, seg, T, x, ld_x, v, ld_v, y, ld_y, d_in, d_out, flags);
  if (st != LORA_OK) return st;
  const int bt = base->dtype;
  const size_t need = lora::fused_workspace_bytes(T, d_in, d_out, bt, flags, pool ? pool->r_cap : 0);
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return LORA_E_SIZE;
    if (reinterpret_cast<uintptr_t>(workspace) & 255u) return LORA_E_ALIGN;
  }
  if (T == 0 || d_out == 0) return LORA_OK;
  return hip_status(lora::launch_fused(*base, pool, const_cast<int32_t*>(seg), T, x, ld_x, v, ld_v, y, ld_y, d_in,
                                       d_out, flags, workspace, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// ---- the allocation-free fused call ----------------------------------------
// Device scratch of lora_fused_linear_noalloc: one copy per GPU (each device
// that loads the library holds its own), kept until the process ends.  Host
// code never passes this name to a kernel or a copy: it is a host-side stand-
// in for the symbol; the device address comes from hipGetSymbolAddress, once
// per device, with that device current.
static __device__ __align__(256) uint8_t scratch[LORA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Device address of this device's scratch (set-up on the first call per device).
hipError_t scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}
}  // namespace

extern "C" {

int lora_fused_linear_noalloc(const lora_base_t* base, const lora_pool_t* pool, const int32_t* seg, int32_t T,
                              const void* x, int32_t ld_x, const float* v, int32_t ld_v, void* y, int32_t ld_y,
                              int32_t d_in, int32_t d_out, int32_t flags, void* stream) {
  const int st = check_fused(base, pool, seg, T, x, ld_x, v, ld_v, y, ld_y, d_in, d_out, flags);
  if (st != LORA_OK) return st;
  const size_t need = lora::fused_workspace_bytes(T, d_in, d_out, base->dtype, flags, pool ? pool->r_cap : 0);
  if (need > LORA_NOALLOC_SCRATCH_BYTES) {
    g_last_error = "lora_fused_linear_noalloc: the call needs " + std::to_string(need) +
                   " bytes of scratch, more than the static " + std::to_string((size_t)LORA_NOALLOC_SCRATCH_BYTES);
    return LORA_E_SIZE;
  }
  if (T == 0 || d_out == 0) return LORA_OK;
  void* ws = nullptr;
  if (need > 0) {
    const int sp = hip_status(scratch_ptr(&ws));
    if (sp != LORA_OK) return sp;
  }
  return hip_status(lora::launch_fused(*base, pool, const_cast<int32_t*>(seg), T, x, ld_x, v, ld_v, y, ld_y, d_in,
                                       d_out, flags, ws, static_cast<hipStream_t>(stream)));
}

size_t lora_fused_slices_workspace_bytes(int32_t n_slices, int32_t T, int32_t d_in, const int32_t* d_out,
                                         int32_t base_dtype, int32_t flags) {
  if (n_slices <= 0 || !d_out || T <= 0 || d_in <= 0) return 0;
  if (base_dtype != LORA_F32 && base_dtype != LORA_BF16 && base_dtype != LORA_FP8_E4M3) return 0;
  for (int s = 0; s < n_slices; ++s)
    if (d_out[s] < 0) return 0;
  // as lora_fused_workspace_bytes: the largest size over every rank capacity
  // (the launch plans with the slices' largest capacity), and no pool
  size_t need = 0;
  for (int rc = 0; rc <= LORA_MAX_RANK; rc += 4) {
    const std::vector<int32_t> rcs(n_slices, rc);
    need = std::max(need, lora::fused_slices_workspace_bytes(T, d_in, d_out, rcs.data(), n_slices, base_dtype, flags));
  }
  return need;
}

int lora_fused_linear_slices(int32_t n_slices, const lora_base_t* bases, const lora_pool_t* pools,
                             const int32_t* seg, int32_t T, const void* x, int32_t ld_x, int32_t d_in,
                             const int32_t* d_out, const float* const* v, const int32_t* ld_v, void* const* y,
                             const int32_t* ld_y, int32_t flags, void* workspace, size_t workspace_bytes,
                             void* stream) {
  if (n_slices < 1 || !bases || !d_out || !y || !ld_y || ((pools != nullptr) != (v != nullptr))) return LORA_E_ARG;
  if (flags & LORA_FLAG_SHRINK_IN_LAUNCH) return LORA_E_ARG;   // (single-projection calls only)
  if (pools && !ld_v) return LORA_E_ARG;
  std::vector<lora::FusedSlice> sl(n_slices);
  std::vector<int32_t> rc(n_slices, 0);
  for (int s = 0; s < n_slices; ++s) {
    const lora_pool_t* pool = pools ? &pools[s] : nullptr;
    const float* vs = v ? v[s] : nullptr;
    const int32_t lv = v ? ld_v[s] : 0;
    const int st = check_fused(&bases[s], pool, seg, T, x, ld_x, vs, lv, y[s], ld_y[s], d_in, d_out[s], flags);
    if (st != LORA_OK) return st;
    if (bases[s].dtype != bases[0].dtype) return LORA_E_DTYPE;
    for (int o = 0; o < s; ++o)
      if (y[o] == y[s]) return LORA_E_ARG;            // each slice writes its own output
    sl[s] = lora::FusedSlice{bases[s], pool, vs, lv, y[s], ld_y[s], d_out[s]};
    rc[s] = pool ? pool->r_cap : 0;
  }
  const int bt = bases[0].dtype;
  const size_t need = lora::fused_slices_workspace_bytes(T, d_in, d_out, rc.data(), n_slices, bt, flags);
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return LORA_E_SIZE;
    if (reinterpret_cast<uintptr_t>(workspace) & 255u) return LORA_E_ALIGN;
  }
  if (T == 0) return LORA_OK;
  return hip_status(lora::launch_fused_slices(sl.data(), n_slices, const_cast<int32_t*>(seg), T, x, ld_x, d_in,
                                              flags, workspace, static_cast<hipStream_t>(stream)));
}

int lora_pool_install(const lora_pool_t* pool, int32_t slot, const void* A, const void* B, int32_t rank,
                      float scale, void* stream) {
  const int st = check_pool(pool);
  if (st != LORA_OK) return st;
  if (slot < 0 || slot >= pool->n_slots || rank < 0 || rank > pool->r_cap) return LORA_E_ARG;
  if (rank > 0 && (!A || !B)) return LORA_E_ARG;
  return hip_status(lora::launch_pool_install(*pool, slot, A, B, rank, scale, static_cast<hipStream_t>(stream)));
}

// ---- concurrent base / adapter work on disjoint CU sets ----------------------

int lora_device_cu_count(int32_t* n_cus) {
  if (!n_cus) return LORA_E_ARG;
  int dev = 0, n = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_status(e);
  *n_cus = n;
  return LORA_OK;
}

int lora_stream_create_cu_masked(const uint32_t* cu_mask, int32_t n_words, void** stream) {
  if (!stream || !cu_mask || n_words <= 0) return LORA_E_ARG;
  *stream = nullptr;
  bool any = false;
  for (int32_t i = 0; i < n_words; ++i) any = any || cu_mask[i] != 0;
  if (!any) return LORA_E_ARG;
  hipStream_t s = nullptr;
  const int st = hip_status(hipExtStreamCreateWithCUMask(&s, (uint32_t)n_words, cu_mask));
  if (st != LORA_OK) return st;
  *stream = s;
  return LORA_OK;
}

int lora_stream_destroy(void* stream) {
  if (!stream) return LORA_E_ARG;
  return hip_status(hipStreamDestroy(static_cast<hipStream_t>(stream)));
}

int lora_quantize_e4m3(const void* x, int32_t T, int32_t d, int32_t ld_x, uint8_t* q, int32_t ld_q, float* s_x,
                       void* stream) {
  if (T < 0 || d < 0 || (T > 0 && (!x || !q || !s_x))) return LORA_E_ARG;
  if (ld_x < d || ld_q < d) return LORA_E_ARG;
  if (d % 16 || ld_x % 8 || ld_q % 16 || !aligned16(x) || !aligned16(q)) return LORA_E_ALIGN;
  if (T == 0 || d == 0) return LORA_OK;
  return hip_status(lora::launch_quantize_e4m3(x, T, d, ld_x, q, ld_q, s_x, static_cast<hipStream_t>(stream)));
}

const char* lora_status_string(int status) {
  switch (status) {
    case LORA_OK: return "ok";
    case LORA_E_ARG: return "invalid argument";
    case LORA_E_ID: return "adapter id out of range";
    case LORA_E_RANK: return "rank capacity out of range";
    case LORA_E_DTYPE: return "unsupported dtype combination";
    case LORA_E_ALIGN: return "pointer or leading dimension not 16-byte aligned";
    case LORA_E_HIP: return "HIP error";
    case LORA_E_SIZE: return "size beyond a limit or buffer too small";
    default: return "unknown status";
  }
}

const char* lora_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
