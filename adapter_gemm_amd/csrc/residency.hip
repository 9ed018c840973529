// Loading one adapter into a pool slot ("LLM-stack book" 7.14.3: the slot is
// filled by an asynchronous copy on a side stream, and the adapter kernels
// run once that stream has passed the copy).  A is one contiguous block of
// rank rows; B goes row by row into the slot's rank-padded rows; the slot's
// rank and scale are written by a one-thread kernel whose arguments carry the
// values, so the refresh needs no host buffer and can be captured in a graph.
#include "common.h"

namespace lora {
namespace {

__global__ void set_slot_kernel(int32_t* slot_rank, float* slot_scale, int slot, int rank, float scale) {
  if (threadIdx.x == 0) {
    slot_rank[slot] = rank;
    slot_scale[slot] = scale;
  }
}

}  // namespace

hipError_t launch_pool_install(const lora_pool_t& pool, int slot, const void* A, const void* B, int rank,
                               float scale, hipStream_t st) {
  const size_t e = pool.dtype == LORA_F32 ? 4 : 2;
  if (rank > 0) {
    uint8_t* Ad = static_cast<uint8_t*>(const_cast<void*>(pool.A)) + (size_t)slot * pool.r_cap * pool.d_in * e;
    hipError_t err = hipMemcpyAsync(Ad, A, (size_t)rank * pool.d_in * e, hipMemcpyDefault, st);
    if (err != hipSuccess) return err;
    uint8_t* Bd = static_cast<uint8_t*>(const_cast<void*>(pool.B)) + (size_t)slot * pool.d_out * pool.r_cap * e;
    err = hipMemcpy2DAsync(Bd, (size_t)pool.r_cap * e, B, (size_t)rank * e, (size_t)rank * e, pool.d_out,
                           hipMemcpyDefault, st);
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(set_slot_kernel, dim3(1), dim3(64), 0, st, const_cast<int32_t*>(pool.slot_rank),
                     const_cast<float*>(pool.slot_scale), slot, rank, scale);
  return hipGetLastError();
}

}  // namespace lora
