// Per-token fp8 (OCP e4m3fn) activation quantisation for the W8A8 base
// product ("EpiLoRA" 2 and Fig. 4: the activations are quantised once per
// token, x -> (x_q, s_x), and the GEMM applies s_x s_w to its result).
//
//   s_x[i]  = amax_k |x[i, k]| / 448           (fp32, correctly rounded)
//   q[i, k] = e4m3( x[i, k] / s_x[i] )          (fp32 division, round to
//                                               nearest even, saturate +-448)
// The quotient is the correctly rounded fp32 x / s_x, formed without a
// division sequence (see e4m3_quot), and the hardware's e4m3 conversion (round
// to nearest even) rounds it after a clamp to +-448, so every code is the one
// stated above.
#include "common.h"

namespace lora {
namespace {

constexpr int kQuantThreads = 256;
constexpr int kRegChunks = 8;     // rows of up to 8 x 2048 values stay in registers

// Correctly rounded x / s from y = RN(1 / s): q1 = RN(x y) is within an ulp
// of x / s, the residual r = x - q1 s then comes out exact from one fma, and
// RN(q1 + r y) is the correctly rounded quotient (Markstein's theorem on the
// final correction step of a division, which needs y correctly rounded and q1
// faithful).  r is exact whenever |x / s| >= 2^-11 and s >= 2^-90 (its bits
// then stay above the fp32 subnormal grid); smaller quotients all encode to
// +-0 whatever their last bits.  The sign is x's (s > 0), set at the end
// because the correction turns x = -0 into +0 (r = +0, and +0 + -0 = +0).
__device__ __forceinline__ float e4m3_quot(float x, float s, float y) {
  const float q1 = x * y;
  const float r = __builtin_fmaf(-q1, s, x);
  return __builtin_copysignf(__builtin_fmaf(r, y, q1), x);
}

// Two quotients to two e4m3fn codes in the low half of the result.
template <bool DIV>
__device__ __forceinline__ uint32_t e4m3x2(float x0, float x1, float s, float y) {
  const float q0 = DIV ? __fdiv_rn(x0, s) : e4m3_quot(x0, s, y);
  const float q1 = DIV ? __fdiv_rn(x1, s) : e4m3_quot(x1, s, y);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(q0, -448.0f, 448.0f),
                                                   __builtin_amdgcn_fmed3f(q1, -448.0f, 448.0f), 0, false) & 0xffffu;
}

// Eight values (one 16-byte load) to eight codes.
template <bool DIV>
__device__ __forceinline__ uint2 e4m3x8(const u32x4_t& u, float s, float y) {
  return uint2{e4m3x2<DIV>(bf16lo(u[0]), bf16hi(u[0]), s, y) | (e4m3x2<DIV>(bf16lo(u[1]), bf16hi(u[1]), s, y) << 16),
               e4m3x2<DIV>(bf16lo(u[2]), bf16hi(u[2]), s, y) | (e4m3x2<DIV>(bf16lo(u[3]), bf16hi(u[3]), s, y) << 16)};
}

// The row's amax from each thread's partial maximum: the wave's, then the
// workgroup's waves through LDS; s_x follows (an all-zero row gets 1).
__device__ __forceinline__ float row_scale(float amax, float* wave_max) {
  const int t = threadIdx.x;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  if ((t & 63) == 0) wave_max[t >> 6] = amax;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kQuantThreads / 64; ++w) amax = fmaxf(amax, wave_max[w]);
  return amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f;
}

// (s is uniform over the workgroup; below 2^-90 the residual could lose bits
// that decide a code, and the division is taken as it stands)
__device__ __forceinline__ bool quot_by_rcp(float s) { return s >= 0x1p-90f; }

// One row per workgroup of four waves, for rows of at most NC x 2048 values
// (a launch of T workgroups: 512 rows already give every CU two).  Thread t
// loads the 8-value groups t, t + 256, ... of the row at once (a group past
// the row loads the row's last one again: every address stays in the row,
// and a repeated value leaves the maximum as it is), keeps them in registers
// while the amax is reduced, then encodes and stores the groups in the row.
template <int NC>
__global__ __launch_bounds__(kQuantThreads) void quant_kernel(const uint16_t* __restrict__ x, int d, int ld_x,
                                                              uint8_t* __restrict__ q, int ld_q,
                                                              float* __restrict__ s_x) {
  __shared__ float wave_max[kQuantThreads / 64];
  const int t = threadIdx.x;
  const int row = blockIdx.x;
  const uint16_t* xr = x + (size_t)row * ld_x;
  u32x4_t u[NC];
#pragma unroll
  for (int j = 0; j < NC; ++j) u[j] = ld128(xr + min(8 * (t + kQuantThreads * j), d - 8));
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < NC; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) amax = fmaxf(amax, fmaxf(fabsf(bf16lo(u[j][e])), fabsf(bf16hi(u[j][e]))));
  const float s = row_scale(amax, wave_max);
  if (t == 0) s_x[row] = s;
  uint8_t* qr = q + (size_t)row * ld_q;
  if (quot_by_rcp(s)) {
    const float y = __fdiv_rn(1.0f, s);
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const int k = 8 * (t + kQuantThreads * j);
      if (k < d) *reinterpret_cast<uint2*>(qr + k) = e4m3x8<false>(u[j], s, y);
    }
  } else {
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const int k = 8 * (t + kQuantThreads * j);
      if (k < d) *reinterpret_cast<uint2*>(qr + k) = e4m3x8<true>(u[j], s, 0.f);
    }
  }
}

// Rows longer than kRegChunks x 2048 values: pass 1 reduces the amax over the
// row, pass 2 re-reads the row (from L2) and encodes it.
__global__ __launch_bounds__(kQuantThreads) void quant_kernel_long(const uint16_t* __restrict__ x, int d, int ld_x,
                                                                   uint8_t* __restrict__ q, int ld_q,
                                                                   float* __restrict__ s_x) {
  __shared__ float wave_max[kQuantThreads / 64];
  const int t = threadIdx.x;
  const int row = blockIdx.x;
  const uint16_t* xr = x + (size_t)row * ld_x;
  float amax = 0.f;
  for (int k = 8 * t; k < d; k += 8 * kQuantThreads) {
    const u32x4_t u = ld128(xr + k);
#pragma unroll
    for (int e = 0; e < 4; ++e) amax = fmaxf(amax, fmaxf(fabsf(bf16lo(u[e])), fabsf(bf16hi(u[e]))));
  }
  const float s = row_scale(amax, wave_max);
  if (t == 0) s_x[row] = s;
  uint8_t* qr = q + (size_t)row * ld_q;
  if (quot_by_rcp(s)) {
    const float y = __fdiv_rn(1.0f, s);
    for (int k = 8 * t; k < d; k += 8 * kQuantThreads)
      *reinterpret_cast<uint2*>(qr + k) = e4m3x8<false>(ld128(xr + k), s, y);
  } else {
    for (int k = 8 * t; k < d; k += 8 * kQuantThreads)
      *reinterpret_cast<uint2*>(qr + k) = e4m3x8<true>(ld128(xr + k), s, 0.f);
  }
}

}  // namespace

hipError_t launch_quantize_e4m3(const void* x, int T, int d, int ld_x, uint8_t* q, int ld_q, float* s_x,
                                hipStream_t st) {
  if (T == 0) return hipSuccess;
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  const int nc = (d + 8 * kQuantThreads - 1) / (8 * kQuantThreads);   // 2048-value chunks of a row
  const dim3 grid(T), block(kQuantThreads);
  static_assert(kRegChunks == 8, "one case per chunk count below");
  switch (nc) {
    case 1: hipLaunchKernelGGL(quant_kernel<1>, grid, block, 0, st, xb, d, ld_x, q, ld_q, s_x); break;
    case 2: hipLaunchKernelGGL(quant_kernel<2>, grid, block, 0, st, xb, d, ld_x, q, ld_q, s_x); break;
    case 3: hipLaunchKernelGGL(quant_kernel<3>, grid, block, 0, st, xb, d, ld_x, q, ld_q, s_x); break;
    case 4: hipLaunchKernelGGL(quant_kernel<4>, grid, block, 0, st, xb, d, ld_x, q, ld_q, s_x); break;
    case 5: hipLaunchKernelGGL(quant_kernel<5>, grid, block, 0, st, xb, d, ld_x, q, ld_q, s_x); break;
    case 6: hipLaunchKernelGGL(quant_kernel<6>, grid, block, 0, st, xb, d, ld_x, q, ld_q, s_x); break;
    case 7: hipLaunchKernelGGL(quant_kernel<7>, grid, block, 0, st, xb, d, ld_x, q, ld_q, s_x); break;
    case 8: hipLaunchKernelGGL(quant_kernel<8>, grid, block, 0, st, xb, d, ld_x, q, ld_q, s_x); break;
    default: hipLaunchKernelGGL(quant_kernel_long, grid, block, 0, st, xb, d, ld_x, q, ld_q, s_x); break;
  }
  return hipGetLastError();
}

}  // namespace lora
