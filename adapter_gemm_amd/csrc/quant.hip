// Per-token fp8 (OCP e4m3fn) activation quantisation for the W8A8 base
// product ("EpiLoRA" 2 and Fig. 4: the activations are quantised once per
// token, x -> (x_q, s_x), and the GEMM applies s_x s_w to its result).
//
//   s_x[i]  = amax_k |x[i, k]| / 448           (fp32, correctly rounded)
//   q[i, k] = e4m3( x[i, k] / s_x[i] )          (fp32 division, round to
//                                               nearest even, saturate +-448)
// One wave per row: pass 1 reduces the row's amax, pass 2 re-reads the row
// (from L2) and writes 16 codes per lane per 128-bit store.  The e4m3
// rounding is done on the fp32 bit pattern so the decision is exactly the
// one stated above.
#include "common.h"

namespace lora {
namespace {

__device__ __forceinline__ uint32_t e4m3_encode(float q) {
  const uint32_t u = __float_as_uint(q);
  const uint32_t sign = (u >> 24) & 0x80u;
  float a = fminf(fabsf(q), 448.0f);
  uint32_t code;
  if (a < 0.015625f) {                       // below 2^-6: subnormal grid of 2^-9
    code = (uint32_t)rintf(a * 512.0f);      // exact scaling, ties to even; 8 -> 0x08 = 2^-6
  } else {
    const uint32_t b = __float_as_uint(a);
    uint32_t E = b >> 23;
    uint32_t m = (b & 0x7fffffu);
    uint32_t m3 = m >> 20;
    const uint32_t rem = m & 0xfffffu;
    if (rem > 0x80000u || (rem == 0x80000u && (m3 & 1u))) ++m3;
    if (m3 == 8u) { m3 = 0; ++E; }
    code = ((E - 120u) << 3) | m3;           // e4m3 exponent = E - 127 + 7
  }
  return code | sign;
}

__global__ __launch_bounds__(256) void quant_kernel(const uint16_t* __restrict__ x, int T, int d, int ld_x,
                                                    uint8_t* __restrict__ q, int ld_q, float* __restrict__ s_x) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= T) return;
  const uint16_t* xr = x + (size_t)row * ld_x;
  float amax = 0.f;
  for (int k = lane * 8; k < d; k += 512) {
    const u32x4_t u = ld128(xr + k);
#pragma unroll
    for (int e = 0; e < 4; ++e) amax = fmaxf(amax, fmaxf(fabsf(bf16lo(u[e])), fabsf(bf16hi(u[e]))));
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  const float s = amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f;
  if (lane == 0) s_x[row] = s;
  uint8_t* qr = q + (size_t)row * ld_q;
  for (int k = lane * 16; k < d; k += 1024) {
    const u32x4_t u0 = ld128(xr + k);
    const u32x4_t u1 = ld128(xr + k + 8);
    u32x4_t out;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const u32x4_t& u = e < 2 ? u0 : u1;
      const int w0 = (e & 1) * 2;
      const uint32_t c0 = e4m3_encode(__fdiv_rn(bf16lo(u[w0]), s));
      const uint32_t c1 = e4m3_encode(__fdiv_rn(bf16hi(u[w0]), s));
      const uint32_t c2 = e4m3_encode(__fdiv_rn(bf16lo(u[w0 + 1]), s));
      const uint32_t c3 = e4m3_encode(__fdiv_rn(bf16hi(u[w0 + 1]), s));
      out[e] = c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
    }
    st128(qr + k, out);
  }
}

}  // namespace

hipError_t launch_quantize_e4m3(const void* x, int T, int d, int ld_x, uint8_t* q, int ld_q, float* s_x,
                                hipStream_t st) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(quant_kernel, dim3((T + 3) / 4), dim3(256), 0, st, static_cast<const uint16_t*>(x), T, d,
                     ld_x, q, ld_q, s_x);
  return hipGetLastError();
}

}  // namespace lora
