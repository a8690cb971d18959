// FP8 (OCP E4M3) copies of bf16 tensors with one scale per problem, for the
// FP8 attention kernel (the project README's open-source plan, "Support FP8
// attention").  scale = max|x| / 448 for the dequantization and
// r = 448 / max|x| (both correctly rounded fp32; 1 for an all-zero problem);
// x8 = E4M3(x * r), the product in fp32 clamped to +-448 and the conversion
// round-to-nearest-even.
#include <math.h>

#include "common.hpp"
#include "internal.hpp"

namespace svg2 {

constexpr int kQuantThreads = 256;
constexpr int kQuantVec = 8;                     // bf16 elements per 16-byte load
constexpr int kQuantUnroll = 4;
constexpr int kQuantPerWG = kQuantThreads * kQuantVec * kQuantUnroll;

__global__ void k_quant_zero(uint32_t* amax, int bh) {
  const int p = blockIdx.x * blockDim.x + threadIdx.x;
  if (p < bh) amax[p] = 0u;
}

// max |x| per problem: non-negative floats order like their bit patterns, so
// an unsigned atomic max of the bits is exact and order-independent.  Each
// work-group covers kAmaxSub blocks of kQuantPerWG elements and issues one
// atomic: atomics on one address are served one at a time, so there are few.
constexpr int kAmaxSub = 16;

__global__ __launch_bounds__(kQuantThreads) void k_quant_amax(const uint16_t* __restrict__ x, size_t per_problem,
                                                              uint32_t* __restrict__ amax) {
  __shared__ float s_red[17];
  const int p = blockIdx.y;
  const uint16_t* xp = x + (size_t)p * per_problem;
  float m = 0.f;
  for (int sb = 0; sb < kAmaxSub; ++sb) {
    const size_t base = ((size_t)blockIdx.x * kAmaxSub + sb) * kQuantPerWG;
    if (base >= per_problem) break;
#pragma unroll
    for (int u = 0; u < kQuantUnroll; ++u) {
      const size_t e = base + ((size_t)u * kQuantThreads + threadIdx.x) * kQuantVec;
      if (e + kQuantVec <= per_problem) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(xp + e);
#pragma unroll
        for (int w = 0; w < 4; ++w) m = fmaxf(m, fmaxf(fabsf(bf16_lo(v[w])), fabsf(bf16_hi(v[w]))));
      } else {
        for (size_t i = e; i < per_problem && i < e + kQuantVec; ++i)
          m = fmaxf(m, fabsf(__uint_as_float((uint32_t)xp[i] << 16)));
      }
    }
  }
  m = wave_max(m);
  if (lane_id() == 0) s_red[threadIdx.x / kWave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float b = 0.f;
    for (int w = 0; w < kQuantThreads / kWave; ++w) b = fmaxf(b, s_red[w]);
    atomicMax(&amax[p], __float_as_uint(b));
  }
}

__global__ __launch_bounds__(kQuantThreads) void k_quant_fp8(const uint16_t* __restrict__ x, size_t per_problem,
                                                             const uint32_t* __restrict__ amax,
                                                             uint8_t* __restrict__ x8, float* __restrict__ scale) {
  const int p = blockIdx.y;
  const float s = quant_ratio(amax[p]);
  if (blockIdx.x == 0 && threadIdx.x == 0) scale[p] = quant_scale(amax[p]);
  const uint16_t* xp = x + (size_t)p * per_problem;
  uint8_t* op = x8 + (size_t)p * per_problem;
  const size_t base = (size_t)blockIdx.x * kQuantPerWG;
#pragma unroll
  for (int u = 0; u < kQuantUnroll; ++u) {
    const size_t e = base + ((size_t)u * kQuantThreads + threadIdx.x) * kQuantVec;
    if (e + kQuantVec <= per_problem) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(xp + e);
      *reinterpret_cast<uint2*>(op + e) = quant8_bf16(v, s);
    } else {
      for (size_t i = e; i < per_problem && i < e + kQuantVec; ++i) {
        const float f = quant_mul(__uint_as_float((uint32_t)xp[i] << 16), s);
        op[i] = (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(f, 0.f, 0, false) & 0xff);
      }
    }
  }
}

hipError_t launch_amax_bf16(const void* x, int bh, int N, int d, uint32_t* amax_ws, hipStream_t s) {
  const size_t per = (size_t)N * d;
  const size_t per_wg = (size_t)kQuantPerWG * kAmaxSub;
  const dim3 grid((unsigned)((per + per_wg - 1) / per_wg), bh);
  hipLaunchKernelGGL(k_quant_zero, dim3((bh + 255) / 256), dim3(256), 0, s, amax_ws, bh);
  hipLaunchKernelGGL(k_quant_amax, grid, dim3(kQuantThreads), 0, s, static_cast<const uint16_t*>(x), per, amax_ws);
  return hipGetLastError();
}

hipError_t launch_quantize_fp8(const void* x, int bh, int N, int d, uint8_t* x8, float* scale, uint32_t* amax_ws,
                               hipStream_t s) {
  const size_t per = (size_t)N * d;
  const dim3 grid((unsigned)((per + kQuantPerWG - 1) / kQuantPerWG), bh);
  if (const hipError_t e = launch_amax_bf16(x, bh, N, d, amax_ws, s); e != hipSuccess) return e;
  hipLaunchKernelGGL(k_quant_fp8, grid, dim3(kQuantThreads), 0, s, static_cast<const uint16_t*>(x), per, amax_ws,
                     x8, scale);
  return hipGetLastError();
}

}  // namespace svg2
