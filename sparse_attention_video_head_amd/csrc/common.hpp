// Device helpers shared by the SVG2 HIP kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace svg2 {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }
// round-to-nearest-even conversion (v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(uint16_t, h);
}
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// two floats -> two bf16 (RNE) in one word: one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// element loaders: T is float or uint16_t (bf16 storage)
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float get(const float* p, size_t i) { return p[i]; }
};
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ float get(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
};

// ---------------------------------------------------------------- wave ops
__device__ __forceinline__ int lane_id() { return __lane_id(); }

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}
template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmax(v, __shfl_xor(v, m));
  return v;
}
// inclusive prefix sum over the 64 lanes (fixed order: Hillis-Steele)
template <typename T>
__device__ __forceinline__ T wave_inclusive_scan(T v) {
  const int l = lane_id();
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    T u = __shfl_up(v, o);
    if (l >= o) v += u;
  }
  return v;
}

// Exclusive prefix sum over a whole work-group (blockDim.x a multiple of 64,
// at most 1024 threads).  `scratch` holds >= 17 T in LDS.  Also returns the
// group total through *total.  Contains __syncthreads.
template <typename T>
__device__ T block_exclusive_scan(T v, T* scratch, T* total) {
  const int l = lane_id();
  const int w = threadIdx.x / kWave;
  const int nw = blockDim.x / kWave;
  T inc = wave_inclusive_scan(v);
  __syncthreads();
  if (l == kWave - 1) scratch[w] = inc;
  __syncthreads();
  if (w == 0) {
    T s = (l < nw) ? scratch[l] : T(0);
    T si = wave_inclusive_scan(s);
    if (l < nw) scratch[l] = si - s;           // exclusive over waves
    if (l == nw - 1) scratch[16] = si;
  }
  __syncthreads();
  T res = scratch[w] + inc - v;
  *total = scratch[16];
  __syncthreads();
  return res;
}

template <typename T>
__device__ T block_sum(T v, T* scratch) {
  T t;
  (void)block_exclusive_scan(v, scratch, &t);
  return t;
}

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// OCP E4M3 with one scale per problem: scale = max|x| / 448 dequantizes,
// r = 448 / max|x| quantizes (both correctly rounded fp32, 1 for an all-zero
// problem); x8 = E4M3(x * r), the product in fp32 clamped to +-448 and the
// conversion round-to-nearest-even.  amax_bits: max|x| as float bits.
constexpr float kE4M3Max = 448.f;

__device__ __forceinline__ float quant_scale(uint32_t amax_bits) {
  const float a = __uint_as_float(amax_bits);
  return a > 0.f ? a / kE4M3Max : 1.f;
}

__device__ __forceinline__ float quant_ratio(uint32_t amax_bits) {
  const float a = __uint_as_float(amax_bits);
  return a > 0.f ? kE4M3Max / a : 1.f;
}

__device__ __forceinline__ float quant_mul(float v, float r) {
  return fminf(fmaxf(v * r, -kE4M3Max), kE4M3Max);
}

// 8 bf16 values (16 bytes) -> 8 E4M3 bytes
__device__ __forceinline__ uint2 quant8_bf16(const u32x4_t& v, float r) {
  int lo = 0, hi = 0;
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(quant_mul(bf16_lo(v[0]), r), quant_mul(bf16_hi(v[0]), r), lo, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(quant_mul(bf16_lo(v[1]), r), quant_mul(bf16_hi(v[1]), r), lo, true);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(quant_mul(bf16_lo(v[2]), r), quant_mul(bf16_hi(v[2]), r), hi, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(quant_mul(bf16_lo(v[3]), r), quant_mul(bf16_hi(v[3]), r), hi, true);
  uint2 w;
  w.x = (uint32_t)lo;
  w.y = (uint32_t)hi;
  return w;
}

}  // namespace svg2
