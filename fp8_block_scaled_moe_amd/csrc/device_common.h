// Device helpers shared by the kernels: number formats and wavefront
// reductions for gfx950 (wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {


constexpr float kFp8Max = 448.f;    // largest finite OCP e4m3 magnitude
constexpr float kAmaxFloor = 1e-10f;
constexpr int kWave = 64;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef int int8v_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// OCP e4m3 bytes of four values, nearest with ties to the even mantissa,
// saturating to +-448, packed low byte first. Clamping to +-448 first and
// then rounding to nearest-even gives exactly the saturating rounding for
// finite inputs; gfx950 converts FP32 pairs to OCP e4m3 natively (round to
// nearest even in the default mode).
__device__ __forceinline__ uint32_t e4m3x4_encode(float a, float b, float c, float d) {
  a = __builtin_amdgcn_fmed3f(a, -kFp8Max, kFp8Max);
  b = __builtin_amdgcn_fmed3f(b, -kFp8Max, kFp8Max);
  c = __builtin_amdgcn_fmed3f(c, -kFp8Max, kFp8Max);
  d = __builtin_amdgcn_fmed3f(d, -kFp8Max, kFp8Max);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

__device__ __forceinline__ uint32_t e4m3x2_encode(float a, float b) {
  a = __builtin_amdgcn_fmed3f(a, -kFp8Max, kFp8Max);
  b = __builtin_amdgcn_fmed3f(b, -kFp8Max, kFp8Max);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// Two e4m3 bytes of `word` (bytes 0,1 when hi == false, bytes 2,3 when true)
// as an exact F16 pair, low byte in .x. gfx950 converts OCP e4m3 natively;
// a unit scale leaves the values unchanged.
template <bool kHi>
__device__ __forceinline__ half2_t e4m3x2_to_f16x2(uint32_t word) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(word, 1.0f, kHi);
}

__device__ __forceinline__ uint16_t bf16_bits(float f) {  // nearest-even, finite f
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_value(uint32_t b) { return __uint_as_float(b << 16); }

template <int W>
__device__ __forceinline__ float group_max(float v) {  // max over aligned groups of W lanes
#pragma unroll
  for (int o = 1; o < W; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

template <int W>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = 1; o < W; o <<= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint64_t w = __shfl_xor(v, o, kWave);
    v = w > v ? w : v;
  }
  return v;
}

// Nontemporal 16-byte load of streamed weights (read once per call).
__device__ __forceinline__ u32x4_t load_stream16(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

}  // namespace moe
