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

// OCP e4m3 byte nearest to v, ties to the even mantissa, magnitudes at or
// beyond the 448/480 midpoint saturating to 448 (0x7E). Finite inputs only.
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  const uint32_t bits = __float_as_uint(v);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const float a = fabsf(v);
  if (!(a < 464.f)) return sign | 0x7Eu;
  int binade = (int)((bits >> 23) & 0xFFu) - 127;  // exponent of a (f32 subnormals read -127)
  int E = binade < -6 ? -6 : binade;                // below 2^-6 the grid is 2^-9
  int q = (int)rintf(ldexpf(a, 3 - E));             // exact scaling, ties-to-even round
  if (q >= 16) { E += 1; q = 8; }                   // rounded into the next binade
  const uint32_t code = q >= 8 ? (uint32_t)(((E + 7) << 3) | (q - 8)) : (uint32_t)q;
  return sign | code;
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
