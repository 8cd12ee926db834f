// E2M1 (FP4) and UE4M3 helpers for the FP4 form of the step
// (nvfp4-megamoe-kernel README, "Data Formats" and bug 2).
#pragma once

#include "device_common.h"

namespace moe {

constexpr float kE2m1Max = 6.f;
constexpr int kFp4Group = 16;  // values per UE4M3 scale

// Nearest E2M1 code of a (sign bit 3, magnitude code 0..7 for 0, 0.5, 1,
// 1.5, 2, 3, 4, 6), ties to the even code, saturating at 6. Each comparison
// places a at or above one midpoint between neighbouring magnitudes; a
// midpoint goes up (>=) when the upper neighbour's code is even and stays
// down (>) when the lower one's is.
__device__ __forceinline__ uint32_t e2m1_encode(float a) {
  const float m = fabsf(a);
  const uint32_t c = (uint32_t)(m > 0.25f) + (uint32_t)(m >= 0.75f) + (uint32_t)(m > 1.25f) +
                     (uint32_t)(m >= 1.75f) + (uint32_t)(m > 2.5f) + (uint32_t)(m >= 3.5f) +
                     (uint32_t)(m > 5.0f);
  return c | ((__float_as_uint(a) >> 28) & 8u);
}

// Value of a UE4M3 (e4m3) byte, exact.
__device__ __forceinline__ float e4m3_value(uint32_t byte) {
  return __builtin_amdgcn_cvt_f32_fp8((int)(byte & 0xFFu), 0);
}

// One 16-value group staged to FP4: scale = e4m3(block_max / 6) (FP32
// quotient, nearest-even, saturating), codes = E2M1 of v / dec(scale), all
// zero when the stored scale is 0. Returns the scale byte; codes packed two
// per byte, element 2i in the low nibble, into packed[0..1].
__device__ __forceinline__ uint32_t stage_fp4_group(const float v[kFp4Group], uint32_t packed[2]) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < kFp4Group; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const uint32_t sbyte = e4m3x2_encode(amax / kE2m1Max, 0.f) & 0xFFu;
  const float s = e4m3_value(sbyte);
  packed[0] = packed[1] = 0u;
#pragma unroll
  for (int i = 0; i < kFp4Group; ++i) {
    const uint32_t c = s > 0.f ? e2m1_encode(v[i] / s) : 0u;
    packed[i / 8] |= c << (4 * (i % 8));
  }
  return sbyte;
}

// Two E2M1 values of byte kByte of `word` as an exact F16 pair (low nibble
// in .x). gfx950 converts packed FP4 natively; a unit scale leaves the
// values unchanged.
template <int kByte>
__device__ __forceinline__ half2_t e2m1x2_to_f16x2(uint32_t word) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, kByte);
}

}  // namespace moe
