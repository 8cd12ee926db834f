// Device pieces shared by the GEMM kernels: problem selection within a launch
// and the F16 MFMA step over one 128-K block.
#pragma once

#include "kernels.h"
#include "device_common.h"

namespace moe {

// The problem this workgroup works on (the dense problem's units come first)
// and its unit index within that problem.
__device__ __forceinline__ GemmProblem select_problem(const GemmArgs& a, int& unit) {
  const bool dense = (int)blockIdx.x < a.units0;
  unit = dense ? (int)blockIdx.x : (int)blockIdx.x - a.units0;
  return dense ? a.p[0] : a.p[1];
}

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));

// A wave's 16 x 128-byte weight block passes through a private LDS tile from
// the load layout (eight lanes per row, 16 B each) into the MFMA layout; the
// row stride of 144 B keeps both the writes and the reads free of bank
// conflicts.
constexpr int kTileStride = kTile + 16;
constexpr int kTileBytes = 16 * kTileStride;

__device__ __forceinline__ half8_t widen8(uint32_t w0, uint32_t w1) {
  const half2_t a = e4m3x2_to_f16x2<false>(w0), b = e4m3x2_to_f16x2<true>(w0);
  const half2_t c = e4m3x2_to_f16x2<false>(w1), d = e4m3x2_to_f16x2<true>(w1);
  return half8_t{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

// Orders this wave's LDS accesses around the tile exchange (a wave's LDS
// operations complete in order; this keeps the compiler from moving them).
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
}

// The 16 rows x 16 routes partial of one 128-K block, exact products summed
// in FP32 by four v_mfma_f32_16x16x32_f16. Lane l (row or route l % 16,
// g = l / 16) supplies bytes 16g..16g+15 (wlo, xlo) and 64+16g..64+16g+15
// (whi, xhi) of its row's and its route's block, so each of the 128 products
// enters exactly once. Result: lane l holds route l % 16, rows 4g..4g+3.
__device__ __forceinline__ float4_t mfma_block(const u32x4_t& wlo, const u32x4_t& whi, const u32x4_t& xlo,
                                               const u32x4_t& xhi) {
  const float4_t zero = {0.f, 0.f, 0.f, 0.f};
  float4_t p = __builtin_amdgcn_mfma_f32_16x16x32_f16(widen8(wlo[0], wlo[1]), widen8(xlo[0], xlo[1]), zero, 0,
                                                      0, 0);
  p = __builtin_amdgcn_mfma_f32_16x16x32_f16(widen8(wlo[2], wlo[3]), widen8(xlo[2], xlo[3]), p, 0, 0, 0);
  p = __builtin_amdgcn_mfma_f32_16x16x32_f16(widen8(whi[0], whi[1]), widen8(xhi[0], xhi[1]), p, 0, 0, 0);
  p = __builtin_amdgcn_mfma_f32_16x16x32_f16(widen8(whi[2], whi[3]), widen8(xhi[2], xhi[3]), p, 0, 0, 0);
  return p;
}

}  // namespace moe
