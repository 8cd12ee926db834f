// The two small steps between and after the GEMMs.
//
// swiglu_requant: the fixed-order sum of GEMM1's split partials, the clamped
// SwiGLU and the FP8 hidden of the vLLM "mega_moe" page's hidden_block:
// up = clamp(u, -L, L), gate = min(g, L), act = gate / (1 + exp(-gate)) * up
// in FP32 operations (the exp correctly rounded), then per 128 values scale = max(amax, 1e-10) / 448 and
// q = e4m3(act / scale). Rows 0..I-1 of GEMM1 are up, I..2I-1 gate.
//
// combine: the fixed-order sum of GEMM2's split partials rounded once to the
// BF16 slot row, and combined[t] = BF16(sum_j w[t, j] * slot[t*k + j]) with
// the FP32 sum taken in pick order -- the routing weights applied once, at
// the end (nvfp4-megamoe-kernel README, slot representation).
#include "kernels.h"
#include "device_common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

// One wave per (route, 128-block of the hidden), two values per lane.
__global__ __launch_bounds__(kThreads) void swiglu_requant_kernel(SwigluArgs a) {
  const int nblk = a.I / kTile;
  const int gw = blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave;
  if (gw >= a.R * nblk) return;  // whole waves exit together
  const int lane = threadIdx.x & (kWave - 1);
  const int r = gw / nblk, c = gw - r * nblk;
  const int j = c * kTile + 2 * lane;
  const size_t row = (size_t)2 * a.I;
  float up0 = 0.f, up1 = 0.f, g0 = 0.f, g1 = 0.f;
  for (int s = 0; s < a.splits; ++s) {
    const float* p = a.part + ((size_t)s * a.R + r) * row;
    const float2 u = *reinterpret_cast<const float2*>(p + j);
    const float2 g = *reinterpret_cast<const float2*>(p + a.I + j);
    up0 += u.x;
    up1 += u.y;
    g0 += g.x;
    g1 += g.y;
  }
  const float L = a.limit;
  up0 = fminf(fmaxf(up0, -L), L);
  up1 = fminf(fmaxf(up1, -L), L);
  g0 = fminf(g0, L);
  g1 = fminf(g1, L);
  // exp rounded once to FP32 from FP64, then the add, divide and product in
  // FP32 in this order: the FP8 codes below are decided from these values.
  const float e0 = (float)exp(-(double)g0), e1 = (float)exp(-(double)g1);
  const float act0 = (g0 / (1.f + e0)) * up0;
  const float act1 = (g1 / (1.f + e1)) * up1;
  const float amax = group_max<kWave>(fmaxf(fabsf(act0), fabsf(act1)));
  const float s = fmaxf(amax, kAmaxFloor) / kFp8Max;
  const uint32_t q = e4m3_encode(act0 / s) | (e4m3_encode(act1 / s) << 8);
  *reinterpret_cast<uint16_t*>(a.hq + (size_t)r * a.I + j) = (uint16_t)q;
  if (lane == 0) a.hs[(size_t)r * nblk + c] = s;
}

// One thread per (token, 8 consecutive hidden columns).
__global__ __launch_bounds__(kThreads) void combine_kernel(CombineArgs a) {
  const int per_row = a.H / 8;
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i >= a.M * per_row) return;
  const int t = i / per_row;
  const int h0 = (i - t * per_row) * 8;
  float acc[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) acc[q] = 0.f;
  for (int j = 0; j < a.k; ++j) {
    const int r = t * a.k + j;
    float v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = 0.f;
    for (int s = 0; s < a.splits; ++s) {
      const float4_t* p =
          reinterpret_cast<const float4_t*>(a.part + ((size_t)s * (a.M * a.k) + r) * a.H + h0);
      const float4_t lo = p[0], hi = p[1];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[q] += lo[q];
        v[4 + q] += hi[q];
      }
    }
    const float w = a.weights[r];
    u32x4_t packed;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t b0 = bf16_bits(v[2 * q]), b1 = bf16_bits(v[2 * q + 1]);
      packed[q] = b0 | (b1 << 16);
      acc[2 * q] = fmaf(w, bf16_value(b0), acc[2 * q]);
      acc[2 * q + 1] = fmaf(w, bf16_value(b1), acc[2 * q + 1]);
    }
    *reinterpret_cast<u32x4_t*>(a.slots + (size_t)r * a.H + h0) = packed;
  }
  u32x4_t out;
#pragma unroll
  for (int q = 0; q < 4; ++q) out[q] = bf16_bits(acc[2 * q]) | (bf16_bits(acc[2 * q + 1]) << 16);
  *reinterpret_cast<u32x4_t*>(a.combined + (size_t)t * a.H + h0) = out;
}

}  // namespace

hipError_t launch_swiglu_requant(const SwigluArgs& a, hipStream_t s) {
  const int waves = a.R * (a.I / kTile);
  const int wpg = kThreads / kWave;
  hipLaunchKernelGGL(swiglu_requant_kernel, dim3((waves + wpg - 1) / wpg), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  const int n = a.M * (a.H / 8);
  hipLaunchKernelGGL(combine_kernel, dim3((n + kThreads - 1) / kThreads), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
