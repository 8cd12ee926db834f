// Device bodies of the two small steps around the GEMMs, launched by the
// kernels of epilogues.hip.
#pragma once

#include "kernels.h"
#include "device_common.h"
#include "fp4_device.h"
#include "stream_device.h"

namespace moe {

__device__ __forceinline__ float bf16_round(float v) { return bf16_value(bf16_bits(v)); }

// One wave: the clamped SwiGLU and the FP8 hidden block of route r, columns
// 128c + 2 lane and + 1, from the GEMM1 sums of its up and gate rows (vLLM
// "mega_moe" page, hidden_block): up = clamp(u, -L, L), gate = min(g, L),
// act = (gate / (1 + exp(-gate))) * up in FP32 operations with the exp
// correctly rounded, scale = max(amax, 1e-10) / 448 over the wave's 128
// values, q = e4m3(act / scale). Used by the separate kernel and by the
// GEMM1 launch that finishes the step itself.
__device__ __forceinline__ void swiglu_finish(float up0, float up1, float g0, float g1, float L, int I,
                                              uint8_t* hq, float* hs, int r, int c, int lane) {
  const int nblk = I / kTile;
  const int j = c * kTile + 2 * lane;
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
  const uint32_t q = e4m3x2_encode(act0 / s, act1 / s);
  *reinterpret_cast<uint16_t*>(hq + (size_t)r * I + j) = (uint16_t)q;
  if (lane == 0) hs[(size_t)r * nblk + c] = s;
}

// Split s of GEMM1's partials for route r, 128-block c of the hidden, this
// lane's two columns: (up, up, gate, gate). Rows 0..I-1 of GEMM1 are up,
// I..2I-1 gate.
__device__ __forceinline__ float4 swiglu_split(const SwigluArgs& a, int r, int c, int lane, int s) {
  const int j = c * kTile + 2 * lane;
  const float* p = a.part + ((size_t)s * a.R + r) * (size_t)(2 * a.I);
  const float2 u = *reinterpret_cast<const float2*>(p + j);
  const float2 g = *reinterpret_cast<const float2*>(p + a.I + j);
  return make_float4(u.x, u.y, g.x, g.y);
}

// One wave: route r, 128-block c of the hidden, from the fixed-order sum of
// GEMM1's split partials; `first` is split 0, read by the caller.
__device__ __forceinline__ void swiglu_route_block(const SwigluArgs& a, int r, int c, int lane, float4 first) {
  float up0 = 0.f + first.x, up1 = 0.f + first.y, g0 = 0.f + first.z, g1 = 0.f + first.w;
#pragma unroll 4
  for (int s = 1; s < a.splits; ++s) {
    const float4 v = swiglu_split(a, r, c, lane, s);
    up0 += v.x;
    up1 += v.y;
    g0 += v.z;
    g1 += v.w;
  }
  swiglu_finish(up0, up1, g0, g1, a.limit, a.I, a.hq, a.hs, r, c, lane);
}

// One wave, shared expert ("shared_expert" page, _DownKernel and
// _group_scale): token t, 128-block c of the shared hidden. gate/up are the
// fixed-order split sums rounded to BF16 (rows 0..Is-1 gate, Is..2Is-1 up);
// gate = min(gate, L), up = clamp(up, -L, L), silu = gate / (1 + exp(-gate))
// in FP32 steps (exp correctly rounded), act = BF16(silu * up); per 128,
// scale = max(amax, 1e-10) / 448, rounded up to a power of two with UE8M0,
// q = e4m3(act * (1 / scale)).
__device__ __forceinline__ void swiglu_shared_block(const SwigluArgs& a, int t, int c, int lane) {
  const int nblk = a.Is / kTile;
  const int j = c * kTile + 2 * lane;
  const size_t row = (size_t)2 * a.Is;
  float g0 = 0.f, g1 = 0.f, up0 = 0.f, up1 = 0.f;
#pragma unroll 4
  for (int s = 0; s < a.ssplits; ++s) {
    const float* p = a.spart + ((size_t)s * a.M + t) * row;
    const float2 g = *reinterpret_cast<const float2*>(p + j);
    const float2 u = *reinterpret_cast<const float2*>(p + a.Is + j);
    g0 += g.x;
    g1 += g.y;
    up0 += u.x;
    up1 += u.y;
  }
  const float L = a.slimit;
  g0 = fminf(bf16_round(g0), L);
  g1 = fminf(bf16_round(g1), L);
  up0 = fminf(fmaxf(bf16_round(up0), -L), L);
  up1 = fminf(fmaxf(bf16_round(up1), -L), L);
  const float e0 = (float)exp(-(double)g0), e1 = (float)exp(-(double)g1);
  const float act0 = bf16_round((g0 / (1.f + e0)) * up0);
  const float act1 = bf16_round((g1 / (1.f + e1)) * up1);
  const float amax = group_max<kWave>(fmaxf(fabsf(act0), fabsf(act1)));
  float s = fmaxf(amax, kAmaxFloor) / kFp8Max;
  if (a.sue8m0) {
    const uint32_t b = __float_as_uint(fmaxf(s, kAmaxFloor));
    s = __uint_as_float(((b >> 23) + ((b & 0x7FFFFFu) != 0u)) << 23);
  }
  const float inv = 1.f / s;
  const uint32_t q = e4m3x2_encode(act0 * inv, act1 * inv);
  *reinterpret_cast<uint16_t*>(a.shq + (size_t)t * a.Is + j) = (uint16_t)q;
  if (lane == 0) a.shs[(size_t)t * nblk + c] = s;
}

// The FP32 total of the stream partials of row n for route r (slot order),
// over columns n and n + 1 (the same tile), written back to slot 0 so that
// slot 0 holds the GEMM's output afterwards.
__device__ __forceinline__ float2 stream_total2(const StreamDesc& d, float* part, int R, int N, int r, int n) {
  const int slots = stream_slots(d, r, n);
  float2 v = {0.f, 0.f};
  for (int s = 0; s < slots; ++s) {
    const float2 p = *reinterpret_cast<const float2*>(part + ((size_t)s * R + r) * N + n);
    v.x += p.x;
    v.y += p.y;
  }
  if (slots > 1) *reinterpret_cast<float2*>(part + (size_t)r * N + n) = v;
  return v;
}

// One wave, FP4 form (nvfp4-megamoe-kernel README: SiLU times up per slot,
// then the activation staged to E2M1 for L2): route r, columns
// [128c, 128c + 128) of the hidden, two per lane. gate/up are GEMM1's FP32
// sums (stream partials added in slot order) rounded to BF16 (gate rows
// first); gate = min(gate, L), up = clamp(up, -L, L); act = BF16(gate /
// (1 + exp(-gate)) * up) in FP32 steps with the exp correctly rounded; then
// per 16 values (eight lanes) the E2M1 codes and the UE4M3 scale.
__device__ __forceinline__ void swiglu_fp4_block(const SwigluArgs& a, int r, int c, int lane) {
  const int j = c * kTile + 2 * lane;
  float* part = const_cast<float*>(a.part);
  const float2 g = stream_total2(a.stream, part, a.R, 2 * a.I, r, j);
  const float2 u = stream_total2(a.stream, part, a.R, 2 * a.I, r, a.I + j);
  const float L = a.limit;
  const float g0 = fminf(bf16_round(g.x), L), g1 = fminf(bf16_round(g.y), L);
  const float u0 = fminf(fmaxf(bf16_round(u.x), -L), L), u1 = fminf(fmaxf(bf16_round(u.y), -L), L);
  const float e0 = (float)exp(-(double)g0), e1 = (float)exp(-(double)g1);
  const float act0 = bf16_round((g0 / (1.f + e0)) * u0);
  const float act1 = bf16_round((g1 / (1.f + e1)) * u1);
  const float amax = group_max<8>(fmaxf(fabsf(act0), fabsf(act1)));
  const uint32_t sbyte = e4m3x2_encode(amax / kE2m1Max, 0.f) & 0xFFu;
  const float s = e4m3_value(sbyte);
  const uint32_t q0 = s > 0.f ? e2m1_encode(act0 / s) : 0u;
  const uint32_t q1 = s > 0.f ? e2m1_encode(act1 / s) : 0u;
  a.hq[((size_t)r * a.I + j) / 2] = (uint8_t)(q0 | (q1 << 4));
  if ((lane & 7) == 0) a.hs4[((size_t)r * a.I + j) / kFp4Group] = (uint8_t)sbyte;
}

// The whole workgroup (256 threads): token t, hidden columns
// [col0, col0 + 64). Each slot value is the fixed-order sum of GEMM2's split
// partials rounded once to BF16; combined = BF16(sum_j w[t, j] * slot_j) with
// the FP32 sum in pick order -- the routing weights applied once, at the end
// (nvfp4-megamoe-kernel README, slot representation). Slots whose expert is
// not local are zero and add nothing. With a shared expert, the otherwise
// idle second wave writes its BF16 output for the same columns. `lds` holds
// k * 64 floats. Contains a barrier: every thread of the workgroup must call
// it.
__device__ __forceinline__ void combine_token_tile(const CombineArgs& a, int t, int col0, float* lds) {
  const int tid = threadIdx.x;
  const int c = tid & 63, jg = tid >> 6;
  const int R = a.M * a.k;
  for (int j = jg; j < a.k; j += 4) {
    const int r = t * a.k + j;
    const int e = a.ids[r] - a.lb;
    float v = 0.f;  // non-local experts: a zero slot, nothing added below
    if (e >= 0 && e < a.lc) {
      const int splits = a.fp4 ? stream_slots(a.stream, r, col0 + c) : a.splits;
#pragma unroll 4
      for (int s = 0; s < splits; ++s) v += a.part[((size_t)s * R + r) * a.H + col0 + c];
    }
    const uint32_t b = bf16_bits(v);
    a.slots[(size_t)r * a.H + col0 + c] = (uint16_t)b;
    lds[j * 64 + c] = bf16_value(b);
  }
  __syncthreads();
  if (tid < 64) {
    float acc = 0.f;
    for (int j = 0; j < a.k; ++j) acc = fmaf(a.weights[(size_t)t * a.k + j], lds[j * 64 + c], acc);
    a.combined[(size_t)t * a.H + col0 + c] = (uint16_t)bf16_bits(acc);
  } else if (tid < 128 && a.spart) {
    // the shared expert's output: fixed-order split sum rounded once to BF16
    float v = 0.f;
    for (int s = 0; s < a.ssplits; ++s) v += a.spart[((size_t)s * a.M + t) * a.H + col0 + c];
    a.shared_out[(size_t)t * a.H + col0 + c] = (uint16_t)bf16_bits(v);
  }
}

}  // namespace moe
