// The SwiGLU/requant and slot/combine steps, each one launch that also covers
// the shared expert when there is one; the arithmetic lives in
// epilogue_device.h. Also the one-time conversion of packed UE8M0 scales.
#include <algorithm>

#include "epilogue_device.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

// One wave per (route, 128-block of the hidden), then one per (token,
// 128-block of the shared hidden).
__global__ __launch_bounds__(kThreads) void swiglu_requant_kernel(SwigluArgs a) {
  // every line of the argument block under one wait (the ids pointer sits in
  // the last): read at first use, a line costs a memory round trip
  asm volatile("" ::"s"(a.part), "s"(a.sue8m0), "s"(a.ids));
  const int nblk = a.I / kTile;
  const int gw = blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int routed = a.R * nblk;
  if (gw < routed) {
    const int r = gw / nblk, c = gw % nblk;
    if (a.fp4) {
      const int e = a.ids[r] - a.lb;
      if (e < 0 || e >= a.lc) return;  // a route of another GPU's expert: nothing to compute
      swiglu_fp4_block(a, r, c, lane);
      return;
    }
    // the first split is read beside the expert id, not after it (its row
    // exists for every route; a route of another GPU's expert drops it)
    const float4 first = swiglu_split(a, r, c, lane, 0);
    const int e = a.ids[r] - a.lb;
    asm volatile("" ::"v"(first.x), "v"(first.y), "v"(first.z), "v"(first.w));  // keeps the read above the exit
    if (e < 0 || e >= a.lc) return;
    swiglu_route_block(a, r, c, lane, first);
    return;
  }
  if (!a.spart) return;
  const int sblk = a.Is / kTile;
  const int w = gw - routed;
  if (w >= a.M * sblk) return;  // whole waves exit together
  swiglu_shared_block(a, w / sblk, w % sblk, lane);
}

// Thread per (row n, K group g): the biased exponent byte of the packed word
// becomes the FP32 scale 2^(byte - 127) (bits byte << 23) of block
// (n / 128, g); every row must carry its block's first row's byte.
__global__ void unpack_ue8m0_kernel(const int32_t* packed, int n, int k, float* out, int32_t* bad) {
  const int groups = k / kTile, words = (groups + 3) / 4;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n * groups) return;
  const int row = i / groups, g = i - row * groups;
  const int lead = row - row % kTile;
  const uint32_t e = ((uint32_t)packed[(size_t)row * words + g / 4] >> (8 * (g % 4))) & 0xFFu;
  const uint32_t e0 = ((uint32_t)packed[(size_t)lead * words + g / 4] >> (8 * (g % 4))) & 0xFFu;
  if (e != e0) atomicOr(bad, 1);
  if (row == lead) out[(size_t)(row / kTile) * groups + g] = __uint_as_float(e << 23);
}

__global__ void zero_words_kernel(int32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

// One workgroup per (token, 64 hidden columns).
__global__ __launch_bounds__(kThreads) void combine_kernel(CombineArgs a) {
  __shared__ float lds[kMaxTopK * 64];
  const int tiles = a.H / 64;
  combine_token_tile(a, blockIdx.x / tiles, (blockIdx.x % tiles) * 64, lds);
}

}  // namespace

hipError_t launch_swiglu_requant(const SwigluArgs& a, hipStream_t s, KernelEvents ev) {
  const int waves = a.R * (a.I / kTile) + (a.spart ? a.M * (a.Is / kTile) : 0);
  const int wpg = kThreads / kWave;
  hipExtLaunchKernelGGL(swiglu_requant_kernel, dim3((waves + wpg - 1) / wpg), dim3(kThreads), 0, s,
                        ev.start, ev.stop, 0, a);
  return hipGetLastError();
}

hipError_t launch_zero_words(int32_t* p, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const unsigned blocks = (unsigned)std::min<size_t>((n + 255) / 256, 1024);
  hipLaunchKernelGGL(zero_words_kernel, dim3(blocks), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s, KernelEvents ev) {
  hipExtLaunchKernelGGL(combine_kernel, dim3(a.M * (a.H / 64)), dim3(kThreads), 0, s,
                        ev.start, ev.stop, 0, a);
  return hipGetLastError();
}

hipError_t launch_unpack_ue8m0(const int32_t* packed, int n, int k, float* out, int32_t* bad,
                               hipStream_t s) {
  const int items = n * (k / kTile);
  hipLaunchKernelGGL(unpack_ue8m0_kernel, dim3((items + 255) / 256), dim3(256), 0, s, packed, n, k, out,
                     bad);
  return hipGetLastError();
}

}  // namespace moe
