// The SwiGLU/requant and slot/combine steps as kernels of their own (used
// when the GEMMs' last-arriver epilogues are switched off). The arithmetic
// lives in epilogue_device.h.
#include "epilogue_device.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

// One wave per (route, 128-block of the hidden).
__global__ __launch_bounds__(kThreads) void swiglu_requant_kernel(SwigluArgs a) {
  const int nblk = a.I / kTile;
  const int gw = blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave;
  if (gw >= a.R * nblk) return;  // whole waves exit together
  swiglu_route_block(a, gw / nblk, gw % nblk, threadIdx.x & (kWave - 1));
}

// One workgroup per (token, 64 hidden columns).
__global__ __launch_bounds__(kThreads) void combine_kernel(CombineArgs a) {
  __shared__ float lds[kMaxTopK * 64];
  const int tiles = a.H / 64;
  combine_token_tile(a, blockIdx.x / tiles, (blockIdx.x % tiles) * 64, lds);
}

}  // namespace

hipError_t launch_swiglu_requant(const SwigluArgs& a, hipStream_t s) {
  const int waves = a.R * (a.I / kTile);
  const int wpg = kThreads / kWave;
  hipLaunchKernelGGL(swiglu_requant_kernel, dim3((waves + wpg - 1) / wpg), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(combine_kernel, dim3(a.M * (a.H / 64)), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
