// The boundary steps of an expert-parallel pipeline in their one-GPU form
// ("kimi_k3 ... ep.comm" page: EpDispatch's MXFP8 quantisation of the
// latent; EpCombine's reduce and RMSNorm, rms_rstd), with the C ABI of
// include/moe_boundary.h.
//
// Both are latency-bound (a few tokens x a few KB): one workgroup per token
// (the quantiser: 256 threads per token and 4096 columns, 16 values a lane;
// the norm: 512 threads, 8 columns a lane per pass), 16-byte loads and
// stores.
#include <hip/hip_runtime.h>

#include "../../include/moe_boundary.h"
#include "device_common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kPerLane = 16;                       // values per lane
constexpr int kCols = kThreads * kPerLane;         // columns per workgroup pass
constexpr int kMxBlock = 32;                       // values per E8M0 scale
constexpr int kE4m3Emax = 8;                       // floor(log2(448))
constexpr int kMaxRanks = 64;
constexpr int kNormThreads = 512;                  // the norm: one pass over D = 3584 at 8 columns a lane
constexpr int kNormWaves = kNormThreads / 64;
constexpr int kLoadBatch = 8;                      // partial rows requested before they are added

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// floor(log2(a)) of a finite a > 0, subnormals included.
__device__ __forceinline__ int floor_log2(float a) {
  const uint32_t u = __float_as_uint(a);
  const int e = (int)((u >> 23) & 0xFFu);
  if (e) return e - 127;
  return (31 - __builtin_clz(u & 0x7FFFFFu)) - 149;  // subnormal: m * 2^-149
}

__device__ __forceinline__ void unpack_bf16x8(const u32x4_t& w, float* v) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_value(w[i] & 0xFFFFu);
    v[2 * i + 1] = bf16_value(w[i] >> 16);
  }
}

// Lane pairs (2l, 2l + 1) share one 32-value block: each lane holds 16 values,
// both find the block max, the even lane stores the scale byte.
__global__ __launch_bounds__(kThreads) void mxfp8_quant_kernel(const uint16_t* x, int D, uint8_t* q,
                                                               uint8_t* sf) {
  const int t = blockIdx.x;
  const int col = blockIdx.y * kCols + threadIdx.x * kPerLane;
  const bool live = col < D;  // D is a multiple of 32: both lanes of a pair agree
  float v[kPerLane];
  float amax = 0.f;
  if (live) {
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(x + (size_t)t * D + col);
    unpack_bf16x8(src[0], v);
    unpack_bf16x8(src[1], v + 8);
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) amax = fmaxf(amax, fabsf(v[i]));
  }
  amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));  // every lane takes part
  if (!live) return;
  int shared = amax > 0.f ? floor_log2(amax) - kE4m3Emax : -127;
  shared = min(max(shared, -127), 127);
  u32x4_t out;
#pragma unroll
  for (int w = 0; w < 4; ++w)  // x * 2^-shared is exact; then nearest-even e4m3, saturating
    out[w] = e4m3x4_encode(ldexpf(v[4 * w], -shared), ldexpf(v[4 * w + 1], -shared),
                           ldexpf(v[4 * w + 2], -shared), ldexpf(v[4 * w + 3], -shared));
  *reinterpret_cast<u32x4_t*>(q + (size_t)t * D + col) = out;
  if ((threadIdx.x & 1) == 0) sf[(size_t)t * (D / kMxBlock) + col / kMxBlock] = (uint8_t)(shared + 127);
}

// One workgroup per token: the FP32 sum of the N partials in order (loads
// issued kLoadBatch rows ahead of the additions), rounded once to BF16 (kept
// in LDS, D values), the FP32 sum of squares (lane, wave, then the waves in
// order), rstd, and the normalised row.
__global__ __launch_bounds__(kNormThreads) void reduce_rmsnorm_kernel(const uint16_t* partials, int N, int D,
                                                                  const uint16_t* gamma, float eps,
                                                                  uint16_t* latent, uint16_t* out) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* lat = reinterpret_cast<uint16_t*>(smem);                           // [D]
  float* part = reinterpret_cast<float*>(smem + (((size_t)D * 2 + 15) & ~(size_t)15));  // [kNormWaves]
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  float sq = 0.f;
  for (int c0 = 0; c0 < D; c0 += kNormThreads * 8) {
    const int col = c0 + tid * 8;  // eight columns per lane and pass (D is a multiple of 8)
    if (col < D) {
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      const uint16_t* row = partials + (size_t)t * N * D + col;
      for (int n0 = 0; n0 < N; n0 += kLoadBatch) {
        u32x4_t w[kLoadBatch];
#pragma unroll
        for (int j = 0; j < kLoadBatch; ++j)
          if (n0 + j < N) w[j] = *reinterpret_cast<const u32x4_t*>(row + (size_t)(n0 + j) * D);
#pragma unroll
        for (int j = 0; j < kLoadBatch; ++j) {  // rank order
          if (n0 + j < N) {
            float v[8];
            unpack_bf16x8(w[j], v);
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] += v[i];
          }
        }
      }
      u32x4_t packed;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t lo = bf16_bits(acc[2 * i]), hi = bf16_bits(acc[2 * i + 1]);
        packed[i] = lo | (hi << 16);
        const float a = bf16_value(lo), b = bf16_value(hi);
        sq = fmaf(a, a, sq);
        sq = fmaf(b, b, sq);
      }
      *reinterpret_cast<u32x4_t*>(lat + col) = packed;
      if (latent) *reinterpret_cast<u32x4_t*>(latent + (size_t)t * D + col) = packed;
    }
  }
  sq = group_sum<kWave>(sq);
  if (lane == 0) part[wave] = sq;
  __syncthreads();
  float total = 0.f;
#pragma unroll
  for (int w = 0; w < kNormWaves; ++w) total += part[w];
  const float rstd = 1.0f / sqrtf(total / (float)D + eps);
  for (int c0 = 0; c0 < D; c0 += kNormThreads * 8) {
    const int col = c0 + tid * 8;
    if (col < D) {
      const u32x4_t xw = *reinterpret_cast<const u32x4_t*>(lat + col);
      const u32x4_t gw = *reinterpret_cast<const u32x4_t*>(gamma + col);
      float xv[8], gv[8];
      unpack_bf16x8(xw, xv);
      unpack_bf16x8(gw, gv);
      u32x4_t o;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        o[i] = (uint32_t)bf16_bits((xv[2 * i] * rstd) * gv[2 * i]) |
               ((uint32_t)bf16_bits((xv[2 * i + 1] * rstd) * gv[2 * i + 1]) << 16);
      *reinterpret_cast<u32x4_t*>(out + (size_t)t * D + col) = o;
    }
  }
}

}  // namespace
}  // namespace moe

extern "C" {

int moe_mxfp8_quantize(const void* x, int32_t T, int32_t D, void* q, void* sf, void* stream) {
  using namespace moe;
  if (T == 0) return MOE_DECODE_OK;  // an empty call: nothing is read or written
  if (T < 0 || !x || !q || !sf || !aligned16(x) || !aligned16(q)) return MOE_DECODE_ERR_INVALID_ARG;
  if (D <= 0 || D % kMxBlock || D > MOE_BOUNDARY_MAX_D) return MOE_DECODE_ERR_UNSUPPORTED;
  const dim3 grid(T, (D + kCols - 1) / kCols);
  hipLaunchKernelGGL(mxfp8_quant_kernel, grid, dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint16_t*>(x), D, static_cast<uint8_t*>(q), static_cast<uint8_t*>(sf));
  return hipGetLastError() == hipSuccess ? MOE_DECODE_OK : MOE_DECODE_ERR_HIP;
}

int moe_reduce_rmsnorm(const void* partials, int32_t T, int32_t N, int32_t D, const void* gamma, float eps,
                       void* latent, void* out, void* stream) {
  using namespace moe;
  if (T == 0) return MOE_DECODE_OK;
  if (T < 0 || !partials || !gamma || !out || !aligned16(partials) || !aligned16(gamma) || !aligned16(out) ||
      (latent && !aligned16(latent)) || !(eps >= 0.f) || !(eps <= 3.4e38f))
    return MOE_DECODE_ERR_INVALID_ARG;
  if (D <= 0 || D % 8 || D > MOE_BOUNDARY_MAX_D || N < 1 || N > kMaxRanks) return MOE_DECODE_ERR_UNSUPPORTED;
  const size_t lds = (((size_t)D * 2 + 15) & ~(size_t)15) + kNormWaves * sizeof(float);
  hipLaunchKernelGGL(reduce_rmsnorm_kernel, dim3(T), dim3(kNormThreads), lds, static_cast<hipStream_t>(stream),
                     static_cast<const uint16_t*>(partials), N, D, static_cast<const uint16_t*>(gamma), eps,
                     static_cast<uint16_t*>(latent), static_cast<uint16_t*>(out));
  return hipGetLastError() == hipSuccess ? MOE_DECODE_OK : MOE_DECODE_ERR_HIP;
}

}  // extern "C"
