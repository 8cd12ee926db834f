// Block-scaled FP8 GEMM over the touched experts, split-K, weight streaming.
//
// The pages' kernel (vLLM "mega_moe" page, module docstring) keeps each
// 128-K block's unscaled partial apart because the FP32 block scales are not
// powers of two and cannot ride inside the matrix instruction; the epilogue
// scales and sums the blocks once. The same rule holds here: every partial
// over one 128-K block is multiplied by (weight scale x activation scale) of
// that block before it joins the running FP32 sum.
//
// Work unit = (distinct expert, 64 weight rows, one K split). Each of the four
// waves of a workgroup owns 16 rows. A touched expert's weights are read once
// for all of its routes (up to 8 or 16 per pass); untouched experts are never
// read. The grid is sized for the largest possible number of distinct
// experts; workgroups past the actual count exit at once, so no host
// synchronisation is needed.
#include "kernels.h"
#include "device_common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kPrefetch = 4;  // 128-K blocks of weights in flight per wave

struct Unit {
  int e, cnt, off, tile, split, kb0, nb;
};

__device__ __forceinline__ bool decode_unit(const GemmArgs& a, Unit& u) {
  const int U = a.b.ctrl[1];
  const int per_expert = a.tiles * a.splits;
  const int unit = blockIdx.x;
  if (unit >= U * per_expert) return false;
  const int ui = unit / per_expert;
  const int rem = unit - ui * per_expert;
  u.tile = rem / a.splits;
  u.split = rem - u.tile * a.splits;
  u.e = a.b.uexp[ui];
  u.cnt = a.b.ucnt[ui];
  u.off = a.b.uoff[ui];
  u.kb0 = u.split * a.ks;
  u.nb = min(a.ks, a.nkb - u.kb0);
  return true;
}

// ---------------------------------------------------------------------------
// VALU inner product: lane (8 per row, 16 bytes each) holds one 128-byte
// block of two rows; e4m3 pairs widen exactly to F16 pairs and v_dot2 adds
// two exact products into FP32.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void gemm_valu_kernel(GemmArgs a) {
  __shared__ __align__(16) _Float16 xh[kValuRoutes * kMaxKs * kTile];
  __shared__ float sc[kValuRoutes * kMaxKs];
  __shared__ int rts[kValuRoutes];

  Unit u;
  if (!decode_unit(a, u)) return;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int rg = lane >> 3, ch = lane & 7;
  const int row_a = u.tile * kRowsPerWg + wave * 16 + rg;
  const uint8_t* pa = a.w + ((size_t)u.e * a.N + row_a) * a.K + (size_t)u.kb0 * kTile + ch * 16;
  const uint8_t* pb = pa + (size_t)8 * a.K;
  const float* wsr =
      a.ws + ((size_t)u.e * (a.N / kTile) + (u.tile * kRowsPerWg) / kTile) * a.nkb + u.kb0;

  for (int c0 = 0; c0 < u.cnt; c0 += kValuRoutes) {
    const int nr = min(kValuRoutes, u.cnt - c0);
    if (c0) __syncthreads();
    if (tid < nr) rts[tid] = a.b.routes[u.off + c0 + tid];
    __syncthreads();
    // Stage the routes' activations for this split as exact F16, and the
    // per-block products of the two scales.
    const int chunks = nr * u.nb * 16;  // 8-byte chunks
    for (int i = tid; i < chunks; i += kThreads) {
      const int r = i / (u.nb * 16), rem = i - r * (u.nb * 16);
      const size_t row = (size_t)(rts[r] / a.act_div);
      const uint2 v = *reinterpret_cast<const uint2*>(a.aq + row * a.K + (size_t)u.kb0 * kTile + rem * 8);
      half2_t* dst = reinterpret_cast<half2_t*>(&xh[r * kMaxKs * kTile + rem * 8]);
      dst[0] = e4m3x2_to_f16x2<false>(v.x);
      dst[1] = e4m3x2_to_f16x2<true>(v.x);
      dst[2] = e4m3x2_to_f16x2<false>(v.y);
      dst[3] = e4m3x2_to_f16x2<true>(v.y);
    }
    for (int i = tid; i < nr * u.nb; i += kThreads) {
      const int r = i / u.nb, b = i - r * u.nb;
      const size_t row = (size_t)(rts[r] / a.act_div);
      sc[r * kMaxKs + b] = wsr[b] * a.as[row * a.nkb + u.kb0 + b];
    }
    __syncthreads();

    float acc_a[kValuRoutes], acc_b[kValuRoutes];
#pragma unroll
    for (int i = 0; i < kValuRoutes; ++i) acc_a[i] = acc_b[i] = 0.f;

    u32x4_t na[kPrefetch], nb_[kPrefetch];
#pragma unroll
    for (int q = 0; q < kPrefetch; ++q) {
      if (q < u.nb) {
        na[q] = load_stream16(pa + q * kTile);
        nb_[q] = load_stream16(pb + q * kTile);
      }
    }
    for (int b0 = 0; b0 < u.nb; b0 += kPrefetch) {
      u32x4_t ca[kPrefetch], cb[kPrefetch];
#pragma unroll
      for (int q = 0; q < kPrefetch; ++q) {
        ca[q] = na[q];
        cb[q] = nb_[q];
      }
#pragma unroll
      for (int q = 0; q < kPrefetch; ++q) {
        const int b = b0 + kPrefetch + q;
        if (b < u.nb) {
          na[q] = load_stream16(pa + (size_t)b * kTile);
          nb_[q] = load_stream16(pb + (size_t)b * kTile);
        }
      }
#pragma unroll
      for (int q = 0; q < kPrefetch; ++q) {
        const int b = b0 + q;
        if (b < u.nb) {
          half2_t wa[8], wb[8];
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            wa[2 * d] = e4m3x2_to_f16x2<false>(ca[q][d]);
            wa[2 * d + 1] = e4m3x2_to_f16x2<true>(ca[q][d]);
            wb[2 * d] = e4m3x2_to_f16x2<false>(cb[q][d]);
            wb[2 * d + 1] = e4m3x2_to_f16x2<true>(cb[q][d]);
          }
#pragma unroll
          for (int i = 0; i < kValuRoutes; ++i) {
            if (i < nr) {
              const half2_t* xp =
                  reinterpret_cast<const half2_t*>(&xh[i * kMaxKs * kTile + b * kTile + ch * 16]);
              float da = 0.f, db = 0.f;
#pragma unroll
              for (int p = 0; p < 8; ++p) {
                const half2_t xv = xp[p];
                da = __builtin_amdgcn_fdot2(wa[p], xv, da, false);
                db = __builtin_amdgcn_fdot2(wb[p], xv, db, false);
              }
              const float s = sc[i * kMaxKs + b];
              acc_a[i] = fmaf(da, s, acc_a[i]);
              acc_b[i] = fmaf(db, s, acc_b[i]);
            }
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kValuRoutes; ++i) {
      if (i < nr) {
        const float sa = group_sum<8>(acc_a[i]);
        const float sb = group_sum<8>(acc_b[i]);
        if (ch == 0) {
          float* dst = a.part + ((size_t)u.split * a.R + rts[i]) * a.N;
          dst[row_a] = sa;
          dst[row_a + 8] = sb;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// MFMA inner product: one v_mfma_f32_16x16x128_f8f6f4 per wave and 128-K
// block gives the 16 rows x 16 routes block partial in FP32; it is scaled and
// added to the running sum at once. Lane l feeds row l % 16 (weights) and
// route l % 16 (activations) with 32 bytes of the block: bytes 16g..16g+15
// and 64+16g..64+16g+15 for g = l / 16. A and B share that byte-to-slot map,
// so the instruction still sums exactly the block's 128 products, while every
// weight load instruction reads 64 contiguous bytes of 16 rows.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void gemm_mfma_kernel(GemmArgs a) {
  __shared__ __align__(16) uint8_t xb[kMfmaRoutes * kMaxKs * kTile];
  __shared__ float sc[kMaxKs * kMfmaRoutes];  // [block][route]
  __shared__ int rts[kMfmaRoutes];

  Unit u;
  if (!decode_unit(a, u)) return;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int col = lane & 15, g = lane >> 4;
  const int row0 = u.tile * kRowsPerWg + wave * 16;
  const uint8_t* pw = a.w + ((size_t)u.e * a.N + row0 + col) * a.K + (size_t)u.kb0 * kTile + g * 16;
  const float* wsr =
      a.ws + ((size_t)u.e * (a.N / kTile) + (u.tile * kRowsPerWg) / kTile) * a.nkb + u.kb0;

  for (int c0 = 0; c0 < u.cnt; c0 += kMfmaRoutes) {
    const int nr = min(kMfmaRoutes, u.cnt - c0);
    if (c0) __syncthreads();
    if (tid < nr) rts[tid] = a.b.routes[u.off + c0 + tid];
    __syncthreads();
    const int chunks = nr * u.nb * 8;  // 16-byte chunks
    for (int i = tid; i < chunks; i += kThreads) {
      const int r = i / (u.nb * 8), rem = i - r * (u.nb * 8);
      const size_t row = (size_t)(rts[r] / a.act_div);
      *reinterpret_cast<u32x4_t*>(&xb[r * kMaxKs * kTile + rem * 16]) =
          *reinterpret_cast<const u32x4_t*>(a.aq + row * a.K + (size_t)u.kb0 * kTile + rem * 16);
    }
    for (int i = tid; i < kMfmaRoutes * u.nb; i += kThreads) {
      const int r = i % kMfmaRoutes, b = i / kMfmaRoutes;
      float v = 0.f;
      if (r < nr) {
        const size_t row = (size_t)(rts[r] / a.act_div);
        v = wsr[b] * a.as[row * a.nkb + u.kb0 + b];
      }
      sc[b * kMfmaRoutes + r] = v;
    }
    __syncthreads();

    const bool live = col < nr;
    const uint8_t* xr = &xb[col * kMaxKs * kTile + g * 16];
    float4_t acc = {0.f, 0.f, 0.f, 0.f};
    const float4_t zero = {0.f, 0.f, 0.f, 0.f};
    u32x4_t nlo[kPrefetch], nhi[kPrefetch];
#pragma unroll
    for (int q = 0; q < kPrefetch; ++q) {
      if (q < u.nb) {
        nlo[q] = load_stream16(pw + q * kTile);
        nhi[q] = load_stream16(pw + q * kTile + 64);
      }
    }
    for (int b0 = 0; b0 < u.nb; b0 += kPrefetch) {
      u32x4_t clo[kPrefetch], chi[kPrefetch];
#pragma unroll
      for (int q = 0; q < kPrefetch; ++q) {
        clo[q] = nlo[q];
        chi[q] = nhi[q];
      }
#pragma unroll
      for (int q = 0; q < kPrefetch; ++q) {
        const int b = b0 + kPrefetch + q;
        if (b < u.nb) {
          nlo[q] = load_stream16(pw + (size_t)b * kTile);
          nhi[q] = load_stream16(pw + (size_t)b * kTile + 64);
        }
      }
#pragma unroll
      for (int q = 0; q < kPrefetch; ++q) {
        const int b = b0 + q;
        if (b < u.nb) {
          u32x4_t xlo = *reinterpret_cast<const u32x4_t*>(xr + b * kTile);
          u32x4_t xhi = *reinterpret_cast<const u32x4_t*>(xr + b * kTile + 64);
          if (!live) xlo = xhi = u32x4_t{0u, 0u, 0u, 0u};
          const int8v_t av = {(int)clo[q][0], (int)clo[q][1], (int)clo[q][2], (int)clo[q][3],
                              (int)chi[q][0], (int)chi[q][1], (int)chi[q][2], (int)chi[q][3]};
          const int8v_t bv = {(int)xlo[0], (int)xlo[1], (int)xlo[2], (int)xlo[3],
                              (int)xhi[0], (int)xhi[1], (int)xhi[2], (int)xhi[3]};
          const float4_t p =
              __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, zero, 0, 0, 0, 0, 0, 0);
          const float s = sc[b * kMfmaRoutes + col];
          acc[0] = fmaf(p[0], s, acc[0]);
          acc[1] = fmaf(p[1], s, acc[1]);
          acc[2] = fmaf(p[2], s, acc[2]);
          acc[3] = fmaf(p[3], s, acc[3]);
        }
      }
    }
    if (live) {
      float* dst = a.part + ((size_t)u.split * a.R + rts[col]) * a.N + row0 + 4 * g;
      *reinterpret_cast<float4_t*>(dst) = acc;
    }
  }
}

}  // namespace

hipError_t launch_gemm_valu(const GemmArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL(gemm_valu_kernel, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gemm_mfma(const GemmArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL(gemm_mfma_kernel, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
