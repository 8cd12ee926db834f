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
// synchronisation is needed. The first weight blocks are requested before
// the activations are staged, so the weight stream starts at once.
#include "kernels.h"
#include "device_common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kPrefetch = 4;  // 128-K blocks of weights in flight per wave
constexpr int kStageBatch = 4;

struct Unit {
  int ui, e, cnt, off, tile, split, kb0, nb;
};

__device__ __forceinline__ bool decode_unit(const GemmArgs& a, Unit& u) {
  const int U = a.b.ctrl[1];
  const int per_expert = a.tiles * a.splits;
  const int unit = blockIdx.x;
  if (unit >= U * per_expert) return false;
  u.ui = unit / per_expert;
  const int rem = unit - u.ui * per_expert;
  u.tile = rem / a.splits;
  u.split = rem - u.tile * a.splits;
  u.e = a.b.uexp[u.ui];
  u.cnt = a.b.ucnt[u.ui];
  u.off = a.b.uoff[u.ui];
  u.kb0 = u.split * a.ks;
  u.nb = min(a.ks, a.nkb - u.kb0);
  return true;
}

// Activations of routes rts[0..nr) for the unit's K range, widened exactly to
// F16 into dst (route r at dst + r * stride halves). Loads of up to
// kStageBatch chunks per thread are issued before any is converted.
__device__ __forceinline__ void stage_f16(const GemmArgs& a, const Unit& u, const int* rts, int nr,
                                          _Float16* dst, int stride) {
  const int per_route = u.nb * 16;  // 8-byte chunks
  const int chunks = nr * per_route;
  for (int base = 0; base < chunks; base += kStageBatch * kThreads) {
    uint2 v[kStageBatch];
#pragma unroll
    for (int q = 0; q < kStageBatch; ++q) {
      const int i = base + q * kThreads + threadIdx.x;
      if (i < chunks) {
        const int r = i / per_route, rem = i - r * per_route;
        const size_t row = (size_t)(rts[r] / a.act_div);
        v[q] = *reinterpret_cast<const uint2*>(a.aq + row * a.K + (size_t)u.kb0 * kTile + rem * 8);
      }
    }
#pragma unroll
    for (int q = 0; q < kStageBatch; ++q) {
      const int i = base + q * kThreads + threadIdx.x;
      if (i < chunks) {
        const int r = i / per_route, rem = i - r * per_route;
        half2_t* d = reinterpret_cast<half2_t*>(dst + r * stride + rem * 8);
        d[0] = e4m3x2_to_f16x2<false>(v[q].x);
        d[1] = e4m3x2_to_f16x2<true>(v[q].x);
        d[2] = e4m3x2_to_f16x2<false>(v[q].y);
        d[3] = e4m3x2_to_f16x2<true>(v[q].y);
      }
    }
  }
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

  u32x4_t na[kPrefetch], nb_[kPrefetch];
  auto prefetch = [&]() {
#pragma unroll
    for (int q = 0; q < kPrefetch; ++q) {
      if (q < u.nb) {
        na[q] = load_stream16(pa + q * kTile);
        nb_[q] = load_stream16(pb + q * kTile);
      }
    }
  };
  prefetch();

  for (int c0 = 0; c0 < u.cnt; c0 += kValuRoutes) {
    const int nr = min(kValuRoutes, u.cnt - c0);
    if (c0) __syncthreads();
    if (tid < nr) rts[tid] = a.b.routes[u.off + c0 + tid];
    __syncthreads();
    // the routes' activations for this split as exact F16, and the per-block
    // products of the two scales
    stage_f16(a, u, rts, nr, xh, kMaxKs * kTile);
    for (int i = tid; i < nr * u.nb; i += kThreads) {
      const int r = i / u.nb, b = i - r * u.nb;
      const size_t row = (size_t)(rts[r] / a.act_div);
      sc[r * kMaxKs + b] = wsr[b] * a.as[row * a.nkb + u.kb0 + b];
    }
    __syncthreads();

    float acc_a[kValuRoutes], acc_b[kValuRoutes];
#pragma unroll
    for (int i = 0; i < kValuRoutes; ++i) acc_a[i] = acc_b[i] = 0.f;

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
    if (c0 + kValuRoutes < u.cnt) prefetch();
  }
}

// ---------------------------------------------------------------------------
// MFMA inner product. Weights and activations widen exactly from e4m3 to F16
// and feed v_mfma_f32_16x16x32_f16: four instructions per wave and 128-K block
// give the 16 rows x 16 routes block partial, which is scaled and added to the
// running FP32 sum at once. (The FP8-input 16x16x128 instruction would take
// the bytes directly, but its internal 128-term sum truncates: measured on
// MI355X up to ~1e-4 of sum |terms|, enough to move FP8 hidden codes; the F16
// instruction's sum is as accurate as FP32 accumulation.)
// Lane l feeds row l % 16 (weights) and route l % 16 (activations) with 32
// values of the block: bytes 16g..16g+15 and 64+16g..64+16g+15, g = l / 16.
// A and B use the same value-to-slot map, so each block's 128 products are
// summed exactly once, and every weight load instruction reads 64 contiguous
// bytes of 16 rows.
// ---------------------------------------------------------------------------
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ half8_t cat4(half2_t a, half2_t b, half2_t c, half2_t d) {
  return half8_t{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

__global__ __launch_bounds__(kThreads) void gemm_mfma_kernel(GemmArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int nrp = a.pass_routes;                    // routes per pass, <= 16
  const int stride = a.ks * kTile + 8;             // halves per route row: +16 B against bank conflicts
  _Float16* xh = reinterpret_cast<_Float16*>(smem);
  float* sc = reinterpret_cast<float*>(smem + (size_t)nrp * stride * 2);  // [ks][16]
  int* rts = reinterpret_cast<int*>(sc + a.ks * kMfmaRoutes);

  Unit u;
  if (!decode_unit(a, u)) return;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int col = lane & 15, g = lane >> 4;
  const int row0 = u.tile * kRowsPerWg + wave * 16;
  const uint8_t* pw = a.w + ((size_t)u.e * a.N + row0 + col) * a.K + (size_t)u.kb0 * kTile + g * 16;
  const float* wsr =
      a.ws + ((size_t)u.e * (a.N / kTile) + (u.tile * kRowsPerWg) / kTile) * a.nkb + u.kb0;

  u32x4_t nlo[kPrefetch], nhi[kPrefetch];
  auto prefetch = [&]() {
#pragma unroll
    for (int q = 0; q < kPrefetch; ++q) {
      if (q < u.nb) {
        nlo[q] = load_stream16(pw + q * kTile);
        nhi[q] = load_stream16(pw + q * kTile + 64);
      }
    }
  };
  prefetch();

  for (int c0 = 0; c0 < u.cnt; c0 += nrp) {
    const int nr = min(nrp, u.cnt - c0);
    if (c0) __syncthreads();
    if (tid < nr) rts[tid] = a.b.routes[u.off + c0 + tid];
    __syncthreads();
    stage_f16(a, u, rts, nr, xh, stride);
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
    // lanes past the pass's routes read route 0's row; their columns are dropped
    const _Float16* xr = xh + (live ? col : 0) * stride + g * 16;
    float4_t acc = {0.f, 0.f, 0.f, 0.f};
    const float4_t zero = {0.f, 0.f, 0.f, 0.f};
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
          const half8_t* xb = reinterpret_cast<const half8_t*>(xr + b * kTile);
          const half8_t x0 = xb[0], x1 = xb[1], x2 = xb[8], x3 = xb[9];  // +0, +8, +64, +72 halves
          const half8_t w0 = cat4(e4m3x2_to_f16x2<false>(clo[q][0]), e4m3x2_to_f16x2<true>(clo[q][0]),
                                  e4m3x2_to_f16x2<false>(clo[q][1]), e4m3x2_to_f16x2<true>(clo[q][1]));
          const half8_t w1 = cat4(e4m3x2_to_f16x2<false>(clo[q][2]), e4m3x2_to_f16x2<true>(clo[q][2]),
                                  e4m3x2_to_f16x2<false>(clo[q][3]), e4m3x2_to_f16x2<true>(clo[q][3]));
          const half8_t w2 = cat4(e4m3x2_to_f16x2<false>(chi[q][0]), e4m3x2_to_f16x2<true>(chi[q][0]),
                                  e4m3x2_to_f16x2<false>(chi[q][1]), e4m3x2_to_f16x2<true>(chi[q][1]));
          const half8_t w3 = cat4(e4m3x2_to_f16x2<false>(chi[q][2]), e4m3x2_to_f16x2<true>(chi[q][2]),
                                  e4m3x2_to_f16x2<false>(chi[q][3]), e4m3x2_to_f16x2<true>(chi[q][3]));
          float4_t p = __builtin_amdgcn_mfma_f32_16x16x32_f16(w0, x0, zero, 0, 0, 0);
          p = __builtin_amdgcn_mfma_f32_16x16x32_f16(w1, x1, p, 0, 0, 0);
          p = __builtin_amdgcn_mfma_f32_16x16x32_f16(w2, x2, p, 0, 0, 0);
          p = __builtin_amdgcn_mfma_f32_16x16x32_f16(w3, x3, p, 0, 0, 0);
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
    if (c0 + nrp < u.cnt) prefetch();
  }
}

}  // namespace

size_t gemm_mfma_lds_bytes(int pass_routes, int ks) {
  return (size_t)pass_routes * (ks * kTile + 8) * 2 + (size_t)ks * kMfmaRoutes * 4 + kMfmaRoutes * 4;
}

hipError_t launch_gemm_valu(const GemmArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL(gemm_valu_kernel, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gemm_mfma(const GemmArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL(gemm_mfma_kernel, dim3(grid), dim3(kThreads),
                     gemm_mfma_lds_bytes(a.pass_routes, a.ks), s, a);
  return hipGetLastError();
}

}  // namespace moe
