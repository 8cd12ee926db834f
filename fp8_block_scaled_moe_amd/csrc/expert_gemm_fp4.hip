// FP4 block-scaled GEMM over the touched local experts (nvfp4-megamoe-kernel
// README, "Data Formats"): packed E2M1 weights [E, N, K/2] with one UE4M3
// scale per 16 values along K, against activations staged to E2M1 with
// their own per-16 scales,
//   out[r, n] = sum_g dec(Sw[e, n, g]) * sum_{i in g} W[e, n, i] * (A[row(r), i] * dec(Sa[row(r), g]))
// with each activation already multiplied by its scale. That product of an
// E2M1 value and a UE4M3 scale has at most six significant bits, so the
// routing kernel stores it exactly as F16. gfx950's native FP4 matrix
// instructions take power-of-two scales per 32 values, not UE4M3 per 16, so
// the weights are widened in software: exactly to F16 pairs, then v_dot2
// multiplies exactly and adds in FP32, and each 16-value group's sum is
// multiplied by its weight scale once.
//
// Work decomposition as in expert_gemm_wg.hip: a workgroup owns 16, 32 or 64
// weight rows of one expert over all of K, its four waves split K into
// `kparts` ranges and add their results through LDS in a fixed order, and
// one FP32 value per (route, row) is written. Per step a wave reads 16 rows x
// 256 values (128 bytes per row, eight lanes per row) plus their 16 scale
// bytes per row; the activations of the pass's routes sit in LDS as F16 for
// the whole K.
#include <algorithm>

#include "fp4_device.h"
#include "gemm_device.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kDepth = 2;           // steps in flight per wave
constexpr int kStepValues = 256;    // K values per step (128 packed bytes per row)
constexpr int kMaxPassRoutes = 8;
constexpr size_t kXLdsBudget = 28 * 1024;  // F16 activations per pass

template <int kRole>
__global__ __launch_bounds__(kThreads) void gemm_fp4_kernel(GemmArgs args) {
  extern __shared__ __align__(16) unsigned char smem[];
  int unit;
  const GemmProblem a = select_problem(args, unit);
  const int kparts = a.kparts;
  const int rows_wg = kRowsPerWg / kparts;
  const int per_expert = a.N / rows_wg;
  const int U = a.dense ? 1 : a.b.ctrl[1];
  if (unit >= U * per_expert) return;  // past the touched experts: the whole workgroup exits
  const int ui = unit / per_expert, tile = unit - ui * per_expert;
  int e, cnt, off;
  if (a.dense) {
    e = 0;
    cnt = a.dense;
    off = 0;
  } else {
    e = a.b.uexp[ui];
    cnt = a.b.ucnt[ui];
    off = a.b.uoff[ui];
  }

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int rgrp = wave / kparts, kp = wave - rgrp * kparts;
  const int row0 = tile * rows_wg + rgrp * 16;
  const int nsteps_all = a.K / kStepValues;
  const int sb0 = (kp * nsteps_all) / kparts;
  const int nsteps = ((kp + 1) * nsteps_all) / kparts - sb0;
  const int rg = lane >> 3, ch = lane & 7;  // rows rg and rg + 8; bytes 16ch..16ch+15 of each row's step
  const int nrp = args.pass_routes;

  _Float16* xh = reinterpret_cast<_Float16*>(smem);                           // [nrp][K]
  float* red = reinterpret_cast<float*>(smem + (size_t)nrp * a.K * 2);         // [4][16][nrp]
  int* rts = reinterpret_cast<int*>(red + 4 * 16 * nrp);                       // [nrp]

  const size_t row_bytes = (size_t)a.K / 2, row_scales = (size_t)a.K / kFp4Group;
  const uint8_t* pw = a.w + ((size_t)e * a.N + row0 + rg) * row_bytes + (size_t)sb0 * (kStepValues / 2) + ch * 16;
  const uint8_t* ps = a.ws8 + ((size_t)e * a.N + row0 + rg) * row_scales +
                      (size_t)sb0 * (kStepValues / kFp4Group) + ch * 2;
  u32x4_t wa[kDepth], wb[kDepth];
  uint32_t sa[kDepth], sb[kDepth];
  auto load = [&](int q, int st) {
    const uint8_t* p = pw + (size_t)st * (kStepValues / 2);
    wa[q] = load_stream16(p);
    wb[q] = load_stream16(p + 8 * row_bytes);
    const uint8_t* s = ps + (size_t)st * (kStepValues / kFp4Group);
    sa[q] = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(s));
    sb[q] = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(s + 8 * row_scales));
  };

  for (int c0 = 0; c0 < cnt; c0 += nrp) {
    const int nr = min(nrp, cnt - c0);
    if (c0) __syncthreads();  // the previous pass is done with xh, red and rts
#pragma unroll
    for (int q = 0; q < kDepth; ++q)
      if (q < nsteps) load(q, q);
    if (tid < nr) rts[tid] = a.dense ? c0 + tid : a.b.routes[off + c0 + tid];
    __syncthreads();
    {  // the pass's activations, F16 for all of K
      const int per_route = a.K / 8;  // 16-byte chunks
      for (int i = tid; i < nr * per_route; i += kThreads) {
        const int r = i / per_route, c = i - r * per_route;
        const _Float16* src = a.ad + (size_t)(rts[r] / a.act_div) * a.K + c * 8;
        *reinterpret_cast<u32x4_t*>(xh + (size_t)r * a.K + c * 8) = *reinterpret_cast<const u32x4_t*>(src);
      }
    }
    __syncthreads();

    float acc_a[kMaxPassRoutes], acc_b[kMaxPassRoutes];
#pragma unroll
    for (int i = 0; i < kMaxPassRoutes; ++i) acc_a[i] = acc_b[i] = 0.f;
    for (int st0 = 0; st0 < nsteps; st0 += kDepth) {
#pragma unroll
      for (int q = 0; q < kDepth; ++q) {
        const int st = st0 + q;
        if (st < nsteps) {
          half2_t w0[16], w1[16];
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            w0[4 * d] = e2m1x2_to_f16x2<0>(wa[q][d]);
            w0[4 * d + 1] = e2m1x2_to_f16x2<1>(wa[q][d]);
            w0[4 * d + 2] = e2m1x2_to_f16x2<2>(wa[q][d]);
            w0[4 * d + 3] = e2m1x2_to_f16x2<3>(wa[q][d]);
            w1[4 * d] = e2m1x2_to_f16x2<0>(wb[q][d]);
            w1[4 * d + 1] = e2m1x2_to_f16x2<1>(wb[q][d]);
            w1[4 * d + 2] = e2m1x2_to_f16x2<2>(wb[q][d]);
            w1[4 * d + 3] = e2m1x2_to_f16x2<3>(wb[q][d]);
          }
          const float s0a = e4m3_value(sa[q]), s1a = e4m3_value(sa[q] >> 8);
          const float s0b = e4m3_value(sb[q]), s1b = e4m3_value(sb[q] >> 8);
          if (st + kDepth < nsteps) load(q, st + kDepth);
          const int k0 = (sb0 + st) * kStepValues + ch * 32;
#pragma unroll
          for (int i = 0; i < kMaxPassRoutes; ++i) {
            if (i < nr) {
              const half2_t* x = reinterpret_cast<const half2_t*>(xh + (size_t)i * a.K + k0);
              float pa0 = 0.f, pa1 = 0.f, pb0 = 0.f, pb1 = 0.f;
#pragma unroll
              for (int j = 0; j < 8; ++j) {
                const half2_t xv0 = x[j], xv1 = x[8 + j];
                pa0 = __builtin_amdgcn_fdot2(w0[j], xv0, pa0, false);
                pb0 = __builtin_amdgcn_fdot2(w1[j], xv0, pb0, false);
                pa1 = __builtin_amdgcn_fdot2(w0[8 + j], xv1, pa1, false);
                pb1 = __builtin_amdgcn_fdot2(w1[8 + j], xv1, pb1, false);
              }
              acc_a[i] = fmaf(pa1, s1a, fmaf(pa0, s0a, acc_a[i]));
              acc_b[i] = fmaf(pb1, s1b, fmaf(pb0, s0b, acc_b[i]));
            }
          }
        }
      }
    }

    // rows rg and rg + 8: the eight lanes of a row hold consecutive 32-value
    // pieces; their sum, then the K parts in a fixed order
#pragma unroll
    for (int i = 0; i < kMaxPassRoutes; ++i) {
      if (i < nr) {
        acc_a[i] = group_sum<8>(acc_a[i]);
        acc_b[i] = group_sum<8>(acc_b[i]);
      }
    }
    if (kparts > 1) {
      if (ch == 0) {
        for (int i = 0; i < nr; ++i) {
          red[(wave * 16 + rg) * nrp + i] = acc_a[i];
          red[(wave * 16 + rg + 8) * nrp + i] = acc_b[i];
        }
      }
      __syncthreads();
      if (kp == 0 && ch == 0) {
        for (int j = 1; j < kparts; ++j) {
          for (int i = 0; i < nr; ++i) {
            acc_a[i] += red[((wave + j) * 16 + rg) * nrp + i];
            acc_b[i] += red[((wave + j) * 16 + rg + 8) * nrp + i];
          }
        }
      }
    }
    if (kp == 0 && ch == 0) {
      for (int i = 0; i < nr; ++i) {
        float* dst = a.part + (size_t)rts[i] * a.N + row0;
        dst[rg] = acc_a[i];
        dst[rg + 8] = acc_b[i];
      }
    }
  }
}

__global__ void codec_check_fp4_kernel(const float* in, uint8_t* q, float* dq, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  q[i] = (uint8_t)e2m1_encode(in[i]);
  const uint32_t c = (uint32_t)i & 15u;
  const int pos = (i >> 4) & 7;  // nibble position in a word: byte pos / 2, high nibble when odd
  const uint32_t word = c << (4 * pos);
  half2_t h;
  switch (pos >> 1) {
    case 0: h = e2m1x2_to_f16x2<0>(word); break;
    case 1: h = e2m1x2_to_f16x2<1>(word); break;
    case 2: h = e2m1x2_to_f16x2<2>(word); break;
    default: h = e2m1x2_to_f16x2<3>(word); break;
  }
  dq[i] = (float)((pos & 1) ? h.y : h.x);
}

}  // namespace

int gemm_fp4_routes_per_pass(int K) {
  return std::max(1, std::min(kMaxPassRoutes, (int)(kXLdsBudget / ((size_t)K * 2))));
}

size_t gemm_fp4_lds_bytes(int K, int routes) {
  return (size_t)routes * K * 2 + (size_t)4 * 16 * routes * 4 + (size_t)routes * 4;
}

hipError_t launch_gemm_fp4(const GemmArgs& a, int role, int grid, hipStream_t s) {
  const size_t lds = gemm_fp4_lds_bytes(a.p[1].K, a.pass_routes);
  if (role == 1)
    hipLaunchKernelGGL(gemm_fp4_kernel<1>, dim3(grid), dim3(kThreads), lds, s, a);
  else
    hipLaunchKernelGGL(gemm_fp4_kernel<2>, dim3(grid), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_codec_check_fp4(const float* in, uint8_t* q, float* dq, int n, hipStream_t s) {
  hipLaunchKernelGGL(codec_check_fp4_kernel, dim3((n + 255) / 256), dim3(256), 0, s, in, q, dq, n);
  return hipGetLastError();
}

}  // namespace moe
