// Block-scaled FP8 GEMM over the touched experts, split-K, weight streaming.
//
// The pages' kernel (vLLM "mega_moe" page, module docstring) keeps each
// 128-K block's unscaled partial apart because the FP32 block scales are not
// powers of two and cannot ride inside the matrix instruction; the epilogue
// scales and sums the blocks once. The same rule holds here: every partial
// over one 128-K block is multiplied by (weight scale x activation scale) of
// that block before it joins the running FP32 sum.
//
// Work unit = (distinct expert, group of `tpw` 64-row tiles, one K split).
// Each of the four waves of a workgroup owns 16 rows of a tile. A touched
// expert's weights are read once for all of its routes (up to 8 or 16 per
// pass); untouched experts are never read. The unit's activations are staged
// once and its tiles are streamed back to back as one sequence of 128-K
// blocks, so staging is paid once per `tpw` tiles. The grid is sized for the
// largest possible number of distinct experts; workgroups past the actual
// count exit at once, so no host synchronisation is needed. The first weight
// blocks are requested before the activations are staged.
//
// A launch may also carry a dense problem -- the shared expert, whose routes
// are the tokens themselves -- whose units run first in the same grid, so the
// shared expert's weights stream beside the routed experts' without a launch
// of their own.
#include <algorithm>

#include "gemm_device.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kPrefetch = 4;  // 128-K blocks of weights in flight per wave
constexpr int kStageBatch = 4;

struct Unit {
  int ui, e, cnt, off, tile0, split, kb0, nb;
};

__device__ __forceinline__ bool decode_unit(const GemmProblem& a, int unit, Unit& u) {
  const int U = a.dense ? 1 : a.b.ctrl[1];
  const int groups = a.tiles / a.tpw;
  const int per_expert = groups * a.splits;
  if (unit >= U * per_expert) return false;
  u.ui = unit / per_expert;
  const int rem = unit - u.ui * per_expert;
  const int group = rem / a.splits;
  u.tile0 = group * a.tpw;
  u.split = rem - group * a.splits;
  if (a.dense) {
    u.e = 0;
    u.cnt = a.dense;
    u.off = 0;
  } else {
    u.e = a.b.uexp[u.ui];
    u.cnt = a.b.ucnt[u.ui];
    u.off = a.b.uoff[u.ui];
  }
  u.kb0 = u.split * a.ks;
  u.nb = min(a.ks, a.nkb - u.kb0);
  return true;
}

// Route index i of the unit's list.
__device__ __forceinline__ int unit_route(const GemmProblem& a, const Unit& u, int i) {
  return a.dense ? i : a.b.routes[u.off + i];
}

// Position of one 128-K block in the unit's stream (tile j, block b).
struct Cursor {
  int j, b;
  __device__ __forceinline__ void next(int nb) {
    if (++b == nb) {
      b = 0;
      ++j;
    }
  }
};

// Weight scales of the unit's tiles (wsl[j * kMaxKs + b]) and activation
// scales of the pass's routes (xsl[r * kMaxKs + b]); the block scale of
// (tile j, route r, block b) is their product.
__device__ __forceinline__ void stage_scales(const GemmProblem& a, const Unit& u, const int* rts, int nr,
                                             float* wsl, float* xsl) {
  const float* ws = a.ws + (size_t)u.e * (a.N / kTile) * a.nkb + u.kb0;
  for (int i = threadIdx.x; i < a.tpw * u.nb; i += kThreads) {
    const int j = i / u.nb, b = i - j * u.nb;
    wsl[j * kMaxKs + b] = ws[(size_t)(((u.tile0 + j) * kRowsPerWg) / kTile) * a.nkb + b];
  }
  for (int i = threadIdx.x; i < nr * u.nb; i += kThreads) {
    const int r = i / u.nb, b = i - r * u.nb;
    const size_t row = (size_t)(rts[r] / a.act_div);
    xsl[r * kMaxKs + b] = a.as[row * a.nkb + u.kb0 + b];
  }
}

// ---------------------------------------------------------------------------
// VALU inner product: lane (8 per row, 16 bytes each) holds one 128-byte
// block of two rows; e4m3 pairs widen exactly to F16 pairs and v_dot2 adds
// two exact products into FP32.
// ---------------------------------------------------------------------------

// kRole only names the instantiation (1: W13 / GEMM1, 2: W2 / GEMM2), so that
// profiles report the two GEMMs apart.
template <int kRole>
__global__ __launch_bounds__(kThreads) void gemm_valu_kernel(GemmArgs args) {
  __shared__ __align__(16) _Float16 xh[kValuRoutes * kMaxKs * kTile];
  __shared__ float xsl[kValuRoutes * kMaxKs];
  __shared__ float wsl[kMaxTpw * kMaxKs];
  __shared__ int rts[kValuRoutes];

  int unit;
  const GemmProblem a = select_problem(args, unit);
  Unit u;
  if (!decode_unit(a, unit, u)) return;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int rg = lane >> 3, ch = lane & 7;
  const int rows_in_tile = wave * 16 + rg;  // and + 8
  const uint8_t* p0 = a.w + ((size_t)u.e * a.N + u.tile0 * kRowsPerWg + rows_in_tile) * a.K +
                      (size_t)u.kb0 * kTile + ch * 16;
  const size_t tile_step = (size_t)kRowsPerWg * a.K;
  const size_t half_step = (size_t)8 * a.K;
  const int nsteps = a.tpw * u.nb;

  u32x4_t na[kPrefetch], nb_[kPrefetch];
  Cursor ld{0, 0};
  auto load_next = [&](int q) {
    const uint8_t* p = p0 + ld.j * tile_step + (size_t)ld.b * kTile;
    na[q] = load_stream16(p);
    nb_[q] = load_stream16(p + half_step);
    ld.next(u.nb);
  };
  auto prefetch = [&]() {
    ld = Cursor{0, 0};
#pragma unroll
    for (int q = 0; q < kPrefetch; ++q)
      if (q < nsteps) load_next(q);
  };
  prefetch();

  for (int c0 = 0; c0 < u.cnt; c0 += kValuRoutes) {
    const int nr = min(kValuRoutes, u.cnt - c0);
    if (c0) __syncthreads();
    if (tid < nr) rts[tid] = unit_route(a, u, c0 + tid);
    __syncthreads();
    // the routes' activations for this split as exact F16, and the scales
    {
      const int per_route = u.nb * 16;  // 8-byte chunks
      const int chunks = nr * per_route;
      for (int base = 0; base < chunks; base += kStageBatch * kThreads) {
        uint2 v[kStageBatch];
#pragma unroll
        for (int q = 0; q < kStageBatch; ++q) {
          const int i = base + q * kThreads + tid;
          if (i < chunks) {
            const int r = i / per_route, rem = i - r * per_route;
            const size_t row = (size_t)(rts[r] / a.act_div);
            v[q] = *reinterpret_cast<const uint2*>(a.aq + row * a.K + (size_t)u.kb0 * kTile + rem * 8);
          }
        }
#pragma unroll
        for (int q = 0; q < kStageBatch; ++q) {
          const int i = base + q * kThreads + tid;
          if (i < chunks) {
            const int r = i / per_route, rem = i - r * per_route;
            half2_t* d = reinterpret_cast<half2_t*>(&xh[r * kMaxKs * kTile + rem * 8]);
            d[0] = e4m3x2_to_f16x2<false>(v[q].x);
            d[1] = e4m3x2_to_f16x2<true>(v[q].x);
            d[2] = e4m3x2_to_f16x2<false>(v[q].y);
            d[3] = e4m3x2_to_f16x2<true>(v[q].y);
          }
        }
      }
    }
    stage_scales(a, u, rts, nr, wsl, xsl);
    __syncthreads();

    float acc_a[kValuRoutes], acc_b[kValuRoutes];
#pragma unroll
    for (int i = 0; i < kValuRoutes; ++i) acc_a[i] = acc_b[i] = 0.f;
    Cursor at{0, 0};
    // Rotating prefetch: the registers of step st are refilled with step
    // st + kPrefetch as soon as they are consumed.
    for (int st0 = 0; st0 < nsteps; st0 += kPrefetch) {
#pragma unroll
      for (int q = 0; q < kPrefetch; ++q) {
        if (st0 + q < nsteps) {
          half2_t wa[8], wb[8];
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            wa[2 * d] = e4m3x2_to_f16x2<false>(na[q][d]);
            wa[2 * d + 1] = e4m3x2_to_f16x2<true>(na[q][d]);
            wb[2 * d] = e4m3x2_to_f16x2<false>(nb_[q][d]);
            wb[2 * d + 1] = e4m3x2_to_f16x2<true>(nb_[q][d]);
          }
          if (st0 + q + kPrefetch < nsteps) load_next(q);
          const int b = at.b;
          const float ws = wsl[at.j * kMaxKs + b];
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
              const float s = ws * xsl[i * kMaxKs + b];
              acc_a[i] = fmaf(da, s, acc_a[i]);
              acc_b[i] = fmaf(db, s, acc_b[i]);
            }
          }
          if (b == u.nb - 1) {  // tile at.j complete: reduce over the 8 lanes of a row, store
            const int row = (u.tile0 + at.j) * kRowsPerWg + rows_in_tile;
#pragma unroll
            for (int i = 0; i < kValuRoutes; ++i) {
              if (i < nr) {
                const float sa = group_sum<8>(acc_a[i]);
                const float sb = group_sum<8>(acc_b[i]);
                if (ch == 0) {
                  float* dst = a.part + ((size_t)u.split * a.R + rts[i]) * a.N;
                  dst[row] = sa;
                  dst[row + 8] = sb;
                }
              }
              acc_a[i] = acc_b[i] = 0.f;
            }
          }
          at.next(u.nb);
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
//
// Weights are loaded exactly as in the VALU kernel -- eight lanes read a
// row's full 128-byte block, 16 B each -- because reading half-lines of
// twice as many rows per instruction measured ~20% slower on MI355X. Each
// wave then passes its 16 x 128-byte block through a private LDS tile (row
// stride 144 B, so the reads below hit every bank once) into the MFMA
// layout: lane l feeds row l % 16 with bytes 16g..16g+15 and 64+16g..64+16g+15
// of the block, g = l / 16, and the activations of route l % 16 with the same
// bytes, so each block's 128 products are summed exactly once.
// ---------------------------------------------------------------------------
template <int kRole>
__global__ __launch_bounds__(kThreads) void gemm_mfma_kernel(GemmArgs args) {
  extern __shared__ __align__(16) unsigned char smem[];
  int unit;
  const GemmProblem a = select_problem(args, unit);
  const int nrp = args.pass_routes;      // routes per pass, <= 16
  const int stride = a.ks * kTile + 16;  // bytes per staged route row: +16 B against bank conflicts
  uint8_t* tiles = smem;                                           // [4 waves][kTileBytes]
  uint8_t* xb = smem + 4 * kTileBytes;                             // [nrp][stride] e4m3
  float* xsl = reinterpret_cast<float*>(xb + (size_t)nrp * stride);  // [16][kMaxKs]
  float* wsl = xsl + kMfmaRoutes * kMaxKs;                         // [kMaxTpw][kMaxKs]
  int* rts = reinterpret_cast<int*>(wsl + kMaxTpw * kMaxKs);

  Unit u;
  if (!decode_unit(a, unit, u)) return;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int rg = lane >> 3, ch = lane & 7;   // load layout
  const int col = lane & 15, g = lane >> 4;  // MFMA layout
  const uint8_t* p0 = a.w + ((size_t)u.e * a.N + u.tile0 * kRowsPerWg + wave * 16 + rg) * a.K +
                      (size_t)u.kb0 * kTile + ch * 16;
  const size_t tile_step = (size_t)kRowsPerWg * a.K;
  const size_t half_step = (size_t)8 * a.K;
  const int nsteps = a.tpw * u.nb;
  uint8_t* tile = tiles + wave * kTileBytes;

  u32x4_t na[kPrefetch], nb_[kPrefetch];
  Cursor ld{0, 0};
  auto load_next = [&](int q) {
    const uint8_t* p = p0 + ld.j * tile_step + (size_t)ld.b * kTile;
    na[q] = load_stream16(p);
    nb_[q] = load_stream16(p + half_step);
    ld.next(u.nb);
  };
  auto prefetch = [&]() {
    ld = Cursor{0, 0};
#pragma unroll
    for (int q = 0; q < kPrefetch; ++q)
      if (q < nsteps) load_next(q);
  };
  prefetch();

  for (int c0 = 0; c0 < u.cnt; c0 += nrp) {
    const int nr = min(nrp, u.cnt - c0);
    if (c0) __syncthreads();
    if (tid < nr) rts[tid] = unit_route(a, u, c0 + tid);
    __syncthreads();
    {  // the routes' activations for this split, e4m3 as stored
      const int per_route = u.nb * 8;  // 16-byte chunks
      const int chunks = nr * per_route;
      for (int base = 0; base < chunks; base += kStageBatch * kThreads) {
        u32x4_t v[kStageBatch];
#pragma unroll
        for (int q = 0; q < kStageBatch; ++q) {
          const int i = base + q * kThreads + tid;
          if (i < chunks) {
            const int r = i / per_route, rem = i - r * per_route;
            const size_t row = (size_t)(rts[r] / a.act_div);
            v[q] = *reinterpret_cast<const u32x4_t*>(a.aq + row * a.K + (size_t)u.kb0 * kTile + rem * 16);
          }
        }
#pragma unroll
        for (int q = 0; q < kStageBatch; ++q) {
          const int i = base + q * kThreads + tid;
          if (i < chunks) {
            const int r = i / per_route, rem = i - r * per_route;
            *reinterpret_cast<u32x4_t*>(xb + r * stride + rem * 16) = v[q];
          }
        }
      }
    }
    stage_scales(a, u, rts, nr, wsl, xsl);
    __syncthreads();

    const bool live = col < nr;
    // lanes past the pass's routes read route 0's row; their columns are dropped
    const uint8_t* xr = xb + (live ? col : 0) * stride + g * 16;
    const float* xs_col = xsl + (live ? col : 0) * kMaxKs;
    float4_t acc = {0.f, 0.f, 0.f, 0.f};
    const float4_t zero = {0.f, 0.f, 0.f, 0.f};
    Cursor at{0, 0};
    for (int st0 = 0; st0 < nsteps; st0 += kPrefetch) {
#pragma unroll
      for (int q = 0; q < kPrefetch; ++q) {
        if (st0 + q < nsteps) {
          // weights: load layout -> tile -> MFMA layout; the registers of
          // step st are refilled with step st + kPrefetch right away
          *reinterpret_cast<u32x4_t*>(tile + rg * kTileStride + ch * 16) = na[q];
          *reinterpret_cast<u32x4_t*>(tile + (rg + 8) * kTileStride + ch * 16) = nb_[q];
          if (st0 + q + kPrefetch < nsteps) load_next(q);
          const int b = at.b;
          wave_lds_fence();
          const u32x4_t wlo = *reinterpret_cast<const u32x4_t*>(tile + col * kTileStride + g * 16);
          const u32x4_t whi = *reinterpret_cast<const u32x4_t*>(tile + col * kTileStride + 64 + g * 16);
          const u32x4_t xlo = *reinterpret_cast<const u32x4_t*>(xr + b * kTile);
          const u32x4_t xhi = *reinterpret_cast<const u32x4_t*>(xr + b * kTile + 64);
          wave_lds_fence();
          const float4_t p = mfma_block(wlo, whi, xlo, xhi);
          const float s = wsl[at.j * kMaxKs + b] * xs_col[b];
          acc[0] = fmaf(p[0], s, acc[0]);
          acc[1] = fmaf(p[1], s, acc[1]);
          acc[2] = fmaf(p[2], s, acc[2]);
          acc[3] = fmaf(p[3], s, acc[3]);
          if (b == u.nb - 1) {  // tile at.j complete
            if (live) {
              const int row = (u.tile0 + at.j) * kRowsPerWg + wave * 16 + 4 * g;
              float* dst = a.part + ((size_t)u.split * a.R + rts[col]) * a.N + row;
              *reinterpret_cast<float4_t*>(dst) = acc;
            }
            acc = zero;
          }
          at.next(u.nb);
        }
      }
    }
    if (c0 + nrp < u.cnt) prefetch();
  }
}

}  // namespace

size_t gemm_mfma_lds_bytes(int pass_routes, int ks) {
  return 4 * (size_t)kTileBytes + (size_t)pass_routes * (ks * kTile + 16) +
         (size_t)(kMfmaRoutes + kMaxTpw) * kMaxKs * 4 + kMfmaRoutes * 4;
}

hipError_t launch_gemm_valu(const GemmArgs& a, int role, int grid, hipStream_t s, KernelEvents ev) {
  if (role == 1)
    hipExtLaunchKernelGGL(gemm_valu_kernel<1>, dim3(grid), dim3(kThreads), 0, s, ev.start, ev.stop, 0, a);
  else
    hipExtLaunchKernelGGL(gemm_valu_kernel<2>, dim3(grid), dim3(kThreads), 0, s, ev.start, ev.stop, 0, a);
  return hipGetLastError();
}

hipError_t launch_gemm_mfma(const GemmArgs& a, int role, int grid, hipStream_t s, KernelEvents ev) {
  const int ks = a.units0 ? std::max(a.p[0].ks, a.p[1].ks) : a.p[1].ks;
  const size_t lds = gemm_mfma_lds_bytes(a.pass_routes, ks);
  if (role == 1)
    hipExtLaunchKernelGGL(gemm_mfma_kernel<1>, dim3(grid), dim3(kThreads), lds, s, ev.start, ev.stop, 0, a);
  else
    hipExtLaunchKernelGGL(gemm_mfma_kernel<2>, dim3(grid), dim3(kThreads), lds, s, ev.start, ev.stop, 0, a);
  return hipGetLastError();
}

}  // namespace moe
