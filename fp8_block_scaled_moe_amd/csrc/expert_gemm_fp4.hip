// FP4 block-scaled GEMM over the touched local experts (nvfp4-megamoe-kernel
// README, "Data Formats"): packed E2M1 weights [E, N, K/2] with one UE4M3
// scale per 16 values along K, against activations staged to E2M1 with their
// own per-16 UE4M3 scales,
//   out[r, n] = sum_g dec(Sw[e, n, g]) * dec(Sa[row(r), g]) * sum_{i in g} W[e, n, i] * A[row(r), i].
//
// On the matrix cores. gfx950's FP4 matrix instructions take power-of-two
// scales per 32 values, not UE4M3 per 16, so the codes are widened to F16 in
// software and the scales applied around v_mfma_f32_4x4x4_16b_f16. Its
// sixteen 4 x 4 x 4 blocks are laid along K: for a wave's 16 rows and one
// 256-value item, instruction (row group g, k step c) gives block b rows
// 4g .. 4g + 3 and the four values 16b + 4c .. 16b + 4c + 3, so block b
// covers exactly scale group b of the item, and a lane's activation operand
// (block b, route x) is the same for all four row groups: the activations
// are widened once per item for the 16 rows, each value times its group's
// scale (an E2M1 value, two significant bits, times a UE4M3 scale, four, is
// exact in F16, between 2^-10 and 2688). The weights are widened as they
// are. A block's four chained instructions then sum the group exactly in
// FP32 (every partial sum is an integer below 2^12 times Sa / 4), and one
// FMA per output multiplies the group sum by the row's weight scale (exact,
// 20 bits) and adds it to the FP32 accumulator: one rounding per group. The
// accumulators' block partials are added across lanes when a tile ends. A job is up
// to kFp4JobRoutes (four) routes of one expert, a block's four columns, so
// an expert's weights are read once for up to four of its routes (decode
// batches rarely give one GPU's expert more; more take further passes).
//
// Work split: the stream of (job, 64-row tile, 256-value step) items is cut
// evenly over the workgroups (stream_device.h), so every workgroup reads the
// same weight bytes however few experts are touched. Each of the four waves
// owns 16 rows of the current tile.
//
// Per item a wave reads 16 rows x 128 bytes with full-line loads (eight lanes
// per row) and passes them through a private LDS tile to lane 4b + x as rows
// x, 4 + x, 8 + x, 12 + x, bytes 8b .. 8b + 7; the 16 rows' scales of group b
// come from a copy reordered once at create (reorder_fp4_scales below) as one
// 16-byte load per lane (the four lanes of a block read the same bytes);
// each lane's activation bytes (8) and scale byte come from L2 straight into
// registers. The job count, the first job descriptors
// and the first route entries are read under one wait at the start, so the
// first weight request follows one memory round trip.
#include <algorithm>

#include "fp4_device.h"
#include "gemm_device.h"
#include "stream_device.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
// Items in flight per wave: three for a long K (150 VGPRs, three waves per
// SIMD), two otherwise (120, four). Measured on MI355X over one GPU's FP4
// share (H = 7168, I = 3072, event timing): GEMM1 (K = 7168) took 13.3
// against 14.8 us at M = 4, 20.6 against 22.1 at M = 16 (4 experts), 41.0
// against 40.7 at M = 16 (9 experts) and 75.7 against 76.4 at M = 64 with
// three rather than two; GEMM2 (K = 3072) 9.8 against 9.2 at M = 4 and 42.8
// against 40.0 at M = 64.
constexpr int kDeepK = 4096;
__host__ __device__ constexpr int fp4_depth(int K) { return K >= kDeepK ? 3 : 2; }
constexpr int kStepValues = 256;                      // K values per item
constexpr int kStepBytes = kStepValues / 2;           // packed bytes of a row's item
constexpr int kStepScales = kStepValues / kFp4Group;  // scale bytes of a row's item
constexpr int kFp4TileStride = kStepBytes + 16;       // LDS row stride (conflict-free)
constexpr int kFp4TileBytes = 16 * kFp4TileStride;
constexpr int kSpec = kThreads;  // job descriptors and route entries read at the start
constexpr int kFp4ScaleBytes = 16 * kStepScales;  // weight scale bytes of a 16-row group and item

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float2_t __attribute__((ext_vector_type(2)));

struct Cursor {
  int j, tile, s;  // job, 64-row tile, K step
};

__device__ __forceinline__ void advance(Cursor& c, int tiles, int steps) {
  if (++c.s == steps) {
    c.s = 0;
    if (++c.tile == tiles) {
      c.tile = 0;
      ++c.j;
    }
  }
}

// The (s, s) F16 pair of byte i of w (a UE4M3 scale), exact.
template <int kByte>
__device__ __forceinline__ half2_t scale_pair(uint32_t w) {
  constexpr uint32_t sel = kByte * 0x00000101u;  // bytes i, i in the low half
  return e4m3x2_to_f16x2<false>(__builtin_amdgcn_perm(w, w, sel));
}

// Four E2M1 values (bytes kB and kB + 1 of w, low nibbles first) times s.
template <int kB>
__device__ __forceinline__ half4_t widen4(uint32_t w, half2_t s) {
  const half2_t lo = e2m1x2_to_f16x2<kB>(w) * s, hi = e2m1x2_to_f16x2<kB + 1>(w) * s;
  return half4_t{lo.x, lo.y, hi.x, hi.y};
}

// The same four values as they are.
template <int kB>
__device__ __forceinline__ half4_t widen4(uint32_t w) {
  const half2_t lo = e2m1x2_to_f16x2<kB>(w), hi = e2m1x2_to_f16x2<kB + 1>(w);
  return half4_t{lo.x, lo.y, hi.x, hi.y};
}

// Bytes 2h and 2h + 1 of w (UE4M3 scales) as FP32, exact.
template <bool kHi>
__device__ __forceinline__ float2_t scale_f32x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, kHi);
}

template <int kRole, int kDepth>
__global__ __launch_bounds__(kThreads) void gemm_fp4_kernel(GemmArgs args) {
  __shared__ __align__(16) unsigned char tiles_lds[4 * kFp4TileBytes];
  __shared__ int4 spec_jobs[kSpec];
  __shared__ int spec_routes[kSpec];
  const GemmProblem& a = args.p[1];
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // uniform: addresses stay scalar

  // One round trip: the job count beside the first job descriptors and route
  // entries (jobs never outnumber routes, so both reads stay in their tables).
  const int nspec = min(a.R, kSpec);
  int4 jd_t = make_int4(0, 0, 0, 0);
  int rt_t = 0;
  if (tid < nspec) {
    jd_t = a.b.jobs[tid];
    rt_t = a.b.routes[tid];
  }
  const int J = a.b.ctrl[2];
  if (tid < nspec) {
    spec_jobs[tid] = jd_t;
    spec_routes[tid] = rt_t;
  }
  __syncthreads();

  const int S = a.K / kStepValues, tiles = a.N / kRowsPerWg;
  const int per_job = tiles * S;  // > kDepth for every accepted shape
  const StreamMap m = stream_map(J, tiles, S, args.stream_wgs);
  if ((int)blockIdx.x >= m.Wa) return;
  const uint32_t lo = stream_begin(blockIdx.x, m), hi = stream_begin(blockIdx.x + 1, m);
  if (lo >= hi) return;  // no items at all
  const int n = (int)(hi - lo);

  const int rg = lane >> 3, ch = lane & 7;  // load layout: rows rg and rg + 8, bytes 16ch..
  const int x = lane & 3, blk = lane >> 2;  // MFMA layout: column / row x of block blk
  const uint32_t row_bytes = (uint32_t)a.K / 2, row_scales = (uint32_t)a.K / kFp4Group;
  uint8_t* tile = tiles_lds + wave * kFp4TileBytes;

  const int j0 = (int)(lo / (uint32_t)per_job), jlast = (int)((hi - 1) / (uint32_t)per_job);
  if (jlast > j0 + 1) return;  // cannot happen: a range holds at most one job's items
  Cursor c{j0, (int)((lo % (uint32_t)per_job) / S), (int)(lo % (uint32_t)S)};  // the item being summed
  Cursor pc = c;                                                               // the next item to request
  int pleft = n;

  // The range's (at most two) jobs: expert and route count (uniform), the
  // route of this lane's column x (the job's first route for columns past
  // the count, whose sums are not written), its activation offsets.
  auto job_of = [&](int j) { return j < nspec ? spec_jobs[j] : a.b.jobs[j]; };
  auto route_at = [&](int i) { return i < nspec ? spec_routes[i] : a.b.routes[i]; };
  const int4 jd0 = job_of(j0), jd1 = jlast > j0 ? job_of(j0 + 1) : jd0;
  const int e0 = __builtin_amdgcn_readfirstlane(jd0.x), e1 = __builtin_amdgcn_readfirstlane(jd1.x);
  const int nr0 = __builtin_amdgcn_readfirstlane(jd0.z), nr1 = __builtin_amdgcn_readfirstlane(jd1.z);
  const int rt0 = route_at(jd0.y + (x < nr0 ? x : 0)), rt1 = route_at(jd1.y + (x < nr1 ? x : 0));
  // 32-bit offsets of this lane's activation bytes and scale byte in step 0
  const uint32_t xo0 = (uint32_t)(rt0 / a.act_div) * row_bytes + blk * 8;
  const uint32_t xo1 = (uint32_t)(rt1 / a.act_div) * row_bytes + blk * 8;
  const uint32_t so0 = (uint32_t)(rt0 / a.act_div) * row_scales + blk;
  const uint32_t so1 = (uint32_t)(rt1 / a.act_div) * row_scales + blk;
  int pe = e0;
  uint32_t pxo = xo0, pso = so0;

  u32x4_t wa[kDepth], wb[kDepth], sw[kDepth];
  uint32_t sx[kDepth];
  uint2 xv[kDepth];
  const uint32_t lane_w = (uint32_t)rg * row_bytes + ch * 16, lane_s = (uint32_t)blk * 16;
  // Requests the item under the requesting cursor into buffer q: the weights
  // and their scales (request_w), then the activations (request_x, which then
  // moves the cursor on). Addresses are a uniform base plus this lane's
  // 32-bit offset. Past the range's end the cursor stays on its last item (a
  // repeat read, from L2).
  auto request_w = [&](int q) {
    const size_t group = (size_t)pe * (a.N / 16) + pc.tile * (kRowsPerWg / 16) + wave;  // 16-row group
    const uint8_t* w = a.w + group * 16 * row_bytes + (size_t)pc.s * kStepBytes;
    const uint8_t* ws = a.ws8 + (group * S + pc.s) * kFp4ScaleBytes;
    wa[q] = load_stream16(w + lane_w);
    wb[q] = load_stream16(w + (lane_w + 8 * row_bytes));
    sw[q] = load_stream16(ws + lane_s);
  };
  auto request_x = [&](int q) {
    const uint8_t* xs = a.aq + (size_t)pc.s * kStepBytes;
    const uint8_t* ss = a.as8 + (size_t)pc.s * kStepScales;
    xv[q] = *reinterpret_cast<const uint2*>(xs + pxo);
    sx[q] = ss[pso];
    if (--pleft > 0) {
      const int pj = pc.j;
      advance(pc, tiles, S);
      if (pc.j != pj) {
        pe = e1;
        pxo = xo1;
        pso = so1;
      }
    }
  };
#pragma unroll
  for (int q = 0; q < kDepth; ++q) {
    request_w(q);
    request_x(q);
  }

  float4_t acc[4] = {};  // row groups 0..3 (rows 4r .. 4r + 3): block blk's sum for route x

  // One item from buffer q; `refill` requests the item kDepth further on.
  // Each register set is refilled once its data is consumed: the weights
  // after they pass through the tile, the activations after the MFMAs.
  auto process = [&](int q, bool refill) {
    *reinterpret_cast<u32x4_t*>(tile + rg * kFp4TileStride + ch * 16) = wa[q];
    *reinterpret_cast<u32x4_t*>(tile + (rg + 8) * kFp4TileStride + ch * 16) = wb[q];
    const u32x4_t ws = sw[q];  // scales of rows 0 .. 15, group blk
    if (refill) request_w(q);
    wave_lds_fence();
    uint2 wr[4];  // rows 4r + x, bytes 8blk .. 8blk + 7
#pragma unroll
    for (int r = 0; r < 4; ++r)
      wr[r] = *reinterpret_cast<const uint2*>(tile + (4 * r + x) * kFp4TileStride + blk * 8);
    wave_lds_fence();
    const half2_t pa = scale_pair<0>(sx[q]);
    const half4_t b0 = widen4<0>(xv[q].x, pa), b1 = widen4<2>(xv[q].x, pa);
    const half4_t b2 = widen4<0>(xv[q].y, pa), b3 = widen4<2>(xv[q].y, pa);
    const float4_t zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      // group blk's exact sum for rows 4r .. 4r + 3 and route x
      float4_t d = __builtin_amdgcn_mfma_f32_4x4x4f16(widen4<0>(wr[r].x), b0, zero, 0, 0, 0);
      d = __builtin_amdgcn_mfma_f32_4x4x4f16(widen4<2>(wr[r].x), b1, d, 0, 0, 0);
      d = __builtin_amdgcn_mfma_f32_4x4x4f16(widen4<0>(wr[r].y), b2, d, 0, 0, 0);
      d = __builtin_amdgcn_mfma_f32_4x4x4f16(widen4<2>(wr[r].y), b3, d, 0, 0, 0);
      const float2_t s01 = scale_f32x2<false>(ws[r]), s23 = scale_f32x2<true>(ws[r]);
      acc[r][0] = fmaf(d[0], s01.x, acc[r][0]);
      acc[r][1] = fmaf(d[1], s01.y, acc[r][1]);
      acc[r][2] = fmaf(d[2], s23.x, acc[r][2]);
      acc[r][3] = fmaf(d[3], s23.y, acc[r][3]);
    }
    if (refill) request_x(q);
  };
  // After item `done` (0-based in the range): at a tile's last step, or the
  // range's last item, the blocks' partials are added across lanes (a fixed
  // butterfly over blocks 0 .. 15) and the live routes' sums go to the
  // tile's partial slot: lane x (block 0) writes rows 4r .. 4r + 3 of the
  // wave's 16 for route x.
  auto finish = [&](int done) {
    if (c.s == S - 1 || done == n - 1) {
      const uint32_t tile_item = ((uint32_t)c.j * tiles + c.tile) * S;
      const int slot = (int)blockIdx.x - stream_owner(tile_item, m);
      const bool first = c.j == j0;
      // the workgroup summing the tile's last step records its slot count
      if (c.s == S - 1 && tid == 0) args.stream_counts[(size_t)c.j * tiles + c.tile] = slot + 1;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = acc[r][i];
          v += __shfl_xor(v, 4, kWave);
          v += __shfl_xor(v, 8, kWave);
          v += __shfl_xor(v, 16, kWave);
          v += __shfl_xor(v, 32, kWave);
          acc[r][i] = v;
        }
        if (blk == 0 && x < (first ? nr0 : nr1)) {
          float* dst = a.part + ((size_t)slot * a.R + (first ? rt0 : rt1)) * a.N + c.tile * kRowsPerWg +
                       wave * 16 + 4 * r;
          *reinterpret_cast<float4_t*>(dst) = acc[r];
        }
        acc[r] = float4_t{0.f, 0.f, 0.f, 0.f};
      }
    }
    advance(c, tiles, S);
  };

  int it = 0;
  for (; it + kDepth <= n; it += kDepth) {
#pragma unroll
    for (int q = 0; q < kDepth; ++q) {
      process(q, true);
      finish(it + q);
    }
  }
#pragma unroll
  for (int q = 0; q < kDepth - 1; ++q)
    if (it + q < n) {
      process(q, false);
      finish(it + q);
    }
}

// The weight scales [rows, K/16] (rows = E * N, a multiple of 16) into the
// kernel's layout: for 16-row group g and item s (256 values), 16 blocks of
// 16 bytes, block b holding the scales of group b of item s in rows 16g ..
// 16g + 15 (byte i: row 16g + i), which is what the lanes of MFMA block b
// read. One thread per output word: word (g * S + s) * 64 + 4b + q holds
// rows 16g + 4q .. 16g + 4q + 3.
__global__ void reorder_fp4_scales_kernel(const uint8_t* src, uint32_t* dst, size_t words, int S) {
  const size_t w = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (w >= words) return;
  const int l = (int)(w % kWave), b = l >> 2, q = l & 3;
  const size_t gs = w / kWave, g = gs / S;
  const int s = (int)(gs - g * S);
  const size_t row_scales = (size_t)S * kStepScales;
  const uint8_t* p = src + (g * 16 + 4 * q) * row_scales + (size_t)s * kStepScales + b;
  dst[w] = (uint32_t)p[0] | ((uint32_t)p[row_scales] << 8) | ((uint32_t)p[2 * row_scales] << 16) |
           ((uint32_t)p[3 * row_scales] << 24);
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

size_t gemm_fp4_lds_bytes(int) { return 4 * (size_t)kFp4TileBytes + kSpec * (sizeof(int4) + sizeof(int)); }

int gemm_fp4_resident_wgs(int K) {
  int dev = 0, cus = 0, per_cu = 0;
  const void* k = fp4_depth(K) == 3 ? reinterpret_cast<const void*>(gemm_fp4_kernel<1, 3>)
                                    : reinterpret_cast<const void*>(gemm_fp4_kernel<1, 2>);
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, kThreads, 0) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return cus * per_cu;
}

hipError_t launch_gemm_fp4(const GemmArgs& a, int role, int grid, hipStream_t s, KernelEvents ev) {
  const bool deep = fp4_depth(a.p[1].K) == 3;
  if (role == 1 && deep)
    hipExtLaunchKernelGGL((gemm_fp4_kernel<1, 3>), dim3(grid), dim3(kThreads), 0, s, ev.start, ev.stop, 0, a);
  else if (role == 1)
    hipExtLaunchKernelGGL((gemm_fp4_kernel<1, 2>), dim3(grid), dim3(kThreads), 0, s, ev.start, ev.stop, 0, a);
  else if (deep)
    hipExtLaunchKernelGGL((gemm_fp4_kernel<2, 3>), dim3(grid), dim3(kThreads), 0, s, ev.start, ev.stop, 0, a);
  else
    hipExtLaunchKernelGGL((gemm_fp4_kernel<2, 2>), dim3(grid), dim3(kThreads), 0, s, ev.start, ev.stop, 0, a);
  return hipGetLastError();
}

hipError_t launch_reorder_fp4_scales(const uint8_t* src, uint8_t* dst, size_t rows, int K, hipStream_t s) {
  const int S = K / kStepValues;
  const size_t words = rows / 16 * S * kWave;
  hipLaunchKernelGGL(reorder_fp4_scales_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, s, src,
                     reinterpret_cast<uint32_t*>(dst), words, S);
  return hipGetLastError();
}

hipError_t launch_codec_check_fp4(const float* in, uint8_t* q, float* dq, int n, hipStream_t s) {
  hipLaunchKernelGGL(codec_check_fp4_kernel, dim3((n + 255) / 256), dim3(256), 0, s, in, q, dq, n);
  return hipGetLastError();
}

}  // namespace moe
