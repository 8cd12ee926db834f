// FP4 block-scaled GEMM over the touched local experts (nvfp4-megamoe-kernel
// README, "Data Formats"): packed E2M1 weights [E, N, K/2] with one UE4M3
// scale per 16 values along K, against activations staged to E2M1 with their
// own per-16 UE4M3 scales,
//   out[r, n] = sum_g dec(Sw[e, n, g]) * dec(Sa[row(r), g]) * sum_{i in g} W[e, n, i] * A[row(r), i].
// gfx950's FP4 matrix instructions take power-of-two scales per 32 values, not
// UE4M3 per 16, so the codes are widened in software, exactly, to F16 pairs:
// v_dot2 multiplies them exactly and adds in FP32, and a 16-value group's sum
// of E2M1 products (a multiple of 1/4 below 600) is exact. Times the
// activation scale it is still exact (at most 16 significant bits); the
// weight scale then joins in one fused multiply-add into the FP32 total.
//
// Work split: the stream of (job, 64-row tile, 256-value step) items is cut
// evenly over the workgroups (stream_device.h), so every workgroup reads the
// same weight bytes however few experts are touched. A job is up to
// kFp4JobRoutes (two) routes of one expert (the routing kernel builds the
// job table), so an expert's weights are read once per two of its routes:
// the inner product costs VALU work per route, and one GPU's share of
// experts sees one or two routes per touched expert at decode batch sizes
// (more routes per expert are the matrix-core path's case). Each of the four
// waves owns 16 rows of the current tile; the jobs' activations (packed codes
// and scale bytes, a ninth of the weight bytes per route and K value) are
// staged in LDS once per job over the whole K. When a tile ends, or the
// workgroup's range does, each wave writes its rows' sums for the job's
// routes to the tile's partial slot.
//
// Per item a wave reads 16 rows x 128 bytes (eight lanes per row; rows rg and
// rg + 8 per lane) plus the rows' 16 scale bytes each, kDepth items ahead of
// use, straight across tile and job boundaries. The weight scales are read
// from a copy reordered once at create (reorder_fp4_scales below): there one
// item's scales of a wave's 16 rows are 256 contiguous bytes in lane order,
// four per lane, so each item costs one coalesced load and every scale line
// is fetched once (read in place, 16 bytes of each row's 128-byte line per
// item, the lines are fetched again for most items).
#include <algorithm>

#include "fp4_device.h"
#include "stream_device.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kDepth = 2;                              // items in flight per wave
constexpr int kStepValues = 256;                       // K values per item
constexpr int kStepBytes = kStepValues / 2;            // packed bytes of a row's item
constexpr int kStepScales = kStepValues / kFp4Group;   // scale bytes of a row's item
constexpr int kJobBufs = 2;                            // jobs staged at once
constexpr int kInfoInts = 2 + kFp4JobRoutes;           // a staged job's route count, expert, routes
constexpr int kStageBatch = 4;                         // 16-byte staging loads in flight per thread

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

// Route i of a job from its routes held in registers (selects, no indexing).
__device__ __forceinline__ int pick_route(const int (&rt)[kFp4JobRoutes], int i) {
  int v = rt[0];
#pragma unroll
  for (int k = 1; k < kFp4JobRoutes; ++k) v = i == k ? rt[k] : v;
  return v;
}

// A job's descriptor {expert, first route entry, count} and routes.
__device__ __forceinline__ void load_job(const GemmProblem& a, int j, int4& jd, int (&rt)[kFp4JobRoutes]) {
  jd = a.b.jobs[j];
#pragma unroll
  for (int i = 0; i < kFp4JobRoutes; ++i) rt[i] = i < jd.z ? a.b.routes[jd.y + i] : 0;
}

// A job's activations over the whole K into an LDS buffer
// ([kFp4JobRoutes][S][128] packed codes, then [kFp4JobRoutes][S][16] scale
// bytes) and its route count, expert and
// routes into `info`. The whole workgroup calls it; a barrier must follow
// before the buffer is read.
__device__ void stage_job(const GemmProblem& a, const int4& jd, const int (&rt)[kFp4JobRoutes], int S,
                          unsigned char* codes, int* info) {
  const int nr = jd.z;
  const int tid = threadIdx.x;
  if (tid == 0) {
    info[0] = nr;
    info[1] = jd.x;
  }
  if (tid < nr) info[2 + tid] = pick_route(rt, tid);
  unsigned char* scales = codes + (size_t)kFp4JobRoutes * S * kStepBytes;
  const int per_route = S * (kStepBytes / 16 + kStepScales / 16);  // 16-byte chunks
  const int total = nr * per_route;
  const size_t row_bytes = (size_t)a.K / 2, row_scales = (size_t)a.K / kFp4Group;
  for (int base = 0; base < total; base += kStageBatch * kThreads) {
    u32x4_t v[kStageBatch];
    unsigned char* dst[kStageBatch];
#pragma unroll
    for (int q = 0; q < kStageBatch; ++q) {
      const int c = base + q * kThreads + tid;
      dst[q] = nullptr;
      if (c < total) {
        const int r = c / per_route, cc = c - r * per_route;
        const size_t row = (size_t)(pick_route(rt, r) / a.act_div);
        const uint8_t* src;
        if (cc < S * (kStepBytes / 16)) {
          src = a.aq + row * row_bytes + (size_t)cc * 16;
          dst[q] = codes + ((size_t)r * S * kStepBytes + (size_t)cc * 16);
        } else {
          const int sc = cc - S * (kStepBytes / 16);
          src = a.as8 + row * row_scales + (size_t)sc * 16;
          dst[q] = scales + ((size_t)r * S * kStepScales + (size_t)sc * 16);
        }
        v[q] = *reinterpret_cast<const u32x4_t*>(src);
      }
    }
#pragma unroll
    for (int q = 0; q < kStageBatch; ++q)
      if (dst[q]) *reinterpret_cast<u32x4_t*>(dst[q]) = v[q];
  }
}

template <int kRole>
__global__ __launch_bounds__(kThreads) void gemm_fp4_kernel(GemmArgs args) {
  extern __shared__ __align__(16) unsigned char smem[];
  const GemmProblem& a = args.p[1];
  const int S = a.K / kStepValues, tiles = a.N / kRowsPerWg;
  const int per_job = tiles * S;  // > kDepth for every accepted shape
  const StreamMap m = stream_map(a.b.ctrl[2], tiles, S, args.stream_wgs);
  if ((int)blockIdx.x >= m.Wa) return;
  const int64_t lo = stream_begin(blockIdx.x, m), hi = stream_begin(blockIdx.x + 1, m);
  if (lo >= hi) return;  // no items at all
  const int n = (int)(hi - lo);

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int rg = lane >> 3, ch = lane & 7;
  const size_t row_bytes = (size_t)a.K / 2;
  const size_t buf_bytes = (size_t)kFp4JobRoutes * S * (kStepBytes + kStepScales);
  int* info = reinterpret_cast<int*>(smem + kJobBufs * buf_bytes);  // [kJobBufs][kInfoInts]

  const int j0 = (int)(lo / per_job), jlast = (int)((hi - 1) / per_job);
  if (jlast > j0 + 1) return;  // cannot happen: a range holds at most one job's items
  Cursor c{j0, (int)((lo % per_job) / S), (int)(lo % S)};  // the item being summed
  Cursor pc = c;                                              // the next item to request
  int pleft = n;

  // The range's (at most two) jobs, read before any weight is requested so
  // that no wait for them queues behind the weight stream; job j sits in
  // buffer j - j0.
  int4 jd0, jd1 = make_int4(0, 0, 0, 0);
  int rt0[kFp4JobRoutes], rt1[kFp4JobRoutes] = {};
  load_job(a, j0, jd0, rt0);
  if (jlast > j0) load_job(a, j0 + 1, jd1, rt1);
  // experts of the two jobs, uniform across the workgroup
  const int e0 = __builtin_amdgcn_readfirstlane(jd0.x), e1 = __builtin_amdgcn_readfirstlane(jd1.x);
  int pe = e0;

  u32x4_t wa[kDepth], wb[kDepth];
  uint32_t sw[kDepth];
  // this lane's offsets within its wave's 16-row group: rows rg (and rg + 8),
  // bytes 16ch.. of an item; four scale bytes per lane in the reordered scales
  const size_t lane_w = (size_t)rg * row_bytes + ch * 16;
  const size_t lane_s = (size_t)lane * 4;
  // Requests the item under the requesting cursor into buffer q; past the
  // range's end the cursor stays on its last item (a repeat read, from L2).
  auto request = [&](int q) {
    const size_t group = (size_t)pe * (a.N / 16) + pc.tile * (kRowsPerWg / 16) + wave;  // 16-row group
    const uint8_t* p = a.w + (group * 16 * row_bytes + (size_t)pc.s * kStepBytes) + lane_w;
    wa[q] = load_stream16(p);
    wb[q] = load_stream16(p + 8 * row_bytes);
    sw[q] = __builtin_nontemporal_load(
        reinterpret_cast<const uint32_t*>(a.ws8 + ((group * S + pc.s) * kWave * 4) + lane_s));
    if (--pleft > 0) {
      const int pj = pc.j;
      advance(pc, tiles, S);
      if (pc.j != pj) pe = e1;
    }
  };
#pragma unroll
  for (int q = 0; q < kDepth; ++q) request(q);

  stage_job(a, jd0, rt0, S, smem, info);
  if (jlast > j0) stage_job(a, jd1, rt1, S, smem + buf_bytes, info + kInfoInts);
  __syncthreads();

  float acc_a[kFp4JobRoutes], acc_b[kFp4JobRoutes];
#pragma unroll
  for (int i = 0; i < kFp4JobRoutes; ++i) acc_a[i] = acc_b[i] = 0.f;

  // One item from buffer q; `refill` requests the item kDepth further on.
  auto process = [&](int q, bool refill) {
    const int buf = c.j - j0;
    const int nr = info[buf * kInfoInts];
    const unsigned char* xc = smem + buf * buf_bytes;
    const unsigned char* xs = xc + (size_t)kFp4JobRoutes * S * kStepBytes;

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
    // weight scales of groups 2ch and 2ch + 1 of rows rg (bytes 0, 1) and rg + 8 (bytes 2, 3)
    const float s0a = e4m3_value(sw[q]), s1a = e4m3_value(sw[q] >> 8);
    const float s0b = e4m3_value(sw[q] >> 16), s1b = e4m3_value(sw[q] >> 24);
    if (refill) request(q);

#pragma unroll
    for (int i = 0; i < kFp4JobRoutes; ++i) {
      if (i < nr) {
        const size_t rs = (size_t)i * S + c.s;
        const u32x4_t xw = *reinterpret_cast<const u32x4_t*>(xc + rs * kStepBytes + ch * 16);
        const uint32_t xsv = *reinterpret_cast<const uint16_t*>(xs + rs * kStepScales + ch * 2);
        float pa0 = 0.f, pb0 = 0.f, pa1 = 0.f, pb1 = 0.f;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const half2_t x0 = e2m1x2_to_f16x2<0>(xw[d]), x1 = e2m1x2_to_f16x2<1>(xw[d]);
          const half2_t x2 = e2m1x2_to_f16x2<2>(xw[d]), x3 = e2m1x2_to_f16x2<3>(xw[d]);
          float& pa = d < 2 ? pa0 : pa1;
          float& pb = d < 2 ? pb0 : pb1;
          pa = __builtin_amdgcn_fdot2(w0[4 * d], x0, pa, false);
          pb = __builtin_amdgcn_fdot2(w1[4 * d], x0, pb, false);
          pa = __builtin_amdgcn_fdot2(w0[4 * d + 1], x1, pa, false);
          pb = __builtin_amdgcn_fdot2(w1[4 * d + 1], x1, pb, false);
          pa = __builtin_amdgcn_fdot2(w0[4 * d + 2], x2, pa, false);
          pb = __builtin_amdgcn_fdot2(w1[4 * d + 2], x2, pb, false);
          pa = __builtin_amdgcn_fdot2(w0[4 * d + 3], x3, pa, false);
          pb = __builtin_amdgcn_fdot2(w1[4 * d + 3], x3, pb, false);
        }
        const float sx0 = e4m3_value(xsv), sx1 = e4m3_value(xsv >> 8);
        acc_a[i] = fmaf(pa1 * sx1, s1a, fmaf(pa0 * sx0, s0a, acc_a[i]));
        acc_b[i] = fmaf(pb1 * sx1, s1b, fmaf(pb0 * sx0, s0b, acc_b[i]));
      }
    }
    return nr;
  };
  // After item `done` (0-based in the range): at a tile's last step, or the
  // range's last item, the rows' sums go to the tile's partial slot (rows rg
  // and rg + 8; the eight lanes of a row hold consecutive 32-value pieces).
  auto finish = [&](int done, int nr) {
    if (c.s == S - 1 || done == n - 1) {
      const int64_t tile_item = ((int64_t)c.j * tiles + c.tile) * S;
      const int slot = (int)blockIdx.x - stream_owner(tile_item, m);
      const int row0 = c.tile * kRowsPerWg + wave * 16;
      const int* rts = info + (c.j - j0) * kInfoInts + 2;
#pragma unroll
      for (int i = 0; i < kFp4JobRoutes; ++i) {
        if (i < nr) {
          const float ta = group_sum<8>(acc_a[i]), tb = group_sum<8>(acc_b[i]);
          if (ch == 0) {
            float* dst = a.part + ((size_t)slot * a.R + rts[i]) * a.N + row0;
            dst[rg] = ta;
            dst[rg + 8] = tb;
          }
        }
        acc_a[i] = acc_b[i] = 0.f;
      }
    }
    advance(c, tiles, S);
  };

  int it = 0;
  for (; it + kDepth <= n; it += kDepth) {
#pragma unroll
    for (int q = 0; q < kDepth; ++q) finish(it + q, process(q, true));
  }
#pragma unroll
  for (int q = 0; q < kDepth - 1; ++q)
    if (it + q < n) finish(it + q, process(q, false));
}

// The weight scales [rows, K/16] (rows = E * N, a multiple of 16) into the
// kernel's layout: for 16-row group g, item s (256 values) and lane l =
// 8 rg + ch, bytes ((g * S + s) * 64 + l) * 4 + {0, 1, 2, 3} = scales of
// groups 2ch and 2ch + 1 (16 values each) of item s in rows 16g + rg, then
// 16g + rg + 8. One thread per output word.
__global__ void reorder_fp4_scales_kernel(const uint8_t* src, uint32_t* dst, size_t words, int S) {
  const size_t w = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (w >= words) return;
  const int l = (int)(w % kWave), rg = l >> 3, ch = l & 7;
  const size_t gs = w / kWave, g = gs / S;
  const int s = (int)(gs - g * S);
  const size_t row_scales = (size_t)S * kStepScales;
  const uint8_t* a = src + (g * 16 + rg) * row_scales + (size_t)s * kStepScales + 2 * ch;
  const uint8_t* b = a + 8 * row_scales;
  dst[w] = (uint32_t)a[0] | ((uint32_t)a[1] << 8) | ((uint32_t)b[0] << 16) | ((uint32_t)b[1] << 24);
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

size_t gemm_fp4_lds_bytes(int K) {
  const size_t S = (size_t)K / kStepValues;
  return kJobBufs * kFp4JobRoutes * S * (kStepBytes + kStepScales) + kJobBufs * kInfoInts * sizeof(int);
}

int gemm_fp4_resident_wgs(int K) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(gemm_fp4_kernel<1>),
                                                   kThreads, gemm_fp4_lds_bytes(K)) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return cus * per_cu;
}

hipError_t launch_gemm_fp4(const GemmArgs& a, int role, int grid, hipStream_t s) {
  const size_t lds = gemm_fp4_lds_bytes(a.p[1].K);
  if (role == 1)
    hipLaunchKernelGGL(gemm_fp4_kernel<1>, dim3(grid), dim3(kThreads), lds, s, a);
  else
    hipLaunchKernelGGL(gemm_fp4_kernel<2>, dim3(grid), dim3(kThreads), lds, s, a);
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
