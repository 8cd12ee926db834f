// Routing, activation quantisation and expert bucketing.
//
// Routing follows the vLLM "mega_moe" page (top_k_pick, _ordered): FP32
// sigmoid scores, FP32 keys score + bias compared through a monotone integer
// image, top_k rounds of a wave-wide maximum with ties to the lower expert,
// weights = picked score / (FP32 sum of picked scores in pick order) * scale.
// The activation quantiser is the same page's epilogue: per 128 values,
// scale = max(amax, 1e-10) / 448 (IEEE divide), optionally rounded up to a
// power of two after flooring it at 1e-10, then v * (1 / scale) encoded to
// e4m3.
//
// Launch: one 1024-thread workgroup per 4 tokens (2 when there are more than
// 4); waves 0..3 (or 0..1, on their own SIMDs) each route one token while the
// other waves quantise the workgroup's tokens' x. With one workgroup the
// routes are grouped by expert right away (by one wave when there are at most
// 64 routes, else through LDS); with several, the last workgroup to arrive
// (atomic counter, reset by that workgroup) does it.
#include "kernels.h"
#include "device_common.h"
#include "fp4_device.h"

namespace moe {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;  // 16
// Tokens per workgroup, one routing wave each, one per SIMD: routing is
// VALU-issue bound (FP64 sigmoid, 64-bit DPP maxima), so two routing waves
// on a SIMD take twice as long (measured on MI355X at M = 8: 11.6 us as two
// workgroups against 13.0 us as one). Up to 4 tokens run in one workgroup
// (no cross-workgroup handoff); more run 2 to a workgroup: on one GPU's FP4
// share (M = 16, E = 384, top-6) the kernel took 17.0 us at 4 tokens per
// workgroup and 13.6 us at 2, and the DeepSeek-V3 shapes at M = 8..64 were
// even (measured on MI355X).
constexpr int kTokensPerWg = 4;
constexpr int kTokensPerWgMany = 2;
__host__ __device__ inline int tokens_per_wg(int M) { return M <= kTokensPerWg ? kTokensPerWg : kTokensPerWgMany; }

// Monotone image of an FP32 value in uint32: a > b as floats (with -0 < +0)
// iff key(a) > key(b). Negatives flip every bit, the rest flip the sign bit.
__device__ __forceinline__ uint32_t ordered_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float sigmoid_f32(float z) {
  // FP32 rounding of the sigmoid evaluated in FP64.
  return (float)(1.0 / (1.0 + exp(-(double)z)));
}

template <int kCtrl>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const int lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)v, kCtrl, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), kCtrl, 0xF, 0xF, false);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int lane) {
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, lane);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), lane);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// Wave-wide maximum: DPP permutations inside each row of 16 lanes (swap
// neighbours, swap pairs, half-row mirror, row mirror), then the four row
// results through readlane. Every lane returns the same value.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = max_u64(v, dpp_u64<0xB1>(v));   // quad_perm [1,0,3,2]
  v = max_u64(v, dpp_u64<0x4E>(v));   // quad_perm [2,3,0,1]
  v = max_u64(v, dpp_u64<0x141>(v));  // row_half_mirror
  v = max_u64(v, dpp_u64<0x140>(v));  // row_mirror
  return max_u64(max_u64(readlane_u64(v, 0), readlane_u64(v, 16)),
                 max_u64(readlane_u64(v, 32), readlane_u64(v, 48)));
}

// One wave: the picks and weights of token t. Lane l holds experts
// l + 64 j for j < kPer (kPer >= E / 64).
template <int kPer>
__device__ void route_token(const RouteQuantArgs& a, int t, int lane, int* ids_l) {
  const int E = a.E;
  float score[kPer];
  uint64_t key[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    score[j] = 0.f;
    key[j] = 0;
    const int e = lane + kWave * j;
    if (e < E) {
      const size_t at = (size_t)t * E + e;
      const float z = a.logits_bf16 ? bf16_value(((const uint16_t*)a.logits)[at])
                                    : ((const float*)a.logits)[at];
      const float s = sigmoid_f32(z);
      const float biased = s + a.bias[e];
      score[j] = s;
      // high word: the key; low word: ~e, so that equal keys favour lower e
      key[j] = ((uint64_t)ordered_key(biased) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
    }
  }
  float total = 0.f;
  int my_id = 0;
  float my_score = 0.f;
  for (int r = 0; r < a.k; ++r) {
    uint64_t best = key[0];
#pragma unroll
    for (int j = 1; j < kPer; ++j) best = max_u64(best, key[j]);
    best = wave_max_u64(best);
    const int winner = (int)(0xFFFFFFFFu - (uint32_t)best);
    const int owner = winner & (kWave - 1);
    const int slot = winner / kWave;
    float s_slot = 0.f;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      if (j == slot) {
        s_slot = score[j];
        if (lane == owner) key[j] = 0;
      }
    }
    const float s = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s_slot), owner));
    total = total + s;
    if (lane == r) {
      my_id = winner;
      my_score = s;
    }
  }
  if (lane < a.k) {
    const float w = (my_score / total) * a.routed_scale;
    const size_t at = (size_t)t * a.k + lane;
    // written through to the device coherence point: another workgroup (on
    // another XCD, with its own L2) may read it in the cross-workgroup handoff
    __hip_atomic_store(a.ids + at, my_id, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    a.weights[at] = w;
    ids_l[at] = my_id;
  }
}

__device__ void route_token_any(const RouteQuantArgs& a, int t, int lane, int* ids_l) {
  const int per = (a.E + kWave - 1) / kWave;
  if (per <= 1) route_token<1>(a, t, lane, ids_l);
  else if (per <= 2) route_token<2>(a, t, lane, ids_l);
  else if (per <= 4) route_token<4>(a, t, lane, ids_l);
  else if (per <= 8) route_token<8>(a, t, lane, ids_l);
  else route_token<16>(a, t, lane, ids_l);
}

// Threads tid0.. (tid0 a multiple of the wave size): the 128-blocks of tokens
// [t0, t0 + ntok), eight lanes per block and sixteen values per lane; loads
// of up to four blocks per lane are issued before any is used.
__device__ void quant_tokens(const RouteQuantArgs& a, int t0, int ntok, int tid0) {
  const int kGroups = (kThreads - tid0) / 8;
  constexpr int kBatch = 4;
  const int group = (threadIdx.x - tid0) / 8, sub = threadIdx.x % 8;
  const int nblk = a.H / kTile;
  const int items = ntok * nblk;
  for (int base = 0; base < items; base += kBatch * kGroups) {
    u32x4_t lo[kBatch], hi[kBatch];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const int item = base + q * kGroups + group;
      if (item < items) {
        const size_t at = (size_t)(t0 + item / nblk) * a.H + (size_t)(item % nblk) * kTile + sub * 16;
        lo[q] = *reinterpret_cast<const u32x4_t*>(a.x + at);
        hi[q] = *reinterpret_cast<const u32x4_t*>(a.x + at + 8);
      }
    }
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const int item = base + q * kGroups + group;
      if (item < items) {  // the same for all eight lanes of a group
        float v[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[2 * i] = bf16_value(lo[q][i] & 0xFFFFu);
          v[2 * i + 1] = bf16_value(lo[q][i] >> 16);
          v[8 + 2 * i] = bf16_value(hi[q][i] & 0xFFFFu);
          v[8 + 2 * i + 1] = bf16_value(hi[q][i] >> 16);
        }
        const int t = t0 + item / nblk, blk = item % nblk;
        const size_t at = (size_t)t * a.H + (size_t)blk * kTile + sub * 16;
        if (a.fp4) {  // this lane's 16 values are one FP4 group
          uint32_t packed[2];
          const uint32_t sbyte = stage_fp4_group(v, packed);
          *reinterpret_cast<uint2*>(a.xq + at / 2) = make_uint2(packed[0], packed[1]);
          a.xs4[at / kFp4Group] = (uint8_t)sbyte;
          continue;
        }
        float amax = kAmaxFloor;
#pragma unroll
        for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
        amax = group_max<8>(amax);
        // scale = amax / 448, optionally rounded up to a power of two; codes
        // = e4m3(v * (1 / scale))
        auto emit = [&](int ue8m0, uint8_t* xq, float* xs) {
          float s = amax / kFp8Max;
          if (ue8m0) {
            const uint32_t b = __float_as_uint(fmaxf(s, kAmaxFloor));
            s = __uint_as_float(((b >> 23) + ((b & 0x7FFFFFu) != 0u)) << 23);
          }
          const float inv = 1.0f / s;
          u32x4_t out;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            out[w] = e4m3x4_encode(v[4 * w] * inv, v[4 * w + 1] * inv, v[4 * w + 2] * inv,
                                   v[4 * w + 3] * inv);
          }
          *reinterpret_cast<u32x4_t*>(xq + at) = out;
          if (sub == 0) xs[(size_t)t * nblk + blk] = s;
        };
        emit(a.ue8m0, a.xq, a.xs);
        if (a.xq2) emit(a.ue8m0_2, a.xq2, a.xs2);  // the shared expert's own scale rule
      }
    }
  }
}

struct Lds {
  uint64_t* mask;  // [E][W] token bitmask of every expert
  int* ids;        // [M*k] picks
  int* first;      // [E] first route slot of each expert
  int* jbase;      // [E] first job of each expert (FP4 form)
  int* scratch;    // [3 * kWaves] per-wave scan totals
};

__device__ __forceinline__ Lds carve(unsigned char* lds, int E, int W, int R) {
  Lds l;
  l.mask = reinterpret_cast<uint64_t*>(lds);
  l.ids = reinterpret_cast<int*>(lds + (size_t)E * W * 8);
  l.first = l.ids + R;
  l.jbase = l.first + E;
  l.scratch = l.jbase + E;
  return l;
}

// Routes of the local experts grouped by expert (local index e - lb),
// experts ascending, each expert's routes in ascending token order (so
// ascending route index).
__device__ void bucket_routes(const RouteQuantArgs& a, const Lds& l) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int E = a.lc, W = a.words, R = a.M * a.k;
  for (int i = tid; i < E * W; i += kThreads) l.mask[i] = 0;
  __syncthreads();
  for (int r = tid; r < R; r += kThreads) {
    const int t = r / a.k;
    const int e = l.ids[r] - a.lb;
    if (e >= 0 && e < E)
      atomicOr(reinterpret_cast<unsigned long long*>(&l.mask[(size_t)e * W + t / 64]), 1ull << (t % 64));
  }
  __syncthreads();
  // thread e owns expert e (E <= kThreads); block-wide exclusive scan of
  // (present, count, jobs) gives each present expert its rank, first slot
  // and first job
  const int jr = a.job_routes;
  int cnt = 0;
  if (tid < E)
    for (int w = 0; w < W; ++w) cnt += __popcll(l.mask[(size_t)tid * W + w]);
  const int present = cnt > 0;
  const int nj = jr > 0 ? (cnt + jr - 1) / jr : 0;
  int inc_p = present, inc_r = cnt, inc_j = nj;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int up_p = __shfl_up(inc_p, o, kWave);
    const int up_r = __shfl_up(inc_r, o, kWave);
    const int up_j = __shfl_up(inc_j, o, kWave);
    if (lane >= o) {
      inc_p += up_p;
      inc_r += up_r;
      inc_j += up_j;
    }
  }
  if (lane == kWave - 1) {
    l.scratch[wave] = inc_p;
    l.scratch[kWaves + wave] = inc_r;
    l.scratch[2 * kWaves + wave] = inc_j;
  }
  __syncthreads();
  int base_p = 0, base_r = 0, base_j = 0, all_p = 0, all_j = 0;
  for (int w = 0; w < kWaves; ++w) {
    const int tp = l.scratch[w], tr = l.scratch[kWaves + w], tj = l.scratch[2 * kWaves + w];
    if (w < wave) {
      base_p += tp;
      base_r += tr;
      base_j += tj;
    }
    all_p += tp;
    all_j += tj;
  }
  if (present) {
    const int u = base_p + inc_p - 1;
    const int o = base_r + inc_r - cnt;
    const int jb = base_j + inc_j - nj;
    a.b.uexp[u] = tid;
    a.b.uoff[u] = o;
    a.b.ucnt[u] = cnt;
    l.first[tid] = o;
    l.jbase[tid] = jb;
    for (int p = 0; p < nj; ++p) a.b.jobs[jb + p] = make_int4(tid, o + p * jr, min(jr, cnt - p * jr), 0);
  }
  if (tid == 0) {
    a.b.ctrl[1] = all_p;
    a.b.ctrl[2] = all_j;
  }
  __syncthreads();
  for (int r = tid; r < R; r += kThreads) {
    const int e = l.ids[r] - a.lb;
    if (e < 0 || e >= E) continue;
    const int t = r / a.k;
    const uint64_t* m = l.mask + (size_t)e * W;
    int before = 0;
    for (int w = 0; w < t / 64; ++w) before += __popcll(m[w]);
    before += __popcll(m[t / 64] & ((1ull << (t % 64)) - 1ull));
    a.b.routes[l.first[e] + before] = r;
    if (jr > 0) a.b.rjob[r] = l.jbase[e] + before / jr;
  }
}

// The same grouping by one wave when there are at most 64 routes: lane r
// holds (local expert << 16) | r (non-local routes sort last as padding), a
// bitonic network over the wave sorts the keys (experts ascending, routes
// ascending within an expert), and the first lane of each expert's run
// writes its bucket. No LDS, no barrier.
__device__ void bucket_routes_wave(const RouteQuantArgs& a, const int* ids, int lane) {
  const int e_own = lane < a.M * a.k ? ids[lane] - a.lb : -1;
  const bool mine = e_own >= 0 && e_own < a.lc;
  const int R = __popcll(__ballot(mine));  // local routes
  uint32_t v = mine ? ((uint32_t)e_own << 16) | (uint32_t)lane : 0xFFFFFFFFu;
#pragma unroll
  for (int k = 2; k <= kWave; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const uint32_t w = (uint32_t)__shfl_xor((int)v, j, kWave);
      const bool ascending = (lane & k) == 0;
      const bool lower = (lane & j) == 0;
      v = (lower == ascending) ? min(v, w) : max(v, w);
    }
  }
  const int e = (int)(v >> 16);
  const int prev = __shfl_up(e, 1, kWave);
  const bool valid = lane < R;
  const bool first = valid && (lane == 0 || e != prev);
  const uint64_t starts = __ballot(first);
  const int route = (int)(v & 0xFFFFu);
  if (valid) a.b.routes[lane] = route;
  const uint64_t later = lane == kWave - 1 ? 0ull : starts >> (lane + 1);
  const int next = later ? lane + 1 + __builtin_ctzll(later) : R;  // end of the run (first lanes)
  if (first) {
    const int u = __popcll(starts & ((1ull << lane) - 1ull));
    a.b.uexp[u] = e;
    a.b.uoff[u] = lane;
    a.b.ucnt[u] = next - lane;
  }
  if (lane == 0) a.b.ctrl[1] = __popcll(starts);
  const int jr = a.job_routes;
  if (jr > 0) {
    // each run cut into jobs of jr entries: a scan of the runs' job counts
    // gives their first jobs; the run's start, end and first job then reach
    // every lane of the run through an inclusive max-scan (all three rise
    // from run to run)
    const int nj = first ? (next - lane + jr - 1) / jr : 0;
    int inc = nj;
    int rs = first ? lane : -1, re = first ? next : -1;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int up = __shfl_up(inc, o, kWave);
      if (lane >= o) inc += up;
    }
    int rb = first ? inc - nj : -1;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int up_s = __shfl_up(rs, o, kWave), up_e = __shfl_up(re, o, kWave), up_b = __shfl_up(rb, o, kWave);
      if (lane >= o) {
        rs = max(rs, up_s);
        re = max(re, up_e);
        rb = max(rb, up_b);
      }
    }
    if (valid) {
      const int pos = lane - rs, j = rb + pos / jr;
      a.b.rjob[route] = j;
      if (pos % jr == 0) a.b.jobs[j] = make_int4(e, lane, min(jr, re - lane), 0);
    }
    const int jobs = __shfl(inc, kWave - 1, kWave);
    if (lane == 0) a.b.ctrl[2] = jobs;
  }
}

__device__ __forceinline__ void bucket_any(const RouteQuantArgs& a, const Lds& l) {
  if (a.M * a.k <= kWave) {
    if (threadIdx.x < kWave) bucket_routes_wave(a, l.ids, threadIdx.x);
  } else {
    bucket_routes(a, l);
  }
}

__global__ __launch_bounds__(kThreads) void route_quant_kernel(RouteQuantArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  __shared__ int is_last;
  const Lds l = carve(lds, a.E, a.words, a.M * a.k);
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int tpw = tokens_per_wg(a.M);
  const int t0 = blockIdx.x * tpw;
  const int ntok = min(tpw, a.M - t0);
  // the routing waves (one per token) and the quantising waves run side by side
  if (wave < tpw) {
    if (wave < ntok) route_token_any(a, t0 + wave, lane, l.ids);
  } else {
    quant_tokens(a, t0, ntok, tpw * kWave);
  }
  if (gridDim.x == 1) {
    __syncthreads();
    bucket_any(a, l);
    return;
  }
  // Count arrivals once this workgroup's picks are published; the last
  // arrival reads every workgroup's picks. The picks were stored at device
  // scope, so waiting for those stores to complete publishes them: no fence
  // here writes back the rest of the L2 (which a release fence would do, at
  // the cost of every dirty line earlier kernels left there).
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0)
    is_last = __hip_atomic_fetch_add(a.b.ctrl, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
              (int)gridDim.x - 1;
  __syncthreads();
  if (!is_last) return;
  if (threadIdx.x == 0) __hip_atomic_store(a.b.ctrl, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (int r = threadIdx.x; r < a.M * a.k; r += kThreads) {
    const int id = __hip_atomic_load(a.ids + r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    l.ids[r] = min(max(id, 0), a.E - 1);  // keeps the bucket indexing in bounds whatever it reads
  }
  __syncthreads();
  bucket_any(a, l);
}

__global__ void codec_check_kernel(const float* in, uint8_t* q, float* dq, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  q[i] = (uint8_t)e4m3x2_encode(in[i], 0.f);
  const uint32_t c = (uint32_t)i & 0xFFu;
  const int variant = (i >> 8) & 3;  // which byte of a word carries the code
  const uint32_t word = c << (8 * variant);
  const half2_t h = variant >= 2 ? e4m3x2_to_f16x2<true>(word) : e4m3x2_to_f16x2<false>(word);
  dq[i] = (float)((variant & 1) ? h.y : h.x);
}

}  // namespace

size_t route_quant_lds_bytes(int E, int words, int routes) {
  return (size_t)E * words * 8 + (size_t)routes * 4 + (size_t)E * 8 + 3 * kWaves * 4;
}

hipError_t launch_route_quant(const RouteQuantArgs& a, hipStream_t s) {
  const int tpw = tokens_per_wg(a.M);
  const int grid = (a.M + tpw - 1) / tpw;
  hipLaunchKernelGGL(route_quant_kernel, dim3(grid), dim3(kThreads),
                     route_quant_lds_bytes(a.E, a.words, a.M * a.k), s, a);
  return hipGetLastError();
}

hipError_t launch_codec_check(const float* in, uint8_t* q, float* dq, int n, hipStream_t s) {
  hipLaunchKernelGGL(codec_check_kernel, dim3((n + 255) / 256), dim3(256), 0, s, in, q, dq, n);
  return hipGetLastError();
}

}  // namespace moe
