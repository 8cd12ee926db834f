// Routing, activation quantisation and expert bucketing: one workgroup per
// token, the last workgroup to finish groups the routes by expert.
//
// Routing follows the vLLM "mega_moe" page (top_k_pick, _ordered): FP32
// sigmoid scores, FP32 keys score + bias compared through a monotone integer
// image, top_k rounds of a wave-wide maximum with ties to the lower expert,
// weights = picked score / (FP32 sum of picked scores in pick order) * scale.
// The activation quantiser is the same page's epilogue: per 128 values,
// scale = max(amax, 1e-10) / 448 (IEEE divide), optionally rounded up to a
// power of two after flooring it at 1e-10, then v * (1 / scale) encoded to
// e4m3.
#include "kernels.h"
#include "device_common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxPerLane = 16;  // experts per lane: E <= 1024

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

// Wave 0 of the token's workgroup: picks and weights of token t.
__device__ void route_token(const RouteQuantArgs& a, int t, int lane) {
  const int E = a.E;
  const int per = (E + kWave - 1) / kWave;
  float score[kMaxPerLane];
  uint64_t key[kMaxPerLane];
#pragma unroll
  for (int j = 0; j < kMaxPerLane; ++j) {
    score[j] = 0.f;
    key[j] = 0;
    const int e = lane + kWave * j;
    if (j < per && e < E) {
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
    uint64_t best = 0;
#pragma unroll
    for (int j = 0; j < kMaxPerLane; ++j)
      if (j < per) best = key[j] > best ? key[j] : best;
    best = wave_max_u64(best);
    const int winner = (int)(0xFFFFFFFFu - (uint32_t)best);
    const int owner = winner & (kWave - 1);
    const int slot = winner / kWave;
    float s_slot = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxPerLane; ++j) {
      if (j == slot) {
        s_slot = score[j];
        if (lane == owner) key[j] = 0;
      }
    }
    const float s = __shfl(s_slot, owner, kWave);
    total = total + s;
    if (lane == r) {
      my_id = winner;
      my_score = s;
    }
  }
  if (lane < a.k) {
    const float w = (my_score / total) * a.routed_scale;
    a.ids[(size_t)t * a.k + lane] = my_id;
    a.weights[(size_t)t * a.k + lane] = w;
  }
}

// Threads [first, first + count) of the workgroup quantise token t: eight
// lanes per 128-block, sixteen values per lane.
__device__ void quant_token(const RouteQuantArgs& a, int t, int first, int count) {
  const int me = threadIdx.x - first;
  const int groups = count / 8;
  const int g = me / 8, sub = me % 8;
  const int nblk = a.H / kTile;
  for (int blk = g; blk < nblk; blk += groups) {
    const size_t base = (size_t)t * a.H + (size_t)blk * kTile + sub * 16;
    const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(a.x + base);
    const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(a.x + base + 8);
    float v[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_value(lo[i] & 0xFFFFu);
      v[2 * i + 1] = bf16_value(lo[i] >> 16);
      v[8 + 2 * i] = bf16_value(hi[i] & 0xFFFFu);
      v[8 + 2 * i + 1] = bf16_value(hi[i] >> 16);
    }
    float amax = kAmaxFloor;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = group_max<8>(amax);
    float s = amax / kFp8Max;
    if (a.ue8m0) {
      const uint32_t b = __float_as_uint(fmaxf(s, kAmaxFloor));
      s = __uint_as_float(((b >> 23) + ((b & 0x7FFFFFu) != 0u)) << 23);
    }
    const float inv = 1.0f / s;
    u32x4_t q;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      q[w] = e4m3_encode(v[4 * w] * inv) | (e4m3_encode(v[4 * w + 1] * inv) << 8) |
             (e4m3_encode(v[4 * w + 2] * inv) << 16) | (e4m3_encode(v[4 * w + 3] * inv) << 24);
    }
    *reinterpret_cast<u32x4_t*>(a.xq + base) = q;
    if (sub == 0) a.xs[(size_t)t * nblk + blk] = s;
  }
}

// The last workgroup: routes grouped by expert, experts in ascending order,
// each expert's routes in ascending token order.
__device__ void bucket_routes(const RouteQuantArgs& a, unsigned char* lds) {
  const int tid = threadIdx.x;
  const int E = a.E, W = a.words, R = a.M * a.k;
  uint64_t* mask = reinterpret_cast<uint64_t*>(lds);               // [E][W]
  int* first = reinterpret_cast<int*>(lds + (size_t)E * W * 8);    // [E]
  int* wave_tot = first + E;                                       // [2][4]

  for (int i = tid; i < E * W; i += kThreads) mask[i] = 0;
  __syncthreads();
  for (int r = tid; r < R; r += kThreads) {
    const int e = __hip_atomic_load(a.ids + r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int t = r / a.k;
    atomicOr(reinterpret_cast<unsigned long long*>(&mask[(size_t)e * W + t / 64]),
             1ull << (t % 64));
  }
  __syncthreads();

  // Each thread owns a contiguous run of experts; a block-wide exclusive scan
  // gives every present expert its rank and its first route slot.
  const int per = (E + kThreads - 1) / kThreads;  // <= 4
  int cnt[4];
  int present = 0, routes = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    cnt[q] = 0;
    const int e = tid * per + q;
    if (q < per && e < E) {
      for (int w = 0; w < W; ++w) cnt[q] += __popcll(mask[(size_t)e * W + w]);
      present += cnt[q] > 0;
      routes += cnt[q];
    }
  }
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  int inc_p = present, inc_r = routes;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int up_p = __shfl_up(inc_p, o, kWave);
    const int up_r = __shfl_up(inc_r, o, kWave);
    if (lane >= o) {
      inc_p += up_p;
      inc_r += up_r;
    }
  }
  if (lane == kWave - 1) {
    wave_tot[wave] = inc_p;
    wave_tot[4 + wave] = inc_r;
  }
  __syncthreads();
  int base_p = 0, base_r = 0, all_p = 0;
  for (int w = 0; w < kThreads / kWave; ++w) {
    if (w < wave) {
      base_p += wave_tot[w];
      base_r += wave_tot[4 + w];
    }
    all_p += wave_tot[w];
  }
  int u = base_p + inc_p - present;
  int o = base_r + inc_r - routes;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = tid * per + q;
    if (q < per && e < E) {
      first[e] = o;
      if (cnt[q] > 0) {
        a.b.uexp[u] = e;
        a.b.uoff[u] = o;
        a.b.ucnt[u] = cnt[q];
        ++u;
        o += cnt[q];
      }
    }
  }
  if (tid == 0) a.b.ctrl[1] = all_p;
  __syncthreads();
  for (int r = tid; r < R; r += kThreads) {
    const int e = __hip_atomic_load(a.ids + r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int t = r / a.k;
    const uint64_t* m = mask + (size_t)e * W;
    int before = 0;
    for (int w = 0; w < t / 64; ++w) before += __popcll(m[w]);
    before += __popcll(m[t / 64] & ((1ull << (t % 64)) - 1ull));
    a.b.routes[first[e] + before] = r;
  }
}

__global__ __launch_bounds__(kThreads) void route_quant_kernel(RouteQuantArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  __shared__ int is_last;
  const int t = blockIdx.x;
  const int wave = threadIdx.x / kWave;
  if (wave == 0) {
    route_token(a, t, threadIdx.x);
  } else {
    quant_token(a, t, kWave, kThreads - kWave);
  }
  // Publish this token's picks, then count arrivals; the last arrival sees
  // every token's picks.
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const int prev = atomicAdd(a.b.ctrl, 1);
    is_last = prev == a.M - 1;
  }
  __syncthreads();
  if (!is_last) return;
  __threadfence();
  if (threadIdx.x == 0) __hip_atomic_store(a.b.ctrl, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  bucket_routes(a, lds);
}

__global__ void codec_check_kernel(const float* in, uint8_t* q, float* dq, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  q[i] = (uint8_t)e4m3_encode(in[i]);
  const uint32_t c = (uint32_t)i & 0xFFu;
  const int variant = (i >> 8) & 3;  // which byte of a word carries the code
  const uint32_t word = c << (8 * variant);
  const half2_t h = variant >= 2 ? e4m3x2_to_f16x2<true>(word) : e4m3x2_to_f16x2<false>(word);
  dq[i] = (float)((variant & 1) ? h.y : h.x);
}

}  // namespace

size_t route_quant_lds_bytes(int E, int words) {
  return (size_t)E * words * 8 + (size_t)E * 4 + 8 * 4;
}

hipError_t launch_route_quant(const RouteQuantArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(route_quant_kernel, dim3(a.M), dim3(kThreads),
                     route_quant_lds_bytes(a.E, a.words), s, a);
  return hipGetLastError();
}

hipError_t launch_codec_check(const float* in, uint8_t* q, float* dq, int n, hipStream_t s) {
  hipLaunchKernelGGL(codec_check_kernel, dim3((n + 255) / 256), dim3(256), 0, s, in, q, dq, n);
  return hipGetLastError();
}

}  // namespace moe
