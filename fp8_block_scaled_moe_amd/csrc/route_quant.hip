// Routing, activation quantisation and expert bucketing (the arithmetic is
// in route_device.h, shared with the routing prologue of the persistent
// GEMM1).
//
// Launch: one 1024-thread routing workgroup per 4 tokens (2 when there are
// more than 4); its waves 0..3 (or 0..1, on their own SIMDs) each route one
// token while its other waves quantise. Workgroups that only quantise follow
// when there are few routing workgroups; all quantising waves share out the
// 128-blocks of every token. With one routing workgroup the routes are
// grouped by expert right away (by one wave when there are at most 64
// routes, else through LDS); with several, the last routing workgroup to
// arrive (atomic counter, reset by that workgroup) does it.
#include <algorithm>

#include "fp4_device.h"
#include "route_device.h"

namespace moe {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;  // 16
// Tokens per workgroup, one routing wave each. Up to 16 tokens are routed
// in one workgroup, so no handoff between workgroups is needed (4 slots at
// M <= 4, the other 12 waves quantising). A routing wave's selection is a
// chain of dependent cross-lane steps, so waves sharing a SIMD overlap
// well: on MI355X the kernel took 6.2 us at DeepSeek-V3 shapes with M = 8
// in one workgroup against 9.0 us over four, and 10.1 against 12.1 us at
// M = 16. Past 16 tokens they run 2 to a workgroup and the last workgroup
// to arrive groups the routes.
constexpr int kTokensPerWgFew = 4;
constexpr int kTokensPerWgOne = 16;  // all waves of a workgroup
constexpr int kTokensPerWgMany = 2;
__host__ __device__ inline int tokens_per_wg(int M) {
  return M <= kTokensPerWgFew ? kTokensPerWgFew : M <= kTokensPerWgOne ? M : kTokensPerWgMany;
}
__host__ __device__ inline int routing_wgs(int M) { return (M + tokens_per_wg(M) - 1) / tokens_per_wg(M); }
// Workgroups that only quantise, launched after the routing ones when the
// routing workgroups' quantising waves would take more than one 128-block
// per eight lanes (4 tokens on one workgroup: 56 blocks each at H = 7168,
// against 96 groups of eight lanes).
constexpr int kMaxQuantWgs = 16;
inline int quant_wgs(int M, int H) {
  const int have = routing_wgs(M) * (kThreads - tokens_per_wg(M) * kWave) / 8;
  const int items = M * (H / kTile);
  return items > have ? std::min((items - have + kThreads / 8 - 1) / (kThreads / 8), kMaxQuantWgs) : 0;
}

// One wave: the picks and weights of token t. Lane l holds experts
// l + 64 j for j < kPer (kPer >= E / 64).
template <int kPer>
__device__ void route_token(const RouteQuantArgs& a, int t, int lane, int* ids_l) {
  // slots past E load expert E - 1 and are never opened
  int at[kPer];
  float z[kPer], bias[kPer], score[kPer];
  uint32_t key[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int e = min(lane + kWave * j, a.E - 1);
    at[j] = t * a.E + e;
    bias[j] = a.bias[e];
  }
  load_logits<kPer>(a.logits, a.logits_bf16, at, z);
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    score[j] = sigmoid_f32(z[j]);
    key[j] = ordered_key(score[j] + bias[j]);
  }
  int my_id;
  float my_score, total;
  pick_top_k<kPer>(key, score, a.E, a.k, lane, my_id, my_score, total);
  if (lane < a.k) {
    const size_t at = (size_t)t * a.k + lane;
    // written through to the device coherence point: another workgroup (on
    // another XCD, with its own L2) may read it in the cross-workgroup handoff
    __hip_atomic_store(a.ids + at, my_id, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    a.weights[at] = pick_weight(my_score, total, a.routed_scale);
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

// The 128-blocks of all M tokens, eight lanes per block and sixteen values
// per lane: group g of `groups` takes blocks g, g + groups, ...; loads of up
// to four blocks per lane are issued before any is used.
__device__ void quant_blocks(const RouteQuantArgs& a, int group, int groups) {
  constexpr int kBatch = 4;
  const int sub = threadIdx.x % 8;
  const int nblk = a.H / kTile;
  const int items = a.M * nblk;
  for (int base = 0; base < items; base += kBatch * groups) {
    u32x4_t lo[kBatch], hi[kBatch];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const int item = base + q * groups + group;
      if (item < items) {
        const size_t at = (size_t)(item / nblk) * a.H + (size_t)(item % nblk) * kTile + sub * 16;
        lo[q] = *reinterpret_cast<const u32x4_t*>(a.x + at);
        hi[q] = *reinterpret_cast<const u32x4_t*>(a.x + at + 8);
      }
    }
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const int item = base + q * groups + group;
      if (item < items) {  // the same for all eight lanes of a group
        float v[16];
        bf16x16_values(lo[q], hi[q], v);
        const int t = item / nblk, blk = item % nblk;
        const size_t at = (size_t)t * a.H + (size_t)blk * kTile + sub * 16;
        if (a.fp4) {  // this lane's 16 values are one FP4 group
          uint32_t packed[2];
          const uint32_t sbyte = stage_fp4_group(v, packed);
          *reinterpret_cast<uint2*>(a.xq + at / 2) = make_uint2(packed[0], packed[1]);
          a.xs4[at / kFp4Group] = (uint8_t)sbyte;
          continue;
        }
        const float amax = block_amax8(v);
        float sc;
        *reinterpret_cast<u32x4_t*>(a.xq + at) = fp8_block_codes(v, amax, a.ue8m0, sc);
        if (sub == 0) a.xs[(size_t)t * nblk + blk] = sc;
        if (a.xq2) {  // the shared expert's own scale rule
          *reinterpret_cast<u32x4_t*>(a.xq2 + at) = fp8_block_codes(v, amax, a.ue8m0_2, sc);
          if (sub == 0) a.xs2[(size_t)t * nblk + blk] = sc;
        }
      }
    }
  }
}

struct Lds {
  int* totals;     // [2 * kWaves] per-wave scan totals
  uint64_t* mask;  // [E][W] token bitmask of every expert
  int* ids;        // [M*k] picks
  int* first;      // [E] first route slot of each expert
  int* jbase;      // [E] first job of each expert
};

__device__ __forceinline__ Lds carve(unsigned char* lds, int E, int W, int R) {
  Lds l;
  l.totals = reinterpret_cast<int*>(lds);  // first: read as 16-byte words
  l.mask = reinterpret_cast<uint64_t*>(lds + 2 * kWaves * 4);
  l.ids = reinterpret_cast<int*>(lds + 2 * kWaves * 4 + (size_t)E * W * 8);
  l.first = l.ids + R;
  l.jbase = l.first + E;
  return l;
}

// Inclusive prefix sum over the lanes of a wave: shifts by 1, 2, 4 and 8
// lanes inside each row of 16 (lanes with no source add nothing), then each
// row adds the totals of the rows before it.
__device__ __forceinline__ int wave_prefix_sum(int v, int lane) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31),
            r2 = __builtin_amdgcn_readlane(v, 47);
  const int row = lane / 16;
  return v + (row > 0 ? r0 : 0) + (row > 1 ? r1 : 0) + (row > 2 ? r2 : 0);
}

// Routes of local expert e (its token mask's popcount).
__device__ __forceinline__ int expert_routes(const Lds& l, int e, int W) {
  int c = 0;
  for (int w = 0; w < W; ++w) c += __popcll(l.mask[(size_t)e * W + w]);
  return c;
}

// Jobs of an expert with c routes, at most jr routes each (none when jr = 0).
__device__ __forceinline__ int expert_jobs(int c, int jr) { return jr > 0 ? (c + jr - 1) / jr : 0; }

// Routes of the local experts grouped by expert (local index e - lb),
// experts ascending, each expert's routes in ascending token order (so
// ascending route index). l.ids holds the picks and l.mask is zero.
// 1. Token masks per expert in LDS.
// 2. Thread e owns expert e (E <= 1024): its route count, presence and job
//    count go through a prefix sum over the wave (presence and routes
//    packed in one word: at most 1024 and 8192), the waves' totals through
//    LDS (none with at most 64 experts: wave 0 alone), giving each expert
//    its rank, first route slot and first job.
// 3. Every route finds its slot from its expert's mask.
// Every index written is checked against the buffers' sizes.
__device__ void bucket_routes(const RouteQuantArgs& a, const Lds& l) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int E = a.lc, W = a.words, R = a.M * a.k, jr = a.job_routes, ucap = min(E, R);
  for (int r = tid; r < R; r += kThreads) {
    const int t = r / a.k;
    const int e = l.ids[r] - a.lb;
    if (e >= 0 && e < E)
      atomicOr(reinterpret_cast<unsigned long long*>(&l.mask[(size_t)e * W + t / 64]), 1ull << (t % 64));
  }
  __syncthreads();
  const bool one_wave = E <= kWave;  // then wave 0 alone, with no totals to exchange
  if (!one_wave || wave == 0) {
    const int cnt = tid < E ? expert_routes(l, tid, W) : 0;
    const int present = cnt > 0 ? 1 : 0, nj = expert_jobs(cnt, jr);
    constexpr int kShift = 11;  // presence in bits 0..10, routes above
    const int ipr = wave_prefix_sum(present | (cnt << kShift), lane), ij = wave_prefix_sum(nj, lane);
    int base_pr = 0, base_j = 0, all_pr = 0, all_j = 0;
    if (one_wave) {
      all_pr = __builtin_amdgcn_readlane(ipr, kWave - 1);
      all_j = __builtin_amdgcn_readlane(ij, kWave - 1);
    } else {
      if (lane == kWave - 1) {
        l.totals[wave] = ipr;
        l.totals[kWaves + wave] = ij;
      }
      __syncthreads();
      const int4* t4 = reinterpret_cast<const int4*>(l.totals);
      int tot[2 * kWaves];
#pragma unroll
      for (int q = 0; q < 2 * kWaves / 4; ++q) {
        const int4 v = t4[q];
        tot[4 * q] = v.x;
        tot[4 * q + 1] = v.y;
        tot[4 * q + 2] = v.z;
        tot[4 * q + 3] = v.w;
      }
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        base_pr += w < wave ? tot[w] : 0;
        base_j += w < wave ? tot[kWaves + w] : 0;
        all_pr += tot[w];
        all_j += tot[kWaves + w];
      }
    }
    if (present) {
      const int pr = base_pr + ipr;
      const int u = (pr & ((1 << kShift) - 1)) - 1, o = (pr >> kShift) - cnt, jb = base_j + ij - nj;
      if (u < ucap) {
        a.b.uexp[u] = tid;
        a.b.uoff[u] = o;
        a.b.ucnt[u] = cnt;
      }
      l.first[tid] = o;
      l.jbase[tid] = jb;
      for (int q = 0; q < nj; ++q)
        if (jb + q < R) a.b.jobs[jb + q] = make_int4(tid, o + q * jr, min(jr, cnt - q * jr), 0);
    }
    if (tid == 0) {
      a.b.ctrl[1] = min(all_pr & ((1 << kShift) - 1), ucap);
      a.b.ctrl[2] = min(all_j, R);
    }
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
    const int slot = l.first[e] + before;
    if (slot < R) a.b.routes[slot] = r;
    if (jr > 0) a.b.rjob[r] = l.jbase[e] + before / jr;
  }
}

__device__ __forceinline__ void bucket_any(const RouteQuantArgs& a, const Lds& l) {
  if (a.M * a.k <= kWave) {
    if (threadIdx.x < kWave) bucket_routes_wave(a.b, l.ids, a.M * a.k, a.lb, a.lc, a.job_routes, threadIdx.x);
  } else {
    bucket_routes(a, l);
  }
}

__global__ __launch_bounds__(kThreads) void route_quant_kernel(RouteQuantArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  __shared__ int is_last;
  // Every line of the argument block is read here, under one wait: read at
  // first use, the bucketing's pointers and the grid size each cost a memory
  // round trip in the middle of the kernel.
  asm volatile("" ::"s"(a.logits), "s"(a.lc), "s"(a.b.rjob), "s"(gridDim.x));
  const Lds l = carve(lds, a.E, a.words, a.M * a.k);
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int tpw = tokens_per_wg(a.M);
  const int gr = routing_wgs(a.M);
  const bool routing = (int)blockIdx.x < gr;
  if (routing && a.M * a.k > kWave)  // the token masks of the grouping (read after a barrier)
    for (int i = threadIdx.x; i < a.lc * a.words; i += kThreads) l.mask[i] = 0;
  // the routing waves (one per token) and the quantising waves run side by
  // side; the quantising waves of every workgroup share out the blocks
  if (routing && wave < tpw) {
    const int t = blockIdx.x * tpw + wave;
    if (t < a.M) route_token_any(a, t, lane, l.ids);
  } else {
    const int qw = kWaves - tpw;  // quantising waves of a routing workgroup
    const int w = routing ? blockIdx.x * qw + wave - tpw : gr * qw + (blockIdx.x - gr) * kWaves + wave;
    quant_blocks(a, w * (kWave / 8) + lane / 8, (gr * qw + (gridDim.x - gr) * kWaves) * (kWave / 8));
  }
  if (!routing) return;
  if (gr == 1) {
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
    is_last = __hip_atomic_fetch_add(a.b.ctrl, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gr - 1;
  __syncthreads();
  if (!is_last) return;
  // Acquire at agent scope: the reads below may not be served from before the
  // count was observed (it invalidates this CU's caches, writes nothing back).
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
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
  return (size_t)E * words * 8 + (size_t)routes * 4 + (size_t)E * 8 + 2 * kWaves * 4;
}

hipError_t launch_route_quant(const RouteQuantArgs& a, hipStream_t s, KernelEvents ev) {
  const int grid = routing_wgs(a.M) + quant_wgs(a.M, a.H);
  hipExtLaunchKernelGGL(route_quant_kernel, dim3(grid), dim3(kThreads),
                        route_quant_lds_bytes(a.E, a.words, a.M * a.k), s, ev.start, ev.stop, 0, a);
  return hipGetLastError();
}

hipError_t launch_codec_check(const float* in, uint8_t* q, float* dq, int n, hipStream_t s) {
  hipLaunchKernelGGL(codec_check_kernel, dim3((n + 255) / 256), dim3(256), 0, s, in, q, dq, n);
  return hipGetLastError();
}

}  // namespace moe
