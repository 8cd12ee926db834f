// Block-scaled FP8 GEMM over the touched experts with the whole K reduction
// inside one workgroup.
//
// Same sum as the split-K kernels (expert_gemm.hip): every 128-K block's
// partial is multiplied by (weight scale x activation scale) of that block
// before it joins the FP32 total ("mega_moe" page, module docstring). What
// differs is where the K sum is finished. Writing split-K partial sums to
// memory in the middle of the weight stream costs far more than their bytes
// on MI355X: the FP32 partials are written back to HBM between the weight
// reads. Measured with every expert taking 16 routes, GEMM1 streamed at
// 6.7 TB/s with the partials kept in L2 and 5.1 TB/s with them written out.
// So here a workgroup owns 16, 32 or 64 weight rows of one expert over all of
// K: its four waves split K into `kparts` contiguous ranges (four row groups
// x one range, two x two, or one x four), and add their 16 x 16 results
// through LDS in a fixed order. One FP32 value per (route, row) leaves the
// chip.
//
// Per step a wave takes one 128-K block of its 16 rows. The weights are read
// with eight lanes per row (full 128-byte segments, nontemporal) and passed
// through a per-wave LDS tile into the MFMA layout. The activations of the
// pass's 16 routes come straight from L2 into registers in the MFMA layout,
// so no LDS staging bounds how much of K a workgroup covers. Both streams are
// requested kDepth steps ahead.
//
// GEMM2 can also finish the layer in the same launch (kFuse): its FP32
// outputs are then stored at device scope, and once a unit's stores have
// completed it counts one arrival per route on (token, column tile). The
// arrival that completes a count (the token's local picks) finds every slot
// value of that tile in memory and writes the tile's BF16 slots and combined
// values, with the arithmetic of the separate combine kernel (weights applied
// once, FP32 sum in pick order). No workgroup ever waits for another.
#include <algorithm>

#include "epilogue_device.h"
#include "gemm_device.h"
#include "route_device.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kDepth = 2;          // 128-K steps in flight per wave (keeps four waves per SIMD)
constexpr int kRoutesPerPass = 16;  // MFMA columns
constexpr int kRedFloats = 4 * kWave * 4;  // the four waves' 16 x 16 results

// Picks of token t whose expert is local.
__device__ __forceinline__ int local_picks(const CombineFuse& f, int t) {
  if (f.all_local) return f.k;
  int n = 0;
  for (int j = 0; j < f.k; ++j) {
    const int e = f.ids[(size_t)t * f.k + j] - f.lb;
    n += e >= 0 && e < f.lc;
  }
  return n;
}

// Whole workgroup: slots and combined values of token t over columns
// [c0, c0 + w) (w <= 64), reading the FP32 slot values of the local picks at
// device scope. Each slot is its GEMM output rounded once to BF16, zero for a
// pick whose expert is not local; combined = BF16(sum_j w[t, j] * slot_j),
// the FP32 sum in pick order (nvfp4-megamoe-kernel README, slot
// representation). `lds` holds k * 64 floats. Contains barriers.
__device__ void combine_tile(const CombineFuse& f, const float* part, int H, int t, int c0, int w, float* lds) {
  const int tid = threadIdx.x;
  for (int i = tid; i < f.k * w; i += kThreads) {
    const int j = i / w, c = i - j * w;
    const size_t r = (size_t)t * f.k + j;
    const int e = f.ids[r] - f.lb;
    float v = 0.f;
    if (e >= 0 && e < f.lc) v += __hip_atomic_load(part + r * H + c0 + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t b = bf16_bits(v);
    f.slots[r * H + c0 + c] = (uint16_t)b;
    lds[j * 64 + c] = bf16_value(b);
  }
  __syncthreads();
  if (tid < w) {
    float acc = 0.f;
    for (int j = 0; j < f.k; ++j) acc = fmaf(f.weights[(size_t)t * f.k + j], lds[j * 64 + tid], acc);
    f.combined[(size_t)t * H + c0 + tid] = bf16_bits(acc);
  }
  __syncthreads();
}

// Workgroup 0 of a fused launch: tokens without a local pick get zero slot
// rows and a zero combined row (no unit counts arrivals for them).
__device__ void zero_unrouted_tokens(const CombineFuse& f, int H, int* list, int& nlist) {
  const int tid = threadIdx.x;
  if (tid == 0) nlist = 0;
  __syncthreads();
  for (int t = tid; t < f.M; t += kThreads)
    if (local_picks(f, t) == 0) list[atomicAdd(&nlist, 1)] = t;
  __syncthreads();
  const int n = nlist, row16 = H / 8;  // 16-byte words per BF16 row
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  for (int q = 0; q < n; ++q) {
    const int t = list[q];
    for (int i = tid; i < (f.k + 1) * row16; i += kThreads) {
      const int j = i / row16, c = i - j * row16;
      uint16_t* row = j < f.k ? f.slots + ((size_t)t * f.k + j) * H : f.combined + (size_t)t * H;
      reinterpret_cast<u32x4_t*>(row)[c] = zero;
    }
  }
  __syncthreads();
}

template <int kRole, bool kFuse>
__global__ __launch_bounds__(kThreads) void gemm_wg_kernel(GemmArgs args) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int nclaim;
  int unit;
  const GemmProblem a = select_problem(args, unit);
  const CombineFuse& f = args.cf;
  const int kparts = a.kparts;
  const int rows_wg = kRowsPerWg / kparts;
  const int per_expert = a.N / rows_wg;
  if (kFuse && !f.all_local && blockIdx.x == 0)
    zero_unrouted_tokens(f, a.N, reinterpret_cast<int*>(smem + 4 * kTileBytes), nclaim);
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
  const int row0 = tile * rows_wg + rgrp * 16;  // this wave's 16 rows
  const int kb0 = (kp * a.nkb) / kparts;
  const int nsteps = ((kp + 1) * a.nkb) / kparts - kb0;
  const int rg = lane >> 3, ch = lane & 7;   // load layout
  const int col = lane & 15, g = lane >> 4;  // MFMA layout

  uint8_t* tile_lds = smem + wave * kTileBytes;                      // [4][kTileBytes]
  float* red = reinterpret_cast<float*>(smem + 4 * kTileBytes);       // [4 waves][64 lanes][4]
  float* wsl = red + kRedFloats;                                      // [4 row groups][nkb]
  float* xsl = wsl + 4 * a.nkb;                                       // [nkb][16]
  int* rts = reinterpret_cast<int*>(xsl + a.nkb * kRoutesPerPass);    // [16]

  // addresses: a uniform base plus a 32-bit offset per lane
  const uint8_t* pw = a.w + ((size_t)e * a.N + tile * rows_wg) * a.K;
  const uint32_t w_lane = (uint32_t)((rgrp * 16 + rg) * a.K + kb0 * kTile + ch * 16);
  const uint32_t half_step = (uint32_t)(8 * a.K);
  u32x4_t wa[kDepth], wb[kDepth], xa[kDepth], xb[kDepth];
  auto load_w = [&](int q, int st) {
    const uint32_t o = w_lane + (uint32_t)st * kTile;
    wa[q] = load_stream16(pw + o);
    wb[q] = load_stream16(pw + (o + half_step));
  };

  for (int c0 = 0; c0 < cnt; c0 += kRoutesPerPass) {
    const int nr = min(kRoutesPerPass, cnt - c0);
    if (c0) __syncthreads();  // the previous pass is done with rts, xsl and red
#pragma unroll
    for (int q = 0; q < kDepth; ++q) {  // unconditional (see step): past the last step, row 0 of aq
      if (q < nsteps) {
        load_w(q, q);
      } else {
        wa[q] = load_stream16(a.aq);
        wb[q] = load_stream16(a.aq + 64);
      }
    }
    if (tid < nr) rts[tid] = a.dense ? c0 + tid : a.b.routes[off + c0 + tid];
    if (c0 == 0) {
      // weight scales of the workgroup's row groups: one 128-row scale block each
      const float* ws = a.ws + (size_t)e * (a.N / kTile) * a.nkb;
      for (int i = tid; i < (kRowsPerWg / 16) * a.nkb; i += kThreads) {
        const int r = i / a.nkb, b = i - r * a.nkb;
        if (r < 4 / kparts) wsl[i] = ws[(size_t)((tile * rows_wg + r * 16) / kTile) * a.nkb + b];
      }
    }
    __syncthreads();

    const bool live = col < nr;
    const int xrow = rts[live ? col : 0] / a.act_div;  // lanes past the routes repeat route 0
    const uint32_t px = (uint32_t)(xrow * a.K + kb0 * kTile + g * 16);
    auto load_x = [&](int q, int st) {
      const uint32_t o = px + (uint32_t)st * kTile;
      xa[q] = *reinterpret_cast<const u32x4_t*>(a.aq + o);
      xb[q] = *reinterpret_cast<const u32x4_t*>(a.aq + (o + 64));
    };
#pragma unroll
    for (int q = 0; q < kDepth; ++q) load_x(q, q < nsteps ? q : 0);
    for (int i = tid; i < nr * a.nkb; i += kThreads) {
      const int r = i / a.nkb, b = i - r * a.nkb;
      xsl[b * kRoutesPerPass + r] = a.as[(size_t)(rts[r] / a.act_div) * a.nkb + b];
    }
    __syncthreads();

    const float* wsr = wsl + rgrp * a.nkb + kb0;
    const float* xsr = xsl + kb0 * kRoutesPerPass + (live ? col : 0);
    float4_t acc = {0.f, 0.f, 0.f, 0.f};
    // One step. Its loads are issued on every step (branches around them
    // make the compiler wait for every load in flight): step st + kDepth, or
    // near the end this lane's activations of step st again (an L2 hit, never
    // used). Each register set is refilled once its data is consumed
    // (weights after the LDS write, activations after the MFMA), so no copy
    // of an in-flight load ties the wait to the newest request.
    auto step = [&](int st, int q) {
      // steps stay in order: the scheduler interleaving two steps' MFMAs
      // needs both steps' activations at once, i.e. a wait for every load
      __builtin_amdgcn_sched_barrier(0);
      *reinterpret_cast<u32x4_t*>(tile_lds + rg * kTileStride + ch * 16) = wa[q];
      *reinterpret_cast<u32x4_t*>(tile_lds + (rg + 8) * kTileStride + ch * 16) = wb[q];
      const bool ahead = st + kDepth < nsteps;
      const int lst = ahead ? st + kDepth : st;
      const uint8_t* wbase = ahead ? pw : a.aq;
      const uint32_t o = (ahead ? w_lane : px) + (uint32_t)lst * kTile;
      wa[q] = load_stream16(wbase + o);
      wb[q] = load_stream16(wbase + (o + (ahead ? half_step : 64u)));
      wave_lds_fence();
      const u32x4_t wlo = *reinterpret_cast<const u32x4_t*>(tile_lds + col * kTileStride + g * 16);
      const u32x4_t whi = *reinterpret_cast<const u32x4_t*>(tile_lds + col * kTileStride + 64 + g * 16);
      wave_lds_fence();
      const float4_t p = mfma_block(wlo, whi, xa[q], xb[q]);
      load_x(q, lst);
      const float s = wsr[st] * xsr[st * kRoutesPerPass];
      acc[0] = fmaf(p[0], s, acc[0]);
      acc[1] = fmaf(p[1], s, acc[1]);
      acc[2] = fmaf(p[2], s, acc[2]);
      acc[3] = fmaf(p[3], s, acc[3]);
    };
    int st0 = 0;
    for (; st0 + kDepth <= nsteps; st0 += kDepth) {
#pragma unroll
      for (int q = 0; q < kDepth; ++q) step(st0 + q, q);
    }
    for (int q = 0; st0 + q < nsteps; ++q) step(st0 + q, q);  // fewer than kDepth steps left

    if (kparts > 1) {  // K parts of a row group added in a fixed order: part 0, 1, ...
      *reinterpret_cast<float4_t*>(red + (wave * kWave + lane) * 4) = acc;
      __syncthreads();
      if (kp == 0) {
        for (int j = 1; j < kparts; ++j) {
          const float4_t o = *reinterpret_cast<const float4_t*>(red + ((wave + j) * kWave + lane) * 4);
          acc[0] += o[0];
          acc[1] += o[1];
          acc[2] += o[2];
          acc[3] += o[3];
        }
      }
    }
    if (kp == 0 && live) {
      float* dst = a.part + (size_t)rts[col] * a.N + row0 + 4 * g;
      if (kFuse && !a.dense) {  // read back by whichever workgroup completes the tile
#pragma unroll
        for (int i = 0; i < 4; ++i) __hip_atomic_store(dst + i, acc[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        *reinterpret_cast<float4_t*>(dst) = acc;
      }
      if (kFuse && a.dense && f.shared_out) {  // the shared expert's output row, rounded once
        uint16_t* so = f.shared_out + (size_t)rts[col] * a.N + row0 + 4 * g;
#pragma unroll
        for (int i = 0; i < 4; ++i) so[i] = bf16_bits(0.f + acc[i]);
      }
    }
  }

  if constexpr (kFuse) {
    if (a.dense) return;
    // This unit's outputs were stored at device scope: once those stores have
    // completed they are visible to the workgroup that completes each count
    // (the pattern of the routing kernel's arrival counter; no release fence,
    // which would write back the whole L2).
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    int* claimed = reinterpret_cast<int*>(red);  // tokens whose tile this unit completes (<= cnt)
    if (tid == 0) nclaim = 0;
    __syncthreads();
    for (int i = tid; i < cnt; i += kThreads) {
      const int t = a.b.routes[off + i] / f.k;
      int32_t* ctr = f.counters + (size_t)t * per_expert + tile;
      if (__hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == local_picks(f, t) - 1) {
        __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // ready for the next call
        claimed[atomicAdd(&nclaim, 1)] = t;
      }
    }
    __syncthreads();
    const int n = nclaim;
    if (n > 0) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // reads after the completed count
    float* lds = reinterpret_cast<float*>(smem);  // the weight tiles' space: k * 64 floats
    for (int q = 0; q < n; ++q) combine_tile(f, a.part, a.N, claimed[q], tile * rows_wg, rows_wg, lds);
  }
}

// ---------------------------------------------------------------------------
// Persistent form of the same kernel for the routed problem. The grid is the
// number of workgroups resident at once (G), and workgroup b takes units b,
// b + G, b + 2G, ... in turn. Units, their rows, K parts and every sum are as
// above, so the outputs are bit-identical; what changes is the weight stream.
// A workgroup that runs one unit spends the start of it with only its first
// kDepth weight steps in flight (routes and scales are staged first), and the
// slot stands empty between workgroups. Here the next unit's routes and
// scales are fetched into registers while the current unit streams, and the
// next unit's first kDepth steps of weights and activations are requested in
// the slots the current unit no longer refills, so each wave's stream runs on
// from one unit into the next. A read probe of this shape (64-row units of
// 3584 B rows, 800 MB) streamed at 6.78 TB/s on 1024 persistent workgroups
// and 6.42 TB/s with one workgroup per unit.
//
// Its units are (job, rows) rather than (expert, rows): the routing kernel
// cuts each expert's routes into jobs of at most 16 (one MFMA pass), so an
// expert with more routes is several jobs, each streaming its weights once,
// as the one-unit kernel's passes do.
//
// Conditions, checked by the host: no dense problem, K blocks a multiple of
// kparts * kDepth (every wave has the same even number of steps) and at most
// kMaxPersistBlocks of them.
constexpr int kMaxPersistBlocks = 64;
constexpr int kSxPerThread = kMaxPersistBlocks * kRoutesPerPass / kThreads;  // activation scales staged per thread

struct UnitRef {
  int e, cnt, off, tile;
};

// Whole workgroup, after a GEMM1 unit of rows [row0, row0 + rows_wg) has
// stored its sums at device scope: one arrival per route of the unit on
// (route, 128-column block); for each count this unit completes, one wave
// reads the block's up and gate sums at device scope and writes its
// activation and FP8 codes (the arithmetic of the separate kernel, its split
// sum of one slice included). Contains barriers.
__device__ void finish_swiglu_blocks(const SwigluFuse& f, const GemmProblem& a, const UnitRef& u, int rows_wg,
                                     int* claimed, int& nclaim, const int32_t* routes) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  // These stores are at the device coherence point once they complete (the
  // next unit's first requests, issued before them, complete too).
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) nclaim = 0;
  __syncthreads();
  const int row0 = u.tile * rows_wg;
  const int c = (row0 < f.I ? row0 : row0 - f.I) / kTile;  // the unit's rows lie in one 128-row block
  const int nblk = f.I / kTile, target = 2 * (kTile / rows_wg);
  if (tid < u.cnt) {
    const int r = routes[u.off + tid];
    int32_t* ctr = f.counters + (size_t)r * nblk + c;
    if (__hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == target - 1) {
      __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // ready for the next call
      claimed[atomicAdd(&nclaim, 1)] = r;
    }
  }
  __syncthreads();
  const int n = nclaim;
  if (n > 0) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // reads after the completed count
  for (int q = wave; q < n; q += kThreads / kWave) {
    const int r = claimed[q];
    const float* p = a.part + (size_t)r * a.N + c * kTile + 2 * lane;
    const float u0 = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const float u1 = __hip_atomic_load(p + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const float g0 = __hip_atomic_load(p + f.I, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const float g1 = __hip_atomic_load(p + f.I + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    swiglu_finish(0.f + u0, 0.f + u1, 0.f + g0, 0.f + g1, f.limit, f.I, f.hq, f.hs, r, c, lane);
  }
}

__host__ __device__ inline size_t wgp_lds_bytes(int nkb) {
  return 4 * (size_t)kTileBytes + kRedFloats * 4 + (size_t)2 * (4 * nkb + nkb * kRoutesPerPass) * 4;
}

// LDS of the routing prologue, after the kernel's own: the jobs, x's FP8
// codes and scales, the picks and the buckets (at most 64 routes).
struct RouteLds {
  uint8_t* xq;  // [M][K]
  float* xs;    // [M][K / 128]
  int* ids;     // [M * k]
  Buckets b;    // routes, uexp, uoff, ucnt, rjob [64], ctrl [4], jobs [64]
};

__host__ __device__ inline size_t route_lds_bytes(int nkb) {
  return (size_t)kWave * 16 + (size_t)kRouteFuseMaxTokens * nkb * (kTile + 4) + (size_t)6 * kWave * 4 + 16;
}

__device__ __forceinline__ RouteLds carve_route(unsigned char* p, int nkb) {
  RouteLds l;
  l.b.jobs = reinterpret_cast<int4*>(p);
  p += kWave * 16;
  l.xq = p;
  p += (size_t)kRouteFuseMaxTokens * nkb * kTile;
  l.xs = reinterpret_cast<float*>(p);
  int* q = reinterpret_cast<int*>(l.xs + kRouteFuseMaxTokens * nkb);
  l.ids = q;
  l.b.routes = q + kWave;
  l.b.uexp = q + 2 * kWave;
  l.b.uoff = q + 3 * kWave;
  l.b.ucnt = q + 4 * kWave;
  l.b.rjob = q + 5 * kWave;
  l.b.ctrl = q + 6 * kWave;
  return l;
}

// Whole workgroup, before its first unit: routing of the M tokens, their
// local routes grouped into jobs of at most 16, and x staged as FP8 codes,
// into this workgroup's LDS, by the routing kernel's own functions. The
// sigmoids of all (token, expert) pairs are shared out over the workgroup
// through `keys_lds` (the kernel's weight tiles, not yet in use); then wave
// t < M takes token t's picks, a chain of dependent wave-wide steps, while
// the other waves quantise x's 128-blocks (eight lanes per block); with
// one token the picking wave lists the jobs right away, with two wave 0
// groups the routes after a barrier. Workgroup 0 also writes the picks,
// weights, expert-ordered buckets, codes and scales to device memory.
// Expert e of a token sits in lane e % 64, slot e / 64 (E <= 64 kPer,
// M * E * 8 bytes within the weight tiles' space, M * k <= 64: checked by
// the host). Contains barriers.
template <int kPer>
__device__ void route_prologue(const RouteFuse& f, const GemmProblem& a, unsigned char* keys_lds, const RouteLds& l) {
  constexpr int kWaves = kThreads / kWave;
  // blocks per group of eight lanes when the waves past the M picking ones quantise
  constexpr int kMinGroups = (kWaves - kRouteFuseMaxTokens) * (kWave / 8);
  constexpr int kQ = (kRouteFuseMaxTokens * kMaxPersistBlocks + kMinGroups - 1) / kMinGroups;
  constexpr int kS = kRouteFuseMaxTokens * kWave * kPer / kThreads;  // sigmoids per thread
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int M = f.M, E = f.E, K = a.K, nkb = a.nkb;
  const bool out = blockIdx.x == 0;
  uint32_t* keys = reinterpret_cast<uint32_t*>(keys_lds);  // [M][E]
  float* scores = reinterpret_cast<float*>(keys + M * E);  // [M][E]

  // every load first: the logits and bias of this thread's pairs, and (waves
  // past the picking ones) the BF16 values of the thread's group's blocks
  // (pairs past M * E load the last one and are not kept)
  int at[kS];
  float z[kS], bias[kS];
#pragma unroll
  for (int q = 0; q < kS; ++q) {
    at[q] = min(tid + q * kThreads, M * E - 1);
    bias[q] = f.bias[at[q] % E];
  }
  load_logits<kS>(f.logits, f.logits_bf16, at, z);
  // quantising waves only: group grp in [0, groups) takes blocks grp,
  // grp + groups, ... of the M * nkb
  const bool quant = wave >= M;
  const int groups = (kWaves - M) * (kWave / 8), sub = lane % 8;
  const int grp = quant ? (wave - M) * (kWave / 8) + lane / 8 : 0;
  const int items = M * nkb;
  u32x4_t lo[kQ], hi[kQ];
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    const int item = grp + q * groups;
    if (quant && item < items) {
      const size_t at = (size_t)(item / nkb) * K + (size_t)(item % nkb) * kTile + sub * 16;
      lo[q] = *reinterpret_cast<const u32x4_t*>(f.x + at);
      hi[q] = *reinterpret_cast<const u32x4_t*>(f.x + at + 8);
    }
  }
#pragma unroll
  for (int q = 0; q < kS; ++q) {
    const int i = tid + q * kThreads;
    if (i < M * E) {
      const float sc = sigmoid_f32(z[q]);
      scores[i] = sc;
      keys[i] = ordered_key(sc + bias[q]);
    }
  }
  __syncthreads();

  if (wave < M) {  // token `wave`'s picks
    const int t = wave;
    uint32_t key[kPer];
    float score[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int e = lane + kWave * j;
      key[j] = 0;
      score[j] = 0.f;
      if (e < E) {
        key[j] = keys[t * E + e];
        score[j] = scores[t * E + e];
      }
    }
    int id;
    float s, total;
    pick_top_k<kPer>(key, score, E, f.k, lane, id, s, total);
    if (lane < f.k) {
      l.ids[t * f.k + lane] = id;
      if (out) {
        f.ids[(size_t)t * f.k + lane] = id;
        f.weights[(size_t)t * f.k + lane] = pick_weight(s, total, f.routed_scale);
      }
    }
    if (M == 1) {
      // One route per expert: this workgroup's jobs are the local picks in
      // pick order, one route each (a GEMM1 sum depends only on its route,
      // not on the job that carries it). The kernels that follow get the
      // expert-ordered buckets from workgroup 0.
      const int e_loc = id - f.lb;
      const uint64_t local = __ballot(lane < f.k && e_loc >= 0 && e_loc < f.lc);
      const int pos = __popcll(local & ((1ull << lane) - 1ull));
      if ((local >> lane) & 1ull) {
        l.b.jobs[pos] = make_int4(e_loc, pos, 1, 0);
        l.b.routes[pos] = lane;
      }
      if (lane == 0) l.b.ctrl[2] = __popcll(local);
      if (out) {
        wave_lds_fence();
        bucket_routes_wave(a.b, l.ids, f.k, f.lb, f.lc, kRoutesPerPass, lane);
      }
    }
  }
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    const int item = grp + q * groups;
    if (quant && item < items) {  // the same for the eight lanes of a group
      float v[16];
      bf16x16_values(lo[q], hi[q], v);
      float sc;
      const u32x4_t c = fp8_block_codes(v, block_amax8(v), f.ue8m0, sc);
      const int t = item / nkb, blk = item % nkb;
      const size_t at = (size_t)t * K + (size_t)blk * kTile + sub * 16;
      *reinterpret_cast<u32x4_t*>(l.xq + at) = c;
      if (sub == 0) l.xs[t * nkb + blk] = sc;
      if (out) {
        *reinterpret_cast<u32x4_t*>(f.xq + at) = c;
        if (sub == 0) f.xs[(size_t)t * nkb + blk] = sc;
      }
    }
  }
  __syncthreads();
  if (M > 1) {
    if (wave == 0) {
      bucket_routes_wave(l.b, l.ids, M * f.k, f.lb, f.lc, kRoutesPerPass, lane);
      if (out) bucket_routes_wave(a.b, l.ids, M * f.k, f.lb, f.lc, kRoutesPerPass, lane);
    }
    __syncthreads();
  }
}

// kRoutePer > 0: the routing prologue runs first (RouteFuse; experts per
// lane), and the jobs, routes and activations come from this workgroup's LDS.
template <int kRole, bool kSwiglu, int kRoutePer>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 4))) void gemm_wgp_kernel(GemmArgs args) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int claimed[kRoutesPerPass];
  __shared__ int nclaim;
  constexpr bool kRoute = kRoutePer > 0;
  const GemmProblem& a = args.p[1];
  int u = blockIdx.x;
  int kparts, rows_wg, per_expert, total;
  int4 job0;
  const int4* jobs;
  const int32_t* routes;
  const uint8_t* aq;  // activation codes [rows, K] and scales [rows, K / 128]
  const float* as;
  if constexpr (kRoute) {
    const RouteLds l = carve_route(smem + wgp_lds_bytes(a.nkb), a.nkb);
    route_prologue<kRoutePer>(args.rf, a, smem, l);
    kparts = a.kparts;
    rows_wg = kRowsPerWg / kparts;
    per_expert = a.N / rows_wg;
    jobs = l.b.jobs;
    routes = l.b.routes;
    aq = l.xq;
    as = l.xs;
    job0 = jobs[min(u / per_expert, kWave - 1)];  // past the count: not used
    total = l.b.ctrl[2] * per_expert;
  } else {
    // The argument lines the first unit needs are read under one wait, and
    // the first unit's job beside the job count: read at first use, each
    // would add a memory round trip before the first weight request. The job
    // index is clamped to the routes (jobs never outnumber them), so the early
    // read stays inside the table; past the count it is not used.
    kparts = a.kparts;  // passed through the read below, so nothing computes ahead of it
    asm volatile("" : "+s"(kparts) : "s"(a.w), "s"(a.b.jobs), "s"(a.b.ctrl), "s"(a.R));
    rows_wg = kRowsPerWg / kparts;
    per_expert = a.N / rows_wg;
    jobs = a.b.jobs;
    routes = a.b.routes;
    aq = a.aq;
    as = a.as;
    job0 = jobs[min(u / per_expert, a.R - 1)];
    total = a.b.ctrl[2] * per_expert;  // jobs x units per job
    asm volatile("" ::"v"(job0.x), "v"(job0.y), "v"(job0.z));  // keeps the read above the exit
  }
  const int j0 = u / per_expert;
  const int G = gridDim.x;
  if (u >= total) return;  // more slots than units: the whole workgroup exits

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int rgrp = wave / kparts, kp = wave - rgrp * kparts;
  const int nkb = a.nkb;
  const int nsteps = nkb / kparts;  // the same for every wave (checked by the host)
  const int kb0 = kp * nsteps;
  const int rg = lane >> 3, ch = lane & 7;   // load layout
  const int col = lane & 15, g = lane >> 4;  // MFMA layout
  const int nsw = (4 / kparts) * nkb;        // weight scales of a unit (row groups x blocks)
  const int stage_floats = 4 * nkb + nkb * kRoutesPerPass;

  uint8_t* tile_lds = smem + wave * kTileBytes;                 // [4][kTileBytes]
  float* red = reinterpret_cast<float*>(smem + 4 * kTileBytes);  // [4 waves][64 lanes][4]
  float* stage = red + kRedFloats;                               // [2][wsl 4 * nkb | xsl nkb * 16]

  auto unit_ref = [&](int v) {
    UnitRef x;
    const int j = v / per_expert;
    x.tile = v - j * per_expert;
    const int4 job = jobs[j];  // {local expert, first index in routes, count <= 16, 0}
    x.e = job.x;
    x.off = job.y;
    x.cnt = job.z;
    return x;
  };
  // Addresses as a uniform base per unit plus a 32-bit offset per lane (a
  // lane's offset into its unit's weights is the same for every unit).
  auto weights_of = [&](const UnitRef& x) { return a.w + ((size_t)x.e * a.N + x.tile * rows_wg) * a.K; };
  const uint32_t w_lane = (uint32_t)((rgrp * 16 + rg) * a.K + kb0 * kTile + ch * 16);
  const uint32_t half_step = (uint32_t)(8 * a.K);

  // Per-thread staging registers: one weight scale (thread < nsw), and the
  // activation scales of route col (blocks tid / 16 + 16 j).
  float sw = 0.f, sx[kSxPerThread];
  int rt_next = 0, xrow_next = 0;
  auto fetch_routes = [&](const UnitRef& x) {  // first level: the route of this lane's column
    rt_next = routes[x.off + (col < x.cnt ? col : 0)];  // lanes past the routes repeat route 0
    xrow_next = rt_next / a.act_div;
    if (tid < nsw) {
      const int r = tid / nkb, b = tid - r * nkb;
      sw = a.ws[((size_t)x.e * (a.N / kTile) + (x.tile * rows_wg + r * 16) / kTile) * nkb + b];
    }
  };
  auto fetch_scales = [&](const UnitRef& x) {  // second level: activation scales of those routes
#pragma unroll
    for (int j = 0; j < kSxPerThread; ++j) {
      const int b = tid / kRoutesPerPass + (kThreads / kRoutesPerPass) * j;
      sx[j] = col < x.cnt && b < nkb ? as[(size_t)xrow_next * nkb + b] : 0.f;
    }
  };
  auto commit = [&](float* st, const UnitRef& x) {
    if (tid < nsw) st[tid] = sw;
#pragma unroll
    for (int j = 0; j < kSxPerThread; ++j) {
      const int b = tid / kRoutesPerPass + (kThreads / kRoutesPerPass) * j;
      if (col < x.cnt && b < nkb) st[4 * nkb + b * kRoutesPerPass + col] = sx[j];
    }
  };

  u32x4_t wa[kDepth], wb[kDepth], xa[kDepth], xb[kDepth];
  auto load_w = [&](const uint8_t* pw, int q, int st) {
    const uint32_t o = w_lane + (uint32_t)st * kTile;
    wa[q] = load_stream16(pw + o);
    wb[q] = load_stream16(pw + (o + half_step));
  };
  auto x_of = [&](int xrow) { return (uint32_t)(xrow * a.K + kb0 * kTile + g * 16); };
  auto load_x = [&](uint32_t px, int q, int st) {
    const uint32_t o = px + (uint32_t)st * kTile;
    xa[q] = *reinterpret_cast<const u32x4_t*>(aq + o);
    xb[q] = *reinterpret_cast<const u32x4_t*>(aq + (o + 64));
  };

  // The first unit: requests, then staging, as the one-unit kernel does.
  UnitRef cur;
  cur.tile = u - j0 * per_expert;
  cur.e = job0.x;
  cur.off = job0.y;
  cur.cnt = job0.z;
  const uint8_t* pw = weights_of(cur);
#pragma unroll
  for (int q = 0; q < kDepth; ++q) load_w(pw, q, q);
  fetch_routes(cur);
  int rt = rt_next;
  uint32_t px = x_of(xrow_next);
#pragma unroll
  for (int q = 0; q < kDepth; ++q) load_x(px, q, q);
  fetch_scales(cur);
  commit(stage, cur);
  __syncthreads();

  for (int buf = 0;; buf ^= 1) {
    const int nu = u + G;
    const bool more = nu < total;
    UnitRef nx = cur;
    if (more) {
      nx = unit_ref(nu);
      fetch_routes(nx);
    }
    const uint8_t* pwn = weights_of(nx);
    const uint32_t pxn = x_of(xrow_next);
    if (more) fetch_scales(nx);

    const float* st_cur = stage + buf * stage_floats;
    const float* wsr = st_cur + rgrp * nkb + kb0;
    const bool live = col < cur.cnt;
    const float* xsr = st_cur + 4 * nkb + kb0 * kRoutesPerPass + (live ? col : 0);
    float4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int st0 = 0; st0 < nsteps; st0 += kDepth) {
#pragma unroll
      for (int q = 0; q < kDepth; ++q) {
        const int st = st0 + q;
        *reinterpret_cast<u32x4_t*>(tile_lds + rg * kTileStride + ch * 16) = wa[q];
        *reinterpret_cast<u32x4_t*>(tile_lds + (rg + 8) * kTileStride + ch * 16) = wb[q];
        // One load path for every step (separate paths cost a full drain of
        // the loads in flight): this unit's step st + kDepth, else the next
        // unit's step q (nsteps is a multiple of kDepth), else, after the last
        // unit, this lane's activations of step st again in both register
        // sets (L2 hits; never used; weights, read nontemporally, would come
        // from HBM again). Each register set is refilled only once its data
        // is consumed (weights after the LDS write, activations after the
        // MFMA), so no copy of an in-flight load ties the wait to the newest
        // request.
        const bool ahead = st + kDepth < nsteps;
        const bool idle = !ahead && !more;
        const uint32_t xsrc = ahead || !more ? px : pxn;
        const int lst = ahead ? st + kDepth : (more ? q : st);
        const uint8_t* wbase = idle ? a.aq : (ahead ? pw : pwn);
        const uint32_t wo = (idle ? px : w_lane) + (uint32_t)lst * kTile;
        wa[q] = load_stream16(wbase + wo);
        wb[q] = load_stream16(wbase + (wo + (idle ? 64u : half_step)));
        wave_lds_fence();
        const u32x4_t wlo = *reinterpret_cast<const u32x4_t*>(tile_lds + col * kTileStride + g * 16);
        const u32x4_t whi = *reinterpret_cast<const u32x4_t*>(tile_lds + col * kTileStride + 64 + g * 16);
        wave_lds_fence();
        const float4_t p = mfma_block(wlo, whi, xa[q], xb[q]);
        load_x(xsrc, q, lst);
        const float s = wsr[st] * xsr[st * kRoutesPerPass];
        acc[0] = fmaf(p[0], s, acc[0]);
        acc[1] = fmaf(p[1], s, acc[1]);
        acc[2] = fmaf(p[2], s, acc[2]);
        acc[3] = fmaf(p[3], s, acc[3]);
      }
    }

    if (kparts > 1) {  // K parts of a row group added in a fixed order: part 0, 1, ...
      *reinterpret_cast<float4_t*>(red + (wave * kWave + lane) * 4) = acc;
      __syncthreads();
      if (kp == 0) {
        for (int j = 1; j < kparts; ++j) {
          const float4_t o = *reinterpret_cast<const float4_t*>(red + ((wave + j) * kWave + lane) * 4);
          acc[0] += o[0];
          acc[1] += o[1];
          acc[2] += o[2];
          acc[3] += o[3];
        }
      }
    }
    if (kp == 0 && live) {
      float* dst = a.part + (size_t)rt * a.N + cur.tile * rows_wg + rgrp * 16 + 4 * g;
      if constexpr (kSwiglu) {  // read back by whichever workgroup completes the block
#pragma unroll
        for (int i = 0; i < 4; ++i) __hip_atomic_store(dst + i, acc[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        *reinterpret_cast<float4_t*>(dst) = acc;
      }
    }
    if constexpr (kSwiglu) finish_swiglu_blocks(args.sf, a, cur, rows_wg, claimed, nclaim, routes);
    if (!more) break;
    commit(stage + (buf ^ 1) * stage_floats, nx);
    __syncthreads();  // the next unit's scales are in place; this unit is done with red and its stage
    u = nu;
    cur = nx;
    pw = pwn;
    px = pxn;
    rt = rt_next;
  }
}

}  // namespace

size_t gemm_wg_lds_bytes(int nkb) {
  return 4 * (size_t)kTileBytes + kRedFloats * 4 + (size_t)4 * nkb * 4 + (size_t)nkb * kRoutesPerPass * 4 +
         kRoutesPerPass * 4;
}

size_t gemm_wgp_lds_bytes(int nkb) { return wgp_lds_bytes(nkb); }

size_t gemm_wgp_route_lds_bytes(int nkb) { return wgp_lds_bytes(nkb) + route_lds_bytes(nkb); }

bool gemm_wgp_route_fits(int nkb, int E) {
  return E >= 1 && E <= 16 * kWave && (size_t)kRouteFuseMaxTokens * E * 8 <= wgp_lds_bytes(nkb) &&
         nkb <= kMaxPersistBlocks;
}

bool gemm_wgp_fits(int nkb, int kparts) {
  return nkb <= kMaxPersistBlocks && kparts >= 1 && 4 % kparts == 0 && nkb % (kparts * kDepth) == 0;
}

int gemm_wgp_resident_wgs(int nkb) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(gemm_wgp_kernel<1, false, 0>),
                                                   kThreads, gemm_wgp_lds_bytes(nkb)) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return cus * per_cu;
}

int gemm_wgp_route_resident_wgs(int nkb, int E) {
  int dev = 0, cus = 0, per_cu = 0;
  const void* k = E <= 4 * kWave ? reinterpret_cast<const void*>(gemm_wgp_kernel<1, false, 4>)
                                 : reinterpret_cast<const void*>(gemm_wgp_kernel<1, false, 16>);
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, kThreads, gemm_wgp_route_lds_bytes(nkb)) !=
          hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return cus * per_cu;
}

hipError_t launch_gemm_wgp(const GemmArgs& a, int role, int grid, hipStream_t s, KernelEvents ev) {
  const GemmProblem& p = a.p[1];
  if (a.units0 || a.cf.on || grid < 1 || !gemm_wgp_fits(p.nkb, p.kparts))
    return hipErrorInvalidValue;
  const size_t lds = gemm_wgp_lds_bytes(p.nkb);
  if (a.rf.on) {
    // every workgroup routes: its LDS holds the jobs, x's codes and the picks
    const RouteFuse& f = a.rf;
    if (role != 1 || a.sf.on || f.M < 1 || f.M > kRouteFuseMaxTokens || f.M * f.k > kWave || f.k < 1 ||
        p.K != p.nkb * kTile || p.act_div != f.k || !gemm_wgp_route_fits(p.nkb, f.E))
      return hipErrorInvalidValue;
    const size_t rlds = gemm_wgp_route_lds_bytes(p.nkb);
    if (f.E <= 4 * kWave)
      hipExtLaunchKernelGGL((gemm_wgp_kernel<1, false, 4>), dim3(grid), dim3(kThreads), rlds, s,
                            ev.start, ev.stop, 0, a);
    else
      hipExtLaunchKernelGGL((gemm_wgp_kernel<1, false, 16>), dim3(grid), dim3(kThreads), rlds, s,
                            ev.start, ev.stop, 0, a);
  } else if (a.sf.on) {
    // the unit's rows must lie in one 128-column block of up or of gate
    if (role != 1 || p.N != 2 * a.sf.I || kTile % (kRowsPerWg / p.kparts) != 0) return hipErrorInvalidValue;
    hipExtLaunchKernelGGL((gemm_wgp_kernel<1, true, 0>), dim3(grid), dim3(kThreads), lds, s,
                          ev.start, ev.stop, 0, a);
  } else if (role == 1) {
    hipExtLaunchKernelGGL((gemm_wgp_kernel<1, false, 0>), dim3(grid), dim3(kThreads), lds, s,
                          ev.start, ev.stop, 0, a);
  } else {
    hipExtLaunchKernelGGL((gemm_wgp_kernel<2, false, 0>), dim3(grid), dim3(kThreads), lds, s,
                          ev.start, ev.stop, 0, a);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_wg(const GemmArgs& a, int role, int grid, hipStream_t s, KernelEvents ev) {
  const int nkb = a.units0 ? std::max(a.p[0].nkb, a.p[1].nkb) : a.p[1].nkb;
  const size_t lds = gemm_wg_lds_bytes(nkb);
  if (a.cf.on) {
    // the combine's LDS (k x 64 floats) and token list reuse the weight tiles
    // and the reduction buffer; output rows are H wide
    if (role != 2 || a.cf.k > kMaxTopK || a.cf.M > kRedFloats || (a.units0 && a.p[0].N != a.p[1].N))
      return hipErrorInvalidValue;
    hipExtLaunchKernelGGL((gemm_wg_kernel<2, true>), dim3(grid), dim3(kThreads), lds, s,
                          ev.start, ev.stop, 0, a);
  } else if (role == 1) {
    hipExtLaunchKernelGGL((gemm_wg_kernel<1, false>), dim3(grid), dim3(kThreads), lds, s,
                          ev.start, ev.stop, 0, a);
  } else {
    hipExtLaunchKernelGGL((gemm_wg_kernel<2, false>), dim3(grid), dim3(kThreads), lds, s,
                          ev.start, ev.stop, 0, a);
  }
  return hipGetLastError();
}

}  // namespace moe
