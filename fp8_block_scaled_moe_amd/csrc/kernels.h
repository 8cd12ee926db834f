// Kernel argument blocks and host-side launchers. Each kernel lives in its
// own translation unit and is launched through the function declared here.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kTile = 128;  // block size of every FP8 scale (K and N)
constexpr int kMaxTopK = 32;

// Events that a launch fills with its kernel's own start and end: the
// timestamps of the kernel's dispatch (hipExtLaunchKernel), not of markers
// queued beside it. Both null: an untimed launch.
struct KernelEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

// Distinct-expert buckets built by the routing kernel (device memory).
struct Buckets {
  int32_t* ctrl;     // [0] arrival counter (self-resetting), [1] U = distinct experts,
                     // [2] J = jobs (when job_routes > 0)
  int32_t* uexp;     // [U] expert ids, ascending
  int32_t* uoff;     // [U] first index of the expert's routes in `routes`
  int32_t* ucnt;     // [U] number of routes of the expert
  int32_t* routes;   // [M*k] route indices (t*k + j) grouped by expert, ascending t
  // Each expert's routes cut into jobs of at most job_routes consecutive
  // entries of `routes`, experts ascending (FP4 form; persistent FP8 GEMMs).
  int4* jobs;        // [J] {local expert, first index in routes, count, 0}
  int32_t* rjob;     // [M*k] job of each local route
};

// Where the epilogues find the FP4 GEMM's partial sums of a tile: the GEMM
// records the partial slots of every (job, 64-row tile) (stream_device.h).
struct StreamDesc {
  const int32_t* counts;  // [J, tiles] partial slots, written by the GEMM
  const int32_t* rjob;    // job of each route
  int R;                  // routes (jobs never outnumber them)
  int tiles;              // N / 64
  int steps;              // K / 256
};

struct RouteQuantArgs {
  const void* logits;   // [M, E] f32 or bf16
  int logits_bf16;
  const float* bias;    // [E]
  const uint16_t* x;    // [M, H] bf16
  int M, E, k, H;
  float routed_scale;
  int ue8m0;
  int words;            // 64-bit token-mask words per expert: ceil(M / 64)
  int32_t* ids;         // [M, k]
  float* weights;       // [M, k]
  uint8_t* xq;          // [M, H]
  float* xs;            // [M, H/128]
  uint8_t* xq2;         // second quantisation of x (shared expert), or nullptr
  float* xs2;
  int ue8m0_2;
  // FP4 staging instead of FP8 (fp4 != 0): packed E2M1 [M, H/2] in xq and
  // UE4M3 bytes [M, H/16] in xs4; jobs of at most job_routes routes.
  int fp4;
  uint8_t* xs4;
  int job_routes;
  int lb, lc;           // local experts [lb, lb + lc): only their routes are bucketed
  Buckets b;
};

struct SwigluArgs {
  float* part;          // [splits, R, 2I] (FP4 form: slot 0 receives the totals)
  int splits, R, I;
  float limit;
  uint8_t* hq;          // [R, I]
  float* hs;            // [R, I/128]
  // Shared expert (spart == nullptr when absent): GEMM partials
  // [ssplits, M, 2Is], gate rows first.
  const float* spart;
  int ssplits, M, Is;
  float slimit;
  int sue8m0;
  uint8_t* shq;         // [M, Is]
  float* shs;           // [M, Is/128]
  // FP4 form (fp4 != 0): GEMM1's partial slots found through `stream`,
  // their total written back to slot 0; gate rows first, BF16 rounding of
  // the GEMM output and of the activation, E2M1 staging per 16 into hq
  // (packed [R, I/2]) and hs4 ([R, I/16] UE4M3 bytes).
  int fp4;
  uint8_t* hs4;
  StreamDesc stream;
  const int32_t* ids;   // [M, k]: routes of non-local experts are skipped
  int lb, lc;
};

struct CombineArgs {
  const float* part;    // [splits, R, H]
  int splits, M, k, H;
  const float* weights; // [M, k]
  uint16_t* slots;      // [M*k, H] bf16
  uint16_t* combined;   // [M, H] bf16
  const float* spart;   // shared expert's down partials [ssplits, M, H], or nullptr
  int ssplits;
  uint16_t* shared_out; // [M, H] bf16
  const int32_t* ids;   // [M, k]: slots of non-local experts are zero
  int lb, lc;
  int fp4;              // GEMM2's partial slots found through `stream`
  StreamDesc stream;
};

// One block-scaled GEMM problem: for every route r of distinct expert u and
// every weight row n,
//   part[split, r, n] = sum_{b in split} ws[e, n/128, b] * as[row(r), b] *
//                       sum_{i in block b} W[e, n, i] * A[row(r), i]
// with row(r) = r / act_div. A routed problem takes its experts and routes
// from the buckets; a dense one (the shared expert) is expert 0 with routes
// 0..dense-1, one per token.
struct GemmProblem {
  const uint8_t* w;     // [E, N, K] e4m3 (FP4 kernel: [E, N, K/2] packed E2M1)
  const float* ws;      // [E, N/128, K/128]
  const uint8_t* ws8;   // FP4 kernel: UE4M3 bytes, reordered (launch_reorder_fp4_scales)
  const uint8_t* as8;   // FP4 kernel: [rows, K/16] UE4M3 bytes of the activations
  const uint8_t* aq;    // [rows, K] e4m3 (FP4 kernel: [rows, K/2] packed E2M1)
  const float* as;      // [rows, K/128]
  float* part;          // [splits, R, N]
  Buckets b;            // routed problems only
  int dense;            // > 0: dense problem of this many routes
  int N, K, nkb;        // nkb = K / 128
  int tiles;            // N / 64
  int splits, ks;       // K splits and 128-blocks per split
  int R;                // routes (row stride of part)
  int act_div;
  int tpw;              // split-K kernels: 64-row tiles streamed per workgroup (divides tiles, <= kMaxTpw)
  int kparts;           // K-in-workgroup kernel: K ranges per row group (1, 2 or 4); 64 / kparts rows
};

// The combine carried out inside the GEMM2 launch (K-in-workgroup kernel):
// each unit, once its outputs are stored at device scope, counts one arrival
// per route on (token, column tile); the arrival that completes a tile's
// count (the token's local picks) writes that tile's slots and combined row.
// Counters reset themselves. Arrays as in CombineArgs.
struct CombineFuse {
  int on;               // 0: plain GEMM (combine_kernel follows)
  int32_t* counters;    // [M, N / rows per workgroup], zero between calls
  const int32_t* ids;   // [M, k]
  const float* weights; // [M, k]
  uint16_t* slots;      // [M*k, H] bf16
  uint16_t* combined;   // [M, H] bf16
  uint16_t* shared_out; // [M, H] bf16, written by the dense units (or nullptr)
  int M, k, lb, lc;
  int all_local;        // lb == 0 and lc == experts: every token has k local picks
};

// The SwiGLU carried out inside the persistent GEMM1 launch: each unit, once
// its outputs are stored at device scope, counts one arrival per route on
// (route, 128-column block of the hidden); the arrival that completes a
// count (the 2 x 128 / rows units holding the block's up and gate rows)
// computes that block's activation and FP8 codes. Counters reset themselves.
struct SwigluFuse {
  int on;               // 0: plain GEMM1 (swiglu_requant_kernel follows)
  int32_t* counters;    // [R, I/128], zero between calls
  int I;
  float limit;
  uint8_t* hq;          // [R, I] e4m3
  float* hs;            // [R, I/128]
};

// Routing and the activation quantisation inside the persistent GEMM1 launch
// (at most kRouteFuseMaxTokens tokens and 64 routes): every workgroup routes
// the M tokens, groups their local routes into jobs and stages x as FP8
// codes in its own LDS before its first unit, with the functions the
// routing kernel runs (route_device.h); workgroup 0 also writes the picks,
// weights, buckets, codes and scales out for the kernels that follow.
// Arrays as in RouteQuantArgs; the buckets are the routed problem's.
constexpr int kRouteFuseMaxTokens = 2;
struct RouteFuse {
  int on;
  const void* logits;   // [M, E] f32 or bf16
  int logits_bf16;
  const float* bias;    // [E]
  const uint16_t* x;    // [M, K] bf16
  int M, E, k;
  float routed_scale;
  int ue8m0;
  int lb, lc;
  int32_t* ids;         // [M, k]
  float* weights;       // [M, k]
  uint8_t* xq;          // [M, K] e4m3 (the routed problem's aq)
  float* xs;            // [M, K/128] (its as)
};

// One GEMM launch: the dense problem's units (if any) come first in the grid,
// then the routed problem's.
struct GemmArgs {
  GemmProblem p[2];     // [0] dense (shared expert), [1] routed
  int units0;           // work units of p[0]; 0 when there is none
  int pass_routes;      // MFMA path: routes staged per pass (<= 16)
  int stream_wgs;       // FP4 kernel: resident workgroups (stream_map)
  int32_t* stream_counts;  // FP4 kernel: [J, tiles] partial slots of each tile, written here
  CombineFuse cf;       // K-in-workgroup GEMM2 only
  SwigluFuse sf;        // persistent GEMM1 only
  RouteFuse rf;         // persistent GEMM1 only
};

// FP4 GEMM: a stream of (job, tile, step) items split evenly over the
// workgroups; partial sums per tile go to part[slot] (stream_device.h).
constexpr int kFp4JobRoutes = 4;  // routes of a job (one pass over an expert's weights): an MFMA block's columns
size_t gemm_fp4_lds_bytes(int K);
// workgroups that are resident at once on the current device (0 on error)
int gemm_fp4_resident_wgs(int K);
hipError_t launch_gemm_fp4(const GemmArgs& a, int role, int grid, hipStream_t s, KernelEvents ev = {});
// Weight scales [rows, K/16] UE4M3 (rows a multiple of 16) into the FP4
// GEMM's layout: per 16-row group and 256-value step, the step's 16 scale
// groups x the 16 rows' bytes (dst holds as many bytes as src).
hipError_t launch_reorder_fp4_scales(const uint8_t* src, uint8_t* dst, size_t rows, int K, hipStream_t s);
hipError_t launch_codec_check_fp4(const float* in, uint8_t* q, float* dq, int n, hipStream_t s);

// Work units of a problem per expert: (tiles / tpw) tile groups x splits.
inline int gemm_units_per_expert(const GemmProblem& p) { return (p.tiles / p.tpw) * p.splits; }

// Maximum 128-blocks of K per split (bounds the LDS staging of activations).
constexpr int kMaxKs = 16;
constexpr int kRowsPerWg = 64;
constexpr int kValuRoutes = 8;   // routes per pass of the VALU inner product
constexpr int kMfmaRoutes = 16;  // routes per pass of the MFMA inner product
constexpr int kMaxTpw = 4;
constexpr size_t kMfmaLdsBudget = 40 * 1024;  // keeps three workgroups per CU
constexpr size_t kMaxRouteLds = 64 * 1024;
constexpr size_t kMaxWgLds = 64 * 1024;

size_t route_quant_lds_bytes(int E, int words, int routes);
hipError_t launch_route_quant(const RouteQuantArgs& a, hipStream_t s, KernelEvents ev = {});
// role: 1 = GEMM1 (W13), 2 = GEMM2 (W2); it only selects the kernel symbol.
hipError_t launch_gemm_valu(const GemmArgs& a, int role, int grid, hipStream_t s, KernelEvents ev = {});
hipError_t launch_gemm_mfma(const GemmArgs& a, int role, int grid, hipStream_t s, KernelEvents ev = {});
size_t gemm_mfma_lds_bytes(int pass_routes, int ks);
// The kernel with the whole K sum inside a workgroup (no split-K partials):
// writes one FP32 value per (route, row) to part[0].
hipError_t launch_gemm_wg(const GemmArgs& a, int role, int grid, hipStream_t s, KernelEvents ev = {});
size_t gemm_wg_lds_bytes(int nkb);
// Its persistent form (routed problem only; its units are the routing
// kernel's jobs of at most kMfmaRoutes routes x rows): `grid` workgroups take
// the units in turn. gemm_wgp_fits: nkb K blocks and kparts K parts are
// within its conditions; resident_wgs is 0 on error.
hipError_t launch_gemm_wgp(const GemmArgs& a, int role, int grid, hipStream_t s, KernelEvents ev = {});
size_t gemm_wgp_lds_bytes(int nkb);
bool gemm_wgp_fits(int nkb, int kparts);
int gemm_wgp_resident_wgs(int nkb);
// The persistent GEMM1 with routing inside (RouteFuse): LDS per workgroup,
// whether E experts fit its routing prologue for nkb K blocks, and its
// resident workgroups (0 on error).
size_t gemm_wgp_route_lds_bytes(int nkb);
bool gemm_wgp_route_fits(int nkb, int E);
int gemm_wgp_route_resident_wgs(int nkb, int E);
// FP32 [n/128, k/128] scales from packed UE8M0 words int32 [n, ceil(k/512)];
// *bad is set nonzero when the rows of a 128-row block disagree.
hipError_t launch_unpack_ue8m0(const int32_t* packed, int n, int k, float* out, int32_t* bad,
                               hipStream_t s);
hipError_t launch_swiglu_requant(const SwigluArgs& a, hipStream_t s, KernelEvents ev = {});
// Zeroes n int32 words at p with a kernel (no memset node under graph capture).
hipError_t launch_zero_words(int32_t* p, size_t n, hipStream_t s);
hipError_t launch_combine(const CombineArgs& a, hipStream_t s, KernelEvents ev = {});
hipError_t launch_codec_check(const float* in, uint8_t* q, float* dq, int n, hipStream_t s);

}  // namespace moe
