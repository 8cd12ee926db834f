// The C ABI: handle creation (validation, workspace, scale conversion), the
// per-call launch plan, and the launches of one routed-expert step.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/moe_decode.h"
#include "kernels.h"
#include "stream_device.h"

using namespace moe;

namespace {

constexpr int kRegions = 21;
constexpr int kStages = 5;  // timing slots: route, GEMM1, SwiGLU, GEMM2, combine
constexpr int kEvents = 2 * kStages;  // start and stop of each timing slot
constexpr int kTargetUnits = 4096;  // work units per GEMM launch to aim for (16 per CU)
constexpr int kDenseTargetUnits = 256;  // units of the shared expert per GEMM launch
constexpr int kWgTargetUnits = 4096;    // K-in-workgroup path: units to aim for (16 per CU)
constexpr int kWgMinPartBlocks = 14;    // shortest per-wave weight stream worth a K part (128-K blocks)
constexpr int kBadFlagWord = 32;        // word of the control region used by create
// Debug stages past the workspace regions: the shared expert's FP32 scales.
constexpr int kStageSharedScale13 = 19, kStageSharedScale2 = 20;
// Most tokens for the persistent K-in-workgroup GEMMs. Measured on MI355X
// (DeepSeek-V3 shapes, layer µs, one workgroup per unit -> persistent):
// M=1 83.8 -> 81.3, M=2 137.6 -> 132.2, M=4 209.4 -> 207.5, M=8 313.9 ->
// 311.3, M=16 441.2 -> 446.4 (units no longer divide evenly over the
// resident workgroups, and a static share cannot even them out).
constexpr int kPersistMaxTokens = 8;
constexpr int kMfmaRouteFuseRoutes = 64;  // routes one wave groups in the GEMM1 routing prologue
// Beyond that, a GEMM whose K is at most this many 128-blocks still runs
// persistent: its units are short next to the per-unit staging. Measured on
// the latent shape (H=3584, I=1024, E=896, top-16, M=64), GEMM2 (8 blocks)
// took 157.4 µs with one workgroup per unit and 139.1 µs persistent; GEMM2
// of the DeepSeek-V3 shape (16 blocks) was even at M=16..64.
constexpr int kPersistShortBlocks = 8;

// Workspace regions (the debug stages use the same numbering).
enum {
  kCtrl, kUexp, kUoff, kUcnt, kRoutes, kXq, kXs, kP1, kHq, kHs, kP2,
  kSXq, kSXs, kSP1, kSHq, kSHs, kSP2,
  kJobs, kRjob,  // the job table and each route's job (FP4 form, persistent FP8 GEMMs)
  kCount,        // fused GEMM2 + combine: arrivals per (token, column tile)
  kSwCount,      // fused GEMM1 + SwiGLU: arrivals per (route, 128-column block)
};

struct Plan {
  int path;
  int s1, ks1, s2, ks2;
  int grid1, grid2;  // whole launches, shared units included
  int umax;
  int pass_routes;  // MFMA path: routes per pass
  int tpw1, tpw2;   // 64-row tiles per workgroup
  // shared expert (all zero without one)
  int ss1, sks1, ss2, sks2, stpw1, stpw2, sunits1, sunits2;
  // K-in-workgroup path: K parts per row group (routed, shared)
  int kp1, kp2, skp1, skp2;
  bool fuse_combine;  // the combine runs inside the GEMM2 launch
  bool fuse_swiglu;   // the SwiGLU runs inside the (persistent) GEMM1 launch
  // K-in-workgroup path: resident workgroups of the persistent GEMM1 / GEMM2
  // launches (0: one workgroup per unit)
  int persist1, persist2;
  bool route1;  // routing and the x quantisation run inside the persistent GEMM1 launch
};

struct Region {
  size_t off, bytes;
};

}  // namespace

struct moe_decode_handle {
  moe_decode_config cfg;
  int device;
  unsigned char* ws;
  size_t ws_bytes;
  Region reg[kRegions];
  int words;
  bool shared_own_quant;  // the shared expert quantises x with its own scale rule
  // shared expert scales converted to FP32 (owned), or the caller's FP32 ones
  float* s13_owned;
  float* s2_owned;
  const float* s13;
  const float* s2;
  int fp4_wgs1, fp4_wgs2;  // FP4 form: resident workgroups of each GEMM launch
  int wgp_wgs1, wgp_wgs2;  // FP8 form: resident workgroups of the persistent GEMM kernels
  int wgp_route_wgs1;      // and of the persistent GEMM1 with routing inside
  // FP4 form: the weight scales reordered for the GEMM kernel (owned)
  uint8_t* fp4_s13;
  uint8_t* fp4_s2;
  bool timing;
  bool timed_run;
  hipEvent_t ev[kEvents];  // slot i: ev[2i] and ev[2i + 1], filled by the slot's kernel
  int ev_slots;            // bit i: slot i's kernel ran in the last timed run
};

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int ceil_div(int a, int b) { return (a + b - 1) / b; }

// K split of one GEMM: at most max_ks blocks per split, enough units to fill
// the chip, splits of equal size where possible.
void choose_split(int units_per_split, int nkb, int forced, int max_ks, int* splits, int* ks) {
  int s = forced > 0 ? forced : ceil_div(kTargetUnits, std::max(units_per_split, 1));
  s = std::max(1, std::min(s, nkb));
  s = std::max(s, ceil_div(nkb, max_ks));
  int k = ceil_div(nkb, s);
  *ks = k;
  *splits = ceil_div(nkb, k);
}

int tiles_per_wg(int tiles, int want) {
  int t = want;
  while (tiles % t) t /= 2;
  return t;
}

// The dense problem (shared expert, M routes, N x K weights): about one unit
// per CU, but split-K partials (splits * M * N * 4 bytes written and read)
// kept within an eighth of the N * K weight bytes unless the LDS bound on
// blocks per split needs more splits.
void plan_dense(int M, int N, int K, int max_ks, int want_tpw, int* splits, int* ks, int* tpw,
                int* units) {
  const int tiles = N / kRowsPerWg, nkb = K / kTile;
  *tpw = tiles_per_wg(tiles, want_tpw);
  const int groups = tiles / *tpw;
  const int cap = std::max(1, K / (32 * M));
  int s = std::min(ceil_div(kDenseTargetUnits, groups), std::min(cap, nkb));
  s = std::max(s, ceil_div(nkb, max_ks));
  *ks = ceil_div(nkb, s);
  *splits = ceil_div(nkb, *ks);
  *units = groups * *splits;
}

// K parts per row group of the K-in-workgroup kernel: the fewest (longest
// weight streams per wave) that give about kWgTargetUnits units, as long as
// each part keeps kWgMinPartBlocks blocks (measured on MI355X: GEMM2's
// 16-block rows streamed at 65.5 us whole and 68.4 us in two parts, GEMM1's
// 56-block rows at 124.6 us whole, 123.3 in two and 122.5 in four parts, at
// 27 experts). A forced value is rounded down to 1, 2 or 4 and kept at two
// blocks per part at least.
int choose_kparts(int experts, int N, int nkb, int forced) {
  int kp = 1;
  if (forced > 0) {
    kp = forced >= 4 ? 4 : (forced >= 2 ? 2 : 1);
    while (kp > 1 && nkb < 2 * kp) kp /= 2;
    return kp;
  }
  while (kp < 4 && experts * (N / (kRowsPerWg / kp)) < kWgTargetUnits && nkb / (2 * kp) >= kWgMinPartBlocks)
    kp *= 2;
  return kp;
}

int local_count(const moe_decode_config& c) { return c.local_experts ? c.local_experts : c.experts; }

// fp4_wgs1/2: the FP4 GEMM launches' resident workgroups, wgp_wgs1/2 those of
// the persistent FP8 GEMMs (0 while only sizing the workspace).
Plan make_plan(const moe_decode_config& c, int M, int fp4_wgs1 = 0, int fp4_wgs2 = 0, int wgp_wgs1 = 0,
               int wgp_wgs2 = 0, int wgp_route_wgs1 = 0) {
  Plan p{};
  const int R = M * c.top_k;
  p.umax = std::min(local_count(c), R);
  if (c.weight_format == MOE_WEIGHTS_NVFP4) {
    // one launch-wide stream over K steps of 256 values: at most
    // stream_max_slots partials per tile; the resident workgroups, or one per
    // route if there are more routes (at most one job each)
    p.path = MOE_GEMM_FP4;
    p.ks1 = c.hidden / (2 * kTile);
    p.ks2 = c.inter / (2 * kTile);
    p.s1 = stream_max_slots(p.ks1);
    p.s2 = stream_max_slots(p.ks2);
    p.kp1 = p.kp2 = 1;
    p.tpw1 = p.tpw2 = kRowsPerWg;
    p.grid1 = std::max(fp4_wgs1, R);
    p.grid2 = std::max(fp4_wgs2, R);
    return p;
  }
  const int tiles1 = 2 * c.inter / kRowsPerWg, tiles2 = c.hidden / kRowsPerWg;
  if (c.gemm_path == MOE_GEMM_AUTO || c.gemm_path == MOE_GEMM_MFMA) {
    // K summed inside the workgroup: no split-K partials leave the chip
    p.path = MOE_GEMM_MFMA;
    p.pass_routes = kMfmaRoutes;
    p.s1 = p.s2 = 1;
    p.kp1 = choose_kparts(p.umax, 2 * c.inter, c.hidden / kTile, c.splits1);
    p.kp2 = choose_kparts(p.umax, c.hidden, c.inter / kTile, c.splits2);
    p.ks1 = ceil_div(c.hidden / kTile, p.kp1);
    p.ks2 = ceil_div(c.inter / kTile, p.kp2);
    p.tpw1 = kRowsPerWg / p.kp1;  // rows per workgroup
    p.tpw2 = kRowsPerWg / p.kp2;
    if (c.shared_inter > 0) {
      p.ss1 = p.ss2 = 1;
      p.skp1 = choose_kparts(1, 2 * c.shared_inter, c.hidden / kTile, p.kp1);
      p.skp2 = choose_kparts(1, c.hidden, c.shared_inter / kTile, p.kp2);
      p.sks1 = ceil_div(c.hidden / kTile, p.skp1);
      p.sks2 = ceil_div(c.shared_inter / kTile, p.skp2);
      p.sunits1 = 2 * c.shared_inter / (kRowsPerWg / p.skp1);
      p.sunits2 = c.hidden / (kRowsPerWg / p.skp2);
    }
    p.grid1 = p.umax * (2 * c.inter / p.tpw1) + p.sunits1;
    p.grid2 = p.umax * (c.hidden / p.tpw2) + p.sunits2;
    p.fuse_combine = c.launch_mode == MOE_LAUNCH_COMBINE_IN_GEMM2;
    // Persistent workgroups where the kernel's conditions hold, for up to
    // kPersistMaxTokens tokens or short K; MOE_GEMM_MFMA asked for by name
    // keeps one workgroup per unit.
    if (c.gemm_path == MOE_GEMM_AUTO && c.shared_inter == 0) {
      const int nkb1 = c.hidden / kTile, nkb2 = c.inter / kTile;
      const bool few = M <= kPersistMaxTokens;
      if (wgp_wgs1 > 0 && (few || nkb1 <= kPersistShortBlocks) && gemm_wgp_fits(nkb1, p.kp1)) {
        // On resident workgroups the units' count no longer sets the grid:
        // the most K parts that keep kWgMinPartBlocks blocks each give finer
        // units and so an even last round (measured on MI355X, DeepSeek-V3
        // M=4: GEMM1 123.9 µs at 2 K parts, 118.5 at 4; M=8: 189.2 at 1,
        // 187.1 at 4).
        if (c.splits1 <= 0) {
          for (int kp = 4; kp > p.kp1; kp /= 2) {
            if (nkb1 / kp >= kWgMinPartBlocks && gemm_wgp_fits(nkb1, kp)) {
              p.kp1 = kp;
              p.ks1 = ceil_div(nkb1, kp);
              p.tpw1 = kRowsPerWg / kp;
              p.grid1 = p.umax * (2 * c.inter / p.tpw1);
              break;
            }
          }
        }
        p.persist1 = std::min(p.grid1, wgp_wgs1);
        p.fuse_swiglu = c.launch_mode == MOE_LAUNCH_SWIGLU_IN_GEMM1;
        // Routing inside the GEMM1 launch: every workgroup routes the few
        // tokens itself (the "mega_moe" page's per-warp routing, here per
        // workgroup) and one wave groups the routes. The workgroups' first
        // weight request waits for that prologue (5.3 us at one token, 9.0
        // at two, against about 0.5 us after a routing launch); measured on
        // MI355X at DeepSeek-V3 shapes, the layer took 73.3 against 78.0 us
        // at one token and 128.2 against 129.0 at two, so MOE_LAUNCH_AUTO
        // takes it at one token.
        const bool want_route = c.launch_mode == MOE_LAUNCH_ROUTE_IN_GEMM1 ||
                                (c.launch_mode == MOE_LAUNCH_AUTO && M == 1);
        p.route1 = want_route && M <= kRouteFuseMaxTokens && M * c.top_k <= kMfmaRouteFuseRoutes &&
                   wgp_route_wgs1 > 0 && gemm_wgp_route_fits(nkb1, c.experts);
        if (p.route1) p.persist1 = std::min(p.grid1, wgp_route_wgs1);
      }
      if (wgp_wgs2 > 0 && !p.fuse_combine && (few || nkb2 <= kPersistShortBlocks) && gemm_wgp_fits(nkb2, p.kp2))
        p.persist2 = std::min(p.grid2, wgp_wgs2);
    }
    return p;
  }
  // MFMA costs the same per weight byte for any number of routes of an
  // expert (up to 16 per pass), VALU dot products cost per route. Measured on
  // MI355X with every expert taking n routes (E=64, H=7168, I=2048), GEMM1
  // streams at 6.69/6.67 TB/s (VALU/MFMA) for n=1, 5.68/5.86 for n=4,
  // 4.10/5.46 for n=8 and 2.01/5.06 for n=16; so MFMA unless every expert has
  // exactly one route (M = 1).
  p.path = c.gemm_path;
  // an expert has at most one route per token
  p.pass_routes = std::min(kMfmaRoutes, M);
  int max_ks = kMaxKs;
  if (p.path == MOE_GEMM_MFMA_SPLITK)
    while (max_ks > 1 && gemm_mfma_lds_bytes(p.pass_routes, max_ks) > kMfmaLdsBudget) --max_ks;
  // Staging a unit's activations costs about as much as streaming a few
  // blocks of weights per route; with many tokens (so many routes per
  // expert) a workgroup streams several tiles per staging.
  const int want = M <= 2 ? 1 : (M <= 8 ? 2 : kMaxTpw);
  p.tpw1 = tiles_per_wg(tiles1, want);
  p.tpw2 = tiles_per_wg(tiles2, want);
  choose_split(p.umax * (tiles1 / p.tpw1), c.hidden / kTile, c.splits1, max_ks, &p.s1, &p.ks1);
  choose_split(p.umax * (tiles2 / p.tpw2), c.inter / kTile, c.splits2, max_ks, &p.s2, &p.ks2);
  p.grid1 = p.umax * (tiles1 / p.tpw1) * p.s1;
  p.grid2 = p.umax * (tiles2 / p.tpw2) * p.s2;
  if (c.shared_inter > 0) {
    plan_dense(M, 2 * c.shared_inter, c.hidden, max_ks, want, &p.ss1, &p.sks1, &p.stpw1, &p.sunits1);
    plan_dense(M, c.hidden, c.shared_inter, max_ks, want, &p.ss2, &p.sks2, &p.stpw2, &p.sunits2);
    p.grid1 += p.sunits1;
    p.grid2 += p.sunits2;
  }
  return p;
}

int validate_config(const moe_decode_config* c) {
  if (!c) return MOE_DECODE_ERR_INVALID_ARG;
  if (!c->w13 || !c->w13_scale || !c->w2 || !c->w2_scale) return MOE_DECODE_ERR_INVALID_ARG;
  if (!aligned16(c->w13) || !aligned16(c->w2) || !aligned16(c->w13_scale) || !aligned16(c->w2_scale))
    return MOE_DECODE_ERR_INVALID_ARG;
  if (!(c->limit > 0.f) || !(c->routed_scale == c->routed_scale)) return MOE_DECODE_ERR_INVALID_ARG;
  if (c->max_tokens < 1) return MOE_DECODE_ERR_INVALID_ARG;
  if (c->hidden <= 0 || c->inter <= 0 || c->experts <= 0 || c->top_k <= 0)
    return MOE_DECODE_ERR_INVALID_ARG;
  if (c->max_tokens > MOE_DECODE_MAX_TOKENS) return MOE_DECODE_ERR_UNSUPPORTED;
  if (c->hidden % kTile || c->inter % kTile) return MOE_DECODE_ERR_UNSUPPORTED;
  if (c->experts > MOE_DECODE_MAX_EXPERTS) return MOE_DECODE_ERR_UNSUPPORTED;
  if (c->top_k > std::min(c->experts, MOE_DECODE_MAX_TOP_K)) return MOE_DECODE_ERR_UNSUPPORTED;
  if (c->logits_dtype != MOE_DTYPE_F32 && c->logits_dtype != MOE_DTYPE_BF16)
    return MOE_DECODE_ERR_UNSUPPORTED;
  if (c->gemm_path < MOE_GEMM_AUTO || c->gemm_path > MOE_GEMM_MFMA) return MOE_DECODE_ERR_UNSUPPORTED;
  if (c->local_begin < 0 || c->local_experts < 0 || c->local_begin + local_count(*c) > c->experts)
    return MOE_DECODE_ERR_INVALID_ARG;
  if (c->weight_format != MOE_WEIGHTS_FP8 && c->weight_format != MOE_WEIGHTS_NVFP4)
    return MOE_DECODE_ERR_UNSUPPORTED;
  if (c->weight_format == MOE_WEIGHTS_NVFP4) {
    const int step = 2 * kTile;  // the FP4 kernel's 256-value steps
    if (c->hidden % step || c->inter % step || c->shared_inter != 0 || c->ue8m0_act ||
        c->gemm_path != MOE_GEMM_AUTO)
      return MOE_DECODE_ERR_UNSUPPORTED;
    for (int K : {c->hidden, c->inter})  // two jobs' activations over the whole K in LDS
      if (gemm_fp4_lds_bytes(K) > kMaxWgLds) return MOE_DECODE_ERR_UNSUPPORTED;
  }
  if (gemm_wg_lds_bytes(std::max(c->hidden, std::max(c->inter, c->shared_inter)) / kTile) > kMaxWgLds)
    return MOE_DECODE_ERR_UNSUPPORTED;
  if (c->splits1 < 0 || c->splits2 < 0) return MOE_DECODE_ERR_INVALID_ARG;
  if (c->launch_mode < MOE_LAUNCH_AUTO || c->launch_mode > MOE_LAUNCH_ROUTE_IN_GEMM1)
    return MOE_DECODE_ERR_UNSUPPORTED;
  {
    const int words = (c->max_tokens + 63) / 64;
    if (route_quant_lds_bytes(c->experts, words, c->max_tokens * c->top_k) > kMaxRouteLds)
      return MOE_DECODE_ERR_UNSUPPORTED;
  }
  if (c->shared_inter < 0) return MOE_DECODE_ERR_INVALID_ARG;
  if (c->shared_inter > 0) {
    if (!c->sw13 || !c->sw13_scale || !c->sw2 || !c->sw2_scale) return MOE_DECODE_ERR_INVALID_ARG;
    if (!aligned16(c->sw13) || !aligned16(c->sw2) || !aligned16(c->sw13_scale) ||
        !aligned16(c->sw2_scale))
      return MOE_DECODE_ERR_INVALID_ARG;
    if (!(c->shared_limit > 0.f)) return MOE_DECODE_ERR_INVALID_ARG;
    if (c->shared_inter % kTile) return MOE_DECODE_ERR_UNSUPPORTED;
    if (c->shared_scale_format != MOE_SCALES_F32 && c->shared_scale_format != MOE_SCALES_UE8M0_PACKED)
      return MOE_DECODE_ERR_UNSUPPORTED;
  }
  return MOE_DECODE_OK;
}

// The workspace regions for every M up to c.max_tokens, each 256-byte
// aligned; returns the total bytes.
size_t layout_workspace(const moe_decode_config& c, Region reg[kRegions], bool* shared_own_quant) {
  const size_t Rcap = (size_t)c.max_tokens * c.top_k;
  const size_t Ucap = std::min<size_t>(local_count(c), Rcap);
  const bool fp4 = c.weight_format == MOE_WEIGHTS_NVFP4;
  size_t p1 = 0, p2 = 0, sp1 = 0, sp2 = 0;
  for (int M = 1; M <= c.max_tokens; ++M) {
    const Plan p = make_plan(c, M);
    p1 = std::max(p1, (size_t)p.s1 * M * c.top_k * 2 * c.inter);
    p2 = std::max(p2, (size_t)p.s2 * M * c.top_k * c.hidden);
    sp1 = std::max(sp1, (size_t)p.ss1 * M * 2 * c.shared_inter);
    sp2 = std::max(sp2, (size_t)p.ss2 * M * c.hidden);
  }
  const size_t H = c.hidden, I = c.inter, Is = c.shared_inter, T = c.max_tokens;
  // the shared expert reuses the routed x quantisation when the rules agree
  const bool own_quant = Is > 0 && (c.shared_ue8m0_act != 0) != (c.ue8m0_act != 0);
  const size_t sizes[kRegions] = {
      64 * sizeof(int32_t),           // control
      Ucap * sizeof(int32_t),         // uexp
      Ucap * sizeof(int32_t),         // uoff
      Ucap * sizeof(int32_t),         // ucnt
      Rcap * sizeof(int32_t),         // routes
      T * H,                          // x_q (FP4: packed, half of it)
      fp4 ? T * (H / 16) : T * (H / kTile) * sizeof(float),  // x_s (FP4: UE4M3 bytes per 16)
      p1 * sizeof(float),             // GEMM1 partials
      Rcap * I,                       // h_q
      fp4 ? Rcap * (I / 16) : Rcap * (I / kTile) * sizeof(float),  // h_s
      p2 * sizeof(float),             // GEMM2 partials
      own_quant ? T * H : 0,          // shared x_q
      own_quant ? T * (H / kTile) * sizeof(float) : 0,  // shared x_s
      sp1 * sizeof(float),            // shared gate_up partials
      T * Is,                         // shared h_q
      T * (Is / kTile) * sizeof(float),  // shared h_s
      sp2 * sizeof(float),            // shared down partials
      Rcap * sizeof(int32_t) * 4,     // job table (at most one job per route)
      Rcap * sizeof(int32_t),         // job of each route
      // arrival counts (at least 16 rows per workgroup); FP4 form: GEMM1's
      // partial slots per (job, 64-row tile), jobs never outnumbering routes
      fp4 ? Rcap * (2 * I / 64) * sizeof(int32_t) : T * (H / 16) * sizeof(int32_t),
      // arrival counts per (route, hidden block); FP4 form: GEMM2's slots per (job, tile)
      fp4 ? Rcap * (H / 64) * sizeof(int32_t) : Rcap * (I / kTile) * sizeof(int32_t),
  };
  size_t off = 0;
  for (int i = 0; i < kRegions; ++i) {
    reg[i] = Region{off, sizes[i]};
    off += (sizes[i] + 255) & ~size_t(255);
  }
  *shared_own_quant = own_quant;
  return off;
}

// Shared-expert scales as FP32: the caller's own, or converted once from the
// packed UE8M0 form into buffers the handle owns. Synchronises the device.
int prepare_shared_scales(moe_decode_handle* h) {
  const moe_decode_config& c = h->cfg;
  if (c.shared_scale_format == MOE_SCALES_F32) {
    h->s13 = static_cast<const float*>(c.sw13_scale);
    h->s2 = static_cast<const float*>(c.sw2_scale);
    return MOE_DECODE_OK;
  }
  const int H = c.hidden, Is = c.shared_inter;
  const size_t n13 = (size_t)(2 * Is / kTile) * (H / kTile), n2 = (size_t)(H / kTile) * (Is / kTile);
  if (hipMalloc(&h->s13_owned, n13 * sizeof(float)) != hipSuccess ||
      hipMalloc(&h->s2_owned, n2 * sizeof(float)) != hipSuccess) {
    (void)hipGetLastError();
    return MOE_DECODE_ERR_OUT_OF_MEMORY;
  }
  int32_t* bad = reinterpret_cast<int32_t*>(h->ws + h->reg[kCtrl].off) + kBadFlagWord;
  int32_t flag = 0;
  if (launch_unpack_ue8m0(static_cast<const int32_t*>(c.sw13_scale), 2 * Is, H, h->s13_owned, bad, nullptr) !=
          hipSuccess ||
      launch_unpack_ue8m0(static_cast<const int32_t*>(c.sw2_scale), H, Is, h->s2_owned, bad, nullptr) !=
          hipSuccess ||
      hipMemcpy(&flag, bad, sizeof(flag), hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemset(bad, 0, sizeof(int32_t)) != hipSuccess || hipDeviceSynchronize() != hipSuccess)
    return MOE_DECODE_ERR_HIP;
  if (flag) return MOE_DECODE_ERR_INVALID_ARG;  // a 128-row block mixes exponent bytes
  h->s13 = h->s13_owned;
  h->s2 = h->s2_owned;
  return MOE_DECODE_OK;
}

// ---- The workspace of moe_decode_run_noalloc ------------------------------
// A file-scope device array: each GPU holds its own copy, at its own
// address, from the library's load on that GPU until the process ends. In
// host code `scratch` names a host-side stand-in, not device memory: device
// addresses come only from the per-device lookup below.
constexpr size_t kScratchBytes = MOE_DECODE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
constexpr int kMaxCachedBlocks = 1024;  // K / 128 values whose resident-workgroup counts are cached

struct DeviceScratch {
  std::once_flag once;
  unsigned char* ptr = nullptr;  // this device's copy of `scratch`
  // resident workgroups of the persistent FP8 GEMM for K / 128 = i, plus one
  // (0: not yet asked)
  std::atomic<int> wgp[kMaxCachedBlocks + 1] = {};
  // the same for the persistent GEMM1 with routing inside, [E > 256][K / 128]
  std::atomic<int> wgp_route[2][kMaxCachedBlocks + 1] = {};
};
DeviceScratch g_dev[kMaxDevices];

// The device copy of `scratch` on device dev (the current device), looked
// up once per device; nullptr if the lookup failed.
unsigned char* device_scratch(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  DeviceScratch& d = g_dev[dev];
  std::call_once(d.once, [&] {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess)
      d.ptr = static_cast<unsigned char*>(p);
    else
      (void)hipGetLastError();
  });
  return d.ptr;
}

int cached_wgp_wgs(int dev, int nkb) {
  if (nkb > kMaxCachedBlocks) return gemm_wgp_resident_wgs(nkb);
  std::atomic<int>& slot = g_dev[dev].wgp[nkb];
  int v = slot.load(std::memory_order_relaxed);
  if (v == 0) {
    v = gemm_wgp_resident_wgs(nkb) + 1;
    slot.store(v, std::memory_order_relaxed);
  }
  return v - 1;
}

int cached_wgp_route_wgs(int dev, int nkb, int E) {
  if (nkb > kMaxCachedBlocks) return gemm_wgp_route_resident_wgs(nkb, E);
  std::atomic<int>& slot = g_dev[dev].wgp_route[E > 256][nkb];  // the kernel for E <= 256 or for more
  int v = slot.load(std::memory_order_relaxed);
  if (v == 0) {
    v = gemm_wgp_route_resident_wgs(nkb, E) + 1;
    slot.store(v, std::memory_order_relaxed);
  }
  return v - 1;
}

// Pointer checks of a run (M >= 1): INVALID_ARG for a NULL or misaligned
// buffer, or a shared_out without a shared expert.
int check_run_pointers(const moe_decode_config& c, const void* x, const void* logits, const float* bias,
                       const void* slots, const int32_t* ids, const float* weights, const void* combined,
                       const void* shared_out) {
  if (!x || !logits || !bias || !slots || !ids || !weights || !combined)
    return MOE_DECODE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(slots) || !aligned16(combined) || !aligned16(logits) ||
      ((uintptr_t)ids & 3u) || ((uintptr_t)weights & 3u) || ((uintptr_t)bias & 3u))
    return MOE_DECODE_ERR_INVALID_ARG;
  if (shared_out && (c.shared_inter == 0 || !aligned16(shared_out))) return MOE_DECODE_ERR_INVALID_ARG;
  return MOE_DECODE_OK;
}

// The five launches of one step on the handle's workspace (h->ws, h->reg);
// the arguments are checked.
int run_layer(moe_decode_handle* h, int32_t M, const void* x, const void* logits, const float* bias,
              void* slots, int32_t* ids, float* weights, void* combined, void* shared_out, hipStream_t s) {
  const bool shared = shared_out != nullptr;

  const moe_decode_config& c = h->cfg;
  const Plan p = make_plan(c, M, h->fp4_wgs1, h->fp4_wgs2, h->wgp_wgs1, h->wgp_wgs2, h->wgp_route_wgs1);
  const int R = M * c.top_k;
  const bool fp4 = c.weight_format == MOE_WEIGHTS_NVFP4;
  const int lb = c.local_begin, lc = local_count(c);
  unsigned char* ws = h->ws;
  auto at = [&](int i) { return ws + h->reg[i].off; };

  auto atf = [&](int i) { return reinterpret_cast<float*>(at(i)); };
  Buckets b;
  b.ctrl = reinterpret_cast<int32_t*>(at(kCtrl));
  b.uexp = reinterpret_cast<int32_t*>(at(kUexp));
  b.uoff = reinterpret_cast<int32_t*>(at(kUoff));
  b.ucnt = reinterpret_cast<int32_t*>(at(kUcnt));
  b.routes = reinterpret_cast<int32_t*>(at(kRoutes));
  b.jobs = reinterpret_cast<int4*>(at(kJobs));
  b.rjob = reinterpret_cast<int32_t*>(at(kRjob));
  uint8_t* xq = at(kXq);
  float* xs = atf(kXs);
  float* p1 = atf(kP1);
  uint8_t* hq = at(kHq);
  float* hs = atf(kHs);
  float* p2 = atf(kP2);
  uint8_t* sxq = h->shared_own_quant ? at(kSXq) : xq;
  float* sxs = h->shared_own_quant ? atf(kSXs) : xs;

  // timed runs: the kernel of timing slot `stage` fills that slot's events
  // with its own start and end
  int slots_run = 0;
  auto events = [&](int stage) -> KernelEvents {
    if (!h->timing) return {};
    slots_run |= 1 << stage;
    return KernelEvents{h->ev[2 * stage], h->ev[2 * stage + 1]};
  };

  hipError_t e = hipSuccess;

  RouteQuantArgs ra;
  ra.logits = logits;
  ra.logits_bf16 = c.logits_dtype == MOE_DTYPE_BF16;
  ra.bias = bias;
  ra.x = static_cast<const uint16_t*>(x);
  ra.M = M;
  ra.E = c.experts;
  ra.k = c.top_k;
  ra.H = c.hidden;
  ra.routed_scale = c.routed_scale;
  ra.ue8m0 = c.ue8m0_act;
  ra.words = (M + 63) / 64;
  ra.ids = ids;
  ra.weights = weights;
  ra.xq = xq;
  ra.xs = xs;
  ra.xq2 = shared && h->shared_own_quant ? sxq : nullptr;
  ra.xs2 = sxs;
  ra.ue8m0_2 = c.shared_ue8m0_act;
  ra.fp4 = fp4;
  ra.xs4 = at(kXs);
  // jobs: the FP4 GEMM's units, and the persistent FP8 GEMMs' (one MFMA pass each)
  ra.job_routes = fp4 ? kFp4JobRoutes : (p.persist1 || p.persist2 ? kMfmaRoutes : 0);
  ra.lb = lb;
  ra.lc = lc;
  ra.b = b;
  if (!p.route1 && e == hipSuccess) e = launch_route_quant(ra, s, events(0));

  SwigluArgs sa;
  sa.part = p1;
  sa.splits = p.s1;
  sa.R = R;
  sa.I = c.inter;
  sa.limit = c.limit;
  sa.hq = hq;
  sa.hs = hs;
  sa.spart = shared ? atf(kSP1) : nullptr;
  sa.ssplits = p.ss1;
  sa.M = M;
  sa.Is = c.shared_inter;
  sa.slimit = c.shared_limit;
  sa.sue8m0 = c.shared_ue8m0_act;
  sa.shq = at(kSHq);
  sa.shs = atf(kSHs);
  sa.fp4 = fp4;
  sa.hs4 = at(kHs);
  sa.stream = StreamDesc{reinterpret_cast<const int32_t*>(at(kCount)), b.rjob, R, 2 * c.inter / kRowsPerWg,
                         c.hidden / (2 * kTile)};
  sa.ids = ids;
  sa.lb = lb;
  sa.lc = lc;

  CombineArgs ca;
  ca.part = p2;
  ca.splits = p.s2;
  ca.M = M;
  ca.k = c.top_k;
  ca.H = c.hidden;
  ca.weights = weights;
  ca.slots = static_cast<uint16_t*>(slots);
  ca.combined = static_cast<uint16_t*>(combined);
  ca.spart = shared ? atf(kSP2) : nullptr;
  ca.ssplits = p.ss2;
  ca.shared_out = static_cast<uint16_t*>(shared_out);
  ca.ids = ids;
  ca.lb = lb;
  ca.lc = lc;
  ca.fp4 = fp4;
  ca.stream = StreamDesc{reinterpret_cast<const int32_t*>(at(kSwCount)), b.rjob, R, c.hidden / kRowsPerWg,
                         c.inter / (2 * kTile)};

  // problem descriptor of N x K weights and their activations
  auto problem = [](const void* w, const void* ws, const uint8_t* aq, const float* as, float* part, int N,
                    int K, int splits, int ks, int R, int act_div, int tpw) {
    GemmProblem q{};
    q.w = static_cast<const uint8_t*>(w);
    q.ws = static_cast<const float*>(ws);
    q.ws8 = static_cast<const uint8_t*>(ws);
    q.aq = aq;
    q.as = as;
    q.part = part;
    q.N = N;
    q.K = K;
    q.nkb = K / kTile;
    q.tiles = N / kRowsPerWg;
    q.splits = splits;
    q.ks = ks;
    q.R = R;
    q.act_div = act_div;
    q.tpw = tpw;
    return q;
  };
  auto launch_gemm = [&](const GemmArgs& g, int role, int grid) {
    const int persist = role == 1 ? p.persist1 : p.persist2;
    const KernelEvents ev = events(role == 1 ? 1 : 3);
    switch (p.path) {
      case MOE_GEMM_FP4: return launch_gemm_fp4(g, role, grid, s, ev);
      case MOE_GEMM_MFMA:
        return persist ? launch_gemm_wgp(g, role, persist, s, ev) : launch_gemm_wg(g, role, grid, s, ev);
      case MOE_GEMM_MFMA_SPLITK: return launch_gemm_mfma(g, role, grid, s, ev);
      default: return launch_gemm_valu(g, role, grid, s, ev);
    }
  };

  GemmArgs g1{};
  g1.p[1] = problem(c.w13, c.w13_scale, xq, xs, p1, 2 * c.inter, c.hidden, p.s1, p.ks1, R, c.top_k, p.tpw1);
  g1.p[1].b = b;
  g1.p[1].kparts = p.kp1;
  g1.p[1].as8 = at(kXs);
  if (fp4) g1.p[1].ws8 = h->fp4_s13;
  g1.pass_routes = p.pass_routes;
  g1.stream_wgs = h->fp4_wgs1;
  g1.stream_counts = reinterpret_cast<int32_t*>(at(kCount));
  if (shared) {
    g1.p[0] = problem(c.sw13, h->s13, sxq, sxs, atf(kSP1), 2 * c.shared_inter, c.hidden, p.ss1, p.sks1, M, 1,
                      p.stpw1);
    g1.p[0].dense = M;
    g1.p[0].kparts = p.skp1;
    g1.units0 = p.sunits1;
  }
  if (p.route1) {
    RouteFuse& f = g1.rf;
    f.on = 1;
    f.logits = logits;
    f.logits_bf16 = ra.logits_bf16;
    f.bias = bias;
    f.x = ra.x;
    f.M = M;
    f.E = c.experts;
    f.k = c.top_k;
    f.routed_scale = c.routed_scale;
    f.ue8m0 = c.ue8m0_act;
    f.lb = lb;
    f.lc = lc;
    f.ids = ids;
    f.weights = weights;
    f.xq = xq;
    f.xs = xs;
  }
  if (p.fuse_swiglu) {
    SwigluFuse& f = g1.sf;
    f.on = 1;
    f.counters = reinterpret_cast<int32_t*>(at(kSwCount));
    f.I = c.inter;
    f.limit = c.limit;
    f.hq = hq;
    f.hs = hs;
  }
  if (e == hipSuccess) e = launch_gemm(g1, 1, p.grid1 - (shared ? 0 : p.sunits1));

  if (!p.fuse_swiglu && e == hipSuccess) e = launch_swiglu_requant(sa, s, events(2));

  GemmArgs g2{};
  g2.p[1] = problem(c.w2, c.w2_scale, hq, hs, p2, c.hidden, c.inter, p.s2, p.ks2, R, 1, p.tpw2);
  g2.p[1].b = b;
  g2.p[1].kparts = p.kp2;
  g2.p[1].as8 = at(kHs);
  if (fp4) g2.p[1].ws8 = h->fp4_s2;
  g2.pass_routes = p.pass_routes;
  g2.stream_wgs = h->fp4_wgs2;
  g2.stream_counts = reinterpret_cast<int32_t*>(at(kSwCount));
  if (shared) {
    g2.p[0] = problem(c.sw2, h->s2, at(kSHq), atf(kSHs), atf(kSP2), c.hidden, c.shared_inter, p.ss2, p.sks2,
                      M, 1, p.stpw2);
    g2.p[0].dense = M;
    g2.p[0].kparts = p.skp2;
    g2.units0 = p.sunits2;
  }
  if (p.fuse_combine) {
    CombineFuse& f = g2.cf;
    f.on = 1;
    f.counters = reinterpret_cast<int32_t*>(at(kCount));
    f.ids = ids;
    f.weights = weights;
    f.slots = ca.slots;
    f.combined = ca.combined;
    f.shared_out = ca.shared_out;
    f.M = M;
    f.k = c.top_k;
    f.lb = lb;
    f.lc = lc;
    f.all_local = lb == 0 && lc == c.experts;
  }
  if (e == hipSuccess) e = launch_gemm(g2, 2, p.grid2 - (shared ? 0 : p.sunits2));

  if (!p.fuse_combine && e == hipSuccess) e = launch_combine(ca, s, events(4));

  h->timed_run = h->timing;
  h->ev_slots = slots_run;
  return e == hipSuccess ? MOE_DECODE_OK : MOE_DECODE_ERR_HIP;
}

}  // namespace

extern "C" {

const char* moe_decode_error_string(int code) {
  switch (code) {
    case MOE_DECODE_OK: return "ok";
    case MOE_DECODE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_DECODE_ERR_UNSUPPORTED: return "unsupported shape or option";
    case MOE_DECODE_ERR_TOO_MANY_TOKENS: return "more tokens than the handle's max_tokens";
    case MOE_DECODE_ERR_HIP: return "HIP runtime error";
    case MOE_DECODE_ERR_OUT_OF_MEMORY: return "out of device memory";
    case MOE_DECODE_ERR_SCRATCH_TOO_SMALL:
      return "the step needs more workspace than the no-allocation buffer holds";
    default: return "unknown error";
  }
}

int moe_decode_create(const moe_decode_config* cfg, moe_decode_t* out) {
  if (!out) return MOE_DECODE_ERR_INVALID_ARG;
  *out = nullptr;
  const int v = validate_config(cfg);
  if (v != MOE_DECODE_OK) return v;
  const moe_decode_config& c = *cfg;

  const bool fp4 = c.weight_format == MOE_WEIGHTS_NVFP4;
  const size_t H = c.hidden, I = c.inter, Is = c.shared_inter;
  moe_decode_handle* h = new (std::nothrow) moe_decode_handle();
  if (!h) return MOE_DECODE_ERR_OUT_OF_MEMORY;
  h->cfg = c;
  h->ws_bytes = layout_workspace(c, h->reg, &h->shared_own_quant);
  h->words = (c.max_tokens + 63) / 64;
  if (hipGetDevice(&h->device) != hipSuccess) {
    delete h;
    return MOE_DECODE_ERR_HIP;
  }
  if (hipMalloc(&h->ws, h->ws_bytes) != hipSuccess) {
    (void)hipGetLastError();
    delete h;
    return MOE_DECODE_ERR_OUT_OF_MEMORY;
  }
  if (hipMemset(h->ws, 0, h->ws_bytes) != hipSuccess) {
    (void)hipFree(h->ws);
    delete h;
    return MOE_DECODE_ERR_HIP;
  }
  for (int i = 0; i < kEvents; ++i) {
    if (hipEventCreate(&h->ev[i]) != hipSuccess) {
      for (int j = 0; j < i; ++j) (void)hipEventDestroy(h->ev[j]);
      (void)hipFree(h->ws);
      delete h;
      return MOE_DECODE_ERR_HIP;
    }
  }
  if (!fp4) {  // 0 (one workgroup per unit) if the query fails
    h->wgp_wgs1 = gemm_wgp_resident_wgs(c.hidden / kTile);
    h->wgp_wgs2 = gemm_wgp_resident_wgs(c.inter / kTile);
    if (gemm_wgp_route_fits(c.hidden / kTile, c.experts))
      h->wgp_route_wgs1 = gemm_wgp_route_resident_wgs(c.hidden / kTile, c.experts);
  }
  if (fp4) {
    h->fp4_wgs1 = gemm_fp4_resident_wgs(c.hidden);
    h->fp4_wgs2 = gemm_fp4_resident_wgs(c.inter);
    if (h->fp4_wgs1 <= 0 || h->fp4_wgs2 <= 0) {
      moe_decode_destroy(h);
      return MOE_DECODE_ERR_HIP;
    }
    // the weight scales, read once here into the kernel's layout
    const size_t El = local_count(c), rows13 = El * 2 * I, rows2 = El * H;
    if (hipMalloc(&h->fp4_s13, rows13 * (H / 16)) != hipSuccess ||
        hipMalloc(&h->fp4_s2, rows2 * (I / 16)) != hipSuccess) {
      (void)hipGetLastError();
      moe_decode_destroy(h);
      return MOE_DECODE_ERR_OUT_OF_MEMORY;
    }
    if (launch_reorder_fp4_scales(static_cast<const uint8_t*>(c.w13_scale), h->fp4_s13, rows13, (int)H,
                                  nullptr) != hipSuccess ||
        launch_reorder_fp4_scales(static_cast<const uint8_t*>(c.w2_scale), h->fp4_s2, rows2, (int)I, nullptr) !=
            hipSuccess ||
        hipDeviceSynchronize() != hipSuccess) {
      moe_decode_destroy(h);
      return MOE_DECODE_ERR_HIP;
    }
  }
  if (Is > 0) {
    const int r = prepare_shared_scales(h);
    if (r != MOE_DECODE_OK) {
      moe_decode_destroy(h);
      return r;
    }
  }
  if (std::getenv("MOE_DECODE_DEBUG")) {
    const Plan p = make_plan(c, c.max_tokens, h->fp4_wgs1, h->fp4_wgs2, h->wgp_wgs1, h->wgp_wgs2,
                             h->wgp_route_wgs1);
    std::fprintf(stderr,
                 "moe_decode: H=%d I=%d E=%d k=%d max_tokens=%d workspace=%zu B; at M=%d: "
                 "path=%d splits1=%d (ks %d) splits2=%d (ks %d) grid1=%d grid2=%d\n",
                 c.hidden, c.inter, c.experts, c.top_k, c.max_tokens, h->ws_bytes, c.max_tokens,
                 p.path, p.s1, p.ks1, p.s2, p.ks2, p.grid1, p.grid2);
  }
  *out = h;
  return MOE_DECODE_OK;
}

void moe_decode_destroy(moe_decode_t h) {
  if (!h) return;
  int prev = 0;
  (void)hipGetDevice(&prev);
  (void)hipSetDevice(h->device);
  (void)hipDeviceSynchronize();
  for (int i = 0; i < kEvents; ++i) (void)hipEventDestroy(h->ev[i]);
  (void)hipFree(h->ws);
  if (h->s13_owned) (void)hipFree(h->s13_owned);
  if (h->s2_owned) (void)hipFree(h->s2_owned);
  if (h->fp4_s13) (void)hipFree(h->fp4_s13);
  if (h->fp4_s2) (void)hipFree(h->fp4_s2);
  (void)hipSetDevice(prev);
  delete h;
}

int moe_decode_plan(moe_decode_t h, int32_t M, int32_t* out, int32_t n) {
  if (!h || !out || n < 9 || M < 1) return MOE_DECODE_ERR_INVALID_ARG;
  if (M > h->cfg.max_tokens) return MOE_DECODE_ERR_TOO_MANY_TOKENS;
  const Plan p = make_plan(h->cfg, M, h->fp4_wgs1, h->fp4_wgs2, h->wgp_wgs1, h->wgp_wgs2, h->wgp_route_wgs1);
  out[0] = p.path;
  out[1] = p.s1;
  out[2] = p.s2;
  const int blk = p.path == MOE_GEMM_FP4 ? 2 : 1;  // the FP4 plan counts 256-value steps
  out[3] = p.ks1 * blk;
  out[4] = p.ks2 * blk;
  out[5] = p.grid1;
  out[6] = p.grid2;
  out[7] = p.tpw1;
  out[8] = p.tpw2;
  if (n >= 15) {
    out[9] = p.ss1;
    out[10] = p.ss2;
    out[11] = p.sks1;
    out[12] = p.sks2;
    out[13] = p.sunits1;
    out[14] = p.sunits2;
  }
  if (n >= 17) {
    out[15] = p.path == MOE_GEMM_MFMA ? p.kp1 : 1;
    out[16] = p.path == MOE_GEMM_MFMA ? p.kp2 : 1;
  }
  if (n >= 18) out[17] = 5 - (p.fuse_combine ? 1 : 0) - (p.fuse_swiglu ? 1 : 0) - (p.route1 ? 1 : 0);
  if (n >= 20) {
    out[18] = p.persist1;
    out[19] = p.persist2;
  }
  return MOE_DECODE_OK;
}

int moe_decode_run(moe_decode_t h, int32_t M, const void* x, const void* logits, const float* bias,
                   void* slots, int32_t* ids, float* weights, void* combined, void* shared_out,
                   void* stream) {
  if (!h) return MOE_DECODE_ERR_INVALID_ARG;
  if (M < 0) return MOE_DECODE_ERR_INVALID_ARG;
  if (M > h->cfg.max_tokens) return MOE_DECODE_ERR_TOO_MANY_TOKENS;
  if (M == 0) return MOE_DECODE_OK;
  const int r = check_run_pointers(h->cfg, x, logits, bias, slots, ids, weights, combined, shared_out);
  if (r != MOE_DECODE_OK) return r;
  return run_layer(h, M, x, logits, bias, slots, ids, weights, combined, shared_out,
                   static_cast<hipStream_t>(stream));
}

int moe_decode_run_noalloc(const moe_decode_config* cfg, int32_t M, const void* x, const void* logits,
                           const float* bias, void* slots, int32_t* ids, float* weights, void* combined,
                           void* shared_out, void* stream) {
  if (!cfg || M < 0) return MOE_DECODE_ERR_INVALID_ARG;
  if (M > MOE_DECODE_MAX_TOKENS) return MOE_DECODE_ERR_TOO_MANY_TOKENS;
  moe_decode_handle h{};  // on the stack; its workspace is this device's scratch
  h.cfg = *cfg;
  moe_decode_config& c = h.cfg;
  c.max_tokens = std::max(M, 1);
  const int v = validate_config(&c);
  if (v != MOE_DECODE_OK) return v;
  // no handle-owned copies: FP4 scales are reordered, and packed shared
  // scales converted, into memory a handle owns
  if (c.weight_format != MOE_WEIGHTS_FP8 || (c.shared_inter > 0 && c.shared_scale_format != MOE_SCALES_F32))
    return MOE_DECODE_ERR_UNSUPPORTED;
  if (M == 0) return MOE_DECODE_OK;
  const int r = check_run_pointers(c, x, logits, bias, slots, ids, weights, combined, shared_out);
  if (r != MOE_DECODE_OK) return r;
  h.ws_bytes = layout_workspace(c, h.reg, &h.shared_own_quant);
  if (h.ws_bytes > kScratchBytes) return MOE_DECODE_ERR_SCRATCH_TOO_SMALL;
  if (hipGetDevice(&h.device) != hipSuccess) return MOE_DECODE_ERR_HIP;
  h.ws = device_scratch(h.device);
  if (!h.ws) return MOE_DECODE_ERR_HIP;
  h.words = (M + 63) / 64;
  h.s13 = static_cast<const float*>(c.sw13_scale);
  h.s2 = static_cast<const float*>(c.sw2_scale);
  h.wgp_wgs1 = cached_wgp_wgs(h.device, c.hidden / kTile);
  h.wgp_wgs2 = cached_wgp_wgs(h.device, c.inter / kTile);
  if (gemm_wgp_route_fits(c.hidden / kTile, c.experts))
    h.wgp_route_wgs1 = cached_wgp_route_wgs(h.device, c.hidden / kTile, c.experts);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // The buffer holds the previous call's data, in that call's layout: clear
  // the arrival counters this step's kernels expect at zero.
  const Plan p = make_plan(c, M, 0, 0, h.wgp_wgs1, h.wgp_wgs2, h.wgp_route_wgs1);
  auto words_of = [&](int i) { return reinterpret_cast<int32_t*>(h.ws + h.reg[i].off); };
  hipError_t e = launch_zero_words(words_of(kCtrl), h.reg[kCtrl].bytes / sizeof(int32_t), s);
  if (e == hipSuccess && p.fuse_combine)
    e = launch_zero_words(words_of(kCount), h.reg[kCount].bytes / sizeof(int32_t), s);
  if (e == hipSuccess && p.fuse_swiglu)
    e = launch_zero_words(words_of(kSwCount), h.reg[kSwCount].bytes / sizeof(int32_t), s);
  if (e != hipSuccess) return MOE_DECODE_ERR_HIP;
  return run_layer(&h, M, x, logits, bias, slots, ids, weights, combined, shared_out, s);
}

int moe_decode_debug_stage(moe_decode_t h, int32_t stage, void* dst, size_t bytes, void* stream) {
  if (!h || !dst || stage < 0) return MOE_DECODE_ERR_INVALID_ARG;
  if (stage == kStageSharedScale13 || stage == kStageSharedScale2) {
    // The shared expert's FP32 block scales as the kernels read them.
    const moe_decode_config& c = h->cfg;
    if (c.shared_inter == 0) return MOE_DECODE_ERR_INVALID_ARG;
    const size_t H = c.hidden / kTile, Is = c.shared_inter / kTile;
    const size_t full = (stage == kStageSharedScale13 ? 2 * Is * H : H * Is) * sizeof(float);
    const hipError_t e = hipMemcpyAsync(dst, stage == kStageSharedScale13 ? h->s13 : h->s2,
                                        std::min(bytes, full), hipMemcpyDeviceToDevice,
                                        static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MOE_DECODE_OK : MOE_DECODE_ERR_HIP;
  }
  if (stage >= kCount) return MOE_DECODE_ERR_INVALID_ARG;
  if (stage >= kSXq && stage <= kSP2 && h->cfg.shared_inter == 0) return MOE_DECODE_ERR_INVALID_ARG;
  if (stage >= kJobs && h->cfg.weight_format != MOE_WEIGHTS_NVFP4) return MOE_DECODE_ERR_INVALID_ARG;
  if (!h->shared_own_quant && (stage == kSXq || stage == kSXs)) stage = stage == kSXq ? kXq : kXs;
  const Region& r = h->reg[stage];
  const size_t n = std::min(bytes, r.bytes);
  const hipError_t e =
      hipMemcpyAsync(dst, h->ws + r.off, n, hipMemcpyDeviceToDevice, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_DECODE_OK : MOE_DECODE_ERR_HIP;
}

int moe_decode_set_timing(moe_decode_t h, int32_t enable) {
  if (!h) return MOE_DECODE_ERR_INVALID_ARG;
  h->timing = enable != 0;
  return MOE_DECODE_OK;
}

int moe_decode_last_timing(moe_decode_t h, float* ms, int32_t n) {
  if (!h || !ms || n < kStages) return MOE_DECODE_ERR_INVALID_ARG;
  for (int i = 0; i < kStages; ++i) ms[i] = 0.f;
  if (!h->timed_run || h->ev_slots == 0) return MOE_DECODE_ERR_INVALID_ARG;
  for (int i = 0; i < kStages; ++i) {
    if (!(h->ev_slots & (1 << i))) continue;
    if (hipEventSynchronize(h->ev[2 * i + 1]) != hipSuccess) return MOE_DECODE_ERR_HIP;
    if (hipEventElapsedTime(&ms[i], h->ev[2 * i], h->ev[2 * i + 1]) != hipSuccess) return MOE_DECODE_ERR_HIP;
  }
  return MOE_DECODE_OK;
}

int moe_decode_debug_codec_fp4(const float* in, uint8_t* q, float* dq, int32_t n, void* stream) {
  if (!in || !q || !dq || n < 0) return MOE_DECODE_ERR_INVALID_ARG;
  if (n == 0) return MOE_DECODE_OK;
  return launch_codec_check_fp4(in, q, dq, n, static_cast<hipStream_t>(stream)) == hipSuccess
             ? MOE_DECODE_OK
             : MOE_DECODE_ERR_HIP;
}

int moe_decode_debug_codec(const float* in, uint8_t* q, float* dq, int32_t n, void* stream) {
  if (!in || !q || !dq || n < 0) return MOE_DECODE_ERR_INVALID_ARG;
  if (n == 0) return MOE_DECODE_OK;
  return launch_codec_check(in, q, dq, n, static_cast<hipStream_t>(stream)) == hipSuccess
             ? MOE_DECODE_OK
             : MOE_DECODE_ERR_HIP;
}

}  // extern "C"
