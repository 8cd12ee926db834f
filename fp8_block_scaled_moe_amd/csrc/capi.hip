// The C ABI: handle creation (validation, workspace, scale conversion), the
// per-call launch plan, and the launches of one routed-expert step.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

#include "../../include/moe_decode.h"
#include "kernels.h"

using namespace moe;

namespace {

constexpr int kEvents = 8;
constexpr int kRegions = 11;
constexpr int kStages = 7;  // timing slots: route, GEMM1, SwiGLU, GEMM2, combine, shared x2
constexpr int kTargetUnits = 4096;  // work units per GEMM launch to aim for (16 per CU)

struct Plan {
  int path;
  int s1, ks1, s2, ks2;
  int grid1, grid2;
  int umax;
  int pass_routes;  // MFMA path: routes per pass
  int tpw1, tpw2;   // 64-row tiles per workgroup
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
  // shared expert scales converted to FP32 (owned), or the caller's FP32 ones
  float* s13_owned;
  float* s2_owned;
  const float* s13;
  const float* s2;
  bool timing;
  bool timed_run;
  hipEvent_t ev[kEvents];
  int ev_stage[kEvents];  // timing slot of the interval that ends at event i
  int ev_count;           // events recorded by the last timed run
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

Plan make_plan(const moe_decode_config& c, int M) {
  Plan p{};
  const int R = M * c.top_k;
  p.umax = std::min(c.experts, R);
  const int tiles1 = 2 * c.inter / kRowsPerWg, tiles2 = c.hidden / kRowsPerWg;
  // MFMA costs the same per weight byte for any number of routes of an
  // expert (up to 16 per pass), VALU dot products cost per route. Measured on
  // MI355X with every expert taking n routes (E=64, H=7168, I=2048), GEMM1
  // streams at 6.69/6.67 TB/s (VALU/MFMA) for n=1, 5.68/5.86 for n=4,
  // 4.10/5.46 for n=8 and 2.01/5.06 for n=16; so MFMA unless every expert has
  // exactly one route (M = 1).
  if (c.gemm_path == MOE_GEMM_AUTO)
    p.path = M == 1 ? MOE_GEMM_VALU : MOE_GEMM_MFMA;
  else
    p.path = c.gemm_path;
  // an expert has at most one route per token
  p.pass_routes = std::min(kMfmaRoutes, M);
  int max_ks = kMaxKs;
  if (p.path == MOE_GEMM_MFMA)
    while (max_ks > 1 && gemm_mfma_lds_bytes(p.pass_routes, max_ks) > kMfmaLdsBudget) --max_ks;
  // Staging a unit's activations costs about as much as streaming a few
  // blocks of weights per route; with many tokens (so many routes per
  // expert) a workgroup streams several tiles per staging.
  const int want = M <= 2 ? 1 : (M <= 8 ? 2 : kMaxTpw);
  auto tiles_per_wg = [&](int tiles) {
    int t = want;
    while (tiles % t) t /= 2;
    return t;
  };
  p.tpw1 = tiles_per_wg(tiles1);
  p.tpw2 = tiles_per_wg(tiles2);
  choose_split(p.umax * (tiles1 / p.tpw1), c.hidden / kTile, c.splits1, max_ks, &p.s1, &p.ks1);
  choose_split(p.umax * (tiles2 / p.tpw2), c.inter / kTile, c.splits2, max_ks, &p.s2, &p.ks2);
  p.grid1 = p.umax * (tiles1 / p.tpw1) * p.s1;
  p.grid2 = p.umax * (tiles2 / p.tpw2) * p.s2;
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
  if (c->splits1 < 0 || c->splits2 < 0) return MOE_DECODE_ERR_INVALID_ARG;
  {
    const int words = (c->max_tokens + 63) / 64;
    if (route_quant_lds_bytes(c->experts, words, c->max_tokens * c->top_k) > kMaxRouteLds)
      return MOE_DECODE_ERR_UNSUPPORTED;
  }
  if (c->shared_inter != 0) {
    // The shared expert is not built into this library yet.
    return MOE_DECODE_ERR_UNSUPPORTED;
  }
  return MOE_DECODE_OK;
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
    default: return "unknown error";
  }
}

int moe_decode_create(const moe_decode_config* cfg, moe_decode_t* out) {
  if (!out) return MOE_DECODE_ERR_INVALID_ARG;
  *out = nullptr;
  const int v = validate_config(cfg);
  if (v != MOE_DECODE_OK) return v;
  const moe_decode_config& c = *cfg;

  // Workspace sized for every M up to max_tokens.
  const size_t Rcap = (size_t)c.max_tokens * c.top_k;
  const size_t Ucap = std::min<size_t>(c.experts, Rcap);
  size_t p1 = 0, p2 = 0;
  for (int M = 1; M <= c.max_tokens; ++M) {
    const Plan p = make_plan(c, M);
    p1 = std::max(p1, (size_t)p.s1 * M * c.top_k * 2 * c.inter);
    p2 = std::max(p2, (size_t)p.s2 * M * c.top_k * c.hidden);
  }
  const size_t H = c.hidden, I = c.inter;
  const size_t sizes[kRegions] = {
      64 * sizeof(int32_t),           // 0 control
      Ucap * sizeof(int32_t),         // 1 uexp
      Ucap * sizeof(int32_t),         // 2 uoff
      Ucap * sizeof(int32_t),         // 3 ucnt
      Rcap * sizeof(int32_t),         // 4 routes
      (size_t)c.max_tokens * H,       // 5 x_q
      (size_t)c.max_tokens * (H / kTile) * sizeof(float),  // 6 x_s
      p1 * sizeof(float),             // 7 GEMM1 partials
      Rcap * I,                       // 8 h_q
      Rcap * (I / kTile) * sizeof(float),  // 9 h_s
      p2 * sizeof(float),             // 10 GEMM2 partials
  };
  moe_decode_handle* h = new (std::nothrow) moe_decode_handle();
  if (!h) return MOE_DECODE_ERR_OUT_OF_MEMORY;
  h->cfg = c;
  size_t off = 0;
  for (int i = 0; i < kRegions; ++i) {
    h->reg[i] = Region{off, sizes[i]};
    off += (sizes[i] + 255) & ~size_t(255);
  }
  h->ws_bytes = off;
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
  if (std::getenv("MOE_DECODE_DEBUG")) {
    const Plan p = make_plan(c, c.max_tokens);
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
  (void)hipSetDevice(prev);
  delete h;
}

int moe_decode_plan(moe_decode_t h, int32_t M, int32_t* out, int32_t n) {
  if (!h || !out || n < 9 || M < 1) return MOE_DECODE_ERR_INVALID_ARG;
  if (M > h->cfg.max_tokens) return MOE_DECODE_ERR_TOO_MANY_TOKENS;
  const Plan p = make_plan(h->cfg, M);
  out[0] = p.path;
  out[1] = p.s1;
  out[2] = p.s2;
  out[3] = p.ks1;
  out[4] = p.ks2;
  out[5] = p.grid1;
  out[6] = p.grid2;
  out[7] = p.tpw1;
  out[8] = p.tpw2;
  return MOE_DECODE_OK;
}

int moe_decode_run(moe_decode_t h, int32_t M, const void* x, const void* logits, const float* bias,
                   void* slots, int32_t* ids, float* weights, void* combined, void* shared_out,
                   void* stream) {
  if (!h) return MOE_DECODE_ERR_INVALID_ARG;
  if (M < 0) return MOE_DECODE_ERR_INVALID_ARG;
  if (M > h->cfg.max_tokens) return MOE_DECODE_ERR_TOO_MANY_TOKENS;
  if (M == 0) return MOE_DECODE_OK;
  if (!x || !logits || !bias || !slots || !ids || !weights || !combined)
    return MOE_DECODE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(slots) || !aligned16(combined) || !aligned16(logits) ||
      ((uintptr_t)ids & 3u) || ((uintptr_t)weights & 3u) || ((uintptr_t)bias & 3u))
    return MOE_DECODE_ERR_INVALID_ARG;
  if (shared_out) return MOE_DECODE_ERR_INVALID_ARG;  // no shared expert in this handle

  const moe_decode_config& c = h->cfg;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Plan p = make_plan(c, M);
  const int R = M * c.top_k;
  unsigned char* ws = h->ws;
  auto at = [&](int i) { return ws + h->reg[i].off; };

  Buckets b;
  b.ctrl = reinterpret_cast<int32_t*>(at(0));
  b.uexp = reinterpret_cast<int32_t*>(at(1));
  b.uoff = reinterpret_cast<int32_t*>(at(2));
  b.ucnt = reinterpret_cast<int32_t*>(at(3));
  b.routes = reinterpret_cast<int32_t*>(at(4));
  uint8_t* xq = at(5);
  float* xs = reinterpret_cast<float*>(at(6));
  float* p1 = reinterpret_cast<float*>(at(7));
  uint8_t* hq = at(8);
  float* hs = reinterpret_cast<float*>(at(9));
  float* p2 = reinterpret_cast<float*>(at(10));

  int evn = 0;
  // records an event closing timing slot `stage` (the first call opens)
  auto mark = [&](int stage) -> hipError_t {
    if (!h->timing) return hipSuccess;
    h->ev_stage[evn] = stage;
    return hipEventRecord(h->ev[evn++], s);
  };

  hipError_t e = mark(-1);

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
  ra.b = b;
  if (e == hipSuccess) e = launch_route_quant(ra, s);
  if (e == hipSuccess) e = mark(0);

  SwigluArgs sa;
  sa.part = p1;
  sa.splits = p.s1;
  sa.R = R;
  sa.I = c.inter;
  sa.limit = c.limit;
  sa.hq = hq;
  sa.hs = hs;

  CombineArgs ca;
  ca.part = p2;
  ca.splits = p.s2;
  ca.M = M;
  ca.k = c.top_k;
  ca.H = c.hidden;
  ca.weights = weights;
  ca.slots = static_cast<uint16_t*>(slots);
  ca.combined = static_cast<uint16_t*>(combined);

  GemmArgs g1;
  g1.w = static_cast<const uint8_t*>(c.w13);
  g1.ws = c.w13_scale;
  g1.aq = xq;
  g1.as = xs;
  g1.part = p1;
  g1.b = b;
  g1.N = 2 * c.inter;
  g1.K = c.hidden;
  g1.nkb = c.hidden / kTile;
  g1.tiles = g1.N / kRowsPerWg;
  g1.splits = p.s1;
  g1.ks = p.ks1;
  g1.R = R;
  g1.act_div = c.top_k;
  g1.pass_routes = p.pass_routes;
  g1.tpw = p.tpw1;
  if (e == hipSuccess)
    e = p.path == MOE_GEMM_MFMA ? launch_gemm_mfma(g1, 1, p.grid1, s) : launch_gemm_valu(g1, 1, p.grid1, s);
  if (e == hipSuccess) e = mark(1);

  if (e == hipSuccess) e = launch_swiglu_requant(sa, s);
  if (e == hipSuccess) e = mark(2);

  GemmArgs g2 = g1;
  g2.w = static_cast<const uint8_t*>(c.w2);
  g2.ws = c.w2_scale;
  g2.aq = hq;
  g2.as = hs;
  g2.part = p2;
  g2.N = c.hidden;
  g2.K = c.inter;
  g2.nkb = c.inter / kTile;
  g2.tiles = g2.N / kRowsPerWg;
  g2.splits = p.s2;
  g2.ks = p.ks2;
  g2.act_div = 1;
  g2.tpw = p.tpw2;
  if (e == hipSuccess)
    e = p.path == MOE_GEMM_MFMA ? launch_gemm_mfma(g2, 2, p.grid2, s) : launch_gemm_valu(g2, 2, p.grid2, s);
  if (e == hipSuccess) e = mark(3);

  if (e == hipSuccess) e = launch_combine(ca, s);
  if (e == hipSuccess) e = mark(4);

  h->timed_run = h->timing;
  h->ev_count = evn;
  return e == hipSuccess ? MOE_DECODE_OK : MOE_DECODE_ERR_HIP;
}

int moe_decode_debug_stage(moe_decode_t h, int32_t stage, void* dst, size_t bytes, void* stream) {
  if (!h || !dst || stage < 0 || stage > 10) return MOE_DECODE_ERR_INVALID_ARG;
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
  if (!h->timed_run || h->ev_count < 2) return MOE_DECODE_ERR_INVALID_ARG;
  const int last = h->ev_count - 1;
  if (hipEventSynchronize(h->ev[last]) != hipSuccess) return MOE_DECODE_ERR_HIP;
  for (int i = 1; i <= last; ++i) {
    float t = 0.f;
    if (hipEventElapsedTime(&t, h->ev[i - 1], h->ev[i]) != hipSuccess) return MOE_DECODE_ERR_HIP;
    ms[h->ev_stage[i]] += t;
  }
  return MOE_DECODE_OK;
}

int moe_decode_debug_codec(const float* in, uint8_t* q, float* dq, int32_t n, void* stream) {
  if (!in || !q || !dq || n < 0) return MOE_DECODE_ERR_INVALID_ARG;
  if (n == 0) return MOE_DECODE_OK;
  return launch_codec_check(in, q, dq, n, static_cast<hipStream_t>(stream)) == hipSuccess
             ? MOE_DECODE_OK
             : MOE_DECODE_ERR_HIP;
}

}  // extern "C"
