// The FP4 GEMM's work split (stream-K style): the items (job, 64-row tile,
// 256-value K step), the step fastest, form one stream of T = J * tiles *
// steps items. Workgroup w of Wa active ones takes items
// [w * T / Wa, (w + 1) * T / Wa), so every workgroup streams the same number
// of weight bytes (to one item) whatever the number of touched experts. Wa is
// at least J, so no range is longer than one job's items and a range touches
// at most two jobs; the launch grid must therefore hold at least J
// workgroups (J is at most the number of routes). A tile whose K steps span
// several workgroups gets one FP32 partial per workgroup, part[slot] with
// slot = w - (first workgroup of the tile); the next kernel adds a tile's
// slots in slot order, a fixed order for a given J.
#pragma once

#include "kernels.h"

namespace moe {

// Fewest items per active workgroup: bounds the partial slots of a tile.
constexpr int kStreamMinSteps = 4;

struct StreamMap {
  int64_t T;  // items
  int Wa;     // active workgroups
};

// wgs: the launch's resident workgroups. Every range holds at least
// kStreamMinSteps items: T / wa >= 4 by the first bound, and when J raises
// wa, T / J = tiles * steps >= 4 for every shape the library accepts.
__host__ __device__ __forceinline__ StreamMap stream_map(int J, int tiles, int steps, int wgs) {
  const int64_t T = (int64_t)J * tiles * steps;
  int64_t wa = T / kStreamMinSteps;
  wa = wa < wgs ? wa : wgs;
  wa = wa > J ? wa : J;
  return StreamMap{T, (int)(wa > 1 ? wa : 1)};
}

__host__ __device__ __forceinline__ int64_t stream_begin(int w, const StreamMap& m) {
  return (int64_t)w * m.T / m.Wa;
}

// The workgroup whose range holds item i (0 <= i < T): the largest w with
// stream_begin(w) <= i.
__host__ __device__ __forceinline__ int stream_owner(int64_t i, const StreamMap& m) {
  return (int)(((i + 1) * m.Wa - 1) / m.T);
}

// Partial slots a tile can have: every active range holds at least
// kStreamMinSteps items, so the steps - 1 item boundaries inside a tile fall
// in at most ceil((steps - 1) / kStreamMinSteps) ranges after the first.
__host__ __device__ __forceinline__ int stream_max_slots(int steps) {
  return (steps - 1 + kStreamMinSteps - 1) / kStreamMinSteps + 1;
}

// Slots of row n's tile for route r, whose job the routing kernel recorded.
// The count is kept within [0, stream_max_slots(steps)] whatever the control
// words hold (no jobs at all gives 0), so a caller's loop over the slots
// stays inside the partial buffer.
__device__ __forceinline__ int stream_slots(const StreamDesc& d, int r, int n) {
  const StreamMap m = stream_map(d.ctrl[2], d.tiles, d.steps, d.wgs);
  if (m.T <= 0) return 0;
  const int64_t base = ((int64_t)d.rjob[r] * d.tiles + n / kRowsPerWg) * d.steps;
  if (base < 0 || base + d.steps > m.T) return 0;
  const int slots = stream_owner(base + d.steps - 1, m) - stream_owner(base, m) + 1;
  return min(max(slots, 0), stream_max_slots(d.steps));
}

}  // namespace moe
