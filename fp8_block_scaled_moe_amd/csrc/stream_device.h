// The FP4 GEMM's work split (stream-K style): the items (job, 64-row tile,
// 256-value K step), the step fastest, form one stream of T = J * tiles *
// steps items. With T = Wa * q + r (0 <= r < Wa), workgroup w of Wa active
// ones takes the q + (w < r) items from w * q + min(w, r) on, so every
// workgroup streams the same number of weight bytes (to one item) whatever
// the number of touched experts. Wa is at least J, so no range is longer than
// one job's items and a range touches at most two jobs; the launch grid must
// therefore hold at least J workgroups (J is at most the number of routes).
// A tile whose K steps span several workgroups gets one FP32 partial per
// workgroup, part[slot] with slot = w - (first workgroup of the tile); the
// workgroup that sums a tile's last step records the tile's slot count, and
// the next kernel adds a tile's slots in slot order, a fixed order for a
// given J. T stays below 2^32 for every shape the library accepts (routes <=
// 8192, tiles <= 1304, steps <= 326), so the arithmetic is 32-bit.
//
// Measured on MI355X (FP4 share, GEMM1): a CU's four resident workgroups end
// in the order they arrived (13.8, 16.0, 18.3 and 21.0 us, the first ones'
// waves winning the SIMDs' issue arbitration), but weighting the shares by
// that order (8:7:6:5) moved the first ones' end to 16.1 us and left the
// last ones' at 21.4 us: a CU is busy until its last workgroup ends either
// way, so the shares stay even.
#pragma once

#include "kernels.h"

namespace moe {

// Fewest items per active workgroup: bounds the partial slots of a tile.
constexpr int kStreamMinSteps = 4;

struct StreamMap {
  uint32_t T;     // items
  int Wa;         // active workgroups
  uint32_t q, r;  // T = Wa * q + r
};

// wgs: the launch's resident workgroups. Every range holds at least
// kStreamMinSteps items: T / wa >= 4 by the first bound, and when J raises
// wa, T / J = tiles * steps >= 4 for every shape the library accepts.
__host__ __device__ __forceinline__ StreamMap stream_map(int J, int tiles, int steps, int wgs) {
  const uint32_t T = (uint32_t)J * (uint32_t)tiles * (uint32_t)steps;
  uint32_t wa = T / kStreamMinSteps;
  wa = wa < (uint32_t)wgs ? wa : (uint32_t)wgs;
  wa = wa > (uint32_t)J ? wa : (uint32_t)J;
  wa = wa > 1 ? wa : 1;
  return StreamMap{T, (int)wa, T / wa, T % wa};
}

__host__ __device__ __forceinline__ uint32_t stream_begin(int w, const StreamMap& m) {
  return (uint32_t)w * m.q + ((uint32_t)w < m.r ? (uint32_t)w : m.r);
}

// The workgroup whose range holds item i (0 <= i < T).
__host__ __device__ __forceinline__ int stream_owner(uint32_t i, const StreamMap& m) {
  const uint32_t big = m.r * (m.q + 1);  // items of the r longer ranges
  return i < big ? (int)(i / (m.q + 1)) : (int)(m.r + (i - big) / m.q);
}

// Partial slots a tile can have: every active range holds at least
// kStreamMinSteps items, so the steps - 1 item boundaries inside a tile fall
// in at most ceil((steps - 1) / kStreamMinSteps) ranges after the first.
__host__ __device__ __forceinline__ int stream_max_slots(int steps) {
  return (steps - 1 + kStreamMinSteps - 1) / kStreamMinSteps + 1;
}

// Slots of row n's tile for route r, as the GEMM recorded them for the
// route's job; kept within [0, stream_max_slots(steps)], so a caller's loop
// over the slots stays inside the partial buffer.
__device__ __forceinline__ int stream_slots(const StreamDesc& d, int r, int n) {
  const int j = d.rjob[r];
  if (j < 0 || j >= d.R) return 0;
  const int slots = d.counts[(size_t)j * d.tiles + n / kRowsPerWg];
  return min(max(slots, 0), stream_max_slots(d.steps));
}

}  // namespace moe
