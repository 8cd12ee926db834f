// Routing and FP8 activation staging, shared by the routing kernel and the
// routing prologue of the persistent GEMM1: both run these same functions,
// so both produce the same picks, weights, buckets and codes.
//
// Routing follows the vLLM "mega_moe" page (top_k_pick, _ordered): FP32
// sigmoid scores, FP32 keys score + bias compared through a monotone integer
// image, the top_k largest keys in order with ties to the lower expert,
// weights = picked score / (FP32 sum of picked scores in pick order) * scale.
// The activation quantiser is the same page's epilogue: per 128 values,
// scale = max(amax, 1e-10) / 448 (IEEE divide), optionally rounded up to a
// power of two after flooring it at 1e-10, then v * (1 / scale) encoded to
// e4m3.
#pragma once

#include "kernels.h"
#include "device_common.h"

namespace moe {

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

// Router logits ([M, E] f32 or bf16) at flat indices at[q] (each in
// bounds), as FP32. Every load is issued before any value is widened, so a
// thread waits for memory once, not once per logit.
template <int kN>
__device__ __forceinline__ void load_logits(const void* logits, int bf16, const int (&at)[kN], float (&z)[kN]) {
  uint32_t raw[kN];
  if (bf16) {
#pragma unroll
    for (int q = 0; q < kN; ++q) raw[q] = ((const uint16_t*)logits)[at[q]];
  } else {
#pragma unroll
    for (int q = 0; q < kN; ++q) raw[q] = ((const uint32_t*)logits)[at[q]];
  }
#pragma unroll
  for (int q = 0; q < kN; ++q) z[q] = __uint_as_float(bf16 ? raw[q] << 16 : raw[q]);
}

// Wave-wide maximum of a uint32: DPP permutations inside each row of 16
// lanes (swap neighbours, swap pairs, half-row mirror, row mirror), then the
// four row results through readlane. Every lane returns the same value.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false));  // row_half_mirror
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false));  // row_mirror
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return max(max(a, b), max(c, d));
}

// Selection by rounds (few experts per lane): a round takes the largest
// remaining key and, among equal keys, the lowest expert: a wave maximum of
// the keys, then the first lane, in expert order, whose remaining key equals
// it (one compare-ballot per slot, lowest slot winning: expert l + 64 j
// grows with j before l). A pick's key becomes 0 and its lane leaves the
// slot's `open` mask, so the maximum needs no mask (every key is >= 0) and a
// later round whose maximum is 0 still skips it. kv[] (0 past E) is
// consumed.
template <int kPer>
__device__ __forceinline__ void pick_by_rounds(uint32_t (&kv)[kPer], const float (&score)[kPer], int E, int k,
                                               int lane, int& id, float& s_mine, float& total) {
  uint64_t open[kPer];  // lanes whose slot j holds an expert not yet picked
#pragma unroll
  for (int j = 0; j < kPer; ++j) open[j] = __ballot(lane + kWave * j < E);
  total = 0.f;
  id = 0;
  s_mine = 0.f;
  for (int r = 0; r < k; ++r) {
    uint32_t m = kv[0];
#pragma unroll
    for (int j = 1; j < kPer; ++j) m = max(m, kv[j]);
    m = wave_max_u32(m);
    int winner = 0;
#pragma unroll
    for (int j = kPer - 1; j >= 0; --j) {  // the lowest slot with a hit is kept
      const uint64_t hit = __ballot(kv[j] == m) & open[j];
      winner = hit ? kWave * j + (int)__builtin_ctzll(hit) : winner;
    }
    const int owner = winner & (kWave - 1), slot = winner / kWave;
    float s_slot = 0.f;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      if (j == slot) {
        s_slot = score[j];
        open[j] &= ~(1ull << owner);
        if (lane == owner) kv[j] = 0;
      }
    }
    const float s = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s_slot), owner));
    total = total + s;
    if (lane == r) {
      id = winner;
      s_mine = s;
    }
  }
}

// Wave-wide minimum of a uint32, as wave_max_u32.
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  v = min(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  v = min(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false));  // row_half_mirror
  v = min(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false));  // row_mirror
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return min(min(a, b), min(c, d));
}

// Selection by a threshold (8 or more experts per lane), the same picks in
// the same order:
// 1. A threshold T: the largest value that at least k keys reach, found one
//    bit at a time (T | bit is kept while at least k keys reach it: a ballot
//    and a popcount per slot, the compares issued before the counts). It
//    lies between L, the smallest of the lanes' largest keys (at least
//    min(E, 64) >= k keys reach L), and the largest key, so the search
//    starts below their common leading bits. It stops as soon as exactly k
//    keys reach T: those are the picks. Slots past E hold key 0, which no
//    candidate (>= 1) counts; the selection below also checks the expert
//    index.
// 2. If it ran through all bits with more than k keys at T, T is the k-th
//    largest key: every key above T is a pick, and the lowest experts with
//    key T make up the rest (experts ascend with the slot, then the lane).
// 3. The picks go to lanes 0..k-1 in expert order: for each slot holding
//    picks, one lane permute (a push) per value to lane (picks of earlier
//    slots + picks of the slot in lower lanes); the other lanes push to
//    lane 63, which no pick uses (k <= 32).
// 4. Each of those lanes counts the picks before its own, an earlier pick
//    having the larger key or the same key and the lower expert; the ranks
//    are a permutation of 0..k-1, and one more push puts pick r in lane r.
// Lane reads come eight at a time, ahead of their use. Measured on MI355X,
// one wave alone (shader clock): 3,500 against 4,150 cycles for the rounds
// at 4 experts per lane and 8 picks, 4,250 against 4,550 at 8 per lane and
// 6 picks, 8,100 against 19,500 at 16 per lane and 16 picks. In the routing
// kernel, where quantising waves share the SIMD, 4 per lane came out
// 0.1-0.2 us slower than the rounds and stays with them; 896 experts top-16
// at 64 tokens took 14.7 us against 18.1.
template <int kPer>
__device__ __forceinline__ void pick_by_threshold(const uint32_t (&kv)[kPer], const float (&score)[kPer], int E, int k,
                                                  int lane, int& id, float& s_mine, float& total) {
  static_assert(kMaxTopK < kWave, "lane 63 takes the pushes of lanes without a pick");
  uint32_t T = 0;
  int n_ge = -1;  // keys reaching T, once a candidate has been kept
  int b = -1;     // the next bit to try
  {
    uint32_t lmax = kv[0];
#pragma unroll
    for (int j = 1; j < kPer; ++j) lmax = max(lmax, kv[j]);
    const uint32_t hi = wave_max_u32(lmax);
    const uint32_t lo = wave_min_u32(lane < E ? lmax : 0xFFFFFFFFu);
    const uint32_t d = hi ^ lo;
    if (d == 0) {
      T = hi;  // k or more lanes share the largest key: T is the k-th key
    } else {
      b = 31 - __builtin_clz(d);
      T = b == 31 ? 0u : (hi & ~((2u << b) - 1u));
    }
  }
  for (; b >= 0 && n_ge != k; --b) {
    const uint32_t c = T | (1u << b);
    uint64_t bal[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) bal[j] = __ballot(kv[j] >= c);
    int n = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) n += __popcll(bal[j]);
    __builtin_amdgcn_sched_group_barrier(0x002, kPer, 0);      // the compares (VALU) first,
    __builtin_amdgcn_sched_group_barrier(0x004, 4 * kPer, 0);  // then the counts (SALU)
    if (n >= k) {
      T = c;
      n_ge = n;
    }
  }

  uint64_t sel[kPer];
  if (n_ge == k) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) sel[j] = __ballot(lane + kWave * j < E && kv[j] >= T);
  } else {
    int need = k;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      sel[j] = __ballot(lane + kWave * j < E && kv[j] > T);
      need -= __popcll(sel[j]);
    }
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      uint64_t tie = __ballot(lane + kWave * j < E && kv[j] == T);
      for (; need > 0 && tie != 0; --need) {
        const uint64_t low = tie & (~tie + 1ull);
        sel[j] |= low;
        tie ^= low;
      }
    }
  }

  int pk = 0, pe = 0, ps = 0;  // lanes below k: key, expert and score bits of a pick
  int base = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const uint64_t m = sel[j];
    if (m != 0) {
      const int cnt = __popcll(m);
      const int below = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      const int to = (((m >> lane) & 1ull) ? base + below : kWave - 1) * 4;
      const int rk = __builtin_amdgcn_ds_permute(to, (int)kv[j]);
      const int rs = __builtin_amdgcn_ds_permute(to, __float_as_int(score[j]));
      const int re = __builtin_amdgcn_ds_permute(to, lane + kWave * j);
      const bool here = lane >= base && lane < base + cnt;
      pk = here ? rk : pk;
      ps = here ? rs : ps;
      pe = here ? re : pe;
      base += cnt;
    }
  }

  const uint64_t mine = ((uint64_t)(uint32_t)pk << 32) | (uint32_t)~pe;
  const int npe = ~pe;
  int rank = 0;
  for (int q0 = 0; q0 < k; q0 += 8) {
    uint64_t other[8];
#pragma unroll
    for (int q = 0; q < 8; ++q)
      other[q] = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(pk, q0 + q) << 32) |
                 (uint32_t)__builtin_amdgcn_readlane(npe, q0 + q);
#pragma unroll
    for (int q = 0; q < 8; ++q) rank += (q0 + q < k && other[q] > mine) ? 1 : 0;
  }
  const int to = (lane < k ? rank : lane) * 4;
  id = __builtin_amdgcn_ds_permute(to, pe);
  s_mine = __int_as_float(__builtin_amdgcn_ds_permute(to, ps));
  total = 0.f;
  for (int r0 = 0; r0 < k; r0 += 8) {
    float v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s_mine), r0 + q));
#pragma unroll
    for (int q = 0; q < 8; ++q) total = r0 + q < k ? total + v[q] : total;
  }
}

// One wave: the k picks of a token (k <= E, k <= 64). Lane l holds experts
// l + 64 j (j < kPer, e < E): key[j] (the ordered image of score + bias)
// and score[j]. The picks are the k largest keys, equal keys ordered by
// expert (lower first), and come out in that order. Lane r < k returns the
// r-th pick and its score, the other lanes 0 and 0; every lane returns the
// FP32 sum of the picked scores taken in pick order.
template <int kPer>
__device__ __forceinline__ void pick_top_k(const uint32_t (&key)[kPer], const float (&score)[kPer], int E, int k,
                                           int lane, int& id, float& s_mine, float& total) {
  uint32_t kv[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) kv[j] = lane + kWave * j < E ? key[j] : 0u;
  if constexpr (kPer >= 8)
    pick_by_threshold<kPer>(kv, score, E, k, lane, id, s_mine, total);
  else
    pick_by_rounds<kPer>(kv, score, E, k, lane, id, s_mine, total);
}

// Routing weight of a pick: its score over the picks' total, times the
// routed scale.
__device__ __forceinline__ float pick_weight(float s, float total, float routed_scale) {
  return (s / total) * routed_scale;
}

// Sixteen BF16 values (two 16-byte words, low half first) as floats.
__device__ __forceinline__ void bf16x16_values(const u32x4_t& lo, const u32x4_t& hi, float (&v)[16]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_value(lo[i] & 0xFFFFu);
    v[2 * i + 1] = bf16_value(lo[i] >> 16);
    v[8 + 2 * i] = bf16_value(hi[i] & 0xFFFFu);
    v[8 + 2 * i + 1] = bf16_value(hi[i] >> 16);
  }
}

// Absolute maximum of a 128-value block held by eight aligned lanes (16
// values each), floored at 1e-10; every lane of the eight returns it.
__device__ __forceinline__ float block_amax8(const float (&v)[16]) {
  float amax = kAmaxFloor;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
  return group_max<8>(amax);
}

// The block's FP8 scale from its absolute maximum: amax / 448, rounded up
// to a power of two when ue8m0 (after flooring at 1e-10); and this lane's
// 16 codes e4m3(v * (1 / scale)).
__device__ __forceinline__ u32x4_t fp8_block_codes(const float (&v)[16], float amax, int ue8m0, float& scale) {
  float s = amax / kFp8Max;
  if (ue8m0) {
    const uint32_t b = __float_as_uint(fmaxf(s, kAmaxFloor));
    s = __uint_as_float(((b >> 23) + ((b & 0x7FFFFFu) != 0u)) << 23);
  }
  const float inv = 1.0f / s;
  u32x4_t out;
#pragma unroll
  for (int w = 0; w < 4; ++w)
    out[w] = e4m3x4_encode(v[4 * w] * inv, v[4 * w + 1] * inv, v[4 * w + 2] * inv, v[4 * w + 3] * inv);
  scale = s;
  return out;
}

// One wave groups at most 64 routes (ids[r] of route r, global expert ids)
// by local expert (e - lb over [0, lc)), experts ascending, each expert's
// routes in ascending route order, without moving data between lanes. Lane
// r holds route r's local expert e. One ballot per bit of e, from the top
// bit down, narrows two masks per lane: the lanes whose expert equals e so
// far (eq) and those already known to be smaller (lt). Then the route's
// place in (expert, route) order is popc(lt) + popc(eq below the lane), the
// first lane of each expert's run (none of eq below it) writes the bucket,
// and the bucket's index is the number of smaller experts' first lanes.
// Non-local routes take no part. With jr > 0 each run is cut into jobs of
// at most jr routes. `out` may point to LDS or to device memory.
__device__ __forceinline__ void bucket_routes_wave(const Buckets& out, const int* ids, int R, int lb, int lc, int jr,
                                                   int lane) {
  const int e = lane < R ? ids[lane] - lb : -1;
  const bool mine = e >= 0 && e < lc;
  const uint64_t below = (1ull << lane) - 1ull;
  uint64_t eq = __ballot(mine), lt = 0;
  const int bits = 32 - __builtin_clz((unsigned)max(lc - 1, 1));
  for (int b = bits - 1; b >= 0; --b) {
    const bool one = mine && ((e >> b) & 1);
    const uint64_t ones = __ballot(one);
    lt |= one ? eq & ~ones : 0ull;
    eq &= one ? ones : ~ones;
  }
  const int pos = __popcll(eq & below);  // place in the expert's run
  const int off = __popcll(lt);          // routes of smaller experts
  const int cnt = __popcll(eq);
  const bool first = mine && pos == 0;
  const uint64_t starts = __ballot(first);
  if (mine) out.routes[off + pos] = lane;
  if (first) {
    const int u = __popcll(starts & lt);
    out.uexp[u] = e;
    out.uoff[u] = off;
    out.ucnt[u] = cnt;
  }
  if (lane == 0) out.ctrl[1] = __popcll(starts);
  if (jr > 0) {
    // a run's first job is the sum of the smaller experts' job counts, taken
    // one bit of the counts at a time (a count is at most 64)
    const int nj = (cnt + jr - 1) / jr;
    int jb = 0, total = 0;
#pragma unroll
    for (int b = 0; b < 7; ++b) {
      const uint64_t has = __ballot(first && ((nj >> b) & 1));
      jb += __popcll(has & lt) << b;
      total += __popcll(has) << b;
    }
    if (mine) {
      out.rjob[lane] = jb + pos / jr;
      if (pos % jr == 0) out.jobs[jb + pos / jr] = make_int4(e, off + pos, min(jr, cnt - pos), 0);
    }
    if (lane == 0) out.ctrl[2] = total;
  }
}

}  // namespace moe
