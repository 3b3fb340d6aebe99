// Top-k + softmax of one token's router logits by one wave, without
// barriers (shared by the single-token and the batched paths).
#pragma once

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

// Batched top-k workgroups are kTopkBlock threads; thread t holds the logits
// of experts kTopkPerThread t .. kTopkPerThread t + kTopkPerThread - 1 while
// it sums the router's partial results.
constexpr int kTopkBlock = 256;
constexpr int kTopkPerThread = kMaxExperts / kTopkBlock;  // keys per thread

struct TopkLds {
  alignas(16) uint64_t cand[2 * kWave];  // candidates; the upper half takes discarded stores
};

// Sum over the 64 lanes by DPP within rows, then the four row sums (the same
// order in every wave, so every workgroup gets the same weights).
__device__ __forceinline__ float wave_sum_rows(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

// Top-k + softmax by ONE wave, without barriers (E <= 1024, k <= 32).  Lane l
// holds experts 16 l .. 16 l + 15 as order-preserving keys (key[m], 0 for an
// absent expert); the selection orders experts by larger logit first, then
// lower index among equal logits.
//  1. T = the k-th largest of the 64 lane maxima (0 when fewer than k lanes
//     hold experts), found bit by bit from the top: a bit stays set when at
//     least k lane maxima are >= the prefix with it (one ballot and one
//     population count per bit, no LDS).  At least k keys are >= T, so every
//     selected key is.
//  2. The present keys >= T (C of them, C >= k; about k + 3 for random
//     logits) are compacted into S.cand as 64-bit composites key << 32 |
//     ~index, which order the experts exactly as the selection does (a
//     larger composite ranks first; composites are distinct).  Entries C ..
//     63 are zero, below every candidate.
//  3. Candidate j (lane j) counts the composites above its own: its rank
//     (the candidates are read from LDS in batches of 32 before any compare,
//     so the reads overlap).  Ranks below k are the selection, written in
//     that order with their softmax weights.
// Returns false, writing nothing, when C > 64 (only with many equal logits
// at the threshold, or E > 64 with fewer than k lanes holding experts); the
// caller then runs topk_softmax_wave_rounds.
__device__ inline bool topk_softmax_wave(const uint32_t (&key)[16], int E, int k, TopkLds& S,
                                         int32_t* idx, float* wts, int32_t* idx_out, float* w_out) {
  const int lane = threadIdx.x & 63;
  const int base = lane * 16;
  // 1. threshold
  uint32_t lm = 0u;
#pragma unroll
  for (int m = 0; m < 16; ++m) lm = umax32(lm, key[m]);
  uint32_t T = 0u;
#pragma unroll
  for (int b = 31; b >= 0; --b) {
    const uint32_t c = T | (1u << b);
    T = __builtin_popcountll(__ballot(lm >= c)) >= k ? c : T;
  }
  // 2. compaction (every lane stores 16 times; non-candidates into the upper half)
  bool take[16];
  uint32_t cnt = 0u;
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    take[m] = base + m < E && key[m] >= T;
    cnt += take[m] ? 1u : 0u;
  }
  const uint32_t incl = wave_incl_scan_u32(cnt);
  const int C = __builtin_amdgcn_readlane((int)incl, kWave - 1);
  if (C > kWave) return false;
  uint32_t pos = incl - cnt;
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    const uint32_t p = take[m] ? pos : (uint32_t)(kWave + lane);
    S.cand[p] = ((uint64_t)key[m] << 32) | (uint64_t)(~(uint32_t)(base + m));
    pos += take[m] ? 1u : 0u;
  }
  if (lane >= C) S.cand[lane] = 0ull;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  // 3. ranks
  const uint64_t mine = S.cand[lane];
  uint32_t rk[4] = {0u, 0u, 0u, 0u};
  for (int h = 0; h < (C <= kWave / 2 ? kWave / 2 : kWave); h += kWave / 2) {
    uint64_t v[kWave / 2];
#pragma unroll
    for (int j = 0; j < kWave / 2; ++j) v[j] = S.cand[h + j];
    __builtin_amdgcn_sched_barrier(0);  // every read issued before the compares
#pragma unroll
    for (int j = 0; j < kWave / 2; ++j) rk[j & 3] += v[j] > mine ? 1u : 0u;
  }
  const int r = (int)((rk[0] + rk[1]) + (rk[2] + rk[3]));
  const bool sel = lane < C && r < k;
  const uint32_t ck = (uint32_t)(mine >> 32);
  const int ci = (int)~(uint32_t)mine;
  const uint64_t first = __ballot(sel && r == 0);  // exactly one lane: the largest logit
  const uint32_t top = (uint32_t)__builtin_amdgcn_readlane((int)ck, (int)__builtin_ctzll(first));
  const float ex = sel ? expf(f32_from_order_key(ck) - f32_from_order_key(top)) : 0.f;
  const float sum = wave_sum_rows(ex);
  if (sel) {
    const float w = ex / sum;
    idx[r] = ci;
    wts[r] = w;
    if (idx_out) idx_out[r] = ci;
    if (w_out) w_out[r] = w;
  }
  return true;
}

// The same selection by k rounds of a wave argmax over (key, lower index):
// exact for any logits (ties included), slower (about 70 instructions a
// round); the fallback when topk_softmax_wave declines.
__device__ inline void topk_softmax_wave_rounds(uint32_t (&key)[16], int E, int k, int32_t* idx,
                                                float* wts, int32_t* idx_out, float* w_out) {
  const int lane = threadIdx.x & 63;
  const int base = lane * 16;
#pragma unroll
  for (int m = 0; m < 16; ++m)
    if (base + m >= E) key[m] = 0u;
  uint32_t sk = 0u;  // this lane's pick of round r (lane r keeps round r's)
  int si = 0;
  for (int r = 0; r < k; ++r) {
    // lane best: the largest key, the lowest index among equals
    uint32_t bk = 0u;
    int bm = 0;
#pragma unroll
    for (int m = 0; m < 16; ++m)
      if (key[m] > bk) {
        bk = key[m];
        bm = m;
      }
    const uint32_t K = wave_max_u32(bk);
    const uint64_t has = __ballot(bk == K);
    const int wl = (int)__builtin_ctzll(has);  // lowest lane: lowest index
    const int wm = __builtin_amdgcn_readlane(bm, wl);
    if (lane == r) {
      sk = K;
      si = wl * 16 + wm;
    }
    if (lane == wl) {
#pragma unroll
      for (int m = 0; m < 16; ++m)
        if (m == wm) key[m] = 0u;
    }
  }
  const bool sel = lane < k;
  const uint32_t top = (uint32_t)__builtin_amdgcn_readlane((int)sk, 0);
  const float ex = sel ? expf(f32_from_order_key(sk) - f32_from_order_key(top)) : 0.f;
  const float sum = wave_sum(ex);
  if (sel) {
    const float w = ex / sum;
    idx[lane] = si;
    wts[lane] = w;
    if (idx_out) idx_out[lane] = si;
    if (w_out) w_out[lane] = w;
  }
}

}  // namespace moe
