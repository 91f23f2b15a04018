// Top-k routing of one token by one 64-lane wave.
//
// Expert routing (warp-decode article, "Background"): experts are ordered by
// logit descending, then expert index ascending, and the first k are kept; the weights are the softmax of the k selected logits
// (softmax over all E renormalised over the selection).
//
// Each logit becomes a 64-bit key: high word = FP32 bits mapped to an
// unsigned order (-0 folded onto +0), low word = ~expert, so the largest key
// is the largest logit and, among equal logits, the lowest index.  k rounds
// of a wave-wide max pick the experts in slot order.
#pragma once

#include "common.h"

namespace moe {

__device__ __forceinline__ uint32_t ordered_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) == 0) u = 0;               // -0 and +0 tie
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_to_float(uint32_t key) {
  uint32_t u = (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key;
  return __uint_as_float(u);
}

// One DPP step of a 64-bit max: combine each lane with the lane CTRL names.
template <int CTRL>
__device__ __forceinline__ uint64_t max_dpp(uint64_t v) {
  const uint32_t lo = static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(v)), CTRL, 0xF, 0xF, false));
  const uint32_t hi = static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(v >> 32)), CTRL, 0xF, 0xF, false));
  const uint64_t o = (static_cast<uint64_t>(hi) << 32) | lo;
  return o > v ? o : v;
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int lane) {
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v)), lane);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v >> 32)), lane);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Wave-wide max of a 64-bit key, returned to every lane.  Within each row of
// 16 lanes: quad swaps (xor 1, xor 2), then half-row and row mirrors; the four
// row maxima are then read into scalar registers and combined.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = max_dpp<0xB1>(v);    // quad_perm [1,0,3,2]
  v = max_dpp<0x4E>(v);    // quad_perm [2,3,0,1]
  v = max_dpp<0x141>(v);   // row_half_mirror
  v = max_dpp<0x140>(v);   // row_mirror
  uint64_t a = readlane_u64(v, 0), b = readlane_u64(v, 16);
  uint64_t c = readlane_u64(v, 32), d = readlane_u64(v, 48);
  a = a > b ? a : b;
  c = c > d ? c : d;
  return a > c ? a : c;
}

// Routes one token.  `lrow` points at its E logits.  On return lanes j < k hold
// (expert of slot j, weight of slot j); other lanes hold (-1, 0).
// R = candidate logits per lane (E <= 64 * R).
template <int R>
__device__ __forceinline__ void route_token(const float* __restrict__ lrow, int E, int k,
                                            int* out_e, float* out_w) {
  const int lane = lane_id();
  uint64_t keys[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int e = lane + kWave * i;
    keys[i] = e < E ? (static_cast<uint64_t>(ordered_key(lrow[e])) << 32) |
                          static_cast<uint64_t>(0xFFFFFFFFu - static_cast<uint32_t>(e))
                    : 0ull;
  }
  int my_e = -1;
  float my_v = 0.0f;
  for (int r = 0; r < k; ++r) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < R; ++i) best = keys[i] > best ? keys[i] : best;
    best = wave_max_u64(best);
#pragma unroll
    for (int i = 0; i < R; ++i) keys[i] = keys[i] == best ? 0ull : keys[i];   // keys are unique
    if (lane == r) {
      my_e = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(best));
      my_v = key_to_float(static_cast<uint32_t>(best >> 32));
    }
  }
  const float v0 = __shfl(my_v, 0, kWave);
  const float ex = lane < k ? expf(my_v - v0) : 0.0f;
  const float den = wave_sum(ex);
  *out_e = my_e;
  *out_w = lane < k ? ex / den : 0.0f;
}

// Dispatch on the number of candidates per lane (E <= 1024).
__device__ __forceinline__ void route_token_any(const float* __restrict__ lrow, int E, int k,
                                                int* out_e, float* out_w) {
  if (E <= 64) route_token<1>(lrow, E, k, out_e, out_w);
  else if (E <= 128) route_token<2>(lrow, E, k, out_e, out_w);
  else if (E <= 256) route_token<4>(lrow, E, k, out_e, out_w);
  else if (E <= 512) route_token<8>(lrow, E, k, out_e, out_w);
  else route_token<16>(lrow, E, k, out_e, out_w);                  // E <= 1024
}

}  // namespace moe
