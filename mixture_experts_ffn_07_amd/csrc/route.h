// Top-k routing of one token by one 64-lane wave.
//
// Expert routing picks each token's experts (warp-decode article,
// "Background"); the pages give neither the selection rule nor the gate
// function, so both are readings: experts are ordered by FP32 logit
// descending, then expert index ascending, and the first k are kept; the
// weights are the softmax of the k selected logits (softmax over all E
// renormalised over the selection).
//
// Each logit becomes a 32-bit key: its FP32 bits mapped to an unsigned order
// (-0 folded onto +0; every finite logit maps above 0, which marks "taken").
// Each of k rounds takes the wave-wide maximum key (DPP), then the lowest
// expert index holding it (wave ballots, experts lane + 64*i scanned by i
// first), so slots come out by logit descending, index ascending.
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

// One DPP step of a 32-bit max: combine each lane with the lane CTRL names.
template <int CTRL>
__device__ __forceinline__ uint32_t max_dpp_u32(uint32_t v) {
  const uint32_t o = static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), CTRL, 0xF, 0xF, false));
  return o > v ? o : v;
}

// Wave-wide max of a 32-bit key, returned to every lane.  Within each row of
// 16 lanes: quad swaps (xor 1, xor 2), then half-row and row mirrors; the four
// row maxima are then read into scalar registers and combined.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max_dpp_u32<0xB1>(v);    // quad_perm [1,0,3,2]
  v = max_dpp_u32<0x4E>(v);    // quad_perm [2,3,0,1]
  v = max_dpp_u32<0x141>(v);   // row_half_mirror
  v = max_dpp_u32<0x140>(v);   // row_mirror
  const uint32_t a = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 0));
  const uint32_t b = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 16));
  const uint32_t c = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 32));
  const uint32_t d = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 48));
  const uint32_t ab = a > b ? a : b, cd = c > d ? c : d;
  return ab > cd ? ab : cd;
}

// Routes one token from its logits already in registers: lane l holds the
// logits of experts l + 64*i in v[i] (any value where l + 64*i >= E).  On
// return lanes j < k hold (expert of slot j, weight of slot j); other lanes
// hold (-1, 0).  R = candidate logits per lane (E <= 64 * R).
template <int R>
__device__ __forceinline__ void route_token_regs(const float (&v)[R], int E, int k, int* out_e,
                                                 float* out_w) {
  const int lane = lane_id();
  uint32_t keys[R];
#pragma unroll
  for (int i = 0; i < R; ++i) keys[i] = lane + kWave * i < E ? ordered_key(v[i]) : 0u;
  int my_e = -1;
  float my_v = 0.0f;
  for (int r = 0; r < k; ++r) {
    uint32_t best = 0;
#pragma unroll
    for (int i = 0; i < R; ++i) best = keys[i] > best ? keys[i] : best;
    best = wave_max_u32(best);
    // lowest expert holding the maximum: first i with a match, then its lowest lane
    int sel = 0;
#pragma unroll
    for (int i = R - 1; i >= 0; --i) {
      const uint64_t b = __ballot(keys[i] == best);
      sel = b ? kWave * i + __builtin_ctzll(b) : sel;
    }
#pragma unroll
    for (int i = 0; i < R; ++i) keys[i] = (lane + kWave * i == sel) ? 0u : keys[i];
    if (lane == r) {
      my_e = sel;
      my_v = key_to_float(best);
    }
  }
  const float v0 = __shfl(my_v, 0, kWave);
  const float ex = lane < k ? expf(my_v - v0) : 0.0f;
  const float den = wave_sum(ex);
  *out_e = my_e;
  *out_w = lane < k ? ex / den : 0.0f;
}

// Loads the E logits of one token (lane l: experts l + 64*i).
template <int R>
__device__ __forceinline__ void load_logits(const float* __restrict__ lrow, int E, float (&v)[R]) {
  const int lane = lane_id();
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int e = lane + kWave * i;
    v[i] = e < E ? lrow[e] : 0.0f;
  }
}

// Routes one token.  `lrow` points at its E logits.
template <int R>
__device__ __forceinline__ void route_token(const float* __restrict__ lrow, int E, int k,
                                            int* out_e, float* out_w) {
  float v[R];
  load_logits<R>(lrow, E, v);
  route_token_regs<R>(v, E, k, out_e, out_w);
}

// Routes tokens t = t0, t0 + step, ... (at most NT of them, t < T) with one wave:
// every token's logits are loaded before the first is routed, so the load
// latencies overlap.  Lanes j < k of token t write (expert, weight) of slot j to
// idx[t*k + j], w[t*k + j].
template <int R, int NT>
__device__ __forceinline__ void route_tokens_wave(const float* __restrict__ logits, int T, int E,
                                                  int k, int t0, int step, int32_t* idx, float* w) {
  float v[NT][R];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int t = t0 + j * step;
    if (t < T) load_logits<R>(logits + static_cast<size_t>(t) * E, E, v[j]);
  }
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int t = t0 + j * step;
    if (t < T) {
      int e;
      float wt;
      route_token_regs<R>(v[j], E, k, &e, &wt);
      if (lane_id() < k) {
        idx[t * k + lane_id()] = e;
        w[t * k + lane_id()] = wt;
      }
    }
  }
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
