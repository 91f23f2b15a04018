// Small-batch decode path: routing + plan, gate_up, down (T <= 64).
//
// Output-centric, after the warp-decode design (warp-decode article, "Key
// points"): the gate_up kernel gives each workgroup 16 neurons (16 gate rows
// and the matching 16 up rows) of one routed expert and every token routed to
// it; the down kernel gives each workgroup 16 output dimensions and sums every
// routed expert's contribution into FP32 accumulators directly, so there is
// neither a per-expert output buffer nor an activation-gather buffer.
//
// On gfx950 the dot products run on MFMA (v_mfma_f32_16x16x32_bf16): a wave
// multiplies 16 weight rows by up to 16 tokens per instruction, so one pass
// over a weight row serves every token routed to that expert at no extra
// HBM traffic.  The eight waves of a workgroup split the reduction dimension
// and their partial sums are added in LDS in a fixed wave order.
//
// The activation handed from gate_up to down is w_j * silu(g) * u in FP32,
// stored as an exact-sum pair of BF16 values (hi = rne(v), lo = rne(v - hi)),
// so the down projection's MFMA sees ~16 significant bits of the FP32 value
// rather than BF16's 8; the FP32 accumulation is untouched.  Pre-multiplying
// by the routing weight lets all routed experts of a token accumulate into
// one MFMA accumulator.
//
// Determinism: expert order (ascending id), token order, the MFMA sequence
// and the cross-wave sum order are all fixed; nothing accumulates through
// atomics (the only atomic is an integer OR that builds expert token masks).
#include "common.h"
#include "internal.h"
#include "route.h"

namespace moe {

namespace {
constexpr int kDecWaves = 8;          // waves per workgroup (split of K)
constexpr int kDecThreads = kDecWaves * kWave;
constexpr int kDownChunk = 4;         // K-steps per batch in down

inline size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }
}  // namespace

DecodeWs decode_ws_layout(int T, int H, int I, int E, int k) {
  DecodeWs L{};
  size_t o = 0;
  const size_t pairs = static_cast<size_t>(T) * k;
  (void)H;
  L.plan_u = o;      o += 256;
  L.plan_e = o;      o = align256(o + sizeof(int32_t) * E);
  L.plan_mask = o;   o = align256(o + sizeof(uint64_t) * E);
  L.idx = o;         o = align256(o + sizeof(int32_t) * pairs);
  L.w = o;           o = align256(o + sizeof(float) * pairs);
  L.hw_hi = o;       o = align256(o + 2 * pairs * I);
  L.hw_lo = o;       o = align256(o + 2 * pairs * I);
  L.total = o;
  return L;
}

// One workgroup: route every token, then list the touched experts in
// ascending order with a 64-bit mask of the tokens routed to each.
__global__ __launch_bounds__(1024) void decode_route_plan(
    const float* __restrict__ logits, int T, int E, int k, int32_t* __restrict__ idx,
    float* __restrict__ wts, int* __restrict__ plan_u, int32_t* __restrict__ plan_e,
    uint64_t* __restrict__ plan_mask) {
  extern __shared__ uint64_t dyn_masks[];          // [E] token masks, then chunk counts
  __shared__ int s_idx[64 * 32];
  const int nchunks = (E + kWave - 1) / kWave;
  int* chunk_off = reinterpret_cast<int*>(dyn_masks + E);
  const int nw = blockDim.x / kWave, wv = wave_id(), lane = lane_id();

  for (int t = wv; t < T; t += nw) {
    int e;
    float wt;
    route_token_any(logits + static_cast<size_t>(t) * E, E, k, &e, &wt);
    if (lane < k) {
      idx[t * k + lane] = e;
      wts[t * k + lane] = wt;
      s_idx[t * k + lane] = e;
    }
  }
  for (int i = threadIdx.x; i < E; i += blockDim.x) dyn_masks[i] = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < T * k; i += blockDim.x)
    atomicOr(reinterpret_cast<unsigned long long*>(&dyn_masks[s_idx[i]]), 1ull << (i / k));
  __syncthreads();
  for (int c = wv; c < nchunks; c += nw) {
    const int e = c * kWave + lane;
    const uint64_t on = __ballot(e < E && dyn_masks[e] != 0);
    if (lane == 0) chunk_off[c] = __popcll(on);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int s = 0;
    for (int c = 0; c < nchunks; ++c) {
      const int v = chunk_off[c];
      chunk_off[c] = s;
      s += v;
    }
    *plan_u = s;
  }
  __syncthreads();
  for (int c = wv; c < nchunks; c += nw) {
    const int e = c * kWave + lane;
    const bool on = e < E && dyn_masks[e] != 0;
    const uint64_t b = __ballot(on);
    if (on) {
      const int r = chunk_off[c] + __popcll(b & ((1ull << lane) - 1));
      plan_e[r] = e;
      plan_mask[r] = dyn_masks[e];
    }
  }
}

// gate_up: work item = (touched expert u, block of 16 neurons).  Workgroups
// stride over items.  Wave wv covers K range [wv*H/8, (wv+1)*H/8).
// TM = token tiles of 16 the batch needs (1, 2 or 4); KC = K-steps whose
// weights are loaded per batch.
template <int TM, int KC>
__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(4, 8))) void decode_gate_up(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wgu,
    const int32_t* __restrict__ idx, const float* __restrict__ wts,
    const int* __restrict__ plan_u, const int32_t* __restrict__ plan_e,
    const uint64_t* __restrict__ plan_mask, int H, int I, int k,
    uint16_t* __restrict__ hw_hi, uint16_t* __restrict__ hw_lo) {
  extern __shared__ float red[];                    // [8 waves][TM][gate/up][4][64]
  __shared__ int tok_list[64];
  const int U = *plan_u;
  const int nrb = I / 16;
  const int items = U * nrb;
  const int wv = wave_id(), ln = lane_id();
  const int col = ln & 15, grp = ln >> 4;
  const int kw = H / kDecWaves;
  const int ksteps = kw / 32;
  const size_t kb = static_cast<size_t>(wv) * kw + grp * 8;
  const bf16x8 zero8 = {};

  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    const int u = item / nrb, rb = item - u * nrb;
    const int e = plan_e[u];
    const uint64_t mask = plan_mask[u];
    const int ntok = __popcll(mask);
    const int tiles = (ntok + 15) >> 4;
    if (wv == 0 && ((mask >> ln) & 1ull)) tok_list[__popcll(mask & ((1ull << ln) - 1))] = ln;
    __syncthreads();
    int tok[TM];
#pragma unroll
    for (int c = 0; c < TM; ++c) {
      const int p = 16 * c + col;
      tok[c] = p < ntok ? tok_list[p] : -1;
    }
    const uint16_t* pg = wgu + (static_cast<size_t>(e) * 2 * I + rb * 16 + col) * H + kb;
    const uint16_t* pu = pg + static_cast<size_t>(I) * H;
    f32x4 ag[TM], au[TM];
#pragma unroll
    for (int c = 0; c < TM; ++c) ag[c] = au[c] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int s0 = 0; s0 < ksteps; s0 += KC) {
      bf16x8 wg[KC], wu[KC];
#pragma unroll
      for (int s = 0; s < KC; ++s) {
        if (s0 + s < ksteps) {
          wg[s] = as_bf16x8(ld16(pg + (s0 + s) * 32));
          wu[s] = as_bf16x8(ld16(pu + (s0 + s) * 32));
        }
      }
#pragma unroll
      for (int c = 0; c < TM; ++c) {
        if (c < tiles) {
          bf16x8 xb[KC];
#pragma unroll
          for (int s = 0; s < KC; ++s)
            xb[s] = (tok[c] >= 0 && s0 + s < ksteps)
                        ? as_bf16x8(ld16(x + static_cast<size_t>(tok[c]) * H + kb + (s0 + s) * 32))
                        : zero8;
#pragma unroll
          for (int s = 0; s < KC; ++s) {
            if (s0 + s < ksteps) {
              ag[c] = mfma16x16x32(wg[s], xb[s], ag[c]);
              au[c] = mfma16x16x32(wu[s], xb[s], au[c]);
            }
          }
        }
      }
    }
#pragma unroll
    for (int c = 0; c < TM; ++c) {
      if (c < tiles) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          red[(((wv * TM + c) * 2 + 0) * 4 + r) * 64 + ln] = ag[c][r];
          red[(((wv * TM + c) * 2 + 1) * 4 + r) * 64 + ln] = au[c][r];
        }
      }
    }
    __syncthreads();
    // Fixed-order sum over waves, SwiGLU, weight, split, store.
    for (int q = threadIdx.x; q < tiles * 256; q += blockDim.x) {
      const int c = q >> 8, within = q & 255;
      const int n = within >> 4, m = within & 15;    // token column n, weight row m
      const int src = 16 * (m >> 2) + n, r = m & 3;
      float g = 0.f, up = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < kDecWaves; ++w2) {
        g += red[(((w2 * TM + c) * 2 + 0) * 4 + r) * 64 + src];
        up += red[(((w2 * TM + c) * 2 + 1) * 4 + r) * 64 + src];
      }
      const int p = c * 16 + n;
      if (p < ntok) {
        const int t = tok_list[p];
        int j = 0;
        while (j < k - 1 && idx[t * k + j] != e) ++j;
        const float hv = wts[t * k + j] * swiglu(g, up);
        const uint32_t hi = f32_to_bf16_rne(hv);
        const uint32_t lo = f32_to_bf16_rne(hv - bf16_to_f32(hi));
        const size_t o = static_cast<size_t>(t * k + j) * I + rb * 16 + m;
        hw_hi[o] = static_cast<uint16_t>(hi);
        hw_lo[o] = static_cast<uint16_t>(lo);
      }
    }
    __syncthreads();
  }
}

// down: workgroup = 8 output dimensions d0..d0+7 of every touched expert (H/8
// workgroups, enough to occupy every CU without splitting the expert sum
// across workgroups).  MFMA rows 0..7 carry those dimensions; lanes of rows
// 8..15 issue no loads (the MFMA work they waste is free: the kernel is bound
// by HBM).  Wave wv covers K range [wv*I/8, (wv+1)*I/8) of each touched expert
// in ascending expert order, loading the weights of UE experts ahead of their
// MFMAs; the eight wave partials are then added in LDS in wave order.
constexpr int kDownRows = 8;

template <int TM>
__device__ __forceinline__ void down_expert(const bf16x8 (&a)[kDownChunk], int s0, int ksteps,
                                            int e, uint64_t mask, int k, int col,
                                            const int* s_idx, size_t kb, int I,
                                            const uint16_t* __restrict__ hw_hi,
                                            const uint16_t* __restrict__ hw_lo, f32x4 (&acc)[TM]) {
  const bf16x8 zero8 = {};
#pragma unroll
  for (int c = 0; c < TM; ++c) {
    const uint32_t bits = static_cast<uint32_t>(mask >> (16 * c)) & 0xFFFFu;
    if (bits == 0) continue;
    const int t = 16 * c + col;
    const bool routed = (bits >> col) & 1u;
    size_t row = 0;
    if (routed) {
      int j = 0;
      while (j < k - 1 && s_idx[t * k + j] != e) ++j;
      row = static_cast<size_t>(t * k + j) * I + kb;
    }
    bf16x8 bh[kDownChunk], bl[kDownChunk];
#pragma unroll
    for (int s = 0; s < kDownChunk; ++s) {
      const bool ok = routed && s0 + s < ksteps;
      bh[s] = ok ? as_bf16x8(ld16(hw_hi + row + (s0 + s) * 32)) : zero8;
      bl[s] = ok ? as_bf16x8(ld16(hw_lo + row + (s0 + s) * 32)) : zero8;
    }
#pragma unroll
    for (int s = 0; s < kDownChunk; ++s) {
      if (s0 + s < ksteps) {
        acc[c] = mfma16x16x32(a[s], bh[s], acc[c]);
        acc[c] = mfma16x16x32(a[s], bl[s], acc[c]);
      }
    }
  }
}

template <int TM, int UE>
__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(4, 8))) void decode_down(
    const uint16_t* __restrict__ wd, const int32_t* __restrict__ idx,
    const int* __restrict__ plan_u, const int32_t* __restrict__ plan_e,
    const uint64_t* __restrict__ plan_mask, const uint16_t* __restrict__ hw_hi,
    const uint16_t* __restrict__ hw_lo, int T, int H, int I, int k, uint16_t* __restrict__ out) {
  extern __shared__ float red[];                    // [8 waves][TM][4][64]
  __shared__ int s_idx[64 * 32];
  for (int i = threadIdx.x; i < T * k; i += blockDim.x) s_idx[i] = idx[i];
  __syncthreads();
  const int U = *plan_u;
  const int wv = wave_id(), ln = lane_id();
  const int col = ln & 15, grp = ln >> 4;
  const bool row_lane = col < kDownRows;
  const int d0 = blockIdx.x * kDownRows;
  const int kw = I / kDecWaves;
  const int ksteps = kw / 32;
  const size_t kb = static_cast<size_t>(wv) * kw + grp * 8;
  const uint16_t* pw = wd + (static_cast<size_t>(d0) + (row_lane ? col : 0)) * I + kb;
  const bf16x8 zero8 = {};
  f32x4 acc[TM];
#pragma unroll
  for (int c = 0; c < TM; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int ub = 0; ub < U; ub += UE) {
    int e[UE];
    uint64_t m[UE];
#pragma unroll
    for (int q = 0; q < UE; ++q) {
      const bool have = ub + q < U;
      e[q] = have ? plan_e[ub + q] : 0;
      m[q] = have ? plan_mask[ub + q] : 0ull;
    }
    for (int s0 = 0; s0 < ksteps; s0 += kDownChunk) {
      bf16x8 a[UE][kDownChunk];
#pragma unroll
      for (int q = 0; q < UE; ++q)
#pragma unroll
        for (int s = 0; s < kDownChunk; ++s)
          a[q][s] = (m[q] != 0 && row_lane && s0 + s < ksteps)
                        ? as_bf16x8(ld16(pw + static_cast<size_t>(e[q]) * H * I + (s0 + s) * 32))
                        : zero8;
#pragma unroll
      for (int q = 0; q < UE; ++q)
        if (m[q] != 0)
          down_expert<TM>(a[q], s0, ksteps, e[q], m[q], k, col, s_idx, kb, I, hw_hi, hw_lo, acc);
    }
  }
  // D rows 0..7 live in lanes with grp < 2
#pragma unroll
  for (int c = 0; c < TM; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[((wv * TM + c) * 4 + r) * 64 + ln] = acc[c][r];
  __syncthreads();
  for (int q = threadIdx.x; q < TM * 16 * kDownRows; q += blockDim.x) {
    const int c = q / (16 * kDownRows), within = q % (16 * kDownRows);
    const int n = within / kDownRows, mm = within % kDownRows;   // token column n, output row mm
    const int src = 16 * (mm >> 2) + n, r = mm & 3;
    float v = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < kDecWaves; ++w2) v += red[((w2 * TM + c) * 4 + r) * 64 + src];
    const int t = 16 * c + n;
    if (t < T) out[static_cast<size_t>(t) * H + d0 + mm] = static_cast<uint16_t>(f32_to_bf16_rne(v));
  }
}

hipError_t launch_decode(const uint16_t* x, const float* logits, const uint16_t* wgu,
                         const uint16_t* wd, int T, int H, int I, int E, int k, uint16_t* out,
                         int32_t* idx, float* w, void* ws, hipStream_t s, int num_cus) {
  const DecodeWs L = decode_ws_layout(T, H, I, E, k);
  char* base = static_cast<char*>(ws);
  int* plan_u = reinterpret_cast<int*>(base + L.plan_u);
  int32_t* plan_e = reinterpret_cast<int32_t*>(base + L.plan_e);
  uint64_t* plan_mask = reinterpret_cast<uint64_t*>(base + L.plan_mask);
  int32_t* idx_p = idx ? idx : reinterpret_cast<int32_t*>(base + L.idx);
  float* w_p = w ? w : reinterpret_cast<float*>(base + L.w);
  uint16_t* hw_hi = reinterpret_cast<uint16_t*>(base + L.hw_hi);
  uint16_t* hw_lo = reinterpret_cast<uint16_t*>(base + L.hw_lo);

  const int nchunks = (E + kWave - 1) / kWave;
  const size_t lds_plan = sizeof(uint64_t) * E + sizeof(int) * nchunks;
  prof_begin(kRoute, s);
  hipLaunchKernelGGL(decode_route_plan, dim3(1), dim3(1024), lds_plan, s, logits, T, E, k, idx_p,
                     w_p, plan_u, plan_e, plan_mask);
  prof_end(kRoute, s);

  const int TM = T <= 16 ? 1 : (T <= 32 ? 2 : 4);   // token tiles the kernels carry
  const long items_upper = static_cast<long>(T * k < E ? T * k : E) * (I / 16);
  const long grid_cap = 2L * num_cus;
  const int grid1 = static_cast<int>(items_upper < grid_cap ? items_upper : grid_cap);
  const size_t lds_gu = sizeof(float) * kDecWaves * TM * 2 * 256;
  const size_t lds_dn = sizeof(float) * kDecWaves * TM * 256;
  const dim3 grid2(H / kDownRows);
  prof_begin(kDecGateUp, s);
  if (TM == 1)
    hipLaunchKernelGGL((decode_gate_up<1, 8>), dim3(grid1), dim3(kDecThreads), lds_gu, s, x, wgu,
                       idx_p, w_p, plan_u, plan_e, plan_mask, H, I, k, hw_hi, hw_lo);
  else if (TM == 2)
    hipLaunchKernelGGL((decode_gate_up<2, 4>), dim3(grid1), dim3(kDecThreads), lds_gu, s, x, wgu,
                       idx_p, w_p, plan_u, plan_e, plan_mask, H, I, k, hw_hi, hw_lo);
  else
    hipLaunchKernelGGL((decode_gate_up<4, 4>), dim3(grid1), dim3(kDecThreads), lds_gu, s, x, wgu,
                       idx_p, w_p, plan_u, plan_e, plan_mask, H, I, k, hw_hi, hw_lo);
  prof_end(kDecGateUp, s);
  prof_begin(kDecDown, s);
  if (TM == 1)
    hipLaunchKernelGGL((decode_down<1, 4>), grid2, dim3(kDecThreads), lds_dn, s, wd, idx_p, plan_u,
                       plan_e, plan_mask, hw_hi, hw_lo, T, H, I, k, out);
  else if (TM == 2)
    hipLaunchKernelGGL((decode_down<2, 2>), grid2, dim3(kDecThreads), lds_dn, s, wd, idx_p, plan_u,
                       plan_e, plan_mask, hw_hi, hw_lo, T, H, I, k, out);
  else
    hipLaunchKernelGGL((decode_down<4, 1>), grid2, dim3(kDecThreads), lds_dn, s, wd, idx_p, plan_u,
                       plan_e, plan_mask, hw_hi, hw_lo, T, H, I, k, out);
  prof_end(kDecDown, s);
  return hipGetLastError();
}

hipError_t decode_set_attributes() {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(decode_gate_up<4, 4>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     sizeof(float) * kDecWaves * 4 * 2 * 256 + 1024);
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(decode_route_plan),
                          hipFuncAttributeMaxDynamicSharedMemorySize,
                          sizeof(uint64_t) * 1024 + sizeof(int) * 16);
  return e;
}

}  // namespace moe
