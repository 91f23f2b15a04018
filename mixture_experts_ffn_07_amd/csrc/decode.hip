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
// The activation handed from gate_up to down is w_j * silu(g) * u, computed in
// FP32 and rounded once to BF16 (the MFMA operand type; the batched path does
// the same); the FP32 accumulation is untouched.  Pre-multiplying by the
// routing weight lets all routed experts of a token add into one sum.
//
// Determinism: expert order (ascending id), token order, the MFMA sequence
// and the cross-wave sum order are all fixed; nothing accumulates through
// atomics (the only atomic is an integer OR that builds expert token masks).
#include "common.h"
#include "internal.h"

namespace moe {

namespace {
constexpr int kDecWaves = 8;          // waves per workgroup (split of K)
constexpr int kDecThreads = kDecWaves * kWave;

inline size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }
}  // namespace

DecodeWs decode_ws_layout(int T, int H, int I, int E, int k) {
  DecodeWs L{};
  size_t o = 0;
  const size_t pairs = static_cast<size_t>(T) * k;
  (void)H;
  L.plan_u = o;      o += 256;
  L.plan_e = o;      o = align256(o + sizeof(int32_t) * E);
  L.plan_off = o;    o = align256(o + sizeof(int32_t) * (E + 1));
  L.plan_pr = o;     o = align256(o + sizeof(uint16_t) * pairs);
  L.idx = o;         o = align256(o + sizeof(int32_t) * pairs);
  L.w = o;           o = align256(o + sizeof(float) * pairs);
  L.hw = o;          o = align256(o + 2 * pairs * I);
  L.total = o;
  return L;
}

// Largest plan a workgroup stages in LDS: touched experts <= E <= 1024,
// routed pairs <= T*k <= 64*32.
constexpr int kMaxPlan = 1024;
constexpr int kMaxPairs = 64 * 32;

// Touched-expert plan, built by every gate_up workgroup from the routing
// result (T*k expert ids, L2-resident), in compressed-row form:
//   s_e[u]                  the u-th touched expert, ascending
//   s_pr[s_off[u] .. s_off[u+1])  the pairs p = t*k + j routed to it, tokens ascending
// Returns U.  `masks` (E words) and `scr` (E + 33 ints) are LDS scratch.  The
// 64-bit token masks are built with integer atomics (the result does not
// depend on their order); everything after is ordered compaction and scans.
__device__ int build_plan(const int32_t* __restrict__ idx, int T, int E, int k, uint64_t* masks,
                          int* scr, int* s_e, int* s_off, uint16_t* s_pr) {
  const int nchunks = (E + kWave - 1) / kWave;      // <= 16
  const int nw = blockDim.x / kWave, wv = wave_id(), lane = lane_id();
  int* map = scr;                                   // [E] expert -> plan position
  int* coff = scr + E;                              // [17] chunk offsets, then per-chunk pair sums
  for (int i = threadIdx.x; i < E; i += blockDim.x) masks[i] = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < T * k; i += blockDim.x)
    atomicOr(reinterpret_cast<unsigned long long*>(&masks[idx[i]]), 1ull << (i / k));
  __syncthreads();
  for (int c = wv; c < nchunks; c += nw) {
    const int e = c * kWave + lane;
    const uint64_t on = __ballot(e < E && masks[e] != 0);
    if (lane == 0) coff[c] = __popcll(on);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int sum = 0;
    for (int c = 0; c < nchunks; ++c) {
      const int v = coff[c];
      coff[c] = sum;
      sum += v;
    }
    coff[16] = sum;
  }
  __syncthreads();
  const int U = coff[16];
  // compaction: expert list and map; each chunk's token counts scanned within the wave
  for (int c = wv; c < nchunks; c += nw) {
    const int e = c * kWave + lane;
    const bool on = e < E && masks[e] != 0;
    const uint64_t b = __ballot(on);
    const int cnt = on ? __popcll(masks[e]) : 0;
    int incl = cnt;                                 // inclusive scan of counts over the chunk's lanes
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int v = __shfl_up(incl, d, kWave);
      if (lane >= d) incl += v;
    }
    if (on) {
      const int r = coff[c] + __popcll(b & ((1ull << lane) - 1));
      s_e[r] = e;
      map[e] = r;
      s_off[r + 1] = incl;                          // chunk-local inclusive sum, fixed up below
    }
  }
  __syncthreads();
  // pair totals of the chunks, scanned, added to the chunk-local sums
  if (threadIdx.x == 0) {
    int sum = 0;
    for (int c = 0; c < nchunks; ++c) {
      const int last = (c + 1 < nchunks ? coff[c + 1] : U) - 1;   // last plan slot of chunk c
      const int tot = last >= coff[c] ? s_off[last + 1] : 0;
      scr[E + 17 + c] = sum;                         // (scratch past coff) chunk base
      sum += tot;
    }
    s_off[0] = 0;
  }
  __syncthreads();
  for (int r = threadIdx.x; r < U; r += blockDim.x) {
    // chunk of plan slot r: largest c with coff[c] <= r
    int c = 0;
    while (c + 1 < nchunks && coff[c + 1] <= r) ++c;
    s_off[r + 1] += scr[E + 17 + c];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < T * k; i += blockDim.x) {
    const int e = idx[i], t = i / k;
    const int pos = s_off[map[e]] + __popcll(masks[e] & ((1ull << t) - 1));
    s_pr[pos] = static_cast<uint16_t>(i);
  }
  __syncthreads();
  return U;
}

// gate_up: work item = (touched expert u, block of 16 neurons); workgroups
// stride over items.  Wave wv covers K range [wv*H/8, (wv+1)*H/8) in chunks
// of KC steps of 32 (KC divides the steps).  The workgroup walks its flat
// sequence of (item, chunk) tasks with the weights of the next task loaded
// into a second register buffer while the current one is multiplied, so the
// weight stream never waits on an epilogue.
template <int TM, int KC>
__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(4, 8))) void decode_gate_up(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wgu,
    const int32_t* __restrict__ idx, const float* __restrict__ wts, int T, int E,
    int* __restrict__ plan_u, int32_t* __restrict__ plan_e, int32_t* __restrict__ plan_off,
    uint16_t* __restrict__ plan_pr, int H, int I, int k, uint16_t* __restrict__ hw) {
  extern __shared__ float red[];                    // [8 waves][TM][gate/up][4][64]
  __shared__ int s_e[kMaxPlan];
  __shared__ int s_off[kMaxPlan + 1];
  __shared__ uint16_t s_pr[kMaxPairs];
  // the plan's scratch (E masks, E + 33 ints) borrows the reduction buffer
  const int U = build_plan(idx, T, E, k, reinterpret_cast<uint64_t*>(red),
                           reinterpret_cast<int*>(reinterpret_cast<uint64_t*>(red) + E), s_e,
                           s_off, s_pr);
  if (blockIdx.x == 0) {                            // the plan for the down kernel
    for (int i = threadIdx.x; i < U; i += blockDim.x) {
      plan_e[i] = s_e[i];
      plan_off[i + 1] = s_off[i + 1];
    }
    for (int i = threadIdx.x; i < T * k; i += blockDim.x) plan_pr[i] = s_pr[i];
    if (threadIdx.x == 0) {
      plan_off[0] = 0;
      *plan_u = U;
    }
  }
  const int nrb = I / 16;
  const int items = U * nrb;
  const int wv = wave_id(), ln = lane_id();
  const int col = ln & 15, grp = ln >> 4;
  const int kw = H / kDecWaves;
  const int nch = kw / 32 / KC;                     // chunks per item
  const int my_items = blockIdx.x < items ? (items - 1 - blockIdx.x) / gridDim.x + 1 : 0;
  const int ntask = my_items * nch;
  const uint32_t kb = static_cast<uint32_t>(wv * kw + grp * 8);

  // weight row offset (elements) of task t's gate row for this lane
  auto task_w = [&](int t) -> const uint16_t* {
    const int j = t / nch, c = t - j * nch;
    const int item = blockIdx.x + j * gridDim.x;
    const int u = item / nrb, rb = item - u * nrb;
    return wgu + (static_cast<size_t>(s_e[u]) * 2 * I + rb * 16 + col) * H + kb + c * KC * 32;
  };
  bf16x8 gA[KC], uA[KC], gB[KC], uB[KC];
  const size_t up_off = static_cast<size_t>(I) * H;
#define GU_ISSUE(G, UU, T)                                             \
  {                                                                    \
    const uint16_t* pg_ = task_w(T);                                   \
    _Pragma("unroll") for (int s = 0; s < KC; ++s) {                   \
      G[s] = as_bf16x8(ld16(pg_ + s * 32));                            \
      UU[s] = as_bf16x8(ld16(pg_ + up_off + s * 32));                  \
    }                                                                  \
  }
  f32x4 ag[TM], au[TM];
  int tok[TM];
  int ntok = 0, tiles = 0;

  auto run_task = [&](const bf16x8 (&G)[KC], const bf16x8 (&UU)[KC], int t) {
    const int j = t / nch, c = t - j * nch;
    const int item = blockIdx.x + j * gridDim.x;
    const int u = item / nrb, rb = item - u * nrb;
    const int base = s_off[u];
    if (c == 0) {
      ntok = s_off[u + 1] - base;
      tiles = (ntok + 15) >> 4;
#pragma unroll
      for (int q = 0; q < TM; ++q) {
        const int p = 16 * q + col;
        tok[q] = s_pr[base + (p < ntok ? p : 0)] / k;   // past the end: a valid token, column discarded
        ag[q] = au[q] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
    const uint32_t ko = kb + c * KC * 32;
#pragma unroll
    for (int q = 0; q < TM; ++q) {
      if (q < tiles) {
        bf16x8 xb[KC];
#pragma unroll
        for (int s = 0; s < KC; ++s) xb[s] = as_bf16x8(ld16(x + static_cast<size_t>(tok[q]) * H + ko + s * 32));
#pragma unroll
        for (int s = 0; s < KC; ++s) {
          ag[q] = mfma16x16x32(G[s], xb[s], ag[q]);
          au[q] = mfma16x16x32(UU[s], xb[s], au[q]);
        }
      }
    }
    if (c != nch - 1) return;
    // epilogue of the item: fixed-order sum over waves, SwiGLU, weight, split, store
#pragma unroll
    for (int q = 0; q < TM; ++q) {
      if (q < tiles) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          red[(((wv * TM + q) * 2 + 0) * 4 + r) * 64 + ln] = ag[q][r];
          red[(((wv * TM + q) * 2 + 1) * 4 + r) * 64 + ln] = au[q][r];
        }
      }
    }
    __syncthreads();
    for (int qq = threadIdx.x; qq < tiles * 256; qq += blockDim.x) {
      const int q = qq >> 8, within = qq & 255;
      const int n = within >> 4, m = within & 15;    // token column n, weight row m
      const int src = 16 * (m >> 2) + n, r = m & 3;
      float g = 0.f, up = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < kDecWaves; ++w2) {
        g += red[(((w2 * TM + q) * 2 + 0) * 4 + r) * 64 + src];
        up += red[(((w2 * TM + q) * 2 + 1) * 4 + r) * 64 + src];
      }
      const int p = q * 16 + n;
      if (p < ntok) {
        const int pr = s_pr[base + p];               // pair t*k + j of this token and expert
        const float hv = wts[pr] * swiglu(g, up);
        hw[static_cast<size_t>(pr) * I + rb * 16 + m] = static_cast<uint16_t>(f32_to_bf16_rne(hv));
      }
    }
    __syncthreads();
  };

  if (ntask > 0) GU_ISSUE(gA, uA, 0)
  for (int t = 0; t < ntask; t += 2) {
    if (t + 1 < ntask) GU_ISSUE(gB, uB, t + 1)
    run_task(gA, uA, t);
    if (t + 1 < ntask) {
      if (t + 2 < ntask) GU_ISSUE(gA, uA, t + 2)
      run_task(gB, uB, t + 1);
    }
  }
#undef GU_ISSUE
}

// down: workgroup = 8 output dimensions d0..d0+7 of every touched expert (H/8
// workgroups, enough to occupy every CU without splitting the expert sum
// across workgroups).  MFMA rows 0..7 carry those dimensions; lanes of rows
// 8..15 issue no weight loads (the MFMA work they waste is free: the kernel
// is bound by memory).  MFMA columns are the tokens routed to the current
// expert, compacted (16 per tile), so every activation load is a routed
// token's row and each expert costs one tile of loads and MFMAs (more only
// for the rare expert with over 16 tokens).  Each wave adds an expert's
// results into its own FP32 accumulator rows in LDS ([token][8 dims]), in
// ascending expert order; the 16 waves' accumulators are added in wave order
// at the end, so the sum order is fixed.  The 16 waves form EGW expert groups
// x KSW K-slices: wave (eg, ks) takes experts u = eg, eg + EGW, ... and the K
// range [ks*I/KSW, (ks+1)*I/KSW) of each, loading the next expert's weights
// and first activation tile while it multiplies the current one.
constexpr int kDownRows = 8;
constexpr int kDownWaves = 16;
constexpr int kDownThreads = kDownWaves * kWave;

template <int KD>
__global__ __launch_bounds__(kDownThreads) void decode_down(
    const uint16_t* __restrict__ wd, const int* __restrict__ plan_u,
    const int32_t* __restrict__ plan_e, const int32_t* __restrict__ plan_off,
    const uint16_t* __restrict__ plan_pr, const uint16_t* __restrict__ hw, int T, int H, int I,
    int k, int KSW, uint16_t* __restrict__ out) {
  extern __shared__ float accl[];                   // [16 waves][T][8 dims]
  __shared__ int s_e[kMaxPlan];
  __shared__ int s_off[kMaxPlan + 1];
  __shared__ uint16_t s_pr[kMaxPairs];
  const int U = *plan_u;
  for (int i = threadIdx.x; i < U; i += blockDim.x) s_e[i] = plan_e[i];
  for (int i = threadIdx.x; i <= U; i += blockDim.x) s_off[i] = plan_off[i];
  for (int i = threadIdx.x; i < T * k; i += blockDim.x) s_pr[i] = plan_pr[i];
  for (int i = threadIdx.x; i < kDownWaves * T * kDownRows; i += blockDim.x) accl[i] = 0.f;
  __syncthreads();
  const int wv = wave_id(), ln = lane_id();
  const int col = ln & 15, grp = ln >> 4;
  const int EGW = kDownWaves / KSW;
  const int ks = wv % KSW, eg = wv / KSW;
  const bool row_lane = col < kDownRows;
  const int d0 = blockIdx.x * kDownRows;
  const int kw = I / KSW;                           // = KD * 32
  const uint32_t kb = static_cast<uint32_t>(ks * kw + grp * 8);
  const uint16_t* pw = wd + (static_cast<size_t>(d0) + (row_lane ? col : 0)) * I + kb;
  float* myacc = accl + wv * T * kDownRows;
  const bf16x8 zero8 = {};
  const int ntask = U > eg ? (U - 1 - eg) / EGW + 1 : 0;

  // add the tile's D rows 0..7 (lanes grp < 2) into token t's accumulator row
  auto accumulate = [&](const f32x4& d, int t, bool on) {
    if (on && grp < 2) {
      f32x4* a = reinterpret_cast<f32x4*>(myacc + t * kDownRows + 4 * grp);
      *a = *a + d;
    }
  };
  bf16x8 aA[KD], aB[KD], bA[KD], bB[KD];
  int pA = 0, pB = 0;                               // pair of this lane's column in the first tile
#define DN_ISSUE(A, B, P, TSK)                                                             \
  {                                                                                        \
    const int u_ = eg + (TSK) * EGW;                                                       \
    const int base_ = s_off[u_];                                                           \
    const uint16_t* p_ = pw + static_cast<size_t>(s_e[u_]) * H * I;                        \
    _Pragma("unroll") for (int s = 0; s < KD; ++s)                                         \
      A[s] = row_lane ? as_bf16x8(ld16(p_ + s * 32)) : zero8;                              \
    const bool on_ = col < s_off[u_ + 1] - base_;                                          \
    P = on_ ? s_pr[base_ + col] : 0;                                                       \
    const size_t r_ = static_cast<size_t>(P) * I + kb;                                     \
    _Pragma("unroll") for (int s = 0; s < KD; ++s)                                         \
      B[s] = on_ ? as_bf16x8(ld16(hw + r_ + s * 32)) : zero8;                              \
  }
#define DN_RUN(A, B, P, TSK)                                                               \
  {                                                                                        \
    const int u_ = eg + (TSK) * EGW;                                                       \
    const int base_ = s_off[u_];                                                           \
    const int nt_ = s_off[u_ + 1] - base_;                                                 \
    f32x4 d_ = {0.f, 0.f, 0.f, 0.f};                                                       \
    _Pragma("unroll") for (int s = 0; s < KD; ++s) d_ = mfma16x16x32(A[s], B[s], d_);      \
    accumulate(d_, P / k, col < nt_);                                                      \
    for (int c0 = 16; c0 < nt_; c0 += 16) {           /* experts with over 16 tokens */    \
      const bool on_ = c0 + col < nt_;                                                     \
      const int pr_ = on_ ? s_pr[base_ + c0 + col] : 0;                                    \
      const size_t r_ = static_cast<size_t>(pr_) * I + kb;                                 \
      bf16x8 bx_[KD];                                                                      \
      _Pragma("unroll") for (int s = 0; s < KD; ++s)                                       \
        bx_[s] = on_ ? as_bf16x8(ld16(hw + r_ + s * 32)) : zero8;                          \
      f32x4 dx_ = {0.f, 0.f, 0.f, 0.f};                                                    \
      _Pragma("unroll") for (int s = 0; s < KD; ++s) dx_ = mfma16x16x32(A[s], bx_[s], dx_); \
      accumulate(dx_, pr_ / k, on_);                                                       \
    }                                                                                      \
  }
  if (ntask > 0) DN_ISSUE(aA, bA, pA, 0)
  for (int t = 0; t < ntask; t += 2) {
    if (t + 1 < ntask) DN_ISSUE(aB, bB, pB, t + 1)
    DN_RUN(aA, bA, pA, t)
    if (t + 1 < ntask) {
      if (t + 2 < ntask) DN_ISSUE(aA, bA, pA, t + 2)
      DN_RUN(aB, bB, pB, t + 1)
    }
  }
#undef DN_ISSUE
#undef DN_RUN
  __syncthreads();
  for (int i = threadIdx.x; i < T * kDownRows; i += blockDim.x) {
    float v = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < kDownWaves; ++w2) v += accl[w2 * T * kDownRows + i];
    const int t = i / kDownRows, mm = i - t * kDownRows;
    out[static_cast<size_t>(t) * H + d0 + mm] = static_cast<uint16_t>(f32_to_bf16_rne(v));
  }
}

hipError_t launch_decode(const uint16_t* x, const float* logits, const uint16_t* wgu,
                         const uint16_t* wd, int T, int H, int I, int E, int k, uint16_t* out,
                         int32_t* idx, float* w, void* ws, hipStream_t s, int num_cus) {
  const DecodeWs L = decode_ws_layout(T, H, I, E, k);
  char* base = static_cast<char*>(ws);
  int* plan_u = reinterpret_cast<int*>(base + L.plan_u);
  int32_t* plan_e = reinterpret_cast<int32_t*>(base + L.plan_e);
  int32_t* plan_off = reinterpret_cast<int32_t*>(base + L.plan_off);
  uint16_t* plan_pr = reinterpret_cast<uint16_t*>(base + L.plan_pr);
  int32_t* idx_p = idx ? idx : reinterpret_cast<int32_t*>(base + L.idx);
  float* w_p = w ? w : reinterpret_cast<float*>(base + L.w);
  uint16_t* hw = reinterpret_cast<uint16_t*>(base + L.hw);

  hipError_t err = launch_route_topk(logits, T, E, k, idx_p, w_p, s);   // brackets kRoute
  if (err != hipSuccess) return err;

  const int TM = T <= 16 ? 1 : (T <= 32 ? 2 : 4);   // token tiles the kernels carry
  const long items_upper = static_cast<long>(T * k < E ? T * k : E) * (I / 16);
  const long grid_cap = 2L * num_cus;
  const int grid1 = static_cast<int>(items_upper < grid_cap ? items_upper : grid_cap);
  // reduction buffer; the plan scratch (E masks + chunk offsets) must fit in it too
  size_t lds_gu = sizeof(float) * kDecWaves * TM * 2 * 256;
  const size_t lds_plan = sizeof(uint64_t) * E + sizeof(int) * (E + 33);
  if (lds_plan > lds_gu) lds_gu = lds_plan;
  const size_t lds_dn = sizeof(float) * kDownWaves * T * kDownRows;
  const int gsteps = H / kDecWaves / 32;
  int KC = gsteps % 4 == 0 ? 4 : (gsteps % 3 == 0 ? 3 : (gsteps % 2 == 0 ? 2 : 1));
  if (TM == 4 && KC == 4) KC = 2;                   // keeps four token tiles within 128 VGPRs
  // down: K-slices per workgroup so that each wave has at most 4 steps of 32
  // (I is a multiple of 256, so I/32 is a multiple of 8 and KSW <= 16 works)
  const int dtotal = I / 32;
  int KSW = 1;
  while (KSW < kDownWaves && (dtotal / KSW > 4 || dtotal % KSW)) KSW *= 2;
  const int KD = dtotal / KSW;
  const dim3 grid2(H / kDownRows);
  prof_begin(kDecGateUp, s);
#define GU_LAUNCH(TMV, KCV)                                                                    \
  hipLaunchKernelGGL((decode_gate_up<TMV, KCV>), dim3(grid1), dim3(kDecThreads), lds_gu, s, x,   \
                     wgu, idx_p, w_p, T, E, plan_u, plan_e, plan_off, plan_pr, H, I, k, hw)
#define GU_KC(TMV)                                        \
  switch (KC) {                                           \
    case 4: GU_LAUNCH(TMV, 4); break;                     \
    case 3: GU_LAUNCH(TMV, 3); break;                     \
    case 2: GU_LAUNCH(TMV, 2); break;                     \
    default: GU_LAUNCH(TMV, 1); break;                    \
  }
  if (TM == 1) { GU_KC(1) } else if (TM == 2) { GU_KC(2) } else { GU_KC(4) }
#undef GU_KC
#undef GU_LAUNCH
  prof_end(kDecGateUp, s);
  prof_begin(kDecDown, s);
#define DN_LAUNCH(KDV)                                                                         \
  hipLaunchKernelGGL((decode_down<KDV>), grid2, dim3(kDownThreads), lds_dn, s, wd, plan_u, plan_e, \
                     plan_off, plan_pr, hw, T, H, I, k, KSW, out)
  switch (KD) {
    case 4: DN_LAUNCH(4); break;
    case 3: DN_LAUNCH(3); break;
    case 2: DN_LAUNCH(2); break;
    default: DN_LAUNCH(1); break;
  }
#undef DN_LAUNCH
  prof_end(kDecDown, s);
  return hipGetLastError();
}

hipError_t decode_set_attributes() {
  const void* tm4[] = {reinterpret_cast<const void*>(decode_gate_up<4, 1>),
                       reinterpret_cast<const void*>(decode_gate_up<4, 2>),
                       reinterpret_cast<const void*>(decode_gate_up<4, 3>),
                       reinterpret_cast<const void*>(decode_gate_up<4, 4>)};
  hipError_t e = hipSuccess;
  for (const void* f : tm4) {
    e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize,
                            sizeof(float) * kDecWaves * 4 * 2 * 256);
    if (e != hipSuccess) return e;
  }
  return e;
}

}  // namespace moe
