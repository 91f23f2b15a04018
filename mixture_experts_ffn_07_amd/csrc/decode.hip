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
#include <atomic>
#include <map>
#include <mutex>
#include <random>
#include <utility>

#include "common.h"
#include "internal.h"
#include "route.h"
#include "tiles.h"

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
  L.flags = o;       o = align256(o + sizeof(uint64_t) * kMaxDecodeGrid);
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

// Workgroup 0 of gate_up writes the plan to global memory for the down kernel.
__device__ void publish_plan(int U, int P, const int* s_e, const int* s_off, const uint16_t* s_pr,
                             int* plan_u, int32_t* plan_e, int32_t* plan_off, uint16_t* plan_pr) {
  for (int i = threadIdx.x; i < U; i += blockDim.x) {
    plan_e[i] = s_e[i];
    plan_off[i + 1] = s_off[i + 1];
  }
  for (int i = threadIdx.x; i < P; i += blockDim.x) plan_pr[i] = s_pr[i];
  if (threadIdx.x == 0) {
    plan_off[0] = 0;
    *plan_u = U;
  }
}

// down: workgroup = 8*NR output dimensions of every touched expert (NR = 1 or
// 2 groups of 8; H/(8*NR) workgroups, enough to occupy every CU without
// splitting the expert sum across workgroups).  The 16x16x32 MFMA is used as
// two 8x8 products side by side: rows 0..7 and 8..15 both carry the 8
// dimensions of a group, rows 0..7 with the first 32 of each 64 K positions
// and rows 8..15 with the second, and columns 0..7 / 8..15 carry the same
// tokens' matching K halves.  The two diagonal 8x8 blocks of D are the wanted
// partial sums (the off-diagonal blocks are discarded), so every lane's weight
// load is useful: per step a wave reads 8 rows x 128 contiguous bytes per
// group.  The tokens are those routed to the current expert (compacted plan
// columns).  A dense load (64 lanes, 16 bytes each) brings the wave's K range
// of several tokens at once into a small wave-private LDS tile, from which
// the lanes read the MFMA layout; with two groups one activation load serves
// both (the activations are re-read by every workgroup, so wider workgroups
// halve that traffic where H leaves enough of them).  Each wave adds an
// expert's results into its own FP32 accumulator rows in LDS ([token][8*NR
// dims]), in ascending expert order, first the half-0 block then the half-1
// block; the 16 waves' accumulators are added in wave order at the end, so the
// sum order is fixed.  The 16 waves form EGW expert groups x KSW K-slices:
// wave (eg, ks) takes experts u = eg, eg + EGW, ... and the K range
// [ks*I/KSW, (ks+1)*I/KSW) of each (64*KD positions), loading the next
// expert's weights and first activations while it multiplies the current one.
constexpr int kDownRows = 8;
constexpr int kDownWaves = 16;
constexpr int kDownThreads = kDownWaves * kWave;

// per-KD geometry of the activation staging tile
template <int KD>
struct DownGeom {
  static constexpr int kCh = 8 * KD;                // 16-byte chunks of one token's K range
  static constexpr int kPerLoad = kWave / kCh;      // tokens one dense load covers
  static constexpr int kTW = 2 * kPerLoad < 8 ? 2 * kPerLoad : 8;   // tokens per MFMA tile
  static constexpr int kRow = kCh + 1;              // padded tile row (chunks): no bank conflicts
  static constexpr int kStage = kTW * kRow;         // chunks per wave
};

// The down phase of one workgroup for output dimensions [d0, d0 + 8*NR): the
// plan (touched experts ascending, their routed pairs in token order) is in
// LDS; `accl` is the dynamic LDS of down_lds_bytes().  NWD waves form EGW
// expert groups x KSW K-slices.  With PRE the weights of each wave's first two
// tasks are loaded before `wait()` returns and the activations only after it:
// the single-launch decode waits there for every workgroup's activations.
template <int KD, int NR, int NWD, bool PRE, typename PE, typename PO, class Wait>
__device__ __forceinline__ void down_phase(
    const uint16_t* __restrict__ wd, int U, const PE* s_e, const PO* s_off,
    const uint16_t* s_pr, const uint8_t* s_tk, const uint16_t* __restrict__ hw, int T, int H,
    int I, int KSW, int d0, float* accl, uint16_t* __restrict__ out, Wait wait) {
  using G = DownGeom<KD>;
  constexpr int RW = kDownRows * NR;                // output dimensions per workgroup
  constexpr int NTD = NWD * kWave;
  for (int i = threadIdx.x; i < NWD * T * RW; i += NTD) accl[i] = 0.f;
  __syncthreads();
  const int wv = __builtin_amdgcn_readfirstlane(wave_id()), ln = lane_id();
  const int col = ln & 15, grp = ln >> 4;
  const int hf = col >> 3, c8 = col & 7;            // K half and row / token within it
  const int EGW = NWD / KSW;
  const int ks = wv % KSW, eg = wv / KSW;
  const int kw = I / KSW;                           // = 64 * KD
  // weights: lane (row c8, half hf, group grp), step s -> K offset 64s + 32hf + 8grp;
  // dimension group r adds 8r rows
  const uint32_t woff = static_cast<uint32_t>((d0 + c8) * I + ks * kw + hf * 32 + grp * 8);
  float* myacc = accl + wv * T * RW;
  i32x4* stage = reinterpret_cast<i32x4*>(accl + NWD * T * RW) + wv * G::kStage;
  // dense activation loads: lane = token slot dc, chunk dq of the wave's K range
  const int dc = ln / G::kCh, dq = ln - dc * G::kCh;
  const bool ld_lane = dc < G::kPerLoad;
  const uint32_t kd = static_cast<uint32_t>(ks * kw + dq * 8);
  i32x4* st0 = stage + dc * G::kRow + dq;           // this lane's slot for the first load
  i32x4* st1 = st0 + G::kPerLoad * G::kRow;         // and for the second
  // MFMA B lane (token c8, half hf, group grp): chunk 8s + 4hf + grp; tokens past the
  // tile read a valid row whose columns are discarded
  const i32x4* bsrc = stage + (c8 < G::kTW ? c8 : G::kTW - 1) * G::kRow + 4 * hf + grp;
  // D: lane (column col, group grp) holds rows 4grp..4grp+3; the wanted block is
  // group half == column half, token c8, dims 4*(grp&1)..+3
  const bool d_lane = (grp >> 1) == hf;
  const int dofs = 4 * (grp & 1);
  const int ntask = U > eg ? (U - 1 - eg) / EGW + 1 : 0;

  bf16x8 aA[NR][KD], aB[NR][KD];
  i32x4 hA0 = {}, hA1 = {}, hB0 = {}, hB1 = {};
  // activations of tokens [c0, c0 + kPerLoad) of the plan entries at `base` (nt of
  // them): every lane loads (lanes past the tokens repeat the last valid one), so
  // the load count is fixed
  auto load_at = [&](int base, int c0, int nt) {
    const int last = nt - 1;
    const int slot = ld_lane && c0 + dc <= last ? c0 + dc : (c0 < last ? c0 : last);
    const uint16_t* p = hw + static_cast<uint32_t>(s_pr[base + slot] * I + kd);
    if constexpr (PRE) {        // written by other workgroups of this launch: device-coherent
      const uint64_t* q = reinterpret_cast<const uint64_t*>(p);
      const uint64_t lo = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint64_t hi = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return i32x4{static_cast<int>(lo), static_cast<int>(lo >> 32), static_cast<int>(hi),
                   static_cast<int>(hi >> 32)};
    }
    return ld16(p);
  };
  auto task_plan = [&](int tsk, int& base, int& nt, int& e) {
    const int u = eg + tsk * EGW;
    base = __builtin_amdgcn_readfirstlane(static_cast<int>(s_off[u]));
    nt = __builtin_amdgcn_readfirstlane(static_cast<int>(s_off[u + 1])) - base;
    e = __builtin_amdgcn_readfirstlane(static_cast<int>(s_e[u]));
  };
  auto issue_w = [&](int tsk, bf16x8 (&A)[NR][KD]) {
    int base, nt, e;
    task_plan(tsk, base, nt, e);
    const uint16_t* pe = wd + static_cast<size_t>(e) * H * I;
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int s = 0; s < KD; ++s)
        A[r][s] = as_bf16x8(ld16_stream(pe + woff + r * kDownRows * I + s * 64));
  };
  auto issue_h = [&](int tsk, i32x4& h0, i32x4& h1) {
    int base, nt, e;
    task_plan(tsk, base, nt, e);
    h0 = load_at(base, 0, nt);
    if (G::kTW > G::kPerLoad && nt > G::kPerLoad) h1 = load_at(base, G::kPerLoad, nt);
  };
  // loads of one task in a fixed order: first activations, weights, optional activations
  auto issue = [&](int tsk, bf16x8 (&A)[NR][KD], i32x4& h0, i32x4& h1) {
    int base, nt, e;
    task_plan(tsk, base, nt, e);
    h0 = load_at(base, 0, nt);
    const uint16_t* pe = wd + static_cast<size_t>(e) * H * I;
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int s = 0; s < KD; ++s)
        A[r][s] = as_bf16x8(ld16_stream(pe + woff + r * kDownRows * I + s * 64));
    if (G::kTW > G::kPerLoad && nt > G::kPerLoad) h1 = load_at(base, G::kPerLoad, nt);
  };
  // stage tokens [c0, c0 + kTW) (already loaded into h0, h1), multiply, accumulate
  auto tile = [&](const bf16x8 (&A)[NR][KD], int base, int c0, int nt, const i32x4& h0,
                  const i32x4& h1) {
    if (ld_lane) {
      *st0 = h0;
      if (G::kTW > G::kPerLoad) *st1 = h1;
    }
    __builtin_amdgcn_wave_barrier();
    bf16x8 b[KD];
#pragma unroll
    for (int s = 0; s < KD; ++s) b[s] = as_bf16x8(bsrc[8 * s]);
    const bool on = d_lane && c8 < G::kTW && c0 + c8 < nt;
    const int t = on ? s_tk[base + c0 + c8] : 0;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KD; ++s) d = mfma16x16x32(A[r][s], b[s], d);
      f32x4* acc = reinterpret_cast<f32x4*>(myacc + t * RW + r * kDownRows + dofs);
      if (on && hf == 0) *acc = *acc + d;           // half-0 block, then half-1 block
      __builtin_amdgcn_wave_barrier();
      if (on && hf == 1) *acc = *acc + d;
      __builtin_amdgcn_wave_barrier();
    }
  };
  auto run = [&](int tsk, const bf16x8 (&A)[NR][KD], const i32x4& h0, const i32x4& h1) {
    int base, nt, e;
    task_plan(tsk, base, nt, e);
    tile(A, base, 0, nt, h0, h1);                   // every touched expert has a token
    if (nt > G::kTW) {                              // experts with more than kTW tokens:
      // the next tile's loads are issued before the current tile waits (fixed count,
      // clamped rows), so their latency overlaps
      i32x4 r0 = load_at(base, G::kTW, nt);
      i32x4 r1 = G::kTW > G::kPerLoad ? load_at(base, G::kTW + G::kPerLoad, nt) : r0;
      for (int c0 = G::kTW; c0 < nt; c0 += G::kTW) {
        const i32x4 n0 = load_at(base, c0 + G::kTW, nt);
        const i32x4 n1 = G::kTW > G::kPerLoad ? load_at(base, c0 + G::kTW + G::kPerLoad, nt) : n0;
        tile(A, base, c0, nt, r0, r1);
        r0 = n0;
        r1 = n1;
      }
    }
  };
  // one task ahead: the loads of task t+1 are in flight while task t multiplies
  int t = 0;
  if (PRE) {
    // the first two tasks' weights before the wait, their activations after it
    if (ntask > 0) issue_w(0, aA);
    if (ntask > 1) issue_w(1, aB);
    wait();
    if (ntask > 0) issue_h(0, hA0, hA1);
    if (ntask > 1) {
      issue_h(1, hB0, hB1);
      run(0, aA, hA0, hA1);
      if (ntask > 2) issue(2, aA, hA0, hA1);
      run(1, aB, hB0, hB1);
      t = 2;
    }
  } else if (ntask > 0) {
    issue(0, aA, hA0, hA1);
  }
  if (t < ntask) {
    for (; t + 2 < ntask; t += 2) {
      issue(t + 1, aB, hB0, hB1);
      run(t, aA, hA0, hA1);
      issue(t + 2, aA, hA0, hA1);
      run(t + 1, aB, hB0, hB1);
    }
    if (t + 1 < ntask) {
      issue(t + 1, aB, hB0, hB1);
      run(t, aA, hA0, hA1);
      run(t + 1, aB, hB0, hB1);
    } else {
      run(t, aA, hA0, hA1);
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < T * RW; i += NTD) {
    float v = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < NWD; ++w2) v += accl[w2 * T * RW + i];
    const int tt = i / RW, mm = i - tt * RW;
    out[static_cast<size_t>(tt) * H + d0 + mm] = static_cast<uint16_t>(f32_to_bf16_rne(v));
  }
}

struct NoWait {
  __device__ void operator()() const {}
};

// Wait of the single-launch decode: every workgroup of the grid has published
// flag == epoch (a 64-bit value unique to the launch, so flags left by earlier
// launches never match).  Wave 0 polls the flags with device-scope loads,
// bounded by kGridWaitPolls rounds.  The activations behind the flags were
// written with device-scope stores that had completed before each flag was
// written, and the down phase reads them with device-scope loads, so no cache
// needs flushing here.  *fail = 1 if the bound was reached.
constexpr int kGridWaitPolls = 1 << 20;
struct GridWait {
  const uint64_t* flags;
  uint64_t epoch;
  int n;
  int* fail;
  __device__ void operator()() const {
    if (wave_id() == 0) {
      bool ok = false;
      for (int it = 0; it < kGridWaitPolls; ++it) {
        bool mine = true;
        for (int i = lane_id(); i < n; i += kWave)
          mine = mine && __hip_atomic_load(flags + i, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT) == epoch;
        ok = __all(mine);
        if (ok) break;
        __builtin_amdgcn_s_sleep(4);
      }
      if (lane_id() == 0) *fail = ok ? 0 : 1;
    }
    __syncthreads();
  }
};

template <int KD, int NR>
__global__ __launch_bounds__(kDownThreads) void decode_down(
    const uint16_t* __restrict__ wd, const int* __restrict__ plan_u,
    const int32_t* __restrict__ plan_e, const int32_t* __restrict__ plan_off,
    const uint16_t* __restrict__ plan_pr, const uint16_t* __restrict__ hw, int T, int H, int I,
    int k, int KSW, uint16_t* __restrict__ out, uint32_t okey) {
  // dynamic LDS: [16 waves][T][RW dims] FP32 accumulators, then [16 waves][kStage] chunks
  extern __shared__ float accl[];
  __shared__ uint16_t s_e[kMaxPlan];                // E <= 1024
  __shared__ uint16_t s_off[kMaxPlan + 1];          // <= T*k <= 2048
  __shared__ uint16_t s_pr[kMaxPairs];
  __shared__ uint8_t s_tk[kMaxPairs];               // token of each plan entry (T <= 64)
  const int U = *plan_u;
  for (int i = threadIdx.x; i < U; i += kDownThreads) s_e[i] = static_cast<uint16_t>(plan_e[i]);
  for (int i = threadIdx.x; i <= U; i += kDownThreads) s_off[i] = static_cast<uint16_t>(plan_off[i]);
  for (int i = threadIdx.x; i < T * k; i += kDownThreads) {
    const int pr = plan_pr[i];
    s_pr[i] = static_cast<uint16_t>(pr);
    s_tk[i] = static_cast<uint8_t>(pr / k);
  }
  down_phase<KD, NR, kDownWaves, false>(wd, U, s_e, s_off, s_pr, s_tk, hw, T, H, I, KSW,
                                         permute_item(blockIdx.x, gridDim.x, okey) * kDownRows * NR,
                                         accl, out, NoWait());
}

// gate_up: work item = (touched expert u, block of NB = 8*NG neurons);
// workgroups stride over items.  The K dimension H is cut into steps of 64
// positions and the eight waves share them (wave wv takes steps
// [wv*S/8, (wv+1)*S/8), S = H/64), walking them in chunks of KC steps.
//
// MFMA layout (two 8x8 products per 16x16x32 instruction): A rows 0..7 are
// the 8 neurons of a neuron group with the first 32 positions of a step, rows
// 8..15 the same neurons with the second 32; B columns 0..7 / 8..15 are up to
// 8 tokens with the same two halves.  The diagonal 8x8 blocks of D are the
// wanted partial sums, added together once per item.  With this layout every
// weight load instruction reads 8 rows x 128 contiguous bytes (whole cache
// lines, streamed with the non-temporal hint) and every activation load 8
// tokens x 128 bytes.
//
// The workgroup walks its flat sequence of (item, chunk) tasks with the
// weights of the next task loaded into a second register buffer while the
// current one is multiplied, so the weight stream never waits on an epilogue.
//
// At T <= 16 (route != 0) the routing runs here too: a separate launch and its
// gap before this kernel cost more than routing two tokens per wave.  Every
// workgroup routes all T tokens (the same routine as moe_route_topk, so the
// result is bit-identical) into LDS past the plan scratch, and workgroup 0
// writes topk_idx / topk_w out.  Otherwise the routing launch has written them
// and each workgroup copies them into the same LDS area.
//
// FUSED (the single-launch decode, T <= 16): after its last item every
// workgroup publishes a flag (its activations written and made visible at
// device scope), and then runs the down phase for output dimensions
// [8*dg, 8*dg + 8), dg = blockIdx.x, blockIdx.x + gridDim.x, ...: the weights of
// each wave's first two down tasks are loaded while it waits for every
// workgroup's flag (they do not depend on the activations), and the rest as in
// decode_down.  The grid is sized from the occupancy query so that every
// workgroup is resident at once on the device; a workgroup that is not yet
// resident (other work holding CUs) is placed as that work retires, since
// nothing it waits for depends on this kernel.  The wait is bounded all the
// same (kGridWaitPolls polls), and a workgroup that gives up writes NaN into
// its outputs.
template <int TM8, int NG, int KC, int NW = kDecWaves, bool FUSED = false, int KD = 3>   // TM8 <= 4: T <= 32
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(4, 8))) void decode_gate_up(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wgu,
    const float* __restrict__ logits, int32_t* __restrict__ idx, float* __restrict__ wts,
    int T, int E, int* __restrict__ plan_u, int32_t* __restrict__ plan_e,
    int32_t* __restrict__ plan_off, uint16_t* __restrict__ plan_pr, int H, int I, int k,
    uint16_t* __restrict__ hw, int route_off, int route, const uint16_t* __restrict__ wd,
    uint16_t* __restrict__ out, uint64_t* __restrict__ flags, uint64_t epoch, int KSW, uint32_t okey) {
  constexpr int kDecWaves = NW;                     // this instantiation's waves
  constexpr int kDecThreads = NW * kWave;
  constexpr int NB = 8 * NG;                        // neurons per item
  // dynamic LDS: two buffers (alternate items) of [8 waves][TM8 tiles][NG groups]
  // [gate/up][4 regs][16 lanes] FP32 per-wave sums, which the plan scratch (E masks,
  // E + 33 ints) borrows first; at byte route_off the routing result [T*k] ids, weights
  extern __shared__ float red[];
  __shared__ int s_e[kMaxPlan];
  __shared__ int s_off[kMaxPlan + 1];
  __shared__ uint16_t s_pr[kMaxPairs];
  __shared__ float s_w[kMaxPairs];                  // routing weight of each plan entry
  int32_t* r_idx = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(red) + route_off);
  float* r_w = reinterpret_cast<float*>(r_idx + T * k);
  if (route) {
    // wave w routes tokens w and w + 8 (T <= 16)
    const int w0 = wave_id();
    constexpr int NTW = (16 + NW - 1) / NW;          // tokens per wave (T <= 16)
    if (E <= 64) route_tokens_wave<1, NTW>(logits, T, E, k, w0, kDecWaves, r_idx, r_w);
    else if (E <= 128) route_tokens_wave<2, NTW>(logits, T, E, k, w0, kDecWaves, r_idx, r_w);
    else if (E <= 256) route_tokens_wave<4, NTW>(logits, T, E, k, w0, kDecWaves, r_idx, r_w);
    else if (E <= 512) route_tokens_wave<8, NTW>(logits, T, E, k, w0, kDecWaves, r_idx, r_w);
    else route_tokens_wave<16, NTW>(logits, T, E, k, w0, kDecWaves, r_idx, r_w);
    __syncthreads();
    if (blockIdx.x == 0) {
      for (int i = threadIdx.x; i < T * k; i += kDecThreads) {
        idx[i] = r_idx[i];
        wts[i] = r_w[i];
      }
    }
  } else {
    for (int i = threadIdx.x; i < T * k; i += kDecThreads) {
      r_idx[i] = idx[i];
      r_w[i] = wts[i];
    }
    __syncthreads();
  }
  const int U = build_plan(r_idx, T, E, k, reinterpret_cast<uint64_t*>(red),
                           reinterpret_cast<int*>(reinterpret_cast<uint64_t*>(red) + E), s_e,
                           s_off, s_pr);
  // (the epilogues then issue no global loads, which would wait on the weight stream)
  for (int i = threadIdx.x; i < T * k; i += kDecThreads) s_w[i] = r_w[s_pr[i]];
  if (blockIdx.x == 0) publish_plan(U, T * k, s_e, s_off, s_pr, plan_u, plan_e, plan_off, plan_pr);
  const int nrb = I / NB;
  const int items = U * nrb;
  const int wv = __builtin_amdgcn_readfirstlane(wave_id()), ln = lane_id();
  const int col = ln & 15, grp = ln >> 4;
  const int hf = col >> 3, c8 = col & 7;
  const int S = H / 64;                             // steps of 64 positions
  const int s0 = wv * S / kDecWaves, s1 = (wv + 1) * S / kDecWaves;
  const int nch = (s1 - s0) / KC;                   // chunks per item (KC divides s1 - s0)
  // FUSED: workgroups take gate_up items from the top of the grid down, so the
  // low-numbered ones, which also do the down phase, hold the fewest items
  const int gb = FUSED ? static_cast<int>(gridDim.x - 1 - blockIdx.x) : static_cast<int>(blockIdx.x);
  const int my_items = gb < items ? (items - 1 - gb) / gridDim.x + 1 : 0;
  // lane's K offset within a step: half hf, 16-byte group grp
  const uint32_t kl = static_cast<uint32_t>(s0 * 64 + hf * 32 + grp * 8);
  const size_t up_off = static_cast<size_t>(I) * H;

  auto item_of = [&](int j, int& u, int& rb) {
    const int item = permute_item(gb + j * gridDim.x, items, okey);
    u = item / nrb;
    rb = item - u * nrb;
  };
  // first weight element of task t (item j, chunk c) for this lane: gate row of group 0
  auto task_w = [&](int t) -> const uint16_t* {
    const int j = t / nch, c = t - j * nch;
    int u, rb;
    item_of(j, u, rb);
    const int e = __builtin_amdgcn_readfirstlane(s_e[u]);
    return wgu + (static_cast<size_t>(e) * 2 * I + rb * NB + c8) * H + kl + c * KC * 64;
  };
  bf16x8 gA[KC][NG], uA[KC][NG], gB[KC][NG], uB[KC][NG];
  bf16x8 xA[KC], xB[KC];                            // first token tile's activations
  uint32_t itk = 0;                                 // this lane's first-tile token, issue side
  // loads of task t: weights, then the first token tile's activations
  auto issue = [&](int t, bf16x8 (&G)[KC][NG], bf16x8 (&UU)[KC][NG], bf16x8 (&XT)[KC]) {
    const int j = t / nch, c = t - j * nch;
    if (c == 0) {                                   // a new item: its first tile's tokens
      int u, rb;
      item_of(j, u, rb);
      const int b = __builtin_amdgcn_readfirstlane(s_off[u]);
      const int n = __builtin_amdgcn_readfirstlane(s_off[u + 1]) - b;
      itk = static_cast<uint32_t>(s_pr[b + (c8 < n ? c8 : 0)] / k);
    }
    const uint16_t* pg = task_w(t);
#pragma unroll
    for (int s = 0; s < KC; ++s) {
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        G[s][g] = as_bf16x8(ld16_stream(pg + static_cast<size_t>(g * 8) * H + s * 64));
        UU[s][g] = as_bf16x8(ld16_stream(pg + up_off + static_cast<size_t>(g * 8) * H + s * 64));
      }
    }
    const uint32_t xo = itk * static_cast<uint32_t>(H) + kl + c * KC * 64;
#pragma unroll
    for (int s = 0; s < KC; ++s) XT[s] = as_bf16x8(ld16(x + xo + s * 64));
  };
  f32x4 ag[TM8][NG], au[TM8][NG];
  uint32_t tkp[(TM8 + 3) / 4];                      // lane's token per tile, packed bytes (T <= 64)
  int ntok = 0, tiles = 0, base = 0;

  // item epilogue: add the two half blocks, then the waves in order; SwiGLU,
  // routing weight, BF16 store.  `have` = this wave holds sums (else zeros).
  // One barrier per item: the buffer alternates, and a wave passes item j+1's
  // barrier only after every wave has finished reading item j's sums.
  auto epilogue = [&](int j, bool have) {
    int u, rb;
    item_of(j, u, rb);
    const int b0 = __builtin_amdgcn_readfirstlane(s_off[u]);
    const int nt = __builtin_amdgcn_readfirstlane(s_off[u + 1]) - b0, nq = (nt + 7) >> 3;
    float* rbuf = red + (j & 1) * (kDecWaves * TM8 * NG * 128);
    const bool wl = col < 8 && grp < 2;             // lanes holding the half-0 block
    const int li = c8 + 8 * grp;
#pragma unroll
    for (int q = 0; q < TM8; ++q) {
      if (q < nq) {
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          f32x4 vg = have ? ag[q][g] : f32x4{0.f, 0.f, 0.f, 0.f};
          f32x4 vu = have ? au[q][g] : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int r = 0; r < 4; ++r) {           // half-1 block sits 40 lanes up
            vg[r] += __shfl_down(vg[r], 40, kWave);
            vu[r] += __shfl_down(vu[r], 40, kWave);
          }
          if (wl) {
            float* dst = rbuf + (((wv * TM8 + q) * NG + g) * 2) * 64 + li;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              dst[r * 16] = vg[r];
              dst[64 + r * 16] = vu[r];
            }
          }
        }
      }
    }
    __syncthreads();
    // one element per thread (TM8 * 8 * NB <= 512): straight-line code, so the
    // compiler has no store loop to drain the weight loads in flight before
    static_assert(TM8 * 8 * NB <= kDecThreads, "one reduction element per thread");
    const int qq = threadIdx.x;
    if (qq < nq * 8 * NB) {
      const int q = qq / (8 * NB), within = qq - q * (8 * NB);
      const int n = within / NB, m = within - n * NB;   // token n of the tile, neuron m
      const int g = m >> 3, mm = m & 7;
      const int r = mm & 3, lsrc = n + 8 * (mm >> 2);
      float gs = 0.f, us = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < kDecWaves; ++w2) {
        const float* src = rbuf + (((w2 * TM8 + q) * NG + g) * 2) * 64 + r * 16 + lsrc;
        gs += src[0];
        us += src[64];
      }
      const int p = q * 8 + n;
      if (p < nt) {
        const int pr = s_pr[b0 + p];                 // pair t*k + j of this token and expert
        const float hv = s_w[b0 + p] * swiglu(gs, us);
        const uint16_t hb = static_cast<uint16_t>(f32_to_bf16_rne(hv));
        uint16_t* hp = hw + static_cast<size_t>(pr) * I + rb * NB + m;
        if constexpr (FUSED)    // device-coherent: read by other workgroups in this launch
          __hip_atomic_store(hp, hb, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else
          *hp = hb;
      }
    }
  };

  auto run_task = [&](const bf16x8 (&G)[KC][NG], const bf16x8 (&UU)[KC][NG],
                      const bf16x8 (&XT)[KC], int t) {
    const int j = t / nch, c = t - j * nch;
    if (c == 0) {
      int u, rb;
      item_of(j, u, rb);
      base = __builtin_amdgcn_readfirstlane(s_off[u]);
      ntok = __builtin_amdgcn_readfirstlane(s_off[u + 1]) - base;
      tiles = (ntok + 7) >> 3;
#pragma unroll
      for (int q = 0; q < (TM8 + 3) / 4; ++q) tkp[q] = 0;
#pragma unroll
      for (int q = 0; q < TM8; ++q) {
        const int p = 8 * q + c8;                   // past the end: a valid token, column discarded
        const uint32_t tk = static_cast<uint32_t>(s_pr[base + (p < ntok ? p : 0)] / k);
        tkp[q >> 2] |= tk << (8 * (q & 3));
#pragma unroll
        for (int g = 0; g < NG; ++g) ag[q][g] = au[q][g] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
#pragma unroll
    for (int q = 0; q < TM8; ++q) {
      if (q < tiles) {
        bf16x8 xb[KC];
        if (q == 0) {
#pragma unroll
          for (int s = 0; s < KC; ++s) xb[s] = XT[s];
        } else {                                    // later tiles: experts with over 8 tokens
          const uint32_t tk = (tkp[q >> 2] >> (8 * (q & 3))) & 0xFFu;
          const uint32_t xo = tk * static_cast<uint32_t>(H) + kl + c * KC * 64;
#pragma unroll
          for (int s = 0; s < KC; ++s) xb[s] = as_bf16x8(ld16(x + xo + s * 64));
        }
#pragma unroll
        for (int s = 0; s < KC; ++s) {
#pragma unroll
          for (int g = 0; g < NG; ++g) {
            ag[q][g] = mfma16x16x32(G[s][g], xb[s], ag[q][g]);
            au[q][g] = mfma16x16x32(UU[s][g], xb[s], au[q][g]);
          }
        }
      }
    }
    if (c == nch - 1) epilogue(j, true);
  };

  if (nch == 0) {                                   // no K steps for this wave (H < 512)
    for (int j = 0; j < my_items; ++j) epilogue(j, false);
  }
  // one task ahead: the loads of task t+1 are in flight while task t multiplies.
  // The steady-state loop issues unconditionally, so the compiler's waits leave
  // the next task's loads in flight.
  const int ntask = my_items * nch;
  if (ntask > 0) {
    issue(0, gA, uA, xA);
    int t = 0;
    for (; t + 2 < ntask; t += 2) {
      issue(t + 1, gB, uB, xB);
      run_task(gA, uA, xA, t);
      issue(t + 2, gA, uA, xA);
      run_task(gB, uB, xB, t + 1);
    }
    if (t + 1 < ntask) {
      issue(t + 1, gB, uB, xB);
      run_task(gA, uA, xA, t);
      run_task(gB, uB, xB, t + 1);
    } else {
      run_task(gA, uA, xA, t);
    }
  }
  if constexpr (FUSED) {
    // publish: every wave waits until its device-coherent activation stores are
    // complete, then one thread writes the flag (no L2-wide writeback needed)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0)
      __hip_atomic_store(flags + blockIdx.x, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int groups = H / kDownRows;
    if (static_cast<int>(blockIdx.x) >= groups) return;      // no output dimensions here
    __shared__ uint8_t s_tk[kMaxPairs];
    __shared__ int s_fail;
    for (int i = threadIdx.x; i < T * k; i += kDecThreads) s_tk[i] = static_cast<uint8_t>(s_pr[i] / k);
    GridWait gw{flags, epoch, static_cast<int>(gridDim.x), &s_fail};
    bool first = true;
    for (int dg0 = blockIdx.x; dg0 < groups; dg0 += gridDim.x) {
      const int dg = permute_item(dg0, groups, okey);
      __syncthreads();                              // the reduction buffer becomes accl
      if (first) {
        down_phase<KD, 1, NW, true>(wd, U, s_e, s_off, s_pr, s_tk, hw, T, H, I, KSW,
                                    dg * kDownRows, red, out, gw);
      } else {
        down_phase<KD, 1, NW, false>(wd, U, s_e, s_off, s_pr, s_tk, hw, T, H, I, KSW,
                                     dg * kDownRows, red, out, NoWait());
      }
      first = false;
      if (s_fail) {                                 // the wait gave up: no silent result
        for (int i = threadIdx.x; i < T * kDownRows; i += kDecThreads)
          out[static_cast<size_t>(i / kDownRows) * H + dg * kDownRows + i % kDownRows] = 0x7FC0;
      }
    }
  }
}

// gate_up for batches with many tokens per expert (T > 32): work item =
// (touched expert u, 16 neurons), MFMA rows = 16 neurons (gate and up
// separately), columns = 16 tokens, so an expert with up to 64 tokens takes
// four column tiles and each weight load serves 16 tokens per MFMA.  Each
// weight load reads 16 rows x 64 bytes, so the loads stay plain (the second
// half of each 128-byte line comes with the next step, from the cache).  Wave
// wv covers K range [wv*H/8, (wv+1)*H/8) in chunks of KC steps of 32; tasks
// and the one-ahead weight buffer as in the narrow kernel.
template <int KC>
__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(4, 8))) void decode_gate_up_wide(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wgu,
    const int32_t* __restrict__ idx, const float* __restrict__ wts, int T, int E,
    int* __restrict__ plan_u, int32_t* __restrict__ plan_e, int32_t* __restrict__ plan_off,
    uint16_t* __restrict__ plan_pr, int H, int I, int k, uint16_t* __restrict__ hw, uint32_t okey) {
  constexpr int TM = 4;                             // 16-token tiles (T <= 64)
  extern __shared__ float red[];                    // [8 waves][TM][gate/up][4][64]
  __shared__ int s_e[kMaxPlan];
  __shared__ int s_off[kMaxPlan + 1];
  __shared__ uint16_t s_pr[kMaxPairs];
  const int U = build_plan(idx, T, E, k, reinterpret_cast<uint64_t*>(red),
                           reinterpret_cast<int*>(reinterpret_cast<uint64_t*>(red) + E), s_e,
                           s_off, s_pr);
  if (blockIdx.x == 0) publish_plan(U, T * k, s_e, s_off, s_pr, plan_u, plan_e, plan_off, plan_pr);
  const int nrb = I / 16;
  const int items = U * nrb;
  const int wv = __builtin_amdgcn_readfirstlane(wave_id()), ln = lane_id();
  const int col = ln & 15, grp = ln >> 4;
  const int kw = H / kDecWaves;
  const int nch = kw / 32 / KC;                     // chunks per item
  const int my_items = blockIdx.x < items ? (items - 1 - blockIdx.x) / gridDim.x + 1 : 0;
  const int ntask = my_items * nch;
  const uint32_t kb = static_cast<uint32_t>(wv * kw + grp * 8);

  auto task_w = [&](int t) -> const uint16_t* {
    const int j = t / nch, c = t - j * nch;
    const int item = permute_item(blockIdx.x + j * gridDim.x, items, okey);
    const int u = item / nrb, rb = item - u * nrb;
    const int e = __builtin_amdgcn_readfirstlane(s_e[u]);
    return wgu + (static_cast<size_t>(e) * 2 * I + rb * 16 + col) * H + kb + c * KC * 32;
  };
  bf16x8 gA[KC], uA[KC], gB[KC], uB[KC];
  const size_t up_off = static_cast<size_t>(I) * H;
  auto issue = [&](int t, bf16x8 (&G)[KC], bf16x8 (&UU)[KC]) {
    const uint16_t* pg = task_w(t);
#pragma unroll
    for (int s = 0; s < KC; ++s) {
      G[s] = as_bf16x8(ld16(pg + s * 32));
      UU[s] = as_bf16x8(ld16(pg + up_off + s * 32));
    }
  };
  f32x4 ag[TM], au[TM];
  int tok[TM];
  int ntok = 0, tiles = 0;
  float wl[2];                                      // routing weights of this thread's two epilogue elements

  auto run_task = [&](const bf16x8 (&G)[KC], const bf16x8 (&UU)[KC], int t) {
    const int j = t / nch, c = t - j * nch;
    const int item = permute_item(blockIdx.x + j * gridDim.x, items, okey);
    const int u = item / nrb, rb = item - u * nrb;
    const int base = __builtin_amdgcn_readfirstlane(s_off[u]);
    if (c == 0) {
      ntok = __builtin_amdgcn_readfirstlane(s_off[u + 1]) - base;
      tiles = (ntok + 15) >> 4;
#pragma unroll
      for (int q = 0; q < TM; ++q) {
        const int p = 16 * q + col;
        tok[q] = s_pr[base + (p < ntok ? p : 0)] / k;   // past the end: a valid token, column discarded
        ag[q] = au[q] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      // loaded here, long before the epilogue needs them, so that waiting for them
      // does not wait for the weight loads issued in between
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int qq = threadIdx.x + h * kDecThreads;
        const int p = (qq >> 8) * 16 + ((qq & 255) >> 4);
        wl[h] = qq < tiles * 256 && p < ntok ? wts[s_pr[base + p]] : 0.f;
      }
    }
    const uint32_t ko = kb + c * KC * 32;
#pragma unroll
    for (int q = 0; q < TM; ++q) {
      if (q < tiles) {
        bf16x8 xb[KC];
#pragma unroll
        for (int s = 0; s < KC; ++s)
          xb[s] = as_bf16x8(ld16(x + static_cast<uint32_t>(tok[q] * H) + ko + s * 32));
#pragma unroll
        for (int s = 0; s < KC; ++s) {
          ag[q] = mfma16x16x32(G[s], xb[s], ag[q]);
          au[q] = mfma16x16x32(UU[s], xb[s], au[q]);
        }
      }
    }
    if (c != nch - 1) return;
    // epilogue of the item: fixed-order sum over waves, SwiGLU, weight, store
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
    // at most TM*256 = 1024 elements: two per thread, unrolled (no store loop)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int qq = threadIdx.x + h * kDecThreads;
      if (qq < tiles * 256) {
        const int q = qq >> 8, within = qq & 255;
        const int n = within >> 4, m = within & 15;  // token column n, weight row m
        const int src = 16 * (m >> 2) + n, r = m & 3;
        float g = 0.f, up = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < kDecWaves; ++w2) {
          g += red[(((w2 * TM + q) * 2 + 0) * 4 + r) * 64 + src];
          up += red[(((w2 * TM + q) * 2 + 1) * 4 + r) * 64 + src];
        }
        const int p = q * 16 + n;
        if (p < ntok) {
          const int pr = s_pr[base + p];
          const float hv = wl[h] * swiglu(g, up);
          hw[static_cast<size_t>(pr) * I + rb * 16 + m] = static_cast<uint16_t>(f32_to_bf16_rne(hv));
        }
      }
    }
    __syncthreads();
  };

  if (ntask > 0) issue(0, gA, uA);
  for (int t = 0; t < ntask; t += 2) {
    if (t + 1 < ntask) issue(t + 1, gB, uB);
    run_task(gA, uA, t);
    if (t + 1 < ntask) {
      if (t + 2 < ntask) issue(t + 2, gA, uA);
      run_task(gB, uB, t + 1);
    }
  }
}

// gate_up for T > 32 with whole-line weight loads (H a multiple of 512): the
// same items, MFMA layout (16 neurons x 16 tokens), tiles and epilogue as
// decode_gate_up_wide, but each task is one 64-position step of the wave's K
// range, and its 16 gate and 16 up rows are read with four loads of 8 rows x
// 128 contiguous bytes (non-temporal), written to a wave-private LDS tile and
// read back in the MFMA layout.  The tile lives in the wave's own slice of the
// reduction buffer: a wave writes that slice only for its own tasks or its own
// partial sums, and the other waves read it only between the epilogue's two
// barriers.  16-byte chunks are XOR-swizzled by row, so the column reads (one
// row per lane) hit distinct banks.
__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(4, 8))) void decode_gate_up_wide_stream(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wgu,
    const int32_t* __restrict__ idx, const float* __restrict__ wts, int T, int E,
    int* __restrict__ plan_u, int32_t* __restrict__ plan_e, int32_t* __restrict__ plan_off,
    uint16_t* __restrict__ plan_pr, int H, int I, int k, uint16_t* __restrict__ hw, uint32_t okey) {
  constexpr int TM = 4;                             // 16-token tiles (T <= 64)
  constexpr int kSlice = TM * 2 * 4 * 64;           // floats per wave in the reduction buffer
  extern __shared__ float red[];                    // [8 waves][TM][gate/up][4][64]
  __shared__ int s_e[kMaxPlan];
  __shared__ int s_off[kMaxPlan + 1];
  __shared__ uint16_t s_pr[kMaxPairs];
  const int U = build_plan(idx, T, E, k, reinterpret_cast<uint64_t*>(red),
                           reinterpret_cast<int*>(reinterpret_cast<uint64_t*>(red) + E), s_e,
                           s_off, s_pr);
  if (blockIdx.x == 0) publish_plan(U, T * k, s_e, s_off, s_pr, plan_u, plan_e, plan_off, plan_pr);
  const int nrb = I / 16;
  const int items = U * nrb;
  const int wv = __builtin_amdgcn_readfirstlane(wave_id()), ln = lane_id();
  const int col = ln & 15, grp = ln >> 4;
  const int kw = H / kDecWaves;                     // a multiple of 64
  const int nch = kw / 64;                          // tasks (steps of 64) per item
  const int my_items = blockIdx.x < items ? (items - 1 - blockIdx.x) / gridDim.x + 1 : 0;
  const int ntask = my_items * nch;
  // whole-line loads: lane = (row ln/8 of an 8-row group, 16-byte chunk ln%8)
  const int lr = ln >> 3, lc = ln & 7;
  const uint32_t wl_off = static_cast<uint32_t>(lr * H + wv * kw + lc * 8);
  i32x4* tilep = reinterpret_cast<i32x4*>(red + wv * kSlice);   // [gate/up][16 rows][8 chunks]
  i32x4* wdst = tilep + lr * 8 + (lc ^ lr);        // + (mat*16 + 8*half) * 8
  // MFMA A lane (row col, group grp), 32-step s2: chunk 4*s2 + grp of row col
  const i32x4* asrc = tilep + col * 8;
  const size_t up_off = static_cast<size_t>(I) * H;
  const uint32_t kb = static_cast<uint32_t>(wv * kw + grp * 8);  // activation lane offset

  i32x4 wA[4], wB[4];                               // [gate/up][row half] whole-line loads
  uint32_t itk = 0;                                 // this lane's first-tile token, load side
  // weights of task t
  auto issue = [&](int t, i32x4 (&W)[4]) {
    const int j = t / nch, c = t - j * nch;
    const int item = permute_item(blockIdx.x + j * gridDim.x, items, okey);
    const int u = item / nrb, rb = item - u * nrb;
    const int e = __builtin_amdgcn_readfirstlane(s_e[u]);
    const uint16_t* pw = wgu + (static_cast<size_t>(e) * 2 * I + rb * 16) * H + wl_off + c * 64;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        W[2 * m + hh] = ld16_stream(pw + m * up_off + static_cast<size_t>(8 * hh) * H);
  };
  float wl[2];                                       // routing weights of this thread's two epilogue elements
  // first token tile's activations of task t (both 32-steps), and at an item's
  // first task the routing weights its epilogue needs; issued before the next
  // task's weights, so that waiting for them leaves those in flight
  auto load_x0 = [&](int t, bf16x8 (&XT)[2]) {
    const int j = t / nch, c = t - j * nch;
    if (c == 0) {
      const int item = permute_item(blockIdx.x + j * gridDim.x, items, okey);
      const int u = item / nrb;
      const int b = __builtin_amdgcn_readfirstlane(s_off[u]);
      const int n = __builtin_amdgcn_readfirstlane(s_off[u + 1]) - b;
      itk = static_cast<uint32_t>(s_pr[b + (col < n ? col : 0)] / k);
      const int nq = (n + 15) >> 4;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int qq = threadIdx.x + h * kDecThreads;
        const int p = (qq >> 8) * 16 + ((qq & 255) >> 4);
        wl[h] = qq < nq * 256 && p < n ? wts[s_pr[b + p]] : 0.f;
      }
    }
    const uint32_t xo = itk * static_cast<uint32_t>(H) + kb + c * 64;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) XT[s2] = as_bf16x8(ld16(x + xo + s2 * 32));
  };
  f32x4 ag[TM], au[TM];
  uint32_t tkp = 0;                                 // this lane's token per tile, packed bytes
  int ntok = 0, tiles = 0;

  auto run_task = [&](const i32x4 (&W)[4], const bf16x8 (&XT)[2], int t) {
    const int j = t / nch, c = t - j * nch;
    const int item = permute_item(blockIdx.x + j * gridDim.x, items, okey);
    const int u = item / nrb, rb = item - u * nrb;
    const int base = __builtin_amdgcn_readfirstlane(s_off[u]);
    if (c == 0) {
      ntok = __builtin_amdgcn_readfirstlane(s_off[u + 1]) - base;
      tiles = (ntok + 15) >> 4;
      tkp = 0;
#pragma unroll
      for (int q = 0; q < TM; ++q) {
        const int p = 16 * q + col;                 // past the end: a valid token, column discarded
        tkp |= static_cast<uint32_t>(s_pr[base + (p < ntok ? p : 0)] / k) << (8 * q);
        ag[q] = au[q] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
    // whole-line weights -> LDS tile -> MFMA layout
#pragma unroll
    for (int i = 0; i < 4; ++i) wdst[i * 64] = W[i];   // (mat*16 + 8*half) rows = 8i rows
    __builtin_amdgcn_wave_barrier();
    bf16x8 ga[2], ua[2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int ch = (4 * s2 + grp) ^ (col & 7);
      ga[s2] = as_bf16x8(asrc[ch]);
      ua[s2] = as_bf16x8(asrc[16 * 8 + ch]);
    }
    __builtin_amdgcn_wave_barrier();
    const uint32_t ko = kb + c * 64;
#pragma unroll
    for (int q = 0; q < TM; ++q) {
      if (q < tiles) {
        bf16x8 xb[2];
        if (q == 0) {
          xb[0] = XT[0];
          xb[1] = XT[1];
        } else {                                    // later tiles: experts with over 16 tokens
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2)
            xb[s2] = as_bf16x8(ld16(x + ((tkp >> (8 * q)) & 0xFFu) * static_cast<uint32_t>(H) + ko + s2 * 32));
        }
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          ag[q] = mfma16x16x32(ga[s2], xb[s2], ag[q]);
          au[q] = mfma16x16x32(ua[s2], xb[s2], au[q]);
        }
      }
    }
    if (c != nch - 1) return;
    // epilogue of the item: fixed-order sum over waves, SwiGLU, weight, store
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
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int qq = threadIdx.x + h * kDecThreads;
      if (qq < tiles * 256) {
        const int q = qq >> 8, within = qq & 255;
        const int n = within >> 4, m = within & 15;  // token column n, weight row m
        const int src = 16 * (m >> 2) + n, r = m & 3;
        float g = 0.f, up = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < kDecWaves; ++w2) {
          g += red[(((w2 * TM + q) * 2 + 0) * 4 + r) * 64 + src];
          up += red[(((w2 * TM + q) * 2 + 1) * 4 + r) * 64 + src];
        }
        const int p = q * 16 + n;
        if (p < ntok) {
          const int pr = s_pr[base + p];
          const float hv = wl[h] * swiglu(g, up);
          hw[static_cast<size_t>(pr) * I + rb * 16 + m] = static_cast<uint16_t>(f32_to_bf16_rne(hv));
        }
      }
    }
    __syncthreads();
  };

  // one task ahead; the steady-state loop issues unconditionally, so the
  // compiler's waits leave the next task's weights in flight
  bf16x8 x0[2];
  if (ntask > 0) {
    issue(0, wA);
    int t = 0;
    for (; t + 2 < ntask; t += 2) {
      load_x0(t, x0);
      issue(t + 1, wB);
      run_task(wA, x0, t);
      load_x0(t + 1, x0);
      issue(t + 2, wA);
      run_task(wB, x0, t + 1);
    }
    load_x0(t, x0);
    if (t + 1 < ntask) {
      issue(t + 1, wB);
      run_task(wA, x0, t);
      load_x0(t + 1, x0);
      run_task(wB, x0, t + 1);
    } else {
      run_task(wA, x0, t);
    }
  }
}

// dynamic LDS of decode_down<KD, NR>
inline size_t down_lds_bytes(int T, int KD, int NR) {
  const int stage = KD == 3 ? DownGeom<3>::kStage
                  : KD == 4 ? DownGeom<4>::kStage
                  : KD == 5 ? DownGeom<5>::kStage : DownGeom<7>::kStage;
  return sizeof(float) * kDownWaves * T * kDownRows * NR + sizeof(i32x4) * kDownWaves * stage;
}

// dynamic LDS of decode_gate_up<TM8, NG, KC>: two buffers of per-wave reduction sums
inline size_t gate_up_lds_bytes(int TM8, int NG) {
  return 2 * sizeof(float) * kDecWaves * TM8 * NG * 2 * 4 * 16;
}

// dynamic LDS of the down phase with nw waves
inline size_t down_lds_bytes_w(int T, int KD, int NR, int nw) {
  const int stage = KD == 3 ? DownGeom<3>::kStage
                  : KD == 4 ? DownGeom<4>::kStage
                  : KD == 5 ? DownGeom<5>::kStage : DownGeom<7>::kStage;
  return sizeof(float) * nw * T * kDownRows * NR + sizeof(i32x4) * nw * stage;
}

// The single-launch decode kernel for a configuration (T <= 16: TM8 <= 2; down
// slices of KD = 3 or 4 steps, i.e. I/64 = 3 or 4 times a power of two up to 8:
// the 5- and 7-step slices do not fit the registers beside the gate_up phase).
const void* fused_kernel(int TM8, int NG, int KC, int KD) {
#define FK(TMV, NGV, KCV, KDV) \
  reinterpret_cast<const void*>(decode_gate_up<TMV, NGV, KCV, kDecWaves, true, KDV>)
#define FK_KD(TMV, NGV, KCV) (KD == 3 ? FK(TMV, NGV, KCV, 3) : FK(TMV, NGV, KCV, 4))
  if (TM8 == 1 && NG == 2) return KC == 2 ? FK_KD(1, 2, 2) : FK_KD(1, 2, 1);
  if (TM8 == 1) return KC == 2 ? FK_KD(1, 1, 2) : FK_KD(1, 1, 1);
  if (NG == 2) return FK_KD(2, 2, 1);
  return FK_KD(2, 1, 1);
#undef FK_KD
#undef FK
}

// Resident workgroups per CU of a kernel (cached per kernel and LDS size; also
// raises the kernel's dynamic LDS limit when it needs more than the default).
hipError_t fused_occupancy(const void* fn, size_t lds, int* bpc) {
  static std::mutex mu;
  static std::map<std::pair<const void*, size_t>, int> cache;
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_pair(fn, lds);
  auto it = cache.find(key);
  if (it != cache.end()) {
    *bpc = it->second;
    return hipSuccess;
  }
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(lds));
  if (e != hipSuccess) return e;
  int n = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, kDecThreads, lds);
  if (e != hipSuccess) return e;
  cache[key] = n;
  *bpc = n;
  return hipSuccess;
}

// A 64-bit value unique to each single-launch decode of this process: the
// workgroups' ready flags carry it, so flags of an earlier launch (or whatever
// a fresh workspace holds, short of a 2^-64 coincidence) never read as ready.
uint64_t next_epoch() {
  static std::atomic<uint64_t> ctr{[] {
    std::random_device rd;
    return ((static_cast<uint64_t>(rd()) << 32) ^ rd()) | 1u;
  }()};
  return ctr.fetch_add(1, std::memory_order_relaxed);
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

  // T <= 16: the gate_up kernel routes the tokens itself; otherwise a routing launch first
  const bool wide = T > 32;
  const int fuse_route = T <= 16;
  if (!fuse_route) {
    const hipError_t err = launch_route_topk(logits, T, E, k, idx_p, w_p, s);   // brackets kRoute
    if (err != hipSuccess) return err;
  }

  // gate_up: T <= 32 takes the narrow kernel (8-token tiles, full-line streamed
  // weights); T > 32 the wide one (16-token tiles)
  const int TM8 = T <= 8 ? 1 : (T <= 16 ? 2 : 4);
  // register budget (128 per lane): weights of two tasks + 16*NG accumulators per tile;
  // one 8-neuron group per item when 16-neuron items would number fewer than sixteen
  // per CU (T <= 10: e.g. T = 8, ~52 touched experts x 48 items): the persistent
  // workgroups then hold about twice as many items, which evens out the last round
  const long pairs_u = T * k < E ? T * k : E;
  const int NG = TM8 <= 2 && pairs_u * (I / 16) >= 16L * num_cus ? 2 : 1;
  const int S = H / 64;                             // a multiple of 4
  // two steps per chunk when every wave's step count is even and registers allow
  const int KC = (S % 16 == 0 && (TM8 == 1 || TM8 == 4)) ? 2 : 1;
  const int gsteps = H / kDecWaves / 32;            // wide kernel: steps of 32 per wave
  const int KCW = gsteps % 2 == 0 ? 2 : 1;
  const long items_upper = pairs_u * (I / (wide ? 16 : 8 * NG));
  const long grid_cap = 2L * num_cus;
  const int grid1 = static_cast<int>(items_upper < grid_cap ? items_upper : grid_cap);
  // reduction buffer; the plan scratch (E masks + chunk offsets) must fit in it too;
  // the narrow kernel keeps its routing result past both
  size_t lds_gu = wide ? sizeof(float) * kDecWaves * 4 * 2 * 256 : gate_up_lds_bytes(TM8, NG);
  const size_t lds_plan = sizeof(uint64_t) * E + sizeof(int) * (E + 33);
  if (lds_plan > lds_gu) lds_gu = lds_plan;
  const int route_off = static_cast<int>((lds_gu + 15) / 16 * 16);
  if (!wide) lds_gu = route_off + static_cast<size_t>(T) * k * (sizeof(int32_t) + sizeof(float));
  // down: K-slices per workgroup (a power of two, so that the 16 waves split into
  // expert groups), the fewest that leave each wave at most 4 steps of 64; I is a
  // multiple of 256 up to 2048, so I/64 is 4, 8, ..., 32, and the two sizes with no
  // such split (I = 1280, 1792) take 4 slices of 5 or 7 steps
  const int dtotal = I / 64;
  int KSW = 1;
  while (KSW < 8 && (dtotal / KSW > 4 || dtotal % KSW)) KSW *= 2;
  if (dtotal % KSW) KSW = 4;
  const int KD = dtotal / KSW;
  // 16 dimensions per workgroup when that still leaves a workgroup per CU (the
  // activations are re-read by every workgroup)
  // (the 5- and 7-step slices keep one group: two would not fit 128 registers)
  const int NR = H / (2 * kDownRows) >= num_cus && KD <= 4 ? 2 : 1;
  const size_t lds_dn = down_lds_bytes(T, KD, NR);
  // The single launch waits on flags compared with a per-launch epoch passed as a
  // kernel argument; a captured graph would replay one epoch, and the flags of
  // the previous replay would already match.  Under stream capture the two
  // launches run instead.
  hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &capture) != hipSuccess) capture = hipStreamCaptureStatusActive;
  if (fuse_route && !wide && (KD == 3 || KD == 4) && capture == hipStreamCaptureStatusNone &&
      (debug_options().flags & kDebugDecodeFused)) {
    // single launch: routing, gate_up and down in one grid of resident workgroups
    uint64_t* flags = reinterpret_cast<uint64_t*>(base + L.flags);
    const size_t lds_f = std::max(lds_gu, down_lds_bytes_w(T, KD, 1, kDecWaves));
    const void* fn = fused_kernel(TM8, NG, KC, KD);
    int bpc = 0;
    hipError_t err = fused_occupancy(fn, lds_f, &bpc);
    if (err != hipSuccess) return err;
    if (bpc >= 1) {
      const int per_cu = bpc < 2 ? bpc : 2;
      int grid = per_cu * num_cus;
      if (grid > kMaxDecodeGrid) grid = kMaxDecodeGrid;
      uint64_t epoch = next_epoch();
      int KSWv = KSW;
      const uint16_t* wd_p = wd;
      uint32_t okey = order_key();
      void* args[] = {const_cast<uint16_t**>(&x), const_cast<uint16_t**>(&wgu),
                      const_cast<float**>(&logits), &idx_p, &w_p, &T, &E, &plan_u, &plan_e,
                      &plan_off, &plan_pr, &H, &I, &k, &hw, const_cast<int*>(&route_off),
                      const_cast<int*>(&fuse_route), const_cast<uint16_t**>(&wd_p), &out, &flags,
                      &epoch, &KSWv, &okey};
      prof_begin(kDecFused, s);
      err = hipLaunchKernel(fn, dim3(grid), dim3(kDecThreads), args, static_cast<unsigned>(lds_f), s);
      prof_end(kDecFused, s);
      if (err != hipSuccess) return err;
      return hipGetLastError();
    }
    // (no residency for the fused kernel: the two-launch path below)
  }
  prof_begin(kDecGateUp, s);
#define GU_LAUNCH(TMV, NGV, KCV)                                                               \
  hipLaunchKernelGGL((decode_gate_up<TMV, NGV, KCV>), dim3(grid1), dim3(kDecThreads), lds_gu, s, \
                     x, wgu, logits, idx_p, w_p, T, E, plan_u, plan_e, plan_off, plan_pr, H, I, \
                     k, hw, route_off, fuse_route, nullptr, nullptr, nullptr, uint64_t{0}, 0, order_key())
#define GU_WIDE(KCV)                                                                            \
  hipLaunchKernelGGL((decode_gate_up_wide<KCV>), dim3(grid1), dim3(kDecThreads), lds_gu, s, x, wgu, \
                     idx_p, w_p, T, E, plan_u, plan_e, plan_off, plan_pr, H, I, k, hw, order_key())
  if (wide && H % 512 == 0) {
    hipLaunchKernelGGL(decode_gate_up_wide_stream, dim3(grid1), dim3(kDecThreads), lds_gu, s, x, wgu,
                       idx_p, w_p, T, E, plan_u, plan_e, plan_off, plan_pr, H, I, k, hw, order_key());
  } else if (wide) {
    if (KCW == 2) GU_WIDE(2); else GU_WIDE(1);
  } else if (TM8 == 1 && NG == 2) {
    if (KC == 2) GU_LAUNCH(1, 2, 2); else GU_LAUNCH(1, 2, 1);
  } else if (TM8 == 1) {
    if (KC == 2) GU_LAUNCH(1, 1, 2); else GU_LAUNCH(1, 1, 1);
  } else if (TM8 == 2 && NG == 2) {
    GU_LAUNCH(2, 2, 1);
  } else if (TM8 == 2) {
    GU_LAUNCH(2, 1, 1);
  } else {
    if (KC == 2) GU_LAUNCH(4, 1, 2); else GU_LAUNCH(4, 1, 1);
  }
#undef GU_WIDE
#undef GU_LAUNCH
  prof_end(kDecGateUp, s);
  prof_begin(kDecDown, s);
#define DN_LAUNCH(KDV, NRV)                                                                    \
  hipLaunchKernelGGL((decode_down<KDV, NRV>), dim3(H / (kDownRows * NRV)), dim3(kDownThreads),    \
                     lds_dn, s, wd, plan_u, plan_e, plan_off, plan_pr, hw, T, H, I, k, KSW, out, order_key())
#define DN_NR(KDV) \
  if (NR == 2) DN_LAUNCH(KDV, 2); else DN_LAUNCH(KDV, 1);
  switch (KD) {
    case 3: DN_NR(3) break;
    case 4: DN_NR(4) break;
    case 5: DN_LAUNCH(5, 1); break;
    case 7: DN_LAUNCH(7, 1); break;
    default: return hipErrorInvalidValue;            // not reachable for valid I
  }
#undef DN_NR
#undef DN_LAUNCH
  prof_end(kDecDown, s);
  return hipGetLastError();
}

hipError_t decode_set_attributes() {
  hipError_t e = hipSuccess;
  // down at T = 64: accumulators plus the staging tiles exceed 64 KB
  const void* dn[] = {reinterpret_cast<const void*>(decode_down<3, 1>),
                      reinterpret_cast<const void*>(decode_down<4, 1>),
                      reinterpret_cast<const void*>(decode_down<5, 1>),
                      reinterpret_cast<const void*>(decode_down<7, 1>),
                      reinterpret_cast<const void*>(decode_down<3, 2>),
                      reinterpret_cast<const void*>(decode_down<4, 2>)};
  const int kds[] = {3, 4, 5, 7, 3, 4}, nrs[] = {1, 1, 1, 1, 2, 2};
  for (int i = 0; i < 6; ++i) {
    e = hipFuncSetAttribute(dn[i], hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(down_lds_bytes(64, kds[i], nrs[i])));
    if (e != hipSuccess) return e;
  }
  return e;
}

}  // namespace moe
