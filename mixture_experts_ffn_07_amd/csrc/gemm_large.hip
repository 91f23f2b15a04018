// Grouped GEMMs for experts that receive many routed rows (hundreds to
// thousands per expert, e.g. one GPU's expert-parallel share of a 2,048
// tokens-per-GPU batch: 64 ranks x 2,048 tokens x top-8 over 384 experts puts
// ~2,731 rows on each of 6 local experts; Mixture-of-Kittens summary, "What is
// 2.37x measured against").  At that size the projections are bound by the
// matrix cores, not by HBM, so the design is the classic LDS-tiled GEMM:
//
//   workgroup tile  256 rows x 256 output columns, K in stages of 64
//                   (gate_up: 128 gate + 128 up neurons of one expert, so the
//                   SwiGLU epilogue finds g and u in the same lane)
//   waves           4 (2 x 2), each 128 x 128 with v_mfma_f32_32x32x16_bf16,
//                   accumulators in AGPRs (256 per lane)
//   operands        both tiles staged in LDS (2 stages x 2 x 32 KB, XOR
//                   swizzled 16-byte chunks: no bank conflicts on the
//                   fragment reads); global loads go through VGPRs one stage
//                   ahead of the LDS writes, which run one stage ahead of the
//                   fragment reads
//   schedule        each MFMA K step interleaves its 16 MFMAs with the next
//                   fragment reads and with the LDS write + global load of the
//                   stage after next, in a fixed order (sched_barrier groups);
//                   one workgroup barrier per stage
//
// LDS writes are the scarce resource on gfx950 (about a quarter of the read
// bandwidth), which is why the tile is as large as the register file allows:
// every staged byte feeds 128 MFMA columns.
#include "common.h"
#include "internal.h"
#include "tiles.h"

namespace moe {

namespace {
constexpr int kLBK = 64;                     // K per stage
constexpr int kLTile = kLargeBM * kLBK;      // elements per operand stage (256 rows x 64)
constexpr size_t kLLds = 2 * 2 * kLTile * sizeof(uint16_t);   // 128 KB
enum { kGateUp = 0, kDownFused = 1, kDownSlots = 2 };

// Tail split.  One workgroup fills a CU, so n items run in ceil(n / ncu)
// rounds; when the last round would leave more than half of the CUs idle, its
// items are cut along K into S slices that run side by side.  Each slice
// writes its FP32 partial tile to the workspace and gemm_large_fixup adds the
// S partials of an item in slice order (fixed, so results stay bit-identical
// run to run) before the usual epilogue.  Items before `full` run whole.
struct TailPlan {
  int full, rem, S;
};
__device__ __forceinline__ TailPlan tail_plan(int n_real, int ncu, int nk) {
  TailPlan p;
  const int rounds = n_real / ncu;
  p.rem = n_real - rounds * ncu;
  p.S = 1;
  if (p.rem > 0 && 2 * p.rem <= ncu && ncu % kXcds == 0)
    p.S = max(1, min(min(8, ncu / p.rem), min(nk / 2, kLargeMaxSlices / p.rem)));
  p.full = p.S > 1 ? rounds * ncu : n_real;
  return p;
}

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// s_waitcnt with only the LDS/scalar counter constrained to 0
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
}  // namespace

// Epilogue of a 256 x 256 tile (see gemm_large_bf16 for the register layout).
template <int KIND>
__device__ __forceinline__ void large_epilogue(const f32x16 (&acc)[4][4], const int* __restrict__ perm,
                                               const float* __restrict__ w, int H, int I, int rbase,
                                               int mcount, int nb, int wm, int wn, int l32, int hi,
                                               uint16_t* __restrict__ hout, float* __restrict__ y,
                                               uint16_t* __restrict__ out) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = wm * 128 + 32 * j + l32;
    if (r >= mcount) continue;
    if (KIND == kGateUp) {
      uint16_t* hr = hout + static_cast<size_t>(rbase + r) * I + nb * 128 + wn * 64 + 4 * hi;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint32_t p[4];
#pragma unroll
          for (int t = 0; t < 4; ++t)
            p[t] = f32_to_bf16_rne(swiglu(acc[i][j][4 * q + t], acc[i + 2][j][4 * q + t]));
          *reinterpret_cast<uint2*>(hr + 32 * i + 8 * q) = make_uint2(p[0] | (p[1] << 16), p[2] | (p[3] << 16));
        }
    } else if (KIND == kDownFused) {
      const int t = perm[rbase + r];        // k = 1: pair id == token
      const float wt_t = w[t];
      uint16_t* orow = out + static_cast<size_t>(t) * H + nb * 256 + wn * 128 + 4 * hi;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint32_t p[4];
#pragma unroll
          for (int t4 = 0; t4 < 4; ++t4) p[t4] = f32_to_bf16_rne(wt_t * acc[i][j][4 * q + t4]);
          *reinterpret_cast<uint2*>(orow + 32 * i + 8 * q) = make_uint2(p[0] | (p[1] << 16), p[2] | (p[3] << 16));
        }
    } else {
      float* yr = y + static_cast<size_t>(rbase + r) * H + nb * 256 + wn * 128 + 4 * hi;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<f32x4*>(yr + 32 * i + 8 * q) =
              f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
    }
  }
}

// KIND kGateUp:    act = x [T,H], wt = W_gate_up [E,2I,H]; writes h [P,I] (sorted rows, BF16).
// KIND kDown*:     act = h [P,I] (sorted rows), wt = W_down [E,H,I]; kDownFused (k = 1)
//                  writes out[t] = bf16(w[t] * y), kDownSlots writes y [P,H] FP32 (sorted rows).
// MFMA operands: A = weight rows (D rows), B = activation rows (D columns).  The
// 32x32x16 result puts, in lane (l32, hi) register 4q+t, weight row 8q + 4hi + t
// and activation row l32 of the 32 x 32 block.  Within each stage of 64, lane
// half hi takes K chunks 2*ks + hi at MFMA K step ks (the same for A and B).
template <int KIND>
__global__ __launch_bounds__(256) void gemm_large_bf16(
    const uint16_t* __restrict__ act, const uint16_t* __restrict__ wt,
    const int* __restrict__ perm, const int2* __restrict__ tiles, const int* __restrict__ n_tiles,
    const int* __restrict__ counts, const int* __restrict__ offsets, const float* __restrict__ w,
    int H, int I, int k, uint16_t* __restrict__ hout, float* __restrict__ y,
    uint16_t* __restrict__ out, float* __restrict__ partial, int ncu) {
  extern __shared__ __align__(16) uint16_t lds[];   // [stage][A, B][256 x 64]
  constexpr bool kGU = KIND == kGateUp;
  const int K = kGU ? H : I;
  const int nblk = kGU ? I / 128 : H / 256;
  const int nk = K / kLBK;
  const int n_real = nblk * *n_tiles;
  const TailPlan plan = tail_plan(n_real, ncu, nk);
  const int L = blockIdx.x;
  int item, kb = 0, ke = nk, slot = -1;
  if (plan.S > 1 && L < plan.full) {
    item = xcd_item(L, plan.full);
  } else if (plan.S > 1) {
    const int t = L - plan.full;
    if (t >= plan.rem * plan.S) return;
    item = plan.full + t % plan.rem;
    const int sl = t / plan.rem;
    kb = sl * nk / plan.S;
    ke = (sl + 1) * nk / plan.S;
    slot = t;
  } else {
    item = real_item(L, nblk, *n_tiles);
    if (item < 0) return;
  }
  const int tile = item / nblk, nb = item - tile * nblk;
  const int2 te = tiles[tile];
  const int e = te.x, m0 = te.y;
  const int mcount = min(kLargeBM, counts[e] - m0);
  const int rbase = offsets[e] + m0;
  const int tid = threadIdx.x, wv = tid >> 6, ln = tid & 63, l32 = ln & 31, hi = ln >> 5;
  const int wm = wv & 1, wn = wv >> 1;

  // Loader: thread covers tile rows wv*64 + 8j + (ln >> 3), j = 0..7, of both
  // operands, 16-byte chunk ln & 7 of each 128-byte row segment.  Rows past the
  // tile's end load the tile's first row (their columns are discarded).
  const int lrow = ln >> 3, lc = ln & 7;
  const uint16_t* __restrict__ abase;
  uint32_t ao;
  if (kGU) {
    const int n0 = nb * 128;
    abase = wt + static_cast<size_t>(e) * 2 * I * H;
    // tile rows 0..127: gate neurons n0.., rows 128..255: up neurons n0..
    ao = static_cast<uint32_t>(((wv < 2 ? n0 + wv * 64 : I + n0 + (wv - 2) * 64) + lrow) * H + lc * 8);
  } else {
    abase = wt + static_cast<size_t>(e) * H * I;
    ao = static_cast<uint32_t>((nb * 256 + wv * 64 + lrow) * I + lc * 8);
  }
  uint32_t bo[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = wv * 64 + 8 * j + lrow;
    const int rr = r < mcount ? r : 0;
    bo[j] = kGU ? static_cast<uint32_t>((perm[rbase + rr] / k) * H + lc * 8)
                : static_cast<uint32_t>((rbase + rr) * I + lc * 8);
  }
  // LDS: row r, 16-byte chunk c at r*64 + ((c ^ (r & 7)) * 8); here r & 7 == lrow
  const int lw = (wv * 64 + lrow) * kLBK + ((lc ^ lrow) * 8);
  // fragment rows of this wave
  int fa[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    fa[i] = ((kGU ? (i >> 1) * 128 + wn * 64 + (i & 1) * 32 : wn * 128 + 32 * i) + l32) * kLBK;
  const int fb = (wm * 128 + l32) * kLBK;
  const int swz = l32 & 7;

  i32x4 stg[16];   // [0..7] weight rows, [8..15] activation rows
#define GLOAD(Q, KT) do {                                                               \
    const uint32_t kk_ = static_cast<uint32_t>(min((KT), ke - 1) * kLBK);               \
    if ((Q) < 8) stg[Q] = ld16(abase + ao + static_cast<uint32_t>((Q) * 8) * K + kk_);  \
    else stg[Q] = ld16(act + bo[(Q) - 8] + kk_);                                        \
  } while (0)
#define LWRITE(Q, KT) do {                                                              \
    uint16_t* st_ = lds + ((KT) & 1) * 2 * kLTile;                                      \
    if ((Q) < 8) *reinterpret_cast<i32x4*>(&st_[lw + (Q) * 8 * kLBK]) = stg[Q];         \
    else *reinterpret_cast<i32x4*>(&st_[kLTile + lw + ((Q) - 8) * 8 * kLBK]) = stg[Q];  \
  } while (0)
#define RDF(PTR) as_bf16x8(*reinterpret_cast<const i32x4*>(PTR))
  // One MFMA K step on fragments (A, B): 8 groups of 2 MFMAs; group g then
  // reads fragment g of the next K step (stage RKT, step RKS) and, for g < NQ,
  // writes staged chunk Q0+g of stage KT+1 to LDS and reloads that chunk from
  // stage KT+2.  sched_barrier keeps this order.
#define PHASE(A, B, NA, NB, RKT, RKS, KT, Q0, NQ) do {                                  \
    const uint16_t* at_ = lds + ((RKT) & 1) * 2 * kLTile;                               \
    const uint16_t* bt_ = at_ + kLTile;                                                 \
    const int so_ = (((2 * (RKS) + hi) ^ swz) * 8);                                     \
    _Pragma("unroll") for (int g = 0; g < 8; ++g) {                                     \
      const int i_ = g >> 1, j0_ = (g & 1) * 2;                                         \
      acc[i_][j0_] = mfma32x32x16(A[i_], B[j0_], acc[i_][j0_]);                         \
      acc[i_][j0_ + 1] = mfma32x32x16(A[i_], B[j0_ + 1], acc[i_][j0_ + 1]);             \
      __builtin_amdgcn_sched_barrier(0);                                                \
      if (g < 4) NA[g] = RDF(&at_[fa[g] + so_]);                                        \
      else NB[g - 4] = RDF(&bt_[fb + 32 * (g - 4) * kLBK + so_]);                       \
      if (g < (NQ)) { LWRITE((Q0) + g, (KT) + 1); GLOAD((Q0) + g, (KT) + 2); }          \
      __builtin_amdgcn_sched_barrier(0);                                                \
    }                                                                                   \
  } while (0)

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
  // prologue: stage 0 into LDS buffer 0, stage 1 into the staging registers
#pragma unroll
  for (int q = 0; q < 16; ++q) GLOAD(q, kb);
#pragma unroll
  for (int q = 0; q < 16; ++q) LWRITE(q, kb);
#pragma unroll
  for (int q = 0; q < 16; ++q) GLOAD(q, kb + 1);
  __syncthreads();
  bf16x8 a0[4], b0[4], a1[4], b1[4];
  {
    const uint16_t* at = lds + (kb & 1) * 2 * kLTile;
    const int so = (hi ^ swz) * 8;
#pragma unroll
    for (int g = 0; g < 4; ++g) a0[g] = RDF(&at[fa[g] + so]);
#pragma unroll
    for (int g = 0; g < 4; ++g) b0[g] = RDF(&at[kLTile + fb + 32 * g * kLBK + so]);
  }
  for (int kt = kb; kt < ke; ++kt) {
    PHASE(a0, b0, a1, b1, kt, 1, kt, 0, 6);
    PHASE(a1, b1, a0, b0, kt, 2, kt, 6, 5);
    PHASE(a0, b0, a1, b1, kt, 3, kt, 11, 5);
    // stage kt+1 is in LDS for every wave, and every wave is done reading stage kt
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    PHASE(a1, b1, a0, b0, kt + 1, 0, kt, 0, 0);
  }
#undef GLOAD
#undef LWRITE
#undef RDF
#undef PHASE

  if (slot >= 0) {
    // tail slice: FP32 partial tile in register order, [64 x f32x4][256 threads]
    f32x4* pp = reinterpret_cast<f32x4*>(partial) + static_cast<size_t>(slot) * 64 * 256 + tid;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          pp[((i * 4 + j) * 4 + q) * 256] =
              f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
    return;
  }
  large_epilogue<KIND>(acc, perm, w, H, I, rbase, mcount, nb, wm, wn, l32, hi, hout, y, out);
}

// Tail fix-up, element-parallel: thread g of the grid takes one f32x4 of the
// partial tile (register order: f32x4 index ((i*4 + j)*4 + q)*256 + tid of the
// GEMM's thread tid) of tail item full + g / per_item, adds it over the S
// slices in slice order and applies that piece of the epilogue.  gate_up pairs
// gate block i with up block i + 2, so one thread takes both (i < 2).
template <int KIND>
__global__ __launch_bounds__(256) void gemm_large_fixup(
    const int* __restrict__ perm, const int2* __restrict__ tiles, const int* __restrict__ n_tiles,
    const int* __restrict__ counts, const int* __restrict__ offsets, const float* __restrict__ w,
    int H, int I, uint16_t* __restrict__ hout, float* __restrict__ y, uint16_t* __restrict__ out,
    const float* __restrict__ partial, int ncu) {
  constexpr bool kGU = KIND == kGateUp;
  constexpr int kPerItem = kGU ? 32 * 256 : 64 * 256;   // threads per tail item
  const int nblk = kGU ? I / 128 : H / 256;
  const int nk = (kGU ? H : I) / kLBK;
  const TailPlan plan = tail_plan(nblk * *n_tiles, ncu, nk);
  const int g = blockIdx.x * 256 + threadIdx.x;
  const int b = g / kPerItem;
  if (plan.S == 1 || b >= plan.rem) return;
  const int f = g - b * kPerItem;            // f32x4 index within the tile (gate half for gate_up)
  const int tid = f & 255, ijq = f >> 8;     // GEMM thread and register block
  const int i = ijq >> 4, j = (ijq >> 2) & 3, q = ijq & 3;
  const int item = plan.full + b;
  const int tile = item / nblk, nb = item - tile * nblk;
  const int2 te = tiles[tile];
  const int e = te.x, m0 = te.y;
  const int mcount = min(kLargeBM, counts[e] - m0);
  const int rbase = offsets[e] + m0;
  const int wv = tid >> 6, ln = tid & 63, l32 = ln & 31, hi = ln >> 5;
  const int wm = wv & 1, wn = wv >> 1;
  const int r = wm * 128 + 32 * j + l32;
  if (r >= mcount) return;
  const f32x4* pp = reinterpret_cast<const f32x4*>(partial) + f;
  f32x4 a = {0.f, 0.f, 0.f, 0.f}, u = {0.f, 0.f, 0.f, 0.f};
  for (int sl = 0; sl < plan.S; ++sl) {
    const size_t base = static_cast<size_t>(sl * plan.rem + b) * 64 * 256;
    a += pp[base];
    if (kGU) u += pp[base + 2 * 16 * 256];   // up block i + 2
  }
  if (kGU) {
    uint16_t* hr = hout + static_cast<size_t>(rbase + r) * I + nb * 128 + wn * 64 + 32 * i + 8 * q + 4 * hi;
    uint32_t p[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) p[t] = f32_to_bf16_rne(swiglu(a[t], u[t]));
    *reinterpret_cast<uint2*>(hr) = make_uint2(p[0] | (p[1] << 16), p[2] | (p[3] << 16));
  } else if (KIND == kDownFused) {
    const int t = perm[rbase + r];
    const float wt_t = w[t];
    uint16_t* o = out + static_cast<size_t>(t) * H + nb * 256 + wn * 128 + 32 * i + 8 * q + 4 * hi;
    uint32_t p[4];
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) p[t4] = f32_to_bf16_rne(wt_t * a[t4]);
    *reinterpret_cast<uint2*>(o) = make_uint2(p[0] | (p[1] << 16), p[2] | (p[3] << 16));
  } else {
    *reinterpret_cast<f32x4*>(y + static_cast<size_t>(rbase + r) * H + nb * 256 + wn * 128 + 32 * i +
                              8 * q + 4 * hi) = a;
  }
}

namespace {
// grid: every item whole, plus room for the tail slices (rem * S - rem < ncu)
int large_grid(int nblk, int max_tiles, int ncu) {
  return (nblk * max_tiles + ncu + kXcds - 1) / kXcds * kXcds;
}
}  // namespace

hipError_t launch_gate_up_large_bf16(const uint16_t* x, const uint16_t* wgu, const int* perm,
                                     const int2* tiles, const int* n_tiles, const int* counts,
                                     const int* offsets, int H, int I, int k, uint16_t* h,
                                     float* partial, int max_tiles, int ncu, hipStream_t s) {
  const int grid = large_grid(I / 128, max_tiles, ncu);
  hipLaunchKernelGGL(gemm_large_bf16<kGateUp>, dim3(grid), dim3(256), kLLds, s, x, wgu, perm,
                     tiles, n_tiles, counts, offsets, nullptr, H, I, k, h, nullptr, nullptr,
                     partial, ncu);
  hipLaunchKernelGGL(gemm_large_fixup<kGateUp>, dim3(ncu / 2 * 32), dim3(256), 0, s, perm, tiles,
                     n_tiles, counts, offsets, nullptr, H, I, h, nullptr, nullptr, partial, ncu);
  return hipGetLastError();
}

hipError_t launch_down_large_bf16(const uint16_t* h, const uint16_t* wd, const int* perm,
                                  const int2* tiles, const int* n_tiles, const int* counts,
                                  const int* offsets, const float* w, int H, int I, int k,
                                  float* y, uint16_t* out, float* partial, int max_tiles, int ncu,
                                  hipStream_t s) {
  const int grid = large_grid(H / 256, max_tiles, ncu);
#define LARGE_DOWN(KD)                                                                        \
  hipLaunchKernelGGL(gemm_large_bf16<KD>, dim3(grid), dim3(256), kLLds, s, h, wd, perm, tiles, \
                     n_tiles, counts, offsets, w, H, I, k, nullptr, y, out, partial, ncu);    \
  hipLaunchKernelGGL(gemm_large_fixup<KD>, dim3(ncu / 2 * 64), dim3(256), 0, s, perm, tiles,   \
                     n_tiles, counts, offsets, w, H, I, nullptr, y, out, partial, ncu)
  if (k == 1) { LARGE_DOWN(kDownFused); } else { LARGE_DOWN(kDownSlots); }
#undef LARGE_DOWN
  return hipGetLastError();
}

hipError_t large_set_attributes() {
  const int bytes = static_cast<int>(kLLds);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_large_bf16<kGateUp>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess)
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_large_bf16<kDownFused>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess)
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_large_bf16<kDownSlots>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  return e;
}

}  // namespace moe
