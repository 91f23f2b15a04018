// Backward pass of the batched layer, BF16.  The Mixture-of-Kittens summary
// measures the layer's backward pass beside its forward pass, in BF16 and in
// MXFP8 ("What is 2.37x measured against"); this is the one-GPU share of it:
// the expert computation of the pairs routed to this GPU.
//
// For every routed pair (t, j) -> expert e, with g, u the gate/up
// pre-activations, a = silu(g) u and w the routing weight:
//   dh      = W_down[e]^T dout[t]                    (the unweighted gradient of a)
//   dw      = a . dh                                 (gradient of the routing weight)
//   dg      = w dh u silu'(g),   du = w dh silu(g)
//   dx[t]  += W_gate_up[e]^T [dg; du]
//   dW_down[e]    += (w dout[t]) a^T
//   dW_gate_up[e] += [dg; du] x[t]^T
//   dlogits[t, m]  = w_m (dw_m - sum_j w_j dw_j) over the selected experts m
//
// Launches, all on the caller's stream, in this order:
//   group_experts   the forward's grouping (64-row M-tiles, stable order)
//   kGU   gu[row]  = [W_gate; W_up][e] x[t]                FP32, recomputed (not stored
//                   by the forward)
//   kDD   dh tile  = W_down[e]^T dout[t]; epilogue: dgu[row] = [dg; du] (BF16) and
//                   one partial dot a . dh per 128 columns
//   kDG   dxs[row] = W_gate_up[e]^T dgu[row]               FP32 per pair (k = 1: dx)
//   sum_pairs       dx[t] = sum_j dxs[row of (t, j)] in slot order, rounded once
//   kWD   dW_down[e]    = sum over the expert's rows of (w dout[t]) a^T     -> BF16
//   kWG   dW_gate_up[e] = sum over the expert's rows of [dg; du] x[t]^T     -> BF16
//   route_bwd       d_topk_w = the partial dots summed in column order; dlogits
//
// Every sum runs in a fixed order (MFMA K order, rows ascending within an
// expert, slots ascending), so repeated runs are bit-identical.
//
// The GEMMs share one LDS-tiled kernel: a workgroup of 4 waves computes an
// MT x 128 tile (MT = 64 routed rows for the three activation-gradient kinds,
// 128 for the weight gradients) in K chunks of 64, double-buffered in LDS.
// Operands whose reduction index is the contiguous one ("rows": x, dout, dgu
// rows, W_gate_up rows) are copied 16 bytes at a time; the others ("cols":
// W_down and W_gate_up read along their output dimension, and every operand
// of the weight gradients, whose reduction runs over routed rows) are read as
// two 16-byte runs of consecutive K rows and transposed into K-contiguous LDS
// rows on the way in (pairs of K packed into 32-bit words).  LDS rows are 128
// bytes with 16-byte chunk c of row r stored at chunk c ^ ((r ^ r >> 3) & 7),
// which keeps both the transposing writes (rows 8 apart) and the MFMA operand
// reads (16 consecutive rows) within two-way bank sharing on the 64 banks.
#include "common.h"
#include "internal.h"
#include "tiles.h"

namespace moe {

namespace {

enum { kGU = 0, kDD = 1, kDG = 2, kWD = 3, kWG = 4 };
constexpr int kBB = 64;          // routed rows per M-tile
constexpr int kKC = 64;          // K chunk (elements)
constexpr int kNT = 128;         // output columns per workgroup
constexpr int kCS32 = kNT + 4;   // FP32 C-tile row stride (elements)
constexpr int kCS16 = kNT + 8;   // BF16 C-tile row stride (elements)

inline size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

struct BwdArgs {
  const uint16_t* x;        // [T, H]
  const uint16_t* wgu;      // [E, 2I, H]
  const uint16_t* wd;       // [E, H, I]
  const uint16_t* dout;     // [T, H]
  const float* w;           // [T*k] routing weights
  const int* perm;          // grouped row -> pair id t*k + j
  const int2* tiles;        // M-tiles (expert, first row)
  const int* n_tiles;
  const int* counts;        // rows per expert
  const int* offsets;       // first grouped row per expert
  float* gu;                // [P, 2I] grouped rows
  uint16_t* dgu;            // [P, 2I] grouped rows
  float* dwp;               // [P, I/128] partial dots
  float* dxs;               // [P, H] grouped rows (k > 1)
  uint16_t* dx;             // [T, H]
  uint16_t* dwgu;           // [E, 2I, H]
  uint16_t* dwd;            // [E, H, I]
  int H, I, E, k;
};

// Element offset of 16-byte chunk c of LDS row r (rows of kKC elements).
__device__ __forceinline__ int swz(int r, int c) { return r * kKC + 8 * (c ^ ((r ^ (r >> 3)) & 7)); }

// Two 16-byte runs of K rows 2p and 2p+1 -> eight 32-bit words (row 2p in the low half).
__device__ __forceinline__ void pack_pairs(const i32x4& v0, const i32x4& v1, uint32_t (&o)[8]) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t a = static_cast<uint32_t>(v0[d]), b = static_cast<uint32_t>(v1[d]);
    o[2 * d] = (a & 0xFFFFu) | (b << 16);
    o[2 * d + 1] = (a >> 16) | (b & 0xFFFF0000u);
  }
}

__device__ __forceinline__ float sigmoidf_(float z) { return 1.0f / (1.0f + __expf(-z)); }

// BF16 x8 (16 bytes) times a scalar, rounded back to BF16.
__device__ __forceinline__ i32x4 scale_bf16x8(i32x4 v, float s) {
  i32x4 r;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t a = static_cast<uint32_t>(v[d]);
    const uint32_t lo = f32_to_bf16_rne(s * bf16_to_f32(a & 0xFFFFu));
    const uint32_t hi = f32_to_bf16_rne(s * bf16_to_f32(a >> 16));
    r[d] = static_cast<int>(lo | (hi << 16));
  }
  return r;
}

// silu(g) * u of 8 FP32 pairs, rounded to BF16 (16 bytes).
__device__ __forceinline__ i32x4 swiglu_bf16x8(const f32x4& g0, const f32x4& g1, const f32x4& u0,
                                               const f32x4& u1) {
  i32x4 r;
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    const uint32_t lo = f32_to_bf16_rne(swiglu(g0[2 * d], u0[2 * d]));
    const uint32_t hi = f32_to_bf16_rne(swiglu(g0[2 * d + 1], u0[2 * d + 1]));
    r[d] = static_cast<int>(lo | (hi << 16));
    const uint32_t lo1 = f32_to_bf16_rne(swiglu(g1[2 * d], u1[2 * d]));
    const uint32_t hi1 = f32_to_bf16_rne(swiglu(g1[2 * d + 1], u1[2 * d + 1]));
    r[2 + d] = static_cast<int>(lo1 | (hi1 << 16));
  }
  return r;
}

template <int KIND>
__global__ __launch_bounds__(256) void bwd_gemm(BwdArgs a) {
  constexpr bool WGRAD = KIND == kWD || KIND == kWG;
  constexpr int MT = WGRAD ? 128 : kBB;
  constexpr int MI = MT / 32;                         // 16-row A blocks per wave
  constexpr int AROW_U = MT * 8 / 256;                // "rows" A units per thread
  constexpr int BROW_U = kNT * 8 / 256;               // "rows" B units per thread (kGU)
  __shared__ __align__(16) uint16_t lds[2 * MT * kKC + 2 * kNT * kKC];
  uint16_t* const As = lds;
  uint16_t* const Bs = lds + 2 * MT * kKC;

  const int tid = threadIdx.x, ln = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = a.H, I = a.I, k = a.k;

  // ---- work item ----
  int e, n0, m0 = 0, mcount = 0, rbase = 0, nchunks;
  if constexpr (!WGRAD) {
    const int N = KIND == kGU ? 2 * I : (KIND == kDD ? I : H);
    const int nblk = N / kNT;
    const int item = real_item(blockIdx.x, nblk, *a.n_tiles);
    if (item < 0) return;
    const int tile = item / nblk;
    n0 = (item - tile * nblk) * kNT;
    const int2 te = a.tiles[tile];
    e = te.x;
    mcount = min(kBB, a.counts[e] - te.y);
    rbase = a.offsets[e] + te.y;
    nchunks = (KIND == kDG ? 2 * I : H) / kKC;
  } else {
    const int M = KIND == kWD ? H : 2 * I;
    const int N = KIND == kWD ? I : H;
    const int mb = M / MT, nb = N / kNT;
    const int n_items = a.E * mb * nb;
    const int item = xcd_item(blockIdx.x, gridDim.x);
    if (item >= n_items) return;
    e = item / (mb * nb);
    const int rem = item - e * (mb * nb);
    m0 = (rem / nb) * MT;
    n0 = (rem % nb) * kNT;
    rbase = a.offsets[e];
    mcount = a.counts[e];                            // the expert's rows = the K range
    nchunks = (mcount + kKC - 1) / kKC;
  }

  // ---- operand sources ----
  // "rows" A (kGU, kDD, kDG): unit u -> (row r = u / 8, chunk u % 8); rows past the
  // tile's end read its first row (their results are never stored)
  const uint16_t* abase = nullptr;
  uint32_t aoff[AROW_U > 0 ? AROW_U : 1] = {};
  if constexpr (!WGRAD) {
    abase = KIND == kGU ? a.x : (KIND == kDD ? a.dout : a.dgu);
#pragma unroll
    for (int i = 0; i < AROW_U; ++i) {
      const int u = tid + 256 * i, r = u >> 3, c = u & 7;
      const int rr = r < mcount ? r : 0;
      const uint32_t row = KIND == kDG ? static_cast<uint32_t>(rbase + rr) * (2 * I)
                                       : static_cast<uint32_t>(a.perm[rbase + rr] / k) * H;
      aoff[i] = row + 8 * c;
    }
  }
  // "rows" B (kGU): W_gate_up[e] rows n0 .. n0+127
  const uint16_t* bbase = nullptr;
  uint32_t boff[4] = {};
  uint32_t bld = 0;                                   // "cols" B: K-row stride
  if constexpr (KIND == kGU) {
    bbase = a.wgu + static_cast<size_t>(e) * 2 * I * H;
#pragma unroll
    for (int i = 0; i < BROW_U; ++i) {
      const int u = tid + 256 * i, r = u >> 3, c = u & 7;
      boff[i] = static_cast<uint32_t>(n0 + r) * H + 8 * c;
    }
  } else if constexpr (KIND == kDD || KIND == kDG) {
    // "cols" B: element (K row kk, column n) of W_down[e] [H, I] (kDD) or
    // W_gate_up[e] [2I, H] (kDG) at kk * ld + n0 + n
    bld = KIND == kDD ? I : H;
    bbase = KIND == kDD ? a.wd + static_cast<size_t>(e) * H * I
                        : a.wgu + static_cast<size_t>(e) * 2 * I * H;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int u = tid + 256 * i, q = u & 15, p = u >> 4;
      boff[i] = static_cast<uint32_t>(2 * p) * bld + n0 + 8 * q;
    }
  }

  // ---- staging registers and their LDS placement ----
  i32x4 ra[WGRAD ? 4 : AROW_U];                      // A: rows units, or 2 cols units x 2 K rows
  i32x4 rb[4];                                        // B: 4 rows units, or 2 cols units x 2 K rows
  f32x4 rg[KIND == kWD ? 16 : 1];                     // kWD B: g and u of 2 units x 2 rows (FP32)
  float rsc[WGRAD ? 4 : 1];                           // kWD A: routing weight per K row
  bool rv[WGRAD ? 4 : 1];                             // K row inside the expert

  auto load_chunk = [&](int ch) {
    if constexpr (!WGRAD) {
#pragma unroll
      for (int i = 0; i < AROW_U; ++i) ra[i] = ld16(abase + aoff[i] + ch * kKC);
      if constexpr (KIND == kGU) {
#pragma unroll
        for (int i = 0; i < BROW_U; ++i) rb[i] = ld16_stream(bbase + boff[i] + ch * kKC);
      } else {
        const uint32_t kof = static_cast<uint32_t>(ch * kKC) * bld;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          rb[2 * i] = ld16_stream(bbase + boff[i] + kof);
          rb[2 * i + 1] = ld16_stream(bbase + boff[i] + kof + bld);
        }
      }
    } else {
      // K rows are the expert's grouped rows rbase + ch*64 + 2p (+1); rows past
      // the expert's end are loaded from its last row and zeroed when packed
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int u = tid + 256 * i, q = u & 15, p = u >> 4;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int kr = ch * kKC + 2 * p + h;
          const int row = rbase + (kr < mcount ? kr : mcount - 1);
          rv[2 * i + h] = kr < mcount;
          if constexpr (KIND == kWD) {
            const int pair = a.perm[row];
            rsc[2 * i + h] = a.w[pair];
            ra[2 * i + h] = ld16(a.dout + static_cast<size_t>(pair / k) * H + m0 + 8 * q);
            const float* gp = a.gu + static_cast<size_t>(row) * (2 * I) + n0 + 8 * q;
            rg[8 * i + 4 * h + 0] = *reinterpret_cast<const f32x4*>(gp);
            rg[8 * i + 4 * h + 1] = *reinterpret_cast<const f32x4*>(gp + 4);
            rg[8 * i + 4 * h + 2] = *reinterpret_cast<const f32x4*>(gp + I);
            rg[8 * i + 4 * h + 3] = *reinterpret_cast<const f32x4*>(gp + I + 4);
          } else {
            ra[2 * i + h] = ld16(a.dgu + static_cast<size_t>(row) * (2 * I) + m0 + 8 * q);
            rb[2 * i + h] = ld16(a.x + static_cast<size_t>(a.perm[row] / k) * H + n0 + 8 * q);
          }
        }
      }
    }
  };

  auto store_chunk = [&](int buf) {
    uint16_t* ab = As + buf * MT * kKC;
    uint16_t* bb = Bs + buf * kNT * kKC;
    if constexpr (!WGRAD) {
#pragma unroll
      for (int i = 0; i < AROW_U; ++i) {
        const int u = tid + 256 * i;
        *reinterpret_cast<i32x4*>(ab + swz(u >> 3, u & 7)) = ra[i];
      }
    }
    if constexpr (KIND == kGU) {
#pragma unroll
      for (int i = 0; i < BROW_U; ++i) {
        const int u = tid + 256 * i;
        *reinterpret_cast<i32x4*>(bb + swz(u >> 3, u & 7)) = rb[i];
      }
    } else {
      // "cols" B (and A for the weight gradients): unit (p, q) holds K rows 2p, 2p+1
      // of columns 8q .. 8q+7; column 8q+j becomes LDS row 8q+j
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int u = tid + 256 * i, q = u & 15, p = u >> 4;
        const int co = (2 * p) & 7, ch = p >> 2;
        uint32_t wb_[8], wa_[8];
        if constexpr (WGRAD) {
          // K rows past the expert's end contribute zero on both sides
          const i32x4 zero = {0, 0, 0, 0};
          i32x4 a0 = ra[2 * i], a1 = ra[2 * i + 1], b0, b1;
          if constexpr (KIND == kWD) {
            a0 = scale_bf16x8(a0, rsc[2 * i]);
            a1 = scale_bf16x8(a1, rsc[2 * i + 1]);
            b0 = swiglu_bf16x8(rg[8 * i + 0], rg[8 * i + 1], rg[8 * i + 2], rg[8 * i + 3]);
            b1 = swiglu_bf16x8(rg[8 * i + 4], rg[8 * i + 5], rg[8 * i + 6], rg[8 * i + 7]);
          } else {
            b0 = rb[2 * i];
            b1 = rb[2 * i + 1];
          }
          if (!rv[2 * i]) a0 = b0 = zero;
          if (!rv[2 * i + 1]) a1 = b1 = zero;
          pack_pairs(a0, a1, wa_);
          pack_pairs(b0, b1, wb_);
        } else {
          pack_pairs(rb[2 * i], rb[2 * i + 1], wb_);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          *reinterpret_cast<uint32_t*>(bb + swz(8 * q + j, ch) + co) = wb_[j];
          if constexpr (WGRAD) *reinterpret_cast<uint32_t*>(ab + swz(8 * q + j, ch) + co) = wa_[j];
        }
      }
    }
  };

  // ---- main loop: wave (wm, wn) computes rows wm*MT/2.. x columns wn*64.. ----
  const int wm = wv & 1, wn = wv >> 1;
  const int fr = ln & 15, fg = ln >> 4;
  f32x4 acc[MI][4];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (nchunks > 0) {
    load_chunk(0);
    store_chunk(0);
  }
  __syncthreads();
  for (int ch = 0; ch < nchunks; ++ch) {
    const int buf = ch & 1;
    const bool more = ch + 1 < nchunks;
    if (more) load_chunk(ch + 1);
    const uint16_t* ab = As + buf * MT * kKC;
    const uint16_t* bb = Bs + buf * kNT * kKC;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int c = 4 * s + fg;
      bf16x8 af[MI], bfr[4];
#pragma unroll
      for (int i = 0; i < MI; ++i)
        af[i] = as_bf16x8(*reinterpret_cast<const i32x4*>(ab + swz(wm * (MT / 2) + 16 * i + fr, c)));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bfr[j] = as_bf16x8(*reinterpret_cast<const i32x4*>(bb + swz(wn * 64 + 16 * j + fr, c)));
      // D rows = B rows (output columns), D columns = A rows: lane holds 4
      // consecutive output columns of one tile row
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(bfr[j], af[i], acc[i][j]);
    }
    if (more) store_chunk(buf ^ 1);
    __syncthreads();
  }

  // ---- C tile through LDS (the operand buffers are free after the last barrier) ----
  // lane: tile row wm*MT/2 + 16i + fr, columns wn*64 + 16j + 4fg .. +3
  if constexpr (!WGRAD) {
    float* Cs = reinterpret_cast<float*>(lds);
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<f32x4*>(Cs + (wm * (MT / 2) + 16 * i + fr) * kCS32 + wn * 64 + 16 * j + 4 * fg) =
            acc[i][j];
  } else {
    uint16_t* Cs = lds;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 v = acc[i][j];
        uint2 p;
        p.x = f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16);
        p.y = f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16);
        *reinterpret_cast<uint2*>(Cs + (wm * (MT / 2) + 16 * i + fr) * kCS16 + wn * 64 + 16 * j + 4 * fg) = p;
      }
  }
  __syncthreads();

  // ---- epilogue: thread = (tile row r, 8 consecutive columns 8*sg) ----
  const int sg = tid & 15;
#pragma unroll 1
  for (int r = tid >> 4; r < MT; r += 16) {
    if constexpr (WGRAD) {
      const uint16_t* Cs = lds;
      const i32x4 v = *reinterpret_cast<const i32x4*>(Cs + r * kCS16 + 8 * sg);
      uint16_t* dst = KIND == kWD
                          ? a.dwd + (static_cast<size_t>(e) * H + m0 + r) * I + n0 + 8 * sg
                          : a.dwgu + (static_cast<size_t>(e) * 2 * I + m0 + r) * H + n0 + 8 * sg;
      st16(dst, v);
    } else {
      const float* Cs = reinterpret_cast<const float*>(lds);
      const f32x4 c0 = *reinterpret_cast<const f32x4*>(Cs + r * kCS32 + 8 * sg);
      const f32x4 c1 = *reinterpret_cast<const f32x4*>(Cs + r * kCS32 + 8 * sg + 4);
      const bool live = r < mcount;
      const size_t grow = static_cast<size_t>(rbase + (live ? r : 0));
      if constexpr (KIND == kGU) {
        if (live) {
          float* dst = a.gu + grow * (2 * I) + n0 + 8 * sg;
          *reinterpret_cast<f32x4*>(dst) = c0;
          *reinterpret_cast<f32x4*>(dst + 4) = c1;
        }
      } else if constexpr (KIND == kDD) {
        // columns n0 + 8sg .. +7 of the intermediate dimension
        const int pair = a.perm[grow];
        const float wt = a.w[pair];
        const float* gp = a.gu + grow * (2 * I) + n0 + 8 * sg;
        const f32x4 g0 = *reinterpret_cast<const f32x4*>(gp);
        const f32x4 g1 = *reinterpret_cast<const f32x4*>(gp + 4);
        const f32x4 u0 = *reinterpret_cast<const f32x4*>(gp + I);
        const f32x4 u1 = *reinterpret_cast<const f32x4*>(gp + I + 4);
        float part = 0.0f;
        uint32_t pg[4], pu[4];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float g = q < 4 ? g0[q] : g1[q - 4];
          const float u = q < 4 ? u0[q] : u1[q - 4];
          const float dh = q < 4 ? c0[q] : c1[q - 4];
          const float sg_ = sigmoidf_(g);
          const float si = g * sg_;
          part = fmaf(si * u, dh, part);
          const float da = wt * dh;
          const uint32_t bg = f32_to_bf16_rne(da * u * (sg_ * (1.0f + g * (1.0f - sg_))));
          const uint32_t bu = f32_to_bf16_rne(da * si);
          if (q & 1) {
            pg[q >> 1] |= bg << 16;
            pu[q >> 1] |= bu << 16;
          } else {
            pg[q >> 1] = bg;
            pu[q >> 1] = bu;
          }
        }
        // partial dot over the 128 columns: the 16 lanes of this row, fixed butterfly
#pragma unroll
        for (int m = 8; m >= 1; m >>= 1) part += __shfl_xor(part, m, kWave);
        if (live) {
          uint16_t* dst = a.dgu + grow * (2 * I) + n0 + 8 * sg;
          st16(dst, i32x4{static_cast<int>(pg[0]), static_cast<int>(pg[1]), static_cast<int>(pg[2]),
                          static_cast<int>(pg[3])});
          st16(dst + I, i32x4{static_cast<int>(pu[0]), static_cast<int>(pu[1]),
                              static_cast<int>(pu[2]), static_cast<int>(pu[3])});
          if (sg == 0) a.dwp[grow * (I / kNT) + n0 / kNT] = part;
        }
      } else {   // kDG
        if (live) {
          if (k > 1) {
            float* dst = a.dxs + grow * H + n0 + 8 * sg;
            *reinterpret_cast<f32x4*>(dst) = c0;
            *reinterpret_cast<f32x4*>(dst + 4) = c1;
          } else {
            const int t = a.perm[grow];               // k = 1: pair id == token
            i32x4 o;
            o[0] = static_cast<int>(f32_to_bf16_rne(c0[0]) | (f32_to_bf16_rne(c0[1]) << 16));
            o[1] = static_cast<int>(f32_to_bf16_rne(c0[2]) | (f32_to_bf16_rne(c0[3]) << 16));
            o[2] = static_cast<int>(f32_to_bf16_rne(c1[0]) | (f32_to_bf16_rne(c1[1]) << 16));
            o[3] = static_cast<int>(f32_to_bf16_rne(c1[2]) | (f32_to_bf16_rne(c1[3]) << 16));
            st16(a.dx + static_cast<size_t>(t) * H + n0 + 8 * sg, o);
          }
        }
      }
    }
  }
}

// dx[t] = sum_j dxs[row of (t, j)] in slot order (FP32), rounded once to BF16.
__global__ __launch_bounds__(256) void sum_pairs(const float* __restrict__ dxs,
                                                 const int* __restrict__ row_of, int T, int H, int k,
                                                 uint16_t* __restrict__ dx) {
  const int t = blockIdx.x;
  const int P = T * k;
  for (int c = threadIdx.x; c < H / 4; c += blockDim.x) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
      const int row = row_of[t * k + j];
      if (static_cast<unsigned>(row) >= static_cast<unsigned>(P)) continue;
      const f32x4 v = *reinterpret_cast<const f32x4*>(dxs + static_cast<size_t>(row) * H + 4 * c);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] += v[i];
    }
    uint2 o;
    o.x = f32_to_bf16_rne(acc[0]) | (f32_to_bf16_rne(acc[1]) << 16);
    o.y = f32_to_bf16_rne(acc[2]) | (f32_to_bf16_rne(acc[3]) << 16);
    *reinterpret_cast<uint2*>(dx + static_cast<size_t>(t) * H + 4 * c) = o;
  }
}

// One wave per token: d_topk_w[t, j] = sum of the pair's partial dots in column
// order; dlogits[t, e] = w_j (dw_j - sum_i w_i dw_i) for e = idx[t, j], else 0.
__global__ __launch_bounds__(64) void route_bwd(const float* __restrict__ dwp,
                                                const int* __restrict__ row_of,
                                                const int32_t* __restrict__ idx,
                                                const float* __restrict__ w, int T, int E, int k,
                                                int nI, float* __restrict__ dtw,
                                                float* __restrict__ dl) {
  __shared__ int s_idx[32];
  __shared__ float s_val[32];
  const int t = blockIdx.x, j = threadIdx.x;
  const int P = T * k;
  float dw = 0.0f, wj = 0.0f;
  if (j < k) {
    const int row = row_of[t * k + j];
    if (static_cast<unsigned>(row) < static_cast<unsigned>(P))
      for (int b = 0; b < nI; ++b) dw += dwp[static_cast<size_t>(row) * nI + b];
    wj = w[t * k + j];
    dtw[t * k + j] = dw;
  }
  const float S = wave_sum(wj * dw);
  if (j < k) {
    s_idx[j] = idx[t * k + j];
    s_val[j] = wj * (dw - S);
  }
  __syncthreads();
  for (int e = j; e < E; e += 64) {
    float v = 0.0f;
    for (int q = 0; q < k; ++q)
      if (s_idx[q] == e) v = s_val[q];
    dl[static_cast<size_t>(t) * E + e] = v;
  }
}

}  // namespace

BackwardWs backward_ws_layout(int T, int H, int I, int E, int k) {
  BackwardWs L{};
  const size_t P = static_cast<size_t>(T) * k;
  L.max_tiles = static_cast<int>(E + (P + kBB - 1) / kBB);
  size_t o = 0;
  L.n_tiles = o;  o += 256;
  L.counts = o;   o = align256(o + sizeof(int) * E);
  L.offsets = o;  o = align256(o + sizeof(int) * (E + 1));
  L.tiles = o;    o = align256(o + sizeof(int) * 2 * L.max_tiles);
  L.perm = o;     o = align256(o + sizeof(int) * P);
  L.row_of = o;   o = align256(o + sizeof(int) * P);
  L.gu = o;       o = align256(o + sizeof(float) * P * 2 * I);
  L.dgu = o;      o = align256(o + sizeof(uint16_t) * P * 2 * I);
  L.dwp = o;      o = align256(o + sizeof(float) * P * (I / kNT));
  L.dxs = o;
  if (k > 1) o = align256(o + sizeof(float) * P * H);
  L.total = o;
  return L;
}

hipError_t launch_backward(const uint16_t* x, const uint16_t* wgu, const uint16_t* wd,
                           const int32_t* idx, const float* w, const uint16_t* dout, int T, int H,
                           int I, int E, int k, uint16_t* dx, uint16_t* dwgu, uint16_t* dwd,
                           float* dtw, float* dlogits, void* ws, hipStream_t s) {
  const BackwardWs L = backward_ws_layout(T, H, I, E, k);
  char* b = static_cast<char*>(ws);
  BwdArgs a{};
  a.x = x;
  a.wgu = wgu;
  a.wd = wd;
  a.dout = dout;
  a.w = w;
  a.perm = reinterpret_cast<int*>(b + L.perm);
  a.tiles = reinterpret_cast<int2*>(b + L.tiles);
  a.n_tiles = reinterpret_cast<int*>(b + L.n_tiles);
  a.counts = reinterpret_cast<int*>(b + L.counts);
  a.offsets = reinterpret_cast<int*>(b + L.offsets);
  a.gu = reinterpret_cast<float*>(b + L.gu);
  a.dgu = reinterpret_cast<uint16_t*>(b + L.dgu);
  a.dwp = reinterpret_cast<float*>(b + L.dwp);
  a.dxs = reinterpret_cast<float*>(b + L.dxs);
  a.dx = dx;
  a.dwgu = dwgu;
  a.dwd = dwd;
  a.H = H;
  a.I = I;
  a.E = E;
  a.k = k;
  const int P = T * k;
  int* row_of = reinterpret_cast<int*>(b + L.row_of);

  hipError_t err = launch_group_experts(idx, P, E, kBB, const_cast<int*>(a.counts),
                                        const_cast<int*>(a.offsets), const_cast<int2*>(a.tiles),
                                        const_cast<int*>(a.n_tiles), const_cast<int*>(a.perm),
                                        row_of, s);
  if (err != hipSuccess) return err;
  auto grid_tiles = [&](int n) {
    return dim3(static_cast<unsigned>((n / kNT * L.max_tiles + kXcds - 1) / kXcds * kXcds));
  };
  auto grid_w = [&](int M, int N) {
    const long long n = static_cast<long long>(E) * (M / 128) * (N / kNT);
    return dim3(static_cast<unsigned>((n + kXcds - 1) / kXcds * kXcds));
  };
  prof_begin(kBwdGateUp, s);
  hipLaunchKernelGGL(bwd_gemm<kGU>, grid_tiles(2 * I), dim3(256), 0, s, a);
  prof_end(kBwdGateUp, s);
  prof_begin(kBwdDown, s);
  hipLaunchKernelGGL(bwd_gemm<kDD>, grid_tiles(I), dim3(256), 0, s, a);
  prof_end(kBwdDown, s);
  prof_begin(kBwdInput, s);
  hipLaunchKernelGGL(bwd_gemm<kDG>, grid_tiles(H), dim3(256), 0, s, a);
  if (k > 1) hipLaunchKernelGGL(sum_pairs, dim3(T), dim3(256), 0, s, a.dxs, row_of, T, H, k, dx);
  prof_end(kBwdInput, s);
  prof_begin(kBwdWDown, s);
  hipLaunchKernelGGL(bwd_gemm<kWD>, grid_w(H, I), dim3(256), 0, s, a);
  prof_end(kBwdWDown, s);
  prof_begin(kBwdWGateUp, s);
  hipLaunchKernelGGL(bwd_gemm<kWG>, grid_w(2 * I, H), dim3(256), 0, s, a);
  prof_end(kBwdWGateUp, s);
  hipLaunchKernelGGL(route_bwd, dim3(T), dim3(64), 0, s, a.dwp, row_of, idx, w, T, E, k, I / kNT,
                     dtw, dlogits);
  return hipGetLastError();
}

}  // namespace moe
