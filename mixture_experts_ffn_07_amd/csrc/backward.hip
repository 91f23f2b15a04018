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
//   group_experts   the forward's grouping (64- or 128-row M-tiles, stable order)
//   kGU   gu[row]  = [W_gate; W_up][e] x[t]                FP32, recomputed when the
//                   caller has not kept the forward's pre-activations
//   kDD   dh tile  = W_down[e]^T dout[t]; epilogue: dgu[row] = [dg; du] (BF16), the
//                   weighted activation wa[row] = w a (BF16) and one partial dot
//                   a . dh per 128 columns
//   kDG   dxs[row] = W_gate_up[e]^T dgu[row]               FP32 per pair (k = 1: dx)
//   sum_pairs       dx[t] = sum_j dxs[row of (t, j)] in slot order, rounded once
//   kWD   dW_down[e]    = sum over the expert's rows of dout[t] (w a)^T     -> BF16
//   kWG   dW_gate_up[e] = sum over the expert's rows of [dg; du] x[t]^T     -> BF16
//   route_bwd       d_topk_w = the partial dots summed in column order; dlogits
//
// Every sum runs in a fixed order (MFMA K order, rows ascending within an
// expert, slots ascending), so repeated runs are bit-identical.
//
// With 256 or more routed rows per expert on average (MFMA-bound) kDD, kDG, kWD
// and kWG run instead on the 256 x 256 large-group GEMM (gemm_large.hip) over a
// second, 256-row tiling of the same grouping: W_down and W_gate_up read as
// stored and transposed in the GEMM's loader for dh and dx (dh goes through
// FP32, then bwd_dh_finish applies kDD's epilogue), and x, dout, [dg; du] and
// w a laid out K-contiguous per expert for the weight gradients.
//
// The three activation-gradient GEMMs share one LDS-tiled kernel (bwd_gemm):
// a workgroup of 4 waves computes a 64-row x 128-column tile in K chunks of
// 64, double-buffered in LDS.  The two weight gradients (bwd_wgrad) reduce
// over an expert's routed rows: a workgroup keeps one 128-column block of its
// n-side operand in LDS and walks 8 blocks of 128 output rows, prefetching the
// next block's operand while the current one multiplies and stores.
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
constexpr int kBB = 64;          // routed rows per M-tile (128 when experts average >= 48 rows)
constexpr int kKC = 64;          // K chunk (elements)
constexpr int kNT = 128;         // output columns per workgroup
constexpr int kCS32 = kNT + 4;   // FP32 C-tile row stride (elements)
constexpr int kMB = 16;          // 128-row output blocks per weight-gradient workgroup
// Weight gradients on the large-group GEMM from this many routed rows per expert
// on average: below it an expert's reduction is one or two 64-row stages and the
// per-block fixed costs dominate (measured at 64 rows: 5.9 -> 10.2 ms for the two
// weight gradients of the GLM-5.2 shape; at 43: 7.3 -> 15.6 ms for Kimi's).
constexpr int kWgradLargeRows = 256;

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
  float* gu;                // [P, 2I] grouped rows (recomputed pre-activations)
  const float* gus;         // or NULL: [P, 2I] pair (slot) order, saved by the forward
  uint16_t* dgu;            // [P, 2I] grouped rows
  uint16_t* wa;             // [P, I] grouped rows: w * silu(g) * u
  float* dwp;               // [P, I/128] partial dots
  float* dxs;               // [P, H] grouped rows (k > 1)
  uint16_t* dx;             // [T, H]
  uint16_t* dwgu;           // [E, 2I, H]
  uint16_t* dwd;            // [E, H, I]
  int H, I, E, k;
  int cb0, ncb, ldx;        // kDG with k > 1: column blocks [cb0, cb0 + ncb) of the kernel's
                            // width (ncb 0: all), written to dxs with row stride ldx from
                            // column cb0 * width
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

// LDS of bwd_gemm<KIND, MT, WN> (dynamic): both operands' two K-chunk buffers
constexpr size_t bwd_lds(int MT, int WN) { return static_cast<size_t>(2 * MT * kKC + 2 * 64 * WN * kKC) * 2; }

// WN: waves along the output columns (64 each): 2 (128 columns, 4 waves) or, for kDG,
// 4 (256 columns, 8 waves), which reads W_gate_up's rows in 512-byte runs instead of
// 256-byte ones (its K rows are 2I apart by H elements).
template <int KIND, int MT, int WN = 2>   // kGU, kDD, kDG; MT = routed rows per M-tile (64 or 128)
__global__ __launch_bounds__(128 * WN) void bwd_gemm(BwdArgs a, uint32_t okey) {
  static_assert(WN == 2 || KIND == kDG || KIND == kDD, "wide tiles: dh and dx only");
  constexpr int NTH = 128 * WN;                       // threads
  constexpr int NTC = 64 * WN;                        // output columns per workgroup
  constexpr int CS32 = NTC + 4;                       // FP32 C-tile row stride (elements)
  constexpr int MI = MT / 32;                         // 16-row A blocks per wave
  constexpr int AROW_U = MT * 8 / NTH;                // "rows" A units per thread
  constexpr int BROW_U = NTC * 8 / NTH;               // "rows" B units per thread (kGU)
  extern __shared__ __align__(16) uint16_t lds[];     // [2][MT x kKC] A, [2][NTC x kKC] B
  uint16_t* const As = lds;
  uint16_t* const Bs = lds + 2 * MT * kKC;

  const int tid = threadIdx.x, ln = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = a.H, I = a.I, k = a.k;

  // ---- work item: (M-tile of MT routed rows, NTC output columns) ----
  const int N = KIND == kGU ? 2 * I : (KIND == kDD ? I : H);
  const int cb0 = KIND == kDG ? a.cb0 : 0;
  const int nblk = KIND == kDG && a.ncb ? a.ncb : N / NTC;
  const int item0 = real_item(blockIdx.x, nblk, *a.n_tiles);
  if (item0 < 0) return;
  const int item = permute_item(item0, nblk * *a.n_tiles, okey);
  const int tile = item / nblk;
  const int n0 = (cb0 + item - tile * nblk) * NTC;
  const int2 te = a.tiles[tile];
  const int e = te.x;
  const int mcount = min(MT, a.counts[e] - te.y);
  const int rbase = a.offsets[e] + te.y;
  const int nchunks = (KIND == kDG ? 2 * I : H) / kKC;

  // ---- operand sources ----
  // "rows" A (kGU, kDD, kDG): unit u -> (row r = u / 8, chunk u % 8); rows past the
  // tile's end read its first row (their results are never stored)
  const uint16_t* const abase = KIND == kGU ? a.x : (KIND == kDD ? a.dout : a.dgu);
  uint32_t aoff[AROW_U];
#pragma unroll
  for (int i = 0; i < AROW_U; ++i) {
    const int u = tid + NTH * i, r = u >> 3, c = u & 7;
    const int rr = r < mcount ? r : 0;
    const uint32_t row = KIND == kDG ? static_cast<uint32_t>(rbase + rr) * (2 * I)
                                     : static_cast<uint32_t>(a.perm[rbase + rr] / k) * H;
    aoff[i] = row + 8 * c;
  }
  // "rows" B (kGU): W_gate_up[e] rows n0 .. n0+127
  const uint16_t* bbase = nullptr;
  uint32_t boff[4] = {};
  uint32_t bld = 0;                                   // "cols" B: K-row stride
  if constexpr (KIND == kGU) {
    bbase = a.wgu + static_cast<size_t>(e) * 2 * I * H;
#pragma unroll
    for (int i = 0; i < BROW_U; ++i) {
      const int u = tid + NTH * i, r = u >> 3, c = u & 7;
      boff[i] = static_cast<uint32_t>(n0 + r) * H + 8 * c;
    }
  } else if constexpr (KIND == kDD || KIND == kDG) {
    // "cols" B: element (K row kk, column n) of W_down[e] [H, I] (kDD) or
    // W_gate_up[e] [2I, H] (kDG) at kk * ld + n0 + n
    bld = KIND == kDD ? I : H;
    bbase = KIND == kDD ? a.wd + static_cast<size_t>(e) * H * I
                        : a.wgu + static_cast<size_t>(e) * 2 * I * H;
#pragma unroll
    for (int i = 0; i < 2; ++i) {                    // NTC/8 column groups x 32 K-row pairs
      const int u = tid + NTH * i, q = u % (NTC / 8), p = u / (NTC / 8);
      boff[i] = static_cast<uint32_t>(2 * p) * bld + n0 + 8 * q;
    }
  }

  // ---- staging registers and their LDS placement ----
  i32x4 ra[AROW_U];
  i32x4 rb[4];                                        // B: 4 rows units, or 2 cols units x 2 K rows

  auto load_chunk = [&](int ch) {
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
  };

  auto store_chunk = [&](int buf) {
    uint16_t* ab = As + buf * MT * kKC;
    uint16_t* bb = Bs + buf * NTC * kKC;
#pragma unroll
    for (int i = 0; i < AROW_U; ++i) {
      const int u = tid + NTH * i;
      *reinterpret_cast<i32x4*>(ab + swz(u >> 3, u & 7)) = ra[i];
    }
    if constexpr (KIND == kGU) {
#pragma unroll
      for (int i = 0; i < BROW_U; ++i) {
        const int u = tid + NTH * i;
        *reinterpret_cast<i32x4*>(bb + swz(u >> 3, u & 7)) = rb[i];
      }
    } else {
      // "cols" B: unit (p, q) holds K rows 2p, 2p+1 of columns 8q .. 8q+7;
      // column 8q+j becomes LDS row 8q+j
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int u = tid + NTH * i, q = u % (NTC / 8), p = u / (NTC / 8);
        uint32_t wb_[8];
        pack_pairs(rb[2 * i], rb[2 * i + 1], wb_);
#pragma unroll
        for (int j = 0; j < 8; ++j)
          *reinterpret_cast<uint32_t*>(bb + swz(8 * q + j, p >> 2) + ((2 * p) & 7)) = wb_[j];
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

  load_chunk(0);
  store_chunk(0);
  __syncthreads();
  for (int ch = 0; ch < nchunks; ++ch) {
    const int buf = ch & 1;
    const bool more = ch + 1 < nchunks;
    if (more) load_chunk(ch + 1);
    const uint16_t* ab = As + buf * MT * kKC;
    const uint16_t* bb = Bs + buf * NTC * kKC;
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

  // ---- C tile through LDS, 64 rows at a time (the operand buffers are free after
  // the last barrier); lane: tile row wm*MT/2 + 16i + fr, columns wn*64 + 16j + 4fg .. +3
  const int sg = tid % (NTC / 8);
#pragma unroll 1
  for (int half = 0; half < MT / 64; ++half) {
    if (MT == 64 || wm == half) {
      float* Cs = reinterpret_cast<float*>(lds);
      const int rl = MT == 64 ? wm * 32 : 0;
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<f32x4*>(Cs + (rl + 16 * i + fr) * CS32 + wn * 64 + 16 * j + 4 * fg) =
              acc[i][j];
    }
    __syncthreads();
  // ---- epilogue: thread = (tile row r, 8 consecutive columns 8*sg) ----
#pragma unroll 1
  for (int rc = tid / (NTC / 8); rc < 64; rc += NTH / (NTC / 8)) {
    const int r = half * 64 + rc;
    {
      const float* Cs = reinterpret_cast<const float*>(lds);
      const f32x4 c0 = *reinterpret_cast<const f32x4*>(Cs + rc * CS32 + 8 * sg);
      const f32x4 c1 = *reinterpret_cast<const f32x4*>(Cs + rc * CS32 + 8 * sg + 4);
      const bool live = r < mcount;
      const size_t grow = static_cast<size_t>(rbase + (live ? r : 0));
      if constexpr (KIND == kGU) {
        if (live) {
          float* dst = a.gu + grow * (2 * I) + n0 + 8 * sg;
          st16_stream(dst, c0);
          st16_stream(dst + 4, c1);
        }
      } else if constexpr (KIND == kDD) {
        // columns n0 + 8sg .. +7 of the intermediate dimension
        const int pair = a.perm[grow];
        const float wt = a.w[pair];
        const float* gp = (a.gus ? a.gus + static_cast<size_t>(pair) * (2 * I) : a.gu + grow * (2 * I)) +
                          n0 + 8 * sg;
        const f32x4 g0 = *reinterpret_cast<const f32x4*>(gp);
        const f32x4 g1 = *reinterpret_cast<const f32x4*>(gp + 4);
        const f32x4 u0 = *reinterpret_cast<const f32x4*>(gp + I);
        const f32x4 u1 = *reinterpret_cast<const f32x4*>(gp + I + 4);
        float part = 0.0f;
        uint32_t pg[4], pu[4], pa[4];
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
          const uint32_t ba = f32_to_bf16_rne(wt * (si * u));
          if (q & 1) {
            pg[q >> 1] |= bg << 16;
            pu[q >> 1] |= bu << 16;
            pa[q >> 1] |= ba << 16;
          } else {
            pg[q >> 1] = bg;
            pu[q >> 1] = bu;
            pa[q >> 1] = ba;
          }
        }
        // partial dot over each 128 columns: their 16 lanes of this row, fixed butterfly
#pragma unroll
        for (int m = 8; m >= 1; m >>= 1) part += __shfl_xor(part, m, kWave);
        if (live) {
          uint16_t* dst = a.dgu + grow * (2 * I) + n0 + 8 * sg;
          st16_stream(dst, i32x4{static_cast<int>(pg[0]), static_cast<int>(pg[1]),
                                 static_cast<int>(pg[2]), static_cast<int>(pg[3])});
          st16_stream(dst + I, i32x4{static_cast<int>(pu[0]), static_cast<int>(pu[1]),
                                     static_cast<int>(pu[2]), static_cast<int>(pu[3])});
          st16_stream(a.wa + grow * I + n0 + 8 * sg,
               i32x4{static_cast<int>(pa[0]), static_cast<int>(pa[1]), static_cast<int>(pa[2]),
                     static_cast<int>(pa[3])});
          if ((sg & 15) == 0) a.dwp[grow * (I / kNT) + (n0 + 8 * sg) / kNT] = part;
        }
      } else {   // kDG
        if (live) {
          if (k > 1) {
            float* dst = a.dxs + grow * a.ldx + (n0 - cb0 * NTC) + 8 * sg;
            st16_stream(dst, c0);
            st16_stream(dst + 4, c1);
          } else {
            const int t = a.perm[grow];               // k = 1: pair id == token
            i32x4 o;
            o[0] = static_cast<int>(pack_bf16x2(c0[0], c0[1]));
            o[1] = static_cast<int>(pack_bf16x2(c0[2], c0[3]));
            o[2] = static_cast<int>(pack_bf16x2(c1[0], c1[1]));
            o[3] = static_cast<int>(pack_bf16x2(c1[2], c1[3]));
            st16(a.dx + static_cast<size_t>(t) * H + n0 + 8 * sg, o);
          }
        }
      }
    }
  }
    __syncthreads();                                  // before the next half reuses Cs
  }
}

// Weight gradients, reduced over an expert's grouped rows r (K, in chunks of
// 64; rows past the expert's end count as zero):
//   kWD: dW_down[e][h][i]    = sum_r dout[t_r][h] * wa[r][i]   (A = dout rows
//        gathered through perm, output rows h; B = wa rows, output columns i)
//   kWG: dW_gate_up[e][c][h] = sum_r dgu[r][c] * x[t_r][h]     (A = dgu rows,
//        output rows c; B = x rows gathered through perm, output columns h)
// Workgroup = (expert, 128 output columns, kMB blocks of 128 output rows).
// With at most two chunks (up to 128 rows: the common case at 40-70 routed
// rows per expert) the B tiles are staged during the first row block and stay
// in LDS (one slot per chunk) for every later row block;
// each row block's A tile is loaded while the previous block multiplies, and
// the finished block leaves through a small per-wave LDS tile: each store
// instruction writes eight whole 128-byte row segments (storing straight from
// the accumulators wrote 64-byte half lines, which the memory system handles
// at a markedly lower rate).
template <int KIND>   // kWD, kWG (at most 256 registers: two workgroups per CU)
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_wgrad(
    BwdArgs a, uint32_t okey) {
  __shared__ __align__(16) uint16_t lds[4 * 128 * kKC];
  constexpr int kWs = 128 + 16;                       // bytes per staged output row (+16: banks)
  __shared__ __align__(16) uint8_t wst[4][16 * kWs];  // per wave: 16 rows x 64 columns, BF16
  uint16_t* const As = lds;                           // [2][128 rows][64 K]
  uint16_t* const Bs = lds + 2 * 128 * kKC;           // [2][128 columns][64 K]
  const int tid = threadIdx.x, ln = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = a.H, I = a.I, k = a.k;
  const int M = KIND == kWD ? H : 2 * I, N = KIND == kWD ? I : H;
  const int mb = M / 128, nb = N / kNT, mgs = (mb + kMB - 1) / kMB;
  const int item = permute_item(xcd_item(blockIdx.x, gridDim.x), gridDim.x, okey);
  if (item >= a.E * nb * mgs) return;
  const int e = item / (nb * mgs);
  const int rem = item - e * (nb * mgs);
  const int n0 = (rem / mgs) * kNT;
  const int mfirst = (rem % mgs) * kMB, mend = min(mb, mfirst + kMB);
  const int cnt = a.counts[e], rbase = a.offsets[e];
  const int nchunks = (cnt + kKC - 1) / kKC;
  const bool bres = nchunks <= 2;                     // B chunk ch stays in LDS slot ch
  uint16_t* const out = KIND == kWD ? a.dwd + static_cast<size_t>(e) * H * I
                                    : a.dwgu + static_cast<size_t>(e) * 2 * I * H;
  const uint16_t* const Ab = KIND == kWD ? a.dout : a.dgu;
  const uint16_t* const Bb = KIND == kWD ? a.wa : a.x;

  // unit i of this thread: u = tid + 256 i -> (K-row pair p = u / 16, 8 columns
  // from 8q, q = u % 16); element offsets of its two K rows in A and in B
  uint32_t aro[4], bro[4];
  bool vld[4];
  auto rows_for = [&](int ch) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int p = (tid + 256 * i) >> 4;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int kr = ch * kKC + 2 * p + h;
        vld[2 * i + h] = kr < cnt;
        const int row = rbase + (kr < cnt ? kr : cnt - 1);
        const uint32_t tok = static_cast<uint32_t>(a.perm[row] / k) * H;
        aro[2 * i + h] = KIND == kWD ? tok : static_cast<uint32_t>(row) * (2 * I);
        bro[2 * i + h] = KIND == kWD ? static_cast<uint32_t>(row) * I : tok;
      }
    }
  };
  i32x4 ra[4], rb[4];
  auto load = [&](int mi, bool with_b) {
    const int m0 = mi * 128;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = (tid + 256 * i) & 15;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        ra[2 * i + h] = ld16(Ab + aro[2 * i + h] + m0 + 8 * q);
        if (with_b) rb[2 * i + h] = ld16(Bb + bro[2 * i + h] + n0 + 8 * q);
      }
    }
  };
  auto stage = [&](int buf, int bslot, bool with_b) {
    uint16_t* ab = As + buf * 128 * kKC;
    uint16_t* bb = Bs + bslot * 128 * kKC;
    const i32x4 zero = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int u = tid + 256 * i, q = u & 15, p = u >> 4;
      uint32_t w_[8];
      pack_pairs(vld[2 * i] ? ra[2 * i] : zero, vld[2 * i + 1] ? ra[2 * i + 1] : zero, w_);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        *reinterpret_cast<uint32_t*>(ab + swz(8 * q + j, p >> 2) + ((2 * p) & 7)) = w_[j];
      if (with_b) {
        pack_pairs(vld[2 * i] ? rb[2 * i] : zero, vld[2 * i + 1] ? rb[2 * i + 1] : zero, w_);
#pragma unroll
        for (int j = 0; j < 8; ++j)
          *reinterpret_cast<uint32_t*>(bb + swz(8 * q + j, p >> 2) + ((2 * p) & 7)) = w_[j];
      }
    }
  };

  const int wm = wv & 1, wn = wv >> 1;
  const int fr = ln & 15, fg = ln >> 4;
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // lane: output row mi*128 + wm*64 + 16i + fr, columns n0 + wn*64 + 16j + 4fg .. +3.
  // Per 16-row group i the wave writes its 16 x 64 block into its LDS tile and
  // reads it back as rows 8s + (ln >> 3), 16-byte chunk ln & 7 (a wave's LDS
  // operations complete in order, so each read sees the writes before it and
  // the next group's writes follow the reads).
  auto store_tile = [&](int mi) {
    uint8_t* st = wst[wv];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<uint2*>(st + fr * kWs + (16 * j + 4 * fg) * 2) =
            make_uint2(pack_bf16x2(acc[i][j][0], acc[i][j][1]), pack_bf16x2(acc[i][j][2], acc[i][j][3]));
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int r = 8 * s + (ln >> 3), c = ln & 7;
        st16_stream(out + static_cast<size_t>(mi * 128 + wm * 64 + 16 * i + r) * N + n0 + wn * 64 + 8 * c,
                    *reinterpret_cast<const i32x4*>(st + r * kWs + 16 * c));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };

  const int total = (mend - mfirst) * nchunks;
  if (total == 0) {                                   // no routed rows: zero gradient
    for (int mi = mfirst; mi < mend; ++mi) store_tile(mi);
    return;
  }
  rows_for(0);
  load(mfirst, true);
  stage(0, 0, true);
  __syncthreads();
  for (int it = 0; it < total; ++it) {
    const int mq = it / nchunks;
    const int mi = mfirst + mq, ch = it - mq * nchunks;
    const int buf = it & 1;
    const bool more = it + 1 < total;
    const int mq1 = (it + 1) / nchunks, ch1 = it + 1 - mq1 * nchunks;
    // B is loaded for every chunk, or (resident) only during the first row block
    const bool nb_load = !bres || mq1 == 0;
    if (more) {
      if (nchunks > 1) rows_for(ch1);
      load(mfirst + mq1, nb_load);
    }
    const uint16_t* ab = As + buf * 128 * kKC;
    const uint16_t* bb = Bs + (bres ? ch : buf) * 128 * kKC;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int c = 4 * s2 + fg;
      bf16x8 af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = as_bf16x8(*reinterpret_cast<const i32x4*>(ab + swz(wm * 64 + 16 * i + fr, c)));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bfr[j] = as_bf16x8(*reinterpret_cast<const i32x4*>(bb + swz(wn * 64 + 16 * j + fr, c)));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(bfr[j], af[i], acc[i][j]);
    }
    if (ch == nchunks - 1) store_tile(mi);
    if (more) {
      stage(buf ^ 1, bres ? ch1 : buf ^ 1, nb_load);
      __syncthreads();
    }
  }
}

// dx[t] = sum_j dxs[row of (t, j)] in slot order (FP32), rounded once to BF16;
// a launch covers dx columns [col0, col0 + cols), dxs holding them with row
// stride ldx from its column 0.
__global__ __launch_bounds__(256) void sum_pairs(const float* __restrict__ dxs,
                                                 const int* __restrict__ row_of, int T, int H, int k,
                                                 uint16_t* __restrict__ dx, uint32_t okey, int col0,
                                                 int cols, int ldx) {
  const int t = permute_item(blockIdx.x, gridDim.x, okey);
  const int P = T * k;
  dx += col0;
  for (int c = threadIdx.x; c < cols / 4; c += blockDim.x) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
      const int row = row_of[t * k + j];
      if (static_cast<unsigned>(row) >= static_cast<unsigned>(P)) continue;
      const f32x4 v = *reinterpret_cast<const f32x4*>(dxs + static_cast<size_t>(row) * ldx + 4 * c);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] += v[i];
    }
    uint2 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
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
                                                float* __restrict__ dl, uint32_t okey) {
  __shared__ int s_idx[32];
  __shared__ float s_val[32];
  const int t = permute_item(blockIdx.x, gridDim.x, okey), j = threadIdx.x;
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

// Large groups: dh (FP32, grouped rows, from the large-group GEMM) -> [dg; du]
// (BF16), w a (BF16) and the partial dots a . dh per 128 columns, with the
// arithmetic of bwd_gemm's kDD epilogue.  Thread = (row, 8 consecutive columns);
// 16 rows x 128 columns per workgroup.
__global__ __launch_bounds__(256) void bwd_dh_finish(BwdArgs a, const float* __restrict__ dh, int P, uint32_t okey) {
  const int I = a.I;
  const int tid = threadIdx.x, sg = tid & 15;
  const int row = permute_item(blockIdx.x, gridDim.x, okey) * 16 + (tid >> 4);
  const int n0 = blockIdx.y * kNT;
  if (row >= P) return;                             // whole 16-lane row groups leave together
  const size_t grow = static_cast<size_t>(row);
  const int pair = a.perm[grow];
  const float wt = a.w[pair];
  const float* gp = (a.gus ? a.gus + static_cast<size_t>(pair) * (2 * I) : a.gu + grow * (2 * I)) +
                    n0 + 8 * sg;
  const f32x4 g0 = *reinterpret_cast<const f32x4*>(gp);
  const f32x4 g1 = *reinterpret_cast<const f32x4*>(gp + 4);
  const f32x4 u0 = *reinterpret_cast<const f32x4*>(gp + I);
  const f32x4 u1 = *reinterpret_cast<const f32x4*>(gp + I + 4);
  const float* hp = dh + grow * I + n0 + 8 * sg;
  const f32x4 c0 = *reinterpret_cast<const f32x4*>(hp);
  const f32x4 c1 = *reinterpret_cast<const f32x4*>(hp + 4);
  float part = 0.0f;
  uint32_t pg[4], pu[4], pa[4];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const float g = q < 4 ? g0[q] : g1[q - 4];
    const float u = q < 4 ? u0[q] : u1[q - 4];
    const float d = q < 4 ? c0[q] : c1[q - 4];
    const float sg_ = sigmoidf_(g);
    const float si = g * sg_;
    part = fmaf(si * u, d, part);
    const float da = wt * d;
    const uint32_t bg = f32_to_bf16_rne(da * u * (sg_ * (1.0f + g * (1.0f - sg_))));
    const uint32_t bu = f32_to_bf16_rne(da * si);
    const uint32_t ba = f32_to_bf16_rne(wt * (si * u));
    if (q & 1) {
      pg[q >> 1] |= bg << 16;
      pu[q >> 1] |= bu << 16;
      pa[q >> 1] |= ba << 16;
    } else {
      pg[q >> 1] = bg;
      pu[q >> 1] = bu;
      pa[q >> 1] = ba;
    }
  }
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) part += __shfl_xor(part, m, kWave);
  uint16_t* dst = a.dgu + grow * (2 * I) + n0 + 8 * sg;
  st16(dst, i32x4{static_cast<int>(pg[0]), static_cast<int>(pg[1]), static_cast<int>(pg[2]),
                  static_cast<int>(pg[3])});
  st16(dst + I, i32x4{static_cast<int>(pu[0]), static_cast<int>(pu[1]), static_cast<int>(pu[2]),
                      static_cast<int>(pu[3])});
  st16(a.wa + grow * I + n0 + 8 * sg,
       i32x4{static_cast<int>(pa[0]), static_cast<int>(pa[1]), static_cast<int>(pa[2]),
             static_cast<int>(pa[3])});
  if (sg == 0) a.dwp[grow * (I / kNT) + n0 / kNT] = part;
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
  L.wa = o;       o = align256(o + sizeof(uint16_t) * P * I);
  L.dwp = o;      o = align256(o + sizeof(float) * P * (I / kNT));
  L.dxs = o;
  if (k > 1) o = align256(o + sizeof(float) * P * H);
  // >= kWgradLargeRows routed rows per expert on average: the weight gradients
  // run on the large-group GEMM over transposed operands (32-bit element offsets
  // into them); >= 256 (MFMA-bound): dh and dx too
  const size_t cols = wgrad_large_cols(static_cast<int>(P), E);
  const size_t rows_max = static_cast<size_t>(H > 2 * I ? H : 2 * I);
  L.large_w = P >= static_cast<size_t>(kWgradLargeRows) * E &&
              rows_max * cols < (static_cast<size_t>(1) << 31);
  L.large_d = P >= static_cast<size_t>(256) * E;
  if (L.large_w) {
    L.koff = o;   o = align256(o + sizeof(int) * (E + 1));
    L.xT = o;     o = align256(o + sizeof(uint16_t) * H * cols);
    L.doutT = o;  o = align256(o + sizeof(uint16_t) * H * cols);
    L.dguT = o;   o = align256(o + sizeof(uint16_t) * 2 * I * cols);
    L.waT = o;    o = align256(o + sizeof(uint16_t) * I * cols);
  }
  if (L.large_d) {
    L.max_tiles256 = static_cast<int>(E + (P + kLargeBM - 1) / kLargeBM);
    L.n_tiles256 = o; o += 256;
    L.tiles256 = o;   o = align256(o + sizeof(int) * 2 * L.max_tiles256);
    L.partial = o;    o = align256(o + sizeof(float) * kLargeMaxSlices * kLargeBM * 256);
    L.dh = o;         o = align256(o + sizeof(float) * P * I);
  }
  L.total = o;
  return L;
}

hipError_t launch_backward(const uint16_t* x, const uint16_t* wgu, const uint16_t* wd,
                           const int32_t* idx, const float* w, const uint16_t* dout,
                           const float* gu_saved, int T, int H, int I, int E, int k,
                           uint16_t* dx, uint16_t* dwgu, uint16_t* dwd, float* dtw,
                           float* dlogits, void* ws, hipStream_t s, int num_cus) {
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
  a.gus = gu_saved;
  a.dgu = reinterpret_cast<uint16_t*>(b + L.dgu);
  a.wa = reinterpret_cast<uint16_t*>(b + L.wa);
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

  // 128-row M-tiles once experts average 48 routed rows or more: an expert's
  // weights are then streamed once per tile for up to 128 rows (fewer second
  // tiles); below that most experts fit one 64-row tile, and the taller tile only
  // adds staging (measured: slower at ~43 rows per expert)
  const bool tall = P >= 48LL * E;
  hipError_t err = launch_group_experts(idx, P, E, tall ? 128 : kBB, const_cast<int*>(a.counts),
                                        const_cast<int*>(a.offsets), const_cast<int2*>(a.tiles),
                                        const_cast<int*>(a.n_tiles), const_cast<int*>(a.perm),
                                        row_of, s);
  if (err != hipSuccess) return err;
  auto grid_tiles = [&](int n) {
    return dim3(static_cast<unsigned>((n / kNT * L.max_tiles + kXcds - 1) / kXcds * kXcds));
  };
  auto grid_w = [&](int M, int N) {
    const long long n = static_cast<long long>(E) * ((M / 128 + kMB - 1) / kMB) * (N / kNT);
    return dim3(static_cast<unsigned>((n + kXcds - 1) / kXcds * kXcds));
  };
  if (!gu_saved) {
    prof_begin(kBwdGateUp, s);
    if (tall) hipLaunchKernelGGL((bwd_gemm<kGU, 128>), grid_tiles(2 * I), dim3(256), bwd_lds(128, 2), s, a, order_key());
    else hipLaunchKernelGGL((bwd_gemm<kGU, 64>), grid_tiles(2 * I), dim3(256), bwd_lds(64, 2), s, a, order_key());
    prof_end(kBwdGateUp, s);
  }
  // large groups: 256-row M-tiles over the same (deterministic) grouping for the
  // large-group GEMMs of dh and dx
  int2* tiles256 = L.large_d ? reinterpret_cast<int2*>(b + L.tiles256) : nullptr;
  int* n_tiles256 = L.large_d ? reinterpret_cast<int*>(b + L.n_tiles256) : nullptr;
  float* partial = L.large_d ? reinterpret_cast<float*>(b + L.partial) : nullptr;
  if (L.large_d) {
    err = launch_group_experts(idx, P, E, kLargeBM, const_cast<int*>(a.counts),
                               const_cast<int*>(a.offsets), tiles256, n_tiles256,
                               const_cast<int*>(a.perm), row_of, s);
    if (err != hipSuccess) return err;
  }
  prof_begin(kBwdDown, s);
  if (L.large_d) {
    // dh on the large-group GEMM (W_down [E][H][I] read in place, transposed in
    // the loader), then the SwiGLU backward, w a and the partial dots elementwise
    float* dh = reinterpret_cast<float*>(b + L.dh);
    err = launch_dh_large(dout, wd, a.perm, tiles256, n_tiles256, a.counts, a.offsets, H, I, k,
                          dh, partial, L.max_tiles256, num_cus, s);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(bwd_dh_finish, dim3((P + 15) / 16, I / kNT), dim3(256), 0, s, a, dh, P, order_key());
  } else if (tall) {
    hipLaunchKernelGGL((bwd_gemm<kDD, 128>), grid_tiles(I), dim3(256), bwd_lds(128, 2), s, a, order_key());
  } else {
    // 8 waves x 256 columns: W_down's rows read in 512-byte runs
    const dim3 g(static_cast<unsigned>((I / 256 * L.max_tiles + kXcds - 1) / kXcds * kXcds));
    hipLaunchKernelGGL((bwd_gemm<kDD, 64, 4>), g, dim3(512), bwd_lds(64, 4), s, a, order_key());
  }
  prof_end(kBwdDown, s);
  prof_begin(kBwdInput, s);
  if (L.large_d) {
    // dx on the large-group GEMM: W_gate_up [E][2I][H] read in place
    err = launch_dgrad_large(a.dgu, wgu, a.perm, tiles256, n_tiles256, a.counts, a.offsets, H,
                             2 * I, k, a.dxs, dx, partial, L.max_tiles256, num_cus, s);
    if (err != hipSuccess) return err;
  } else {
    // column parts (column_parts): each part's FP32 per-pair slice is summed right
    // after its launch, while it is still in the last-level cache (T 2048, k 8,
    // H 7168: 7 parts).  64-row tiles: workgroups of 8 waves x 256 columns, two per
    // CU (W_gate_up's rows read in 512-byte runs: Kimi shape 4.05 -> 3.73 ms); 128-row
    // tiles keep 4 waves x 128 columns, two per CU (the wide form fits one per CU
    // there and ran 11% slower on the GLM shape).
    const int dw = tall ? kNT : 256;
    const int parts = k > 1 ? column_parts(static_cast<size_t>(P), H, dw, L.max_tiles,
                                           8 * num_cus)
                            : 1;
    const int hq = H / parts;
    for (int q = 0; q < parts; ++q) {
      BwdArgs ap = a;
      ap.cb0 = q * (hq / dw);
      ap.ncb = hq / dw;
      ap.ldx = hq;
      const dim3 g(static_cast<unsigned>((hq / dw * L.max_tiles + kXcds - 1) / kXcds * kXcds));
      if (tall) hipLaunchKernelGGL((bwd_gemm<kDG, 128>), g, dim3(256), bwd_lds(128, 2), s, ap, order_key());
      else hipLaunchKernelGGL((bwd_gemm<kDG, 64, 4>), g, dim3(512), bwd_lds(64, 4), s, ap, order_key());
      if (k > 1)
        hipLaunchKernelGGL(sum_pairs, dim3(T), dim3(256), 0, s, a.dxs, row_of, T, H, k, dx,
                           order_key(), q * hq, hq, hq);
    }
  }
  if (L.large_d && k > 1)
    hipLaunchKernelGGL(sum_pairs, dim3(T), dim3(256), 0, s, a.dxs, row_of, T, H, k, dx, order_key(),
                       0, H, H);
  prof_end(kBwdInput, s);
  if (L.large_w) {
    err = launch_wgrad_large(x, dout, a.dgu, a.wa, a.perm, a.counts, a.offsets, P, H, I, E, k,
                             reinterpret_cast<int*>(b + L.koff), reinterpret_cast<uint16_t*>(b + L.xT),
                             reinterpret_cast<uint16_t*>(b + L.doutT),
                             reinterpret_cast<uint16_t*>(b + L.dguT),
                             reinterpret_cast<uint16_t*>(b + L.waT), dwgu, dwd, num_cus, s);
    if (err != hipSuccess) return err;
  } else {
    prof_begin(kBwdWDown, s);
    hipLaunchKernelGGL(bwd_wgrad<kWD>, grid_w(H, I), dim3(256), 0, s, a, order_key());
    prof_end(kBwdWDown, s);
    prof_begin(kBwdWGateUp, s);
    hipLaunchKernelGGL(bwd_wgrad<kWG>, grid_w(2 * I, H), dim3(256), 0, s, a, order_key());
    prof_end(kBwdWGateUp, s);
  }
  hipLaunchKernelGGL(route_bwd, dim3(T), dim3(64), 0, s, a.dwp, row_of, idx, w, T, E, k, I / kNT,
                     dtw, dlogits, order_key());
  return hipGetLastError();
}

// ===========================================================================
// MXFP8 backward.  Every product takes both operands MX-quantized along its own
// reduction axis (blocks of 32): dh = W_down^T dout along H, dx = W_gate_up^T
// [dg; du] along 2I, both weight gradients along the expert's routed pairs.  All
// five products run on the large-tile MXFP8 GEMM (gemm_large.hip) over one
// 256-row tiling of the grouping; the kernels here re-quantize the weights
// along their other axis, finish dh into [dg; du], and lay out the pair-axis
// operands.
namespace {

// E4M3 code -> FP32 (exact): sign, 4-bit exponent with bias 7 (0: subnormal
// m * 2^-9), 3-bit mantissa.  Codes come from MX encoders, so never NaN.
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20))
                    : static_cast<float>(m) * 0.001953125f;
  return (c & 0x80u) ? -v : v;
}

// Eight values of one MX block row (the block spans the four lanes xor 1, 2 of
// a lane quad): amax over the quad, scale, eight E4M3 codes; returns the scale
// code.
__device__ __forceinline__ uint32_t mx_quad_encode(const float (&v)[8], uint32_t& lo, uint32_t& hi) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));
  amax = fmaxf(amax, __shfl_xor(amax, 2, kWave));
  const int sx = mx_scale_exp(amax);
  const float inv = exp2_neg(sx);
  lo = f32x4_to_e4m3x4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
  hi = f32x4_to_e4m3x4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
  return static_cast<uint32_t>(sx + 127);
}

// dst[b] = the MX encoding along R of src[b]^T: src codes [B][R][C] with scales
// [B][R][C/32] (blocks along C) are decoded exactly and re-encoded as dst codes
// [B][C][R] with scales [B][C][R/32] (blocks along R).  A workgroup takes 64U
// rows (R a multiple of 64U) and J consecutive blocks of 128 columns (C a multiple
// of 128J), one block at a time as U 64-row tiles through LDS, with the next
// block's loads in flight while the current one is converted and stored: every
// load covers whole 128-byte lines of source rows; the codes of the 128 output
// rows collect in LDS and leave as whole row lines, and each output row's 2U scale
// bytes in one store.  With counts, matrices b with counts[b] == 0 are skipped
// (their copy is left as is).
template <int U, int J>                             // 64-row tiles, 128-column blocks per workgroup
__global__ __launch_bounds__(256) void mx_requant_t(const uint8_t* __restrict__ src,
                                                    const uint8_t* __restrict__ src_s, int R, int C,
                                                    uint8_t* __restrict__ dst,
                                                    uint8_t* __restrict__ dst_s,
                                                    const int* __restrict__ counts, uint32_t okey) {
  // the scale store below writes a row's 2U scale bytes as one 4- or 8-byte word
  static_assert(U == 2 || U == 4, "64U-row workgroups with U = 2 or 4");
  constexpr int kOt = 64 * U + 16;                  // bytes per staged output row (+16: banks)
  __shared__ float tl[128][64 + 1];                 // [c][r]
  __shared__ __align__(16) uint8_t ot[128 * kOt];   // [c][64U codes]
  __shared__ __align__(8) uint8_t ssc[128][2 * U];  // [c][block of 32 rows]
  const int cb = permute_item(blockIdx.x, gridDim.x, okey) * J, r0 = blockIdx.y * 64 * U;
  const size_t b = blockIdx.z;
  if (counts && counts[b] == 0) return;             // no pair reads this expert's copy
  const int tid = threadIdx.x;
  const int q = tid & 7, rl = tid >> 3;             // load: rows rl and rl + 32 of a tile, 16 codes at 16q
  i32x4 v[U][2], vn[U][2];
  int sc[U][2], sn[U][2];
  auto load = [&](int c0, i32x4 (&V)[U][2], int (&S)[U][2]) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const size_t row = b * R + r0 + 64 * u + 32 * h + rl;
        V[u][h] = ld16(src + row * C + c0 + 16 * q);
        S[u][h] = src_s[row * (C / 32) + (c0 + 16 * q) / 32];
      }
  };
  load(cb * 128, v, sc);
  const int c = tid >> 1, hb = tid & 1;             // encode: out row c, block hb of the tile's 64 rows
#pragma unroll 1
  for (int jj = 0; jj < J; ++jj) {
    const int c0 = (cb + jj) * 128;
    if (jj + 1 < J) load(c0 + 128, vn, sn);         // the next block's codes in flight
    if (jj) __syncthreads();                        // the previous block's rows are stored
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (u) __syncthreads();                       // the previous tile is read out
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        // decode: the hardware E4M3 pair conversion (exact), times 2^(scale - 127)
        const float scl = ldexpf(1.0f, sc[u][h] - 127);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const f32x2 f0 = __builtin_amdgcn_cvt_pk_f32_fp8(v[u][h][d], false);   // bytes 0, 1
          const f32x2 f1 = __builtin_amdgcn_cvt_pk_f32_fp8(v[u][h][d], true);    // bytes 2, 3
          tl[16 * q + 4 * d][32 * h + rl] = f0.x * scl;
          tl[16 * q + 4 * d + 1][32 * h + rl] = f0.y * scl;
          tl[16 * q + 4 * d + 2][32 * h + rl] = f1.x * scl;
          tl[16 * q + 4 * d + 3][32 * h + rl] = f1.y * scl;
        }
      }
      __syncthreads();
      float val[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) val[i] = tl[c][32 * hb + i];
      float amax = 0.f;
#pragma unroll
      for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(val[i]));
      const int sx = mx_scale_exp(amax);
      const float inv = exp2_neg(sx);
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const float* w = val + 16 * g;
        *reinterpret_cast<i32x4*>(&ot[c * kOt + 64 * u + 32 * hb + 16 * g]) =
             i32x4{static_cast<int>(f32x4_to_e4m3x4(w[0] * inv, w[1] * inv, w[2] * inv, w[3] * inv)),
                   static_cast<int>(f32x4_to_e4m3x4(w[4] * inv, w[5] * inv, w[6] * inv, w[7] * inv)),
                   static_cast<int>(f32x4_to_e4m3x4(w[8] * inv, w[9] * inv, w[10] * inv, w[11] * inv)),
                   static_cast<int>(f32x4_to_e4m3x4(w[12] * inv, w[13] * inv, w[14] * inv, w[15] * inv))};
      }
      ssc[c][2 * u + hb] = static_cast<uint8_t>(sx + 127);
    }
    __syncthreads();
    // 128 rows x 64U bytes: lane ln of wave wv stores bytes [16 (ln % 4U), +16) of row
    // 32 wv + (16 / U) s + ln / 4U, so each store instruction writes whole row lines
    {
      const int wv = tid >> 6, ln = tid & 63;
#pragma unroll
      for (int s = 0; s < 2 * U; ++s) {
        const int row = 32 * wv + (16 / U) * s + ln / (4 * U), off = 16 * (ln % (4 * U));
        st16_stream(dst + (b * C + c0 + row) * static_cast<size_t>(R) + r0 + off,
                    *reinterpret_cast<const i32x4*>(&ot[row * kOt + off]));
      }
    }
    if (tid < 128) {
      uint8_t* sp = dst_s + (b * C + c0 + tid) * (R / 32) + r0 / 32;
      if constexpr (U == 4) *reinterpret_cast<uint2*>(sp) = *reinterpret_cast<const uint2*>(&ssc[tid][0]);
      else *reinterpret_cast<uint32_t*>(sp) = *reinterpret_cast<const uint32_t*>(&ssc[tid][0]);
    }
    if (jj + 1 < J) {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          v[u][h] = vn[u][h];
          sc[u][h] = sn[u][h];
        }
    }
  }
}

// The MXFP8 backward's dh finish, per grouped row r (thread = 8 columns, 16
// rows x 128 columns per workgroup): from g, u (FP32, grouped rows [P][2I]) and
// dh = W_down^T dout (FP32 [P][I]): a = silu(g) u and da = w dh, dg = da u
// silu'(g), du = da silu(g); writes a and [dg; du] in FP32 (the pair-axis
// operands of the weight gradients), [dg; du] MX-encoded along 2I (dx's
// operand), and the partial dots a . dh per 128 columns (d topk_w).
__global__ __launch_bounds__(256) void mx_dh_finish(const float* __restrict__ gu,
                                                    const float* __restrict__ dh,
                                                    const int* __restrict__ perm,
                                                    const float* __restrict__ w, int P, int I,
                                                    float* __restrict__ aout,
                                                    float* __restrict__ dgu,
                                                    uint8_t* __restrict__ dguq,
                                                    uint8_t* __restrict__ dgus,
                                                    float* __restrict__ dwp, uint32_t okey) {
  const int tid = threadIdx.x, sg = tid & 15;
  const int row = permute_item(blockIdx.x, gridDim.x, okey) * 16 + (tid >> 4);
  const int n0 = blockIdx.y * kNT;
  if (row >= P) return;                             // whole 16-lane row groups leave together
  const size_t grow = static_cast<size_t>(row);
  const float wt = w[perm[grow]];
  const float* gp = gu + grow * (2 * I) + n0 + 8 * sg;
  const float* hp = dh + grow * I + n0 + 8 * sg;
  float dg[8], du[8], av[8];
  float part = 0.0f;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const float g = gp[q], u = gp[I + q], d = hp[q];
    const float sgm = sigmoidf_(g);
    const float si = g * sgm;
    av[q] = si * u;
    part = fmaf(av[q], d, part);
    const float da = wt * d;
    dg[q] = da * u * (sgm * (1.0f + g * (1.0f - sgm)));
    du[q] = da * si;
  }
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) part += __shfl_xor(part, m, kWave);
  float* ap = aout + grow * I + n0 + 8 * sg;
  float* dp = dgu + grow * (2 * I) + n0 + 8 * sg;
#pragma unroll
  for (int q = 0; q < 8; q += 4) {
    *reinterpret_cast<f32x4*>(ap + q) = f32x4{av[q], av[q + 1], av[q + 2], av[q + 3]};
    *reinterpret_cast<f32x4*>(dp + q) = f32x4{dg[q], dg[q + 1], dg[q + 2], dg[q + 3]};
    *reinterpret_cast<f32x4*>(dp + I + q) = f32x4{du[q], du[q + 1], du[q + 2], du[q + 3]};
  }
  uint32_t lo, hi;
  const uint32_t sgc = mx_quad_encode(dg, lo, hi);
  *reinterpret_cast<uint2*>(dguq + grow * (2 * I) + n0 + 8 * sg) = make_uint2(lo, hi);
  const uint32_t suc = mx_quad_encode(du, lo, hi);
  *reinterpret_cast<uint2*>(dguq + grow * (2 * I) + I + n0 + 8 * sg) = make_uint2(lo, hi);
  if ((sg & 3) == 0) {
    dgus[grow * (2 * I / 32) + (n0 + 8 * sg) / 32] = static_cast<uint8_t>(sgc);
    dgus[grow * (2 * I / 32) + (I + n0 + 8 * sg) / 32] = static_cast<uint8_t>(suc);
  }
  if (sg == 0) dwp[grow * (I / kNT) + n0 / kNT] = part;
}

// Pair-axis operand of a weight gradient: dst[c][koff[e] + r] = the MX encoding,
// along the routed pairs of expert e (blocks of 32 from koff[e], padding zero),
// of element c of the expert's r-th routed row.  SRC 0: x[token] (BF16); 1:
// w * dout[token] (BF16 dout, FP32 routing weight); 2: grouped FP32 rows
// (src32, row stride ld).  Workgroup = 128 pairs (four blocks, all of one
// expert: koff is padded to 128) x 64 rows c, so each row c gets a whole
// 128-byte line of codes and one 4-byte store of its four scales; the scales
// go out transposed ([KPT/128][rows] dwords: the workgroup's 64 dwords are
// consecutive).
template <int SRC>
__global__ __launch_bounds__(256) void mx_pair_t(const uint16_t* __restrict__ src16,
                                                 const float* __restrict__ src32, int ld,
                                                 const int* __restrict__ perm,
                                                 const float* __restrict__ w, int k,
                                                 const int* __restrict__ counts,
                                                 const int* __restrict__ offsets,
                                                 const int* __restrict__ koff, int E,
                                                 uint8_t* __restrict__ dst,
                                                 uint8_t* __restrict__ dst_s, uint32_t okey) {
  __shared__ float tl[64][128 + 1];                 // [c][pair]
  const int KPT = koff[E];
  const int g0 = permute_item(blockIdx.x, gridDim.x, okey) * 128, c0 = blockIdx.y * 64;
  if (g0 >= KPT) return;
  int lo = 0, hi = E - 1;                           // last e with koff[e] <= g0
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (koff[mid] <= g0) lo = mid; else hi = mid - 1;
  }
  const int e = lo;
  const int cnt = counts[e], base = offsets[e], r0 = g0 - koff[e];
  const int tid = threadIdx.x;
  if (SRC < 2) {
    i32x4 raw[4];
    float sc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {                   // pair p, 8 values at 8ch
      const int idx = tid + 256 * u, p = idx >> 3, ch = idx & 7;
      raw[u] = i32x4{0, 0, 0, 0};
      sc[u] = 0.f;
      if (r0 + p < cnt) {
        const int pr = perm[base + r0 + p];
        raw[u] = ld16(src16 + static_cast<size_t>(pr / k) * ld + c0 + 8 * ch);
        sc[u] = SRC == 1 ? w[pr] : 1.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int idx = tid + 256 * u, p = idx >> 3, ch = idx & 7;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t v = static_cast<uint32_t>(raw[u][i]);
        tl[8 * ch + 2 * i][p] = sc[u] * bf16_to_f32(v & 0xFFFFu);
        tl[8 * ch + 2 * i + 1][p] = sc[u] * bf16_to_f32(v >> 16);
      }
    }
  } else {
#pragma unroll
    for (int u = 0; u < 8; ++u) {                   // pair p, 4 values at 4ch
      const int idx = tid + 256 * u, p = idx >> 4, ch = idx & 15;
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (r0 + p < cnt)
        v = *reinterpret_cast<const f32x4*>(src32 + static_cast<size_t>(base + r0 + p) * ld + c0 + 4 * ch);
#pragma unroll
      for (int i = 0; i < 4; ++i) tl[4 * ch + i][p] = v[i];
    }
  }
  __syncthreads();
  const int c = tid >> 2, q = tid & 3;              // out row c; block b: pairs 32b + 8q .. + 7
  const size_t orow = static_cast<size_t>(c0 + c);
  uint32_t scodes = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = tl[c][32 * b + 8 * q + i];
    uint32_t clo, chi;
    scodes |= mx_quad_encode(v, clo, chi) << (8 * b);
    *reinterpret_cast<uint2*>(dst + orow * KPT + g0 + 32 * b + 8 * q) = make_uint2(clo, chi);
  }
  // scale dwords transposed, [KPT/128][rows]: a stage's dwords of consecutive rows are
  // consecutive for the weight-gradient GEMMs' loaders
  if (q == 0) reinterpret_cast<uint32_t*>(dst_s)[static_cast<size_t>(g0 / 128) * (gridDim.y * 64) + orow] = scodes;
}

inline size_t a256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

}  // namespace

MxBackwardWs mx_backward_ws_layout(int T, int H, int I, int E, int k) {
  MxBackwardWs L{};
  const size_t P = static_cast<size_t>(T) * k;
  L.max_tiles = static_cast<int>(E + (P + kLargeBM - 1) / kLargeBM);
  L.kpt_max = (P + static_cast<size_t>(E) * 127 + 127) / 128 * 128;
  size_t o = 0;
  L.n_tiles = o;  o += 256;
  L.counts = o;   o = a256(o + sizeof(int) * E);
  L.offsets = o;  o = a256(o + sizeof(int) * (E + 1));
  L.tiles = o;    o = a256(o + sizeof(int) * 2 * L.max_tiles);
  L.perm = o;     o = a256(o + sizeof(int) * P);
  L.row_of = o;   o = a256(o + sizeof(int) * P);
  L.koff = o;     o = a256(o + sizeof(int) * (E + 1));
  L.xq = o;       o = a256(o + static_cast<size_t>(T) * H);
  L.xs = o;       o = a256(o + static_cast<size_t>(T) * H / 32);
  L.dq = o;       o = a256(o + static_cast<size_t>(T) * H);
  L.ds = o;       o = a256(o + static_cast<size_t>(T) * H / 32);
  L.wdT = o;      o = a256(o + static_cast<size_t>(E) * I * H);
  L.wdTs = o;     o = a256(o + static_cast<size_t>(E) * I * H / 32);
  L.wguT = o;     o = a256(o + static_cast<size_t>(E) * H * 2 * I);
  L.wguTs = o;    o = a256(o + static_cast<size_t>(E) * H * 2 * I / 32);
  L.gu = o;       o = a256(o + sizeof(float) * P * 2 * I);
  L.dh = o;       o = a256(o + sizeof(float) * P * I);
  L.a = o;        o = a256(o + sizeof(float) * P * I);
  L.dgu = o;      o = a256(o + sizeof(float) * P * 2 * I);
  L.dguq = o;     o = a256(o + P * 2 * I);
  L.dgus = o;     o = a256(o + P * 2 * I / 32);
  L.dwp = o;      o = a256(o + sizeof(float) * P * (I / kNT));
  L.dxs = o;
  if (k > 1) o = a256(o + sizeof(float) * P * H);
  L.partial = o;  o = a256(o + sizeof(float) * kLargeMaxSlices * kLargeBM * 256);
  L.aT = o;       o = a256(o + static_cast<size_t>(I) * L.kpt_max);
  L.aTs = o;      o = a256(o + static_cast<size_t>(I) * L.kpt_max / 32);
  L.dyT = o;      o = a256(o + static_cast<size_t>(H) * L.kpt_max);
  L.dyTs = o;     o = a256(o + static_cast<size_t>(H) * L.kpt_max / 32);
  L.xT = o;       o = a256(o + static_cast<size_t>(H) * L.kpt_max);
  L.xTs = o;      o = a256(o + static_cast<size_t>(H) * L.kpt_max / 32);
  L.dguT = o;     o = a256(o + static_cast<size_t>(2 * I) * L.kpt_max);
  L.dguTs = o;    o = a256(o + static_cast<size_t>(2 * I) * L.kpt_max / 32);
  L.max_tiles64 = static_cast<int>(E + (P + 63) / 64);
  L.n_tiles64 = o; o += 256;
  L.tiles64 = o;  o = a256(o + sizeof(int) * 2 * L.max_tiles64);
  // transposed scale dwords for the 256-row large-tile projections (the recompute, dh
  // and dx when experts average >= 256 routed pairs; dx also at k = 1)
  L.sct = o;
  if (P >= static_cast<size_t>(kLargeBM) * E || k == 1) {
    const size_t gu = static_cast<size_t>(E) * 2 * I * (H / 32) + P * (H / 32);
    const size_t dx = static_cast<size_t>(E) * H * (2 * I / 32) + P * (2 * I / 32);
    o = a256(o + (gu > dx ? gu : dx));
  }
  L.total = o;
  return L;
}

// 64-row tiles per re-encoding workgroup (2: 52 KB of LDS, three workgroups per CU)
// and its 128-column blocks (the next one's loads in flight meanwhile; I and H are
// multiples of 256, so 2 divides both block counts)
constexpr int kRqU = 2;
constexpr int kRqJ = 2;

hipError_t launch_backward_mx(const uint16_t* x, const uint8_t* wgu, const uint8_t* wgus,
                              const uint8_t* wd, const uint8_t* wds, const int32_t* idx,
                              const float* w, const uint16_t* dout, int T, int H, int I, int E,
                              int k, uint16_t* dx, uint16_t* dwgu, uint16_t* dwd, float* dtw,
                              float* dlogits, void* ws, hipStream_t s, int num_cus) {
  const MxBackwardWs L = mx_backward_ws_layout(T, H, I, E, k);
  char* b = static_cast<char*>(ws);
  auto P8 = [&](size_t off) { return reinterpret_cast<uint8_t*>(b + off); };
  auto PF = [&](size_t off) { return reinterpret_cast<float*>(b + off); };
  int* counts = reinterpret_cast<int*>(b + L.counts);
  int* offsets = reinterpret_cast<int*>(b + L.offsets);
  int2* tiles = reinterpret_cast<int2*>(b + L.tiles);
  int* n_tiles = reinterpret_cast<int*>(b + L.n_tiles);
  int* perm = reinterpret_cast<int*>(b + L.perm);
  int* row_of = reinterpret_cast<int*>(b + L.row_of);
  int* koff = reinterpret_cast<int*>(b + L.koff);
  float* partial = PF(L.partial);
  uint32_t* sct = reinterpret_cast<uint32_t*>(b + L.sct);
  const int P = T * k;
  hipError_t err = launch_group_experts(idx, P, E, kLargeBM, counts, offsets, tiles, n_tiles, perm,
                                        row_of, s);
  // x and dout along H; the weights re-encoded along their output axes
  if (err != hipSuccess) return err;
  prof_begin(kBwdRequant, s);
  err = launch_quant_mx(x, T, H, P8(L.xq), P8(L.xs), s);
  if (err == hipSuccess) err = launch_quant_mx(dout, T, H, P8(L.dq), P8(L.ds), s);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((mx_requant_t<kRqU, kRqJ>), dim3(I / (128 * kRqJ), H / (64 * kRqU), E), dim3(256), 0, s, wd, wds, H, I, P8(L.wdT),
                     P8(L.wdTs), counts, order_key());
  hipLaunchKernelGGL((mx_requant_t<kRqU, kRqJ>), dim3(H / (128 * kRqJ), 2 * I / (64 * kRqU), E), dim3(256), 0, s, wgu, wgus, 2 * I, H,
                     P8(L.wguT), P8(L.wguTs), counts, order_key());
  prof_end(kBwdRequant, s);
  // Experts averaging fewer than 256 routed pairs: the pre-activations, dh and dx on the
  // batched MXFP8 kernel's 64-row tiles (whole-line weight streams; the 256-row tile spends
  // most of its rows on padding there), over a second tiling of the same grouping
  const bool rows64 = static_cast<int64_t>(P) < static_cast<int64_t>(kLargeBM) * E;
  int2* tiles64 = reinterpret_cast<int2*>(b + L.tiles64);
  int* n_tiles64 = reinterpret_cast<int*>(b + L.n_tiles64);
  if (rows64) {
    err = launch_group_experts(idx, P, E, 64, counts, offsets, tiles64, n_tiles64, perm, row_of, s);
    if (err != hipSuccess) return err;
  }
  // the forward's pre-activations, then dh and its finish
  prof_begin(kBwdGateUp, s);
  if (rows64)
    err = launch_mx_gate_up_raw_rows(P8(L.xq), P8(L.xs), wgu, wgus, perm, tiles64, n_tiles64,
                                     L.max_tiles64, counts, offsets, H, I, k, PF(L.gu), s, num_cus);
  else
    err = launch_gate_up_raw_large_mx(P8(L.xq), P8(L.xs), wgu, wgus, perm, tiles, n_tiles, counts,
                                      offsets, H, I, k, PF(L.gu), partial, L.max_tiles, num_cus, s,
                                      T, E, sct);
  prof_end(kBwdGateUp, s);
  if (err != hipSuccess) return err;
  prof_begin(kBwdDown, s);
  if (rows64) {
    err = launch_mx_rows_gather(P8(L.dq), P8(L.ds), P8(L.wdT), P8(L.wdTs), perm, tiles64, n_tiles64,
                                L.max_tiles64, counts, offsets, H, I, k, PF(L.dh), s, num_cus);
  } else {
    err = launch_dh_large_mx(P8(L.dq), P8(L.ds), P8(L.wdT), P8(L.wdTs), perm, tiles, n_tiles, counts,
                             offsets, H, I, k, PF(L.dh), partial, L.max_tiles, num_cus, s, T, E, sct);
  }
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(mx_dh_finish, dim3((P + 15) / 16, I / kNT), dim3(256), 0, s, PF(L.gu), PF(L.dh),
                     perm, w, P, I, PF(L.a), PF(L.dgu), P8(L.dguq), P8(L.dgus), PF(L.dwp),
                     order_key());
  prof_end(kBwdDown, s);
  // dx (rows64, k > 1: FP32 per grouped row into dxs, then the slot sum; T 2048, k 8, E 384:
  // the whole backward 32.6 -> 32.0 ms)
  prof_begin(kBwdInput, s);
  if (rows64 && k > 1) {
    err = launch_mx_rows_down(P8(L.dguq), P8(L.dgus), P8(L.wguT), P8(L.wguTs), perm, tiles64,
                              n_tiles64, L.max_tiles64, counts, offsets, H, 2 * I, k, PF(L.dxs), s,
                              num_cus);
  } else {
    err = launch_dgrad_large_mx(P8(L.dguq), P8(L.dgus), P8(L.wguT), P8(L.wguTs), perm, tiles, n_tiles,
                                counts, offsets, H, 2 * I, k, PF(L.dxs), dx, partial, L.max_tiles,
                                num_cus, s, T, E, sct);
  }
  if (err != hipSuccess) return err;
  if (k > 1)
    hipLaunchKernelGGL(sum_pairs, dim3(T), dim3(256), 0, s, PF(L.dxs), row_of, T, H, k, dx, order_key(),
                       0, H, H);
  prof_end(kBwdInput, s);
  // weight gradients over pair-axis operands (the segment timed as dw_gate_up
  // covers the pair-axis encodings and both weight gradients' single launch)
  prof_begin(kBwdWGateUp, s);
  err = launch_koff_mx(counts, E, koff, s);
  if (err != hipSuccess) return err;
  const unsigned gb = static_cast<unsigned>(L.kpt_max / 128);
  hipLaunchKernelGGL(mx_pair_t<1>, dim3(gb, H / 64), dim3(256), 0, s, dout, nullptr, H, perm, w, k,
                     counts, offsets, koff, E, P8(L.dyT), P8(L.dyTs), order_key());
  hipLaunchKernelGGL(mx_pair_t<2>, dim3(gb, I / 64), dim3(256), 0, s, nullptr, PF(L.a), I, perm, w, k,
                     counts, offsets, koff, E, P8(L.aT), P8(L.aTs), order_key());
  hipLaunchKernelGGL(mx_pair_t<0>, dim3(gb, H / 64), dim3(256), 0, s, x, nullptr, H, perm, w, k,
                     counts, offsets, koff, E, P8(L.xT), P8(L.xTs), order_key());
  hipLaunchKernelGGL(mx_pair_t<2>, dim3(gb, 2 * I / 64), dim3(256), 0, s, nullptr, PF(L.dgu), 2 * I,
                     perm, w, k, counts, offsets, koff, E, P8(L.dguT), P8(L.dguTs), order_key());
  // experts averaging at most one 128-pair K stage: 128 x 128 tiles, several workgroups
  // per CU; longer pair runs keep the 256 x 256 tile and its pipelined K loop
  const bool small = static_cast<int64_t>(T) * k <= 128LL * E;
  err = launch_wgrad_large_mx(P8(L.aT), P8(L.aTs), P8(L.dyT), P8(L.dyTs), P8(L.xT), P8(L.xTs),
                              P8(L.dguT), P8(L.dguTs), koff, H, I, E, dwgu, dwd, small, num_cus, s);
  prof_end(kBwdWGateUp, s);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(route_bwd, dim3(T), dim3(64), 0, s, PF(L.dwp), row_of, idx, w, T, E, k, I / kNT,
                     dtw, dlogits, order_key());
  return hipGetLastError();
}


hipError_t backward_set_attributes() {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(bwd_gemm<kDG, 64, 4>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(bwd_lds(64, 4)));
  if (e == hipSuccess)
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(bwd_gemm<kDD, 64, 4>),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(bwd_lds(64, 4)));
  return e;
}

}  // namespace moe
