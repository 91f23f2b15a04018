// Batched path: expert grouping, grouped gate_up / down GEMMs on MFMA, and a
// fixed-order combine (T in the thousands, e.g. 2,048 tokens per GPU as in the
// Mixture-of-Kittens summary, "What is 2.37x measured against").
//
// Data flow (all on the caller's stream, no host synchronisation):
//   group_experts   topk_idx -> per-expert counts and offsets, the stable
//                   permutation perm (sorted row -> token*k + slot; experts
//                   ascending, tokens ascending within an expert), its inverse
//                   row_of, and the list of M-tiles (expert, first row).
//   gate_up GEMM    h[row] = silu(x[tok] . Wg[e]) * (x[tok] . Wu[e]); the x
//                   rows are gathered through perm inside the operand loads,
//                   so no gathered copy of x exists.
//   down GEMM       y[row] = W_down[e] . h[row]   (FP32, sorted order); with
//                   k = 1 it writes out[t] = bf16(w * y) directly instead.
//   combine         out[t] = sum_{j=0..k-1} w[t,j] * y[row_of[t,j]] in slot
//                   order, FP32, rounded once to BF16.
//
// The workloads this path serves move every resident expert's weights once
// (33.8 GB for 384 experts at H=7168, I=2048) against ~43 rows per expert, so
// the GEMMs are bound by HBM, not by MFMA: each wave streams its own weight
// rows straight from HBM into MFMA operand registers (no LDS round trip), and
// the gathered activation rows come from L2.  Work items are ordered so that
// the items sharing one expert's activation rows run on the same XCD (same
// L2): workgroups are dispatched to the 8 XCDs round-robin by linear id.
#include "common.h"
#include "internal.h"

namespace moe {

namespace {
constexpr int kBM = 64;            // rows (routed pairs) per M-tile
constexpr int kGuNeurons = 128;    // neurons per gate_up workgroup (4 waves x 32)
constexpr int kDnRows = 256;       // output dims per down workgroup (4 waves x 64)
constexpr int kXcds = 8;
constexpr int kStagesBf16 = 2;   // register pipeline depth of the BF16 GEMMs
constexpr int kStagesMx = 2;     // and of the MXFP8 GEMMs

inline size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }
}  // namespace

BatchedWs batched_ws_layout(int T, int H, int I, int E, int k, int dtype) {
  (void)I;
  (void)dtype;
  BatchedWs L{};
  const size_t P = static_cast<size_t>(T) * k;
  L.max_tiles = static_cast<int>(E + (P + kBM - 1) / kBM);
  size_t o = 0;
  L.n_tiles = o;   o += 256;
  L.counts = o;    o = align256(o + sizeof(int) * E);
  L.offsets = o;   o = align256(o + sizeof(int) * (E + 1));
  L.tiles = o;     o = align256(o + sizeof(int) * 2 * L.max_tiles);
  L.perm = o;      o = align256(o + sizeof(int) * P);
  L.row_of = o;    o = align256(o + sizeof(int) * P);
  L.y = o;
  if (k > 1) o = align256(o + sizeof(float) * P * H);
  L.total = o;
  return L;
}

// ---------------------------------------------------------------------------
// Expert grouping.  Workgroup e builds the full expert histogram in LDS
// (integer atomics: the totals do not depend on their order), takes its own
// offset and tile offset from the counts of experts < e, then walks the pairs
// in order and compacts those routed to e with wave ballots, so the order
// inside an expert is ascending pair id (= ascending token).  Pairs whose id
// is out of range get row_of = P (ignored downstream) from workgroup 0.
__global__ __launch_bounds__(1024) void group_experts(
    const int32_t* __restrict__ idx, int P, int E, int BM, int* __restrict__ counts,
    int* __restrict__ offsets, int2* __restrict__ tiles, int* __restrict__ n_tiles,
    int* __restrict__ perm, int* __restrict__ row_of) {
  __shared__ int hist[1024];
  __shared__ int s_red[2][16];
  __shared__ int s_wcnt[16];
  const int tid = threadIdx.x, wv = wave_id(), lane = lane_id();
  const int e = blockIdx.x;
  for (int i = tid; i < E; i += blockDim.x) hist[i] = 0;
  __syncthreads();
  for (int i = tid; i < P; i += blockDim.x) {
    const unsigned v = static_cast<unsigned>(idx[i]);
    if (v < static_cast<unsigned>(E)) atomicAdd(&hist[v], 1);
    else if (e == 0) row_of[i] = P;
  }
  __syncthreads();
  // offsets of expert e: sum of counts and of tile counts over experts < e
  int c_sum = 0, t_sum = 0;
  for (int i = tid; i < e; i += blockDim.x) {
    c_sum += hist[i];
    t_sum += (hist[i] + BM - 1) / BM;
  }
  for (int m = 32; m >= 1; m >>= 1) {
    c_sum += __shfl_xor(c_sum, m, kWave);
    t_sum += __shfl_xor(t_sum, m, kWave);
  }
  if (lane == 0) {
    s_red[0][wv] = c_sum;
    s_red[1][wv] = t_sum;
  }
  __syncthreads();
  int off = 0, toff = 0;
  const int nw = blockDim.x / kWave;
  for (int w = 0; w < nw; ++w) {
    off += s_red[0][w];
    toff += s_red[1][w];
  }
  const int cnt = hist[e];
  const int ntile = (cnt + BM - 1) / BM;
  if (tid == 0) {
    counts[e] = cnt;
    offsets[e] = off;
    if (e == E - 1) {
      offsets[E] = off + cnt;
      *n_tiles = toff + ntile;
    }
  }
  for (int q = tid; q < ntile; q += blockDim.x) tiles[toff + q] = make_int2(e, q * BM);
  // ordered compaction of the pairs routed to e
  int running = 0;
  for (int base = 0; base < P; base += blockDim.x) {
    const int i = base + tid;
    const bool match = i < P && idx[i] == e;
    const uint64_t b = __ballot(match);
    if (lane == 0) s_wcnt[wv] = __popcll(b);
    __syncthreads();
    int before = 0, total = 0;
    for (int w = 0; w < nw; ++w) {
      const int c = s_wcnt[w];
      before += w < wv ? c : 0;
      total += c;
    }
    if (match) {
      const int pos = off + running + before + __popcll(b & ((1ull << lane) - 1));
      perm[pos] = i;
      row_of[i] = pos;
    }
    running += total;
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Work-item order: item L of a 1-D grid (dispatched to XCD L % 8) takes the
// (L % 8)-th eighth of the item space, so consecutive items - the N-blocks of
// one M-tile - share an XCD.  n_items must be a multiple of 8.
__device__ __forceinline__ int xcd_item(int L, int n_items) {
  return (L % kXcds) * (n_items / kXcds) + L / kXcds;
}

// gate_up, BF16: workgroup = (M-tile, 128 neurons); wave = 32 neurons (16
// gate rows + 16 up rows in two groups) x 64 rows.  MFMA 16x16x32: A = weight
// rows (lane: row col, K chunk grp), B = activation rows, D[row][token].
// The K loop is double-buffered in registers: the loads of step ks + 1 are
// issued before the MFMAs of step ks, so every wave keeps a step of weights
// in flight while it computes.  Rows past the tile's end load the tile's first row;
// their MFMA columns are computed and discarded (columns never mix).
template <int D>
__global__ __launch_bounds__(256) void gemm_gate_up_bf16(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wgu,
    const int* __restrict__ perm, const int2* __restrict__ tiles, const int* __restrict__ n_tiles,
    const int* __restrict__ counts, const int* __restrict__ offsets, int H, int I, int k,
    int n_items, uint16_t* __restrict__ h) {
  const int nblk = I / kGuNeurons;
  const int item = xcd_item(blockIdx.x, n_items);
  const int tile = item / nblk, nb_i = item - tile * nblk;
  if (tile >= *n_tiles) return;
  const int2 te = tiles[tile];
  const int e = te.x, m0 = te.y;
  const int mcount = min(kBM, counts[e] - m0);
  const int rbase = offsets[e] + m0;
  const int wv = wave_id(), ln = lane_id(), col = ln & 15, grp = ln >> 4;
  const int nb = nb_i * kGuNeurons + wv * 32;

  const uint16_t* __restrict__ wb = wgu + static_cast<size_t>(e) * 2 * I * H;
  uint32_t og[2], ou[2], ox[4];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    og[q] = static_cast<uint32_t>((nb + 16 * q + col) * H + grp * 8);
    ou[q] = og[q] + static_cast<uint32_t>(I * H);
  }
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int r = 16 * g + col;
    ox[g] = static_cast<uint32_t>((perm[rbase + (r < mcount ? r : 0)] / k) * H + grp * 8);
  }
  f32x4 ag[2][4], au[2][4];
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int g = 0; g < 4; ++g) ag[q][g] = au[q][g] = f32x4{0.f, 0.f, 0.f, 0.f};

  bf16x8 bg[D][2], bu[D][2], bx[D][4];
#define GU_LOAD(S, KO)                                                    \
  {                                                                       \
    _Pragma("unroll") for (int q = 0; q < 2; ++q) {                       \
      bg[S][q] = as_bf16x8(ld16(wb + og[q] + (KO)));                      \
      bu[S][q] = as_bf16x8(ld16(wb + ou[q] + (KO)));                      \
    }                                                                     \
    _Pragma("unroll") for (int g = 0; g < 4; ++g) bx[S][g] = as_bf16x8(ld16(x + ox[g] + (KO))); \
  }
  const int ksteps = H / 32;
#define GU_MMA(S)                                                             \
  _Pragma("unroll") for (int q = 0; q < 2; ++q)                               \
  _Pragma("unroll") for (int g = 0; g < 4; ++g) {                             \
    ag[q][g] = mfma16x16x32(bg[S][q], bx[S][g], ag[q][g]);                    \
    au[q][g] = mfma16x16x32(bu[S][q], bx[S][g], au[q][g]);                    \
  }
  GU_LOAD(0, 0)
  const int kpairs = ksteps & ~1;
  for (int ks = 0; ks < kpairs; ks += 2) {
    GU_LOAD(1, (ks + 1) * 32)
    GU_MMA(0)
    GU_LOAD(0, min(ks + 2, ksteps - 1) * 32)
    GU_MMA(1)
  }
  if (ksteps & 1) { GU_MMA(0) }
#undef GU_MMA
#undef GU_LOAD
  // SwiGLU epilogue: lane holds neurons nb+16q+4grp+{0..3} of row 16g+col
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int r = 16 * g + col;
    if (r >= mcount) continue;
    uint16_t* hr = h + static_cast<size_t>(rbase + r) * I + nb + 4 * grp;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      uint32_t p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = f32_to_bf16_rne(swiglu(ag[q][g][i], au[q][g][i]));
      uint2 v;
      v.x = p[0] | (p[1] << 16);
      v.y = p[2] | (p[3] << 16);
      *reinterpret_cast<uint2*>(hr + 16 * q) = v;
    }
  }
}

// down, BF16: workgroup = (M-tile, 256 output dims); wave = 64 dims (4 groups)
// x 64 rows; the same double-buffered K loop.  FUSED (k = 1): out[t] = bf16(w[t] * y)
// with t = perm[row].
template <bool FUSED, int D>
__global__ __launch_bounds__(256) void gemm_down_bf16(
    const uint16_t* __restrict__ h, const uint16_t* __restrict__ wd,
    const int* __restrict__ perm, const int2* __restrict__ tiles, const int* __restrict__ n_tiles,
    const int* __restrict__ counts, const int* __restrict__ offsets, const float* __restrict__ w,
    int H, int I, int n_items, float* __restrict__ y, uint16_t* __restrict__ out) {
  const int nblk = H / kDnRows;
  const int item = xcd_item(blockIdx.x, n_items);
  const int tile = item / nblk, db_i = item - tile * nblk;
  if (tile >= *n_tiles) return;
  const int2 te = tiles[tile];
  const int e = te.x, m0 = te.y;
  const int mcount = min(kBM, counts[e] - m0);
  const int rbase = offsets[e] + m0;
  const int wv = wave_id(), ln = lane_id(), col = ln & 15, grp = ln >> 4;
  const int db = db_i * kDnRows + wv * 64;

  const uint16_t* __restrict__ wb = wd + static_cast<size_t>(e) * H * I;
  const uint16_t* __restrict__ hb = h + static_cast<size_t>(rbase) * I;
  uint32_t ow[4], oh[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) ow[q] = static_cast<uint32_t>((db + 16 * q + col) * I + grp * 8);
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int r = 16 * g + col;
    oh[g] = static_cast<uint32_t>((r < mcount ? r : 0) * I + grp * 8);
  }
  f32x4 acc[4][4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int g = 0; g < 4; ++g) acc[q][g] = f32x4{0.f, 0.f, 0.f, 0.f};

  bf16x8 ba[D][4], bb[D][4];
#define DN_LOAD(S, KO)                                                                   \
  {                                                                                      \
    _Pragma("unroll") for (int q = 0; q < 4; ++q) ba[S][q] = as_bf16x8(ld16(wb + ow[q] + (KO))); \
    _Pragma("unroll") for (int g = 0; g < 4; ++g) bb[S][g] = as_bf16x8(ld16(hb + oh[g] + (KO))); \
  }
  const int ksteps = I / 32;
#define DN_MMA(S)                                                             \
  _Pragma("unroll") for (int q = 0; q < 4; ++q)                               \
  _Pragma("unroll") for (int g = 0; g < 4; ++g)                               \
    acc[q][g] = mfma16x16x32(ba[S][q], bb[S][g], acc[q][g]);
  DN_LOAD(0, 0)
  const int kpairs = ksteps & ~1;
  for (int ks = 0; ks < kpairs; ks += 2) {
    DN_LOAD(1, (ks + 1) * 32)
    DN_MMA(0)
    DN_LOAD(0, min(ks + 2, ksteps - 1) * 32)
    DN_MMA(1)
  }
  if (ksteps & 1) { DN_MMA(0) }
#undef DN_MMA
#undef DN_LOAD
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int r = 16 * g + col;
    if (r >= mcount) continue;
    if (FUSED) {
      const int t = perm[rbase + r];         // k = 1: pair id == token
      const float wt = w[t];
      uint16_t* orow = out + static_cast<size_t>(t) * H + db + 4 * grp;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint2 v;
        v.x = f32_to_bf16_rne(wt * acc[q][g][0]) | (f32_to_bf16_rne(wt * acc[q][g][1]) << 16);
        v.y = f32_to_bf16_rne(wt * acc[q][g][2]) | (f32_to_bf16_rne(wt * acc[q][g][3]) << 16);
        *reinterpret_cast<uint2*>(orow + 16 * q) = v;
      }
    } else {
      float* yr = y + static_cast<size_t>(rbase + r) * H + db + 4 * grp;
#pragma unroll
      for (int q = 0; q < 4; ++q) *reinterpret_cast<f32x4*>(yr + 16 * q) = acc[q][g];
    }
  }
}

// combine: out[t] = sum_j w[t,j] * y[row_of[t*k+j]] in slot order (FP32 FMA
// chain starting from 0), rounded once to BF16.  One workgroup per token.
__global__ __launch_bounds__(256) void combine_slots(const float* __restrict__ y,
                                                     const int* __restrict__ row_of,
                                                     const float* __restrict__ w, int T, int H,
                                                     int k, uint16_t* __restrict__ out) {
  const int t = blockIdx.x;
  const int P = T * k;
  for (int c = threadIdx.x; c < H / 4; c += blockDim.x) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
      const int row = row_of[t * k + j];
      if (static_cast<unsigned>(row) >= static_cast<unsigned>(P)) continue;
      const float wj = w[t * k + j];
      const f32x4 v = *reinterpret_cast<const f32x4*>(y + static_cast<size_t>(row) * H + 4 * c);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = fmaf(wj, v[i], acc[i]);
    }
    uint2 o;
    o.x = f32_to_bf16_rne(acc[0]) | (f32_to_bf16_rne(acc[1]) << 16);
    o.y = f32_to_bf16_rne(acc[2]) | (f32_to_bf16_rne(acc[3]) << 16);
    *reinterpret_cast<uint2*>(out + static_cast<size_t>(t) * H + 4 * c) = o;
  }
}


// ---------------------------------------------------------------------------
// MXFP8.  Blocks of 32 along K share one E8M0 scale 2^s, s = floor(log2 amax)
// - 8 (OCP Microscaling v1.0); codes are E4M3 of v / 2^s, round to nearest
// even, saturated.  The MX forward of the Mixture-of-Kittens summary ("What is
// 2.37x measured against") quantizes both GEMM operands; the activation h is
// quantized here from the FP32 SwiGLU value, never through BF16.

// moe_quantize_mxfp8: four lanes per block of 32 (8 BF16 values each).
__global__ __launch_bounds__(256) void quant_mx_rows(const uint16_t* __restrict__ src,
                                                     int64_t n_blocks, uint8_t* __restrict__ codes,
                                                     uint8_t* __restrict__ scales) {
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t blk = tid >> 2;
  const int part = static_cast<int>(tid & 3);
  const bool live = blk < n_blocks;
  i32x4 raw = {0, 0, 0, 0};
  if (live) raw = ld16(src + blk * 32 + part * 8);
  float v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = static_cast<uint32_t>(raw[i]);
    v[2 * i] = bf16_to_f32(w & 0xFFFFu);
    v[2 * i + 1] = bf16_to_f32(w >> 16);
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));
  amax = fmaxf(amax, __shfl_xor(amax, 2, kWave));
  const int sexp = mx_scale_exp(amax);
  const float inv = exp2_neg(sexp);
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) lo |= f32_to_e4m3(v[i] * inv) << (8 * i);
#pragma unroll
  for (int i = 0; i < 4; ++i) hi |= f32_to_e4m3(v[4 + i] * inv) << (8 * i);
  if (live) {
    *reinterpret_cast<uint2*>(codes + blk * 32 + part * 8) = make_uint2(lo, hi);
    if (part == 0) scales[blk] = static_cast<uint8_t>(sexp + 127);
  }
}

// gate_up, MXFP8: workgroup = (M-tile, 128 neurons); wave = 32 neurons (one
// MX block of h) x 64 rows.  Per 128-wide K chunk a lane loads two 16-byte
// pieces of its weight row and of its activation row, plus the row's scale
// byte for block g of the chunk; double-buffered as the BF16 kernel.
template <int D>
__global__ __launch_bounds__(256) void gemm_gate_up_mx(
    const uint8_t* __restrict__ x, const uint8_t* __restrict__ xs,
    const uint8_t* __restrict__ wgu, const uint8_t* __restrict__ wgus,
    const int* __restrict__ perm, const int2* __restrict__ tiles, const int* __restrict__ n_tiles,
    const int* __restrict__ counts, const int* __restrict__ offsets, int H, int I, int k,
    int n_items, uint8_t* __restrict__ h, uint8_t* __restrict__ hs) {
  const int nblk = I / kGuNeurons;
  const int item = xcd_item(blockIdx.x, n_items);
  const int tile = item / nblk, nb_i = item - tile * nblk;
  if (tile >= *n_tiles) return;
  const int2 te = tiles[tile];
  const int e = te.x, m0 = te.y;
  const int mcount = min(kBM, counts[e] - m0);
  const int rbase = offsets[e] + m0;
  const int wv = wave_id(), ln = lane_id(), col = ln & 15, grp = ln >> 4;
  const int nb = nb_i * kGuNeurons + wv * 32;
  const int KB = H / 32;                               // scale bytes per row

  const uint8_t* __restrict__ wb = wgu + static_cast<size_t>(e) * 2 * I * H;
  const uint8_t* __restrict__ wsb = wgus + static_cast<size_t>(e) * 2 * I * KB;
  uint32_t og[2], ou[2], osg[2], osu[2], ox[4], osx[4];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int rg = nb + 16 * q + col, ru = rg + I;
    og[q] = static_cast<uint32_t>(rg * H + 16 * grp);
    ou[q] = static_cast<uint32_t>(ru * H + 16 * grp);
    osg[q] = static_cast<uint32_t>(rg * KB + grp);
    osu[q] = static_cast<uint32_t>(ru * KB + grp);
  }
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int r = 16 * g + col;
    const int tok = perm[rbase + (r < mcount ? r : 0)] / k;
    ox[g] = static_cast<uint32_t>(tok * H + 16 * grp);
    osx[g] = static_cast<uint32_t>(tok * KB + grp);
  }
  f32x4 ag[2][4], au[2][4];
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int g = 0; g < 4; ++g) ag[q][g] = au[q][g] = f32x4{0.f, 0.f, 0.f, 0.f};

  i32x8 bg[D][2], bu[D][2], bx[D][4];
  int sg[D][2], su[D][2], sx[D][4];
#define GUM_LOAD(S, KC)                                                               \
  {                                                                                   \
    const int ko = (KC) * 128, so = (KC) * 4;                                         \
    _Pragma("unroll") for (int q = 0; q < 2; ++q) {                                   \
      bg[S][q] = cat8(ld16(wb + og[q] + ko), ld16(wb + og[q] + ko + 64));             \
      bu[S][q] = cat8(ld16(wb + ou[q] + ko), ld16(wb + ou[q] + ko + 64));             \
      sg[S][q] = wsb[osg[q] + so];                                                    \
      su[S][q] = wsb[osu[q] + so];                                                    \
    }                                                                                 \
    _Pragma("unroll") for (int g = 0; g < 4; ++g) {                                   \
      bx[S][g] = cat8(ld16(x + ox[g] + ko), ld16(x + ox[g] + ko + 64));               \
      sx[S][g] = xs[osx[g] + so];                                                     \
    }                                                                                 \
  }
  const int chunks = H / 128;
#define GUM_MMA(S)                                                                      \
  _Pragma("unroll") for (int q = 0; q < 2; ++q)                                         \
  _Pragma("unroll") for (int g = 0; g < 4; ++g) {                                       \
    ag[q][g] = mfma_mx16x16x128(bg[S][q], bx[S][g], sg[S][q], sx[S][g], ag[q][g]);      \
    au[q][g] = mfma_mx16x16x128(bu[S][q], bx[S][g], su[S][q], sx[S][g], au[q][g]);      \
  }
  GUM_LOAD(0, 0)
  const int kpairs = chunks & ~1;
  for (int kc = 0; kc < kpairs; kc += 2) {
    GUM_LOAD(1, kc + 1)
    GUM_MMA(0)
    GUM_LOAD(0, min(kc + 2, chunks - 1))
    GUM_MMA(1)
  }
  if (chunks & 1) { GUM_MMA(0) }
#undef GUM_MMA
#undef GUM_LOAD
  // SwiGLU, then MX-quantize the 32 neurons [nb, nb+32) of each row: lanes
  // col + 16*grp (grp = 0..3) hold them (4 per q group each).
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int r = 16 * g + col;
    float a[2][4];
    float amax = 0.f;
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[q][i] = swiglu(ag[q][g][i], au[q][g][i]);
        amax = fmaxf(amax, fabsf(a[q][i]));
      }
    amax = fmaxf(amax, __shfl_xor(amax, 16, kWave));
    amax = fmaxf(amax, __shfl_xor(amax, 32, kWave));
    if (r >= mcount) continue;
    const int sexp = mx_scale_exp(amax);
    const float inv = exp2_neg(sexp);
    uint8_t* hr = h + static_cast<size_t>(rbase + r) * I + nb + 4 * grp;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      uint32_t wq = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) wq |= f32_to_e4m3(a[q][i] * inv) << (8 * i);
      *reinterpret_cast<uint32_t*>(hr + 16 * q) = wq;
    }
    if (grp == 0) hs[static_cast<size_t>(rbase + r) * (I / 32) + nb / 32] = static_cast<uint8_t>(sexp + 127);
  }
}

// down, MXFP8: as the BF16 down kernel with 128-wide scaled K chunks.
template <bool FUSED, int D>
__global__ __launch_bounds__(256) void gemm_down_mx(
    const uint8_t* __restrict__ h, const uint8_t* __restrict__ hs,
    const uint8_t* __restrict__ wd, const uint8_t* __restrict__ wds,
    const int* __restrict__ perm, const int2* __restrict__ tiles, const int* __restrict__ n_tiles,
    const int* __restrict__ counts, const int* __restrict__ offsets, const float* __restrict__ w,
    int H, int I, int n_items, float* __restrict__ y, uint16_t* __restrict__ out) {
  const int nblk = H / kDnRows;
  const int item = xcd_item(blockIdx.x, n_items);
  const int tile = item / nblk, db_i = item - tile * nblk;
  if (tile >= *n_tiles) return;
  const int2 te = tiles[tile];
  const int e = te.x, m0 = te.y;
  const int mcount = min(kBM, counts[e] - m0);
  const int rbase = offsets[e] + m0;
  const int wv = wave_id(), ln = lane_id(), col = ln & 15, grp = ln >> 4;
  const int db = db_i * kDnRows + wv * 64;
  const int KB = I / 32;

  const uint8_t* __restrict__ wb = wd + static_cast<size_t>(e) * H * I;
  const uint8_t* __restrict__ wsb = wds + static_cast<size_t>(e) * H * KB;
  const uint8_t* __restrict__ hb = h + static_cast<size_t>(rbase) * I;
  const uint8_t* __restrict__ hsb = hs + static_cast<size_t>(rbase) * KB;
  uint32_t ow[4], osw[4], oh[4], osh[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = db + 16 * q + col;
    ow[q] = static_cast<uint32_t>(row * I + 16 * grp);
    osw[q] = static_cast<uint32_t>(row * KB + grp);
  }
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int r = 16 * g + col;
    const int rr = r < mcount ? r : 0;
    oh[g] = static_cast<uint32_t>(rr * I + 16 * grp);
    osh[g] = static_cast<uint32_t>(rr * KB + grp);
  }
  f32x4 acc[4][4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int g = 0; g < 4; ++g) acc[q][g] = f32x4{0.f, 0.f, 0.f, 0.f};

  i32x8 ba[D][4], bb[D][4];
  int sa[D][4], sb[D][4];
#define DNM_LOAD(S, KC)                                                               \
  {                                                                                   \
    const int ko = (KC) * 128, so = (KC) * 4;                                         \
    _Pragma("unroll") for (int q = 0; q < 4; ++q) {                                   \
      ba[S][q] = cat8(ld16(wb + ow[q] + ko), ld16(wb + ow[q] + ko + 64));             \
      sa[S][q] = wsb[osw[q] + so];                                                    \
    }                                                                                 \
    _Pragma("unroll") for (int g = 0; g < 4; ++g) {                                   \
      bb[S][g] = cat8(ld16(hb + oh[g] + ko), ld16(hb + oh[g] + ko + 64));             \
      sb[S][g] = hsb[osh[g] + so];                                                    \
    }                                                                                 \
  }
  const int chunks = I / 128;
#define DNM_MMA(S)                                                                       \
  _Pragma("unroll") for (int q = 0; q < 4; ++q)                                          \
  _Pragma("unroll") for (int g = 0; g < 4; ++g)                                          \
    acc[q][g] = mfma_mx16x16x128(ba[S][q], bb[S][g], sa[S][q], sb[S][g], acc[q][g]);
  DNM_LOAD(0, 0)
  const int kpairs = chunks & ~1;
  for (int kc = 0; kc < kpairs; kc += 2) {
    DNM_LOAD(1, kc + 1)
    DNM_MMA(0)
    DNM_LOAD(0, min(kc + 2, chunks - 1))
    DNM_MMA(1)
  }
  if (chunks & 1) { DNM_MMA(0) }
#undef DNM_MMA
#undef DNM_LOAD
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int r = 16 * g + col;
    if (r >= mcount) continue;
    if (FUSED) {
      const int t = perm[rbase + r];
      const float wt = w[t];
      uint16_t* orow = out + static_cast<size_t>(t) * H + db + 4 * grp;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint2 v;
        v.x = f32_to_bf16_rne(wt * acc[q][g][0]) | (f32_to_bf16_rne(wt * acc[q][g][1]) << 16);
        v.y = f32_to_bf16_rne(wt * acc[q][g][2]) | (f32_to_bf16_rne(wt * acc[q][g][3]) << 16);
        *reinterpret_cast<uint2*>(orow + 16 * q) = v;
      }
    } else {
      float* yr = y + static_cast<size_t>(rbase + r) * H + db + 4 * grp;
#pragma unroll
      for (int q = 0; q < 4; ++q) *reinterpret_cast<f32x4*>(yr + 16 * q) = acc[q][g];
    }
  }
}

// ---------------------------------------------------------------------------
namespace {
struct BatchedPtrs {
  int *n_tiles, *counts, *offsets, *perm, *row_of;
  int2* tiles;
  float* y;
};
BatchedPtrs batched_ptrs(void* ws, const BatchedWs& L) {
  char* b = static_cast<char*>(ws);
  BatchedPtrs p;
  p.n_tiles = reinterpret_cast<int*>(b + L.n_tiles);
  p.counts = reinterpret_cast<int*>(b + L.counts);
  p.offsets = reinterpret_cast<int*>(b + L.offsets);
  p.tiles = reinterpret_cast<int2*>(b + L.tiles);
  p.perm = reinterpret_cast<int*>(b + L.perm);
  p.row_of = reinterpret_cast<int*>(b + L.row_of);
  p.y = reinterpret_cast<float*>(b + L.y);
  return p;
}
int round_up(int v, int m) { return (v + m - 1) / m * m; }
}  // namespace

hipError_t launch_gate_up_batched(const void* x, const uint8_t* xs, const void* wgu,
                                  const uint8_t* wgus, const int32_t* idx, int T, int H, int I,
                                  int E, int k, int dtype, void* h, uint8_t* hs, void* ws,
                                  hipStream_t s, int num_cus) {
  (void)num_cus;
  const BatchedWs L = batched_ws_layout(T, H, I, E, k, dtype);
  const BatchedPtrs p = batched_ptrs(ws, L);
  const int P = T * k;
  prof_begin(kGroup, s);
  hipLaunchKernelGGL(group_experts, dim3(E), dim3(1024), 0, s, idx, P, E, kBM, p.counts,
                     p.offsets, p.tiles, p.n_tiles, p.perm, p.row_of);
  prof_end(kGroup, s);
  const int n_items = round_up((I / kGuNeurons) * L.max_tiles, kXcds);
  prof_begin(kGemmGateUp, s);
  if (dtype == 0)
    hipLaunchKernelGGL(gemm_gate_up_bf16<kStagesBf16>, dim3(n_items), dim3(256), 0, s,
                       static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(wgu), p.perm,
                       p.tiles, p.n_tiles, p.counts, p.offsets, H, I, k, n_items,
                       static_cast<uint16_t*>(h));
  else
    hipLaunchKernelGGL(gemm_gate_up_mx<kStagesMx>, dim3(n_items), dim3(256), 0, s,
                       static_cast<const uint8_t*>(x), xs, static_cast<const uint8_t*>(wgu), wgus,
                       p.perm, p.tiles, p.n_tiles, p.counts, p.offsets, H, I, k, n_items,
                       static_cast<uint8_t*>(h), hs);
  prof_end(kGemmGateUp, s);
  return hipGetLastError();
}

hipError_t launch_down_batched(const void* h, const uint8_t* hs, const void* wd,
                               const uint8_t* wds, const int32_t* idx, const float* w, int T,
                               int H, int I, int E, int k, int dtype, uint16_t* out, void* ws,
                               hipStream_t s, int num_cus) {
  (void)idx; (void)num_cus;
  const BatchedWs L = batched_ws_layout(T, H, I, E, k, dtype);
  const BatchedPtrs p = batched_ptrs(ws, L);
  const int n_items = round_up((H / kDnRows) * L.max_tiles, kXcds);
  prof_begin(kGemmDown, s);
  if (dtype != 0) {
    const uint8_t* hc = static_cast<const uint8_t*>(h);
    const uint8_t* wc = static_cast<const uint8_t*>(wd);
    if (k == 1)
      hipLaunchKernelGGL((gemm_down_mx<true, kStagesMx>), dim3(n_items), dim3(256), 0, s, hc, hs, wc, wds,
                         p.perm, p.tiles, p.n_tiles, p.counts, p.offsets, w, H, I, n_items, p.y,
                         out);
    else
      hipLaunchKernelGGL((gemm_down_mx<false, kStagesMx>), dim3(n_items), dim3(256), 0, s, hc, hs, wc, wds,
                         p.perm, p.tiles, p.n_tiles, p.counts, p.offsets, w, H, I, n_items, p.y,
                         out);
  } else if (k == 1)
    hipLaunchKernelGGL((gemm_down_bf16<true, kStagesBf16>), dim3(n_items), dim3(256), 0, s,
                       static_cast<const uint16_t*>(h), static_cast<const uint16_t*>(wd), p.perm,
                       p.tiles, p.n_tiles, p.counts, p.offsets, w, H, I, n_items, p.y, out);
  else
    hipLaunchKernelGGL((gemm_down_bf16<false, kStagesBf16>), dim3(n_items), dim3(256), 0, s,
                       static_cast<const uint16_t*>(h), static_cast<const uint16_t*>(wd), p.perm,
                       p.tiles, p.n_tiles, p.counts, p.offsets, w, H, I, n_items, p.y, out);
  prof_end(kGemmDown, s);
  if (k > 1) {
    prof_begin(kCombine, s);
    hipLaunchKernelGGL(combine_slots, dim3(T), dim3(256), 0, s, p.y, p.row_of, w, T, H, k, out);
    prof_end(kCombine, s);
  }
  return hipGetLastError();
}

hipError_t launch_quant_mx(const uint16_t* src, int64_t rows, int K, uint8_t* codes,
                           uint8_t* scales, hipStream_t s) {
  const int64_t n_blocks = rows * (K / 32);
  const int64_t threads = n_blocks * 4;
  const int64_t grid = (threads + 255) / 256;
  prof_begin(kQuant, s);
  hipLaunchKernelGGL(quant_mx_rows, dim3(static_cast<unsigned>(grid)), dim3(256), 0, s, src,
                     n_blocks, codes, scales);
  prof_end(kQuant, s);
  return hipGetLastError();
}

hipError_t batched_set_attributes() { return hipSuccess; }

}  // namespace moe
