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
#include "tiles.h"

namespace moe {

namespace {
constexpr int kBM = 64;            // rows (routed pairs) per M-tile
constexpr int kTallBM = 128;       // BF16, experts averaging 48+ rows

inline size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }
}  // namespace

bool use_large_tiles(int T, int H, int I, int E, int k, int dtype) {
  const int64_t P = static_cast<int64_t>(T) * k;
  return (dtype == 0 || dtype == 1) && P >= static_cast<int64_t>(kLargeBM) * E && H % 256 == 0 &&
         I % 128 == 0;
}

BatchedWs batched_ws_layout(int T, int H, int I, int E, int k, int dtype) {
  BatchedWs L{};
  const size_t P = static_cast<size_t>(T) * k;
  // BF16 takes 128-row tiles when experts average 48 routed rows or more (with
  // 64-row tiles about half of them would stream their weights twice)
  L.bm = use_large_tiles(T, H, I, E, k, dtype) ? kLargeBM
         : dtype == 0 && P >= 48 * static_cast<size_t>(E) ? kTallBM : kBM;
  L.max_tiles = static_cast<int>(E + (P + L.bm - 1) / L.bm);
  size_t o = 0;
  L.n_tiles = o;   o += 256;
  L.counts = o;    o = align256(o + sizeof(int) * E);
  L.offsets = o;   o = align256(o + sizeof(int) * (E + 1));
  L.tiles = o;     o = align256(o + sizeof(int) * 2 * L.max_tiles);
  L.perm = o;      o = align256(o + sizeof(int) * P);
  L.row_of = o;    o = align256(o + sizeof(int) * P);
  L.y = o;
  if (k > 1) o = align256(o + sizeof(float) * P * H);
  L.partial = o;
  if (L.bm == kLargeBM) o = align256(o + sizeof(float) * kLargeMaxSlices * kLargeBM * 256);
  L.sct = o;                 // MXFP8 large tiles: transposed scale dwords
  if (L.bm == kLargeBM && dtype == 1) o = align256(o + mx_scales_t_bytes(static_cast<int>(P), H, I, E));
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
    int* __restrict__ perm, int* __restrict__ row_of, uint32_t okey) {
  __shared__ int hist[1024];
  __shared__ int s_red[2][16];
  __shared__ int s_wcnt[16];
  const int tid = threadIdx.x, wv = wave_id(), lane = lane_id();
  const int e = permute_item(blockIdx.x, gridDim.x, okey);
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

// Batched BF16 projections with a whole-line weight stream (both gate_up and
// down): workgroup = (M-tile of 64 routed rows, NW waves); each wave owns two
// groups of 16 weight rows - gate_up (KIND 0): 16 neurons' gate rows and their
// up rows; down (KIND 1, 2): 32 output dimensions - and all 64 rows of the
// tile.  Each 64-position K step of a wave reads its 32 weight rows as four
// loads of 8 rows x 128 contiguous bytes (whole cache lines, non-temporal: the
// weights are read once per M-tile); a plain 16x16x32 A operand would take 16
// rows x 64 bytes per load, half lines, which stream markedly slower.  Each
// 8-row load goes through a wave-private 2 KB LDS tile (16-byte chunks
// XOR-swizzled by row, so the one-row-per-lane reads hit distinct banks) and is
// read back in the A layout, one 16-row group at a time.  The tile's 64
// activation rows (gathered through perm for gate_up, contiguous in h for
// down) are staged in LDS in 128-wide K chunks, double-buffered and shared by
// the waves; the next step's weights are in flight while a step multiplies.
// Rows past the tile's end load the tile's first row; their MFMA columns are
// computed and discarded (columns never mix).
// Epilogues: KIND 0 SwiGLU -> h (BF16); KIND 3 the same, and also the FP32
// pre-activations g and u of each pair in slot order (for the backward pass);
// KIND 1 FP32 y per slot; KIND 2 (k = 1) out[t] = bf16(w[t] * y) with t = perm[row].
// A launch covers the output column blocks [cb0, cb0 + ncb) of NW * RPW outputs
// each (ncb 0: all of them); KIND 1 writes y with row stride ldy, its column 0
// being output column cb0 * NW * RPW.
constexpr int kSXC = 128;                // K chunk of the staged activations
constexpr int kSXRS = kSXC + 8;          // padded LDS row stride (elements)
enum { kProjGateUp = 0, kProjDown = 1, kProjDownFused = 2, kProjGateUpSave = 3, kProjGatherRows = 4,
       kProjGateUpRaw = 5 };

// BM = 128 (experts averaging 48 routed rows or more, where 64-row tiles would
// stream about half the experts' weights twice): the tile's 128 rows in eight
// 16-row groups, and each wave owns ONE group of 16 weight rows - gate_up: 8
// neurons' gate rows then their up rows, so a lane pairs its gate values with
// the up values of lane + 32; down: 16 output dimensions - which keeps the
// accumulators (and registers) of the 64-row form.
template <int KIND, int NW, int BM = 64, int NGW = 2>   // (128 registers: with NW = 8, two workgroups share a CU)
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(BM == 128 && NGW == 2 ? 2 : 4, 8))) void gemm_bf16s(
    const uint16_t* __restrict__ act, const uint16_t* __restrict__ wt,
    const int* __restrict__ perm, const int2* __restrict__ tiles, const int* __restrict__ n_tiles,
    const int* __restrict__ counts, const int* __restrict__ offsets, const float* __restrict__ w,
    int H, int I, int k, uint16_t* __restrict__ hout, float* __restrict__ y,
    uint16_t* __restrict__ out, float* __restrict__ gu, uint32_t okey, int cb0, int ncb, int ldy) {
  constexpr bool GU = KIND == kProjGateUp || KIND == kProjGateUpSave;
  constexpr bool ONE = NGW == 1;         // one 16-row weight group per wave
  constexpr int NT = NW * 64;
  constexpr int G = BM / 16;             // 16-row groups of the tile
  constexpr int RPW = (GU ? 16 : 32) * NGW / 2;           // outputs per wave
  constexpr int LPT = BM * (kSXC / 8) / NT;               // 16-byte activation loads per thread
  __shared__ __align__(16) uint16_t xs[2][BM * kSXRS];
  __shared__ __align__(16) i32x4 wtl[NW][16 * 8];         // per wave: [16 rows][8 chunks]
  const int K = GU ? H : I;              // reduction length
  const int N = GU ? I : H;              // outputs
  const int nblk = ncb ? ncb : N / (NW * RPW);
  const int item0 = real_item(blockIdx.x, nblk, *n_tiles);
  if (item0 < 0) return;
  const int item = permute_item(item0, nblk * *n_tiles, okey);
  const int tile = item / nblk, nb_i = item - tile * nblk;
  const int2 te = tiles[tile];
  const int e = te.x, m0 = te.y;
  const int mcount = min(BM, counts[e] - m0);
  const int rbase = offsets[e] + m0;
  const int tid = threadIdx.x, ln = tid & 63, col = ln & 15, grp = ln >> 4;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nb = (cb0 + nb_i) * NW * RPW + wv * RPW;      // the wave's first output
  // the wave's 16-row weight groups (BM 64: two; BM 128: one, rows 0-7 from row0
  // and rows 8-15 from row1)
  const int row0 = nb, row1 = GU ? I + nb : nb + (ONE ? 8 : 16);

  // whole-line loads: lane = (row lr of an 8-row group, 16-byte chunk lc)
  const int lr = ln >> 3, lc = ln & 7;
  const uint16_t* __restrict__ wb = wt + static_cast<size_t>(e) * (GU ? 2 * I : H) * K;
  constexpr int NWL = 2 * NGW;                            // 8-row weight loads per step
  uint32_t ow[NWL];                                       // BM 64: group 0 rows 0-7, 8-15, group 1 rows 0-7, 8-15
#pragma unroll
  for (int i = 0; i < NWL; ++i)
    ow[i] = ONE ? static_cast<uint32_t>(((i == 0 ? row0 : row1) + lr) * K + lc * 8)
                 : static_cast<uint32_t>(((i < 2 ? row0 : row1) + 8 * (i & 1) + lr) * K + lc * 8);
  i32x4* tw = wtl[wv];
  i32x4* wdst = tw + lr * 8 + (lc ^ lr);                  // + 64 for rows 8-15
  // A lane (row col, group grp), 32-half hh: chunk 4*hh + grp of row col
  const i32x4* asrc = tw + col * 8;
  const int sw = col & 7;

  // cooperative activation loader: chunk c = tid + i*NT -> (row c/16, 16-byte column c%16)
  uint32_t oxl[LPT];
  int lrow[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int c = tid + i * NT, r = c >> 4, rr = r < mcount ? r : 0;
    lrow[i] = r * kSXRS + (c & 15) * 8;
    const int arow = GU ? perm[rbase + rr] / k : rbase + rr;
    oxl[i] = static_cast<uint32_t>(arow * K + (c & 15) * 8);
  }
  i32x4 xr[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) xr[i] = ld16(act + oxl[i]);
#pragma unroll
  for (int i = 0; i < LPT; ++i) *reinterpret_cast<i32x4*>(&xs[0][lrow[i]]) = xr[i];

  f32x4 acc0[G], acc1[ONE ? 1 : G];                       // [row group g of the tile]
#pragma unroll
  for (int g = 0; g < G; ++g) acc0[g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int g = 0; g < (ONE ? 1 : G); ++g) acc1[g] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nsteps = K / 64;
  i32x4 wA[NWL], wB[NWL];
#pragma unroll
  for (int i = 0; i < NWL; ++i) wA[i] = ld16_stream(wb + ow[i]);
  __syncthreads();

  // one 64-position step: weights W (already loaded), activations from xs[buf] at
  // chunk offset st*64
  auto step = [&](const i32x4 (&W)[NWL], int buf, int st) {
    const uint16_t* xb = &xs[buf][col * kSXRS + st * 64 + grp * 8];
    if (!ONE) {
      bf16x8 bx[G][2];
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          bx[g][hh] = as_bf16x8(*reinterpret_cast<const i32x4*>(xb + 16 * g * kSXRS + hh * 32));
#pragma unroll
      for (int m = 0; m < 2; ++m) {                       // row group 0, then 1
        wdst[0] = W[2 * m];
        wdst[64] = W[2 * m + 1];
        __builtin_amdgcn_wave_barrier();
        bf16x8 a[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) a[hh] = as_bf16x8(asrc[(4 * hh + grp) ^ sw]);
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            if (m == 0) acc0[g] = mfma16x16x32(a[hh], bx[g][hh], acc0[g]);
            else acc1[(ONE ? 0 : g)] = mfma16x16x32(a[hh], bx[g][hh], acc1[(ONE ? 0 : g)]);
          }
      }
    } else {
      wdst[0] = W[0];
      wdst[64] = W[1];
      __builtin_amdgcn_wave_barrier();
      bf16x8 a[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) a[hh] = as_bf16x8(asrc[(4 * hh + grp) ^ sw]);
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int g = 0; g < G; ++g) {
        bf16x8 bx[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          bx[hh] = as_bf16x8(*reinterpret_cast<const i32x4*>(xb + 16 * g * kSXRS + hh * 32));
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) acc0[g] = mfma16x16x32(a[hh], bx[hh], acc0[g]);
      }
    }
  };
  const int nchunk = K / kSXC;
  for (int c = 0; c < nchunk; ++c) {
    const int buf = c & 1;
    const bool more = c + 1 < nchunk;
    if (more) {
#pragma unroll
      for (int i = 0; i < LPT; ++i) xr[i] = ld16(act + oxl[i] + (c + 1) * kSXC);
    }
    // steps 2c (weights in wA) and 2c+1 (wB); the step after each is loaded first
    // (clamped to the last step, a harmless repeat, so the load count is fixed)
    const uint32_t k1 = static_cast<uint32_t>((2 * c + 1) * 64);
    const uint32_t k2 = static_cast<uint32_t>(min(2 * c + 2, nsteps - 1) * 64);
#pragma unroll
    for (int i = 0; i < NWL; ++i) wB[i] = ld16_stream(wb + ow[i] + k1);
    step(wA, buf, 0);
#pragma unroll
    for (int i = 0; i < NWL; ++i) wA[i] = ld16_stream(wb + ow[i] + k2);
    step(wB, buf, 1);
    if (more) {
#pragma unroll
      for (int i = 0; i < LPT; ++i) *reinterpret_cast<i32x4*>(&xs[buf ^ 1][lrow[i]]) = xr[i];
    }
    __syncthreads();
  }
  // epilogue.  BM 64: lane holds outputs nb+4grp+{0..3} (group 0) and
  // row1+4grp+{0..3} (group 1) of tile row 16g+col.  BM 128: lane holds weight
  // rows 4grp+{0..3} of the wave's group - gate_up: gate of neurons nb+4grp+i for
  // grp < 2, up of neurons nb+4(grp-2)+i for grp >= 2; down: outputs nb+4grp+i.
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int r = 16 * g + col;
    f32x4 up;
    if (ONE && GU) {                                      // up values of lane + 32 (all lanes take part)
#pragma unroll
      for (int i = 0; i < 4; ++i) up[i] = __shfl_xor(acc0[g][i], 32, kWave);
    } else {
      up = acc1[ONE ? 0 : g];
    }
    if (r >= mcount || (ONE && GU && grp >= 2)) continue;
    if (GU) {
      uint16_t* hr = hout + static_cast<size_t>(rbase + r) * I + nb + 4 * grp;
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = swiglu(acc0[g][i], up[i]);
      uint2 v;
      v.x = pack_bf16x2(p[0], p[1]);
      v.y = pack_bf16x2(p[2], p[3]);
      st8_stream(hr, v);
      if (KIND == kProjGateUpSave) {                      // FP32 g and u of the pair, slot order
        float* gp = gu + static_cast<size_t>(perm[rbase + r]) * (2 * I) + nb + 4 * grp;
        st16_stream(gp, acc0[g]);
        st16_stream(gp + I, up);
      }
    } else if (KIND == kProjDownFused) {
      const int t = perm[rbase + r];                      // k = 1: pair id == token
      const float wt_ = w[t];
      uint16_t* orow = out + static_cast<size_t>(t) * H + nb + 4 * grp;
#pragma unroll
      for (int m = 0; m < NGW; ++m) {
        const f32x4 a = m == 0 ? acc0[g] : up;
        uint2 v;
        v.x = pack_bf16x2(wt_ * a[0], wt_ * a[1]);
        v.y = pack_bf16x2(wt_ * a[2], wt_ * a[3]);
        *reinterpret_cast<uint2*>(orow + 16 * m) = v;
      }
    } else {
      float* yr = y + static_cast<size_t>(rbase + r) * ldy + (nb - cb0 * NW * RPW) + 4 * grp;
      st16_stream(yr, acc0[g]);
      if (!ONE) st16_stream(yr + 16, up);
    }
  }
}

// combine: out[t] = sum_j w[t,j] * y[row_of[t*k+j]] in slot order (FP32 FMA
// chain starting from 0), rounded once to BF16.  Workgroup (x, y): token x,
// column chunk y of gridDim.y (small batches split the columns so that the
// launch still spreads over the CUs); a launch covers the output columns [col0,
// col0 + cols), y holding them with row stride ldy from its column 0.
__global__ __launch_bounds__(256) void combine_slots(const float* __restrict__ y,
                                                     const int* __restrict__ row_of,
                                                     const float* __restrict__ w, int T, int H,
                                                     int k, uint16_t* __restrict__ out, uint32_t okey,
                                                     int col0, int cols, int ldy) {
  const int t = permute_item(blockIdx.x, gridDim.x, okey);
  const int P = T * k;
  out += col0;
  const int c4 = cols / 4, c_lo = blockIdx.y * c4 / gridDim.y, c_hi = (blockIdx.y + 1) * c4 / gridDim.y;
  for (int c = c_lo + threadIdx.x; c < c_hi; c += blockDim.x) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
      const int row = row_of[t * k + j];
      if (static_cast<unsigned>(row) >= static_cast<unsigned>(P)) continue;
      const float wj = w[t * k + j];
      const f32x4 v = *reinterpret_cast<const f32x4*>(y + static_cast<size_t>(row) * ldy + 4 * c);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = fmaf(wj, v[i], acc[i]);
    }
    uint2 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
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
                                                     uint8_t* __restrict__ scales, uint32_t okey) {
  const int64_t tid = static_cast<int64_t>(permute_item(blockIdx.x, gridDim.x, okey)) * blockDim.x +
                      threadIdx.x;
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
  const uint32_t lo = f32x4_to_e4m3x4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
  const uint32_t hi = f32x4_to_e4m3x4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
  if (live) {
    *reinterpret_cast<uint2*>(codes + blk * 32 + part * 8) = make_uint2(lo, hi);
    if (part == 0) scales[blk] = static_cast<uint8_t>(sexp + 127);
  }
}

// Batched MXFP8 projections with a whole-line weight stream, the layout of
// gemm_bf16s for FP8 codes: workgroup = (M-tile of 64 routed rows, NW waves),
// each wave owning two groups of 16 weight rows (gate_up, KIND 0: 16 neurons'
// gate and up rows; down, KIND 1 / 2: 32 output dimensions).  A 128-position
// chunk of a row is 128 bytes: the wave reads its 32 rows as four loads of 8
// rows x 128 contiguous bytes (non-temporal), passes them through a
// wave-private 2 KB LDS tile (16-byte chunks XOR-swizzled by row) and reads
// back the 32-byte A operand of the block-scaled 16x16x128 MFMA.  The rows'
// E8M0 scale bytes come 8 per row per 256-position stage (two chunks) in one
// load per 16-row group.  The tile's activation codes and scale bytes are
// staged in LDS in 256-position stages, double-buffered and shared by the
// waves.  The gate_up epilogue quantizes h to MX: a 32-neuron block spans the
// wave pair (2m, 2m+1), whose per-row maxima meet in LDS.
constexpr int kMXC = 256;                // K stage of the staged MX codes (two chunks)
constexpr int kMRS = kMXC + 16;          // padded LDS row stride (bytes)
constexpr int kMSC = kMXC / 32;          // scale bytes per row per stage
constexpr int kMCH = kMXC / 16;          // 16-byte code chunks per row per stage

template <int KIND, int NW>   // (128 registers, as gemm_bf16s)
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(4, 8))) void gemm_mx_s(
    const uint8_t* __restrict__ act, const uint8_t* __restrict__ acts,
    const uint8_t* __restrict__ wt, const uint8_t* __restrict__ wts,
    const int* __restrict__ perm, const int2* __restrict__ tiles, const int* __restrict__ n_tiles,
    const int* __restrict__ counts, const int* __restrict__ offsets, const float* __restrict__ w,
    int H, int I, int k, uint8_t* __restrict__ hout, uint8_t* __restrict__ hsout,
    float* __restrict__ y, uint16_t* __restrict__ out, uint32_t okey, int cb0, int ncb, int ldy) {
  constexpr int NT = NW * 64;
  constexpr bool GU = KIND == kProjGateUp || KIND == kProjGateUpRaw;   // gate and up rows
  constexpr int RPW = GU ? 16 : 32;                       // outputs per wave
  constexpr int LPT = kBM * kMCH / NT;                    // 16-byte code loads per thread
  __shared__ __align__(16) uint8_t xl[2][kBM * kMRS];
  __shared__ __align__(16) uint8_t sl[2][kBM * kMSC];
  __shared__ __align__(16) i32x4 wtl[NW][16 * 8];         // per wave: [16 rows][8 chunks]
  __shared__ float s_amax[KIND == kProjGateUp ? NW : 1][kBM];
  // kProjGatherRows (the backward's dh = W_down^T dout): activation rows gathered by
  // token as gate_up's (K = H), one weight matrix [E][I][H] as down's (outputs I),
  // FP32 per grouped row as down's slot output (row stride ldy)
  // kProjGateUpRaw (the backward's pre-activations): gate_up's product, FP32 g and u of
  // each grouped row into y [P][2I] instead of h
  constexpr bool GATHER = GU || KIND == kProjGatherRows;
  const int K = GATHER ? H : I;                           // reduction length
  const int N = GATHER ? I : H;                           // outputs
  const int KB = K / 32;                                  // scale bytes per row
  const int nblk = ncb ? ncb : N / (NW * RPW);
  const int item0 = real_item(blockIdx.x, nblk, *n_tiles);
  if (item0 < 0) return;
  const int item = permute_item(item0, nblk * *n_tiles, okey);
  const int tile = item / nblk, nb_i = item - tile * nblk;
  const int2 te = tiles[tile];
  const int e = te.x, m0 = te.y;
  const int mcount = min(kBM, counts[e] - m0);
  const int rbase = offsets[e] + m0;
  const int tid = threadIdx.x, ln = tid & 63, col = ln & 15, grp = ln >> 4;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nb = (cb0 + nb_i) * NW * RPW + wv * RPW;      // the wave's first output
  const int row0 = nb, row1 = GU ? I + nb : nb + 16;
  const size_t wrows = GU ? 2 * static_cast<size_t>(I) : static_cast<size_t>(N);

  // whole-line loads: lane = (row lr of an 8-row group, 16-byte chunk lc)
  const int lr = ln >> 3, lc = ln & 7;
  const uint8_t* __restrict__ wb = wt + static_cast<size_t>(e) * wrows * K;
  const uint8_t* __restrict__ wsb = wts + static_cast<size_t>(e) * wrows * KB;
  uint32_t ow[4];                                         // group 0 rows 0-7, 8-15, group 1 rows 0-7, 8-15
#pragma unroll
  for (int i = 0; i < 4; ++i)
    ow[i] = static_cast<uint32_t>(((i < 2 ? row0 : row1) + 8 * (i & 1) + lr) * K + lc * 16);
  // weight scale bytes: lane (row col, group grp) of each 16-row group.  16 waves
  // (large batches) load them four stages at a time: the lane takes the 8 bytes of
  // stage 4w + grp of its row, so the four lanes of a row read one 32-byte piece
  // and a row's line is touched once per four stages, and the stage's bytes reach
  // the other lanes of the row by lane shuffles (every lane reading the stage's 8
  // bytes, stage by stage, made the scale lines ~5% of the DeepSeek-shaped
  // gate_up's time).  8 waves (small batches, where the shuffles' latency showed
  // and the line traffic did not) keep the stage-by-stage loads.
  constexpr bool kPieces = NW == 16;
  const uint32_t osw0 = static_cast<uint32_t>((row0 + col) * KB);
  const uint32_t osw1 = static_cast<uint32_t>((row1 + col) * KB);
  i32x4* tw = wtl[wv];
  i32x4* wdst = tw + lr * 8 + (lc ^ lr);                  // + 64 for rows 8-15
  const i32x4* asrc = tw + col * 8;
  const int sw = col & 7;

  // loaders: codes chunk c = tid + i*NT -> (row c/kMCH, 16-byte column c%kMCH);
  // scales: thread tid < 64 loads row tid's kMSC scale bytes of the stage
  uint32_t oxl[LPT];
  int lrow[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int c = tid + i * NT, r = c / kMCH, rr = r < mcount ? r : 0;
    lrow[i] = r * kMRS + (c % kMCH) * 16;
    const int arow = GATHER ? perm[rbase + rr] / k : rbase + rr;
    oxl[i] = static_cast<uint32_t>(arow * K + (c % kMCH) * 16);
  }
  const bool sload = tid < kBM;
  const int srow = tid < mcount ? tid : 0;
  const uint32_t osl =
      sload ? static_cast<uint32_t>((GATHER ? perm[rbase + srow] / k : rbase + srow) * KB)
            : 0u;
  i32x4 xr[LPT];
  uint2 sr = make_uint2(0u, 0u);
#pragma unroll
  for (int i = 0; i < LPT; ++i) xr[i] = ld16(act + oxl[i]);
  if (sload) sr = *reinterpret_cast<const uint2*>(acts + osl);
#pragma unroll
  for (int i = 0; i < LPT; ++i) *reinterpret_cast<i32x4*>(&xl[0][lrow[i]]) = xr[i];
  if (sload) *reinterpret_cast<uint2*>(&sl[0][tid * kMSC]) = sr;

  f32x4 acc0[4], acc1[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) acc0[g] = acc1[g] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nchunk = K / 128;
  i32x4 wA[4], wB[4];
  uint2 scA0, scA1;                                       // scale bytes of groups 0 / 1
#pragma unroll
  for (int i = 0; i < 4; ++i) wA[i] = ld16_stream(wb + ow[i]);
  const int nstage = K / kMXC;
  {
    const uint32_t s0 = kPieces ? static_cast<uint32_t>(min(grp, nstage - 1) * kMSC) : 0u;
    scA0 = *reinterpret_cast<const uint2*>(wsb + osw0 + s0);
    scA1 = *reinterpret_cast<const uint2*>(wsb + osw1 + s0);
  }
  __syncthreads();

  // one 128-position chunk cc (0 or 1) of stage buffer buf: weights W, block scales
  // sa0 / sa1 of this lane's rows.  One row group at a time (its A operand, then
  // the four B fragments); the empty asm statements keep each MFMA at its place,
  // where the compiler would otherwise sink them all to the end of the stage and
  // hold every operand live (beyond the 128 registers of 16 waves per CU).
  auto chunk = [&](const i32x4 (&W)[4], int buf, int cc, int sa0, int sa1) {
    const uint8_t* xcur = &xl[buf][col * kMRS + cc * 128 + 16 * grp];
    const uint8_t* scur = &sl[buf][col * kMSC + cc * 4 + grp];
#pragma unroll
    for (int m = 0; m < 2; ++m) {                         // row group 0, then 1
      wdst[0] = W[2 * m];
      wdst[64] = W[2 * m + 1];
      __builtin_amdgcn_wave_barrier();
      const i32x8 a = cat8(asrc[grp ^ sw], asrc[(4 + grp) ^ sw]);
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint8_t* p_ = xcur + (16 * g) * kMRS;
        const i32x8 bx = cat8(*reinterpret_cast<const i32x4*>(p_), *reinterpret_cast<const i32x4*>(p_ + 64));
        const int sx = scur[(16 * g) * kMSC];
        if (m == 0) {
          acc0[g] = mfma_mx16x16x128(a, bx, sa0, sx, acc0[g]);
          asm volatile("" : "+v"(acc0[g]));
        } else {
          acc1[g] = mfma_mx16x16x128(a, bx, sa1, sx, acc1[g]);
          asm volatile("" : "+v"(acc1[g]));
        }
      }
    }
  };
  for (int st = 0; st < nstage; ++st) {
    const int buf = st & 1;
    const bool more = st + 1 < nstage;
    if (more) {
#pragma unroll
      for (int i = 0; i < LPT; ++i) xr[i] = ld16(act + oxl[i] + (st + 1) * kMXC);
      if (sload) sr = *reinterpret_cast<const uint2*>(acts + osl + (st + 1) * kMSC);
    }
    // chunks 2st (weights in wA) and 2st+1 (wB); the chunk after each is loaded
    // first (clamped to the last chunk / stage, a harmless repeat: fixed load count)
    const uint32_t k1 = static_cast<uint32_t>((2 * st + 1) * 128);
    const uint32_t k2 = static_cast<uint32_t>(min(2 * st + 2, nchunk - 1) * 128);
#pragma unroll
    for (int i = 0; i < 4; ++i) wB[i] = ld16_stream(wb + ow[i] + k1);
    // this stage's 8 scale bytes of the lane's rows (kPieces: from lane (col, st & 3))
    uint32_t c0x = scA0.x, c0y = scA0.y, c1x = scA1.x, c1y = scA1.y;
    if (kPieces) {
      const int src = col + 16 * (st & 3);
      c0x = static_cast<uint32_t>(__shfl(static_cast<int>(c0x), src, kWave));
      c0y = static_cast<uint32_t>(__shfl(static_cast<int>(c0y), src, kWave));
      c1x = static_cast<uint32_t>(__shfl(static_cast<int>(c1x), src, kWave));
      c1y = static_cast<uint32_t>(__shfl(static_cast<int>(c1y), src, kWave));
    }
    const int b1_0 = static_cast<int>((c0y >> (8 * grp)) & 0xFFu);   // chunk 1's scale bytes
    const int b1_1 = static_cast<int>((c1y >> (8 * grp)) & 0xFFu);
    chunk(wA, buf, 0, static_cast<int>((c0x >> (8 * grp)) & 0xFFu),
          static_cast<int>((c1x >> (8 * grp)) & 0xFFu));
#pragma unroll
    for (int i = 0; i < 4; ++i) wA[i] = ld16_stream(wb + ow[i] + k2);
    if (!kPieces || (st & 3) == 3) {                      // the next stage's bytes / four stages' pieces
      const uint32_t s2 = static_cast<uint32_t>(min(st + 1 + (kPieces ? grp : 0), nstage - 1) * kMSC);
      scA0 = *reinterpret_cast<const uint2*>(wsb + osw0 + s2);
      scA1 = *reinterpret_cast<const uint2*>(wsb + osw1 + s2);
    }
    chunk(wB, buf, 1, b1_0, b1_1);
    if (more) {
#pragma unroll
      for (int i = 0; i < LPT; ++i) *reinterpret_cast<i32x4*>(&xl[buf ^ 1][lrow[i]]) = xr[i];
      if (sload) *reinterpret_cast<uint2*>(&sl[buf ^ 1][tid * kMSC]) = sr;
    }
    __syncthreads();
  }
  if (KIND == kProjGateUp) {
    // SwiGLU; per-row maximum over this wave's 16 neurons (lanes col + 16*grp),
    // combined with the partner wave's through LDS, gives the MX scale of the
    // 32-neuron block; then each wave encodes its own 16 neurons.
    float a[4][4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float amax = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[g][i] = swiglu(acc0[g][i], acc1[g][i]);
        amax = fmaxf(amax, fabsf(a[g][i]));
      }
      amax = fmaxf(amax, __shfl_xor(amax, 16, kWave));
      amax = fmaxf(amax, __shfl_xor(amax, 32, kWave));
      if (grp == 0) s_amax[KIND == kProjGateUp ? wv : 0][16 * g + col] = amax;
    }
    __syncthreads();
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int r = 16 * g + col;
      if (r >= mcount) continue;
      const float amax = fmaxf(s_amax[KIND == kProjGateUp ? wv : 0][r],
                               s_amax[KIND == kProjGateUp ? (wv ^ 1) : 0][r]);
      const int sexp = mx_scale_exp(amax);
      const float inv = exp2_neg(sexp);
      const uint32_t wq = f32x4_to_e4m3x4(a[g][0] * inv, a[g][1] * inv, a[g][2] * inv, a[g][3] * inv);
      *reinterpret_cast<uint32_t*>(hout + static_cast<size_t>(rbase + r) * I + nb + 4 * grp) = wq;
      if (grp == 0 && (wv & 1) == 0)
        hsout[static_cast<size_t>(rbase + r) * (I / 32) + nb / 32] = static_cast<uint8_t>(sexp + 127);
    }
  } else if (KIND == kProjGateUpRaw) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int r = 16 * g + col;
      if (r >= mcount) continue;
      float* gp = y + static_cast<size_t>(rbase + r) * (2 * I) + nb + 4 * grp;
      st16_stream(gp, acc0[g]);
      st16_stream(gp + I, acc1[g]);
    }
  } else {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int r = 16 * g + col;
      if (r >= mcount) continue;
      if (KIND == kProjDownFused) {
        const int t = perm[rbase + r];                    // k = 1: pair id == token
        const float wt_ = w[t];
        uint16_t* orow = out + static_cast<size_t>(t) * H + nb + 4 * grp;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const f32x4 a = m == 0 ? acc0[g] : acc1[g];
          uint2 v;
          v.x = pack_bf16x2(wt_ * a[0], wt_ * a[1]);
          v.y = pack_bf16x2(wt_ * a[2], wt_ * a[3]);
          *reinterpret_cast<uint2*>(orow + 16 * m) = v;
        }
      } else {
        float* yr = y + static_cast<size_t>(rbase + r) * ldy + (nb - cb0 * NW * RPW) + 4 * grp;
        st16_stream(yr, acc0[g]);
        st16_stream(yr + 16, acc1[g]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
namespace {
struct BatchedPtrs {
  int *n_tiles, *counts, *offsets, *perm, *row_of;
  int2* tiles;
  float *y, *partial;
  uint32_t* sct;
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
  p.partial = reinterpret_cast<float*>(b + L.partial);
  p.sct = reinterpret_cast<uint32_t*>(b + L.sct);
  return p;
}
int round_up(int v, int m) { return (v + m - 1) / m * m; }
// combine_slots grid: one workgroup per token and, for batches of fewer tokens than
// two per CU, column chunks of at least 256 columns (T 32, H 2048: 8 chunks, 9.9 ->
// ~4 us on the decode-sized MXFP8 shape)
dim3 combine_grid(int T, int cols, int num_cus) {
  int ch = T > 0 ? (2 * num_cus + T - 1) / T : 1;
  ch = ch < 1 ? 1 : ch > cols / 256 ? cols / 256 : ch;
  return dim3(static_cast<unsigned>(T), static_cast<unsigned>(ch < 1 ? 1 : ch));
}
}  // namespace

hipError_t launch_gate_up_batched(const void* x, const uint8_t* xs, const void* wgu,
                                  const uint8_t* wgus, const int32_t* idx, int T, int H, int I,
                                  int E, int k, int dtype, void* h, uint8_t* hs, void* ws,
                                  hipStream_t s, int num_cus, float* gu) {
  const BatchedWs L = batched_ws_layout(T, H, I, E, k, dtype);
  const BatchedPtrs p = batched_ptrs(ws, L);
  const int P = T * k;
  prof_begin(kGroup, s);
  hipLaunchKernelGGL(group_experts, dim3(E), dim3(1024), 0, s, idx, P, E, L.bm, p.counts,
                     p.offsets, p.tiles, p.n_tiles, p.perm, p.row_of, order_key());
  prof_end(kGroup, s);
  if (L.bm == kLargeBM) {
    prof_begin(kGemmGateUp, s);
    const hipError_t e =
        dtype == 0
            ? launch_gate_up_large_bf16(static_cast<const uint16_t*>(x),
                                        static_cast<const uint16_t*>(wgu), p.perm, p.tiles,
                                        p.n_tiles, p.counts, p.offsets, H, I, k,
                                        static_cast<uint16_t*>(h), p.partial, L.max_tiles, num_cus, s,
                                        gu)
            : launch_gate_up_large_mx(static_cast<const uint8_t*>(x), xs,
                                      static_cast<const uint8_t*>(wgu), wgus, p.perm, p.tiles,
                                      p.n_tiles, p.counts, p.offsets, H, I, k,
                                      static_cast<uint8_t*>(h), hs, p.partial, L.max_tiles,
                                      num_cus, s, T, E, p.sct);
    prof_end(kGemmGateUp, s);
    return e;
  }
  prof_begin(kGemmGateUp, s);
  if (L.bm == kTallBM) {
    // 8 waves x 16 neurons = 128 neurons per workgroup, 128-row tiles
    const int n_tall = round_up((I / 128) * L.max_tiles, kXcds);
    if (gu)
      hipLaunchKernelGGL((gemm_bf16s<kProjGateUpSave, 8, kTallBM>), dim3(n_tall), dim3(512), 0, s,
                         static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(wgu), p.perm,
                         p.tiles, p.n_tiles, p.counts, p.offsets, nullptr, H, I, k,
                         static_cast<uint16_t*>(h), nullptr, nullptr, gu, order_key(), 0, 0, 0);
    else
      hipLaunchKernelGGL((gemm_bf16s<kProjGateUp, 8, kTallBM>), dim3(n_tall), dim3(512), 0, s,
                         static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(wgu), p.perm,
                         p.tiles, p.n_tiles, p.counts, p.offsets, nullptr, H, I, k,
                         static_cast<uint16_t*>(h), nullptr, nullptr, nullptr, order_key(), 0, 0, 0);
    prof_end(kGemmGateUp, s);
    return hipGetLastError();
  }
  // 16 waves x 16 neurons = 256 neurons per workgroup (I is a multiple of 256);
  // when that gives fewer than four workgroups per CU (decode-sized batches: about
  // one M-tile per touched expert) 8 waves x 16 neurons instead, twice the items
  const bool narrow = (I / 256) * L.max_tiles < 4 * num_cus;
  const int n_items = round_up((I / 256) * L.max_tiles, kXcds);
  const int n_items8 = round_up((I / 128) * L.max_tiles, kXcds);
  if (narrow && dtype == 0 && gu)
    hipLaunchKernelGGL((gemm_bf16s<kProjGateUpSave, 8>), dim3(n_items8), dim3(512), 0, s,
                       static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(wgu), p.perm,
                       p.tiles, p.n_tiles, p.counts, p.offsets, nullptr, H, I, k,
                       static_cast<uint16_t*>(h), nullptr, nullptr, gu, order_key(), 0, 0, 0);
  else if (narrow && dtype == 0)
    hipLaunchKernelGGL((gemm_bf16s<kProjGateUp, 8>), dim3(n_items8), dim3(512), 0, s,
                       static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(wgu), p.perm,
                       p.tiles, p.n_tiles, p.counts, p.offsets, nullptr, H, I, k,
                       static_cast<uint16_t*>(h), nullptr, nullptr, nullptr, order_key(), 0, 0, 0);
  else if (narrow)
    hipLaunchKernelGGL((gemm_mx_s<kProjGateUp, 8>), dim3(n_items8), dim3(512), 0, s,
                       static_cast<const uint8_t*>(x), xs, static_cast<const uint8_t*>(wgu), wgus,
                       p.perm, p.tiles, p.n_tiles, p.counts, p.offsets, nullptr, H, I, k,
                       static_cast<uint8_t*>(h), hs, nullptr, nullptr, order_key(), 0, 0, 0);
  else if (dtype == 0 && gu)
    hipLaunchKernelGGL((gemm_bf16s<kProjGateUpSave, 16>), dim3(n_items), dim3(1024), 0, s,
                       static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(wgu), p.perm,
                       p.tiles, p.n_tiles, p.counts, p.offsets, nullptr, H, I, k,
                       static_cast<uint16_t*>(h), nullptr, nullptr, gu, order_key(), 0, 0, 0);
  else if (dtype == 0)
    hipLaunchKernelGGL((gemm_bf16s<kProjGateUp, 16>), dim3(n_items), dim3(1024), 0, s,
                       static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(wgu), p.perm,
                       p.tiles, p.n_tiles, p.counts, p.offsets, nullptr, H, I, k,
                       static_cast<uint16_t*>(h), nullptr, nullptr, nullptr, order_key(), 0, 0, 0);
  else
    hipLaunchKernelGGL((gemm_mx_s<kProjGateUp, 16>), dim3(n_items), dim3(1024), 0, s,
                       static_cast<const uint8_t*>(x), xs, static_cast<const uint8_t*>(wgu), wgus,
                       p.perm, p.tiles, p.n_tiles, p.counts, p.offsets, nullptr, H, I, k,
                       static_cast<uint8_t*>(h), hs, nullptr, nullptr, order_key(), 0, 0, 0);
  prof_end(kGemmGateUp, s);
  return hipGetLastError();
}

// The small-tile down projection and the combine run in column parts when k > 1
// (column_parts): part q's down launch writes the FP32 slot values of its
// H / parts output columns into the head of the slot buffer (row stride
// H / parts), and the combine of those columns reads them right after.
// Measured down + combine, T 2048, k 8: H 7168 E 384 BF16 2,245 -> 2,128 us (7
// parts; 4: 2,180; 14: 2,137; 28: 2,400, the per-launch tails taking over),
// whole forward step 5.74 -> 5.65 ms; H 6144 E 256 BF16 128-row tiles
// 1,390 -> 1,360 us (4 parts; 3: 1,345; 6: 1,460).  The MXFP8 down (16-wave
// workgroups, one per CU) stays whole: at H 7168 I 3072 its 7-part form, faster
// alone (1,713 -> 1,650 us), made the whole step slower (4.64 -> 4.68 ms; 2
// parts 4.72).

hipError_t launch_down_batched(const void* h, const uint8_t* hs, const void* wd,
                               const uint8_t* wds, const int32_t* idx, const float* w, int T,
                               int H, int I, int E, int k, int dtype, uint16_t* out, void* ws,
                               hipStream_t s, int num_cus) {
  (void)idx;
  const BatchedWs L = batched_ws_layout(T, H, I, E, k, dtype);
  const BatchedPtrs p = batched_ptrs(ws, L);
  prof_begin(kGemmDown, s);
  if (L.bm == kLargeBM) {
    hipError_t e =
        dtype == 0
            ? launch_down_large_bf16(static_cast<const uint16_t*>(h),
                                     static_cast<const uint16_t*>(wd), p.perm, p.tiles, p.n_tiles,
                                     p.counts, p.offsets, w, H, I, k, p.y, out, p.partial,
                                     L.max_tiles, num_cus, s)
            : launch_down_large_mx(static_cast<const uint8_t*>(h), hs,
                                   static_cast<const uint8_t*>(wd), wds, p.perm, p.tiles,
                                   p.n_tiles, p.counts, p.offsets, w, H, I, k, p.y, out,
                                   p.partial, L.max_tiles, num_cus, s, T, E, p.sct);
    if (e == hipSuccess && k > 1) {
      hipLaunchKernelGGL(combine_slots, combine_grid(T, H, num_cus), dim3(256), 0, s, p.y, p.row_of, w, T,
                         H, k, out, order_key(), 0, H, H);
      e = hipGetLastError();
    }
    prof_end(kGemmDown, s);
    return e;
  }
  // output dims per workgroup: BF16 8 waves x 32, two workgroups per CU (a CU stays
  // busy while one of them starts its next item: measured ~4% faster than one
  // 16-wave workgroup); MXFP8 16 waves x 32, where the 8-wave form measured slower
  // on large batches (8 x 32 when H is not a multiple of 512, or when 16-wave
  // items would leave fewer than four workgroups per CU); BF16 128-row tiles 8 x 32
  const bool wide = dtype == 1 && H % 512 == 0 && (H / 512) * L.max_tiles >= 4 * num_cus;
  const int dims = wide ? 512 : 256;
  // BF16 (two 8-wave workgroups per CU): four rounds are 8 * num_cus items
  const int parts = k > 1 && dtype == 0
                        ? column_parts(static_cast<size_t>(T) * k, H, dims, L.max_tiles, 8 * num_cus)
                        : 1;
  const int hq = H / parts, ncb = hq / dims;
  const dim3 grid(round_up(ncb * L.max_tiles, kXcds)), block(2 * dims);
  const uint16_t* hb = static_cast<const uint16_t*>(h);
  const uint16_t* wb = static_cast<const uint16_t*>(wd);
  const uint8_t* hm = static_cast<const uint8_t*>(h);
  const uint8_t* wm = static_cast<const uint8_t*>(wd);
  for (int q = 0; q < parts; ++q) {
    const int cb0 = q * ncb;
#define DOWN_ARGS_B p.perm, p.tiles, p.n_tiles, p.counts, p.offsets, w, H, I, k, nullptr, p.y, out, \
                    nullptr, order_key(), cb0, ncb, hq
#define DOWN_ARGS_M p.perm, p.tiles, p.n_tiles, p.counts, p.offsets, w, H, I, k, nullptr, nullptr, \
                    p.y, out, order_key(), cb0, ncb, hq
    if (L.bm == kTallBM) {
      if (k == 1) hipLaunchKernelGGL((gemm_bf16s<kProjDownFused, 8, kTallBM>), grid, block, 0, s, hb, wb, DOWN_ARGS_B);
      else hipLaunchKernelGGL((gemm_bf16s<kProjDown, 8, kTallBM>), grid, block, 0, s, hb, wb, DOWN_ARGS_B);
    } else if (dtype == 0) {
      if (k == 1) hipLaunchKernelGGL((gemm_bf16s<kProjDownFused, 8>), grid, block, 0, s, hb, wb, DOWN_ARGS_B);
      else hipLaunchKernelGGL((gemm_bf16s<kProjDown, 8>), grid, block, 0, s, hb, wb, DOWN_ARGS_B);
    } else if (wide) {
      if (k == 1) hipLaunchKernelGGL((gemm_mx_s<kProjDownFused, 16>), grid, block, 0, s, hm, hs, wm, wds, DOWN_ARGS_M);
      else hipLaunchKernelGGL((gemm_mx_s<kProjDown, 16>), grid, block, 0, s, hm, hs, wm, wds, DOWN_ARGS_M);
    } else {
      if (k == 1) hipLaunchKernelGGL((gemm_mx_s<kProjDownFused, 8>), grid, block, 0, s, hm, hs, wm, wds, DOWN_ARGS_M);
      else hipLaunchKernelGGL((gemm_mx_s<kProjDown, 8>), grid, block, 0, s, hm, hs, wm, wds, DOWN_ARGS_M);
    }
#undef DOWN_ARGS_B
#undef DOWN_ARGS_M
    if (k > 1)
      hipLaunchKernelGGL(combine_slots, combine_grid(T, hq, num_cus), dim3(256), 0, s, p.y, p.row_of, w,
                         T, H, k, out, order_key(), q * hq, hq, hq);
  }
  prof_end(kGemmDown, s);
  return hipGetLastError();
}

hipError_t launch_mx_rows_down(const uint8_t* act, const uint8_t* acts, const uint8_t* wt,
                               const uint8_t* wts, const int* perm, const int2* tiles,
                               const int* n_tiles, int max_tiles, const int* counts,
                               const int* offsets, int N, int K, int k, float* y, hipStream_t s,
                               int num_cus) {
  // as the MXFP8 down projection of launch_down_batched (N plays H, K plays I)
  const bool wide = N % 512 == 0 && (N / 512) * max_tiles >= 4 * num_cus;
  const int dims = wide ? 512 : 256;
  const dim3 grid(round_up((N / dims) * max_tiles, kXcds)), block(2 * dims);
  if (wide)
    hipLaunchKernelGGL((gemm_mx_s<kProjDown, 16>), grid, block, 0, s, act, acts, wt, wts, perm, tiles,
                       n_tiles, counts, offsets, nullptr, N, K, k, nullptr, nullptr, y, nullptr,
                       order_key(), 0, N / dims, N);
  else
    hipLaunchKernelGGL((gemm_mx_s<kProjDown, 8>), grid, block, 0, s, act, acts, wt, wts, perm, tiles,
                       n_tiles, counts, offsets, nullptr, N, K, k, nullptr, nullptr, y, nullptr,
                       order_key(), 0, N / dims, N);
  return hipGetLastError();
}

hipError_t launch_mx_rows_gather(const uint8_t* act, const uint8_t* acts, const uint8_t* wt,
                                 const uint8_t* wts, const int* perm, const int2* tiles,
                                 const int* n_tiles, int max_tiles, const int* counts,
                                 const int* offsets, int K, int N, int k, float* y, hipStream_t s,
                                 int num_cus) {
  // act rows gathered by token (perm / k), y [P][N]; the kernel's (H, I) are (K, N)
  const bool wide = N % 512 == 0 && (N / 512) * max_tiles >= 4 * num_cus;
  const int dims = wide ? 512 : 256;
  const dim3 grid(round_up((N / dims) * max_tiles, kXcds)), block(2 * dims);
  if (wide)
    hipLaunchKernelGGL((gemm_mx_s<kProjGatherRows, 16>), grid, block, 0, s, act, acts, wt, wts, perm,
                       tiles, n_tiles, counts, offsets, nullptr, K, N, k, nullptr, nullptr, y, nullptr,
                       order_key(), 0, N / dims, N);
  else
    hipLaunchKernelGGL((gemm_mx_s<kProjGatherRows, 8>), grid, block, 0, s, act, acts, wt, wts, perm,
                       tiles, n_tiles, counts, offsets, nullptr, K, N, k, nullptr, nullptr, y, nullptr,
                       order_key(), 0, N / dims, N);
  return hipGetLastError();
}

hipError_t launch_mx_gate_up_raw_rows(const uint8_t* x, const uint8_t* xs, const uint8_t* wgu,
                                     const uint8_t* wgus, const int* perm, const int2* tiles,
                                     const int* n_tiles, int max_tiles, const int* counts,
                                     const int* offsets, int H, int I, int k, float* gu,
                                     hipStream_t s, int num_cus) {
  // as the MXFP8 gate_up of launch_gate_up_batched: 16 or 8 waves of 16 neurons
  const int n16 = round_up((I / 256) * max_tiles, kXcds);
  if ((I / 256) * max_tiles >= 4 * num_cus) {
    hipLaunchKernelGGL((gemm_mx_s<kProjGateUpRaw, 16>), dim3(n16), dim3(1024), 0, s, x, xs, wgu, wgus,
                       perm, tiles, n_tiles, counts, offsets, nullptr, H, I, k, nullptr, nullptr, gu,
                       nullptr, order_key(), 0, 0, 0);
  } else {
    const int n8 = round_up((I / 128) * max_tiles, kXcds);
    hipLaunchKernelGGL((gemm_mx_s<kProjGateUpRaw, 8>), dim3(n8), dim3(512), 0, s, x, xs, wgu, wgus,
                       perm, tiles, n_tiles, counts, offsets, nullptr, H, I, k, nullptr, nullptr, gu,
                       nullptr, order_key(), 0, 0, 0);
  }
  return hipGetLastError();
}

hipError_t launch_group_experts(const int32_t* idx, int P, int E, int BM, int* counts, int* offsets,
                                int2* tiles, int* n_tiles, int* perm, int* row_of, hipStream_t s) {
  prof_begin(kGroup, s);
  hipLaunchKernelGGL(group_experts, dim3(E), dim3(1024), 0, s, idx, P, E, BM, counts, offsets,
                     tiles, n_tiles, perm, row_of, order_key());
  prof_end(kGroup, s);
  return hipGetLastError();
}

hipError_t launch_quant_mx(const uint16_t* src, int64_t rows, int K, uint8_t* codes,
                           uint8_t* scales, hipStream_t s) {
  const int64_t n_blocks = rows * (K / 32);
  const int64_t threads = n_blocks * 4;
  const int64_t grid = (threads + 255) / 256;
  prof_begin(kQuant, s);
  hipLaunchKernelGGL(quant_mx_rows, dim3(static_cast<unsigned>(grid)), dim3(256), 0, s, src,
                     n_blocks, codes, scales, order_key());
  prof_end(kQuant, s);
  return hipGetLastError();
}

hipError_t batched_set_attributes() { return large_set_attributes(); }

}  // namespace moe
