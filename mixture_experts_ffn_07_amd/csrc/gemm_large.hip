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
//
// The same BF16 kernel serves the backward pass of such batches: dx = [dg; du]
// W_gate_up with W_gate_up transposed (kDownPlain, kDownSlots), dh = W_down^T
// dout with W_down transposed and the dout rows gathered (kBwdDh), and both
// weight gradients over transposed, zero-padded operands (kWgradDown,
// kWgradGateUp); the transposes and the column-offset scan are at the end.
#include "common.h"
#include "internal.h"
#include "tiles.h"

namespace moe {

namespace {
constexpr int kLBK = 64;                     // K per stage
constexpr int kLTile = kLargeBM * kLBK;      // elements per operand stage (256 rows x 64)
constexpr size_t kLLds = 2 * 2 * kLTile * sizeof(uint16_t);   // 128 KB
enum { kGateUp = 0, kDownFused = 1, kDownSlots = 2, kGateUpSave = 3, kWgradGateUp = 4, kWgradDown = 5, kDownPlain = 6, kBwdDh = 7,
       kGateUpRaw = 8 };   // kGateUpRaw: FP32 g and u per grouped row (no activation)

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

// Item order.  Items are (M-tile, N-block) pairs; an XCD runs a contiguous run
// of item numbers, 32 at a time.  Numbering N-blocks fastest would make those
// 32 one or two M-tiles against ~32 different weight blocks (about 34 distinct
// operand blocks per K stage in the XCD's L2); numbering groups of
// kLargeGroupM M-tiles with the M-tile fastest makes them 8 M-tiles x 4
// N-blocks (12 distinct blocks), so each staged block is shared by more CUs.
// (Measured over group sizes 2, 4, 6, 8 and 16: 8 is best for MXFP8 and level
// with 4 for BF16.)
constexpr int kLargeGroupM = 8;
__device__ __forceinline__ void large_coords(int item, int nblk, int n_tiles, int& tile, int& nb) {
  const int grp = item / (kLargeGroupM * nblk);
  const int r = item - grp * kLargeGroupM * nblk;
  const int t0 = grp * kLargeGroupM;
  const int gm = min(kLargeGroupM, n_tiles - t0);
  nb = r / gm;
  tile = t0 + (r - nb * gm);
}

// Workgroup -> item across XCDs.  One workgroup fills a CU, so the ncu
// workgroups resident at a time are consecutive; mapping each such round to one
// contiguous run of items (XCD x, = L mod 8, taking the x-th chunk of it) keeps
// every CU on the same one or two experts at a time, whose operands then stay in
// the last-level cache (spreading the XCDs over the whole item range put six
// experts' weights, 352 MB on the BF16 EP share, in flight at once).  n is a
// multiple of 8; a last partial round keeps the contiguous-per-XCD split.
__device__ __forceinline__ int round_item(int L, int n, int ncu) {
  if (ncu < kXcds || ncu % kXcds) return xcd_item(L, n);
  const int full = n / ncu * ncu;
  if (L < full) {
    const int r = L / ncu, w = L - r * ncu;
    return r * ncu + (w % kXcds) * (ncu / kXcds) + w / kXcds;
  }
  return full + xcd_item(L - full, n - full);
}
__device__ __forceinline__ int round_real_item(int L, int nblk, int n_tiles, int ncu) {
  const int n_real = (nblk * n_tiles + kXcds - 1) / kXcds * kXcds;
  if (L >= n_real) return -1;
  const int item = round_item(L, n_real, ncu);
  return item / nblk < n_tiles ? item : -1;
}

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// s_waitcnt with only the LDS/scalar counter constrained to 0
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
}  // namespace

// Weight-gradient epilogue: the wave's 128 (B rows) x 128 (A columns) block of
// dW, BF16, through LDS so that global stores are 16 bytes per lane along dW
// rows (a wave stores 4 rows x 256 bytes at a time).  Lane (l32, hi) holds A
// column 32i + 8q + 4hi + t and B row 32j + l32 of the block (register 4q + t of
// acc[i][j]).  Two passes of 64 rows through the wave's own 17 KB of LDS; the
// caller has made the LDS free (no wave still reads its K stages).
constexpr int kWgStage = 272;                  // bytes per staged row: 256 + 16
constexpr int kWgLds = 4 * 64 * kWgStage;      // 68 KB for the workgroup
__device__ __forceinline__ void wgrad_store(const f32x16 (&acc)[4][4], uint8_t* lds,
                                            uint16_t* __restrict__ dw, int cols, int row0,
                                            int col0, int wv, int ln) {
  uint8_t* st = lds + wv * 64 * kWgStage;
  const int l32 = ln & 31, hi = ln >> 5;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x16& a = acc[i][2 * half + jj];
          const uint32_t p0 = pack_bf16x2(a[4 * q], a[4 * q + 1]);
          const uint32_t p1 = pack_bf16x2(a[4 * q + 2], a[4 * q + 3]);
          *reinterpret_cast<uint2*>(st + (32 * jj + l32) * kWgStage + (32 * i + 8 * q + 4 * hi) * 2) =
              make_uint2(p0, p1);
        }
    // one wave's LDS operations complete in order: the reads see the writes above
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int r = 4 * u + (ln >> 4), c = ln & 15;
      const i32x4 v = *reinterpret_cast<const i32x4*>(st + r * kWgStage + c * 16);
      *reinterpret_cast<i32x4*>(dw + static_cast<size_t>(row0 + 64 * half + r) * cols + col0 + c * 8) = v;
    }
  }
}

// Epilogue of a 256 x 256 tile (see gemm_large_bf16 for the register layout).
template <int KIND>
__device__ __forceinline__ void large_epilogue(const f32x16 (&acc)[4][4], const int* __restrict__ perm,
                                               const float* __restrict__ w, int H, int I, int rbase,
                                               int mcount, int nb, int wm, int wn, int l32, int hi,
                                               uint16_t* __restrict__ hout, float* __restrict__ y,
                                               uint16_t* __restrict__ out, float* __restrict__ gu) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = wm * 128 + 32 * j + l32;
    if (r >= mcount) continue;
    if (KIND == kGateUp || KIND == kGateUpSave || KIND == kGateUpRaw) {
      if (KIND == kGateUpSave || KIND == kGateUpRaw) {   // FP32 g and u: slot order / grouped rows
        const size_t grow = KIND == kGateUpSave ? static_cast<size_t>(perm[rbase + r])
                                                : static_cast<size_t>(rbase + r);
        float* gp = gu + grow * (2 * I) + nb * 128 + wn * 64 + 4 * hi;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            *reinterpret_cast<f32x4*>(gp + 32 * i + 8 * q) =
                f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
            *reinterpret_cast<f32x4*>(gp + I + 32 * i + 8 * q) =
                f32x4{acc[i + 2][j][4 * q], acc[i + 2][j][4 * q + 1], acc[i + 2][j][4 * q + 2],
                      acc[i + 2][j][4 * q + 3]};
          }
      }
      if (KIND == kGateUpRaw) continue;
      uint16_t* hr = hout + static_cast<size_t>(rbase + r) * I + nb * 128 + wn * 64 + 4 * hi;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float p[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) p[t] = swiglu(acc[i][j][4 * q + t], acc[i + 2][j][4 * q + t]);
          *reinterpret_cast<uint2*>(hr + 32 * i + 8 * q) = make_uint2(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]));
        }
    } else if (KIND == kDownFused || KIND == kDownPlain) {
      const int t = perm[rbase + r];        // k = 1: pair id == token
      const float wt_t = KIND == kDownFused ? w[t] : 1.0f;
      uint16_t* orow = out + static_cast<size_t>(t) * H + nb * 256 + wn * 128 + 4 * hi;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float p[4];
#pragma unroll
          for (int t4 = 0; t4 < 4; ++t4) p[t4] = wt_t * acc[i][j][4 * q + t4];
          *reinterpret_cast<uint2*>(orow + 32 * i + 8 * q) = make_uint2(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]));
        }
    } else {
      // kDownSlots: y [P, H]; kBwdDh: dh [P, I]
      float* yr = y + static_cast<size_t>(rbase + r) * (KIND == kBwdDh ? I : H) + nb * 256 + wn * 128 + 4 * hi;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<f32x4*>(yr + 32 * i + 8 * q) =
              f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
    }
  }
}

// 8 x 8 transpose of BF16 values held in registers: t[i] (i < 8) holds 8 values
// of row i of a block (two per dword, the lower index in the low half); after
// the call t[j] holds column j (row 2p in the low and 2p+1 in the high half of
// dword p).  One byte permute per dword swaps the 16-bit halves between row
// pairs; the rest is dword renaming.
__device__ __forceinline__ void transpose8x8_bf16(i32x4 (&t)[16]) {
  uint32_t s[8][4];
#pragma unroll
  for (int p = 0; p < 4; ++p)
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t a = static_cast<uint32_t>(t[2 * p][m]), b = static_cast<uint32_t>(t[2 * p + 1][m]);
      s[2 * p][m] = __builtin_amdgcn_perm(b, a, 0x05040100u);       // low halves of a, b
      s[2 * p + 1][m] = __builtin_amdgcn_perm(b, a, 0x07060302u);   // high halves of a, b
    }
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) t[j][q] = static_cast<int>(s[2 * q + (j & 1)][j >> 1]);
}

// KIND kGateUp:    act = x [T,H], wt = W_gate_up [E,2I,H]; writes h [P,I] (sorted rows, BF16).
// KIND kDown*:     act = h [P,I] (sorted rows), wt = W_down [E,H,I]; kDownFused (k = 1)
//                  writes out[t] = bf16(w[t] * y), kDownSlots writes y [P,H] FP32 (sorted rows).
// MFMA operands: A = weight rows (D rows), B = activation rows (D columns).  The
// 32x32x16 result puts, in lane (l32, hi) register 4q+t, weight row 8q + 4hi + t
// and activation row l32 of the 32 x 32 block.  Within each stage of 64, lane
// half hi takes K chunks 2*ks + hi at MFMA K step ks (the same for A and B).
// KIND kWgradGateUp / kWgradDown (weight gradients of the backward pass): A and
// B are transposed copies [rows][KPT] whose columns hold the routed rows of
// expert e in offsets[e] .. offsets[e+1] (zero-padded to multiples of 64; KPT =
// offsets[E]): kWgradGateUp A = x^T (rows h), B = [dg; du]^T (rows c), writes
// dW_gate_up[e][c][h]; kWgradDown A = (w a)^T (rows i), B = dout^T (rows h),
// writes dW_down[e][h][i].  A workgroup takes expert e, 256 A rows and 256 B rows
// and reduces over the expert's columns only (no K split).
// AT: the A operand is stored transposed, [E][K][N] with the output dimension N
// contiguous (the backward's dh reads W_down [E][H][I] and its dx W_gate_up
// [E][2I][H] in place).  A thread then loads an 8 (K) x 8 (output) block of each
// stage as eight 16-byte row pieces (a half-wave covers 512 contiguous bytes of a
// K row), transposes it in registers and writes 8 output rows' 16-byte K chunks;
// those rows share their low 3 bits, so the A tile's chunk swizzle also XORs in
// row bits 3..5 (slot = chunk ^ (row & 7) ^ ((row >> 3) & 7)).
template <int KIND, bool AT = false>
__global__ __launch_bounds__(256) void gemm_large_bf16(
    const uint16_t* __restrict__ act, const uint16_t* __restrict__ wt,
    const int* __restrict__ perm, const int2* __restrict__ tiles, const int* __restrict__ n_tiles,
    const int* __restrict__ counts, const int* __restrict__ offsets, const float* __restrict__ w,
    int H, int I, int k, uint16_t* __restrict__ hout, float* __restrict__ y,
    uint16_t* __restrict__ out, float* __restrict__ partial, int ncu, float* __restrict__ gu,
    int E, uint32_t okey) {
  extern __shared__ __align__(16) uint16_t lds[];   // [stage][A, B][256 x 64]
  constexpr bool kGU = KIND == kGateUp || KIND == kGateUpSave;
  constexpr bool kWG = KIND == kWgradGateUp || KIND == kWgradDown;
  constexpr bool kDH = KIND == kBwdDh;   // backward dh = W_down^T dout: gathered dout rows, K = H
  const int K = kWG ? offsets[E] : (kGU || kDH ? H : I);    // row stride of both operands
  const int nA = KIND == kWgradGateUp ? H / 256 : I / 256;       // (weight gradients)
  const int nB = KIND == kWgradGateUp ? 2 * I / 256 : H / 256;
  const int nblk = kGU ? I / 128 : kDH ? I / 256 : H / 256;
  const int nk = K / kLBK;
  const int L = blockIdx.x;
  int item, kb = 0, ke = nk, slot = -1;
  int e, nb, bb = 0, mcount = kLargeBM, rbase = 0;
  if (kWG) {
    const int per = nA * nB, n_w = E * per;
    const int n_pad = (n_w + kXcds - 1) / kXcds * kXcds;
    if (L >= n_pad) return;
    item = permute_item(round_item(L, n_pad, ncu), n_pad, okey);
    if (item >= n_w) return;
    e = item / per;
    large_coords(item - e * per, nA, nB, bb, nb);
    kb = offsets[e] / kLBK;
    ke = offsets[e + 1] / kLBK;
  } else {
    const int n_real = nblk * *n_tiles;
    const TailPlan plan = tail_plan(n_real, ncu, nk);
    if (plan.S > 1 && L < plan.full) {
      item = permute_item(round_item(L, plan.full, ncu), plan.full, okey);
    } else if (plan.S > 1) {
      const int t0 = L - plan.full;
      if (t0 >= plan.rem * plan.S) return;
      const int t = permute_item(t0, plan.rem * plan.S, okey);
      item = plan.full + t % plan.rem;
      const int sl = t / plan.rem;
      kb = sl * nk / plan.S;
      ke = (sl + 1) * nk / plan.S;
      slot = t;
    } else {
      item = round_real_item(L, nblk, *n_tiles, ncu);
      if (item < 0) return;
      item = permute_item(item, nblk * *n_tiles, okey);
    }
    int tile;
    large_coords(item, nblk, *n_tiles, tile, nb);
    const int2 te = tiles[tile];
    e = te.x;
    const int m0 = te.y;
    mcount = min(kLargeBM, counts[e] - m0);
    rbase = offsets[e] + m0;
  }
  const int tid = threadIdx.x, wv = tid >> 6, ln = tid & 63, l32 = ln & 31, hi = ln >> 5;
  const int wm = wv & 1, wn = wv >> 1;

  // Loader: thread covers tile rows wv*64 + 8j + (ln >> 3), j = 0..7, of both
  // operands, 16-byte chunk ln & 7 of each 128-byte row segment.  Rows past the
  // tile's end load the tile's first row (their columns are discarded).
  const int lrow = ln >> 3, lc = ln & 7;
  const uint16_t* __restrict__ abase;
  uint32_t ao;
  if (kWG) {
    abase = wt;
    ao = static_cast<uint32_t>((nb * 256 + wv * 64 + lrow) * K + lc * 8);
  } else if (kGU) {
    const int n0 = nb * 128;
    abase = wt + static_cast<size_t>(e) * 2 * I * H;
    // tile rows 0..127: gate neurons n0.., rows 128..255: up neurons n0..
    ao = static_cast<uint32_t>(((wv < 2 ? n0 + wv * 64 : I + n0 + (wv - 2) * 64) + lrow) * H + lc * 8);
  } else if (AT) {
    // stored [K][ldw]: thread = K rows 8*kb8 .. +7 of the stage, outputs 8*ob8 .. +7
    abase = wt + static_cast<size_t>(e) * H * I;
    ao = static_cast<uint32_t>(8 * (2 * wv + (ln >> 5)) * (kDH ? I : H) + nb * 256 + 8 * (ln & 31));
  } else {
    // down: wt = W_down [E][H][I] (rows h, K = I); kDH: W_down transposed [E][I][H]
    abase = wt + static_cast<size_t>(e) * H * I;
    ao = static_cast<uint32_t>((nb * 256 + wv * 64 + lrow) * K + lc * 8);
  }
  const int ldw = kDH ? I : H;                    // (AT) row stride of the stored A
  // (AT) LDS element offsets of this thread's 8 output rows' K chunk: row 8*ob8 + j,
  // chunk kb8 at slot kb8 ^ j ^ (ob8 & 7)
  const int at_row0 = 8 * (ln & 31) * kLBK, at_kb = 2 * wv + (ln >> 5), at_hs = (ln & 31) & 7;
  uint32_t bo[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = wv * 64 + 8 * j + lrow;
    const int rr = r < mcount ? r : 0;
    bo[j] = kWG ? static_cast<uint32_t>((bb * 256 + r) * K + lc * 8)
          : kGU || kDH ? static_cast<uint32_t>((perm[rbase + rr] / k) * H + lc * 8)
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
  int swa[4];                                     // A fragment swizzles (AT: + row bits 3..5)
#pragma unroll
  for (int i = 0; i < 4; ++i) swa[i] = AT ? swz ^ ((4 * i + (l32 >> 3)) & 7) : swz;

  i32x4 stg[16];   // [0..7] weight rows, [8..15] activation rows
#define GLOAD(Q, KT) do {                                                               \
    const uint32_t kk_ = static_cast<uint32_t>(min((KT), ke - 1) * kLBK);               \
    if ((Q) < 8 && AT) stg[Q] = ld16(abase + ao + (kk_ + (Q)) * static_cast<uint32_t>(ldw)); \
    else if ((Q) < 8) stg[Q] = ld16(abase + ao + static_cast<uint32_t>((Q) * 8) * K + kk_); \
    else stg[Q] = ld16(act + bo[(Q) - 8] + kk_);                                        \
  } while (0)
  // (AT: the first A chunk of a stage transposes all eight in place)
#define LWRITE(Q, KT) do {                                                              \
    uint16_t* st_ = lds + ((KT) & 1) * 2 * kLTile;                                      \
    if ((Q) < 8 && AT) {                                                                \
      if ((Q) == 0) transpose8x8_bf16(stg);                                             \
      *reinterpret_cast<i32x4*>(&st_[at_row0 + (Q) * kLBK + ((at_kb ^ (Q) ^ at_hs) * 8)]) = stg[Q]; \
    } else if ((Q) < 8) *reinterpret_cast<i32x4*>(&st_[lw + (Q) * 8 * kLBK]) = stg[Q]; \
    else *reinterpret_cast<i32x4*>(&st_[kLTile + lw + ((Q) - 8) * 8 * kLBK]) = stg[Q];  \
  } while (0)
#define RDF(PTR) as_bf16x8(*reinterpret_cast<const i32x4*>(PTR))
  // One MFMA K step on fragments (A, B): 8 groups of 2 MFMAs; groups 0..3 then
  // read fragments A g and B g of the next K step (stage RKT, step RKS: all of
  // them in the first half, so they have landed when the next step starts)
  // and, for g < NQ, write staged chunk Q0+g of stage WKT to LDS and reload that
  // chunk from stage WKT+1.  sched_barrier keeps this order.
#define PHASE(A, B, NA, NB, RKT, RKS, WKT, Q0, NQ) do {                                 \
    const uint16_t* at_ = lds + ((RKT) & 1) * 2 * kLTile;                               \
    const uint16_t* bt_ = at_ + kLTile;                                                 \
    const int so_ = (((2 * (RKS) + hi) ^ swz) * 8);                                     \
    const int ka_ = 2 * (RKS) + hi;                                                     \
    _Pragma("unroll") for (int g = 0; g < 8; ++g) {                                     \
      const int i_ = g >> 1, j0_ = (g & 1) * 2;                                         \
      acc[i_][j0_] = mfma32x32x16(A[i_], B[j0_], acc[i_][j0_]);                         \
      acc[i_][j0_ + 1] = mfma32x32x16(A[i_], B[j0_ + 1], acc[i_][j0_ + 1]);             \
      __builtin_amdgcn_sched_barrier(0);                                                \
      if (g < 4) {                                                                      \
        NA[g] = RDF(&at_[fa[g] + ((ka_ ^ swa[g]) * 8)]);                                \
        NB[g] = RDF(&bt_[fb + 32 * g * kLBK + so_]);                                    \
      }                                                                                 \
      if (g < (NQ)) { LWRITE((Q0) + g, WKT); GLOAD((Q0) + g, (WKT) + 1); }              \
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
  // The LDS writes of stage s+1 are spread over the four K steps that may
  // write its buffer: the last step of stage s-1 (chunks 12..15, after the
  // barrier that ends the reads of stage s-1) and the first three of stage s
  // (chunks 0..11, before the barrier that publishes stage s+1).  Prologue:
  // stage kb in LDS, chunks 12..15 of stage kb+1 in LDS, the staging registers
  // holding chunks 0..11 of stage kb+1 and 12..15 of stage kb+2.  (An expert
  // with no routed rows has an empty range: its weight gradient is zero.)
  if (ke > kb) {
#pragma unroll
  for (int q = 0; q < 16; ++q) GLOAD(q, kb);
#pragma unroll
  for (int q = 0; q < 16; ++q) LWRITE(q, kb);
#pragma unroll
  for (int q = 0; q < 16; ++q) GLOAD(q, kb + 1);
#pragma unroll
  for (int q = 12; q < 16; ++q) { LWRITE(q, kb + 1); GLOAD(q, kb + 2); }
  __syncthreads();
  bf16x8 a0[4], b0[4], a1[4], b1[4];
  {
    const uint16_t* at = lds + (kb & 1) * 2 * kLTile;
    const int so = (hi ^ swz) * 8;
#pragma unroll
    for (int g = 0; g < 4; ++g) a0[g] = RDF(&at[fa[g] + ((hi ^ swa[g]) * 8)]);
#pragma unroll
    for (int g = 0; g < 4; ++g) b0[g] = RDF(&at[kLTile + fb + 32 * g * kLBK + so]);
  }
  for (int kt = kb; kt < ke; ++kt) {
    PHASE(a0, b0, a1, b1, kt, 1, kt + 1, 0, 4);
    PHASE(a1, b1, a0, b0, kt, 2, kt + 1, 4, 4);
    PHASE(a0, b0, a1, b1, kt, 3, kt + 1, 8, 4);
    // stage kt+1 is in LDS for every wave, and every wave is done reading stage kt
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    PHASE(a1, b1, a0, b0, kt + 1, 0, kt + 2, 12, 4);
  }
  }
#undef GLOAD
#undef LWRITE
#undef RDF
#undef PHASE

  if (kWG) {
    // dW[e][B row][A row], BF16
    const int colsA = nA * 256;
    __syncthreads();                               // every wave is done with the K stages
    wgrad_store(acc, reinterpret_cast<uint8_t*>(lds), out + static_cast<size_t>(e) * (nB * 256) * colsA,
                colsA, bb * 256 + wm * 128, nb * 256 + wn * 128, wv, ln);
    return;
  }
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
  large_epilogue<KIND>(acc, perm, w, H, I, rbase, mcount, nb, wm, wn, l32, hi, hout, y, out, gu);
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
    const float* __restrict__ partial, int ncu, int nk, float* __restrict__ gu, uint32_t okey) {
  constexpr bool kGU = KIND == kGateUp || KIND == kGateUpSave || KIND == kGateUpRaw;
  constexpr int kPerItem = kGU ? 32 * 256 : 64 * 256;   // threads per tail item
  const int nblk = kGU ? I / 128 : KIND == kBwdDh ? I / 256 : H / 256;
  const TailPlan plan = tail_plan(nblk * *n_tiles, ncu, nk);
  const int g = permute_item(blockIdx.x, gridDim.x, okey) * 256 + threadIdx.x;
  const int b = g / kPerItem;
  if (plan.S == 1 || b >= plan.rem) return;
  const int f = g - b * kPerItem;            // f32x4 index within the tile (gate half for gate_up)
  const int tid = f & 255, ijq = f >> 8;     // GEMM thread and register block
  const int i = ijq >> 4, j = (ijq >> 2) & 3, q = ijq & 3;
  const int item = plan.full + b;
  int tile, nb;
  large_coords(item, nblk, *n_tiles, tile, nb);
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
    if (KIND == kGateUpSave || KIND == kGateUpRaw) {   // FP32 g and u: slot order / grouped rows
      const size_t grow = KIND == kGateUpSave ? static_cast<size_t>(perm[rbase + r])
                                              : static_cast<size_t>(rbase + r);
      float* gp = gu + grow * (2 * I) + nb * 128 + wn * 64 + 32 * i + 8 * q + 4 * hi;
      *reinterpret_cast<f32x4*>(gp) = a;
      *reinterpret_cast<f32x4*>(gp + I) = u;
    }
    if (KIND == kGateUpRaw) return;
    uint16_t* hr = hout + static_cast<size_t>(rbase + r) * I + nb * 128 + wn * 64 + 32 * i + 8 * q + 4 * hi;
    float p[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) p[t] = swiglu(a[t], u[t]);
    *reinterpret_cast<uint2*>(hr) = make_uint2(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]));
  } else if (KIND == kDownFused || KIND == kDownPlain) {
    const int t = perm[rbase + r];
    const float wt_t = KIND == kDownFused ? w[t] : 1.0f;
    uint16_t* o = out + static_cast<size_t>(t) * H + nb * 256 + wn * 128 + 32 * i + 8 * q + 4 * hi;
    float p[4];
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) p[t4] = wt_t * a[t4];
    *reinterpret_cast<uint2*>(o) = make_uint2(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]));
  } else {
    *reinterpret_cast<f32x4*>(y + static_cast<size_t>(rbase + r) * (KIND == kBwdDh ? I : H) + nb * 256 + wn * 128 + 32 * i +
                              8 * q + 4 * hi) = a;
  }
}


// SwiGLU + MX quantization of one 32-neuron block of one token row: the lane
// pair (l32, hi = 0/1) holds neurons 8q + 4hi + t (register 4q + t) of gate
// block g and up block u.  Scale from the block's amax (OCP Microscaling v1.0
// rule), codes E4M3 of v * 2^-s; the hi = 0 lane writes the scale byte.  Both
// lanes of a pair always take the same branch (same row).
__device__ __forceinline__ void mx_store_block(const f32x16& g, const f32x16& u, int r, int mcount,
                                               int rbase, int n, int hi, int I,
                                               uint8_t* __restrict__ hq, uint8_t* __restrict__ hs) {
  if (r >= mcount) return;
  float v[16];
  float amax = 0.f;
#pragma unroll
  for (int x = 0; x < 16; ++x) {
    v[x] = swiglu(g[x], u[x]);
    amax = fmaxf(amax, fabsf(v[x]));
  }
  amax = fmaxf(amax, __shfl_xor(amax, 32, kWave));
  const int sx = mx_scale_exp(amax);
  const float inv = exp2_neg(sx);
  uint8_t* hr = hq + static_cast<size_t>(rbase + r) * I + n + 4 * hi;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    *reinterpret_cast<uint32_t*>(hr + 8 * q) =
        f32x4_to_e4m3x4(v[4 * q] * inv, v[4 * q + 1] * inv, v[4 * q + 2] * inv, v[4 * q + 3] * inv);
  }
  if (hi == 0) hs[static_cast<size_t>(rbase + r) * (I / 32) + n / 32] = static_cast<uint8_t>(sx + 127);
}

// ---------------------------------------------------------------------------
// MXFP8 (E4M3 codes, one E8M0 scale per 32 along K).  Same tile, waves and
// pipeline as the BF16 kernel, in bytes: a stage is 128 K (128-byte row
// segments, the same LDS layout), plus the stage's 4 scale bytes of each of the
// 256 rows of both operands (one dword per row).  MFMA
// v_mfma_scale_f32_32x32x64_f8f6f4: lane (l32, hi) holds bytes [16hi, +16) of
// K block 0 and of K block 1 of the 64-wide K step, and supplies the scale of
// block hi of its row; so at K step ks of a stage, lane hi takes 16-byte
// chunks 4ks + hi and 4ks + 2 + hi, and scale byte 2ks + hi of its row's dword
// (shifted down by 8 hi, then selected with opsel 2ks).
namespace {
constexpr int kMBK = 128;                                  // K per stage
constexpr int kMTile = kLargeBM * kMBK;                    // bytes per operand stage
constexpr size_t kMLds = 2 * 2 * kMTile + 2 * 2 * kLargeBM * 4;   // data + scales: 132 KB
static_assert(kWgLds <= kMLds && kWgLds <= kLLds, "weight-gradient staging fits the K stages' LDS");

template <int OPSEL>
__device__ __forceinline__ f32x16 mfma_mx32(i32x8 a, i32x8 b, int sa, int sb, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, OPSEL, sa, OPSEL, sb);
}
}  // namespace

// KIND kGateUp:  act = x codes [T,H] + scales [T,H/32]; wt = W_gate_up codes [E,2I,H] +
//                scales [E,2I,H/32]; writes h codes [P,I] + scales [P,I/32] (sorted rows),
//                quantized from the FP32 SwiGLU values.
// KIND kGateUpRaw: the same product; writes the FP32 g and u of each grouped row to
//                y [P, 2I] (the backward's pre-activations).
// KIND kDown*:   act = h codes + scales; wt = W_down codes [E,H,I] + scales [E,H,I/32]
//                (the backward's dx: act = [dg; du] codes [P, 2I], wt = W_gate_up
//                re-quantized along 2I and transposed, [E, H, 2I], with I passed as 2I).
// KIND kBwdDh:   act = dout codes [T, H] gathered by token; wt = W_down re-quantized
//                along H and transposed, [E, I, H]; writes FP32 dh [P, I] (grouped rows).
// KIND kWgradDown / kWgradGateUp: weight gradients over pair-axis operands [rows][KPT]
//                (codes [rows][KPT] + scale dwords [KPT/128][rows], expert e's routed pairs in columns
//                offsets[e] .. offsets[e+1], zero-padded to multiples of 128; KPT =
//                offsets[E]): kWgradDown A = a^T (rows i), B = (w dout)^T (rows h),
//                writes dW_down[e][h][i]; kWgradGateUp A = x^T (rows h), B = [dg; du]^T
//                (rows c), writes dW_gate_up[e][c][h]; BF16, no K split.
// TS: the scale dwords (4 bytes per row and 128-wide K stage) transposed, so a
// stage's 256 dwords of an operand are consecutive (1 KB) instead of one per
// row, 4 bytes out of each row's scale line (with row-major scales the scale
// lines took ~10% of the MFMA-bound gate_up's time).  Projections: wt_s
// [E][K/128][rows of A] and act_s [K/128][ldsc] by grouped row, made by
// mx_scales_t; weight gradients: both [KPT/128][rows] as the pair-axis encoder
// writes them (ldsc = rows of B).
template <int KIND, bool TS = false>
__global__ __launch_bounds__(256) void gemm_large_mx(
    const uint8_t* __restrict__ act, const uint8_t* __restrict__ act_s,
    const uint8_t* __restrict__ wt, const uint8_t* __restrict__ wt_s,
    const int* __restrict__ perm, const int2* __restrict__ tiles, const int* __restrict__ n_tiles,
    const int* __restrict__ counts, const int* __restrict__ offsets, const float* __restrict__ w,
    int H, int I, int k, uint8_t* __restrict__ hq, uint8_t* __restrict__ hs,
    float* __restrict__ y, uint16_t* __restrict__ out, float* __restrict__ partial, int ncu,
    int E, uint32_t okey, int ldsc) {
  extern __shared__ __align__(16) uint8_t ldm[];   // [stage][A, B][256 x 128] then [stage][A, B][256] dwords
  uint32_t* lsc = reinterpret_cast<uint32_t*>(ldm + 2 * 2 * kMTile);
  constexpr bool kGU = KIND == kGateUp || KIND == kGateUpRaw;   // gate/up rows, gathered x
  constexpr bool kWG = KIND == kWgradGateUp || KIND == kWgradDown;
  constexpr bool kDH = KIND == kBwdDh;               // gathered dout rows, W_down^T rows
  constexpr bool kGather = kGU || kDH;
  const int K = kWG ? offsets[E] : (kGather ? H : I);
  const int KSB = K / 32;                          // scale bytes per row
  const int nA = KIND == kWgradGateUp ? H / 256 : I / 256;       // (weight gradients)
  const int nB = KIND == kWgradGateUp ? 2 * I / 256 : H / 256;
  const int nblk = kGU ? I / 128 : kDH ? I / 256 : H / 256;
  const int nk = K / kMBK;
  const int L = blockIdx.x;
  int item, kb = 0, ke = nk, slot = -1;
  int e, nb, bb = 0, mcount = kLargeBM, rbase = 0;
  if (kWG) {
    const int per = nA * nB, n_w = E * per;
    const int n_pad = (n_w + kXcds - 1) / kXcds * kXcds;
    if (L >= n_pad) return;
    item = permute_item(round_item(L, n_pad, ncu), n_pad, okey);
    if (item >= n_w) return;
    e = item / per;
    large_coords(item - e * per, nA, nB, bb, nb);
    kb = offsets[e] / kMBK;
    ke = offsets[e + 1] / kMBK;
  } else {
    const int n_real = nblk * *n_tiles;
    const TailPlan plan = tail_plan(n_real, ncu, nk);
    if (plan.S > 1 && L < plan.full) {
      item = permute_item(round_item(L, plan.full, ncu), plan.full, okey);
    } else if (plan.S > 1) {
      const int t0 = L - plan.full;
      if (t0 >= plan.rem * plan.S) return;
      const int t = permute_item(t0, plan.rem * plan.S, okey);
      item = plan.full + t % plan.rem;
      const int sl = t / plan.rem;
      kb = sl * nk / plan.S;
      ke = (sl + 1) * nk / plan.S;
      slot = t;
    } else {
      item = round_real_item(L, nblk, *n_tiles, ncu);
      if (item < 0) return;
      item = permute_item(item, nblk * *n_tiles, okey);
    }
    int tile;
    large_coords(item, nblk, *n_tiles, tile, nb);
    const int2 te = tiles[tile];
    e = te.x;
    const int m0 = te.y;
    mcount = min(kLargeBM, counts[e] - m0);
    rbase = offsets[e] + m0;
  }
  const int tid = threadIdx.x, wv = tid >> 6, ln = tid & 63, l32 = ln & 31, hi = ln >> 5;
  const int wm = wv & 1, wn = wv >> 1;

  // data loader as in the BF16 kernel (16-byte chunk ln & 7 of rows wv*64 + 8j + (ln >> 3))
  const int lrow = ln >> 3, lc = ln & 7;
  const uint8_t* __restrict__ abase;
  const uint8_t* __restrict__ asb;
  uint32_t ao, so_a, so_b;
  const int n0 = nb * 128;
  if (kWG) {
    abase = wt;
    asb = wt_s;
    ao = static_cast<uint32_t>((nb * 256 + wv * 64 + lrow) * K + lc * 16);
    so_a = static_cast<uint32_t>((nb * 256 + tid) * (TS ? 1 : KSB));
  } else if (kGU) {
    abase = wt + static_cast<size_t>(e) * 2 * I * H;
    asb = wt_s + static_cast<size_t>(e) * 2 * I * KSB;       // (TS: [nk][2I] dwords of expert e)
    ao = static_cast<uint32_t>(((wv < 2 ? n0 + wv * 64 : I + n0 + (wv - 2) * 64) + lrow) * H + lc * 16);
    so_a = static_cast<uint32_t>((tid < 128 ? n0 + tid : I + n0 + tid - 128) * (TS ? 1 : KSB));
  } else {
    // down: [E][H][K = I] rows h; kDH: [E][I][K = H] rows i
    abase = wt + static_cast<size_t>(e) * H * I;
    asb = wt_s + static_cast<size_t>(e) * (kDH ? I : H) * KSB;
    ao = static_cast<uint32_t>((nb * 256 + wv * 64 + lrow) * K + lc * 16);
    so_a = static_cast<uint32_t>((nb * 256 + tid) * (TS ? 1 : KSB));
  }
  uint32_t bo[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = wv * 64 + 8 * j + lrow;
    const int rr = r < mcount ? r : 0;
    bo[j] = kWG ? static_cast<uint32_t>((bb * 256 + r) * K + lc * 16)
          : kGather ? static_cast<uint32_t>((perm[rbase + rr] / k) * H + lc * 16)
                    : static_cast<uint32_t>((rbase + rr) * I + lc * 16);
  }
  {
    const int rr = tid < mcount ? tid : 0;         // scale loader: thread = tile row
    so_b = TS ? static_cast<uint32_t>(kWG ? bb * 256 + tid : rbase + rr)   // (TS: row of act_s's columns)
              : static_cast<uint32_t>((kWG ? bb * 256 + tid : kGather ? perm[rbase + rr] / k : rbase + rr) *
                                      KSB);
  }
  const int lw = (wv * 64 + lrow) * kMBK + ((lc ^ lrow) * 16);
  int fa[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) fa[i] = (kGU ? (i >> 1) * 128 + wn * 64 + (i & 1) * 32 : wn * 128 + 32 * i) + l32;
  const int fb = wm * 128 + l32;
  const int swz = l32 & 7;

  i32x4 stg[16];
  uint32_t sst[2];
  // (TS) rows of A's transposed scales: W_gate_up 2I, W_down H, W_down^T I; weight
  // gradients x^T H, (w a)^T I
  const uint32_t ra_rows = static_cast<uint32_t>(
      kWG ? (KIND == kWgradGateUp ? H : I) : kGU ? 2 * I : kDH ? I : H);
#define GLOAD(Q, KT) do {                                                               \
    const uint32_t kk_ = static_cast<uint32_t>(min((KT), ke - 1) * kMBK);               \
    if ((Q) < 8) stg[Q] = ld16(abase + ao + static_cast<uint32_t>((Q) * 8) * K + kk_);  \
    else stg[Q] = ld16(act + bo[(Q) - 8] + kk_);                                        \
  } while (0)
#define SLOAD(KT) do {                                                                  \
    const uint32_t ks_ = static_cast<uint32_t>(min((KT), ke - 1));                     \
    if (TS) {                                                                           \
      sst[0] = reinterpret_cast<const uint32_t*>(asb)[ks_ * ra_rows + so_a];                \
      sst[1] = reinterpret_cast<const uint32_t*>(act_s)[ks_ * static_cast<uint32_t>(ldsc) + so_b]; \
    } else {                                                                            \
      sst[0] = *reinterpret_cast<const uint32_t*>(asb + so_a + 4 * ks_);                \
      sst[1] = *reinterpret_cast<const uint32_t*>(act_s + so_b + 4 * ks_);              \
    }                                                                                   \
  } while (0)
#define LWRITE(Q, KT) do {                                                              \
    uint8_t* st_ = ldm + ((KT) & 1) * 2 * kMTile;                                       \
    if ((Q) < 8) *reinterpret_cast<i32x4*>(&st_[lw + (Q) * 8 * kMBK]) = stg[Q];         \
    else *reinterpret_cast<i32x4*>(&st_[kMTile + lw + ((Q) - 8) * 8 * kMBK]) = stg[Q];  \
  } while (0)
#define SWRITE(KT) do {                                                                 \
    uint32_t* sc_ = lsc + ((KT) & 1) * 2 * kLargeBM;                                    \
    sc_[tid] = sst[0];                                                                  \
    sc_[kLargeBM + tid] = sst[1];                                                       \
  } while (0)
  // fragment piece P (0..15) of stage RKT, K step RKS: fragment P >> 1 (A 0..3, B 4..7), half P & 1
#define RDP(F, P, RKT, RKS) do {                                                        \
    const uint8_t* at_ = ldm + ((RKT) & 1) * 2 * kMTile;                                \
    const int fr_ = (P) >> 1, h_ = (P) & 1;                                             \
    const int row_ = fr_ < 4 ? fa[fr_] : fb + 32 * (fr_ - 4);                           \
    const uint8_t* src_ = (fr_ < 4 ? at_ : at_ + kMTile) + row_ * kMBK +               \
                          (((4 * (RKS) + 2 * h_ + hi) ^ swz) * 16);                     \
    const i32x4 v_ = *reinterpret_cast<const i32x4*>(src_);                             \
    _Pragma("unroll") for (int u_ = 0; u_ < 4; ++u_) F[fr_][4 * h_ + u_] = v_[u_];      \
  } while (0)
#define RDS(SC, RKT) do {                                                               \
    const uint32_t* sc_ = lsc + ((RKT) & 1) * 2 * kLargeBM;                             \
    _Pragma("unroll") for (int i_ = 0; i_ < 4; ++i_) SC[i_] = sc_[fa[i_]] >> (8 * hi);  \
    _Pragma("unroll") for (int j_ = 0; j_ < 4; ++j_)                                    \
      SC[4 + j_] = sc_[kLargeBM + fb + 32 * j_] >> (8 * hi);                            \
  } while (0)

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
  // LDS writes of stage s+1 are split between the second K step of stage s-1
  // (chunks 0..7) and the first of stage s (chunks 8..15 and the scales), as in
  // the BF16 kernel.  Prologue: stage kb and chunks 0..7 of stage kb+1 in LDS;
  // registers holding chunks 8..15 and the scales of stage kb+1 and chunks 0..7
  // of stage kb+2.  (A weight-gradient expert with no rows has an empty range:
  // its block is zero.)  A weight-gradient item of a single stage (an expert
  // with at most 128 routed pairs) loads it once and multiplies: the pipelined
  // form would wait on three load round trips of that same stage (its loads of
  // the next stages are clamped to the last one).
  if (kWG && ke - kb == 1) {
#pragma unroll
    for (int q = 0; q < 16; ++q) GLOAD(q, kb);
    SLOAD(kb);
#pragma unroll
    for (int q = 0; q < 16; ++q) LWRITE(q, kb);
    SWRITE(kb);
    __syncthreads();
    i32x8 f0[8], f1[8];
    uint32_t sc[8];
#pragma unroll
    for (int p = 0; p < 16; ++p) RDP(f0, p, kb, 0);
#pragma unroll
    for (int p = 0; p < 16; ++p) RDP(f1, p, kb, 1);
    RDS(sc, kb);
#pragma unroll
    for (int g = 0; g < 16; ++g)
      acc[g >> 2][g & 3] = mfma_mx32<0>(f0[g >> 2], f0[4 + (g & 3)], static_cast<int>(sc[g >> 2]),
                                        static_cast<int>(sc[4 + (g & 3)]), acc[g >> 2][g & 3]);
#pragma unroll
    for (int g = 0; g < 16; ++g)
      acc[g >> 2][g & 3] = mfma_mx32<2>(f1[g >> 2], f1[4 + (g & 3)], static_cast<int>(sc[g >> 2]),
                                        static_cast<int>(sc[4 + (g & 3)]), acc[g >> 2][g & 3]);
  } else if (ke > kb) {
#pragma unroll
  for (int q = 0; q < 16; ++q) GLOAD(q, kb);
  SLOAD(kb);
#pragma unroll
  for (int q = 0; q < 16; ++q) LWRITE(q, kb);
  SWRITE(kb);
#pragma unroll
  for (int q = 0; q < 16; ++q) GLOAD(q, kb + 1);
  SLOAD(kb + 1);
#pragma unroll
  for (int q = 0; q < 8; ++q) { LWRITE(q, kb + 1); GLOAD(q, kb + 2); }
  __syncthreads();
  i32x8 f0[8], f1[8];          // fragments: [0..3] A, [4..7] B
  uint32_t sc[8], scn[8];      // scales of the current / next stage
#pragma unroll
  for (int p = 0; p < 16; ++p) RDP(f0, p, kb, 0);
  RDS(sc, kb);
  for (int kt = kb; kt < ke; ++kt) {
    // K step 0: MFMAs on f0; read K step 1 into f1 (two pieces per MFMA over the
    // first half); chunks 8..15 and scales of stage kt+1 to LDS, each chunk
    // reloaded from stage kt+2
#pragma unroll
    for (int g = 0; g < 16; ++g) {
      const int i = g >> 2, j = g & 3;
      acc[i][j] = mfma_mx32<0>(f0[i], f0[4 + j], static_cast<int>(sc[i]), static_cast<int>(sc[4 + j]), acc[i][j]);
      __builtin_amdgcn_sched_barrier(0);
      if (g < 8) { RDP(f1, 2 * g, kt, 1); RDP(f1, 2 * g + 1, kt, 1); }
      if (g & 1) { LWRITE(8 + (g >> 1), kt + 1); GLOAD(8 + (g >> 1), kt + 2); }
      if (g == 14) { SWRITE(kt + 1); SLOAD(kt + 2); }
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    // K step 1: MFMAs on f1; read K step 0 of stage kt+1 into f0, and its
    // scales; chunks 0..7 of stage kt+2 to LDS, each reloaded from stage kt+3
#pragma unroll
    for (int g = 0; g < 16; ++g) {
      const int i = g >> 2, j = g & 3;
      acc[i][j] = mfma_mx32<2>(f1[i], f1[4 + j], static_cast<int>(sc[i]), static_cast<int>(sc[4 + j]), acc[i][j]);
      __builtin_amdgcn_sched_barrier(0);
      if (g < 8) { RDP(f0, 2 * g, kt + 1, 0); RDP(f0, 2 * g + 1, kt + 1, 0); }
      if (g == 0) RDS(scn, kt + 1);
      if (g & 1) { LWRITE(g >> 1, kt + 2); GLOAD(g >> 1, kt + 3); }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) sc[q] = scn[q];
  }
  }
#undef GLOAD
#undef SLOAD
#undef LWRITE
#undef SWRITE
#undef RDP
#undef RDS

  if (kWG) {
    // dW[e][B row][A row], BF16
    const int colsA = nA * 256;
    __syncthreads();                               // every wave is done with the K stages
    wgrad_store(acc, ldm, out + static_cast<size_t>(e) * (nB * 256) * colsA,
                colsA, bb * 256 + wm * 128, nb * 256 + wn * 128, wv, ln);
    return;
  }

  if (slot >= 0) {
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
  if (KIND == kGateUp) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 2; ++i) mx_store_block(acc[i][j], acc[i + 2][j], wm * 128 + 32 * j + l32, mcount,
                                                 rbase, n0 + wn * 64 + 32 * i, hi, I, hq, hs);
  } else if (KIND == kGateUpRaw) {
    large_epilogue<KIND>(acc, perm, w, H, I, rbase, mcount, nb, wm, wn, l32, hi, nullptr, nullptr, out, y);
  } else {
    large_epilogue<KIND>(acc, perm, w, H, I, rbase, mcount, nb, wm, wn, l32, hi, nullptr, y, out, nullptr);
  }
}

// Tail fix-up of the MXFP8 gate_up: workgroup (item b, block i, token group j) -
// 8 per tail item - sums the slices of gate block i and up block i + 2 for its
// 32 x 32 piece and quantizes it as the GEMM epilogue does.
__global__ __launch_bounds__(256) void gemm_large_mx_fixup_gate_up(
    const int2* __restrict__ tiles, const int* __restrict__ n_tiles,
    const int* __restrict__ counts, const int* __restrict__ offsets, int H, int I,
    uint8_t* __restrict__ hq, uint8_t* __restrict__ hs, const float* __restrict__ partial, int ncu,
    int nk, uint32_t okey) {
  const int nblk = I / 128;
  const TailPlan plan = tail_plan(nblk * *n_tiles, ncu, nk);
  const int pb = permute_item(blockIdx.x, gridDim.x, okey);
  const int b = pb >> 3, i = (pb >> 2) & 1, j = pb & 3;
  if (plan.S == 1 || b >= plan.rem) return;
  const int item = plan.full + b;
  int tile, nb;
  large_coords(item, nblk, *n_tiles, tile, nb);
  const int2 te = tiles[tile];
  const int e = te.x, m0 = te.y;
  const int mcount = min(kLargeBM, counts[e] - m0);
  const int rbase = offsets[e] + m0;
  const int tid = threadIdx.x, wv = tid >> 6, ln = tid & 63, l32 = ln & 31, hi = ln >> 5;
  f32x16 g = {}, u = {};
  for (int sl = 0; sl < plan.S; ++sl) {
    const f32x4* pp = reinterpret_cast<const f32x4*>(partial) +
                      static_cast<size_t>(sl * plan.rem + b) * 64 * 256 + tid;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 vg = pp[((i * 4 + j) * 4 + q) * 256];
      const f32x4 vu = pp[(((i + 2) * 4 + j) * 4 + q) * 256];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        g[4 * q + t] += vg[t];
        u[4 * q + t] += vu[t];
      }
    }
  }
  mx_store_block(g, u, (wv & 1) * 128 + 32 * j + l32, mcount, rbase,
                 nb * 128 + (wv >> 1) * 64 + 32 * i, hi, I, hq, hs);
}

// Weight gradients of experts averaging at most 128 routed pairs (the MXFP8
// backward at T 2048, k 8, E 384: one K stage per expert): 128 x 128 dW tiles,
// four waves of 64 x 64 (64 accumulator registers per lane, so two workgroups
// share a CU - the 256 x 256 tile of gemm_large_mx runs one per CU, which waits
// for its loads and drains its stores with nothing else to do).  A workgroup
// takes one 128-row block of B (dW rows) and kW1Run consecutive 128-row blocks
// of A (dW columns): for a single-stage expert the B block stays in LDS, and the
// next A block's loads fly while the current block multiplies and its dW block
// is stored.  Operands and products as gemm_large_mx's weight-gradient kinds
// (`bm`: its act, B rows = dW rows; `am`: its wt, A rows = dW columns; the same
// block-scaled 32x32x64 MFMA on the same fragments, K steps in the same order),
// so the result is bit-identical; experts with more than one stage take each A
// block's stages one at a time.  A wave's finished 64 x 64 block leaves through
// its own LDS region as eight whole 128-byte row segments per store instruction.
constexpr int kW1Run = 4;                                  // A blocks per workgroup
constexpr int kW1Tile = 128 * kMBK;                        // bytes per operand stage
constexpr int kW1Row = 128 + 16;                           // bytes per staged dW row (+16: banks)
constexpr int kW1Stage = 2 * kW1Tile + 2 * 128 * 4;        // A, B codes and their scale dwords
constexpr int kW1Lds = kW1Stage + 4 * 64 * kW1Row;         // + dW staging: 69 KB
template <int KIND>
__global__ __launch_bounds__(256) void wgrad_mx_t128(
    const uint8_t* __restrict__ bm, const uint8_t* __restrict__ bms, const uint8_t* __restrict__ am,
    const uint8_t* __restrict__ ams, const int* __restrict__ offsets, int H, int I, int E,
    uint16_t* __restrict__ out, uint32_t okey) {
  static_assert(KIND == kWgradGateUp || KIND == kWgradDown, "weight-gradient kinds");
  extern __shared__ __align__(16) uint8_t ldm[];    // [A, B][128 x 128], [A, B][128] dwords; dW staging
  uint32_t* lsc = reinterpret_cast<uint32_t*>(ldm + 2 * kW1Tile);
  const int K = offsets[E];                          // row stride of both operands' codes
  const int nA = KIND == kWgradGateUp ? H / 128 : I / 128;   // a multiple of kW1Run
  const int nB = KIND == kWgradGateUp ? 2 * I / 128 : H / 128;
  const int nG = nA / kW1Run;
  const int per = nG * nB, n_w = E * per;
  const int n_pad = (n_w + kXcds - 1) / kXcds * kXcds;
  const int L = blockIdx.x;
  if (L >= n_pad) return;
  const int item = permute_item(xcd_item(L, n_pad), n_pad, okey);
  if (item >= n_w) return;
  const int e = item / per;
  int bb, ng;
  large_coords(item - e * per, nG, nB, bb, ng);
  const int kb = offsets[e] / kMBK, ke = offsets[e + 1] / kMBK;
  const int tid = threadIdx.x, wv = tid >> 6, ln = tid & 63, l32 = ln & 31, hi = ln >> 5;
  const int wm = wv & 1, wn = wv >> 1;               // B rows 64 wm .., A rows 64 wn ..
  // loader: chunk u = tid + 256 i of an operand block -> row u >> 3, 16-byte chunk
  // u & 7, LDS slot (u & 7) ^ (row & 7); scale dwords ([K/128][rows] per operand,
  // as the pair-axis encoder writes them): thread tid < 128 the A block's row tid,
  // the others the B block's row tid - 128
  uint32_t ro[4];
  int lw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int u = tid + 256 * i, r = u >> 3, c = u & 7;
    ro[i] = static_cast<uint32_t>(r * K + c * 16);
    lw[i] = r * kMBK + ((c ^ (r & 7)) * 16);
  }
  const bool sa_lane = tid < 128;
  const uint32_t b_off = static_cast<uint32_t>(bb * 128 * K);
  i32x4 ra[4], rb[4];
  uint32_t rs;
  auto load_a = [&](int nb, int kt) {               // A block nb, stage kt (and, tid < 128, its scales)
    const uint8_t* p = am + static_cast<uint32_t>(nb * 128 * K) + static_cast<uint32_t>(kt * kMBK);
#pragma unroll
    for (int i = 0; i < 4; ++i) ra[i] = ld16(p + ro[i]);
    if (sa_lane) rs = reinterpret_cast<const uint32_t*>(ams)[static_cast<uint32_t>(kt * (nA * 128) + nb * 128 + tid)];
  };
  auto load_b = [&](int kt) {                       // B block, stage kt (and, tid >= 128, its scales)
    const uint8_t* p = bm + b_off + static_cast<uint32_t>(kt * kMBK);
#pragma unroll
    for (int i = 0; i < 4; ++i) rb[i] = ld16(p + ro[i]);
    if (!sa_lane) rs = reinterpret_cast<const uint32_t*>(bms)[static_cast<uint32_t>(kt * (nB * 128) + bb * 128 + tid - 128)];
  };
  auto put_a = [&] {
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<i32x4*>(&ldm[lw[i]]) = ra[i];
    if (sa_lane) lsc[tid] = rs;
  };
  auto put_b = [&] {
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<i32x4*>(&ldm[kW1Tile + lw[i]]) = rb[i];
    if (!sa_lane) lsc[tid] = rs;
  };
  f32x16 acc[2][2];
  auto zero = [&] {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
  };
  // fragments: A rows 64 wn + 32 i + l32, B rows 64 wm + 32 j + l32 (gemm_large_mx's
  // pieces: at K step ks lane hi takes chunks 4 ks + hi and 4 ks + 2 + hi)
  const int swz = l32 & 7;
  auto multiply = [&] {
    uint32_t sc[4];
#pragma unroll
    for (int i = 0; i < 2; ++i) sc[i] = lsc[64 * wn + 32 * i + l32] >> (8 * hi);
#pragma unroll
    for (int j = 0; j < 2; ++j) sc[2 + j] = lsc[128 + 64 * wm + 32 * j + l32] >> (8 * hi);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      i32x8 f[4];                                   // [0, 1] A, [2, 3] B
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const int fr = p >> 1, h = p & 1;
        const int row = fr < 2 ? 64 * wn + 32 * fr + l32 : 64 * wm + 32 * (fr - 2) + l32;
        const i32x4 v = *reinterpret_cast<const i32x4*>((fr < 2 ? ldm : ldm + kW1Tile) + row * kMBK +
                                                        (((4 * ks + 2 * h + hi) ^ swz) * 16));
#pragma unroll
        for (int u = 0; u < 4; ++u) f[fr][4 * h + u] = v[u];
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int i = g >> 1, j = g & 1;
        if (ks == 0)
          acc[i][j] = mfma_mx32<0>(f[i], f[2 + j], static_cast<int>(sc[i]), static_cast<int>(sc[2 + j]), acc[i][j]);
        else
          acc[i][j] = mfma_mx32<2>(f[i], f[2 + j], static_cast<int>(sc[i]), static_cast<int>(sc[2 + j]), acc[i][j]);
      }
    }
  };
  // dW[e][B row][A row], BF16: lane (l32, hi) holds A row (dW column) 32 i + 8 q + 4 hi + t
  // and B row (dW row) 32 j + l32 of the wave's block (register 4 q + t of acc[i][j])
  const int cols = nA * 128;
  uint16_t* dw = out + static_cast<size_t>(e) * (nB * 128) * cols + static_cast<size_t>(bb * 128 + 64 * wm) * cols;
  uint8_t* st = ldm + kW1Stage + wv * 64 * kW1Row;
  auto store = [&](int nb) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<uint2*>(st + (32 * j + l32) * kW1Row + (32 * i + 8 * q + 4 * hi) * 2) =
              make_uint2(pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]),
                         pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]));
    // a wave's LDS operations complete in order: the reads see the writes above
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int r = 8 * s + (ln >> 3), c = ln & 7;
      st16_stream(dw + static_cast<size_t>(r) * cols + nb * 128 + 64 * wn + 8 * c,
                  *reinterpret_cast<const i32x4*>(st + r * kW1Row + 16 * c));
    }
  };

  const int nb0 = ng * kW1Run;
  zero();
  if (ke - kb == 1) {
    // the B block stays in LDS; A block m + 1 is loaded while block m multiplies
    // and is stored
    load_b(kb);
    put_b();
    load_a(nb0, kb);
    put_a();
    load_a(nb0 + 1, kb);
    __syncthreads();
    for (int m = 0; m < kW1Run; ++m) {
      multiply();
      __syncthreads();                              // every wave is done reading A block m
      if (m + 1 < kW1Run) {
        put_a();
        if (m + 2 < kW1Run) load_a(nb0 + m + 2, kb);
      }
      store(nb0 + m);
      zero();
      __syncthreads();                              // A block m + 1 is in LDS
    }
  } else {
    for (int m = 0; m < kW1Run; ++m) {
      for (int kt = kb; kt < ke; ++kt) {
        load_b(kt);
        load_a(nb0 + m, kt);
        __syncthreads();                            // every wave is done reading the last stage
        put_b();
        put_a();
        __syncthreads();
        multiply();
      }
      store(nb0 + m);                               // (an expert with no pairs: zeros)
      zero();
    }
  }
}

// Scale dwords (the 4 E8M0 bytes of one 128-wide K stage) transposed for the
// large-tile MXFP8 GEMM, weights and activations in one launch:
//   wout[e][kt][r] = win[e][r][kt]                    (r < wrows, E experts)
//   aout[kt][r]    = ain[perm ? perm[r] / k : r][kt]  (r < P; with perm - the
//                    activation rows gathered into grouped order - only the
//                    routed pairs r < offsets[E], the rest left alone)
// Tiles of 64 rows x 32 stages through LDS, reads and writes along rows of
// their own layout; the first E * (weight tiles per expert) workgroups take the
// weights.
__global__ __launch_bounds__(256) void mx_scales_t(const uint32_t* __restrict__ win, int wrows,
                                                   int E, const uint32_t* __restrict__ ain, int P,
                                                   int nk, const int* __restrict__ perm, int k,
                                                   const int* __restrict__ offsets,
                                                   uint32_t* __restrict__ wout,
                                                   uint32_t* __restrict__ aout) {
  __shared__ uint32_t t[64][33];
  const int tk = (nk + 31) / 32, twr = (wrows + 63) / 64;
  const int nwt = E * twr * tk;
  const bool wpart = static_cast<int>(blockIdx.x) < nwt;
  const int b = wpart ? blockIdx.x : blockIdx.x - nwt;
  const int per = wpart ? twr * tk : 0;
  const int e = wpart ? b / per : 0;
  const int rem = wpart ? b - e * per : b;
  const int r0 = (rem / tk) * 64, k0 = (rem % tk) * 32;
  const int rows = wpart ? wrows : P;
  const int nrows = wpart || !perm ? rows : min(P, offsets[E]);
  const uint32_t* __restrict__ ib = wpart ? win + static_cast<size_t>(e) * wrows * nk : ain;
  uint32_t* __restrict__ ob = wpart ? wout + static_cast<size_t>(e) * nk * wrows : aout;
  for (int i = threadIdx.x; i < 64 * 32; i += 256) {
    const int rr = i >> 5, kk = i & 31, r = r0 + rr, kt = k0 + kk;
    if (r < nrows && kt < nk) {
      const int src = !wpart && perm ? perm[r] / k : r;
      t[rr][kk] = ib[static_cast<size_t>(src) * nk + kt];
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 32; i += 256) {
    const int kk = i >> 6, rr = i & 63, r = r0 + rr, kt = k0 + kk;
    if (r < nrows && kt < nk) ob[static_cast<size_t>(kt) * rows + r] = t[rr][kk];
  }
}

size_t mx_scales_t_bytes(int P, int H, int I, int E) {
  const size_t gu = static_cast<size_t>(E) * 2 * I * (H / 32) + static_cast<size_t>(P) * (H / 32);
  const size_t dn = static_cast<size_t>(E) * H * (I / 32) + static_cast<size_t>(P) * (I / 32);
  return gu > dn ? gu : dn;
}

namespace {
// transposed weight scales [E][K/128][rows] at sct, activation scales [K/128][P] after them
void transpose_scales(const uint8_t* ws_, int rows, int K, const uint8_t* as_, int P,
                      const int* perm, int k, const int* offsets, int E, uint32_t* sct,
                      hipStream_t s) {
  const int nk = K / 128, tk = (nk + 31) / 32;
  const int nblk = E * ((rows + 63) / 64) * tk + ((P + 63) / 64) * tk;
  hipLaunchKernelGGL(mx_scales_t, dim3(nblk), dim3(256), 0, s, reinterpret_cast<const uint32_t*>(ws_),
                     rows, E, reinterpret_cast<const uint32_t*>(as_), P, nk, perm, k, offsets, sct,
                     sct + static_cast<size_t>(E) * nk * rows);
}

// grid: every item whole, plus room for the tail slices (rem * S - rem < ncu)
int large_grid(int nblk, int max_tiles, int ncu) {
  return (nblk * max_tiles + ncu + kXcds - 1) / kXcds * kXcds;
}
}  // namespace

hipError_t launch_gate_up_large_bf16(const uint16_t* x, const uint16_t* wgu, const int* perm,
                                     const int2* tiles, const int* n_tiles, const int* counts,
                                     const int* offsets, int H, int I, int k, uint16_t* h,
                                     float* partial, int max_tiles, int ncu, hipStream_t s,
                                     float* gu) {
  const int grid = large_grid(I / 128, max_tiles, ncu);
#define LARGE_GU(KG)                                                                          \
  hipLaunchKernelGGL(gemm_large_bf16<KG>, dim3(grid), dim3(256), kLLds, s, x, wgu, perm,       \
                     tiles, n_tiles, counts, offsets, nullptr, H, I, k, h, nullptr, nullptr,  \
                     partial, ncu, gu, 0, order_key());                                                    \
  hipLaunchKernelGGL(gemm_large_fixup<KG>, dim3(ncu / 2 * 32), dim3(256), 0, s, perm, tiles,   \
                     n_tiles, counts, offsets, nullptr, H, I, h, nullptr, nullptr, partial, ncu, \
                     H / kLBK, gu, order_key())
  if (gu) { LARGE_GU(kGateUpSave); } else { LARGE_GU(kGateUp); }
#undef LARGE_GU
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
                     n_tiles, counts, offsets, w, H, I, k, nullptr, y, out, partial, ncu,     \
                     nullptr, 0, order_key());                                                             \
  hipLaunchKernelGGL(gemm_large_fixup<KD>, dim3(ncu / 2 * 64), dim3(256), 0, s, perm, tiles,   \
                     n_tiles, counts, offsets, w, H, I, nullptr, y, out, partial, ncu, I / kLBK, \
                     nullptr, order_key())
  if (k == 1) { LARGE_DOWN(kDownFused); } else { LARGE_DOWN(kDownSlots); }
#undef LARGE_DOWN
  return hipGetLastError();
}

hipError_t launch_gate_up_large_mx(const uint8_t* x, const uint8_t* xs, const uint8_t* wgu,
                                   const uint8_t* wgus, const int* perm, const int2* tiles,
                                   const int* n_tiles, const int* counts, const int* offsets, int H,
                                   int I, int k, uint8_t* hq, uint8_t* hs, float* partial,
                                   int max_tiles, int ncu, hipStream_t s, int T, int E,
                                   uint32_t* sct) {
  const int grid = large_grid(I / 128, max_tiles, ncu);
  const int P = T * k;
  transpose_scales(wgus, 2 * I, H, xs, P, perm, k, offsets, E, sct, s);
  const uint8_t* wst = reinterpret_cast<const uint8_t*>(sct);
  const uint8_t* xst = reinterpret_cast<const uint8_t*>(sct + static_cast<size_t>(E) * (H / 128) * 2 * I);
  hipLaunchKernelGGL((gemm_large_mx<kGateUp, true>), dim3(grid), dim3(256), kMLds, s, x, xst, wgu, wst,
                     perm, tiles, n_tiles, counts, offsets, nullptr, H, I, k, hq, hs, nullptr,
                     nullptr, partial, ncu, 0, order_key(), P);
  hipLaunchKernelGGL(gemm_large_mx_fixup_gate_up, dim3(ncu / 2 * 8), dim3(256), 0, s, tiles,
                     n_tiles, counts, offsets, H, I, hq, hs, partial, ncu, H / kMBK, order_key());
  return hipGetLastError();
}

hipError_t launch_down_large_mx(const uint8_t* hq, const uint8_t* hs, const uint8_t* wd,
                                const uint8_t* wds, const int* perm, const int2* tiles,
                                const int* n_tiles, const int* counts, const int* offsets,
                                const float* w, int H, int I, int k, float* y, uint16_t* out,
                                float* partial, int max_tiles, int ncu, hipStream_t s, int T,
                                int E, uint32_t* sct) {
  const int grid = large_grid(H / 256, max_tiles, ncu);
  const int P = T * k;
  // h's rows are already grouped: its scales transpose without a gather
  transpose_scales(wds, H, I, hs, P, nullptr, 1, offsets, E, sct, s);
  const uint8_t* wst = reinterpret_cast<const uint8_t*>(sct);
  const uint8_t* hst = reinterpret_cast<const uint8_t*>(sct + static_cast<size_t>(E) * (I / 128) * H);
#define LARGE_DOWN_MX(KD)                                                                     \
  hipLaunchKernelGGL((gemm_large_mx<KD, true>), dim3(grid), dim3(256), kMLds, s, hq, hst, wd, wst, \
                     perm, tiles, n_tiles, counts, offsets, w, H, I, k, nullptr, nullptr, y,  \
                     out, partial, ncu, 0, order_key(), P);                                   \
  hipLaunchKernelGGL(gemm_large_fixup<KD>, dim3(ncu / 2 * 64), dim3(256), 0, s, perm, tiles,   \
                     n_tiles, counts, offsets, w, H, I, nullptr, y, out, partial, ncu, I / kMBK, \
                     nullptr, order_key())
  if (k == 1) { LARGE_DOWN_MX(kDownFused); } else { LARGE_DOWN_MX(kDownSlots); }
#undef LARGE_DOWN_MX
  return hipGetLastError();
}

// ---- MXFP8 backward on the large-tile GEMM (launched from backward.hip) ----

hipError_t launch_gate_up_raw_large_mx(const uint8_t* xq, const uint8_t* xs, const uint8_t* wgu,
                                       const uint8_t* wgus, const int* perm, const int2* tiles,
                                       const int* n_tiles, const int* counts, const int* offsets,
                                       int H, int I, int k, float* gu, float* partial,
                                       int max_tiles, int ncu, hipStream_t s, int T, int E,
                                       uint32_t* sct) {
  const int grid = large_grid(I / 128, max_tiles, ncu);
  const int P = T * k;
  transpose_scales(wgus, 2 * I, H, xs, P, perm, k, offsets, E, sct, s);
  const uint8_t* wst = reinterpret_cast<const uint8_t*>(sct);
  const uint8_t* xst = reinterpret_cast<const uint8_t*>(sct + static_cast<size_t>(E) * (H / 128) * 2 * I);
  hipLaunchKernelGGL((gemm_large_mx<kGateUpRaw, true>), dim3(grid), dim3(256), kMLds, s, xq, xst, wgu, wst,
                     perm, tiles, n_tiles, counts, offsets, nullptr, H, I, k, nullptr, nullptr, gu,
                     nullptr, partial, ncu, 0, order_key(), P);
  hipLaunchKernelGGL(gemm_large_fixup<kGateUpRaw>, dim3(ncu / 2 * 32), dim3(256), 0, s, perm, tiles,
                     n_tiles, counts, offsets, nullptr, H, I, nullptr, nullptr, nullptr, partial,
                     ncu, H / kMBK, gu, order_key());
  return hipGetLastError();
}

hipError_t launch_dh_large_mx(const uint8_t* dq, const uint8_t* ds, const uint8_t* wdT,
                              const uint8_t* wdTs, const int* perm, const int2* tiles,
                              const int* n_tiles, const int* counts, const int* offsets, int H,
                              int I, int k, float* dh, float* partial, int max_tiles, int ncu,
                              hipStream_t s, int T, int E, uint32_t* sct) {
  const int grid = large_grid(I / 256, max_tiles, ncu);
  const int P = T * k;
  transpose_scales(wdTs, I, H, ds, P, perm, k, offsets, E, sct, s);
  const uint8_t* wst = reinterpret_cast<const uint8_t*>(sct);
  const uint8_t* dst_ = reinterpret_cast<const uint8_t*>(sct + static_cast<size_t>(E) * (H / 128) * I);
  hipLaunchKernelGGL((gemm_large_mx<kBwdDh, true>), dim3(grid), dim3(256), kMLds, s, dq, dst_, wdT, wst, perm,
                     tiles, n_tiles, counts, offsets, nullptr, H, I, k, nullptr, nullptr, dh,
                     nullptr, partial, ncu, 0, order_key(), P);
  hipLaunchKernelGGL(gemm_large_fixup<kBwdDh>, dim3(ncu / 2 * 64), dim3(256), 0, s, perm, tiles,
                     n_tiles, counts, offsets, nullptr, H, I, nullptr, dh, nullptr, partial, ncu,
                     H / kMBK, nullptr, order_key());
  return hipGetLastError();
}

hipError_t launch_dgrad_large_mx(const uint8_t* aq, const uint8_t* as, const uint8_t* wT,
                                 const uint8_t* wTs, const int* perm, const int2* tiles,
                                 const int* n_tiles, const int* counts, const int* offsets, int H,
                                 int K, int k, float* y, uint16_t* out, float* partial,
                                 int max_tiles, int ncu, hipStream_t s, int T, int E,
                                 uint32_t* sct) {
  const int grid = large_grid(H / 256, max_tiles, ncu);
  const int P = T * k;
  transpose_scales(wTs, H, K, as, P, nullptr, 1, offsets, E, sct, s);   // rows grouped already
  const uint8_t* wst = reinterpret_cast<const uint8_t*>(sct);
  const uint8_t* ast = reinterpret_cast<const uint8_t*>(sct + static_cast<size_t>(E) * (K / 128) * H);
#define DGRAD_MX(KD)                                                                          \
  hipLaunchKernelGGL((gemm_large_mx<KD, true>), dim3(grid), dim3(256), kMLds, s, aq, ast, wT, wst, perm, \
                     tiles, n_tiles, counts, offsets, nullptr, H, K, k, nullptr, nullptr, y,  \
                     out, partial, ncu, 0, order_key(), P);                                     \
  hipLaunchKernelGGL(gemm_large_fixup<KD>, dim3(ncu / 2 * 64), dim3(256), 0, s, perm, tiles,   \
                     n_tiles, counts, offsets, nullptr, H, K, nullptr, y, out, partial, ncu,   \
                     K / kMBK, nullptr, order_key())
  if (k == 1) { DGRAD_MX(kDownPlain); } else { DGRAD_MX(kDownSlots); }
#undef DGRAD_MX
  return hipGetLastError();
}

hipError_t launch_wgrad_large_mx(const uint8_t* aT, const uint8_t* aTs, const uint8_t* dyT,
                                 const uint8_t* dyTs, const uint8_t* xT, const uint8_t* xTs,
                                 const uint8_t* dguT, const uint8_t* dguTs, const int* koff,
                                 int H, int I, int E, uint16_t* dwgu, uint16_t* dwd, bool small,
                                 int ncu, hipStream_t s) {
  // 128 x 128 tiles, two workgroups per CU (runs of kW1Run A blocks: H and I multiples of 512)
  if (small && (I / 128) % kW1Run == 0 && (H / 128) % kW1Run == 0) {
    const int nd1 = (E * (I / 128 / kW1Run) * (H / 128) + kXcds - 1) / kXcds * kXcds;
    hipLaunchKernelGGL(wgrad_mx_t128<kWgradDown>, dim3(nd1), dim3(256), kW1Lds, s, dyT, dyTs, aT,
                       aTs, koff, H, I, E, dwd, order_key());
    const int ng1 = (E * (H / 128 / kW1Run) * (2 * I / 128) + kXcds - 1) / kXcds * kXcds;
    hipLaunchKernelGGL(wgrad_mx_t128<kWgradGateUp>, dim3(ng1), dim3(256), kW1Lds, s, dguT, dguTs,
                       xT, xTs, koff, H, I, E, dwgu, order_key());
    return hipGetLastError();
  }
  const int nd = (E * (I / 256) * (H / 256) + kXcds - 1) / kXcds * kXcds;
  hipLaunchKernelGGL((gemm_large_mx<kWgradDown, true>), dim3(nd), dim3(256), kMLds, s, dyT, dyTs, aT, aTs,
                     nullptr, nullptr, nullptr, nullptr, koff, nullptr, H, I, 1, nullptr, nullptr,
                     nullptr, dwd, nullptr, ncu, E, order_key(), H);
  const int ng = (E * (H / 256) * (2 * I / 256) + kXcds - 1) / kXcds * kXcds;
  hipLaunchKernelGGL((gemm_large_mx<kWgradGateUp, true>), dim3(ng), dim3(256), kMLds, s, dguT, dguTs, xT,
                     xTs, nullptr, nullptr, nullptr, nullptr, koff, nullptr, H, I, 1, nullptr,
                     nullptr, nullptr, dwgu, nullptr, ncu, E, order_key(), 2 * I);
  return hipGetLastError();
}

namespace {
// Column offsets of the weight-gradient operands: koff[e] = sum over e' < e of
// counts[e'] rounded up to 64, koff[E] = KPT.  One wave: each lane sums a run of
// experts, then an exclusive scan over the lanes.
__global__ __launch_bounds__(64) void wgrad_koff(const int* __restrict__ counts, int E,
                                                 int* __restrict__ koff, int pad) {
  const int ln = threadIdx.x;
  const int per = (E + 63) / 64, e0 = ln * per, e1 = min(E, e0 + per);
  int sum = 0;
  for (int e = e0; e < e1; ++e) sum += (counts[e] + pad - 1) / pad * pad;
  int incl = sum;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(incl, d, kWave);
    if (ln >= d) incl += v;
  }
  int run = incl - sum;
  for (int e = e0; e < e1; ++e) {
    koff[e] = run;
    run += (counts[e] + pad - 1) / pad * pad;
  }
  if (ln == 63) koff[E] = incl;
}

// Gather-transpose for the weight gradients: dst[c][koff[e] + r] = element c of
// expert e's r-th routed row, 0 for r in [counts[e], padded end).  TOKEN: the row
// is token perm[offsets[e] + r] / k of src (x, dout); otherwise grouped row
// offsets[e] + r (dgu, w a).  Workgroup = 64 routed rows x 64 columns, through
// an LDS tile; 16-byte loads along the source rows, 16-byte stores along dst rows.
template <bool TOKEN>
__global__ __launch_bounds__(256) void wgrad_transpose(
    const uint16_t* __restrict__ src, int C, const int* __restrict__ perm, int k,
    const int* __restrict__ counts, const int* __restrict__ offsets,
    const int* __restrict__ koff, int E, uint16_t* __restrict__ dst, uint32_t okey) {
  __shared__ __align__(16) uint16_t tl[64][64 + 8];
  const int KPT = koff[E];
  const int g0 = permute_item(blockIdx.x, gridDim.x, okey) * 64, c0 = blockIdx.y * 64;
  if (g0 >= KPT) return;
  int lo = 0, hi = E - 1;                         // last e with koff[e] <= g0 (ranges non-empty)
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (koff[mid] <= g0) lo = mid; else hi = mid - 1;
  }
  const int e = lo, r0 = g0 - koff[e], cnt = counts[e], goff = offsets[e];
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int ch = tid + 256 * u, r = ch >> 3, cc = ch & 7;
    i32x4 v = {0, 0, 0, 0};
    if (r0 + r < cnt) {
      const int gr = goff + r0 + r;
      const int row = TOKEN ? perm[gr] / k : gr;
      v = ld16(src + static_cast<size_t>(row) * C + c0 + cc * 8);
    }
    *reinterpret_cast<i32x4*>(&tl[r][cc * 8]) = v;
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int ch = tid + 256 * u, c = ch >> 3, rc = ch & 7;
    uint32_t p[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
      p[t] = static_cast<uint32_t>(tl[rc * 8 + 2 * t][c]) | (static_cast<uint32_t>(tl[rc * 8 + 2 * t + 1][c]) << 16);
    *reinterpret_cast<uint4*>(dst + static_cast<size_t>(c0 + c) * KPT + g0 + rc * 8) =
        make_uint4(p[0], p[1], p[2], p[3]);
  }
}

}  // namespace

size_t wgrad_large_cols(int P, int E) {
  return static_cast<size_t>(P) + static_cast<size_t>(kLBK - 1) * E;
}

hipError_t launch_wgrad_large(const uint16_t* x, const uint16_t* dout, const uint16_t* dgu,
                              const uint16_t* wa, const int* perm, const int* counts,
                              const int* offsets, int P, int H, int I, int E, int k, int* koff,
                              uint16_t* xT, uint16_t* doutT, uint16_t* dguT, uint16_t* waT,
                              uint16_t* dwgu, uint16_t* dwd, int ncu, hipStream_t s) {
  const unsigned gtiles = static_cast<unsigned>((wgrad_large_cols(P, E) + 63) / 64);
  hipLaunchKernelGGL(wgrad_koff, dim3(1), dim3(64), 0, s, counts, E, koff, kLBK);
  auto grid_w = [&](int nA, int nB) {
    return dim3(static_cast<unsigned>((E * nA * nB + kXcds - 1) / kXcds * kXcds));
  };
  prof_begin(kBwdWDown, s);
  hipLaunchKernelGGL(wgrad_transpose<false>, dim3(gtiles, I / 64), dim3(256), 0, s, wa, I, perm, k,
                     counts, offsets, koff, E, waT, order_key());
  hipLaunchKernelGGL(wgrad_transpose<true>, dim3(gtiles, H / 64), dim3(256), 0, s, dout, H, perm, k,
                     counts, offsets, koff, E, doutT, order_key());
  hipLaunchKernelGGL(gemm_large_bf16<kWgradDown>, grid_w(I / 256, H / 256), dim3(256), kLLds, s,
                     doutT, waT, perm, nullptr, nullptr, counts, koff, nullptr, H, I, k, nullptr,
                     nullptr, dwd, nullptr, ncu, nullptr, E, order_key());
  prof_end(kBwdWDown, s);
  prof_begin(kBwdWGateUp, s);
  hipLaunchKernelGGL(wgrad_transpose<true>, dim3(gtiles, H / 64), dim3(256), 0, s, x, H, perm, k,
                     counts, offsets, koff, E, xT, order_key());
  hipLaunchKernelGGL(wgrad_transpose<false>, dim3(gtiles, 2 * I / 64), dim3(256), 0, s, dgu, 2 * I,
                     perm, k, counts, offsets, koff, E, dguT, order_key());
  hipLaunchKernelGGL(gemm_large_bf16<kWgradGateUp>, grid_w(H / 256, 2 * I / 256), dim3(256), kLLds,
                     s, dguT, xT, perm, nullptr, nullptr, counts, koff, nullptr, H, I, k, nullptr,
                     nullptr, dwgu, nullptr, ncu, nullptr, E, order_key());
  prof_end(kBwdWGateUp, s);
  return hipGetLastError();
}

hipError_t launch_dh_large(const uint16_t* dout, const uint16_t* wd, const int* perm,
                           const int2* tiles, const int* n_tiles, const int* counts,
                           const int* offsets, int H, int I, int k, float* dh, float* partial,
                           int max_tiles, int ncu, hipStream_t s) {
  const int grid = large_grid(I / 256, max_tiles, ncu);
  hipLaunchKernelGGL((gemm_large_bf16<kBwdDh, true>), dim3(grid), dim3(256), kLLds, s, dout, wd, perm,
                     tiles, n_tiles, counts, offsets, nullptr, H, I, k, nullptr, dh, nullptr,
                     partial, ncu, nullptr, 0, order_key());
  hipLaunchKernelGGL(gemm_large_fixup<kBwdDh>, dim3(ncu / 2 * 64), dim3(256), 0, s, perm, tiles,
                     n_tiles, counts, offsets, nullptr, H, I, nullptr, dh, nullptr, partial, ncu,
                     H / kLBK, nullptr, order_key());
  return hipGetLastError();
}

hipError_t launch_dgrad_large(const uint16_t* act, const uint16_t* w_in, const int* perm,
                              const int2* tiles, const int* n_tiles, const int* counts,
                              const int* offsets, int H, int K, int k, float* y, uint16_t* out,
                              float* partial, int max_tiles, int ncu, hipStream_t s) {
  const int grid = large_grid(H / 256, max_tiles, ncu);
#define DGRAD(KD)                                                                             \
  hipLaunchKernelGGL((gemm_large_bf16<KD, true>), dim3(grid), dim3(256), kLLds, s, act, w_in, perm, tiles, \
                     n_tiles, counts, offsets, nullptr, H, K, k, nullptr, y, out, partial, ncu,  \
                     nullptr, 0, order_key());                                                                \
  hipLaunchKernelGGL(gemm_large_fixup<KD>, dim3(ncu / 2 * 64), dim3(256), 0, s, perm, tiles,      \
                     n_tiles, counts, offsets, nullptr, H, K, nullptr, y, out, partial, ncu,      \
                     K / kLBK, nullptr, order_key())
  if (k == 1) { DGRAD(kDownPlain); } else { DGRAD(kDownSlots); }
#undef DGRAD
  return hipGetLastError();
}

// Column offsets of the pair-axis operands padded to 128 (the MX stage).
hipError_t launch_koff_mx(const int* counts, int E, int* koff, hipStream_t s) {
  hipLaunchKernelGGL(wgrad_koff, dim3(1), dim3(64), 0, s, counts, E, koff, kMBK);
  return hipGetLastError();
}

hipError_t large_set_attributes() {
  const int bytes = static_cast<int>(kLLds);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_large_bf16<kGateUp>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess)
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_large_bf16<kGateUpSave>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess)
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_large_bf16<kBwdDh, true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess)
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_large_bf16<kDownPlain, true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess)
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_large_bf16<kDownSlots, true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess)
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_large_bf16<kWgradGateUp>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess)
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_large_bf16<kWgradDown>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess)
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_large_bf16<kDownFused>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess)
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_large_bf16<kDownSlots>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  const int mbytes = static_cast<int>(kMLds);
  if (e == hipSuccess)
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_large_mx<kGateUp, true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, mbytes);
  if (e == hipSuccess)
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_large_mx<kDownFused, true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, mbytes);
  if (e == hipSuccess)
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_large_mx<kDownSlots, true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, mbytes);
  const void* mx_bwd[] = {reinterpret_cast<const void*>(gemm_large_mx<kGateUpRaw, true>),
                          reinterpret_cast<const void*>(gemm_large_mx<kBwdDh, true>),
                          reinterpret_cast<const void*>(gemm_large_mx<kDownPlain, true>),
                          reinterpret_cast<const void*>(gemm_large_mx<kWgradDown, true>),
                          reinterpret_cast<const void*>(gemm_large_mx<kWgradGateUp, true>)};
  for (const void* f : mx_bwd)
    if (e == hipSuccess) e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, mbytes);
  const void* t128[] = {reinterpret_cast<const void*>(wgrad_mx_t128<kWgradDown>),
                        reinterpret_cast<const void*>(wgrad_mx_t128<kWgradGateUp>)};
  for (const void* f : t128)
    if (e == hipSuccess) e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, kW1Lds);
  return e;
}

}  // namespace moe
