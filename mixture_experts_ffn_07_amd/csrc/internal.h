// Launch wrappers between the C ABI (abi.cpp) and the kernels (*.hip).
// Arguments have been validated by the caller; each returns hipGetLastError()
// after its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Timing hook set by moe_profile_kernel (per calling thread): launches of
// kernel `id` are bracketed by the two events when they are set.
struct ProfileHook {
  int kernel = 0;
  hipEvent_t start = nullptr, stop = nullptr;
};
ProfileHook& profile_hook();

// Test and debugging options set by moe_set_debug_options (per calling thread).
struct DebugOptions {
  unsigned flags = 0;      // kDebugPermute | kDebugDecodeFused
  uint32_t seed = 0;       // permutation of the workgroup -> work-item order
};
constexpr unsigned kDebugPermute = 1u;
constexpr unsigned kDebugDecodeFused = 2u;
DebugOptions& debug_options();
// The work-item permutation key of the calling thread's launches (0: none).
inline uint32_t order_key() {
  const DebugOptions& o = debug_options();
  return (o.flags & kDebugPermute) ? ((o.seed * 2654435761u) | 1u) : 0u;
}
inline void prof_begin(int id, hipStream_t s) {
  const ProfileHook& h = profile_hook();
  if (h.kernel == id && h.start) (void)hipEventRecord(h.start, s);
}
inline void prof_end(int id, hipStream_t s) {
  const ProfileHook& h = profile_hook();
  if (h.kernel == id && h.stop) (void)hipEventRecord(h.stop, s);
}
// Column parts of a grouped GEMM that writes FP32 per-pair rows (rows x cols)
// for a fixed-order slot sum that reads them right after: the sum runs after
// each part's launch, and a part's slice (at most kYPartBytes, rewritten in
// place by the next part) stays in the 256 MB last-level cache between its
// write and its read instead of mixing the whole buffer's writes into the
// weight stream.  Each part is a launch of its own with its own tail, so parts
// keep at least min_items workgroups (cw: columns per workgroup item; max_tiles
// bounds the M-tiles).  Returns the part count (1: one launch).
constexpr size_t kYPartBytes = size_t(72) << 20;
inline int column_parts(size_t rows, int cols, int cw, int max_tiles, int min_items) {
  const int nblk = cols / cw;
  int parts = 1;
  for (int q = 1; q <= nblk; ++q) {
    if (nblk % q) continue;
    if (static_cast<int64_t>(nblk / q) * max_tiles < min_items) break;
    parts = q;
    if (rows * static_cast<size_t>(cols / q) * sizeof(float) <= kYPartBytes) break;
  }
  return parts;
}

enum KernelId { kRoute = 1, kDecGateUp = 2, kDecDown = 3, kGroup = 4, kQuant = 5,
                kGemmGateUp = 6, kGemmDown = 7, kCombine = 8, kBwdGateUp = 9, kBwdDown = 10,
                kBwdInput = 11, kBwdWDown = 12, kBwdWGateUp = 13, kDecFused = 14,
                kBwdRequant = 15,
                kKernelCount = 16 };

// Library-owned device scratch (scratch.hip): kStaticScratchBytes per GPU for
// the entry points that allocate nothing.  static_scratch(dev) gives its device
// address on device `dev`, which must be the current device; the address is
// taken with hipGetSymbolAddress on the first call for that device.
constexpr size_t kStaticScratchBytes = size_t(4) << 20;
constexpr int kMaxDevices = 64;
hipError_t static_scratch(int dev, void** ptr);

// Byte layout of the decode workspace.
// flags: one 64-bit ready flag per workgroup of the single-launch decode.
constexpr int kMaxDecodeGrid = 4096;
struct DecodeWs {
  size_t plan_u, plan_e, plan_off, plan_pr, idx, w, hw, flags, total;
};
DecodeWs decode_ws_layout(int T, int H, int I, int E, int k);

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* idx, float* w,
                             hipStream_t s);

hipError_t launch_decode(const uint16_t* x, const float* logits, const uint16_t* wgu,
                         const uint16_t* wd, int T, int H, int I, int E, int k, uint16_t* out,
                         int32_t* idx, float* w, void* ws, hipStream_t s, int num_cus);

// Byte layout of the batched workspace.  bm = rows per M-tile (64, or
// kLargeBM when the large-group GEMMs run).
struct BatchedWs {
  size_t counts, offsets, perm, row_of, tiles, n_tiles, y, partial, sct, total;
  int max_tiles, bm;
};
BatchedWs batched_ws_layout(int T, int H, int I, int E, int k, int dtype);

// Large-group GEMMs (gemm_large.hip): chosen when the routed rows per expert
// average at least kLargeBM, i.e. when the projections are MFMA-bound.
// Tail items may be split along K into at most kLargeMaxSlices FP32 partial
// tiles of 256 x 256 (the `partial` workspace region).
constexpr int kLargeBM = 256;
constexpr int kLargeMaxSlices = 256;
bool use_large_tiles(int T, int H, int I, int E, int k, int dtype);
hipError_t launch_gate_up_large_bf16(const uint16_t* x, const uint16_t* wgu, const int* perm,
                                     const int2* tiles, const int* n_tiles, const int* counts,
                                     const int* offsets, int H, int I, int k, uint16_t* h,
                                     float* partial, int max_tiles, int ncu, hipStream_t s,
                                     float* gu);   // gu: also keep the FP32 pre-activations
hipError_t launch_down_large_bf16(const uint16_t* h, const uint16_t* wd, const int* perm,
                                  const int2* tiles, const int* n_tiles, const int* counts,
                                  const int* offsets, const float* w, int H, int I, int k,
                                  float* y, uint16_t* out, float* partial, int max_tiles, int ncu,
                                  hipStream_t s);
// The MXFP8 launchers first transpose the weights' and the activations' scale
// dwords into sct (mx_scales_t_bytes(T*k, H, I, E) bytes of workspace).
size_t mx_scales_t_bytes(int P, int H, int I, int E);
hipError_t launch_gate_up_large_mx(const uint8_t* x, const uint8_t* xs, const uint8_t* wgu,
                                   const uint8_t* wgus, const int* perm, const int2* tiles,
                                   const int* n_tiles, const int* counts, const int* offsets, int H,
                                   int I, int k, uint8_t* hq, uint8_t* hs, float* partial,
                                   int max_tiles, int ncu, hipStream_t s, int T, int E,
                                   uint32_t* sct);
hipError_t launch_down_large_mx(const uint8_t* hq, const uint8_t* hs, const uint8_t* wd,
                                const uint8_t* wds, const int* perm, const int2* tiles,
                                const int* n_tiles, const int* counts, const int* offsets,
                                const float* w, int H, int I, int k, float* y, uint16_t* out,
                                float* partial, int max_tiles, int ncu, hipStream_t s, int T,
                                int E, uint32_t* sct);
// Weight gradients of the backward pass for large groups (>= 256 routed rows
// per expert): koff [E+1] ints, and transposed operands of wgrad_large_cols(P, E)
// columns each - xT, doutT [H][cols], dguT [2I][cols], waT [I][cols].
size_t wgrad_large_cols(int P, int E);
// dh[r][i] = sum_h W_down[e][h][i] dout[perm[r] / k][h] for each grouped row r
// (256-row M-tiles) on the large-group GEMM; wd = W_down [E][H][I] as stored
// (the loader transposes it).
hipError_t launch_dh_large(const uint16_t* dout, const uint16_t* wd, const int* perm,
                           const int2* tiles, const int* n_tiles, const int* counts,
                           const int* offsets, int H, int I, int k, float* dh, float* partial,
                           int max_tiles, int ncu, hipStream_t s);
// Data gradient of a projection on the large-group GEMM: for each grouped row r
// (256-row M-tiles), D[r][n] = sum_c act[r][c] w_in[e][c][n], c < K, n < H
// (w_in [E][K][H] as stored: W_gate_up with K = 2I); k = 1 writes
// out[perm[r]] = bf16(D), k > 1 writes y[r] = D (FP32).
hipError_t launch_dgrad_large(const uint16_t* act, const uint16_t* w_in, const int* perm,
                              const int2* tiles, const int* n_tiles, const int* counts,
                              const int* offsets, int H, int K, int k, float* y, uint16_t* out,
                              float* partial, int max_tiles, int ncu, hipStream_t s);
hipError_t launch_wgrad_large(const uint16_t* x, const uint16_t* dout, const uint16_t* dgu,
                              const uint16_t* wa, const int* perm, const int* counts,
                              const int* offsets, int P, int H, int I, int E, int k, int* koff,
                              uint16_t* xT, uint16_t* doutT, uint16_t* dguT, uint16_t* waT,
                              uint16_t* dwgu, uint16_t* dwd, int ncu, hipStream_t s);
hipError_t large_set_attributes();

// Stable expert grouping of the T*k routed pairs into M-tiles of BM rows
// (batched.hip); used by the forward and the backward.
hipError_t launch_group_experts(const int32_t* idx, int P, int E, int BM, int* counts, int* offsets,
                                int2* tiles, int* n_tiles, int* perm, int* row_of, hipStream_t s);

// Byte layout of the backward workspace (backward.hip).
struct BackwardWs {
  size_t counts, offsets, tiles, n_tiles, perm, row_of, gu, dgu, wa, dwp, dxs, total;
  size_t koff, xT, doutT, dguT, waT;   // large groups: the weight gradients' operands
  size_t tiles256, n_tiles256, partial;         // large groups: dx on the large-group GEMM
  size_t dh;                                     // large groups: dh on the large-group GEMM
  int max_tiles, max_tiles256;
  bool large_w;                        // weight gradients on the large-group GEMM
  bool large_d;                        // dh and dx on the large-group GEMM
};
BackwardWs backward_ws_layout(int T, int H, int I, int E, int k);
// gu_saved: NULL (the pre-activations are recomputed) or [T*k, 2I] FP32, slot order
hipError_t launch_backward(const uint16_t* x, const uint16_t* wgu, const uint16_t* wd,
                           const int32_t* idx, const float* w, const uint16_t* dout,
                           const float* gu_saved, int T, int H, int I, int E, int k,
                           uint16_t* dx, uint16_t* dwgu, uint16_t* dwd, float* dtw,
                           float* dlogits, void* ws, hipStream_t s, int num_cus);

hipError_t launch_quant_mx(const uint16_t* src, int64_t rows, int K, uint8_t* codes,
                           uint8_t* scales, hipStream_t s);

// MXFP8 backward (backward.hip): workspace layout and launch.  kpt_max bounds the
// pair-axis operands' columns (routed pairs, each expert padded to 128).
struct MxBackwardWs {
  size_t n_tiles, counts, offsets, tiles, perm, row_of, koff, xq, xs, dq, ds, wdT, wdTs, wguT,
      wguTs, gu, dh, a, dgu, dguq, dgus, dwp, dxs, partial, aT, aTs, dyT, dyTs, xT, xTs, dguT,
      dguTs, n_tiles64, tiles64, sct, total;
  size_t kpt_max;
  int max_tiles, max_tiles64;
};
MxBackwardWs mx_backward_ws_layout(int T, int H, int I, int E, int k);
hipError_t launch_backward_mx(const uint16_t* x, const uint8_t* wgu, const uint8_t* wgus,
                              const uint8_t* wd, const uint8_t* wds, const int32_t* idx,
                              const float* w, const uint16_t* dout, int T, int H, int I, int E,
                              int k, uint16_t* dx, uint16_t* dwgu, uint16_t* dwd, float* dtw,
                              float* dlogits, void* ws, hipStream_t s, int num_cus);
// The large-tile MXFP8 GEMM's backward products (gemm_large.hip).
hipError_t launch_gate_up_raw_large_mx(const uint8_t* xq, const uint8_t* xs, const uint8_t* wgu,
                                       const uint8_t* wgus, const int* perm, const int2* tiles,
                                       const int* n_tiles, const int* counts, const int* offsets,
                                       int H, int I, int k, float* gu, float* partial,
                                       int max_tiles, int ncu, hipStream_t s, int T, int E,
                                       uint32_t* sct);
hipError_t launch_dh_large_mx(const uint8_t* dq, const uint8_t* ds, const uint8_t* wdT,
                              const uint8_t* wdTs, const int* perm, const int2* tiles,
                              const int* n_tiles, const int* counts, const int* offsets, int H,
                              int I, int k, float* dh, float* partial, int max_tiles, int ncu,
                              hipStream_t s, int T, int E, uint32_t* sct);
hipError_t launch_dgrad_large_mx(const uint8_t* aq, const uint8_t* as, const uint8_t* wT,
                                 const uint8_t* wTs, const int* perm, const int2* tiles,
                                 const int* n_tiles, const int* counts, const int* offsets, int H,
                                 int K, int k, float* y, uint16_t* out, float* partial,
                                 int max_tiles, int ncu, hipStream_t s, int T, int E,
                                 uint32_t* sct);
hipError_t launch_wgrad_large_mx(const uint8_t* aT, const uint8_t* aTs, const uint8_t* dyT,
                                 const uint8_t* dyTs, const uint8_t* xT, const uint8_t* xTs,
                                 const uint8_t* dguT, const uint8_t* dguTs, const int* koff,
                                 int H, int I, int E, uint16_t* dwgu, uint16_t* dwd, bool small,
                                 int ncu, hipStream_t s);
hipError_t launch_koff_mx(const int* counts, int E, int* koff, hipStream_t s);

// gu: NULL, or (BF16, small groups only) [T*k, 2I] FP32 pre-activations out, slot order
hipError_t launch_gate_up_batched(const void* x, const uint8_t* xs, const void* wgu,
                                  const uint8_t* wgus, const int32_t* idx, int T, int H, int I,
                                  int E, int k, int dtype, void* h, uint8_t* hs, void* ws,
                                  hipStream_t s, int num_cus, float* gu = nullptr);

// MXFP8 grouped rows x weights^T with FP32 per-row output (the batched down kernel
// on 64-row tiles): y[row][n] = sum_k act[row][k] wt[e][n][k] for the grouped rows
// of each expert, act [P][K] codes + scales [P][K/32], wt [E][N][K] + [E][N][K/32].
hipError_t launch_mx_rows_down(const uint8_t* act, const uint8_t* acts, const uint8_t* wt,
                               const uint8_t* wts, const int* perm, const int2* tiles,
                               const int* n_tiles, int max_tiles, const int* counts,
                               const int* offsets, int N, int K, int k, float* y, hipStream_t s,
                               int num_cus);
// The same with activation rows gathered by token (perm / k): y[row][n] = sum_k
// act[perm[row] / k][k] wt[e][n][k], act [T][K].
hipError_t launch_mx_rows_gather(const uint8_t* act, const uint8_t* acts, const uint8_t* wt,
                                 const uint8_t* wts, const int* perm, const int2* tiles,
                                 const int* n_tiles, int max_tiles, const int* counts,
                                 const int* offsets, int K, int N, int k, float* y, hipStream_t s,
                                 int num_cus);
// MXFP8 gate_up product of grouped rows (x gathered by token), FP32 g and u per grouped
// row into gu [P][2I] (the backward's pre-activations), on 64-row tiles.
hipError_t launch_mx_gate_up_raw_rows(const uint8_t* x, const uint8_t* xs, const uint8_t* wgu,
                                     const uint8_t* wgus, const int* perm, const int2* tiles,
                                     const int* n_tiles, int max_tiles, const int* counts,
                                     const int* offsets, int H, int I, int k, float* gu,
                                     hipStream_t s, int num_cus);
hipError_t launch_down_batched(const void* h, const uint8_t* hs, const void* wd,
                               const uint8_t* wds, const int32_t* idx, const float* w, int T,
                               int H, int I, int E, int k, int dtype, uint16_t* out, void* ws,
                               hipStream_t s, int num_cus);

}  // namespace moe
