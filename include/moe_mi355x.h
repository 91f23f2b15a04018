/*
 * moe_mi355x.h -- C ABI of the routed Mixture-of-Experts FFN layer for one
 * AMD Instinct MI355X (gfx950).
 *
 * The layer (warp-decode article on picklee.vercel.app, sections "Background"
 * and "Key points"; Mixture-of-Kittens summary on asapai.co.kr, sections
 * "What is 2.37x measured against" and "Determinism on par with
 * performance"): every token is routed to k experts chosen from its router
 * logits; each routed expert applies its gate/up projection, the SwiGLU
 * activation and its down projection; the routed experts' outputs are summed
 * with the routing weights into the token's output, accumulating in FP32 in
 * a fixed order so that the same inputs always give the same bytes.
 *
 * Conventions shared by every call
 *   - Shapes: T tokens, H hidden size, I expert intermediate size, E experts,
 *     k experts per token.  Row-major; the reduction dimension of every weight
 *     matrix is contiguous.
 *   - BF16 values are passed as uint16_t bit patterns.  FP8 E4M3 codes and
 *     E8M0 scale codes are uint8_t.  MX blocks are 32 consecutive elements
 *     along the reduction dimension.
 *   - Every pointer argument is a device pointer unless stated otherwise; the
 *     caller owns all memory.  The library allocates nothing and keeps no
 *     state between calls except a cached device-property query.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Every call only enqueues work on `stream` and returns; no call waits
 *     for the device.
 *   - Errors: arguments are validated on the host before anything is
 *     enqueued.  A failure returns a negative moe_status and leaves a message
 *     for moe_last_error() (per calling thread); nothing was enqueued.
 *     A launch failure reported by the HIP runtime returns MOE_ERR_HIP.
 *   - Device contents are not validated: expert ids must lie in [0, E) and
 *     logits must be finite, otherwise results are undefined.
 *   - Determinism: identical inputs, shapes and device give byte-identical
 *     outputs.  No kernel accumulates floating point values with atomics.
 *   - All device pointers must be 16-byte aligned.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = -1,        /* a required pointer is NULL                    */
  MOE_ERR_SHAPE = -2,       /* a size is out of range or not a multiple      */
  MOE_ERR_ALIGN = -3,       /* a device pointer is not 16-byte aligned       */
  MOE_ERR_WORKSPACE = -4,   /* workspace NULL or smaller than required       */
  MOE_ERR_UNSUPPORTED = -5, /* a valid request this library does not serve   */
  MOE_ERR_HIP = -6          /* the HIP runtime reported an error             */
} moe_status;

typedef enum {
  MOE_BF16 = 0,   /* BF16 activations and weights                         */
  MOE_MXFP8 = 1,  /* E4M3 codes with one E8M0 scale per 32 along K          */
  /* not element types: they make the enum span every int, so that an unknown
   * value passed by a caller is a valid value of the type that the library
   * rejects (MOE_ERR_SHAPE) rather than undefined behaviour in C++ */
  MOE_DTYPE_RANGE_MIN_ = -0x7FFFFFFF - 1,
  MOE_DTYPE_RANGE_MAX_ = 0x7FFFFFFF
} moe_dtype;

/*
 * moe_route_topk -- top-k expert routing (warp-decode article, "Background":
 * expert routing picks each token's experts; "Key points": the routed
 * experts).  The pages name the step but give no gate function, selection
 * rule or tie-break; this library reads them as: select on the FP32 logits,
 * order by (logit descending, index ascending), and weight the k selected
 * experts by softmax renormalised over them.
 *
 *   logits   [T, E] float32, finite
 *   topk_idx [T, k] int32 out: slot j holds the j-th expert in the order
 *            (logit descending, expert index ascending); +0 and -0 tie, so the
 *            lower index wins
 *   topk_w   [T, k] float32 out: exp(l_j - l_0) / sum_i exp(l_i - l_0) over the
 *            k selected logits (softmax over all E then renormalised over k)
 * Limits: T >= 0 (T = 0 enqueues nothing), 1 <= k <= min(E, 32), E <= 1024.
 * Index selection compares FP32 values exactly, so it is bit-exact.
 */
int moe_route_topk(const float* logits, int T, int E, int k,
                   int32_t* topk_idx, float* topk_w, void* stream);

/*
 * moe_decode_forward -- the whole layer for a small decode batch
 * (warp-decode article, "Key points": two kernels, gate_up and down, each
 * output-centric, routed experts' contributions summed directly into FP32
 * accumulators, no per-expert output buffer and no activation-gather buffer;
 * Mixture-of-Kittens summary, "One kernel swallowed the layer's comm+compute":
 * no kernel-launch boundaries inside the layer).  At T <= 16 routing runs
 * inside gate_up (two launches); at larger T routing, gate_up and down are three
 * launches.  A single-launch form (routing, gate_up, a bounded device-wide wait
 * on per-workgroup ready flags, down) is available through
 * moe_set_debug_options(MOE_DEBUG_DECODE_FUSED) for T <= 16 and I/64 a power of
 * two times 3 or 4; it is not the default because it measured no faster.
 *
 *   x           [T, H] BF16
 *   logits      [T, E] float32
 *   w_gate_up   [E, 2I, H] BF16: rows [0, I) gate, rows [I, 2I) up
 *   w_down      [E, H, I] BF16
 *   out         [T, H] BF16 out: FP32 sum, rounded to nearest even once
 *   topk_idx    [T, k] int32 out, may be NULL (then kept in the workspace)
 *   topk_w      [T, k] float32 out, may be NULL
 *   workspace   >= moe_decode_workspace_bytes(T, H, I, E, k) bytes of device
 *               memory, contents ignored on entry and overwritten
 * Limits: 1 <= T <= 64 and I <= 2048 (otherwise MOE_ERR_UNSUPPORTED: use the
 * batched calls), H and I multiples of 256, 1 <= k <= min(E, 32), E <= 1024,
 * 2*I*H < 2^31 (MOE_ERR_SHAPE otherwise).
 * Only the weights of experts that some token routes to are read.
 */
int moe_decode_forward(const uint16_t* x, const float* logits,
                       const uint16_t* w_gate_up, const uint16_t* w_down,
                       int T, int H, int I, int E, int k,
                       uint16_t* out, int32_t* topk_idx, float* topk_w,
                       void* workspace, size_t workspace_bytes, void* stream);

size_t moe_decode_workspace_bytes(int T, int H, int I, int E, int k);

/*
 * moe_decode_forward_noalloc -- moe_decode_forward for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * and harnesses that forbid hipMalloc.  Same arguments, results and bytes as
 * moe_decode_forward, without the workspace: the kernels use a scratch array
 * the library owns, MOE_STATIC_SCRATCH_BYTES on every GPU it runs on (held
 * until the process ends).  This call allocates nothing.
 *
 * Limit: moe_decode_workspace_bytes(T, H, I, E, k) <= MOE_STATIC_SCRATCH_BYTES
 * (about T*k*I <= 2^21; MOE_ERR_UNSUPPORTED otherwise), besides the limits of
 * moe_decode_forward.
 * All calls on one GPU share its scratch array, which keeps the last call's
 * contents (every byte a call reads there, it has written first): calls that
 * can overlap on one GPU (on different streams, or from different threads)
 * race and must be ordered by the caller.
 */
#define MOE_STATIC_SCRATCH_BYTES (4u << 20)
int moe_decode_forward_noalloc(const uint16_t* x, const float* logits,
                               const uint16_t* w_gate_up, const uint16_t* w_down,
                               int T, int H, int I, int E, int k,
                               uint16_t* out, int32_t* topk_idx, float* topk_w, void* stream);

/*
 * moe_quantize_mxfp8 -- MX block quantization of a BF16 matrix along its
 * last dimension (the "MXFP8" forward of the Mixture-of-Kittens summary,
 * "What is 2.37x measured against"; block rule of OCP Microscaling v1.0).
 *
 *   src    [rows, K] BF16
 *   codes  [rows, K] uint8 E4M3 out
 *   scales [rows, K/32] uint8 E8M0 out
 * Per block of 32: s = floor(log2(max |v|)) - 8 clamped to [-127, 127]
 * (an all-zero block takes s = -127); code = E4M3 of v / 2^s rounded to
 * nearest even and saturated to +-448, sign bit copied from v.
 * Limits: rows >= 0, K a positive multiple of 32.
 */
int moe_quantize_mxfp8(const uint16_t* src, int64_t rows, int K,
                       uint8_t* codes, uint8_t* scales, void* stream);

/*
 * moe_gate_up_3d_batched -- gate/up projection and SwiGLU for every routed
 * (token, slot) pair of a large batch, as one grouped GEMM over experts
 * (warp-decode article, "Key points": kernel moe_gate_up_3d_batched;
 * Mixture-of-Kittens summary: expert compute of the MoE layer forward at
 * 2,048 tokens per GPU, BF16 and MXFP8).
 *
 *   x          [T, H]: BF16 (dtype MOE_BF16) or E4M3 codes (MOE_MXFP8)
 *   x_scales   [T, H/32] E8M0 (MOE_MXFP8 only, else ignored)
 *   w_gate_up  [E, 2I, H]: BF16 or E4M3 codes; rows [0, I) gate, [I, 2I) up
 *   w_gate_up_scales [E, 2I, H/32] E8M0 (MOE_MXFP8 only)
 *   topk_idx   [T, k] int32 from moe_route_topk
 *   h          [T*k, I] out, rows in expert-grouped order (row r holds the
 *              pair perm[r]; experts ascending, tokens ascending within an
 *              expert): BF16 (MOE_BF16) or E4M3 codes (MOE_MXFP8), the
 *              activation silu(g) * u computed in FP32 and rounded once
 *   h_scales   [T*k, I/32] E8M0 out (MOE_MXFP8 only)
 *   workspace  >= moe_workspace_bytes(T, H, I, E, k, dtype) bytes; this call
 *              writes the expert grouping into it, and moe_down_3d_batched
 *              must be given the same workspace and topk_idx, later on the
 *              same stream (MXFP8 with >= 256 routed pairs per expert on
 *              average: both calls also keep transposed copies of the weights'
 *              and the activations' scale bytes there)
 * Limits: T >= 1, H and I multiples of 256, 1 <= k <= min(E, 32), E <= 1024;
 * T*H, T*k*H, T*k*I and 2*I*H each below 2^31 (the kernels' 32-bit element
 * offsets).  MOE_ERR_SHAPE otherwise.
 */
int moe_gate_up_3d_batched(const void* x, const uint8_t* x_scales,
                           const void* w_gate_up, const uint8_t* w_gate_up_scales,
                           const int32_t* topk_idx,
                           int T, int H, int I, int E, int k, moe_dtype dtype,
                           void* h, uint8_t* h_scales,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_down_3d_batched -- down projection of every routed pair and the
 * routing-weighted combine into each token's output (warp-decode article,
 * "Key points": kernel moe_down_3d_batched; Mixture-of-Kittens summary,
 * "Determinism on par with performance": a fixed floating-point order).
 *
 *   h, h_scales      as written by moe_gate_up_3d_batched
 *   w_down           [E, H, I]: BF16 or E4M3 codes
 *   w_down_scales    [E, H, I/32] E8M0 (MOE_MXFP8 only)
 *   topk_idx, topk_w [T, k] from moe_route_topk
 *   out              [T, H] BF16 out: out[t] = sum over slots j = 0..k-1, in that
 *                    order, of topk_w[t, j] * y[t, j], in FP32, rounded once
 *   workspace        the workspace given to moe_gate_up_3d_batched
 * Limits as for moe_gate_up_3d_batched.
 */
int moe_down_3d_batched(const void* h, const uint8_t* h_scales,
                        const void* w_down, const uint8_t* w_down_scales,
                        const int32_t* topk_idx, const float* topk_w,
                        int T, int H, int I, int E, int k, moe_dtype dtype,
                        uint16_t* out,
                        void* workspace, size_t workspace_bytes, void* stream);

size_t moe_workspace_bytes(int T, int H, int I, int E, int k, moe_dtype dtype);

/*
 * moe_gate_up_3d_batched_train -- moe_gate_up_3d_batched (BF16) that also keeps
 * what the backward pass needs: the FP32 gate/up pre-activations of every
 * routed pair (Mixture-of-Kittens summary, "Where pull was faster than push":
 * the backward reuses forward activations rather than recomputing them).
 *
 *   x, w_gate_up, topk_idx, h, workspace   as for moe_gate_up_3d_batched with
 *              dtype MOE_BF16
 *   gu         [T*k, 2I] FP32 out, row t*k + j (slot order): [g; u] of pair
 *              (t, j), g = W_gate[e] x[t], u = W_up[e] x[t] summed in FP32
 *              (the values h was computed from); pass it to moe_backward_batched
 * moe_down_3d_batched follows with the same workspace, as after
 * moe_gate_up_3d_batched.  Limits as for moe_gate_up_3d_batched, and
 * T*k*2I < 2^31 (MOE_ERR_SHAPE otherwise).
 */
int moe_gate_up_3d_batched_train(const uint16_t* x, const uint16_t* w_gate_up,
                                 const int32_t* topk_idx, int T, int H, int I, int E, int k,
                                 uint16_t* h, float* gu,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_backward_batched -- backward pass of the whole layer for a large batch,
 * BF16 (Mixture-of-Kittens summary, "What is 2.37x measured against": the
 * MoE layer's backward pass, measured beside its forward pass at 2,048 tokens
 * per GPU).  The gradient is that of the exact layer for the scalar
 * sum(dout * out), with the top-k selection held fixed: for each routed pair
 * (t, j) -> e, with g, u = gate/up pre-activations of x[t], a = silu(g) * u,
 * y = W_down[e] a and w = topk_w[t, j],
 *   d_topk_w[t, j] = dout[t] . y
 *   dg = w (W_down[e]^T dout[t]) * u * silu'(g),  du = w (W_down[e]^T dout[t]) * silu(g)
 *   dx[t]          = sum over j of W_gate[e]^T dg + W_up[e]^T du
 *   dw_down[e]     = sum over e's pairs of (w dout[t]) a^T
 *   dw_gate_up[e]  = sum over e's pairs of [dg; du] x[t]^T
 *   dlogits[t, m]  = w_m (d_topk_w[t, m's slot] - sum_j w_j d_topk_w[t, j]) for
 *                    the k selected experts m (softmax renormalised over them),
 *                    0 for every other expert.
 * The gate/up pre-activations come from gu_saved (as written by
 * moe_gate_up_3d_batched_train) or, when it is NULL, are recomputed from x.
 * All sums accumulate in FP32 in a fixed order; dx and both weight gradients
 * are rounded once to BF16.
 *
 *   x [T, H], w_gate_up [E, 2I, H], w_down [E, H, I]  BF16, as for the forward
 *   topk_idx, topk_w [T, k]   from moe_route_topk
 *   dout       [T, H] BF16    gradient of the layer output
 *   gu_saved   [T*k, 2I] FP32 from moe_gate_up_3d_batched_train, or NULL
 *   dx         [T, H] BF16 out
 *   dw_gate_up [E, 2I, H] BF16 out (zero for experts no token routes to)
 *   dw_down    [E, H, I] BF16 out (likewise)
 *   d_topk_w   [T, k] FP32 out
 *   dlogits    [T, E] FP32 out
 *   workspace  >= moe_backward_workspace_bytes(T, H, I, E, k) bytes.  With 256 or
 *              more routed rows per expert on average (the expert-parallel
 *              share of a large batch) it also holds K-contiguous copies of x,
 *              dout and the intermediate gradients, an FP32 copy of W_down^T
 *              dout and a 64 MiB K-split buffer (about 2*T*k*(2H + 3I) +
 *              4*T*k*I bytes + 64 MiB), which the large-tile GEMMs of that case
 *              read (the weights are read in place).
 * Limits: T >= 1, H and I multiples of 256, 1 <= k <= min(E, 32), E <= 1024.
 */
int moe_backward_batched(const uint16_t* x, const uint16_t* w_gate_up, const uint16_t* w_down,
                         const int32_t* topk_idx, const float* topk_w, const uint16_t* dout,
                         const float* gu_saved, int T, int H, int I, int E, int k,
                         uint16_t* dx, uint16_t* dw_gate_up, uint16_t* dw_down,
                         float* d_topk_w, float* dlogits,
                         void* workspace, size_t workspace_bytes, void* stream);

size_t moe_backward_workspace_bytes(int T, int H, int I, int E, int k);

/*
 * moe_backward_batched_mxfp8 -- backward pass of the MXFP8 layer
 * (Mixture-of-Kittens summary, "What is 2.37x measured against": the MoE
 * layer's backward in MXFP8, beside the BF16 one).  The gradients are those of
 * moe_backward_batched for the MXFP8 layer (pre-activations g, u = W_gate_up x
 * from the E4M3 weights and x MX-quantized along H), with every matrix product
 * taking both operands MX-quantized (blocks of 32, the moe_quantize_mxfp8 rule)
 * along its own reduction axis - a reading of the page, which gives the
 * backward's speed only:
 *   dh = W_down^T dout          dout and W_down's columns along H
 *   dx = W_gate_up^T [dg; du]   [dg; du] and W_gate_up's columns along 2I
 *   dw_down, dw_gate_up         both operands along the expert's routed pairs
 *                               (token order, blocks of 32 from its first pair)
 * from the decoded weights, the BF16 x and dout, and the FP32 a = silu(g) u and
 * [dg; du]; d_topk_w = a . (W_down^T dout).  Sums accumulate in FP32 in a fixed
 * order; dx and both weight gradients are rounded once to BF16.
 *
 *   x, dout [T, H] BF16; w_gate_up [E, 2I, H] and w_down [E, H, I] E4M3 codes
 *   with E8M0 scales [E, 2I, H/32] and [E, H, I/32], as for the MXFP8 forward;
 *   topk_idx, topk_w, dx, dw_gate_up, dw_down, d_topk_w, dlogits as for
 *   moe_backward_batched (the weight gradients BF16)
 *   workspace  >= moe_backward_mxfp8_workspace_bytes(T, H, I, E, k): the
 *              grouping, x and dout encoded along H, both weights re-encoded
 *              along their output axis (transposed copies, ~1.03 x the weight
 *              bytes), FP32 pre-activations, dh, a and [dg; du] per routed pair,
 *              the pair-axis operands, a 64 MiB K-split buffer and (>= 256
 *              routed pairs per expert on average, or k = 1) transposed copies
 *              of the projections' scale bytes
 * Limits: as for moe_backward_batched, and max(H, 2I) * (T*k + 128*E) < 2^31.
 */
int moe_backward_batched_mxfp8(const uint16_t* x, const uint8_t* w_gate_up,
                               const uint8_t* w_gate_up_scales, const uint8_t* w_down,
                               const uint8_t* w_down_scales, const int32_t* topk_idx,
                               const float* topk_w, const uint16_t* dout,
                               int T, int H, int I, int E, int k,
                               uint16_t* dx, uint16_t* dw_gate_up, uint16_t* dw_down,
                               float* d_topk_w, float* dlogits,
                               void* workspace, size_t workspace_bytes, void* stream);

size_t moe_backward_mxfp8_workspace_bytes(int T, int H, int I, int E, int k);

/*
 * Kernel timing hook for benchmarks and profilers (not on any page).
 * moe_profile_kernel(kernel, start, stop): from now on, the calling thread's
 * launches of `kernel` are bracketed by hipEventRecord(start) and
 * hipEventRecord(stop) on the launch stream; `start`/`stop` are hipEvent_t
 * passed as void*, created by the caller.  kernel = MOE_KERNEL_NONE (or NULL
 * events) switches the hook off.  Returns MOE_OK or MOE_ERR_SHAPE for an
 * unknown kernel id.
 */
typedef enum {
  MOE_KERNEL_NONE = 0,
  MOE_KERNEL_ROUTE = 1,          /* moe_route_topk, and routing+plan in decode */
  MOE_KERNEL_DECODE_GATE_UP = 2,
  MOE_KERNEL_DECODE_DOWN = 3,
  MOE_KERNEL_GROUP = 4,          /* expert grouping of the batched path        */
  MOE_KERNEL_QUANT = 5,          /* moe_quantize_mxfp8                         */
  MOE_KERNEL_GEMM_GATE_UP = 6,
  MOE_KERNEL_GEMM_DOWN = 7,      /* batched down projection and the weighted combine
                                    (which runs interleaved with it in column parts) */
  MOE_KERNEL_COMBINE = 8,        /* reserved: the combine is timed within GEMM_DOWN */
  MOE_KERNEL_BWD_GATE_UP = 9,    /* backward: recomputed gate/up pre-activations */
  MOE_KERNEL_BWD_DOWN = 10,      /* backward: W_down^T dout and the SwiGLU step  */
  MOE_KERNEL_BWD_INPUT = 11,     /* backward: dx (and the slot sum)              */
  MOE_KERNEL_BWD_WDOWN = 12,     /* backward: dw_down                            */
  MOE_KERNEL_BWD_WGATE_UP = 13,  /* backward: dw_gate_up                         */
  MOE_KERNEL_DECODE_FUSED = 14,  /* single-launch decode (T <= 16): the whole layer */
  MOE_KERNEL_BWD_REQUANT = 15,   /* MXFP8 backward: x, dout and both weights encoded
                                    along the backward's reduction axes           */
  MOE_KERNEL_COUNT = 16
} moe_kernel_id;

int moe_profile_kernel(int kernel, void* start_event, void* stop_event);

/*
 * Test and debugging options (not on any page), for the calling thread's later
 * calls until changed:
 *   MOE_DEBUG_PERMUTE_ORDER  every grouped and decode kernel visits its work
 *                            items in an order permuted by `seed` (a different
 *                            workgroup -> item assignment); results must not change
 *   MOE_DEBUG_DECODE_FUSED   moe_decode_forward at T <= 16 runs as one launch
 *                            (routing, gate_up, a device-wide wait, down) instead
 *                            of two; not on a capturing stream (its wait keys on a
 *                            per-launch value that a graph would replay): there the
 *                            two launches run
 * flags = 0 restores the defaults.  Returns MOE_OK, or MOE_ERR_SHAPE for
 * unknown bits.
 */
#define MOE_DEBUG_PERMUTE_ORDER 1u
#define MOE_DEBUG_DECODE_FUSED 2u
int moe_set_debug_options(unsigned flags, uint32_t seed);

/* Static text for a moe_status value. */
const char* moe_status_string(int status);

/* Detail of the calling thread's last failure ("" if none).  Host memory owned
 * by the library, valid until the thread's next call. */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
