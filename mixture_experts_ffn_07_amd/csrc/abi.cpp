// C ABI of the library: host-side validation, workspace sizing and dispatch.
// Every check runs before any HIP call, so the checks work on a host without
// a GPU.  The HIP runtime is first touched by the first valid launch.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/moe_mi355x.h"
#include "internal.h"

namespace moe {
hipError_t decode_set_attributes();
hipError_t batched_set_attributes();
hipError_t backward_set_attributes();

ProfileHook& profile_hook() {
  thread_local ProfileHook hook;
  return hook;
}

DebugOptions& debug_options() {
  thread_local DebugOptions opts;
  return opts;
}
}  // namespace moe

static_assert(MOE_STATIC_SCRATCH_BYTES == moe::kStaticScratchBytes,
              "the header's scratch size must match the array's");
static_assert(MOE_DEBUG_PERMUTE_ORDER == moe::kDebugPermute &&
              MOE_DEBUG_DECODE_FUSED == moe::kDebugDecodeFused, "debug option bits");
static_assert(MOE_KERNEL_COUNT == moe::kKernelCount, "kernel ids");

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return MOE_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Device properties and one-time kernel attributes, per device.
struct DeviceInfo {
  int num_cus = 0;
  bool ready = false;
  void* scratch = nullptr;   // this device's copy of the library-owned scratch array
};
std::mutex g_mu;
DeviceInfo g_dev[moe::kMaxDevices];

int device_info(int* num_cus, void** scratch = nullptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= moe::kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "device ordinal %d", dev);
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceInfo& d = g_dev[dev];
  if (!d.ready) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    if (std::string(prop.gcnArchName).rfind("gfx950", 0) != 0)
      return fail(MOE_ERR_UNSUPPORTED, "device %d is %s; this library is built for gfx950", dev,
                  prop.gcnArchName);
    e = moe::decode_set_attributes();
    if (e == hipSuccess) e = moe::batched_set_attributes();
    if (e == hipSuccess) e = moe::backward_set_attributes();
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "hipFuncSetAttribute: %s", hipGetErrorString(e));
    // the device address of this device's scratch array (the device is current)
    e = moe::static_scratch(dev, &d.scratch);
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "hipGetSymbolAddress: %s", hipGetErrorString(e));
    d.num_cus = prop.multiProcessorCount;
    d.ready = true;
  }
  *num_cus = d.num_cus;
  if (scratch) *scratch = d.scratch;
  return MOE_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

int check_common(int T, int H, int I, int E, int k, int hmul, int imul) {
  if (T < 0) return fail(MOE_ERR_SHAPE, "T=%d < 0", T);
  if (E < 1 || E > 1024) return fail(MOE_ERR_SHAPE, "E=%d outside [1, 1024]", E);
  if (k < 1 || k > E || k > 32) return fail(MOE_ERR_SHAPE, "k=%d outside [1, min(E=%d, 32)]", k, E);
  if (H <= 0 || H % hmul) return fail(MOE_ERR_SHAPE, "H=%d is not a positive multiple of %d", H, hmul);
  if (I <= 0 || I % imul) return fail(MOE_ERR_SHAPE, "I=%d is not a positive multiple of %d", I, imul);
  return MOE_OK;
}

// Element offsets the kernels form in 32-bit arithmetic: rows of x (T*H), of
// the routed-pair buffers h and y (T*k*I, T*k*H) and of one expert's weights
// (2I*H).  Each must stay below 2^31.
int check_offsets(int T, int H, int I, int k) {
  const long long lim = 1LL << 31;
  if (static_cast<long long>(T) * H >= lim) return fail(MOE_ERR_SHAPE, "T*H reaches 2^31");
  if (static_cast<long long>(T) * k * H >= lim) return fail(MOE_ERR_SHAPE, "T*k*H reaches 2^31");
  if (static_cast<long long>(T) * k * I >= lim) return fail(MOE_ERR_SHAPE, "T*k*I reaches 2^31");
  if (2LL * I * H >= lim) return fail(MOE_ERR_SHAPE, "2*I*H reaches 2^31");
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "null pointer";
    case MOE_ERR_SHAPE: return "invalid shape";
    case MOE_ERR_ALIGN: return "misaligned pointer";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_UNSUPPORTED: return "unsupported";
    case MOE_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

int moe_profile_kernel(int kernel, void* start_event, void* stop_event) {
  if (kernel < 0 || kernel >= moe::kKernelCount)
    return fail(MOE_ERR_SHAPE, "unknown kernel id %d", kernel);
  moe::ProfileHook& h = moe::profile_hook();
  h.kernel = (start_event && stop_event) ? kernel : 0;
  h.start = static_cast<hipEvent_t>(start_event);
  h.stop = static_cast<hipEvent_t>(stop_event);
  return ok();
}

int moe_set_debug_options(unsigned flags, uint32_t seed) {
  if (flags & ~(MOE_DEBUG_PERMUTE_ORDER | MOE_DEBUG_DECODE_FUSED))
    return fail(MOE_ERR_SHAPE, "unknown debug option bits 0x%x", flags);
  moe::DebugOptions& o = moe::debug_options();
  o.flags = flags;
  o.seed = seed;
  return ok();
}

int moe_route_topk(const float* logits, int T, int E, int k, int32_t* topk_idx, float* topk_w,
                   void* stream) {
  if (T < 0) return fail(MOE_ERR_SHAPE, "T=%d < 0", T);
  if (E < 1 || E > 1024) return fail(MOE_ERR_SHAPE, "E=%d outside [1, 1024]", E);
  if (k < 1 || k > E || k > 32) return fail(MOE_ERR_SHAPE, "k=%d outside [1, min(E=%d, 32)]", k, E);
  if (T == 0) return ok();
  if (!logits || !topk_idx || !topk_w) return fail(MOE_ERR_NULL, "logits, topk_idx and topk_w are required");
  int cus = 0;
  if (int st = device_info(&cus)) return st;
  return hip_status(moe::launch_route_topk(logits, T, E, k, topk_idx, topk_w,
                                           static_cast<hipStream_t>(stream)),
                    "moe_route_topk launch");
}

size_t moe_decode_workspace_bytes(int T, int H, int I, int E, int k) {
  if (T < 1 || T > 64 || H <= 0 || I <= 0 || E < 1 || k < 1) return 0;
  return moe::decode_ws_layout(T, H, I, E, k).total;
}

int moe_decode_forward(const uint16_t* x, const float* logits, const uint16_t* w_gate_up,
                       const uint16_t* w_down, int T, int H, int I, int E, int k, uint16_t* out,
                       int32_t* topk_idx, float* topk_w, void* workspace, size_t workspace_bytes,
                       void* stream) {
  if (int st = check_common(T, H, I, E, k, 256, 256)) return st;
  if (T == 0) return fail(MOE_ERR_SHAPE, "T=0: nothing to decode");
  if (T > 64) return fail(MOE_ERR_UNSUPPORTED, "T=%d > 64: use the batched calls", T);
  if (I > 2048) return fail(MOE_ERR_UNSUPPORTED, "I=%d > 2048: use the batched calls", I);
  if (int st = check_offsets(T, H, I, k)) return st;
  if (!x || !logits || !w_gate_up || !w_down || !out)
    return fail(MOE_ERR_NULL, "x, logits, w_gate_up, w_down and out are required");
  if (!workspace) return fail(MOE_ERR_WORKSPACE, "workspace is NULL");
  const size_t need = moe::decode_ws_layout(T, H, I, E, k).total;
  if (workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, need);
  if (!aligned16(x) || !aligned16(w_gate_up) || !aligned16(w_down) || !aligned16(out) ||
      !aligned16(workspace) || !aligned16(logits) || (topk_idx && !aligned16(topk_idx)) ||
      (topk_w && !aligned16(topk_w)))
    return fail(MOE_ERR_ALIGN, "device pointers must be 16-byte aligned");
  int cus = 0;
  if (int st = device_info(&cus)) return st;
  return hip_status(moe::launch_decode(x, logits, w_gate_up, w_down, T, H, I, E, k, out, topk_idx,
                                       topk_w, workspace, static_cast<hipStream_t>(stream), cus),
                    "moe_decode_forward launch");
}

int moe_decode_forward_noalloc(const uint16_t* x, const float* logits, const uint16_t* w_gate_up,
                               const uint16_t* w_down, int T, int H, int I, int E, int k,
                               uint16_t* out, int32_t* topk_idx, float* topk_w, void* stream) {
  if (int st = check_common(T, H, I, E, k, 256, 256)) return st;
  if (T == 0) return fail(MOE_ERR_SHAPE, "T=0: nothing to decode");
  if (T > 64) return fail(MOE_ERR_UNSUPPORTED, "T=%d > 64: use the batched calls", T);
  if (I > 2048) return fail(MOE_ERR_UNSUPPORTED, "I=%d > 2048: use the batched calls", I);
  if (int st = check_offsets(T, H, I, k)) return st;
  const size_t need = moe::decode_ws_layout(T, H, I, E, k).total;
  if (need > moe::kStaticScratchBytes)
    return fail(MOE_ERR_UNSUPPORTED,
                "workspace of %zu bytes exceeds the library's %zu-byte scratch (T*k*I too "
                "large): use moe_decode_forward with a caller workspace",
                need, moe::kStaticScratchBytes);
  if (!x || !logits || !w_gate_up || !w_down || !out)
    return fail(MOE_ERR_NULL, "x, logits, w_gate_up, w_down and out are required");
  if (!aligned16(x) || !aligned16(w_gate_up) || !aligned16(w_down) || !aligned16(out) ||
      !aligned16(logits) || (topk_idx && !aligned16(topk_idx)) || (topk_w && !aligned16(topk_w)))
    return fail(MOE_ERR_ALIGN, "device pointers must be 16-byte aligned");
  int cus = 0;
  void* ws = nullptr;
  if (int st = device_info(&cus, &ws)) return st;
  return hip_status(moe::launch_decode(x, logits, w_gate_up, w_down, T, H, I, E, k, out, topk_idx,
                                       topk_w, ws, static_cast<hipStream_t>(stream), cus),
                    "moe_decode_forward_noalloc launch");
}

size_t moe_workspace_bytes(int T, int H, int I, int E, int k, moe_dtype dtype) {
  if (T < 1 || H <= 0 || I <= 0 || E < 1 || k < 1 || (dtype != MOE_BF16 && dtype != MOE_MXFP8))
    return 0;
  return moe::batched_ws_layout(T, H, I, E, k, dtype).total;
}

int moe_quantize_mxfp8(const uint16_t* src, int64_t rows, int K, uint8_t* codes, uint8_t* scales,
                       void* stream) {
  if (rows < 0) return fail(MOE_ERR_SHAPE, "rows=%lld < 0", static_cast<long long>(rows));
  if (K <= 0 || K % 32) return fail(MOE_ERR_SHAPE, "K=%d is not a positive multiple of 32", K);
  if (rows == 0) return ok();
  if (!src || !codes || !scales) return fail(MOE_ERR_NULL, "src, codes and scales are required");
  if (!aligned16(src) || !aligned16(codes) || !aligned16(scales))
    return fail(MOE_ERR_ALIGN, "device pointers must be 16-byte aligned");
  int cus = 0;
  if (int st = device_info(&cus)) return st;
  return hip_status(moe::launch_quant_mx(src, rows, K, codes, scales,
                                         static_cast<hipStream_t>(stream)),
                    "moe_quantize_mxfp8 launch");
}

static int check_batched(int T, int H, int I, int E, int k, moe_dtype dtype, const void* ws,
                         size_t ws_bytes) {
  if (int st = check_common(T, H, I, E, k, 256, 256)) return st;
  if (T < 1) return fail(MOE_ERR_SHAPE, "T=%d < 1", T);
  if (dtype != MOE_BF16 && dtype != MOE_MXFP8) return fail(MOE_ERR_SHAPE, "dtype=%d", dtype);
  if (static_cast<long long>(T) * k > (1LL << 30)) return fail(MOE_ERR_SHAPE, "T*k too large");
  // the kernels form 32-bit element offsets into x, h, y and one expert's weights
  if (int st = check_offsets(T, H, I, k)) return st;
  if (!ws) return fail(MOE_ERR_WORKSPACE, "workspace is NULL");
  const size_t need = moe::batched_ws_layout(T, H, I, E, k, dtype).total;
  if (ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes < %zu required", ws_bytes, need);
  if (!aligned16(ws)) return fail(MOE_ERR_ALIGN, "workspace must be 16-byte aligned");
  return MOE_OK;
}

int moe_gate_up_3d_batched(const void* x, const uint8_t* x_scales, const void* w_gate_up,
                           const uint8_t* w_gate_up_scales, const int32_t* topk_idx, int T, int H,
                           int I, int E, int k, moe_dtype dtype, void* h, uint8_t* h_scales,
                           void* workspace, size_t workspace_bytes, void* stream) {
  if (int st = check_batched(T, H, I, E, k, dtype, workspace, workspace_bytes)) return st;
  if (!x || !w_gate_up || !topk_idx || !h)
    return fail(MOE_ERR_NULL, "x, w_gate_up, topk_idx and h are required");
  if (dtype == MOE_MXFP8 && (!x_scales || !w_gate_up_scales || !h_scales))
    return fail(MOE_ERR_NULL, "MXFP8 needs x_scales, w_gate_up_scales and h_scales");
  if (!aligned16(x) || !aligned16(w_gate_up) || !aligned16(topk_idx) || !aligned16(h) ||
      (dtype == MOE_MXFP8 &&
       (!aligned16(x_scales) || !aligned16(w_gate_up_scales) || !aligned16(h_scales))))
    return fail(MOE_ERR_ALIGN, "device pointers must be 16-byte aligned");
  int cus = 0;
  if (int st = device_info(&cus)) return st;
  return hip_status(moe::launch_gate_up_batched(x, x_scales, w_gate_up, w_gate_up_scales, topk_idx,
                                                T, H, I, E, k, dtype, h, h_scales, workspace,
                                                static_cast<hipStream_t>(stream), cus),
                    "moe_gate_up_3d_batched launch");
}

int moe_down_3d_batched(const void* h, const uint8_t* h_scales, const void* w_down,
                        const uint8_t* w_down_scales, const int32_t* topk_idx,
                        const float* topk_w, int T, int H, int I, int E, int k, moe_dtype dtype,
                        uint16_t* out, void* workspace, size_t workspace_bytes, void* stream) {
  if (int st = check_batched(T, H, I, E, k, dtype, workspace, workspace_bytes)) return st;
  if (!h || !w_down || !topk_idx || !topk_w || !out)
    return fail(MOE_ERR_NULL, "h, w_down, topk_idx, topk_w and out are required");
  if (dtype == MOE_MXFP8 && (!h_scales || !w_down_scales))
    return fail(MOE_ERR_NULL, "MXFP8 needs h_scales and w_down_scales");
  if (!aligned16(h) || !aligned16(w_down) || !aligned16(topk_idx) || !aligned16(topk_w) ||
      !aligned16(out) || (dtype == MOE_MXFP8 && (!aligned16(h_scales) || !aligned16(w_down_scales))))
    return fail(MOE_ERR_ALIGN, "device pointers must be 16-byte aligned");
  int cus = 0;
  if (int st = device_info(&cus)) return st;
  return hip_status(moe::launch_down_batched(h, h_scales, w_down, w_down_scales, topk_idx, topk_w,
                                             T, H, I, E, k, dtype, out, workspace,
                                             static_cast<hipStream_t>(stream), cus),
                    "moe_down_3d_batched launch");
}

size_t moe_backward_workspace_bytes(int T, int H, int I, int E, int k) {
  if (T < 1 || H <= 0 || I <= 0 || E < 1 || k < 1) return 0;
  return moe::backward_ws_layout(T, H, I, E, k).total;
}

int moe_backward_batched(const uint16_t* x, const uint16_t* w_gate_up, const uint16_t* w_down,
                         const int32_t* topk_idx, const float* topk_w, const uint16_t* dout,
                         const float* gu_saved, int T, int H, int I, int E, int k,
                         uint16_t* dx, uint16_t* dw_gate_up,
                         uint16_t* dw_down, float* d_topk_w, float* dlogits, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (int st = check_common(T, H, I, E, k, 256, 256)) return st;
  if (T < 1) return fail(MOE_ERR_SHAPE, "T=%d < 1", T);
  if (static_cast<long long>(T) * k > (1LL << 24))
    return fail(MOE_ERR_SHAPE, "T*k=%lld > 2^24", static_cast<long long>(T) * k);
  if (static_cast<long long>(T) * k * H >= (1LL << 31) ||
      static_cast<long long>(T) * k * 2 * I >= (1LL << 31) ||
      2LL * I * H >= (1LL << 31))
    return fail(MOE_ERR_SHAPE, "T*k*H, T*k*2I or 2I*H reaches 2^31");
  if (!x || !w_gate_up || !w_down || !topk_idx || !topk_w || !dout || !dx || !dw_gate_up ||
      !dw_down || !d_topk_w || !dlogits)
    return fail(MOE_ERR_NULL, "every input and output pointer is required");
  if (!workspace) return fail(MOE_ERR_WORKSPACE, "workspace is NULL");
  const size_t need = moe::backward_ws_layout(T, H, I, E, k).total;
  if (workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, need);
  if (!aligned16(x) || !aligned16(w_gate_up) || !aligned16(w_down) || !aligned16(topk_idx) ||
      !aligned16(topk_w) || !aligned16(dout) || !aligned16(dx) || !aligned16(dw_gate_up) ||
      !aligned16(dw_down) || !aligned16(d_topk_w) || !aligned16(dlogits) ||
      !aligned16(workspace) || (gu_saved && !aligned16(gu_saved)))
    return fail(MOE_ERR_ALIGN, "device pointers must be 16-byte aligned");
  int cus = 0;
  if (int st = device_info(&cus)) return st;
  return hip_status(moe::launch_backward(x, w_gate_up, w_down, topk_idx, topk_w, dout, gu_saved,
                                         T, H, I, E, k, dx, dw_gate_up, dw_down, d_topk_w,
                                         dlogits, workspace, static_cast<hipStream_t>(stream), cus),
                    "moe_backward_batched launch");
}

size_t moe_backward_mxfp8_workspace_bytes(int T, int H, int I, int E, int k) {
  if (T < 1 || H <= 0 || I <= 0 || E < 1 || k < 1) return 0;
  return moe::mx_backward_ws_layout(T, H, I, E, k).total;
}

int moe_backward_batched_mxfp8(const uint16_t* x, const uint8_t* w_gate_up,
                               const uint8_t* w_gate_up_scales, const uint8_t* w_down,
                               const uint8_t* w_down_scales, const int32_t* topk_idx,
                               const float* topk_w, const uint16_t* dout, int T, int H, int I,
                               int E, int k, uint16_t* dx, uint16_t* dw_gate_up, uint16_t* dw_down,
                               float* d_topk_w, float* dlogits, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (int st = check_common(T, H, I, E, k, 256, 256)) return st;
  if (T < 1) return fail(MOE_ERR_SHAPE, "T=%d < 1", T);
  if (static_cast<long long>(T) * k > (1LL << 24))
    return fail(MOE_ERR_SHAPE, "T*k=%lld > 2^24", static_cast<long long>(T) * k);
  if (int st = check_offsets(T, H, I, k)) return st;
  if (static_cast<long long>(T) * k * 2 * I >= (1LL << 31))
    return fail(MOE_ERR_SHAPE, "T*k*2I reaches 2^31");
  // pair-axis operands: rows x (routed pairs, each expert padded to 128) below 2^31
  {
    const size_t cols = static_cast<size_t>(T) * k + static_cast<size_t>(128) * E;
    const size_t rows = static_cast<size_t>(H > 2 * I ? H : 2 * I);
    if (rows * cols >= (static_cast<size_t>(1) << 31))
      return fail(MOE_ERR_SHAPE, "max(H, 2I) * (T*k + 128*E) reaches 2^31");
  }
  if (!x || !w_gate_up || !w_gate_up_scales || !w_down || !w_down_scales || !topk_idx ||
      !topk_w || !dout || !dx || !dw_gate_up || !dw_down || !d_topk_w || !dlogits)
    return fail(MOE_ERR_NULL, "every input and output pointer is required");
  if (!workspace) return fail(MOE_ERR_WORKSPACE, "workspace is NULL");
  const size_t need = moe::mx_backward_ws_layout(T, H, I, E, k).total;
  if (workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, need);
  if (!aligned16(x) || !aligned16(w_gate_up) || !aligned16(w_gate_up_scales) ||
      !aligned16(w_down) || !aligned16(w_down_scales) || !aligned16(topk_idx) ||
      !aligned16(topk_w) || !aligned16(dout) || !aligned16(dx) || !aligned16(dw_gate_up) ||
      !aligned16(dw_down) || !aligned16(d_topk_w) || !aligned16(dlogits) || !aligned16(workspace))
    return fail(MOE_ERR_ALIGN, "device pointers must be 16-byte aligned");
  int cus = 0;
  if (int st = device_info(&cus)) return st;
  return hip_status(moe::launch_backward_mx(x, w_gate_up, w_gate_up_scales, w_down, w_down_scales,
                                            topk_idx, topk_w, dout, T, H, I, E, k, dx, dw_gate_up,
                                            dw_down, d_topk_w, dlogits, workspace,
                                            static_cast<hipStream_t>(stream), cus),
                    "moe_backward_batched_mxfp8 launch");
}

int moe_gate_up_3d_batched_train(const uint16_t* x, const uint16_t* w_gate_up,
                                 const int32_t* topk_idx, int T, int H, int I, int E, int k,
                                 uint16_t* h, float* gu, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  if (int st = check_batched(T, H, I, E, k, MOE_BF16, workspace, workspace_bytes)) return st;
  if (!x || !w_gate_up || !topk_idx || !h || !gu)
    return fail(MOE_ERR_NULL, "x, w_gate_up, topk_idx, h and gu are required");
  if (static_cast<long long>(T) * k * 2 * I >= (1LL << 31))
    return fail(MOE_ERR_SHAPE, "T*k*2I reaches 2^31");
  if (!aligned16(x) || !aligned16(w_gate_up) || !aligned16(topk_idx) || !aligned16(h) ||
      !aligned16(gu))
    return fail(MOE_ERR_ALIGN, "device pointers must be 16-byte aligned");
  int cus = 0;
  if (int st = device_info(&cus)) return st;
  return hip_status(moe::launch_gate_up_batched(x, nullptr, w_gate_up, nullptr, topk_idx, T, H, I,
                                                E, k, MOE_BF16, h, nullptr, workspace,
                                                static_cast<hipStream_t>(stream), cus, gu),
                    "moe_gate_up_3d_batched_train launch");
}

}  // extern "C"
