// moe_route_topk: one wave per token, four tokens per workgroup.
#include "common.h"
#include "internal.h"
#include "route.h"
#include "tiles.h"

namespace moe {

__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T,
                                                         int E, int k, int32_t* __restrict__ idx,
                                                         float* __restrict__ w, uint32_t okey) {
  const int t0 = blockIdx.x * (blockDim.x / kWave) + wave_id();
  if (t0 >= T) return;
  const int t = permute_item(t0, T, okey);
  int e;
  float wt;
  route_token_any(logits + static_cast<size_t>(t) * E, E, k, &e, &wt);
  const int lane = lane_id();
  if (lane < k) {
    idx[static_cast<size_t>(t) * k + lane] = e;
    w[static_cast<size_t>(t) * k + lane] = wt;
  }
}

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* idx, float* w,
                             hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int per_block = 4;
  prof_begin(kRoute, s);
  hipLaunchKernelGGL(route_topk_kernel, dim3((T + per_block - 1) / per_block),
                     dim3(per_block * kWave), 0, s, logits, T, E, k, idx, w, order_key());
  prof_end(kRoute, s);
  return hipGetLastError();
}

}  // namespace moe
