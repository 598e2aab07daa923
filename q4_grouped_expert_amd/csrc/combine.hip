// Top-k weighted combine back to token order:
// out[t] = y[R+t] (shared expert, weight 1) + sum_k w[t,k] * y[inv_pos[t*K+k]],
// fp32, in that order.  One workgroup per token, 16-byte accesses.
#include "common.hpp"

namespace moeq4 {

__global__ __launch_bounds__(256) void combine_kernel(CombineArgs c) {
  const int t = blockIdx.x;
  const int H = c.H, K = c.K;
  float wk[MOE_MAX_TOPK];
  const float* rows[MOE_MAX_TOPK];
#pragma unroll
  for (int k = 0; k < MOE_MAX_TOPK; ++k) {
    wk[k] = 0.0f;
    rows[k] = c.y;
    if (k < K) {
      wk[k] = c.topk_w[(size_t)t * K + k];
      rows[k] = c.y + (size_t)c.inv_pos[(size_t)t * K + k] * H;
    }
  }
  const float* ysh = c.y + (size_t)(c.R + t) * H;
  for (int col = 4 * threadIdx.x; col < H; col += 4 * blockDim.x) {
    f32x4 acc = c.has_shared ? *reinterpret_cast<const f32x4*>(ysh + col) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < MOE_MAX_TOPK; ++k) {
      if (k < K) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(rows[k] + col);
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] = __builtin_fmaf(wk[k], v[q], acc[q]);
      }
    }
    *reinterpret_cast<f32x4*>(c.out + (size_t)t * H + col) = acc;
  }
}

hipError_t launch_combine(const CombineArgs& c, hipStream_t stream) {
  hipLaunchKernelGGL(combine_kernel, dim3(c.T), dim3(256), 0, stream, c);
  return hipGetLastError();
}

}  // namespace moeq4
