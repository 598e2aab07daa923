// Top-k weighted combine back to token order:
// out[t] = y[R+t] (shared expert, weight 1) + sum_k w[t,k] * y[inv_pos[t*K+k]],
// fp32, in that order.  One workgroup per token; a thread covers 8 columns
// per pass with 16-byte accesses, and K is a template parameter so that all
// K+1 row loads of a pass are in flight together.
#include <utility>

#include "common.hpp"

namespace moeq4 {

namespace {

template <int K>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs c) {
  const int t = blockIdx.x;
  const int H = c.H;
  float wk[K];
  const float* rows[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    wk[k] = c.topk_w[(size_t)t * K + k];
    rows[k] = c.y + (size_t)c.inv_pos[(size_t)t * K + k] * H;
  }
  const float* ysh = c.y + (size_t)(c.R + t) * H;
  for (int col = 8 * threadIdx.x; col < H; col += 8 * blockDim.x) {
    f32x4 a0 = f32x4{0.f, 0.f, 0.f, 0.f}, a1 = a0;
    if (c.has_shared) {
      a0 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(ysh + col));
      a1 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(ysh + col + 4));
    }
    f32x4 v0[K], v1[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      v0[k] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(rows[k] + col));
      v1[k] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(rows[k] + col + 4));
    }
#pragma unroll
    for (int k = 0; k < K; ++k)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        a0[q] = __builtin_fmaf(wk[k], v0[k][q], a0[q]);
        a1[q] = __builtin_fmaf(wk[k], v1[k][q], a1[q]);
      }
    *reinterpret_cast<f32x4*>(c.out + (size_t)t * H + col) = a0;
    *reinterpret_cast<f32x4*>(c.out + (size_t)t * H + col + 4) = a1;
  }
}

template <int K>
bool launch_one(const CombineArgs& c, hipStream_t stream) {
  hipLaunchKernelGGL(combine_kernel<K>, dim3(c.T), dim3(256), 0, stream, c);
  return true;
}

template <int... Ks>
hipError_t launch_k(const CombineArgs& c, hipStream_t stream, std::integer_sequence<int, Ks...>) {
  const bool launched = ((c.K == Ks + 1 && launch_one<Ks + 1>(c, stream)) || ...);
  return launched ? hipGetLastError() : hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_combine(const CombineArgs& c, hipStream_t stream) {
  return launch_k(c, stream, std::make_integer_sequence<int, MOE_MAX_TOPK>{});
}

}  // namespace moeq4
