// Top-k weighted combine back to token order:
// out[t] = y[R+t] (shared expert, weight 1) + sum_k w[t,k] * y[inv_pos[t*K+k]],
// fp32, in that order.  One workgroup per token; a thread covers 8 columns
// per pass (16-byte accesses for fp32 y, one 16-byte access for bf16 y), and
// K is a template parameter so that all K+1 row loads of a pass are in
// flight together.
#include <utility>

#include "common.hpp"

namespace moeq4 {

namespace {

// 8 consecutive elements of row `row` at column `col`, as fp32.
template <bool kBf16>
__device__ __forceinline__ void load8(const void* y, size_t row, int H, int col, f32x4& lo, f32x4& hi) {
  if constexpr (kBf16) {
    const u32x4 v = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(y) + row * H + col));
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      lo[2 * i] = __uint_as_float(v[i] << 16);
      lo[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
      hi[2 * i] = __uint_as_float(v[i + 2] << 16);
      hi[2 * i + 1] = __uint_as_float(v[i + 2] & 0xFFFF0000u);
    }
  } else {
    const float* p = reinterpret_cast<const float*>(y) + row * H + col;
    lo = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    hi = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + 4));
  }
}

template <int K, bool kBf16>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs c) {
  const int t = blockIdx.x;
  const int H = c.H;
  float wk[K];
  size_t rows[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    wk[k] = c.topk_w[(size_t)t * K + k];
    rows[k] = (size_t)c.inv_pos[(size_t)t * K + k];
  }
  const size_t rsh = (size_t)c.R + t;
  for (int col = 8 * threadIdx.x; col < H; col += 8 * blockDim.x) {
    f32x4 a0 = f32x4{0.f, 0.f, 0.f, 0.f}, a1 = a0;
    if (c.has_shared) load8<kBf16>(c.y, rsh, H, col, a0, a1);
    f32x4 v0[K], v1[K];
#pragma unroll
    for (int k = 0; k < K; ++k) load8<kBf16>(c.y, rows[k], H, col, v0[k], v1[k]);
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
  if (c.y_bf16) hipLaunchKernelGGL((combine_kernel<K, true>), dim3(c.T), dim3(256), 0, stream, c);
  else hipLaunchKernelGGL((combine_kernel<K, false>), dim3(c.T), dim3(256), 0, stream, c);
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
