// Unfused variant of the expert weights: a separate kernel writes every
// weight of the experts that have rows as bf16 to memory, for a bf16 grouped
// GEMM to read back.  The pages measure the fused in-GEMM dequant against
// exactly this write-then-read path ("Perplexity Lily 오픈소스 공개",
// alltoptrend.co.kr, section 5-1; "Apple silicon용 Lily, Qwen 추론 최적화",
// aitrends.kr, section "Qwen 구조와 Prefill 경로").  Decode rule as in the
// GEMM: w = bf16_rne(fma(q, scale, bias)) in fp32.
//
// One thread turns 16 consecutive weights of a row (8 code bytes) into 32
// bytes of bf16; the kernel streams codes in and bf16 out, HBM-bound.
#include "common.hpp"
#include "gemm_common.hpp"

namespace moeq4 {

namespace {
using namespace gemm;

constexpr int kDqThreads = 256;
constexpr int kDqPerThread = 16;  // weights per thread

__global__ __launch_bounds__(kDqThreads) void dequant_q4_kernel(DequantArgs d, int blocks_per_exp) {
  const int e = blockIdx.x / blocks_per_exp;
  const int blk = blockIdx.x - e * blocks_per_exp;
  if (d.counts && d.counts[e] == 0) return;  // no rows: its weights are never read
  const size_t per_exp = (size_t)d.N * d.K;
  const size_t i0 = ((size_t)blk * kDqThreads + threadIdx.x) * kDqPerThread;  // first weight, inside one row
  if (i0 >= per_exp) return;
  const int gpr = d.K / 64;
  const size_t n = i0 / d.K;
  const int k = (int)(i0 - n * d.K);
  const size_t eo = (size_t)e * per_exp;
  const u32x2 c = *reinterpret_cast<const u32x2*>(d.codes + (eo + i0) / 2);
  const size_t g = (size_t)e * d.N * gpr + n * gpr + k / 64;
  const float s = bf16_bits_to_f32(d.scales[g]), b = bf16_bits_to_f32(d.biases[g]);
  const bf16x8 w0 = dequant8(c[0], s, b), w1 = dequant8(c[1], s, b);
  u32x4* dst = reinterpret_cast<u32x4*>(d.out + eo + i0);
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4, w0), dst);
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4, w1), dst + 1);
}

}  // namespace

hipError_t launch_dequant(const DequantArgs& d, hipStream_t stream) {
  const size_t per_exp = (size_t)d.N * d.K;
  const int blocks_per_exp = (int)((per_exp + (size_t)kDqThreads * kDqPerThread - 1) / ((size_t)kDqThreads * kDqPerThread));
  hipLaunchKernelGGL(dequant_q4_kernel, dim3(d.n_exp * blocks_per_exp), dim3(kDqThreads), 0, stream, d,
                     blocks_per_exp);
  return hipGetLastError();
}

}  // namespace moeq4
