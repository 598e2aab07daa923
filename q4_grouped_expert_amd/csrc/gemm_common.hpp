// Device helpers shared by the grouped Q4 GEMM kernels (gfx950 / CDNA4).
#pragma once

#include "common.hpp"

namespace moeq4 {
namespace gemm {

constexpr uint32_t kOob = 0x80000000u;  // buffer offset that reads as zero
constexpr int kRsrcFlags = 0x00020000;  // raw buffer, 32-bit data format

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, kRsrcFlags);
}

// 8 codes (element 2i in the low nibble of byte i, 2i+1 in the high) ->
// bf16(fma(q, s, b)) for each, in element order.  After the nibble masks
// every byte holds one code q in its low four bits; read as an fp8 E4M3 byte
// that is q * 2^-9 exactly (codes 0..7 are the subnormals m * 2^-9, codes
// 8..15 the first normal binade (1 + m/8) * 2^-6), so the packed fp8
// conversion with scale 2^9 turns two bytes into two exact float codes per
// instruction.  The masks are applied in asm so the compiler keeps them.
__device__ __forceinline__ bf16x8 dequant8(uint32_t d, float s, float b) {
  uint32_t lo, hi;
  asm("v_and_b32 %0, 0x0f0f0f0f, %1" : "=v"(lo) : "v"(d));
  asm("v_lshrrev_b32 %0, 4, %1\n\tv_and_b32 %0, 0x0f0f0f0f, %0" : "=&v"(hi) : "v"(d));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const f32x2 e02 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(lo, 512.0f, false);  // elements 0, 2
  const f32x2 e46 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(lo, 512.0f, true);   // elements 4, 6
  const f32x2 e13 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hi, 512.0f, false);  // elements 1, 3
  const f32x2 e57 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hi, 512.0f, true);   // elements 5, 7
  u32x4 r;
  r[0] = pack_bf16x2(__builtin_fmaf(e02[0], s, b), __builtin_fmaf(e13[0], s, b));
  r[1] = pack_bf16x2(__builtin_fmaf(e02[1], s, b), __builtin_fmaf(e13[1], s, b));
  r[2] = pack_bf16x2(__builtin_fmaf(e46[0], s, b), __builtin_fmaf(e57[0], s, b));
  r[3] = pack_bf16x2(__builtin_fmaf(e46[1], s, b), __builtin_fmaf(e57[1], s, b));
  return __builtin_bit_cast(bf16x8, r);
}

// Accumulate and start-of-tile forms of v_mfma_f32_16x16x32_bf16.  The
// first reduction step of a tile uses the inline constant 0 as accumulator
// input instead of zero-initialized registers, which lets the register
// allocator keep every accumulator in place across the k-loop.
__device__ __forceinline__ void mfma_acc(f32x4& c, const bf16x8& a, const bf16x8& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void mfma_first(f32x4& c, const bf16x8& a, const bf16x8& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
}

// s_waitcnt that bounds only the vector-memory counter (gfx9 encoding: vmcnt
// in bits 3:0 and 15:14; expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt has six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// A gate/up launch of the fused-combine layer also clears `out` (read by the
// down launch that follows on the stream): block b of the grid clears its
// share, 16 bytes per thread and step.
__device__ __forceinline__ void zero_share(const GemmArgs& g) {
  if (!g.zero_out) return;
  const size_t per = ((g.zero_n + gridDim.x - 1) / gridDim.x + 3) & ~size_t(3);
  const size_t z0 = (size_t)blockIdx.x * per;
  const size_t z1 = z0 + per < g.zero_n ? z0 + per : g.zero_n;
  for (size_t i = z0 + 4 * threadIdx.x; i < z1; i += 4 * blockDim.x)
    *reinterpret_cast<f32x4*>(g.zero_out + i) = f32x4{0.f, 0.f, 0.f, 0.f};
}

// Down-GEMM output row p (grouped order): where its elements go in g.c and,
// for the fused combine, the weight it is added with.  Routed row p holds
// (t, k) = sorted_idx[p]; shared-expert rows p >= R hold token p - R with
// weight 1.
struct DownRow {
  size_t base;  // element offset of the row's first column in g.c
  float w;
};
__device__ __forceinline__ DownRow down_row(const GemmArgs& g, int p) {
  if (g.out_mode != kOutCombine) return DownRow{(size_t)p * g.N, 1.0f};
  if (p < g.R) {
    const int s = g.sorted_idx[p];
    return DownRow{(size_t)(s / g.topk) * g.N, g.topk_w[s]};
  }
  return DownRow{(size_t)(p - g.R) * g.N, 1.0f};
}

// Four consecutive output columns col..col+3 of a down row: stored as fp32
// or bf16 (RNE) y, or weighted and added into out with fp32 atomics.
__device__ __forceinline__ void store_down4(const GemmArgs& g, const DownRow& r, int col, const f32x4& v) {
  if (g.out_mode == kOutBf16) {
    uint16_t* y = reinterpret_cast<uint16_t*>(g.c) + r.base + col;
    *reinterpret_cast<u32x2*>(y) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  } else if (g.out_mode == kOutCombine) {
    float* o = reinterpret_cast<float*>(g.c) + r.base + col;
#pragma unroll
    for (int i = 0; i < 4; ++i) unsafeAtomicAdd(o + i, r.w * v[i]);
  } else {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(g.c) + r.base + col) = v;
  }
}

}  // namespace gemm
}  // namespace moeq4
