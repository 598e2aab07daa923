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
// bf16(fma(q, s, b)) for each, in element order.  The nibble masks are
// applied in asm so the compiler converts bytes with v_cvt_f32_ubyte{0..3}.
__device__ __forceinline__ bf16x8 dequant8(uint32_t d, float s, float b) {
  uint32_t lo, hi;
  asm("v_and_b32 %0, 0x0f0f0f0f, %1" : "=v"(lo) : "v"(d));
  asm("v_lshrrev_b32 %0, 4, %1\n\tv_and_b32 %0, 0x0f0f0f0f, %0" : "=&v"(hi) : "v"(d));
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float q0 = (float)((lo >> (8 * i)) & 0xFFu);
    const float q1 = (float)((hi >> (8 * i)) & 0xFFu);
    r[i] = pack_bf16x2(__builtin_fmaf(q0, s, b), __builtin_fmaf(q1, s, b));
  }
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

}  // namespace gemm
}  // namespace moeq4
