// Routing kernels: router logits + top-k, then histogram -> exclusive scan ->
// stable scatter -> tile block map, all on the device so the host never
// waits inside the layer ("Perplexity Lily 오픈소스 공개", alltoptrend.co.kr,
// section 5-2; "Apple silicon용 Lily, Qwen 추론 최적화", aitrends.kr, section
// "GPU 상주와 메모리 절감").
#include <math.h>

#include <type_traits>

#include "common.hpp"

namespace moeq4 {

// ---------------------------------------------------------------------------
// Router logits and top-k.
//
// Logit contract: l[t,e] is one fp32 chain over the hidden axis: acc = 0,
// then acc = acc + x[t,h] * Wr[e,h] for h = 0, 1, ..., H-1, then + bias[e].
// A bf16 x bf16 product is exact in fp32, so an fma chain in that order
// rounds exactly like "acc = acc + x*w"; every implementation that keeps the
// order gets bit-identical logits and hence bit-identical expert ids.
//
// Computing all T*E logits on the fp32 VALU costs 2*T*H*E flops.  Instead:
//  1. approximate logits a[t,e] with bf16 MFMA (fp32 accumulation, any
//     internal order), the hidden axis cut into ns equal splits whose
//     partial sums are added in order, then the bias;
//  2. bound both errors: |a - exact| <= da and |canonical - exact| <= dc,
//     with sum_h |x w| <= ||x_t|| * max_e ||w_e|| =: S (Cauchy-Schwarz),
//     da = 34 (H/32 + ns + 1) 2^-23 S  (each 32-product MFMA step off by at
//     most 33 fp32 ulps of its inputs, for any summation order or
//     truncation; each split adds at most one more step's worth, and the
//     ns - 1 adds of partial sums one ulp of S each),
//     dc = (H + 2) 2^-24 S  (bounds the rounding of an fp32 sum of H terms
//     in any order, the bias add included);
//  3. with tau = the K-th largest a[t,.], every expert outside
//     {e : a[t,e] >= tau - 2 (da + dc)} has a canonical logit strictly below
//     the K-th largest canonical logit, so it cannot be selected;
//  4. compute the canonical logits of the candidates only (about K+1 per
//     token) and select the top-k among them exactly.
// The result equals the full canonical computation, ties included.  When
// softmax weights run over all E experts (norm_topk = 0) every expert is a
// candidate.
// ---------------------------------------------------------------------------

namespace {
constexpr int kSelTokens = 16;                    // tokens per selection workgroup
constexpr int kXfStride = MOE_MAX_REDUCTION + 4;  // fp32 per token row in LDS (16-byte pad)
}  // namespace

// ||w_e||_2 of router row e, and the row copied piece-major:
// wt[p][e][0..7] = Wr[e][8p .. 8p+7] (p < H/8), so that piece p of
// neighbouring experts shares a cache line.  One wave.
__device__ __forceinline__ void router_row_prep(const uint16_t* __restrict__ wr, int H, int E, int e, int lane,
                                                float* __restrict__ wnorm, uint16_t* __restrict__ wt) {
  // H <= 2048: at most four 16-byte pieces per lane, all loaded before use
  u32x4 v[MOE_MAX_REDUCTION / 512];
#pragma unroll
  for (int i = 0; i < MOE_MAX_REDUCTION / 512; ++i) {
    const int h = 8 * lane + 512 * i;
    v[i] = h < H ? *reinterpret_cast<const u32x4*>(wr + (size_t)e * H + h) : u32x4{0u, 0u, 0u, 0u};
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < MOE_MAX_REDUCTION / 512; ++i) {
    const int h = 8 * lane + 512 * i;
    if (h < H) *reinterpret_cast<u32x4*>(wt + ((size_t)(h / 8) * E + e) * 8) = v[i];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float lo = bf16_bits_to_f32(v[i][q] & 0xFFFFu), hi = bf16_bits_to_f32(v[i][q] >> 16);
      s = __builtin_fmaf(lo, lo, s);
      s = __builtin_fmaf(hi, hi, s);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
  if (lane == 0) wnorm[e] = sqrtf(s);
}

namespace {
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcFlags = 0x00020000;
constexpr uint32_t kOob = 0x80000000u;  // buffer offset that reads as zero
__device__ __forceinline__ rsrc_t rsrc_of(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, kRsrcFlags);
}
// 16-byte-chunk swizzle of a 128-byte LDS row (conflict-free MFMA fragment
// reads for 16 consecutive rows); an involution.
__device__ __forceinline__ int rswz(int row, int c) { return c ^ (row & 7) ^ ((row >> 3) & 1); }
constexpr int kLgTile = 64;  // tokens and experts per approximate-logits workgroup
constexpr int kMaxLogitSplits = 8;  // hidden-axis splits of the approximate logits
constexpr int kLgK = 64;     // hidden columns per stage
constexpr int kLgRing = 4;   // LDS ring slots (loads run kLgRing - 1 stages ahead)
// s_waitcnt that bounds only the vector-memory counter (gfx9 encoding: vmcnt
// in bits 3:0 and 15:14; expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt has six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// s_waitcnt lgkmcnt(0) alone (vmcnt 63 and expcnt 7 leave those counters
// unconstrained).

// Order-preserving map of an fp32 value to uint32 (-0 is taken as +0 first,
// so equal values get equal keys) and its inverse.
__device__ __forceinline__ uint32_t fkey(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float fkey_inv(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}
// Sum over the 64 lanes, every lane getting the total, in a fixed order that
// only the norms' bound relies on: DPP within rows of 16, then the row-pair
// and half-wave swaps (with both operands the same register, a swap leaves a
// block's value in one output and its neighbour's in the other).
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float v) {
  return __uint_as_float((uint32_t)__builtin_amdgcn_update_dpp(0, (int)__float_as_uint(v), kCtrl, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_sum_f32(float a) {
  a = a + dpp_f32<0xB1>(a);   // quad_perm [1,0,3,2]
  a = a + dpp_f32<0x4E>(a);   // quad_perm [2,3,0,1]
  a = a + dpp_f32<0x141>(a);  // row_half_mirror
  a = a + dpp_f32<0x140>(a);  // row_mirror
  const uint32_t u = __float_as_uint(a);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  a = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  const uint32_t w = __float_as_uint(a);
  const auto h = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return __uint_as_float(h[0]) + __uint_as_float(h[1]);
}
// Lanes below this one in the wave.
__device__ __forceinline__ uint64_t lanes_below() {
  return (1ull << __lane_id()) - 1ull;
}
}  // namespace

// ---------------------------------------------------------------------------
// Approximate router logits a[t,e] = sum_h x[t,h] w[e,h] (+ bias) on bf16 MFMA
// with fp32 accumulation.
//
// One workgroup: 64 tokens x 64 experts; wave w owns the 32 x 32 quadrant
// (tokens 32 (w & 1).., experts 32 (w >> 1)..) as 2 x 2 MFMA tiles.  Token
// and router rows stream through a 4-slot LDS ring of 64-column stages
// filled by direct-to-LDS loads three stages ahead.  Every MFMA adds a
// 32-product step to its fp32 accumulator, the structure the selection
// kernel's error bound assumes.
//
// Block order: consecutive workgroup ids land on consecutive XCDs, so id b
// takes token tile 8 (b / 8 / neb) + b % 8 and expert tile (b / 8) % neb:
// the neb workgroups that share a token tile run on one XCD and share its
// L2.  Ids past the last token tile exit at once.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void route_logits_kernel(RouteArgs a, int ntb, int neb, int nsplit,
                                                           float* __restrict__ alog, float* __restrict__ wnorm,
                                                           uint16_t* __restrict__ wt, int32_t* __restrict__ hist,
                                                           int hist_len) {
  constexpr int kRows = 2 * kLgTile;            // token rows, then router rows
  constexpr int kSlot = kRows * kLgK;           // bf16 elements per ring slot
  __shared__ __attribute__((aligned(16))) uint16_t ring[kLgRing * kSlot];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // What the selection kernel (the next launch) reads besides the logits:
  // cleared expert histograms, router-row norms and the piece-major router
  // copy, spread over the whole grid (wave 0 of block b takes experts b,
  // b + grid, ...), before any block exits.
  for (int i = blockIdx.x * 256 + tid; i < hist_len; i += gridDim.x * 256) hist[i] = 0;
  if (wave == 0)
    for (int e = blockIdx.x; e < a.E; e += gridDim.x) router_row_prep(a.w_router, a.H, a.E, e, lane, wnorm, wt);
  const int ln = lane & 15, lg = lane >> 4;
  // split of the hidden axis outermost, then the token-tile / expert-tile
  // order described above
  const int base = (ntb + 7) / 8 * 8 * neb;
  const int split = blockIdx.x / base, bb = blockIdx.x - split * base;
  const int q = bb >> 3;
  const int tb = (q / neb) * 8 + (bb & 7), eb = q % neb;
  if (tb >= ntb) return;
  const int t0 = tb * kLgTile, e0 = eb * kLgTile;
  const int T = a.T, H = a.H, E = a.E;
  const int nk = H / kLgK / nsplit;  // stages of this split
  const int kbase = split * nk;      // its first stage
  const rsrc_t x_rs = rsrc_of(a.x, (uint32_t)T * H * 2u);
  const rsrc_t w_rs = rsrc_of(a.w_router, (uint32_t)E * H * 2u);

  // DMA plan per stage: wave w fills token rows 16w + 8i + lane/8 and router
  // rows 16w + 8i + lane/8 (i < 2); lane l writes 16 B at physical chunk l%8
  // of its row, fetching the logical chunk the swizzle maps there.  Rows
  // past T or E read as zero.
  uint32_t xoff[2], woff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 16 * wave + 8 * i + (lane >> 3);
    xoff[i] = t0 + r < T ? ((uint32_t)(t0 + r) * H + 8u * rswz(r, lane & 7)) * 2u : kOob;
    woff[i] = e0 + r < E ? ((uint32_t)(e0 + r) * H + 8u * rswz(r, lane & 7)) * 2u : kOob;
  }
  constexpr int kDmaPerStage = 4;  // direct-to-LDS loads per wave per stage
  auto dma = [&](int slot, int kt) {
    uint16_t* S = ring + slot * kSlot;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          x_rs, (__attribute__((address_space(3))) void*)(S + (16 * wave + 8 * i) * kLgK), 16, xoff[i],
          (kbase + kt) * kLgK * 2, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          w_rs, (__attribute__((address_space(3))) void*)(S + (kLgTile + 16 * wave + 8 * i) * kLgK), 16, woff[i],
          (kbase + kt) * kLgK * 2, 0, 0);
    }
  };

  const int wm = wave & 1, wn = wave >> 1;
  f32x4 acc[2][2];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[m][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto stage = [&](int slot) {
    const uint16_t* S = ring + slot * kSlot;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      bf16x8 av[2], bv[2];
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int r = 32 * wm + 16 * m + ln;
        av[m] = *reinterpret_cast<const bf16x8*>(&S[r * kLgK + rswz(r, 2 * lg + st) * 8]);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = 32 * wn + 16 * j + ln;
        bv[j] = *reinterpret_cast<const bf16x8*>(&S[(kLgTile + r) * kLgK + rswz(r, 2 * lg + st) * 8]);
      }
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[m][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[m], bv[j], acc[m][j], 0, 0, 0);
    }
  };

  // Stage kt DMAs stage kt + R - 1 (R = kLgRing slots) into the slot read in
  // stage kt - 1 (free since the last barrier), computes on slot kt % R, then
  // waits until only the DMAs of its last R - 2 stages are in flight (so
  // stage kt + 1 has landed) and meets the other waves at the barrier.  Past
  // the last stage the DMAs repeat the last one, keeping the count per stage
  // fixed; no other vector-memory access runs inside the loop, so the count
  // is exact.
  constexpr int R = kLgRing;
  const int last = nk - 1;
#pragma unroll
  for (int s0 = 0; s0 < R - 1; ++s0) dma(s0, min(s0, last));
  wait_vmcnt<(R - 2) * kDmaPerStage>();
  __builtin_amdgcn_s_barrier();
  int kt = 0;
  for (; kt + R <= nk; kt += R) {
#pragma unroll
    for (int u = 0; u < R; ++u) {
      dma((u + R - 1) % R, min(kt + u + R - 1, last));
      stage(u);
      wait_vmcnt<(R - 2) * kDmaPerStage>();
      __builtin_amdgcn_s_barrier();
    }
  }
#pragma unroll
  for (int u = 0; u < R - 1; ++u) {
    if (kt + u < nk) {
      dma((u + R - 1) % R, min(kt + u + R - 1, last));
      stage(u);
      wait_vmcnt<(R - 2) * kDmaPerStage>();
      __builtin_amdgcn_s_barrier();
    }
  }
  wait_vmcnt<0>();  // no direct-to-LDS write outlives the workgroup

  // this split's partial sums (the selection kernel adds the splits in order,
  // then the bias); MFMA layout: lane holds rows 4*lg+i, column ln
  float* part = alog + (size_t)split * T * E;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int e = e0 + 32 * wn + 16 * j + ln;
    if (e < E) {
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = t0 + 32 * wm + 16 * m + 4 * lg + i;
          if (t < T) part[(size_t)t * E + e] = acc[m][j][i];
        }
    }
  }
}

namespace {
// acc <- fma(x[q], w[q], acc) for q = 0..7 in order, w eight packed bf16.
// One asm block, so the compiler cannot unpack a piece of w early (it does
// so to free registers, and then has to wait for loads still in flight).
__device__ __forceinline__ float chain8(float acc, float4 x0, float4 x1, u32x4 w) {
  float t0, t1;
  asm("v_lshlrev_b32 %[t0], 16, %[w0]\n\t"
      "v_and_b32 %[t1], 0xffff0000, %[w0]\n\t"
      "v_fmac_f32 %[acc], %[xa], %[t0]\n\t"
      "v_fmac_f32 %[acc], %[xb], %[t1]\n\t"
      "v_lshlrev_b32 %[t0], 16, %[w1]\n\t"
      "v_and_b32 %[t1], 0xffff0000, %[w1]\n\t"
      "v_fmac_f32 %[acc], %[xc], %[t0]\n\t"
      "v_fmac_f32 %[acc], %[xd], %[t1]\n\t"
      "v_lshlrev_b32 %[t0], 16, %[w2]\n\t"
      "v_and_b32 %[t1], 0xffff0000, %[w2]\n\t"
      "v_fmac_f32 %[acc], %[xe], %[t0]\n\t"
      "v_fmac_f32 %[acc], %[xf], %[t1]\n\t"
      "v_lshlrev_b32 %[t0], 16, %[w3]\n\t"
      "v_and_b32 %[t1], 0xffff0000, %[w3]\n\t"
      "v_fmac_f32 %[acc], %[xg], %[t0]\n\t"
      "v_fmac_f32 %[acc], %[xh], %[t1]"
      : [acc] "+v"(acc), [t0] "=&v"(t0), [t1] "=&v"(t1)
      : [w0] "v"(w[0]), [w1] "v"(w[1]), [w2] "v"(w[2]), [w3] "v"(w[3]), [xa] "v"(x0.x), [xb] "v"(x0.y),
        [xc] "v"(x0.z), [xd] "v"(x0.w), [xe] "v"(x1.x), [xf] "v"(x1.y), [xg] "v"(x1.z), [xh] "v"(x1.w));
  return acc;
}
// m[j] = mask of the lanes whose k[j] >= c[j] (c wave-uniform), for four
// tokens j.  The four compares sit in one block so that they issue back to
// back and the scalar unit reads their masks after one wait, instead of one
// vector-to-scalar wait per compare.  The outputs are early-clobber: a mask
// written early must not land on a threshold register a later compare reads.
__device__ __forceinline__ void ballot_ge4(uint64_t (&m)[4], const uint32_t (&k)[4], const uint32_t (&c)[4]) {
  asm("v_cmp_le_u32_e64 %0, %4, %8\n\tv_cmp_le_u32_e64 %1, %5, %9\n\t"
      "v_cmp_le_u32_e64 %2, %6, %10\n\tv_cmp_le_u32_e64 %3, %7, %11"
      : "=&s"(m[0]), "=&s"(m[1]), "=&s"(m[2]), "=&s"(m[3])
      : "s"(c[0]), "s"(c[1]), "s"(c[2]), "s"(c[3]), "v"(k[0]), "v"(k[1]), "v"(k[2]), "v"(k[3]));
}
}  // namespace

// ---------------------------------------------------------------------------
// Selection: candidates from the approximate logits, canonical logits for the
// candidates only, exact top-k, combine weights, expert histogram.
//
// One workgroup = 16 tokens; in the per-token steps wave w owns tokens
// 4w .. 4w+3.  The candidate chains (token, expert) of all 16 tokens are
// listed in expert order and run one per lane, each a full sequential fp32
// chain over the hidden axis: the token row comes from LDS as fp32 (rows
// padded by 16 bytes so that 16 different rows hit 16 different bank
// groups), the router row from the piece-major copy wt, where a wave's
// experts, being sorted, share cache lines.  Router pieces stream P pieces
// ahead of use in registers.
// ---------------------------------------------------------------------------
template <int NSPLIT>
__global__ __launch_bounds__(256) void route_select_kernel(RouteArgs a, const float* __restrict__ alog,
                                                           const float* __restrict__ wn,
                                                           const uint16_t* __restrict__ wt,
                                                           int32_t* __restrict__ hist, int ngp) {
  constexpr int TB = kSelTokens;
  constexpr int TPW = TB / 4;                 // tokens per wave in the per-token steps
  static_assert(TPW == 4, "the candidate search handles four tokens per wave");
  constexpr int NP = MOE_MAX_REDUCTION / 512;  // 16-byte row pieces per lane
  __shared__ __attribute__((aligned(16))) float xf[TB * kXfStride];
  // candidates per token, in the order their chains finish: fkey of the
  // canonical logit, and the expert
  __shared__ uint32_t ckv[TB][MOE_MAX_EXPERTS];
  __shared__ uint8_t cke[TB][MOE_MAX_EXPERTS];
  __shared__ uint32_t emask[MOE_MAX_EXPERTS];  // bit tk: expert e is a candidate of token tk
  __shared__ int estart[MOE_MAX_EXPERTS + 1];  // chains of the experts below e
  __shared__ int wsum[4];
  __shared__ int ccount[TB], cfill[TB];
  __shared__ float lmax[TB];      // largest canonical logit per token
  __shared__ float evs[TB][16];  // softmax terms by slot (tokens with at most 16 candidates)
  __shared__ float wmax_s, xn_s[TB];
  __shared__ int bhist[MOE_MAX_EXPERTS];
  __shared__ float bias_s[MOE_MAX_EXPERTS];  // router bias (read after the chains without a global load)

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t0 = blockIdx.x * TB;
  const int T = a.T, H = a.H, E = a.E, K = a.K;
  const rsrc_t x_rs = rsrc_of(a.x, (uint32_t)T * H * 2u);
  const rsrc_t w_rs = rsrc_of(wt, (uint32_t)E * H * 2u);

  bhist[tid] = 0;
  emask[tid] = 0u;
  if (tid < TB) cfill[tid] = 0;
  // router bias: loaded now, stored to LDS once the row loads are issued
  const float rb = a.router_bias && tid < E ? a.router_bias[tid] : 0.0f;

  // ---- token rows of wave w to fp32 in LDS, their norms; approximate logits
  // of its tokens (lane holding experts 4 lane .. 4 lane + 3); all loads of
  // the step are issued before any is used
  float av[TPW][4];
  {
    // this lane's four experts' partial sums, one 16-byte load per split and
    // token (experts past E read what follows in the array, or zeros past
    // its end, and are masked below)
    const rsrc_t a_rs = rsrc_of(alog, (uint32_t)NSPLIT * T * E * 4u);
    u32x4 v[TPW][NP];
    u32x4 pa[TPW][NSPLIT];
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const int t = t0 + TPW * wave + j;
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        const int h = 8 * lane + 512 * i;
        const uint32_t off = t < T && h < H ? ((uint32_t)t * H + h) * 2u : kOob;
        v[j][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(x_rs, off, 0, 0));
      }
#pragma unroll
      for (int sp = 0; sp < NSPLIT; ++sp) {
        const uint32_t off = t < T && 4 * lane < E ? (((uint32_t)sp * T + t) * E + 4 * lane) * 4u : kOob;
        pa[j][sp] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(a_rs, off, 0, 0));
      }
    }
    // the approximate logits: the hidden-axis splits added in order (the
    // bias follows in the candidate step)
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const bool tv = t0 + TPW * wave + j < T;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float v = __uint_as_float(pa[j][0][q]);
#pragma unroll
        for (int sp = 1; sp < NSPLIT; ++sp) v += __uint_as_float(pa[j][sp][q]);
        av[j][q] = tv && 4 * lane + q < E ? v : 0.0f;
      }
    }
    float wv[MOE_MAX_EXPERTS / 64];
    if (wave == 0) {
#pragma unroll
      for (int i = 0; i < MOE_MAX_EXPERTS / 64; ++i) wv[i] = lane + 64 * i < E ? wn[lane + 64 * i] : 0.0f;
    }
    bias_s[tid] = rb;
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const int tk = TPW * wave + j;
      float s2 = 0.0f;
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        const int h = 8 * lane + 512 * i;
        if (h < H) {
          float f[8];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            f[2 * q] = bf16_bits_to_f32(v[j][i][q] & 0xFFFFu);
            f[2 * q + 1] = bf16_bits_to_f32(v[j][i][q] >> 16);
          }
#pragma unroll
          for (int q = 0; q < 8; ++q) s2 = __builtin_fmaf(f[q], f[q], s2);
          float4* dst = reinterpret_cast<float4*>(&xf[tk * kXfStride + h]);
          dst[0] = float4{f[0], f[1], f[2], f[3]};
          dst[1] = float4{f[4], f[5], f[6], f[7]};
        }
      }
      s2 = wave_sum_f32(s2);
      if (lane == 0) xn_s[tk] = sqrtf(s2);
    }
    if (wave == 0) {
      float m = 0.0f;
#pragma unroll
      for (int i = 0; i < MOE_MAX_EXPERTS / 64; ++i) m = fmaxf(m, wv[i]);
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
      if (lane == 0) wmax_s = m;
    }
  }
  __syncthreads();

  // ---- candidates of the wave's tokens -----------------------------------
  // tau_j <= the K-th largest approximate logit of token j.  Each lane takes
  // the largest of its four keys; the K-th largest of these lane maxima is at
  // most the K-th largest key (the K largest lane maxima are K different
  // keys).  th = the largest 16-bit key prefix with at least K lane maxima at
  // or above it, built bit by bit (wave-uniform, the wave's tokens side by
  // side), so th << 16 is at most the K-th largest key; a lower tau only
  // widens the candidate set.  With fewer than K lanes holding keys
  // (E < 4K) no prefix qualifies and every expert is a candidate.
  {
    if (a.router_bias) {
#pragma unroll
      for (int j = 0; j < TPW; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (4 * lane + q < E) av[j][q] = av[j][q] + bias_s[4 * lane + q];
    }
    uint32_t mk[TPW], th[TPW];
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const bool tvalid = t0 + TPW * wave + j < T;
      uint32_t m = 0u;
#pragma unroll
      for (int q = 0; q < 4; ++q) m = max(m, tvalid && 4 * lane + q < E ? fkey(av[j][q]) >> 16 : 0u);
      mk[j] = m;
      th[j] = 0u;
    }
#pragma unroll
    for (int bit = 15; bit >= 0; --bit) {
      uint32_t c[TPW];
#pragma unroll
      for (int j = 0; j < TPW; ++j) c[j] = th[j] | (1u << bit);
      uint64_t m[TPW];
      ballot_ge4(m, mk, c);
#pragma unroll
      for (int j = 0; j < TPW; ++j)
        if (__popcll(m[j]) >= K) th[j] = c[j];
    }
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const int tk = TPW * wave + j;
      const bool tvalid = t0 + tk < T;
      const float tau = th[j] ? fkey_inv(th[j] << 16) : -INFINITY;
      float win;
      if (!a.norm_topk) {
        win = INFINITY;
      } else {
        const float S = xn_s[tk] * wmax_s * 1.001f;
        const float da = 34.0f * (float)(H / 32 + NSPLIT + 1) * 0x1p-23f * S;
        const float dc = (float)(H + 2) * 0x1p-24f * S;
        win = 2.1f * (da + dc) + 0x1p-20f * (fabsf(tau) + 1.0f);
      }
      int total = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bool f = tvalid && 4 * lane + q < E && av[j][q] >= tau - win;
        total += __popcll(__ballot(f));
        if (f) atomicOr(&emask[4 * lane + q], 1u << tk);
      }
      if (lane == 0) ccount[tk] = total;
    }
  }
  __syncthreads();

  // ---- chain list in expert order: exclusive scan of the candidate counts
  {
    const int n = __popc(emask[tid]);
    int inc = n;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(inc, o);
      if (lane >= o) inc += u;
    }
    if (lane == 63) wsum[wave] = inc;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w) base += wsum[w];
    estart[tid] = base + inc - n;
    if (tid == MOE_MAX_EXPERTS - 1) estart[MOE_MAX_EXPERTS] = base + inc;
  }
  __syncthreads();

  // ---- canonical logits: acc = 0, acc += x[t,h] * Wr[e,h] for h ascending,
  // then + bias; bf16 x bf16 products are exact in fp32, so each fma rounds
  // exactly like "acc = acc + x*w".  Chain c runs on thread c % 256 of pass
  // c / 256; piece p (columns 8p .. 8p+7) of expert e sits at wt + (p E + e) 8.
  const int npc = H / 8;
  auto chains = [&](auto depth) {
    constexpr int P = decltype(depth)::value;
    const int nch = estart[MOE_MAX_EXPERTS];
    for (int c0 = 0; c0 < nch; c0 += 256) {
      const int c = c0 + tid;
      const bool live = c < nch;
      // expert: the last e with estart[e] <= c; token: the (c - estart[e])-th
      // set bit of emask[e]
      int lo = 0, hi = MOE_MAX_EXPERTS;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int mid = (lo + hi) >> 1;
        if (estart[mid] <= c) lo = mid;
        else hi = mid;
      }
      const int e = lo;
      uint32_t m = live ? emask[e] : 1u;
      for (int r = live ? c - estart[e] : 0; r > 0; --r) m &= m - 1u;
      const int tk = __builtin_ctz(m);
      const uint32_t voff = live ? (uint32_t)e * 16u : kOob;
      const float* xr = &xf[tk * kXfStride];
      const uint32_t pstride = (uint32_t)E * 16u;  // bytes from one piece to the next
      // first group in piece order (the loop's waits assume wb[i] was issued
      // i-th, on entry as on the back edge)
      u32x4 wb[P];
#pragma unroll
      for (int i = 0; i < P; ++i) {
        wb[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(w_rs, voff, i * pstride, 0));
        __builtin_amdgcn_sched_barrier(0);
      }
      float acc = 0.0f;
      uint32_t vo = voff;
      for (int p0 = 0; p0 < npc; p0 += P) {
        const int nxt = p0 + P < npc ? p0 + P : p0;  // the last group re-reads itself
#pragma unroll
        for (int i = 0; i < P; ++i) {
          const float4 x0 = *reinterpret_cast<const float4*>(&xr[8 * (p0 + i)]);
          const float4 x1 = *reinterpret_cast<const float4*>(&xr[8 * (p0 + i) + 4]);
          acc = chain8(acc, x0, x1, wb[i]);
          // Reload wb[i] only after its last use: the empty asm makes the
          // offset depend on acc, so the scheduler cannot hoist the load (a
          // hoisted load needs a second register set, copied back behind a
          // full wait at the loop's back edge).
          asm("" : "+v"(vo) : "v"(acc));
          wb[i] = __builtin_bit_cast(u32x4,
                                     __builtin_amdgcn_raw_buffer_load_b128(w_rs, vo, (nxt + i) * pstride, 0));
        }
      }
      if (live) {
        if (a.router_bias) acc = acc + bias_s[e];
        const int slot = atomicAdd(&cfill[tk], 1);
        ckv[tk][slot] = fkey(acc);
        cke[tk][slot] = (uint8_t)e;
      }
    }
  };
  if (npc % 16 == 0)
    chains(std::integral_constant<int, 16>{});
  else
    chains(std::integral_constant<int, 8>{});
  __syncthreads();

  // ---- exact top-k of each token among its candidates --------------------
  // A candidate's slot is the number of its token's candidates with a larger
  // key (logit, then lower expert; keys are distinct); the K smallest slots
  // are the selection, already in slot order.  Combine weights: exp(l - max)
  // over the sum of exp(l - max) of the selection (norm_topk) or of every
  // expert, the sums taken across lanes.
  auto ckey = [&](int tk, int c) -> unsigned long long {
    return ((unsigned long long)ckv[tk][c] << 8) | (unsigned)(255 - cke[tk][c]);
  };
  auto emit = [&](int t, int rank, int e, float w) {
    a.out.topk_ids[(size_t)t * K + rank] = e;
    a.out.topk_w[(size_t)t * K + rank] = w;
    atomicAdd(&bhist[e], 1);
  };
  bool small = true;
#pragma unroll
  for (int j = 0; j < TPW; ++j) small = small && ccount[TPW * wave + j] <= 16;
  if (small) {
    // the wave's tokens side by side, 16 lanes each, one candidate per lane
    const int j = lane >> 4, sl = lane & 15;
    const int tk = TPW * wave + j;
    const int C = ccount[tk];  // 0 for tokens past T
    const bool valid = sl < C;
    const unsigned long long my = valid ? ckey(tk, sl) : 0ull;
    int n = 0;
#pragma unroll
    for (int o = 0; o < 16; ++o) n += o < C && ckey(tk, o) > my ? 1 : 0;
    const float v = fkey_inv((uint32_t)(my >> 8));
    if (valid && n == 0) lmax[tk] = v;
    __builtin_amdgcn_wave_barrier();
    const float ev = valid ? expf(v - lmax[tk]) : 0.0f;
    // the sum runs over the terms placed by slot, in a fixed tree, so the
    // weights do not depend on the order the chains finished in
    if (valid) evs[tk][n] = ev;
    __builtin_amdgcn_wave_barrier();
    float part = sl < C && (!a.norm_topk || sl < K) ? evs[tk][sl] : 0.0f;
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) part += __shfl_xor(part, o, 16);
    if (valid && n < K) emit(t0 + tk, n, 255 - (int)(my & 255ull), ev / part);
  } else {
#pragma unroll 1
    for (int j = 0; j < TPW; ++j) {
      const int tk = TPW * wave + j;
      const int C = ccount[tk];
      float v[MOE_MAX_EXPERTS / 64];
      int me[MOE_MAX_EXPERTS / 64], rank[MOE_MAX_EXPERTS / 64];
#pragma unroll
      for (int r = 0; r < MOE_MAX_EXPERTS / 64; ++r) {
        const int c = lane + 64 * r;
        rank[r] = K;
        me[r] = 0;
        v[r] = 0.0f;
        if (64 * r < C) {
          const unsigned long long my = c < C ? ckey(tk, c) : 0ull;
          int n = 0;
#pragma unroll 4
          for (int o = 0; o < C; ++o) n += ckey(tk, o) > my ? 1 : 0;
          me[r] = 255 - (int)(my & 255ull);
          v[r] = fkey_inv((uint32_t)(my >> 8));
          if (c < C) {
            rank[r] = n;
            if (n == 0) lmax[tk] = v[r];
          }
        }
      }
      __builtin_amdgcn_wave_barrier();
      const float mx = C > 0 ? lmax[tk] : 0.0f;
      // terms placed by slot (over the keys, which every lane has read; same
      // element type, so the stores stay behind those reads), then summed in
      // a fixed tree: lane l adds slots 4l .. 4l+3
      float ev[MOE_MAX_EXPERTS / 64];
#pragma unroll
      for (int r = 0; r < MOE_MAX_EXPERTS / 64; ++r) {
        ev[r] = 0.0f;
        if (lane + 64 * r < C) {
          ev[r] = expf(v[r] - mx);
          ckv[tk][rank[r]] = __float_as_uint(ev[r]);
        }
      }
      __builtin_amdgcn_wave_barrier();
      const int nterm = a.norm_topk ? K : C;
      float part = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * lane + i < nterm) part += __uint_as_float(ckv[tk][4 * lane + i]);
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) part += __shfl_xor(part, o);
#pragma unroll
      for (int r = 0; r < MOE_MAX_EXPERTS / 64; ++r)
        if (rank[r] < K) emit(t0 + tk, rank[r], me[r], ev[r] / part);
    }
  }
  // LDS-only barrier: the histogram atomics above must land, the global
  // stores need not
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  // this workgroup's tokens lie in one histogram group of kHistTokens;
  // hist is [E][ngp]
  if (tid < E && bhist[tid]) atomicAdd(&hist[(size_t)tid * ngp + t0 / kHistTokens], bhist[tid]);
}

// ---------------------------------------------------------------------------
// Group offsets, tile block map and stable scatter (sorted_idx / inv_pos).
//
// hist[e][g] holds the rows of expert e among the tokens of group g (64
// tokens each); rows are ngp = ng rounded up to 4 ints long.  One workgroup
// per group, one thread per expert: it sums its expert's row of hist into the
// total count and the rows that earlier groups own, and a workgroup-wide
// exclusive scan of the totals gives the expert group offsets.  The four
// waves place the group's rows (lane l: token l of the group; wave w: slots
// w, w + 4, ...): a (t, k) row goes to offsets[e] + (rows of e in earlier
// groups) + (earlier tokens of this group that chose e, from a 64-bit LDS
// mask).  The expert ids are loaded before the histogram rows, so both loads
// are in flight together.  Workgroup 0 also writes counts, offsets and the
// block map (each expert's tiles of at most kTileRows rows, then the shared
// expert's).  When lmap is set, the last workgroup lists the same tiles again
// in launch order: most 16-row subtiles first (a GEMM workgroup's time grows
// with them), so the grouped GEMM starts the longest tiles first and ends on
// the shortest; or, with launch_rows below kTileRows, every expert's rows cut
// into pieces of at most launch_rows rows for the small-prompt GEMMs, in the
// same order (full pieces first, then the partial ones by subtile count);
// n_launch entries in all.
// Places come from ballots (the lanes with the same subtile count, the bits
// of the full-tile counts) and a scan over the 16 counts, so the list is
// stored in the same phase as the block map.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(MOE_MAX_EXPERTS) void route_group_kernel(const int32_t* __restrict__ hist, int ngp,
                                                                      int T, int K, int E, int has_shared,
                                                                      moe_route_out out, int32_t* __restrict__ lmap,
                                                                      int32_t* __restrict__ n_launch, int launch_rows) {
  __shared__ int wsum[MOE_MAX_EXPERTS / 64][2];
  __shared__ int before_s[MOE_MAX_EXPERTS], off_s[MOE_MAX_EXPERTS];
  __shared__ unsigned long long mask[MOE_MAX_EXPERTS];
  constexpr int BM = kTileRows;
  constexpr int kSub = BM / 16;  // launch order: subtile counts 1..kSub, bucket kSub - count
  __shared__ int4 pw[kSub];      // launch order: partial tiles of bucket b in wave w (.x .. .w)
  __shared__ int wfull[MOE_MAX_EXPERTS / 64];  // launch order: full tiles of the experts of wave w
  const int e = threadIdx.x;
  const int lane = e & 63, wave = e >> 6;
  const int g = blockIdx.x;
  // the last workgroup also lists the launch order (every workgroup has the
  // whole histogram; the first one writes the block map)
  const bool order = g == (int)gridDim.x - 1 && lmap != nullptr;
  // a piece list (launch_rows < BM): pieces of at most LR rows, in the same
  // order as tiles (full pieces first, then the partial ones by subtile count)
  const bool pieces = launch_rows < BM;
  const int LR = pieces ? launch_rows : BM;

  mask[e] = 0ull;
  if (lane < kSub) reinterpret_cast<int*>(&pw[lane])[wave] = 0;  // each wave clears its own column
  // this thread's (token, slot) rows: token g*64 + lane, slots wave + 4j
  constexpr int kSlotsPerWave = (MOE_MAX_TOPK + 3) / 4;
  const int t = g * kHistTokens + lane;
  int my[kSlotsPerWave];
#pragma unroll
  for (int j = 0; j < kSlotsPerWave; ++j) {
    const int k = wave + 4 * j;
    const int id = t < T && k < K ? out.topk_ids[(size_t)t * K + k] : -1;
    my[j] = (unsigned)id < (unsigned)E ? id : -1;  // ids are produced in range; the check keeps indexing safe
  }
  // per-expert total and the part owned by groups before g; a row of hist
  // (ngp ints, 16-byte aligned, zero past ng) is read 64 groups per round,
  // all loads of a round in flight together
  int run = 0, before = 0;
  if (e < E) {
    const int4* row = reinterpret_cast<const int4*>(hist + (size_t)e * ngp);
    for (int g0 = 0; g0 < ngp; g0 += 64) {
      int4 v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = g0 + 4 * i < ngp ? row[g0 / 4 + i] : int4{0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int gi = g0 + 4 * i;
        before += (gi < g ? v[i].x : 0) + (gi + 1 < g ? v[i].y : 0) + (gi + 2 < g ? v[i].z : 0) +
                  (gi + 3 < g ? v[i].w : 0);
        run += v[i].x + v[i].y + v[i].z + v[i].w;
      }
    }
  }
  const int nt = (run + BM - 1) / BM;
  // workgroup-wide exclusive scans of counts and tile counts
  int ic = run, it = nt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int vc = __shfl_up(ic, o), vt = __shfl_up(it, o);
    if (lane >= o) {
      ic += vc;
      it += vt;
    }
  }
  if (lane == 63) {
    wsum[wave][0] = ic;
    wsum[wave][1] = it;
  }
  // launch order, part 1: this expert's full tiles and its last, partial tile
  // (rem rows, bucket bp); per bucket, the wave's experts with such a tile
  const int nfull = run / LR, rem = run - nfull * LR;
  const int bp = kSub - ((rem + 15) >> 4);
  uint64_t same_b = 0;  // lanes of this wave whose partial tile is in bucket bp
  if (order) {
    // the lanes with a partial tile in the same bucket: one ballot per bit of bp
    same_b = __builtin_amdgcn_ballot_w64(rem > 0);
#pragma unroll
    for (int bit = 0; (1 << bit) < kSub; ++bit) {
      const bool on = (bp >> bit) & 1;
      const uint64_t m = __builtin_amdgcn_ballot_w64(on);
      same_b &= on ? m : ~m;
    }
    // the first such lane records the bucket's count in this wave (pw starts at zero)
    if (rem > 0 && (same_b & lanes_below()) == 0) reinterpret_cast<int*>(&pw[bp])[wave] = (int)__popcll(same_b);
  }
  int fbw = 0;  // full tiles of the lanes below in this wave (launch order only)
  if (order) {
    // one ballot per bit of the full-tile count (at most ceil(T / LR))
    int wtot = 0;
    for (int bit = 0; (1 << bit) <= (T + LR - 1) / LR; ++bit) {
      const uint64_t m = __builtin_amdgcn_ballot_w64((nfull >> bit) & 1);
      fbw += (int)__popcll(m & lanes_below()) << bit;
      wtot += (int)__popcll(m) << bit;
    }
    if (lane == 0) wfull[wave] = wtot;
  }
  __syncthreads();
  int bc = 0, bt = 0;
  for (int w = 0; w < wave; ++w) {
    bc += wsum[w][0];
    bt += wsum[w][1];
  }
  const int off = bc + ic - run;
  const int tst = bt + it - nt;
  before_s[e] = before;
  off_s[e] = off;
  if (g == 0) {
    if (e < E) {
      out.counts[e] = run;
      out.offsets[e] = off;
      for (int i = 0; i < nt; ++i) {
        int32_t* bm = out.block_map + 4 * (tst + i);
        bm[0] = e;
        bm[1] = off + i * BM;
        bm[2] = min(BM, run - i * BM);
        bm[3] = 0;
      }
    }
    if (e == MOE_MAX_EXPERTS - 1) {
      // totals over all lanes (lanes >= E contribute 0)
      const int R = bc + ic;
      const int tiles = bt + it;
      const int nsh = has_shared ? (T + BM - 1) / BM : 0;
      out.offsets[E] = R;
      *out.n_tiles = tiles + nsh;
      for (int i = 0; i < nsh; ++i) {
        int32_t* bm = out.block_map + 4 * (tiles + i);
        bm[0] = E;
        bm[1] = R + i * BM;
        bm[2] = min(BM, T - i * BM);
        bm[3] = 0;
      }
    }
  }
  // ---- launch order, part 2: every tile's place, stored with the block map ----
  // (with pieces, a full tile is a full piece of LR rows)
  // bucket 0 (16 subtiles): the experts' full tiles in expert order, the
  // shared expert's full tiles, then the partial tiles of 16 subtiles;
  // buckets 1.. : partial tiles in expert order, the shared expert's last
  if (order) {
    int fb = 0, ftot = 0;  // full tiles of the experts in earlier waves, and of all
#pragma unroll
    for (int w = 0; w < MOE_MAX_EXPERTS / 64; ++w) {
      const int v = wfull[w];
      fb += w < wave ? v : 0;
      ftot += v;
    }
    const int sfull = has_shared ? T / LR : 0;
    const int srem = has_shared ? T - sfull * LR : 0;
    const int sb = kSub - ((srem + 15) >> 4);  // bucket of the shared expert's partial tile
    // lane q of each 16-lane row: bucket q (routed partial tiles nq, those of
    // earlier waves bq); a scan over the row gives the bucket's first place
    // (bucket 0 opens with every full tile), then each thread reads its own
    const int q = lane & (kSub - 1);
    const int4 cq = pw[q];
    const int nq = cq.x + cq.y + cq.z + cq.w;
    const int bq = (wave > 0 ? cq.x : 0) + (wave > 1 ? cq.y : 0) + (wave > 2 ? cq.z : 0);
    const int sz = nq + (srem > 0 && sb == q ? 1 : 0);
    int inc = sz;
#pragma unroll
    for (int o = 1; o < kSub; o <<= 1) {
      const int v = __shfl_up(inc, o, kSub);
      if (q >= o) inc += v;
    }
    const int startq = ftot + sfull + inc - sz;
    const int st_p = __shfl(startq, bp & (kSub - 1)), bw = __shfl(bq, bp & (kSub - 1));
    const int st_s = __shfl(startq, sb & (kSub - 1)), nb_s = __shfl(nq, sb & (kSub - 1));
    const int ntot = ftot + sfull + __shfl(inc, kSub - 1);  // every tile or piece (lane 15 holds the buckets' total)
    if (e == 0 && n_launch) *n_launch = ntot;
    const int f0 = fb + fbw;  // place of this expert's first full tile
    for (int i = 0; i < nfull; ++i)
      *reinterpret_cast<int4*>(lmap + 4 * (f0 + i)) = int4{e, off + i * LR, LR, 0};
    if (rem > 0) {
      const int pos = st_p + bw + (int)__popcll(same_b & lanes_below());
      *reinterpret_cast<int4*>(lmap + 4 * pos) = int4{e, off + nfull * LR, rem, 0};
    }
    if (e == MOE_MAX_EXPERTS - 1 && has_shared) {
      const int R = bc + ic;  // total routed rows: the last thread's inclusive scan
      for (int i = 0; i < sfull; ++i)
        *reinterpret_cast<int4*>(lmap + 4 * (ftot + i)) = int4{E, R + i * LR, LR, 0};
      if (srem > 0) *reinterpret_cast<int4*>(lmap + 4 * (st_s + nb_s)) = int4{E, R + sfull * LR, srem, 0};
    }
  }
  // ---- scatter of this group's rows -------------------------------------------
#pragma unroll
  for (int j = 0; j < kSlotsPerWave; ++j)
    if (my[j] >= 0) atomicOr(&mask[my[j]], 1ull << lane);
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kSlotsPerWave; ++j) {
    const int x = my[j];
    if (x >= 0) {
      const int k = wave + 4 * j;
      const int rank = __popcll(mask[x] & lanes_below());
      const int p = off_s[x] + before_s[x] + rank;
      out.sorted_idx[p] = t * K + k;
      out.inv_pos[(size_t)t * K + k] = p;
    }
  }
}

namespace {
size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }
struct RouteWs {
  size_t hist, wn, wt, alog, total;
};
// expert-histogram row length: 64-token groups rounded up to 4
int hist_row(int T) { return ((T + kHistTokens - 1) / kHistTokens + 3) & ~3; }
// splits of the hidden axis for the approximate logits: as many as keep the
// grid at or below one workgroup per CU (at most 8, each a whole number of
// 64-column stages), so short prompts fill the chip
int logit_splits(int T, int H, int E) {
  const int ntb = (T + kLgTile - 1) / kLgTile, neb = (E + kLgTile - 1) / kLgTile;
  const int base = (ntb + 7) / 8 * 8 * neb;
  int ns = 1;
  while (ns < kMaxLogitSplits && base * ns * 2 <= 256 && (H / kLgK) % (ns * 2) == 0) ns *= 2;
  return ns;
}
RouteWs route_ws_layout(int T, int H, int E) {
  const size_t ng = (size_t)hist_row(T);
  RouteWs L;
  L.hist = 0;                                                     // expert histograms [E][64-token groups]
  L.wn = align256(ng * (size_t)E * sizeof(int32_t));             // router row norms
  L.wt = L.wn + align256(MOE_MAX_EXPERTS * sizeof(float));        // piece-major router copy [H/8][E][8] bf16
  L.alog = L.wt + align256((size_t)E * H * sizeof(uint16_t));     // approximate logits [T][E]
  L.total = L.alog + align256((size_t)logit_splits(T, H, E) * T * E * sizeof(float));
  return L;
}
}  // namespace

size_t route_workspace_bytes(int T, int H, int E) { return route_ws_layout(T, H, E).total; }

hipError_t launch_route(const RouteArgs& a, void* ws, hipStream_t stream) {
  const int ng = (a.T + kHistTokens - 1) / kHistTokens, ngp = hist_row(a.T);
  const RouteWs L = route_ws_layout(a.T, a.H, a.E);
  char* base = reinterpret_cast<char*>(ws);
  int32_t* hist = reinterpret_cast<int32_t*>(base + L.hist);
  float* wn = reinterpret_cast<float*>(base + L.wn);
  uint16_t* wt = reinterpret_cast<uint16_t*>(base + L.wt);
  float* alog = reinterpret_cast<float*>(base + L.alog);
  const int ntb = (a.T + kLgTile - 1) / kLgTile, neb = (a.E + kLgTile - 1) / kLgTile;
  const int ns = logit_splits(a.T, a.H, a.E);
  hipLaunchKernelGGL(route_logits_kernel, dim3((ntb + 7) / 8 * 8 * neb * ns), dim3(256), 0, stream, a, ntb, neb, ns,
                     alog, wn, wt, hist, ngp * a.E);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const dim3 sel_grid((a.T + kSelTokens - 1) / kSelTokens);
  switch (ns) {
    case 1: hipLaunchKernelGGL(route_select_kernel<1>, sel_grid, dim3(256), 0, stream, a, alog, wn, wt, hist, ngp); break;
    case 2: hipLaunchKernelGGL(route_select_kernel<2>, sel_grid, dim3(256), 0, stream, a, alog, wn, wt, hist, ngp); break;
    case 4: hipLaunchKernelGGL(route_select_kernel<4>, sel_grid, dim3(256), 0, stream, a, alog, wn, wt, hist, ngp); break;
    default: hipLaunchKernelGGL(route_select_kernel<8>, sel_grid, dim3(256), 0, stream, a, alog, wn, wt, hist, ngp); break;
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(route_group_kernel, dim3(ng), dim3(MOE_MAX_EXPERTS), 0, stream, hist, ngp, a.T, a.K, a.E,
                     a.has_shared, a.out, a.launch_map, a.n_launch, a.launch_rows);
  return hipGetLastError();
}

}  // namespace moeq4
