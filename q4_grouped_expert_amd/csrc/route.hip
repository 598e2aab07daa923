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
// Logit contract: l[t,e] is an fp32 sum in a fixed order.  The hidden axis
// splits into blocks of 64 columns; s_b = sum of x[t,h] * Wr[e,h] over block
// b in ascending h, from 0; l = s_0 + s_1 + ... in block order, from 0; then
// + bias[e].  A bf16 x bf16 product is exact in fp32, so an fma chain in that
// order rounds exactly like "s = s + x*w"; every implementation that keeps
// the order gets bit-identical logits and hence bit-identical expert ids.
//
// Computing all T*E logits on the fp32 VALU costs 2*T*H*E flops.  Instead:
//  1. approximate logits a[t,e] with bf16 MFMA (fp32 accumulation, any
//     internal order);
//  2. bound both errors: |a - exact| <= da and |canonical - exact| <= dc,
//     with sum_h |x w| <= ||x_t|| * max_e ||w_e|| =: S (Cauchy-Schwarz),
//     da = 34 (H/32 + 1) 2^-23 S  (each 32-product MFMA step off by at most
//     33 fp32 ulps of its inputs, for any summation order or truncation),
//     dc = (H + 2) 2^-24 S  (bounds any order of fp32 summation of H terms,
//     the blocked order included);
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
constexpr int kSelTokens = 4;    // tokens per selection workgroup (one wave each)
constexpr int kLogitBlock = 64;  // columns per block of the canonical logit order
}  // namespace

// ||w_e||_2 of every router row, one wave per expert; the workgroups also
// clear the expert histograms that the selection kernel accumulates into.
__global__ __launch_bounds__(64) void route_wnorm_kernel(const uint16_t* __restrict__ wr, int H, float* wn,
                                                         int32_t* __restrict__ hist, int hist_len) {
  const int e = blockIdx.x, lane = threadIdx.x;
  for (int i = e * 64 + lane; i < hist_len; i += gridDim.x * 64) hist[i] = 0;
  // H <= 2048: at most four 16-byte pieces per lane, all loaded before use
  u32x4 v[MOE_MAX_REDUCTION / 512];
#pragma unroll
  for (int i = 0; i < MOE_MAX_REDUCTION / 512; ++i) {
    const int h = 8 * lane + 512 * i;
    v[i] = h < H ? *reinterpret_cast<const u32x4*>(wr + (size_t)e * H + h) : u32x4{0u, 0u, 0u, 0u};
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < MOE_MAX_REDUCTION / 512; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float lo = bf16_bits_to_f32(v[i][q] & 0xFFFFu), hi = bf16_bits_to_f32(v[i][q] >> 16);
      s = __builtin_fmaf(lo, lo, s);
      s = __builtin_fmaf(hi, hi, s);
    }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
  if (lane == 0) wn[e] = sqrtf(s);
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
constexpr int kLgK = 64;     // hidden columns per stage
// s_waitcnt that bounds only the vector-memory counter (gfx9 encoding: vmcnt
// in bits 3:0 and 15:14; expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt has six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// s_waitcnt lgkmcnt(0) alone (vmcnt 63 and expcnt 7 leave those counters
// unconstrained).
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4)); }
// Order-preserving map of an fp32 value to uint32 (-0 is taken as +0 first,
// so equal values get equal keys) and its inverse.
__device__ __forceinline__ uint32_t fkey(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float fkey_inv(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
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
// and router rows stream through a 3-slot LDS ring of 64-column stages
// filled by direct-to-LDS loads two stages ahead.  Every MFMA adds a
// 32-product step to its fp32 accumulator, the structure the selection
// kernel's error bound assumes.
//
// Block order: consecutive workgroup ids land on consecutive XCDs, so id b
// takes token tile 8 (b / 8 / neb) + b % 8 and expert tile (b / 8) % neb:
// the neb workgroups that share a token tile run on one XCD and share its
// L2.  Ids past the last token tile exit at once.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void route_logits_kernel(RouteArgs a, int ntb, int neb, float* __restrict__ alog) {
  constexpr int kRows = 2 * kLgTile;            // token rows, then router rows
  constexpr int kSlot = kRows * kLgK;           // bf16 elements per ring slot
  __shared__ __attribute__((aligned(16))) uint16_t ring[3 * kSlot];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 15, lg = lane >> 4;
  const int q = blockIdx.x >> 3;
  const int tb = (q / neb) * 8 + (blockIdx.x & 7), eb = q % neb;
  if (tb >= ntb) return;
  const int t0 = tb * kLgTile, e0 = eb * kLgTile;
  const int T = a.T, H = a.H, E = a.E;
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
          kt * kLgK * 2, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          w_rs, (__attribute__((address_space(3))) void*)(S + (kLgTile + 16 * wave + 8 * i) * kLgK), 16, woff[i],
          kt * kLgK * 2, 0, 0);
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

  // Stage kt DMAs stage kt+2 into the slot read in stage kt-1 (free since
  // the last barrier), computes on slot kt%3, then waits until only its own
  // DMAs of this stage are in flight (so stage kt+1 has landed) and meets
  // the other waves at the barrier.  Past the last stage the DMAs repeat
  // the last one, keeping the count per stage fixed; no other vector-memory
  // access runs inside the loop, so the count is exact.
  const int nk = H / kLgK;
  const int last = nk - 1;
  dma(0, 0);
  dma(1, min(1, last));
  wait_vmcnt<kDmaPerStage>();
  __builtin_amdgcn_s_barrier();
  int kt = 0;
  for (; kt + 3 <= nk; kt += 3) {
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      dma((u + 2) % 3, min(kt + u + 2, last));
      stage(u);
      wait_vmcnt<kDmaPerStage>();
      __builtin_amdgcn_s_barrier();
    }
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    if (kt + u < nk) {
      dma((u + 2) % 3, min(kt + u + 2, last));
      stage(u);
      wait_vmcnt<kDmaPerStage>();
      __builtin_amdgcn_s_barrier();
    }
  }
  wait_vmcnt<0>();  // no direct-to-LDS write outlives the workgroup

  // approximate logits (+ bias); MFMA layout: lane holds rows 4*lg+i, column ln
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int e = e0 + 32 * wn + 16 * j + ln;
    if (e < E) {
      const float rb = a.router_bias ? a.router_bias[e] : 0.0f;
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = t0 + 32 * wm + 16 * m + 4 * lg + i;
          if (t < T) alog[(size_t)t * E + e] = acc[m][j][i] + rb;
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
}  // namespace

// ---------------------------------------------------------------------------
// Selection: candidates from the approximate logits, canonical logits for the
// candidates only, exact top-k, combine weights, expert histogram.
//
// One workgroup = 4 tokens; wave w owns token w in the per-token steps.  The
// canonical logits of all the workgroup's candidates are spread as pairs of
// chains over the waves: lane l of a pair computes block l % 32 of chain
// l / 32 (one block sum, a 64-step fma chain), the block sums meet in LDS
// and lane 0 of each half adds them in block order.  Token rows sit in LDS
// as fp32 with each block's 16-byte chunks rotated by the block index, so
// the 16 lanes of an LDS cycle read 16 different bank groups.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void route_select_kernel(RouteArgs a, const float* __restrict__ alog,
                                                           const float* __restrict__ wn,
                                                           int32_t* __restrict__ hist, int ngp) {
  constexpr int TB = kSelTokens;
  __shared__ __attribute__((aligned(16))) float xf[TB * MOE_MAX_REDUCTION];
  // canonical logits of the candidates as keys: fkey(logit) << 8 | 255 - e
  // (larger key = larger logit, then lower expert; E <= 256)
  __shared__ unsigned long long ck[TB][MOE_MAX_EXPERTS];
  __shared__ short cand[TB][MOE_MAX_EXPERTS];
  // block sums of a wave's last (up to) 4 chain pairs, [pair % 4][lane]
  __shared__ __attribute__((aligned(16))) float part[TB][4][64];
  __shared__ float selv[TB][MOE_MAX_TOPK];
  __shared__ int ccount[TB];
  __shared__ float wmax_s, xn_s[TB];
  __shared__ int bhist[MOE_MAX_EXPERTS];
  __shared__ float bias_s[MOE_MAX_EXPERTS];  // router bias (read in the chain loop without a global load)

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t0 = blockIdx.x * TB;
  const int T = a.T, H = a.H, E = a.E, K = a.K;
  const int nblk = H / kLogitBlock;
  const rsrc_t x_rs = rsrc_of(a.x, (uint32_t)T * H * 2u);
  const rsrc_t w_rs = rsrc_of(a.w_router, (uint32_t)E * H * 2u);
  // fp32 position of column h of token row r in LDS
  auto xpos = [&](int r, int h) {
    const int b = h >> 6, q = (h >> 2) & 15;
    return r * MOE_MAX_REDUCTION + 64 * b + 4 * (q ^ (b & 15));
  };

  bhist[tid] = 0;
  bias_s[tid] = a.router_bias && tid < E ? a.router_bias[tid] : 0.0f;
  const int t = t0 + wave;
  const bool tvalid = t < T;
  // approximate logits of token w, lane holding experts 4 lane .. 4 lane + 3
  // (loaded now so their latency overlaps the token row's)
  float av[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = 4 * lane + j;
    av[j] = tvalid && e < E ? alog[(size_t)t * E + e] : 0.0f;
  }
  // ---- token row of wave w to fp32 in LDS, its norm; largest router-row norm
  {
    const bool tv = tvalid;
    u32x4 v[MOE_MAX_REDUCTION / 512];
#pragma unroll
    for (int i = 0; i < MOE_MAX_REDUCTION / 512; ++i) {
      const int h = 8 * lane + 512 * i;
      const uint32_t off = tv && h < H ? ((uint32_t)t * H + h) * 2u : kOob;
      v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(x_rs, off, 0, 0));
    }
    float wv[MOE_MAX_EXPERTS / 64];
    if (wave == 0) {
#pragma unroll
      for (int i = 0; i < MOE_MAX_EXPERTS / 64; ++i) wv[i] = lane + 64 * i < E ? wn[lane + 64 * i] : 0.0f;
    }
    float s2 = 0.0f;
#pragma unroll
    for (int i = 0; i < MOE_MAX_REDUCTION / 512; ++i) {
      const int h = 8 * lane + 512 * i;
      if (h < H) {
        float f[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          f[2 * q] = bf16_bits_to_f32(v[i][q] & 0xFFFFu);
          f[2 * q + 1] = bf16_bits_to_f32(v[i][q] >> 16);
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) s2 = __builtin_fmaf(f[q], f[q], s2);
        *reinterpret_cast<float4*>(&xf[xpos(wave, h)]) = float4{f[0], f[1], f[2], f[3]};
        *reinterpret_cast<float4*>(&xf[xpos(wave, h + 4)]) = float4{f[4], f[5], f[6], f[7]};
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) s2 += __shfl_xor(s2, o);
    if (lane == 0) xn_s[wave] = sqrtf(s2);
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

  // ---- candidates of token w ---------------------------------------------
  {
    const float* v = av;
    uint32_t key[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) key[j] = tvalid && 4 * lane + j < E ? fkey(v[j]) >> 16 : 0u;
    // tau <= the K-th largest approximate logit: th = the largest 16-bit key
    // prefix with at least K keys at or above it, built bit by bit
    // (wave-uniform); th << 16 is at most the K-th largest key, and a lower
    // tau only widens the candidate set
    uint32_t th = 0;
    for (int bit = 15; bit >= 0; --bit) {
      const uint32_t c = th | (1u << bit);
      int n = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) n += __popcll(__ballot(key[j] >= c));
      if (n >= K) th = c;
    }
    const float tau = fkey_inv(th << 16);
    float win;
    if (!a.norm_topk) {
      win = INFINITY;
    } else {
      const float S = xn_s[wave] * wmax_s * 1.001f;
      const float da = 34.0f * (float)(H / 32 + 1) * 0x1p-23f * S;
      const float dc = (float)(H + 2) * 0x1p-24f * S;
      win = 2.1f * (da + dc) + 0x1p-20f * (fabsf(tau) + 1.0f);
    }
    // compact the candidates in expert order
    bool f[4];
    uint64_t bal[4];
    int below = 0, total = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f[j] = tvalid && 4 * lane + j < E && v[j] >= tau - win;
      bal[j] = __ballot(f[j]);
      below += __popcll(bal[j] & lanes_below());
      total += __popcll(bal[j]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (f[j]) cand[wave][below++] = (short)(4 * lane + j);
    if (lane == 0) ccount[wave] = total;
  }
  __syncthreads();

  // ---- canonical logits of all candidates, two chains per wave pass ------
  {
    int cst[TB + 1];
    cst[0] = 0;
#pragma unroll
    for (int i = 0; i < TB; ++i) cst[i + 1] = cst[i] + ccount[i];
    const int nchain = cst[TB];
    const int npair = (nchain + 1) / 2;
    const int half = lane >> 5, b = lane & 31;
    // chain c -> (token slot, expert); row offset of this lane's block, or
    // an offset that reads zeros
    auto locate = [&](int c, int& tk, int& slot, int& e) {
      tk = 0;
#pragma unroll
      for (int i = 1; i < TB; ++i) tk += c >= cst[i] ? 1 : 0;
      slot = c - cst[tk];
      e = cand[tk][slot];
    };
    auto row_off = [&](int p) -> uint32_t {
      const int c = 2 * p + half;
      if (p >= npair || c >= nchain || b >= nblk) return kOob;
      int tk, slot, e;
      locate(c, tk, slot, e);
      return ((uint32_t)e * H + kLogitBlock * b) * 2u;
    };
    auto load = [&](u32x4 (&w)[8], uint32_t off) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        w[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(w_rs, off, 16 * i, 0));
    };
    // block sum of pair p from this lane's router block w
    auto block_sum = [&](const u32x4 (&w)[8], int p) -> float {
      const int c = 2 * p + half;
      int tk = 0;
#pragma unroll
      for (int i = 1; i < TB; ++i) tk += c >= cst[i] ? 1 : 0;
      float sb = 0.0f;
      const float* xr = &xf[tk * MOE_MAX_REDUCTION + kLogitBlock * b];
      const int sw = b & 15;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float4 x0 = *reinterpret_cast<const float4*>(&xr[4 * ((2 * i) ^ sw)]);
        const float4 x1 = *reinterpret_cast<const float4*>(&xr[4 * ((2 * i + 1) ^ sw)]);
        sb = chain8(sb, x0, x1, w[i]);
      }
      return sb;
    };
    // Block sums go to LDS, one row of 64 per pair; after every 4th pair of
    // the wave (and after its last) lane j < 8 adds the block sums of chain
    // j of those pairs in block order, so the 32-add chains of 8 chains run
    // side by side.  p0 is the wave's first pair of the batch, n its size.
    auto combine = [&](int p0, int n) {
      __builtin_amdgcn_wave_barrier();
      const int j = lane;          // chain 2 (p0 + TB (j / 2)) + j % 2
      const int pj = p0 + TB * (j >> 1);
      const int c = 2 * pj + (j & 1);
      if (j < 2 * n && c < nchain) {
        int tk, slot, e;
        locate(c, tk, slot, e);
        const float* row = &part[wave][j >> 1][32 * (j & 1)];
        float ps[32];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float4 q = *reinterpret_cast<const float4*>(&row[4 * i]);
          ps[4 * i] = q.x;
          ps[4 * i + 1] = q.y;
          ps[4 * i + 2] = q.z;
          ps[4 * i + 3] = q.w;
        }
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < 32; ++i)
          if (i < nblk) acc = acc + ps[i];
        if (a.router_bias) acc = acc + bias_s[e];
        ck[tk][slot] = ((unsigned long long)fkey(acc) << 8) | (unsigned)(255 - e);
      }
      __builtin_amdgcn_wave_barrier();
    };
    u32x4 wa[8], wb[8];
    uint32_t offa = row_off(wave);
    load(wa, offa);
    int it = 0;  // pairs of this wave so far
    for (int p = wave; p < npair; p += 2 * TB) {
      uint32_t offb = row_off(p + TB);
      load(wb, offb);
      const float sa = block_sum(wa, p);
      // the reload of wa must follow its last use (else a second register
      // set and a full wait at the back edge): tie its offset to sa
      offa = row_off(p + 2 * TB);
      asm("" : "+v"(offa) : "v"(sa));
      load(wa, offa);
      part[wave][it & 3][lane] = sa;
      ++it;
      if (p + TB < npair) {
        part[wave][it & 3][lane] = block_sum(wb, p + TB);
        ++it;
      }
      if ((it & 3) == 0) combine(wave + TB * (it - 4), 4);
    }
    if (it & 3) combine(wave + TB * (it & ~3), it & 3);
  }
  __syncthreads();

  // ---- exact top-k of token w among its candidates -----------------------
  // A candidate's slot is the number of its token's candidates with a larger
  // key (keys are distinct); the K smallest slots are the selection, already
  // in slot order.
  if (tvalid) {
    const int C = ccount[wave];
    const unsigned long long* kw = ck[wave];
    unsigned long long mine[MOE_MAX_EXPERTS / 64];
    int rank[MOE_MAX_EXPERTS / 64];
#pragma unroll
    for (int r = 0; r < MOE_MAX_EXPERTS / 64; ++r) {
      const int c = lane + 64 * r;
      mine[r] = c < C ? kw[c] : 0ull;
      rank[r] = C;
      if (64 * r < C) {
        int n = 0;
#pragma unroll 4
        for (int o = 0; o < C; ++o) n += kw[o] > mine[r] ? 1 : 0;
        rank[r] = n;
        if (c < C && n < K) selv[wave][n] = fkey_inv((uint32_t)(mine[r] >> 8));
      }
    }
    __builtin_amdgcn_wave_barrier();
    const float mx = selv[wave][0];
    float den = 0.0f;
    if (a.norm_topk) {
      for (int k = 0; k < K; ++k) den += expf(selv[wave][k] - mx);
    } else {
      float sum = 0.0f;
#pragma unroll
      for (int r = 0; r < MOE_MAX_EXPERTS / 64; ++r)
        if (lane + 64 * r < C) sum += expf(fkey_inv((uint32_t)(mine[r] >> 8)) - mx);
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
      den = sum;
    }
#pragma unroll
    for (int r = 0; r < MOE_MAX_EXPERTS / 64; ++r) {
      if (lane + 64 * r < C && rank[r] < K) {
        const int e = 255 - (int)(mine[r] & 255ull);
        a.out.topk_ids[(size_t)t * K + rank[r]] = e;
        a.out.topk_w[(size_t)t * K + rank[r]] = expf(selv[wave][rank[r]] - mx) / den;
        atomicAdd(&bhist[e], 1);
      }
    }
  }
  __syncthreads();
  // this workgroup's tokens lie in one histogram group of kHistTokens;
  // hist is [E][ngp]
  if (tid < E && bhist[tid]) atomicAdd(&hist[(size_t)tid * ngp + t0 / kHistTokens], bhist[tid]);
}

// ---------------------------------------------------------------------------
// Group offsets, tile block map and stable scatter (sorted_idx / inv_pos).
//
// hist[e][g] holds the rows of expert e among the tokens of group g (64
// tokens each); rows are ngp = ng rounded up to 4 ints long.  One workgroup per group, one thread per expert: it sums its
// expert's row of hist into the total count and the rows that earlier groups
// own, a workgroup-wide exclusive scan of the totals gives the expert group
// offsets, and the first wave places the group's rows: a (t, k) row goes to
// offsets[e] + (rows of e in earlier groups) + (earlier tokens of this group
// that chose e, from a 64-bit LDS mask).  Workgroup 0 also writes counts,
// offsets and the block map (each expert's tiles of at most kTileRows rows,
// then the shared expert's).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(MOE_MAX_EXPERTS) void route_group_kernel(const int32_t* __restrict__ hist, int ngp,
                                                                      int T, int K, int E, int has_shared,
                                                                      moe_route_out out) {
  __shared__ int wsum[MOE_MAX_EXPERTS / 64][2];
  __shared__ int before_s[MOE_MAX_EXPERTS], off_s[MOE_MAX_EXPERTS];
  __shared__ unsigned long long mask[MOE_MAX_EXPERTS];
  const int e = threadIdx.x;
  const int lane = e & 63, wave = e >> 6;
  const int g = blockIdx.x;
  constexpr int BM = kTileRows;

  mask[e] = 0ull;
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
  // ---- scatter of this group's rows (first wave, one lane per token) ------
  const int t = g * kHistTokens + lane;
  const bool valid = wave == 0 && t < T;
  int my[MOE_MAX_TOPK];
#pragma unroll
  for (int k = 0; k < MOE_MAX_TOPK; ++k) {
    my[k] = 0;
    if (valid && k < K) {
      const int id = out.topk_ids[(size_t)t * K + k];
      my[k] = (unsigned)id < (unsigned)E ? id : 0;  // ids are produced in range; clamp keeps indexing safe
      atomicOr(&mask[my[k]], 1ull << lane);
    }
  }
  __syncthreads();
  if (valid) {
#pragma unroll
    for (int k = 0; k < MOE_MAX_TOPK; ++k) {
      if (k < K) {
        const int x = my[k];
        const int rank = __popcll(mask[x] & lanes_below());
        const int p = off_s[x] + before_s[x] + rank;
        out.sorted_idx[p] = t * K + k;
        out.inv_pos[(size_t)t * K + k] = p;
      }
    }
  }
}

namespace {
size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }
struct RouteWs {
  size_t hist, wn, alog, total;
};
// expert-histogram row length: 64-token groups rounded up to 4
int hist_row(int T) { return ((T + kHistTokens - 1) / kHistTokens + 3) & ~3; }
RouteWs route_ws_layout(int T, int E) {
  const size_t ng = (size_t)hist_row(T);
  RouteWs L;
  L.hist = 0;                                                     // expert histograms [E][64-token groups]
  L.wn = align256(ng * (size_t)E * sizeof(int32_t));             // router row norms
  L.alog = L.wn + align256(MOE_MAX_EXPERTS * sizeof(float));      // approximate logits [T][E]
  L.total = L.alog + align256((size_t)T * E * sizeof(float));
  return L;
}
}  // namespace

size_t route_workspace_bytes(int T, int E) { return route_ws_layout(T, E).total; }

hipError_t launch_route(const RouteArgs& a, void* ws, hipStream_t stream) {
  const int ng = (a.T + kHistTokens - 1) / kHistTokens, ngp = hist_row(a.T);
  const RouteWs L = route_ws_layout(a.T, a.E);
  char* base = reinterpret_cast<char*>(ws);
  int32_t* hist = reinterpret_cast<int32_t*>(base + L.hist);
  float* wn = reinterpret_cast<float*>(base + L.wn);
  float* alog = reinterpret_cast<float*>(base + L.alog);
  hipLaunchKernelGGL(route_wnorm_kernel, dim3(a.E), dim3(64), 0, stream, a.w_router, a.H, wn, hist, ngp * a.E);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int ntb = (a.T + kLgTile - 1) / kLgTile, neb = (a.E + kLgTile - 1) / kLgTile;
  hipLaunchKernelGGL(route_logits_kernel, dim3((ntb + 7) / 8 * 8 * neb), dim3(256), 0, stream, a, ntb, neb, alog);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(route_select_kernel, dim3((a.T + kSelTokens - 1) / kSelTokens), dim3(256), 0, stream, a, alog,
                     wn, hist, ngp);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(route_group_kernel, dim3(ng), dim3(MOE_MAX_EXPERTS), 0, stream, hist, ngp, a.T, a.K, a.E,
                     a.has_shared, a.out);
  return hipGetLastError();
}

}  // namespace moeq4
