// Routing kernels: router logits + top-k (one pass over x and the router
// weight), then histogram -> exclusive scan -> stable scatter -> tile block
// map, all on the device so the host never waits inside the layer
// ("Perplexity Lily 오픈소스 공개", alltoptrend.co.kr, section 5-2;
// "Apple silicon용 Lily, Qwen 추론 최적화", aitrends.kr, section
// "GPU 상주와 메모리 절감").
#include <math.h>

#include <type_traits>

#include "common.hpp"

namespace moeq4 {

// ---------------------------------------------------------------------------
// Router logits and top-k.
//
// Logit contract: l[t,e] = sum_h x[t,h] * Wr[e,h] in fp32 with h strictly
// ascending, then + bias[e].  A bf16 x bf16 product is exact in fp32, so an
// fma chain in that order rounds exactly like "acc = acc + x*w"; every
// implementation that keeps the order gets bit-identical logits and hence
// bit-identical expert ids.
//
// Computing all T*E chains on the fp32 VALU costs 2*T*H*E flops.  Instead:
//  1. approximate logits a[t,e] with bf16 MFMA (fp32 accumulation, any
//     internal order);
//  2. bound both errors: |a - exact| <= da and |canonical - exact| <= dc,
//     with sum_h |x w| <= ||x_t|| * max_e ||w_e|| (Cauchy-Schwarz),
//     da = 34 (H/32 + 1) 2^-23 S  (each 32-product MFMA step off by at most
//     33 fp32 ulps of its inputs, for any summation order or truncation),
//     dc = (H + 2) 2^-24 S  (sequential fp32 summation);
//  3. with tau = the K-th largest a[t,.], every expert outside
//     {e : a[t,e] >= tau - 2 (da + dc)} has a canonical logit strictly below
//     the K-th largest canonical logit, so it cannot be selected;
//  4. recompute the canonical chains for the candidates only (about K+2 per
//     token) and select the top-k among them exactly.
// The result equals the full canonical computation, ties included.  When
// softmax weights run over all E experts (norm_topk = 0) every expert is a
// candidate.
// ---------------------------------------------------------------------------

// ||w_e||_2 of every router row, one wave per expert.
__global__ __launch_bounds__(64) void route_wnorm_kernel(const uint16_t* __restrict__ wr, int H, float* wn) {
  const int e = blockIdx.x, lane = threadIdx.x;
  float s = 0.0f;
  for (int h = 8 * lane; h < H; h += 512) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(wr + (size_t)e * H + h);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float lo = bf16_bits_to_f32(v[q] & 0xFFFFu), hi = bf16_bits_to_f32(v[q] >> 16);
      s = __builtin_fmaf(lo, lo, s);
      s = __builtin_fmaf(hi, hi, s);
    }
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
constexpr int kXfPad = 4;    // fp32 padding per staged token row (bank spread)
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
// Selection: candidates from the approximate logits, canonical fp32 chains
// for the candidates only, exact top-k and combine weights, and this block's
// expert histogram.  One workgroup = 16 tokens, 16 lanes per token for the
// per-token steps; the chains of all 16 tokens are packed one per lane.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void route_select_kernel(RouteArgs a, const float* __restrict__ alog,
                                                           const float* __restrict__ wn,
                                                           int32_t* __restrict__ hist) {
  constexpr int TB = kRouteTokens;  // 16 tokens
  // token rows in fp32 (padded rows spread the chains' reads over the banks)
  __shared__ __attribute__((aligned(16))) float xf[TB * (MOE_MAX_REDUCTION + kXfPad)];
  __shared__ float lv[TB][MOE_MAX_EXPERTS];  // canonical values of the candidates
  __shared__ short cand[TB][MOE_MAX_EXPERTS];
  __shared__ int ccount[TB], cstart[TB + 1];
  __shared__ float wmax_s, xn_s[TB];
  __shared__ int bhist[MOE_MAX_EXPERTS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 15, lg = lane >> 4;
  const int t0 = blockIdx.x * TB;
  const int T = a.T, H = a.H, E = a.E, K = a.K;
  const int xstride = H + kXfPad;
  const rsrc_t x_rs = rsrc_of(a.x, (uint32_t)T * H * 2u);
  const rsrc_t w_rs = rsrc_of(a.w_router, (uint32_t)E * H * 2u);

  bhist[tid] = 0;
  // ---- token rows to fp32 in LDS, their norms; largest router-row norm ---
  // 16 lanes per token, 16-byte pieces 128 columns apart; each lane issues
  // up to 16 loads before it converts any, so a 2048-column row costs one
  // memory latency.
  {
    const int tt = tid >> 4, seg = tid & 15;
    const bool tv = t0 + tt < T;
    float s2 = 0.0f;
    for (int hb = 0; hb < H; hb += 2048) {
      u32x4 v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int h = hb + 128 * i + 8 * seg;
        const uint32_t off = tv && h < H ? (uint32_t)((t0 + tt) * H + h) * 2u : kOob;
        v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(x_rs, off, 0, 0));
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int h = hb + 128 * i + 8 * seg;
        if (h < H) {
          float f[8];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            f[2 * q] = bf16_bits_to_f32(v[i][q] & 0xFFFFu);
            f[2 * q + 1] = bf16_bits_to_f32(v[i][q] >> 16);
          }
#pragma unroll
          for (int q = 0; q < 8; ++q) s2 = __builtin_fmaf(f[q], f[q], s2);
          float4* dst = reinterpret_cast<float4*>(&xf[tt * xstride + h]);
          dst[0] = float4{f[0], f[1], f[2], f[3]};
          dst[1] = float4{f[4], f[5], f[6], f[7]};
        }
      }
    }
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) s2 += __shfl_xor(s2, o, 16);
    if (seg == 0) xn_s[tt] = sqrtf(s2);
    if (wave == 0) {
      float m = 0.0f;
      for (int e = lane; e < E; e += 64) m = fmaxf(m, wn[e]);
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
      if (lane == 0) wmax_s = m;
    }
  }
  __syncthreads();

  // ---- candidates per token (16 lanes per token) ------------------------
  const int tok = 4 * wave + lg;  // this 16-lane group's token
  const bool tvalid = t0 + tok < T;
  {
    float v[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int e = 16 * ln + q;
      v[q] = (tvalid && e < E) ? alog[(size_t)(t0 + tok) * E + e] : -INFINITY;
    }
    uint32_t taken = 0;
    float tau = -INFINITY;
    for (int k = 0; k < K; ++k) {
      float bv = -INFINITY;
      int bq = -1;
#pragma unroll
      for (int q = 0; q < 16; ++q)
        if (!((taken >> q) & 1u) && (bq < 0 || v[q] > bv)) {
          bv = v[q];
          bq = q;
        }
      float gv = bv;
      int gl = bq >= 0 ? ln : 16;
#pragma unroll
      for (int o = 8; o >= 1; o >>= 1) {
        const float ov = __shfl_xor(gv, o, 16);
        const int ol = __shfl_xor(gl, o, 16);
        if (ov > gv || (ov == gv && ol < gl)) {
          gv = ov;
          gl = ol;
        }
      }
      if (gl == ln && bq >= 0) taken |= 1u << bq;
      tau = gv;
    }
    float win;
    if (!a.norm_topk) {
      win = INFINITY;
    } else {
      const float S = xn_s[tok] * wmax_s * 1.001f;
      const float da = 34.0f * (float)(H / 32 + 1) * 0x1p-23f * S;
      const float dc = (float)(H + 2) * 0x1p-24f * S;
      win = 2.1f * (da + dc) + 0x1p-20f * (fabsf(tau) + 1.0f);
    }
    uint32_t m = 0;
#pragma unroll
    for (int q = 0; q < 16; ++q)
      if (16 * ln + q < E && v[q] >= tau - win) m |= 1u << q;
    const int cnt = __popc(m);
    int incl = cnt;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const int u = __shfl_up(incl, o, 16);
      if (ln >= o) incl += u;
    }
    int pos = incl - cnt;
#pragma unroll
    for (int q = 0; q < 16; ++q)
      if ((m >> q) & 1u) cand[tok][pos++] = (short)(16 * ln + q);
    if (ln == 15) ccount[tok] = tvalid ? incl : 0;
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int t = 0; t < TB; ++t) {
      cstart[t] = run;
      run += ccount[t];
    }
    cstart[TB] = run;
  }
  __syncthreads();

  // ---- canonical chains: l = sum_h x[t,h] w[e,h] in fp32, h ascending ------
  // Chain c of the block's list runs on thread c % 256 (batch c / 256); the
  // router row streams from L2 in 16-byte pieces P pieces ahead (P = 16, or
  // 8 where H is not a multiple of 128, since the unrolled body walks whole
  // groups of P pieces), the token row comes from LDS.  bf16 x bf16
  // products are exact in fp32, so each fma rounds exactly like
  // "acc = acc + x*w".
  const int npc = H / 8;
  auto chains = [&](auto depth) {
    constexpr int P = decltype(depth)::value;
    const int total = cstart[TB];
    for (int c = tid; c < ((total + 255) / 256) * 256; c += 256) {
      const bool live = c < total;
      int tk = 0;
#pragma unroll
      for (int t = 1; t < TB; ++t) tk += (live && c >= cstart[t]) ? 1 : 0;
      const int slot = c - cstart[tk];
      const int e = live ? cand[tk][slot] : 0;
      uint32_t wrow = live ? (uint32_t)e * H * 2u : kOob;
      const float* xr = &xf[tk * xstride];
      // first group in piece order (the loop's waits assume wb[i] was issued
      // i-th, on entry as on the back edge)
      u32x4 wb[P];
#pragma unroll
      for (int i = 0; i < P; ++i) {
        wb[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(w_rs, wrow, 16 * i, 0));
        __builtin_amdgcn_sched_barrier(0);
      }
      float acc = 0.0f;
      for (int p0 = 0; p0 < npc; p0 += P) {
        const int nxt = p0 + P < npc ? p0 + P : p0;  // the last group re-reads itself
#pragma unroll
        for (int i = 0; i < P; ++i) {
          const float4 x0 = *reinterpret_cast<const float4*>(&xr[8 * (p0 + i)]);
          const float4 x1 = *reinterpret_cast<const float4*>(&xr[8 * (p0 + i) + 4]);
          acc = chain8(acc, x0, x1, wb[i]);
          // Reload wb[i] only after its last use: the empty asm makes the
          // row offset depend on acc, so the scheduler cannot hoist the load
          // (a hoisted load needs a second register set, copied back behind
          // a full wait at the loop's back edge).
          asm("" : "+v"(wrow) : "v"(acc));
          wb[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(w_rs, wrow, 16 * (nxt + i), 0));
        }
      }
      if (live) lv[tk][slot] = a.router_bias ? acc + a.router_bias[e] : acc;
    }
  };
  if (npc % 16 == 0)
    chains(std::integral_constant<int, 16>{});
  else
    chains(std::integral_constant<int, 8>{});
  __syncthreads();
  const int C = ccount[tok];

  // ---- exact top-k among the candidates ----------------------------------
  if (tvalid) {
    const int t = t0 + tok;
    uint32_t taken = 0;  // bit r: candidate ln + 16 r taken
    float sel_v[MOE_MAX_TOPK];
    int sel_e[MOE_MAX_TOPK];
#pragma unroll
    for (int k = 0; k < MOE_MAX_TOPK; ++k) {
      sel_v[k] = 0.0f;
      sel_e[k] = 0;
      if (k < K) {
        float bv = -INFINITY;
        int be = 0x7fffffff, br = -1;
        for (int r = 0; ln + 16 * r < C; ++r) {
          if ((taken >> r) & 1u) continue;
          const int cc = ln + 16 * r;
          const float vv = lv[tok][cc];
          const int ee = cand[tok][cc];
          if (br < 0 || vv > bv || (vv == bv && ee < be)) {
            bv = vv;
            be = ee;
            br = r;
          }
        }
        float gv = bv;
        int ge = br >= 0 ? be : 0x7fffffff;
#pragma unroll
        for (int o = 8; o >= 1; o >>= 1) {
          const float ov = __shfl_xor(gv, o, 16);
          const int oe = __shfl_xor(ge, o, 16);
          if (oe != 0x7fffffff && (ov > gv || (ov == gv && oe < ge) || ge == 0x7fffffff)) {
            gv = ov;
            ge = oe;
          }
        }
        if (br >= 0 && be == ge) taken |= 1u << br;
        sel_v[k] = gv;
        sel_e[k] = ge;
      }
    }
    const float mx = sel_v[0];
    float den = 0.0f;
    if (a.norm_topk) {
#pragma unroll
      for (int k = 0; k < MOE_MAX_TOPK; ++k)
        if (k < K) den += expf(sel_v[k] - mx);
    } else {
      float s = 0.0f;
      for (int cc = ln; cc < C; cc += 16) s += expf(lv[tok][cc] - mx);
#pragma unroll
      for (int o = 8; o >= 1; o >>= 1) s += __shfl_xor(s, o, 16);
      den = s;
    }
#pragma unroll
    for (int k = 0; k < MOE_MAX_TOPK; ++k) {
      if (k < K && ln == k) {
        a.out.topk_ids[(size_t)t * K + k] = sel_e[k];
        a.out.topk_w[(size_t)t * K + k] = expf(sel_v[k] - mx) / den;
        atomicAdd(&bhist[sel_e[k]], 1);
      }
    }
  }
  __syncthreads();
  if (tid < E) hist[(size_t)blockIdx.x * E + tid] = bhist[tid];
}

// ---------------------------------------------------------------------------
// Exclusive scan of the expert histogram and the tile block map.
//
// hist[b][e] holds router workgroup b's count for expert e; it is rewritten
// in place into the exclusive prefix over b (the rows of e that earlier
// workgroups own), counts[e] is the total, offsets the exclusive scan over e
// and the block map lists each expert's tiles of at most kTileRows rows, then
// the shared expert's.  One workgroup, one lane per expert.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(MOE_MAX_EXPERTS) void route_scan_kernel(int32_t* __restrict__ hist, int nblk, int T,
                                                                     int K, int E, int has_shared,
                                                                     moe_route_out out) {
  __shared__ int wsum[MOE_MAX_EXPERTS / 64][2];
  const int e = threadIdx.x;
  const int lane = e & 63, wave = e >> 6;
  constexpr int BM = kTileRows;

  int run = 0;
  if (e < E) {
    int b = 0;
    for (; b + 8 <= nblk; b += 8) {
      int v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = hist[(size_t)(b + i) * E + e];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        hist[(size_t)(b + i) * E + e] = run;
        run += v[i];
      }
    }
    for (; b < nblk; ++b) {
      const int v = hist[(size_t)b * E + e];
      hist[(size_t)b * E + e] = run;
      run += v;
    }
  }
  const int nt = (run + BM - 1) / BM;
  // block-wide exclusive scans of counts and tile counts
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

// ---------------------------------------------------------------------------
// Stable scatter.  Router workgroup b's tokens land at
//   offsets[e] + (rows of e owned by workgroups < b) + (rank inside b),
// the rank being the number of earlier tokens of the same 16-token block that
// chose e (a 16-bit LDS mask per expert; a token's experts are distinct).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void route_scatter_kernel(const int32_t* __restrict__ hist, int T, int K, int E,
                                                           moe_route_out out) {
  __shared__ uint32_t mask[MOE_MAX_EXPERTS];
  const int lane = threadIdx.x;
  const int b = blockIdx.x;
  for (int e = lane; e < E; e += 64) mask[e] = 0u;
  __syncthreads();
  const int t = b * kRouteTokens + lane;
  const bool valid = lane < kRouteTokens && t < T;
  int my[MOE_MAX_TOPK];
#pragma unroll
  for (int k = 0; k < MOE_MAX_TOPK; ++k) {
    my[k] = 0;
    if (valid && k < K) {
      const int e = out.topk_ids[(size_t)t * K + k];
      my[k] = (unsigned)e < (unsigned)E ? e : 0;  // ids are produced in range; clamp keeps indexing safe
      atomicOr(&mask[my[k]], 1u << lane);
    }
  }
  __syncthreads();
  if (valid) {
#pragma unroll
    for (int k = 0; k < MOE_MAX_TOPK; ++k) {
      if (k < K) {
        const int e = my[k];
        const int rank = __popc(mask[e] & ((1u << lane) - 1u));
        const int p = out.offsets[e] + hist[(size_t)b * E + e] + rank;
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
RouteWs route_ws_layout(int T, int E) {
  const size_t nb = (size_t)(T + kRouteTokens - 1) / kRouteTokens;
  RouteWs L;
  L.hist = 0;                                                     // per-block expert histograms
  L.wn = align256(nb * (size_t)E * sizeof(int32_t));             // router row norms
  L.alog = L.wn + align256(MOE_MAX_EXPERTS * sizeof(float));      // approximate logits [T][E]
  L.total = L.alog + align256((size_t)T * E * sizeof(float));
  return L;
}
}  // namespace

size_t route_workspace_bytes(int T, int E) { return route_ws_layout(T, E).total; }

hipError_t launch_route(const RouteArgs& a, void* ws, hipStream_t stream) {
  const int nb = (a.T + kRouteTokens - 1) / kRouteTokens;
  const RouteWs L = route_ws_layout(a.T, a.E);
  char* base = reinterpret_cast<char*>(ws);
  int32_t* hist = reinterpret_cast<int32_t*>(base + L.hist);
  float* wn = reinterpret_cast<float*>(base + L.wn);
  float* alog = reinterpret_cast<float*>(base + L.alog);
  hipLaunchKernelGGL(route_wnorm_kernel, dim3(a.E), dim3(64), 0, stream, a.w_router, a.H, wn);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int ntb = (a.T + kLgTile - 1) / kLgTile, neb = (a.E + kLgTile - 1) / kLgTile;
  hipLaunchKernelGGL(route_logits_kernel, dim3((ntb + 7) / 8 * 8 * neb), dim3(256), 0, stream, a, ntb, neb, alog);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(route_select_kernel, dim3(nb), dim3(256), 0, stream, a, alog, wn, hist);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(MOE_MAX_EXPERTS), 0, stream, hist, nb, a.T, a.K, a.E,
                     a.has_shared, a.out);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(route_scatter_kernel, dim3(nb), dim3(64), 0, stream, hist, a.T, a.K, a.E, a.out);
  return hipGetLastError();
}

}  // namespace moeq4
