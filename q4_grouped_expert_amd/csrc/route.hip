// Routing kernels: router logits + top-k (one pass over x and the router
// weight), then histogram -> exclusive scan -> stable scatter -> tile block
// map, all on the device so the host never waits inside the layer
// ("Perplexity Lily 오픈소스 공개", alltoptrend.co.kr, section 5-2;
// "Apple silicon용 Lily, Qwen 추론 최적화", aitrends.kr, section
// "GPU 상주와 메모리 절감").
#include <math.h>

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
__device__ __forceinline__ rsrc_t rsrc_of(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, kRsrcFlags);
}
constexpr int kWChunk = 64;  // hidden columns of the router weight staged per LDS chunk
// 16-byte chunk swizzle of a 128-byte LDS row (rows are experts)
__device__ __forceinline__ int wswz(int row, int c) { return c ^ (row & 7); }
}  // namespace

__global__ __launch_bounds__(256) void route_topk_kernel(RouteArgs a, int32_t* __restrict__ hist,
                                                         const float* __restrict__ wn) {
  constexpr int TB = kRouteTokens;  // 16 tokens
  __shared__ __attribute__((aligned(16))) uint16_t xs[TB * MOE_MAX_REDUCTION];          // token rows, bf16
  __shared__ __attribute__((aligned(16))) uint16_t wsm[2][MOE_MAX_EXPERTS * kWChunk];   // router chunk ring
  __shared__ __attribute__((aligned(16))) float lv[TB][MOE_MAX_EXPERTS];  // approx logits, then exact values
  __shared__ short cand[TB][MOE_MAX_EXPERTS];
  __shared__ int ccount[TB];
  __shared__ float xnorm[TB];
  __shared__ float wmax_s;
  __shared__ int bhist[MOE_MAX_EXPERTS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 15, lg = lane >> 4;
  const int t0 = blockIdx.x * TB;
  const int T = a.T, H = a.H, E = a.E, K = a.K;
  const rsrc_t x_rs = rsrc_of(a.x, (uint32_t)T * H * 2u);
  const rsrc_t w_rs = rsrc_of(a.w_router, (uint32_t)E * H * 2u);

  bhist[tid] = 0;
  // ---- phase 0: stage the 16 token rows (bf16) and their 2-norms ----------
  {
    const int tt = tid >> 4, seg = tid & 15;
    float s2 = 0.0f;
    for (int h = 8 * seg; h < H; h += 128) {
      const u32x4 v = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(x_rs, (uint32_t)((t0 + tt) * H + h) * 2u, 0, 0));
      *reinterpret_cast<u32x4*>(&xs[tt * H + h]) = v;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float lo = bf16_bits_to_f32(v[q] & 0xFFFFu), hi = bf16_bits_to_f32(v[q] >> 16);
        s2 = __builtin_fmaf(lo, lo, s2);
        s2 = __builtin_fmaf(hi, hi, s2);
      }
    }
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) s2 += __shfl_xor(s2, o, 16);
    if (seg == 0) xnorm[tt] = sqrtf(s2);
    if (wave == 0) {
      float m = 0.0f;
      for (int e = lane; e < E; e += 64) m = fmaxf(m, wn[e]);
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
      if (lane == 0) wmax_s = m;
    }
  }

  // ---- phase 1: approximate logits on the matrix cores ---------------------
  // rows = the 16 tokens, columns = experts 64*wave + 16j + ln (j = 0..3)
  {
    f32x4 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint32_t xo = (uint32_t)((t0 + ln) * H + 8 * lg) * 2u;
    uint32_t wo[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) wo[j] = (uint32_t)((64 * wave + 16 * j + ln) * H + 8 * lg) * 2u;
#pragma unroll 8
    for (int k0 = 0; k0 < H; k0 += 32) {
      const bf16x8 av = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(x_rs, xo, k0 * 2, 0));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x8 bv = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(w_rs, wo[j], k0 * 2, 0));
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[j], 0, 0, 0);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 64 * wave + 16 * j + ln;
      const float rb = (a.router_bias && e < E) ? a.router_bias[e] : 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) lv[4 * lg + i][e] = e < E ? acc[j][i] + rb : -INFINITY;
    }
  }
  __syncthreads();

  // ---- phase 2: candidates per token (16 lanes per token) ------------------
  const int tok = 4 * wave + lg;  // this 16-lane group's token
  const bool tvalid = t0 + tok < T;
  {
    float v[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) v[q] = lv[tok][16 * ln + q];
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
      const float S = xnorm[tok] * wmax_s * 1.001f;
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

  // ---- phase 3: canonical chains for the candidates -------------------------
  // Router rows are streamed in 64-column chunks through an LDS ring (one
  // full cache line per row and chunk); every 16-lane group runs the chains
  // of its token's candidates, 16 at a time.
  int maxc = 0;
#pragma unroll
  for (int t = 0; t < TB; ++t) maxc = max(maxc, ccount[t]);
  const int C = ccount[tok];
  for (int base = 0; base < maxc; base += 16) {
    const int c = base + ln;
    const bool live = c < C;
    const int e = live ? cand[tok][c] : 0;
    float acc = 0.0f;
    // 256 rows x 128 B per chunk: lane -> row tid/8 + 32*i, 16-byte chunk tid%8.
    // The next chunk's loads go out before this chunk's chains and land in
    // LDS after them, so their latency hides under the arithmetic.
    u32x4 wreg[8];
    auto load_w = [&](int h0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = (tid >> 3) + 32 * i, ch = tid & 7;
        wreg[i] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(w_rs, (uint32_t)(r * H + h0 + 8 * ch) * 2u, 0, 0));
      }
    };
    auto store_w = [&](int buf) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = (tid >> 3) + 32 * i, ch = tid & 7;
        *reinterpret_cast<u32x4*>(&wsm[buf][r * kWChunk + wswz(r, ch) * 8]) = wreg[i];
      }
    };
    load_w(0);
    store_w(0);
    __syncthreads();
    for (int h0 = 0; h0 < H; h0 += kWChunk) {
      const int buf = (h0 / kWChunk) & 1;
      const bool more = h0 + kWChunk < H;
      if (more) load_w(h0 + kWChunk);
      if (live) {
#pragma unroll
        for (int ch = 0; ch < 8; ++ch) {
          const u32x4 xv = *reinterpret_cast<const u32x4*>(&xs[tok * H + h0 + 8 * ch]);
          const u32x4 wv = *reinterpret_cast<const u32x4*>(&wsm[buf][e * kWChunk + wswz(e, ch) * 8]);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc = __builtin_fmaf(bf16_bits_to_f32(xv[q] & 0xFFFFu), bf16_bits_to_f32(wv[q] & 0xFFFFu), acc);
            acc = __builtin_fmaf(bf16_bits_to_f32(xv[q] >> 16), bf16_bits_to_f32(wv[q] >> 16), acc);
          }
        }
      }
      if (more) store_w(buf ^ 1);
      __syncthreads();
    }
    if (live) lv[tok][c] = (a.router_bias ? acc + a.router_bias[e] : acc);
  }
  __syncthreads();

  // ---- phase 4: exact top-k among the candidates ----------------------------
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

size_t route_workspace_bytes(int T, int E) {
  const size_t nb = (size_t)(T + kRouteTokens - 1) / kRouteTokens;
  return nb * (size_t)E * sizeof(int32_t) + 256 * sizeof(float);  // block histograms + router row norms
}

hipError_t launch_route(const RouteArgs& a, void* ws, hipStream_t stream) {
  const int nb = (a.T + kRouteTokens - 1) / kRouteTokens;
  int32_t* hist = reinterpret_cast<int32_t*>(ws);
  float* wn = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + (size_t)nb * a.E * sizeof(int32_t));
  hipLaunchKernelGGL(route_wnorm_kernel, dim3(a.E), dim3(64), 0, stream, a.w_router, a.H, wn);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(route_topk_kernel, dim3(nb), dim3(256), 0, stream, a, hist, wn);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(MOE_MAX_EXPERTS), 0, stream, hist, nb, a.T, a.K, a.E,
                     a.has_shared, a.out);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(route_scatter_kernel, dim3(nb), dim3(64), 0, stream, hist, a.T, a.K, a.E, a.out);
  return hipGetLastError();
}

}  // namespace moeq4
