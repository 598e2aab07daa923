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
// ascending (+ bias[e] afterwards).  A bf16 x bf16 product is exact in fp32,
// so each fma below rounds exactly like "acc = acc + x*w"; every
// implementation that keeps this order gets bit-identical logits and hence
// bit-identical expert ids.  The work therefore runs on the fp32 VALU, one
// independent accumulation chain per (token, expert) pair.
//
// Workgroup: 256 lanes = 4 waves, 16 tokens.  Wave w owns tokens 4w..4w+3,
// lane l owns experts 4l..4l+3 (E <= 256), i.e. 16 chains per lane.  The
// router weight chunk [32 h][256 e] and the token chunk [32 h][16 t] are
// staged in LDS as fp32, transposed so a lane's 4 experts (or a wave's 4
// tokens) are one 16-byte LDS read.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void route_logits_topk_kernel(RouteArgs a) {
  __shared__ __attribute__((aligned(16))) float xs[kRouteChunk][kRouteTokens];
  __shared__ __attribute__((aligned(16))) float ws[kRouteChunk][MOE_MAX_EXPERTS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int t0 = blockIdx.x * kRouteTokens;
  const int T = a.T, H = a.H, E = a.E, K = a.K;

  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;

  for (int h0 = 0; h0 < H; h0 += kRouteChunk) {
    // router weight row e = tid, kRouteChunk bf16 (16 B per 8)
    if (tid < E) {
      const u32x4* src = reinterpret_cast<const u32x4*>(a.w_router + (size_t)tid * H + h0);
#pragma unroll
      for (int c = 0; c < kRouteChunk / 8; ++c) {
        u32x4 v = src[c];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          ws[c * 8 + 2 * q][tid] = bf16_bits_to_f32(v[q] & 0xFFFFu);
          ws[c * 8 + 2 * q + 1][tid] = bf16_bits_to_f32(v[q] >> 16);
        }
      }
    } else {
#pragma unroll
      for (int h = 0; h < kRouteChunk; ++h) ws[h][tid] = 0.0f;
    }
    // tokens: 16 x kRouteChunk bf16, 16 B per lane
    constexpr int kCh = kRouteChunk / 8;
    if (tid < kRouteTokens * kCh) {
      const int tt = tid / kCh, c = tid % kCh;
      const int t = t0 + tt;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (t < T) v = *reinterpret_cast<const u32x4*>(a.x + (size_t)t * H + h0 + 8 * c);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        xs[c * 8 + 2 * q][tt] = bf16_bits_to_f32(v[q] & 0xFFFFu);
        xs[c * 8 + 2 * q + 1][tt] = bf16_bits_to_f32(v[q] >> 16);
      }
    }
    __syncthreads();
#pragma unroll 8
    for (int h = 0; h < kRouteChunk; ++h) {
      const f32x4 xv = *reinterpret_cast<const f32x4*>(&xs[h][4 * wave]);
      const f32x4 wv = *reinterpret_cast<const f32x4*>(&ws[h][4 * lane]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(xv[i], wv[j], acc[i][j]);
    }
    __syncthreads();
  }

  float bias[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = 4 * lane + j;
    bias[j] = (a.router_bias && e < E) ? a.router_bias[e] : 0.0f;
  }

  // Top-k per token: K rounds of a wave-wide argmax (logit descending,
  // expert ascending on ties).  The chosen order is the slot order.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + 4 * wave + i;
    if (t >= T) continue;  // uniform across the wave
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * lane + j;
      v[j] = (e < E) ? (a.router_bias ? acc[i][j] + bias[j] : acc[i][j]) : -INFINITY;
    }
    uint32_t taken = 0;
    float sel_v[MOE_MAX_TOPK];
    int sel_e[MOE_MAX_TOPK];
#pragma unroll
    for (int k = 0; k < MOE_MAX_TOPK; ++k) {
      sel_v[k] = 0.0f;
      sel_e[k] = 0;
      if (k < K) {
        float bv = -INFINITY;
        int be = 0x7fffffff;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e = 4 * lane + j;
          if (e < E && !((taken >> j) & 1u)) {
            // the last clause keeps the pick a valid, untaken expert even if a
            // logit is NaN (non-finite inputs give unspecified, in-range ids)
            if (v[j] > bv || (v[j] == bv && e < be) || be == 0x7fffffff) {
              bv = v[j];
              be = e;
            }
          }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
          const float ov = __shfl_xor(bv, off);
          const int oe = __shfl_xor(be, off);
          if (oe != 0x7fffffff && (ov > bv || (ov == bv && oe < be) || be == 0x7fffffff)) {
            bv = ov;
            be = oe;
          }
        }
        if ((be >> 2) == lane) taken |= 1u << (be & 3);
        sel_v[k] = bv;
        sel_e[k] = be;
      }
    }
    const float m = sel_v[0];
    float den = 0.0f;
    if (a.norm_topk) {
#pragma unroll
      for (int k = 0; k < MOE_MAX_TOPK; ++k)
        if (k < K) den += expf(sel_v[k] - m);
    } else {
      float s = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (4 * lane + j < E) s += expf(v[j] - m);
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
      den = s;
    }
#pragma unroll
    for (int k = 0; k < MOE_MAX_TOPK; ++k) {
      if (k < K && lane == k) {
        a.out.topk_ids[(size_t)t * K + k] = sel_e[k];
        a.out.topk_w[(size_t)t * K + k] = expf(sel_v[k] - m) / den;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Grouping: histogram, exclusive scan, block map and a stable scatter, in one
// workgroup of 1024 lanes.
//
// Stability without ordered atomics: tokens are processed in passes of 1024;
// in a pass every expert gets a 1024-bit LDS mask of the tokens that chose it
// (a token's experts are distinct, so one bit per token suffices).  The rank
// of token t inside expert e's group is the popcount of e's mask below t,
// plus a running cursor carried across passes.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kGroupThreads) void route_group_kernel(const int32_t* __restrict__ ids, int T,
                                                                    int K, int E, int has_shared,
                                                                    moe_route_out out) {
  constexpr int kWords = kGroupThreads / 64;
  __shared__ int cnt[MOE_MAX_EXPERTS];
  __shared__ int off[MOE_MAX_EXPERTS + 1];
  __shared__ int tstart[MOE_MAX_EXPERTS + 1];
  __shared__ int cursor[MOE_MAX_EXPERTS];
  __shared__ unsigned long long bits[MOE_MAX_EXPERTS][kWords];

  const int tid = threadIdx.x;
  const int R = T * K;
  constexpr int BM = kTileRows;

  for (int e = tid; e < E; e += kGroupThreads) cnt[e] = 0;
  __syncthreads();
  // ids come from the router kernel and are always in [0, E); the clamp only
  // guarantees in-bounds indexing if that buffer were ever corrupted
  auto expert_of = [&](int e) { return (unsigned)e < (unsigned)E ? e : 0; };
  for (int r = tid; r < R; r += kGroupThreads) atomicAdd(&cnt[expert_of(ids[r])], 1);
  __syncthreads();

  if (tid < 64) {  // wave 0: scans of counts and of tiles per expert, 4 experts per lane
    int c[4], nt[4];
    int sc = 0, st = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * tid + j;
      c[j] = e < E ? cnt[e] : 0;
      nt[j] = (c[j] + BM - 1) / BM;
      sc += c[j];
      st += nt[j];
    }
    int isc = sc, ist = st;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(isc, o);
      const int w = __shfl_up(ist, o);
      if (tid >= o) {
        isc += v;
        ist += w;
      }
    }
    int ex = isc - sc, et = ist - st;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * tid + j;
      if (e < E) {
        off[e] = ex;
        tstart[e] = et;
      }
      ex += c[j];
      et += nt[j];
    }
    if (tid == 63) {
      off[E] = isc;
      tstart[E] = ist;
    }
  }
  __syncthreads();

  for (int e = tid; e < E; e += kGroupThreads) {
    out.counts[e] = cnt[e];
    out.offsets[e] = off[e];
    cursor[e] = off[e];
    const int nt = (cnt[e] + BM - 1) / BM;
    for (int i = 0; i < nt; ++i) {
      int32_t* b = out.block_map + 4 * (tstart[e] + i);
      b[0] = e;
      b[1] = off[e] + i * BM;
      b[2] = min(BM, cnt[e] - i * BM);
      b[3] = 0;
    }
  }
  const int nsh = has_shared ? (T + BM - 1) / BM : 0;
  for (int i = tid; i < nsh; i += kGroupThreads) {
    int32_t* b = out.block_map + 4 * (tstart[E] + i);
    b[0] = E;
    b[1] = R + i * BM;
    b[2] = min(BM, T - i * BM);
    b[3] = 0;
  }
  if (tid == 0) {
    out.offsets[E] = off[E];
    *out.n_tiles = tstart[E] + nsh;
  }
  __syncthreads();

  unsigned long long* flat = &bits[0][0];
  for (int c0 = 0; c0 < T; c0 += kGroupThreads) {
    for (int i = tid; i < E * kWords; i += kGroupThreads) flat[i] = 0ull;
    __syncthreads();
    const int t = c0 + tid;
    const bool valid = t < T;
    const int word = tid >> 6;
    const unsigned long long bit = 1ull << (tid & 63);
    int my[MOE_MAX_TOPK];
#pragma unroll
    for (int k = 0; k < MOE_MAX_TOPK; ++k) {
      my[k] = 0;
      if (valid && k < K) {
        my[k] = expert_of(ids[(size_t)t * K + k]);
        atomicOr(&bits[my[k]][word], bit);
      }
    }
    __syncthreads();
    if (valid) {
#pragma unroll
      for (int k = 0; k < MOE_MAX_TOPK; ++k) {
        if (k < K) {
          const int e = my[k];
          int rank = __popcll(bits[e][word] & (bit - 1ull));
          for (int w = 0; w < word; ++w) rank += __popcll(bits[e][w]);
          const int p = cursor[e] + rank;
          out.sorted_idx[p] = t * K + k;
          out.inv_pos[(size_t)t * K + k] = p;
        }
      }
    }
    __syncthreads();
    for (int e = tid; e < E; e += kGroupThreads) {
      int s = 0;
#pragma unroll
      for (int w = 0; w < kWords; ++w) s += __popcll(bits[e][w]);
      cursor[e] += s;
    }
    __syncthreads();
  }
}

hipError_t launch_route(const RouteArgs& a, hipStream_t stream) {
  const int nb = (a.T + kRouteTokens - 1) / kRouteTokens;
  hipLaunchKernelGGL(route_logits_topk_kernel, dim3(nb), dim3(256), 0, stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(route_group_kernel, dim3(1), dim3(kGroupThreads), 0, stream, a.out.topk_ids, a.T, a.K,
                     a.E, a.has_shared, a.out);
  return hipGetLastError();
}

}  // namespace moeq4
