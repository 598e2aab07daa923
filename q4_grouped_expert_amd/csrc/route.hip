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
__global__ __launch_bounds__(256) void route_logits_topk_kernel(RouteArgs a, int32_t* __restrict__ hist) {
  __shared__ __attribute__((aligned(16))) float xs[2][kRouteChunk][kRouteTokens];
  __shared__ __attribute__((aligned(16))) float ws[2][kRouteChunk][MOE_MAX_EXPERTS];
  __shared__ int bhist[MOE_MAX_EXPERTS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int t0 = blockIdx.x * kRouteTokens;
  const int T = a.T, H = a.H, E = a.E, K = a.K;
  constexpr int kCh = kRouteChunk / 8;  // 16-byte pieces per row and chunk

  bhist[tid] = 0;

  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;

  // Chunk staging, one chunk ahead: router row e = tid (kCh x 16 B) and, for
  // lanes < 16*kCh, one 16-byte piece of a token row.
  u32x4 wreg[kCh];
  u32x4 xreg = {0u, 0u, 0u, 0u};
  const int xt = tid / kCh, xc = tid % kCh;
  const bool xlane = tid < kRouteTokens * kCh && t0 + xt < T;
  auto load_chunk = [&](int h0) {
    if (tid < E) {
      const u32x4* src = reinterpret_cast<const u32x4*>(a.w_router + (size_t)tid * H + h0);
#pragma unroll
      for (int c = 0; c < kCh; ++c) wreg[c] = src[c];
    }
    if (xlane) xreg = *reinterpret_cast<const u32x4*>(a.x + (size_t)(t0 + xt) * H + h0 + 8 * xc);
  };
  auto store_chunk = [&](int buf) {
#pragma unroll
    for (int c = 0; c < kCh; ++c) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t v = tid < E ? wreg[c][q] : 0u;
        ws[buf][c * 8 + 2 * q][tid] = bf16_bits_to_f32(v & 0xFFFFu);
        ws[buf][c * 8 + 2 * q + 1][tid] = bf16_bits_to_f32(v >> 16);
      }
    }
    if (tid < kRouteTokens * kCh) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        xs[buf][xc * 8 + 2 * q][xt] = bf16_bits_to_f32(xreg[q] & 0xFFFFu);
        xs[buf][xc * 8 + 2 * q + 1][xt] = bf16_bits_to_f32(xreg[q] >> 16);
      }
    }
  };
  auto compute = [&](int buf) {
#pragma unroll 8
    for (int h = 0; h < kRouteChunk; ++h) {
      const f32x4 xv = *reinterpret_cast<const f32x4*>(&xs[buf][h][4 * wave]);
      const f32x4 wv = *reinterpret_cast<const f32x4*>(&ws[buf][h][4 * lane]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(xv[i], wv[j], acc[i][j]);
    }
  };

  const int nch = H / kRouteChunk;
  load_chunk(0);
  store_chunk(0);
  __syncthreads();
  for (int c = 0; c < nch; c += 2) {
    if (c + 1 < nch) load_chunk((c + 1) * kRouteChunk);
    compute(0);
    if (c + 1 < nch) store_chunk(1);
    __syncthreads();
    if (c + 1 < nch) {
      if (c + 2 < nch) load_chunk((c + 2) * kRouteChunk);
      compute(1);
      if (c + 2 < nch) store_chunk(0);
      __syncthreads();
    }
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
        atomicAdd(&bhist[sel_e[k]], 1);
      }
    }
  }
  __syncthreads();
  // this workgroup's expert histogram (16 tokens)
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
  return nb * (size_t)E * sizeof(int32_t);
}

hipError_t launch_route(const RouteArgs& a, void* ws, hipStream_t stream) {
  const int nb = (a.T + kRouteTokens - 1) / kRouteTokens;
  int32_t* hist = reinterpret_cast<int32_t*>(ws);
  hipLaunchKernelGGL(route_logits_topk_kernel, dim3(nb), dim3(256), 0, stream, a, hist);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(MOE_MAX_EXPERTS), 0, stream, hist, nb, a.T, a.K, a.E,
                     a.has_shared, a.out);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(route_scatter_kernel, dim3(nb), dim3(64), 0, stream, hist, a.T, a.K, a.E, a.out);
  return hipGetLastError();
}

}  // namespace moeq4
