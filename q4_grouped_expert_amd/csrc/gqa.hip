// Batch-1 decode attention with grouped KV heads (gfx950 / CDNA4).
//
// For query head h of G = HQ / HKV per KV head g = h / G:
//   s_j = scale * q_h . K_g[j],  p = softmax(s),  out_h = sum_j p_j V_g[j]
// over a KV cache in fixed blocks of 32 tokens (K token-major, V
// dimension-major inside a block).  The step is bound by reading the cache
// ("Perplexity Lily 오픈소스 공개", alltoptrend.co.kr, section 6-2; "Apple
// silicon용 Lily, Qwen 추론 최적화", aitrends.kr, section "Decode의 토큰 단위
// 최적화"), so:
//  * GQA packing: the G query heads of a KV head are the 16 columns of one
//    MFMA tile, so each K and V row is loaded once for all of them;
//  * the context is split over many waves (a few 32-token blocks each, about
//    1024 waves in all) and the partial softmax sums are merged, first
//    across the 4 waves of a workgroup in LDS, then across workgroups by a
//    second kernel (flash-decoding);
//  * QK^T: v_mfma_f32_16x16x32_bf16 with K rows as the A operand (16 tokens
//    x 32 dims, one 16-byte load per lane straight from the block) and the
//    queries as B.  MFMA row i of tile t is token 8(i/4) + 4t + i%4 of the
//    block, so the result leaves each lane with 8 consecutive tokens of one
//    head: exactly the B operand the PV product needs, with no data movement;
//  * PV: the dimension-major V block is the A operand (dims x 8 consecutive
//    tokens, one 16-byte load per lane) and the lane's own probabilities the
//    B operand, split into a bf16 high and low part (two MFMAs) so the
//    weights keep about 16 significant bits;
//  * the online softmax runs in the log2 domain with v_exp_f32; per head the
//    running max and sum need only two cross-lane shuffles per block.
#include <math.h>

#include "common.hpp"
#include "gqa_decode.h"

namespace moeq4 {
namespace {

constexpr int kGqaWaves = 4;
constexpr int kGqaThreads = 64 * kGqaWaves;
// context splits to aim for: about 4 waves per CU (measured against 2 and 16:
// fewer splits leave less to merge, more of them hide load latency better)
constexpr int kTargetWaves = 1024;
constexpr int kMaxGroup = 16;       // query heads per KV head: the 16 columns of an MFMA tile

struct GqaPlan {
  int nb;    // cache blocks in use
  int bpw;   // blocks per wave
  int wgs;   // workgroups per KV head
  int G;     // query heads per KV head
};

GqaPlan make_plan(const gqa_decode_desc& d) {
  GqaPlan p;
  p.G = d.HQ / d.HKV;
  p.nb = (d.L + GQA_BLOCK - 1) / GQA_BLOCK;
  const long total = (long)p.nb * d.HKV;
  p.bpw = (int)(total > kTargetWaves ? (total + kTargetWaves - 1) / kTargetWaves : 1);
  const int waves = (p.nb + p.bpw - 1) / p.bpw;
  p.wgs = (waves + kGqaWaves - 1) / kGqaWaves;
  return p;
}

struct GqaArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  float* out;
  float* pm;  // [parts][G] running max (log2 domain)
  float* pl;  // [parts][G] sum of weights
  float* po;  // [parts][G][D] weighted sum of values
  int L, HKV, G, nb, bpw, wgs;
  float scale_log2;  // scale * log2(e)
};

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }

template <int D>
__global__ __launch_bounds__(kGqaThreads, 2) void gqa_split_kernel(GqaArgs a) {
  constexpr int KS = D / 32;  // QK reduction steps
  constexpr int DT = D / 16;  // PV output tiles
  __shared__ float cm[kGqaWaves][kMaxGroup];
  __shared__ float cl[kGqaWaves][kMaxGroup];
  __shared__ __attribute__((aligned(16))) float co[kGqaWaves][kMaxGroup][D];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 15;  // B/D column: the head; A row: token or dim
  const int c = lane >> 4;  // k-group: dims 8c.. of a QK step, tokens 8c.. of a block
  const int g = blockIdx.x / a.wgs, w = blockIdx.x % a.wgs;
  const int G = a.G;
  const int blk0 = (w * kGqaWaves + wave) * a.bpw;
  const int blk1 = min(blk0 + a.bpw, a.nb);

  // queries of the group as the B operand of QK (columns past G are zero)
  u32x4 qop[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s)
    qop[s] = j < G ? ld16(a.q + ((size_t)(g * G + j) * D + 32 * s + 8 * c)) : u32x4{0u, 0u, 0u, 0u};

  f32x4 acc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;

  for (int blk = blk0; blk < blk1; ++blk) {
    const uint16_t* kb = a.k + ((size_t)blk * a.HKV + g) * GQA_BLOCK * D;
    const uint16_t* vb = a.v + ((size_t)blk * a.HKV + g) * D * GQA_BLOCK;
    u32x4 kop[2][KS];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int tok = 8 * (j >> 2) + 4 * tt + (j & 3);
#pragma unroll
      for (int s = 0; s < KS; ++s) kop[tt][s] = ld16(kb + (size_t)tok * D + 32 * s + 8 * c);
    }
    u32x4 vop[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t) vop[t] = ld16(vb + (size_t)(16 * t + j) * GQA_BLOCK + 8 * c);

    // scores: lane holds tokens 8c + 4tt + r of head j
    f32x4 sc[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      sc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kop[tt][0]),
                                                       __builtin_bit_cast(bf16x8, qop[0]),
                                                       f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
      for (int s = 1; s < KS; ++s)
        sc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kop[tt][s]),
                                                         __builtin_bit_cast(bf16x8, qop[s]), sc[tt], 0, 0, 0);
    }
    const int tok0 = blk * GQA_BLOCK + 8 * c;
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float sv = sc[e >> 2][e & 3] * a.scale_log2;
      x[e] = (tok0 + e < a.L) ? sv : -INFINITY;
    }
    float mb = x[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mb = fmaxf(mb, x[e]);
    mb = fmaxf(mb, __shfl_xor(mb, 16));
    mb = fmaxf(mb, __shfl_xor(mb, 32));
    const float m_new = fmaxf(m_run, mb);  // finite: every block holds a token below L
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float p[8], ps = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = __builtin_amdgcn_exp2f(x[e] - m_new);
      ps += p[e];
    }
    l_run = l_run * alpha + ps;
#pragma unroll
    for (int t = 0; t < DT; ++t) acc[t] *= alpha;
    bf16x8 ph, pl;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ph[e] = (__bf16)p[e];
      pl[e] = (__bf16)(p[e] - (float)ph[e]);
    }
    if (blk * GQA_BLOCK + GQA_BLOCK > a.L) {
      // entries past L in the last block may hold anything: zero them
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        const uint32_t keep = (tok0 + 2 * wd < a.L ? 0x0000ffffu : 0u) | (tok0 + 2 * wd + 1 < a.L ? 0xffff0000u : 0u);
#pragma unroll
        for (int t = 0; t < DT; ++t) vop[t][wd] &= keep;
      }
    }
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vop[t]), ph, acc[t], 0, 0, 0);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vop[t]), pl, acc[t], 0, 0, 0);
    }
    m_run = m_new;
  }

  // this wave's sums: head j, dims 16t + 4c + r
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (c == 0) {
    cm[wave][j] = m_run;
    cl[wave][j] = l_run;
  }
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) co[wave][j][16 * t + 4 * c + r] = acc[t][r];
  __syncthreads();

  // merge the 4 waves (a wave with no block has max -inf and weight 0;
  // wave 0 always has one)
  const size_t part = (size_t)g * a.wgs + w;
  for (int idx = threadIdx.x; idx < G * D; idx += kGqaThreads) {
    const int h = idx / D, d = idx % D;
    float M = cm[0][h];
#pragma unroll
    for (int wv = 1; wv < kGqaWaves; ++wv) M = fmaxf(M, cm[wv][h]);
    float o = 0.0f, l = 0.0f;
#pragma unroll
    for (int wv = 0; wv < kGqaWaves; ++wv) {
      const float f = __builtin_amdgcn_exp2f(cm[wv][h] - M);
      o += f * co[wv][h][d];
      l += f * cl[wv][h];
    }
    a.po[(part * G + h) * D + d] = o;
    if (d == 0) {
      a.pm[part * G + h] = M;
      a.pl[part * G + h] = l;
    }
  }
}

// out[h][d] = sum over the head's partials of 2^(m_p - M) o_p / the same sum
// of l_p.  Workgroup (h, slice) takes 64 dims of query head h.  No load
// waits for the maximum: every thread first loads its share of the partials'
// maxima and weights and the first kCombinePre partial outputs of its column
// (one round trip for up to 4 * kCombinePre partials), then M and the weight
// sum are reduced across lanes and waves, and each of the 4 waves sums every
// fourth partial of its 64 dims; longer lists continue with 8 loads in
// flight.  The 4 wave sums are added in wave order.
constexpr int kMaxParts = 1024;  // partials per head the combine holds in LDS
constexpr int kCombineDims = 64;
constexpr int kCombinePre = 32;  // partial outputs per thread loaded up front

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__global__ __launch_bounds__(256) void gqa_combine_kernel(GqaArgs a, int D) {
  constexpr int kPer = kMaxParts / 256;
  __shared__ float f[kMaxParts];
  __shared__ float wred[2][4];
  __shared__ float part_o[4][kCombineDims];
  const int nslice = D / kCombineDims;
  const int h = blockIdx.x / nslice, slice = blockIdx.x % nslice;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int G = a.G, g = h / G, hl = h % G;
  const int n = a.wgs;
  const float* pm = a.pm + (size_t)g * n * G + hl;
  const float* pl = a.pl + (size_t)g * n * G + hl;
  const int dd = t & (kCombineDims - 1), qq = t / kCombineDims;
  const int d = slice * kCombineDims + dd;
  const size_t stride = (size_t)G * D;
  const float* po = a.po + ((size_t)g * n * G + hl) * D + d;

  float mv[kPer], lv[kPer], pre[kCombinePre];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int w = t + 256 * i;
    mv[i] = w < n ? pm[(size_t)w * G] : -INFINITY;
    lv[i] = w < n ? pl[(size_t)w * G] : 0.0f;
  }
#pragma unroll
  for (int u = 0; u < kCombinePre; ++u) {
    const int w = qq + 4 * u;
    pre[u] = w < n ? po[(size_t)w * stride] : 0.0f;
  }

  float M = fmaxf(fmaxf(mv[0], mv[1]), fmaxf(mv[2], mv[3]));
  M = wave_max(M);
  if (lane == 0) wred[0][wave] = M;
  __syncthreads();
  M = fmaxf(fmaxf(wred[0][0], wred[0][1]), fmaxf(wred[0][2], wred[0][3]));
  float l = 0.0f;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int w = t + 256 * i;
    if (w < n) {
      const float fw = __builtin_amdgcn_exp2f(mv[i] - M);
      f[w] = fw;
      l += fw * lv[i];
    }
  }
  l = wave_sum(l);
  if (lane == 0) wred[1][wave] = l;
  __syncthreads();
  l = (wred[1][0] + wred[1][1]) + (wred[1][2] + wred[1][3]);

  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < kCombinePre; ++u) {
    const int w = qq + 4 * u;
    if (w < n) o[u % 8] += f[w] * pre[u];
  }
  int w = qq + 4 * kCombinePre;
  for (; w + 28 < n; w += 32) {
#pragma unroll
    for (int u = 0; u < 8; ++u) o[u] += f[w + 4 * u] * po[(size_t)(w + 4 * u) * stride];
  }
  for (; w < n; w += 4) o[((w - qq) / 4) % 8] += f[w] * po[(size_t)w * stride];
  part_o[qq][dd] = ((o[0] + o[1]) + (o[2] + o[3])) + ((o[4] + o[5]) + (o[6] + o[7]));
  __syncthreads();
  if (qq == 0)
    a.out[(size_t)h * D + d] =
        n > 0 ? ((part_o[0][dd] + part_o[1][dd]) + (part_o[2][dd] + part_o[3][dd])) / l : 0.0f;
}

inline bool misaligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

int check_desc(const gqa_decode_desc* d) {
  if (!d) return MOE_ERR_INVALID_ARGUMENT;
  if (d->L < 0 || d->HQ <= 0 || d->HKV <= 0 || d->D <= 0) return MOE_ERR_INVALID_ARGUMENT;
  if (d->HQ % d->HKV != 0 || d->HQ / d->HKV > kMaxGroup || (d->D != 128 && d->D != 256))
    return MOE_ERR_UNSUPPORTED_SHAPE;
  return MOE_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace
}  // namespace moeq4

extern "C" int gqa_decode_workspace_size(const gqa_decode_desc* d, size_t* bytes) {
  using namespace moeq4;
  const int rc = check_desc(d);
  if (rc != MOE_OK) return rc;
  if (!bytes) return MOE_ERR_INVALID_ARGUMENT;
  const GqaPlan p = make_plan(*d);
  const size_t parts = (size_t)p.wgs * d->HKV;
  *bytes = 2 * align256(parts * p.G * sizeof(float)) + align256(parts * p.G * (size_t)d->D * sizeof(float));
  return MOE_OK;
}

extern "C" int gqa_decode_attention(const gqa_decode_desc* d, const uint16_t* q, const uint16_t* k_cache,
                                    const uint16_t* v_cache, float* out, void* ws, size_t ws_bytes, void* stream) {
  using namespace moeq4;
  int rc = check_desc(d);
  if (rc != MOE_OK) return rc;
  if (!q || !out || (d->L > 0 && (!k_cache || !v_cache || !ws))) return MOE_ERR_INVALID_ARGUMENT;
  if (misaligned16(q) || misaligned16(out) ||
      (d->L > 0 && (misaligned16(k_cache) || misaligned16(v_cache) || misaligned16(ws))))
    return MOE_ERR_MISALIGNED;
  size_t need = 0;
  gqa_decode_workspace_size(d, &need);
  if (d->L > 0 && ws_bytes < need) return MOE_ERR_WORKSPACE_TOO_SMALL;
  const GqaPlan p = make_plan(*d);
  if (p.wgs > kMaxParts) return MOE_ERR_UNSUPPORTED_SHAPE;
  const size_t parts = (size_t)p.wgs * d->HKV;
  char* wsb = static_cast<char*>(ws);
  GqaArgs a;
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.out = out;
  a.pm = d->L > 0 ? reinterpret_cast<float*>(wsb) : nullptr;
  a.pl = d->L > 0 ? reinterpret_cast<float*>(wsb + align256(parts * p.G * sizeof(float))) : nullptr;
  a.po = d->L > 0 ? reinterpret_cast<float*>(wsb + 2 * align256(parts * p.G * sizeof(float))) : nullptr;
  a.L = d->L;
  a.HKV = d->HKV;
  a.G = p.G;
  a.nb = p.nb;
  a.bpw = p.bpw;
  a.wgs = p.wgs;
  a.scale_log2 = d->scale * 1.4426950408889634f;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (p.wgs > 0) {
    const dim3 grid((unsigned)(p.wgs * d->HKV));
    if (d->D == 256) hipLaunchKernelGGL(gqa_split_kernel<256>, grid, dim3(kGqaThreads), 0, s, a);
    else hipLaunchKernelGGL(gqa_split_kernel<128>, grid, dim3(kGqaThreads), 0, s, a);
  }
  hipLaunchKernelGGL(gqa_combine_kernel, dim3(d->HQ * (d->D / kCombineDims)), dim3(256), 0, s, a, (int)d->D);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}
