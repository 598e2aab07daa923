// Decode-shape MoE layer: at most 16 tokens per call, the step after prefill
// on the same layer ("Perplexity Lily 오픈소스 공개", alltoptrend.co.kr,
// section 6: one token at a time, bound by the bytes moved per token;
// "Apple silicon용 Lily, Qwen 추론 최적화", aitrends.kr, section
// "Decode의 토큰 단위 최적화").  It computes exactly what the prefill layer
// computes (same routing rule, same bf16 weights, fp32 accumulation) and
// reads only the weights of the experts the tokens chose.
//
// gfx950 mapping
//  * Router: no candidate filter.  One wave per (token, 64 experts), one
//    lane per expert, each lane the exact sequential fp32 chain over the
//    hidden axis.  The router matrix is kept, once per model, as an fp32
//    piece-major copy wf[h/4][e][4], so the 64 lanes read 1 KB of
//    consecutive memory per step and need no bf16 unpack: four fma per
//    16-byte load, the pieces streamed 32 ahead in registers.  The token
//    row sits in LDS as fp32 and is read a group of pieces at a time.
//  * Top-k and grouping: one workgroup.  Wave t selects token t's experts by
//    K rounds of a wave-wide maximum over (logit, lower expert) keys and
//    forms the weights; then the workgroup builds counts, offsets, the stable
//    permutation and the block map (one tile per expert with rows, then the
//    shared expert) from the at most 256 (token, slot) pairs.
//  * Expert GEMVs: a workgroup of 8 waves owns one tile (<= 16 rows of one
//    expert) and 16 weight rows (gate/up: 16 gate rows and the matching 16
//    up rows; down: 32 output columns as two subtiles) and splits the
//    reduction into 8 contiguous ranges of 64-column quant groups, one per
//    wave.  Each wave dequantizes its part of the weights (fma(q, s, b) in
//    fp32, rounded to bf16) as the A operand of v_mfma_f32_16x16x32_bf16
//    with the tile's activation rows as the B operand; all of a wave's loads
//    are issued before the first MFMA.  The 8 partial 16x16 results are
//    added in wave order through LDS, so the result does not depend on
//    timing.
//  * Combine: the prefill combine kernel.
#include <math.h>

#include <type_traits>

#include "common.hpp"
#include "gemm_common.hpp"

namespace moeq4 {

namespace {
using namespace gemm;

constexpr int kDecWaves = 8;
constexpr int kDecThreads = 64 * kDecWaves;
constexpr int kDecMaxGroupsPerWave = MOE_MAX_REDUCTION / 64 / kDecWaves;  // 4

// Maximum of v over the 64 lanes of the wave, returned to every lane: DPP
// row shifts build each row's maximum in its lane 15, two row broadcasts
// carry them to lane 63 (the identity is 0, below every value used here).
template <int kCtrl, int kRowMask, int kBankMask>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kCtrl, kRowMask, kBankMask, false);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  uint32_t r = v;
  r = max(r, dpp_u32<0x111, 0xf, 0xf>(v));  // row_shr:1
  r = max(r, dpp_u32<0x112, 0xf, 0xf>(v));  // row_shr:2
  r = max(r, dpp_u32<0x113, 0xf, 0xf>(v));  // row_shr:3
  r = max(r, dpp_u32<0x114, 0xf, 0xe>(r));  // row_shr:4, banks 1-3
  r = max(r, dpp_u32<0x118, 0xf, 0xc>(r));  // row_shr:8, banks 2-3
  r = max(r, dpp_u32<0x142, 0xa, 0xf>(r));  // row_bcast:15 into rows 1 and 3
  r = max(r, dpp_u32<0x143, 0xc, 0xf>(r));  // row_bcast:31 into rows 2 and 3
  return (uint32_t)__builtin_amdgcn_readlane((int)r, 63);
}

// Order-preserving map of an fp32 value to uint32 (-0 taken as +0).
__device__ __forceinline__ uint32_t dec_fkey(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------------------
// wf[p][e][0..3] = Wr[e][4p .. 4p+3] as fp32 (p < H/4).  One wave per expert.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void decode_prep_kernel(const uint16_t* __restrict__ wr, int H, int E,
                                                         float* __restrict__ wf) {
  const int e = blockIdx.x;
  for (int p = threadIdx.x; p < H / 4; p += 64) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(wr + (size_t)e * H + 4 * p);
    const float4 f{bf16_bits_to_f32(v[0] & 0xFFFFu), bf16_bits_to_f32(v[0] >> 16), bf16_bits_to_f32(v[1] & 0xFFFFu),
                   bf16_bits_to_f32(v[1] >> 16)};
    *reinterpret_cast<float4*>(wf + ((size_t)p * E + e) * 4) = f;
  }
}

// ---------------------------------------------------------------------------
// Logits of 64 experts of one token per wave: l[e] = one fp32 chain over h
// in ascending order, then + bias.  Lanes past E run a copy of expert E-1's
// chain (every load stays in range) and store nothing.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void decode_logits_kernel(const uint16_t* __restrict__ x,
                                                           const float* __restrict__ wf,
                                                           const float* __restrict__ rb, int H, int E,
                                                           float* __restrict__ logits) {
  __shared__ __attribute__((aligned(16))) float xf[MOE_MAX_REDUCTION];
  const int neb = (E + 63) / 64;
  const int t = blockIdx.x / neb, eb = blockIdx.x - t * neb;
  const int lane = threadIdx.x;
  const int e = eb * 64 + lane;
  for (int h = 8 * lane; h < H; h += 512) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(x + (size_t)t * H + h);
    float4* dst = reinterpret_cast<float4*>(&xf[h]);
    dst[0] = float4{bf16_bits_to_f32(v[0] & 0xFFFFu), bf16_bits_to_f32(v[0] >> 16), bf16_bits_to_f32(v[1] & 0xFFFFu),
                    bf16_bits_to_f32(v[1] >> 16)};
    dst[1] = float4{bf16_bits_to_f32(v[2] & 0xFFFFu), bf16_bits_to_f32(v[2] >> 16), bf16_bits_to_f32(v[3] & 0xFFFFu),
                    bf16_bits_to_f32(v[3] >> 16)};
  }
  __syncthreads();
  // Router pieces of 4 columns (np = H/4, a multiple of 16) stream P ahead in
  // registers (32 when np allows, else 16).  The chain is bound by the
  // latency of 2048 dependent fma (measured about 14 clocks each on gfx950,
  // with nothing independent to issue between them); deeper prefetch does
  // not shorten it.  The last group re-reads itself so the loop has no
  // conditions.  The token row sits in LDS as fp32
  // (the same address for every lane: a broadcast read), 16 pieces of it
  // read ahead of their fma.  bf16 x bf16 products are exact in fp32, so each fma rounds
  // exactly like acc = acc + x*w.
  const int np = H / 4;
  const int ec = e < E ? e : E - 1;
  const float* col = wf + (size_t)ec * 4;
  const size_t pstride = (size_t)E * 4;
  auto chain = [&](auto depth) {
    constexpr int P = decltype(depth)::value;
    float4 wb[P];
#pragma unroll
    for (int i = 0; i < P; ++i) {
      wb[i] = *reinterpret_cast<const float4*>(col + i * pstride);
      __builtin_amdgcn_sched_barrier(0);  // keep every load at its place: P in flight
    }
    float acc = 0.0f;
    for (int p0 = 0; p0 < np; p0 += P) {
      const int nxt = p0 + P < np ? p0 + P : p0;
      float4 xv[16];
#pragma unroll
      for (int i = 0; i < P; ++i) {
        if (i % 16 == 0) {
          // the token row for the next 16 pieces, read before their first fma
#pragma unroll
          for (int u = 0; u < 16; ++u) xv[u] = *reinterpret_cast<const float4*>(&xf[4 * (p0 + i + u)]);
          __builtin_amdgcn_sched_barrier(0);
        }
        acc = __builtin_fmaf(xv[i % 16].x, wb[i].x, acc);
        acc = __builtin_fmaf(xv[i % 16].y, wb[i].y, acc);
        acc = __builtin_fmaf(xv[i % 16].z, wb[i].z, acc);
        acc = __builtin_fmaf(xv[i % 16].w, wb[i].w, acc);
        // reload wb[i] only after its last use (the empty asm ties the
        // address to acc, so the load cannot be hoisted into a second
        // register set)
        const float* src = col + (size_t)(nxt + i) * pstride;
        asm("" : "+v"(src) : "v"(acc));
        wb[i] = *reinterpret_cast<const float4*>(src);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    return acc;
  };
  const float acc = np % 32 == 0 ? chain(std::integral_constant<int, 32>{}) : chain(std::integral_constant<int, 16>{});
  if (e < E) logits[(size_t)t * E + e] = rb ? acc + rb[e] : acc;
}

// ---------------------------------------------------------------------------
// Top-k, weights and grouping for at most 16 tokens in one workgroup.
//
// Wave t (token t) holds experts 4 l .. 4 l + 3 in lane l as keys
// fkey(logit) << 8 | 255 - e (larger = larger logit, then lower expert) and
// takes K rounds of a wave-wide maximum, each removing the winner: the
// winners in order are the slots.  Weights: exp(l - l_max) over the sum of
// exp(l - l_max) of the selection (norm_topk) or of every expert, the sums
// in a fixed lane tree.  Then, for the at most 256 (token, slot) pairs:
// counts, offsets, stable sorted_idx / inv_pos, the block map (one tile per
// expert with rows, in expert order, then the shared expert's) and n_tiles.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void decode_group_kernel(const float* __restrict__ logits, int T, int K, int E,
                                                            int norm_topk, int has_shared, moe_route_out out) {
  __shared__ int sid[MOE_MAX_EXPERTS];
  __shared__ int wsum[MOE_MAX_EXPERTS / 64][2];
  __shared__ int off_s[MOE_MAX_EXPERTS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  if (wave < T) {
    const int t = wave;
    unsigned long long kq[4];
    float lv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = 4 * lane + q;
      lv[q] = e < E ? logits[(size_t)t * E + e] : 0.0f;
      kq[q] = e < E ? ((unsigned long long)dec_fkey(lv[q]) << 8) | (unsigned)(255 - e) : 0ull;
    }
    float mysel = 0.0f;  // lane k < K: the slot-k logit
    for (int k = 0; k < K; ++k) {
      // the wave's largest key: largest logit key, then among the lanes that
      // hold it the largest 255 - e (the lowest expert)
      unsigned long long lm = kq[0];
#pragma unroll
      for (int q = 1; q < 4; ++q) lm = kq[q] > lm ? kq[q] : lm;
      const uint32_t hi = wave_max_u32((uint32_t)(lm >> 8));
      const uint32_t lo = wave_max_u32((uint32_t)(lm >> 8) == hi ? (uint32_t)(lm & 255ull) : 0u);
      const unsigned long long m = ((unsigned long long)hi << 8) | lo;
      const int e = 255 - (int)lo;
      if (lane == k) {
        out.topk_ids[(size_t)t * K + k] = e;
        sid[t * K + k] = e;
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (kq[q] == m) kq[q] = 0ull;  // taken (keys are distinct)
      // the slot-k logit, from the lane that holds expert e
      float val = 0.0f;
#pragma unroll
      for (int q = 0; q < 4; ++q) val = (4 * lane + q == e) ? lv[q] : val;
      val = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(val), e >> 2));
      if (lane == k) mysel = val;
    }
    const float mx = __shfl(mysel, 0);
    float part = 0.0f, ev = 0.0f;
    if (norm_topk) {
      ev = lane < K ? expf(mysel - mx) : 0.0f;
      part = ev;
    } else {
      ev = lane < K ? expf(mysel - mx) : 0.0f;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (4 * lane + q < E) part += expf(lv[q] - mx);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) part += __shfl_xor(part, o);
    if (lane < K) out.topk_w[(size_t)t * K + lane] = ev / part;
  }
  __syncthreads();

  // ---- grouping of the R = T*K pairs (threads 0..255, one per expert) ------
  const int R = T * K;  // <= 256
  int c = 0, ne = 0;
  if (tid < MOE_MAX_EXPERTS) {
    for (int i = 0; i < R; ++i) c += sid[i] == tid ? 1 : 0;
    ne = c > 0 ? 1 : 0;
  }
  int ic = c, in = ne;  // inclusive scans of counts and of non-empty experts
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int vc = __shfl_up(ic, o), vn = __shfl_up(in, o);
    if (lane >= o) {
      ic += vc;
      in += vn;
    }
  }
  if (lane == 63 && wave < MOE_MAX_EXPERTS / 64) {
    wsum[wave][0] = ic;
    wsum[wave][1] = in;
  }
  __syncthreads();
  if (tid < MOE_MAX_EXPERTS) {
    int bc = 0, bn = 0;
    for (int w = 0; w < wave; ++w) {
      bc += wsum[w][0];
      bn += wsum[w][1];
    }
    const int off = bc + ic - c, tile = bn + in - ne;
    off_s[tid] = off;
    if (tid < E) {
      out.counts[tid] = c;
      out.offsets[tid] = off;
      if (c) {
        int32_t* bm = out.block_map + 4 * tile;
        bm[0] = tid;
        bm[1] = off;
        bm[2] = c;
        bm[3] = 0;
      }
    }
    if (tid == MOE_MAX_EXPERTS - 1) {
      const int tiles = bn + in;
      out.offsets[E] = R;
      if (has_shared) {
        int32_t* bm = out.block_map + 4 * tiles;
        bm[0] = E;
        bm[1] = R;
        bm[2] = T;
        bm[3] = 0;
      }
      *out.n_tiles = tiles + (has_shared ? 1 : 0);
    }
  }
  __syncthreads();
  if (tid < R) {
    const int x = sid[tid];
    int rank = 0;
    for (int i = 0; i < tid; ++i) rank += sid[i] == x ? 1 : 0;
    const int p = off_s[x] + rank;
    out.sorted_idx[p] = tid;
    out.inv_pos[tid] = p;
  }
}

// ---------------------------------------------------------------------------
// Split-reduction GEMV of one tile (<= 16 rows) against 16 weight rows per
// subtile (two subtiles), see the header comment.
// ---------------------------------------------------------------------------
template <bool kGateUp>
__global__ __launch_bounds__(kDecThreads) void decode_gemv_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) f32x4 part[kDecWaves][2][64];
  const int nslice = kGateUp ? g.I / 16 : g.N / 32;
  const int tile = blockIdx.x / nslice, sl = blockIdx.x - tile * nslice;
  if (kGateUp) zero_share(g);
  // the block-map entry is read together with n_tiles (entries past n_tiles
  // lie inside the map and are not used)
  const int4 bm = *reinterpret_cast<const int4*>(g.block_map + 4 * tile);
  if (tile >= *g.n_tiles) return;
  const int e = bm.x, row0 = bm.y, nrows = bm.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 15, lg = lane >> 4;
  const int Kd = g.Kdim, gpr = Kd / 64;
  const uint32_t cpr = (uint32_t)Kd / 2;
  const uint8_t* codes;
  const uint16_t* scl;
  const uint16_t* bia;
  if (e < g.E) {
    codes = g.codes + (size_t)e * g.N * cpr;
    scl = g.scales + (size_t)e * g.N * gpr;
    bia = g.biases + (size_t)e * g.N * gpr;
  } else {
    codes = g.s_codes;
    scl = g.s_scales;
    bia = g.s_biases;
  }
  const rsrc_t c_rs = make_rsrc(codes, (uint32_t)g.N * cpr);
  const rsrc_t s_rs = make_rsrc(scl, (uint32_t)g.N * gpr * 2u);
  const rsrc_t b_rs = make_rsrc(bia, (uint32_t)g.N * gpr * 2u);
  const uint32_t a_rows = kGateUp ? (uint32_t)g.T : (uint32_t)(g.R + g.T);
  const rsrc_t a_rs = make_rsrc(g.a, a_rows * (uint32_t)Kd * 2u);

  // weight rows of this lane (subtile j): gate/up: gate row 16 sl + ln and up
  // row I + 16 sl + ln; down: output columns 32 sl + 16 j + ln
  uint32_t wrow[2];
  if (kGateUp) {
    wrow[0] = (uint32_t)(16 * sl + ln);
    wrow[1] = (uint32_t)(g.I + 16 * sl + ln);
  } else {
    wrow[0] = (uint32_t)(32 * sl + ln);
    wrow[1] = (uint32_t)(32 * sl + 16 + ln);
  }
  // activation column ln of the MFMA: row ln of the tile (gate/up: its
  // token's x row; down: h row row0 + ln); columns past the tile read zeros
  uint32_t aoff = kOob;
  if (ln < nrows) {
    const int p = row0 + ln;
    int src;
    if (kGateUp) src = (p < g.R) ? g.sorted_idx[p] / g.topk : p - g.R;
    else src = p;
    aoff = (uint32_t)src * (uint32_t)Kd * 2u;
  }
  // per-lane part of the activation offsets (columns 16 lg + 8 st of a group)
  const uint32_t aoff_l[2] = {aoff == kOob ? kOob : aoff + 32u * lg, aoff == kOob ? kOob : aoff + 32u * lg + 16u};
  // this wave's quant groups: [g0, g1)
  const int g0 = (gpr * wave) / kDecWaves, g1 = (gpr * (wave + 1)) / kDecWaves;
  f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  if (g0 < g1) {
    u32x2 cw[kDecMaxGroupsPerWave][2];
    uint32_t sw[kDecMaxGroupsPerWave][2], bw[kDecMaxGroupsPerWave][2];
    u32x4 av[kDecMaxGroupsPerWave][2];
    // every load of the wave first (at most 4 groups: gpr <= 32)
#pragma unroll
    for (int i = 0; i < kDecMaxGroupsPerWave; ++i) {
      const int gi = g0 + i;
      if (gi < g1) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          cw[i][j] = __builtin_bit_cast(
              u32x2, __builtin_amdgcn_raw_buffer_load_b64(c_rs, wrow[j] * cpr + 8u * lg, gi * 32, 0));
          sw[i][j] = __builtin_amdgcn_raw_buffer_load_b16(s_rs, wrow[j] * (uint32_t)gpr * 2u, gi * 2, 0);
          bw[i][j] = __builtin_amdgcn_raw_buffer_load_b16(b_rs, wrow[j] * (uint32_t)gpr * 2u, gi * 2, 0);
        }
        // activation columns 16 lg .. 16 lg + 15 of the group: the k order
        // of the code word (the same permutation on both operands)
#pragma unroll
        for (int st = 0; st < 2; ++st)
          av[i][st] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(a_rs, aoff_l[st], gi * 128, 0));
      }
    }
#pragma unroll
    for (int i = 0; i < kDecMaxGroupsPerWave; ++i) {
      if (g0 + i < g1) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const float s = bf16_bits_to_f32(sw[i][j] & 0xFFFFu), b = bf16_bits_to_f32(bw[i][j] & 0xFFFFu);
#pragma unroll
          for (int st = 0; st < 2; ++st)
            mfma_acc(acc[j], dequant8(cw[i][j][st], s, b), __builtin_bit_cast(bf16x8, av[i][st]));
        }
      }
    }
  }
  // lane holds weight rows 4 lg .. 4 lg + 3 of each subtile for tile row ln;
  // the partials of the 8 waves are added in wave order
  part[wave][0][lane] = acc[0];
  part[wave][1][lane] = acc[1];
  __syncthreads();
  if (wave != 0 || ln >= nrows) return;
  f32x4 s0 = part[0][0][lane], s1 = part[0][1][lane];
#pragma unroll
  for (int w = 1; w < kDecWaves; ++w) {
    s0 += part[w][0][lane];
    s1 += part[w][1][lane];
  }
  const int r = row0 + ln;
  if (kGateUp) {
    uint32_t hv[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      float o[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const float gv = s0[2 * i + q], uv = s1[2 * i + q];
        o[q] = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * uv;
      }
      hv[i] = pack_bf16x2(o[0], o[1]);
    }
    uint16_t* h = reinterpret_cast<uint16_t*>(g.c);
    *reinterpret_cast<u32x2*>(&h[(size_t)r * g.I + 16 * sl + 4 * lg]) = u32x2{hv[0], hv[1]};
  } else {
    const DownRow dr = down_row(g, r);
    store_down4(g, dr, 32 * sl + 4 * lg, s0);
    store_down4(g, dr, 32 * sl + 16 + 4 * lg, s1);
  }
}

}  // namespace

hipError_t launch_decode_prep(const uint16_t* wr, int H, int E, float* wf, hipStream_t stream) {
  hipLaunchKernelGGL(decode_prep_kernel, dim3(E), dim3(64), 0, stream, wr, H, E, wf);
  return hipGetLastError();
}

hipError_t launch_decode_route(const DecodeRouteArgs& a, hipStream_t stream) {
  const int neb = (a.E + 63) / 64;
  hipLaunchKernelGGL(decode_logits_kernel, dim3(a.T * neb), dim3(64), 0, stream, a.x, a.wf, a.router_bias, a.H, a.E,
                     a.logits);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(decode_group_kernel, dim3(1), dim3(1024), 0, stream, a.logits, a.T, a.K, a.E, a.norm_topk,
                     a.has_shared, a.out);
  return hipGetLastError();
}

hipError_t launch_decode_gemv(const GemmArgs& g, bool gate_up, hipStream_t stream) {
  const int nslice = gate_up ? g.I / 16 : g.N / 32;
  if (gate_up)
    hipLaunchKernelGGL(decode_gemv_kernel<true>, dim3(g.max_tiles * nslice), dim3(kDecThreads), 0, stream, g);
  else
    hipLaunchKernelGGL(decode_gemv_kernel<false>, dim3(g.max_tiles * nslice), dim3(kDecThreads), 0, stream, g);
  return hipGetLastError();
}

}  // namespace moeq4
