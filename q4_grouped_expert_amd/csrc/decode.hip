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
//    hidden axis.  The router matrix is kept, once per model, as a bf16
//    piece-major copy wt[h/8][e][8], so the 64 lanes read 1 KB of
//    consecutive memory per step: eight fma per 16-byte load, the pieces
//    streamed 32 ahead in registers.  Each piece is unpacked to fp32 while
//    the previous piece's fma run (a dependent fma waits about 11 clocks on
//    gfx950; the unpacks fill those gaps).  The token row sits in LDS as fp32
//    and is read three pieces ahead.
//  * Top-k and grouping: one workgroup.  Wave t selects token t's experts by
//    K rounds of a wave-wide maximum over (logit, lower expert) keys and
//    forms the weights; then the workgroup builds counts, offsets, the stable
//    permutation and the block map (one tile per expert with rows, then the
//    shared expert) from the at most 256 (token, slot) pairs.
//  * Expert GEMVs: a workgroup owns one tile (<= 16 rows of one expert) and
//    32 weight rows (gate/up: 16 gate rows and the matching 16 up rows; down:
//    32 output columns as two subtiles) and splits the reduction into
//    contiguous ranges of at most 4 quant groups (64 columns each), one per
//    wave: 8 waves for a 2048-column reduction, 4 up to 1024, with the LDS
//    sized to match.  The work is a few MB spread over the whole chip, so the limit is
//    the number of memory requests, not bytes: each wave fetches its codes
//    as whole 128-byte row segments straight into LDS (8 lanes per segment),
//    the tile's scales and biases arrive as one 1 KB copy per table half,
//    and every load of the workgroup is in flight before the first wait.
//    Each wave dequantizes its codes (fma(q, s, b) in fp32, rounded to bf16)
//    as the A operand of v_mfma_f32_16x16x32_bf16 with the tile's activation
//    rows as the B operand.  The waves' partial 16x16 results are added in
//    wave order through LDS, so the result does not depend on timing.
//  * Combine: the prefill combine kernel.
#include <math.h>

#include <type_traits>

#include "common.hpp"
#include "gemm_common.hpp"

namespace moeq4 {

namespace {
using namespace gemm;

constexpr int kGvGroupsPerWave = 4;  // quant groups of the reduction per GEMV wave at most

// Maximum of v over the 64 lanes of the wave, returned to every lane: DPP
// exchanges inside each row of 16 lanes, then the row-pair and half-wave
// swaps (with both operands the same register, a swap leaves a block's
// value in one output and its neighbour's in the other).
template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kCtrl, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t a) {
  a = max(a, dpp_u32<0xB1>(a));   // quad_perm [1,0,3,2]
  a = max(a, dpp_u32<0x4E>(a));   // quad_perm [2,3,0,1]
  a = max(a, dpp_u32<0x141>(a));  // row_half_mirror
  a = max(a, dpp_u32<0x140>(a));  // row_mirror
  const auto r = __builtin_amdgcn_permlane16_swap(a, a, false, false);
  a = max((uint32_t)r[0], (uint32_t)r[1]);
  const auto h = __builtin_amdgcn_permlane32_swap(a, a, false, false);
  return max((uint32_t)h[0], (uint32_t)h[1]);
}

// Order-preserving map of an fp32 value to uint32 (-0 taken as +0).
__device__ __forceinline__ uint32_t dec_fkey(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------------------
// wt[p][e][0..7] = Wr[e][8p .. 8p+7] (p < H/8).  One wave per expert.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void decode_prep_kernel(const uint16_t* __restrict__ wr, int H, int E,
                                                         uint16_t* __restrict__ wt) {
  const int e = blockIdx.x;
  for (int p = threadIdx.x; p < H / 8; p += 64)
    *reinterpret_cast<u32x4*>(wt + ((size_t)p * E + e) * 8) = *reinterpret_cast<const u32x4*>(wr + (size_t)e * H + 8 * p);
}

// acc <- fma(x[q], u[q], acc) for q = 0..3 in order (u: fp32 weights), while
// the four bf16 weights packed in w0, w1 are unpacked into n.  The unpacks do
// not depend on acc and issue in the gaps between the dependent fma; one asm
// block keeps that interleaving.
__device__ __forceinline__ float chain4_unpack(float acc, float4 x, float u0, float u1, float u2, float u3,
                                               uint32_t w0, uint32_t w1, float& n0, float& n1, float& n2,
                                               float& n3) {
  asm("v_fmac_f32 %[acc], %[xa], %[u0]\n\t"
      "v_lshlrev_b32 %[n0], 16, %[w0]\n\t"
      "v_fmac_f32 %[acc], %[xb], %[u1]\n\t"
      "v_and_b32 %[n1], 0xffff0000, %[w0]\n\t"
      "v_fmac_f32 %[acc], %[xc], %[u2]\n\t"
      "v_lshlrev_b32 %[n2], 16, %[w1]\n\t"
      "v_fmac_f32 %[acc], %[xd], %[u3]\n\t"
      "v_and_b32 %[n3], 0xffff0000, %[w1]"
      : [acc] "+v"(acc), [n0] "=&v"(n0), [n1] "=&v"(n1), [n2] "=&v"(n2), [n3] "=&v"(n3)
      : [xa] "v"(x.x), [xb] "v"(x.y), [xc] "v"(x.z), [xd] "v"(x.w), [u0] "v"(u0), [u1] "v"(u1), [u2] "v"(u2),
        [u3] "v"(u3), [w0] "v"(w0), [w1] "v"(w1));
  return acc;
}

// ---------------------------------------------------------------------------
// Logits of 64 experts of one token per wave: l[e] = one fp32 chain over h
// in ascending order, then + bias.  Lanes past E run a copy of expert E-1's
// chain (every load stays in range) and store nothing.
// ---------------------------------------------------------------------------
template <int P>
__device__ __forceinline__ float logit_chain(rsrc_t w_rs, uint32_t voff, uint32_t pstride, int npc, const float* xf) {
  // Ring of P packed pieces: slot q % P holds piece q.  Piece q + 1 is
  // unpacked while piece q runs its fma, and its slot is then reloaded with
  // piece q + 1 + P.  Buffer loads count against the vector-memory counter
  // only (a generic pointer load would also count against the LDS counter, so
  // every read of the token row would wait for all loads in flight).  A
  // single wave issues one instruction every few clocks, so the loop keeps
  // its per-piece bookkeeping to a minimum: only the last block of P pieces
  // clamps its load offsets to the last piece, and the token row carries
  // three zero pieces after its end for the reads ahead.
  u32x4 wb[P];
#pragma unroll
  for (int i = 0; i < P; ++i) {
    wb[i] = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(w_rs, voff, (uint32_t)min(i, npc - 1) * pstride, 0));
    __builtin_amdgcn_sched_barrier(0);  // keep every load at its place: P in flight
  }
  float u[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    u[2 * k] = __uint_as_float(wb[0][k] << 16);
    u[2 * k + 1] = __uint_as_float(wb[0][k] & 0xFFFF0000u);
  }
  uint32_t vo = voff;
  wb[0] = __builtin_bit_cast(
      u32x4, __builtin_amdgcn_raw_buffer_load_b128(w_rs, vo, (uint32_t)min(P, npc - 1) * pstride, 0));
  // the token row of piece q in slot q % 4, read three pieces ahead (an LDS
  // read takes longer than one piece's fma)
  float4 xr[4][2];
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    xr[k][0] = *reinterpret_cast<const float4*>(&xf[8 * k]);
    xr[k][1] = *reinterpret_cast<const float4*>(&xf[8 * k + 4]);
  }
  float acc = 0.0f;
  // one block of P pieces from p0; kLast: the block whose reloads would pass
  // the last piece
  auto block = [&](auto last, int p0) {
    constexpr bool kLast = decltype(last)::value;
    const float* xb = xf + 8 * (p0 + 3);
    const uint32_t sbase = (uint32_t)(p0 + 1 + P) * pstride;
#pragma unroll
    for (int i = 0; i < P; ++i) {
      xr[(i + 3) % 4][0] = *reinterpret_cast<const float4*>(xb + 8 * i);
      xr[(i + 3) % 4][1] = *reinterpret_cast<const float4*>(xb + 8 * i + 4);
      __builtin_amdgcn_sched_barrier(0);  // the reads go out before this piece's fma
      const u32x4 w = wb[(i + 1) % P];
      float n[8];
      acc = chain4_unpack(acc, xr[i % 4][0], u[0], u[1], u[2], u[3], w[0], w[1], n[0], n[1], n[2], n[3]);
      acc = chain4_unpack(acc, xr[i % 4][1], u[4], u[5], u[6], u[7], w[2], w[3], n[4], n[5], n[6], n[7]);
      // reload the slot just unpacked only now (the empty asm ties the
      // offset to acc, so the load cannot be hoisted into a second register
      // set)
      asm("" : "+v"(vo) : "v"(acc));
      const uint32_t soff = kLast ? (uint32_t)min(p0 + i + 1 + P, npc - 1) * pstride : sbase + (uint32_t)i * pstride;
      wb[(i + 1) % P] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(w_rs, vo, soff, 0));
#pragma unroll
      for (int k = 0; k < 8; ++k) u[k] = n[k];
    }
  };
  int p0 = 0;
  for (; p0 + P < npc; p0 += P) block(std::false_type{}, p0);
  block(std::true_type{}, p0);
  return acc;
}

// Token t's row of x into LDS as fp32, then three zero pieces (read ahead
// past the end), by the threads [first, first + n).
__device__ __forceinline__ void token_row_to_lds(const uint16_t* __restrict__ x, int t, int H, float* xf, int i,
                                                 int n) {
  if (i < 24) xf[H + i] = 0.0f;
  for (int h = 8 * i; h < H; h += 8 * n) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(x + (size_t)t * H + h);
    float4* dst = reinterpret_cast<float4*>(&xf[h]);
    dst[0] = float4{bf16_bits_to_f32(v[0] & 0xFFFFu), bf16_bits_to_f32(v[0] >> 16), bf16_bits_to_f32(v[1] & 0xFFFFu),
                    bf16_bits_to_f32(v[1] >> 16)};
    dst[1] = float4{bf16_bits_to_f32(v[2] & 0xFFFFu), bf16_bits_to_f32(v[2] >> 16), bf16_bits_to_f32(v[3] & 0xFFFFu),
                    bf16_bits_to_f32(v[3] >> 16)};
  }
}

// The logit of expert e (this lane) against the token row xf: the exact
// chain, then + bias.  Lanes past E run a copy of expert E-1's chain (every
// load stays in range); the caller stores nothing for them.  bf16 x bf16
// products are exact in fp32, so each fma rounds exactly like acc = acc + x*w.
__device__ __forceinline__ float lane_logit(const uint16_t* __restrict__ wt, const float* __restrict__ rb, int H,
                                           int E, int e, const float* xf) {
  const int npc = H / 8;  // pieces, a multiple of 8
  const int ec = e < E ? e : E - 1;
  const rsrc_t w_rs = make_rsrc(wt, (uint32_t)E * (uint32_t)H * 2u);
  const uint32_t voff = (uint32_t)ec * 16u, pstride = (uint32_t)E * 16u;  // bytes
  const float acc = npc % 32 == 0 ? logit_chain<32>(w_rs, voff, pstride, npc, xf)
                                  : logit_chain<8>(w_rs, voff, pstride, npc, xf);
  return rb && e < E ? acc + rb[e] : acc;
}

__global__ __launch_bounds__(64) void decode_logits_kernel(const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ wt,
                                                           const float* __restrict__ rb, int H, int E,
                                                           float* __restrict__ logits) {
  __shared__ __attribute__((aligned(16))) float xf[MOE_MAX_REDUCTION + 24];
  const int neb = (E + 63) / 64;
  const int t = blockIdx.x / neb, eb = blockIdx.x - t * neb;
  const int lane = threadIdx.x;
  const int e = eb * 64 + lane;
  token_row_to_lds(x, t, H, xf, lane, 64);
  __syncthreads();
  const float l = lane_logit(wt, rb, H, E, e, xf);
  if (e < E) logits[(size_t)t * E + e] = l;
}

// ---------------------------------------------------------------------------
// Top-k, weights and grouping for at most 16 tokens in one workgroup.
//
// Wave t (token t) holds experts 4 l .. 4 l + 3 in lane l as order-preserving
// keys of their logits and takes K rounds: the wave-wide maximum key, then
// the lowest lane holding it (a ballot) and that lane's lowest expert with
// it, which is the lowest expert with the largest logit; the winner's key is
// removed and the winners in order are the slots.  Weights: exp(l - l_max)
// over the sum of exp(l - l_max) of the selection (norm_topk) or of every
// expert, the sums in a fixed lane tree.  Then, for the at most 256
// (token, slot) pairs, one per thread: each wave finds the lanes whose pair
// has the same expert with eight ballots (one per bit of the expert index),
// which gives a pair's rank among the earlier pairs of its wave and each
// expert's count per wave; counts, offsets, the stable sorted_idx / inv_pos,
// the block map (one tile per expert with rows, in expert order, then the
// shared expert's) and n_tiles follow from those.
// ---------------------------------------------------------------------------
constexpr int kPairWaves = MOE_MAX_EXPERTS / 64;  // waves of (token, slot) pairs, R <= 256
struct GroupLds {
  int sid[MOE_MAX_EXPERTS];
  int wsum[MOE_MAX_EXPERTS / 64][2];
  int off_s[MOE_MAX_EXPERTS];
  int cntw[kPairWaves][MOE_MAX_EXPERTS];  // pairs of wave w with expert e
};

// Called by every thread of a workgroup of at least max(T, 4) waves; logits
// [T][E] in global memory or LDS, complete and visible to the workgroup.
__device__ __forceinline__ void group_body(const float* logits, int T, int K, int E, int norm_topk, int has_shared,
                                           const moe_route_out& out, GroupLds& sm) {
  auto& sid = sm.sid;
  auto& wsum = sm.wsum;
  auto& off_s = sm.off_s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // every count of a pair wave starts at zero (the waves past T are idle now)
  for (int i = tid; i < kPairWaves * MOE_MAX_EXPERTS; i += blockDim.x) (&sm.cntw[0][0])[i] = 0;

  if (wave < T) {
    const int t = wave;
    uint32_t kq[4];
    float lv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = 4 * lane + q;
      lv[q] = e < E ? logits[(size_t)t * E + e] : 0.0f;
      kq[q] = e < E ? dec_fkey(lv[q]) : 0u;  // every logit's key is above 0
    }
    float mysel = 0.0f;  // lane k < K: the slot-k logit and expert
    int myid = 0;
    for (int k = 0; k < K; ++k) {
      const uint32_t lm = max(max(kq[0], kq[1]), max(kq[2], kq[3]));
      const uint32_t m = wave_max_u32(lm);
      // lane l holds experts 4l..4l+3, so the lowest lane holding the key
      // holds the lowest expert with it
      const int wl = __builtin_ctzll(__builtin_amdgcn_ballot_w64(lm == m));
      const int qf = kq[0] == m ? 0 : kq[1] == m ? 1 : kq[2] == m ? 2 : 3;
      const int qs = __builtin_amdgcn_readlane(qf, wl);
      const float lq = qs == 0 ? lv[0] : qs == 1 ? lv[1] : qs == 2 ? lv[2] : lv[3];
      const float val = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lq), wl));
      const bool mine = lane == wl;
#pragma unroll
      for (int q = 0; q < 4; ++q) kq[q] = (mine && q == qs) ? 0u : kq[q];  // taken
      if (lane == k) {
        myid = 4 * wl + qs;
        mysel = val;
      }
    }
    if (lane < K) {
      out.topk_ids[(size_t)t * K + lane] = myid;
      sid[t * K + lane] = myid;
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

  // ---- grouping of the R = T*K pairs -----------------------------------------
  const int R = T * K;  // <= 256
  int x = 0, rank = 0;  // thread i < R: pair i's expert and its rank among the wave's earlier pairs
  if (tid < R) {
    x = sid[tid];
    uint64_t same = __builtin_amdgcn_ballot_w64(true);
#pragma unroll
    for (int b = 0; b < 8; ++b) {  // expert indices are below 256
      const bool bit = (x >> b) & 1;
      const uint64_t m = __builtin_amdgcn_ballot_w64(bit);
      same &= bit ? m : ~m;
    }
    rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(same >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)same, 0u));
    if (rank == 0) sm.cntw[wave][x] = __popcll(same);
  }
  __syncthreads();
  int c = 0, ne = 0;  // thread e < 256: expert e's pairs
  if (tid < MOE_MAX_EXPERTS) {
#pragma unroll
    for (int w = 0; w < kPairWaves; ++w) c += sm.cntw[w][tid];
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
    for (int w = 0; w < wave; ++w) rank += sm.cntw[w][x];  // the expert's pairs in earlier waves
    const int p = off_s[x] + rank;
    out.sorted_idx[p] = tid;
    out.inv_pos[tid] = p;
  }
}

__global__ __launch_bounds__(1024) void decode_group_kernel(const float* __restrict__ logits, int T, int K, int E,
                                                            int norm_topk, int has_shared, moe_route_out out) {
  __shared__ GroupLds sm;
  group_body(logits, T, K, E, norm_topk, has_shared, out, sm);
}

// ---------------------------------------------------------------------------
// Router and grouping in one workgroup for at most kDecFusedTokens tokens:
// wave w computes the logits of token w / neb, experts 64 (w % neb) ..
// (every chain on its own wave, as in the two-kernel form), into LDS; then
// the workgroup runs the grouping above.  One launch fewer.
// ---------------------------------------------------------------------------
constexpr int kDecFusedTokens = 2;  // 8 waves at most: 256 registers per lane for the chain

__global__ __launch_bounds__(512) void decode_route_fused_kernel(const uint16_t* __restrict__ x,
                                                                  const uint16_t* __restrict__ wt,
                                                                  const float* __restrict__ rb, int T, int H, int E,
                                                                  int K, int norm_topk, int has_shared,
                                                                  moe_route_out out) {
  __shared__ __attribute__((aligned(16))) float xf[kDecFusedTokens][MOE_MAX_REDUCTION + 24];
  __shared__ float lg[kDecFusedTokens * MOE_MAX_EXPERTS];
  __shared__ GroupLds sm;
  const int neb = (E + 63) / 64;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nw = blockDim.x >> 6;
  // token rows: the waves share them out, token t to waves t, t + T, ...
  for (int t = 0; t < T; ++t)
    if (wave % T == t) token_row_to_lds(x, t, H, xf[t], tid - 64 * wave + 64 * (wave / T), 64 * ((nw - t + T - 1) / T));
  __syncthreads();
  if (wave < T * neb) {
    const int t = wave / neb, eb = wave - t * neb;
    const int e = eb * 64 + lane;
    const float l = lane_logit(wt, rb, H, E, e, xf[t]);
    if (e < E) lg[t * E + e] = l;
  }
  __syncthreads();
  group_body(lg, T, K, E, norm_topk, has_shared, out, sm);
}

// ---------------------------------------------------------------------------
// Split-reduction GEMV of one tile (<= 16 rows) against 32 weight rows, see
// the header comment.
// ---------------------------------------------------------------------------
// NW waves, each taking at most MG = kGvGroupsPerWave quant groups of the
// reduction: 8 waves and 36 KB for a 2048-column reduction (four workgroups
// per CU), 4 waves and 18 KB up to 1024 columns (eight per CU)
template <int NW, int MG>
struct GemvLds {
  static constexpr int kSegs = MG * 32 / 128;  // 128-byte code segments per row and wave
  // codes of each wave: [segment * 4 + row block][row in block][16-byte chunk];
  // once a wave's products are done, the start of its range holds its
  // partial sums ([2][64] f32x4)
  uint8_t cl[NW][kSegs * 4][1024];
  uint16_t ssh[32 * NW * MG];  // [32 rows][gpr] scales
  uint16_t bsh[32 * NW * MG];  // and biases
  static_assert(2 * 64 * sizeof(f32x4) <= kSegs * 4 * 1024, "a wave's partial sums fit its code range");
};

template <bool kGateUp, int NW, int MG>
__device__ __forceinline__ void gemv_body(const GemmArgs& g, GemvLds<NW, MG>& sm) {
  constexpr int kGvSegs = GemvLds<NW, MG>::kSegs;
  auto& cl = sm.cl;
  auto& ssh = sm.ssh;
  auto& bsh = sm.bsh;
  // wave w's partial sums, in the code range it alone reads
  auto part = [&](int w, int j) { return reinterpret_cast<f32x4*>(&cl[w][0][0]) + 64 * j; };
  const int nslice = kGateUp ? g.I / 16 : g.N / 32;
  const int tile = blockIdx.x / nslice, sl = blockIdx.x - tile * nslice;
  if (kGateUp) zero_share(g);
  // The block-map entry and the tile count arrive after one memory latency:
  // the exit test reads both (entries past n_tiles lie inside the map; every
  // live entry has rows), so neither load waits for the other.
  const int4 bm = *reinterpret_cast<const int4*>(g.block_map + 4 * tile);
  const int nt = *g.n_tiles;
  if (tile >= nt || bm.z <= 0) return;
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

  // Weight row r (0..31) of the slice: gate/up: gate rows 16 sl + r for
  // r < 16, the matching up rows I + 16 sl + r - 16 after them; down: output
  // columns 32 sl + r.  Rows 0..15 and 16..31 are each contiguous.
  auto wrow_of = [&](int r) -> uint32_t {
    if (kGateUp) return (uint32_t)((r < 16 ? 0 : g.I - 16) + 16 * sl + r);
    return (uint32_t)(32 * sl + r);
  };
  // tile row ln's activation row (gate/up: its token, through sorted_idx;
  // down: h row row0 + ln); loaded first, so waiting for it leaves the DMAs
  // issued after it in flight
  const bool arow = ln < nrows;
  int sidx = 0;
  if (kGateUp && arow && row0 + ln < g.R) sidx = g.sorted_idx[row0 + ln];
  __builtin_amdgcn_sched_barrier(0);

  // ---- the tile's scale and bias tables ([32 rows][gpr] each): wave w < 4
  // copies half w & 1 (16 rows, 32 gpr bytes <= 1 KB) of table w >> 1; only
  // the lanes inside the half copy (the two halves' LDS ranges are adjacent)
  {
    const int half = wave & 1;
    const uint32_t bytes = 32u * (uint32_t)gpr;
    uint16_t* dst = (wave < 2 ? ssh : bsh) + half * 16 * gpr;
    if (wave < 4 && 16u * lane < bytes)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wave < 2 ? s_rs : b_rs, (__attribute__((address_space(3))) void*)dst,
                                               16, wrow_of(16 * half) * (uint32_t)gpr * 2u + 16u * lane, 0, 0, 0);
  }
  // ---- this wave's codes: quant groups [g0, g1) (at most MG), as
  // whole 128-byte segments of each of the 32 rows.  DMA (s, rb) fills rows
  // 8 rb .. 8 rb + 7 with segment s: lane l lands at row 8 rb + l/8,
  // physical chunk l%8, and fetches logical chunk (l%8) ^ (l/8), so that the
  // 16 rows one read touches spread over the banks.  Chunks past g1 read
  // zeros.
  const int g0 = (gpr * wave) / NW, g1 = (gpr * (wave + 1)) / NW;
  const int ng = g1 - g0;
  {
    const int r8 = lane >> 3;
    const int c = (lane & 7) ^ r8;
#pragma unroll
    for (int sg = 0; sg < kGvSegs; ++sg)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const uint32_t b = 128u * sg + 16u * c;  // byte of the wave's row range
        const uint32_t off = b < 32u * (uint32_t)ng ? wrow_of(8 * rb + r8) * cpr + 32u * g0 + b : kOob;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            c_rs, (__attribute__((address_space(3))) void*)&cl[wave][sg * 4 + rb][0], 16, off, 0, 0, 0);
      }
  }
  // ---- activations as the B operand: lane (ln, lg) holds tile row ln,
  // columns 64 g + 16 lg + 8 st of group g for MFMA step st (the k order of
  // the code word; the same permutation on both operands); rows past the
  // tile and groups past g1 read zeros
  uint32_t aoff = kOob;
  if (arow) {
    const int p = row0 + ln;
    const int src = kGateUp ? (p < g.R ? sidx / g.topk : p - g.R) : p;
    aoff = (uint32_t)src * (uint32_t)Kd * 2u + 32u * lg;
  }
  u32x4 av[MG][2];
#pragma unroll
  for (int i = 0; i < MG; ++i)
#pragma unroll
    for (int st = 0; st < 2; ++st)
      av[i][st] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(a_rs, i < ng ? aoff + 16u * st : kOob, (g0 + i) * 128, 0));
  wait_vmcnt<0>();
  __syncthreads();  // every wave's table copy has landed

  f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int i = 0; i < MG; ++i) {
    if (i < ng) {
      const int sg = i / 4;
      const int c = 2 * (i % 4) + (lg >> 1);  // logical chunk of the segment
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = 16 * j + ln;  // row of the slice
        const int r8 = r & 7;
        const u32x2 cw = *reinterpret_cast<const u32x2*>(&cl[wave][sg * 4 + (r >> 3)][r8 * 128 + (c ^ r8) * 16 +
                                                                                      8 * (lg & 1)]);
        const float sv = bf16_bits_to_f32(ssh[r * gpr + g0 + i]), bv = bf16_bits_to_f32(bsh[r * gpr + g0 + i]);
#pragma unroll
        for (int st = 0; st < 2; ++st)
          mfma_acc(acc[j], dequant8(cw[st], sv, bv), __builtin_bit_cast(bf16x8, av[i][st]));
      }
    }
  }
  // lane holds weight rows 4 lg .. 4 lg + 3 of each subtile for tile row ln;
  // the partials of the 4 waves are added in wave order
  // (a wave's LDS operations run in order, so these writes follow its own
  // last reads of that range)
  part(wave, 0)[lane] = acc[0];
  part(wave, 1)[lane] = acc[1];
  __syncthreads();
  if (wave != 0 || ln >= nrows) return;
  f32x4 s0 = part(0, 0)[lane], s1 = part(0, 1)[lane];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    s0 += part(w, 0)[lane];
    s1 += part(w, 1)[lane];
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

template <bool kGateUp, int NW>
__global__ __launch_bounds__(64 * NW) void decode_gemv_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) GemvLds<NW, kGvGroupsPerWave> sm;
  gemv_body<kGateUp, NW, kGvGroupsPerWave>(g, sm);
}

}  // namespace

hipError_t launch_decode_prep(const uint16_t* wr, int H, int E, uint16_t* wt, hipStream_t stream) {
  hipLaunchKernelGGL(decode_prep_kernel, dim3(E), dim3(64), 0, stream, wr, H, E, wt);
  return hipGetLastError();
}

hipError_t launch_decode_route(const DecodeRouteArgs& a, hipStream_t stream) {
  const int neb = (a.E + 63) / 64;
  if (a.T <= kDecFusedTokens) {
    const int waves = a.T * neb > 4 ? a.T * neb : 4;  // the grouping needs 256 threads
    hipLaunchKernelGGL(decode_route_fused_kernel, dim3(1), dim3(64 * waves), 0, stream, a.x, a.wt, a.router_bias, a.T,
                       a.H, a.E, a.K, a.norm_topk, a.has_shared, a.out);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(decode_logits_kernel, dim3(a.T * neb), dim3(64), 0, stream, a.x, a.wt, a.router_bias, a.H, a.E,
                     a.logits);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(decode_group_kernel, dim3(1), dim3(1024), 0, stream, a.logits, a.T, a.K, a.E, a.norm_topk,
                     a.has_shared, a.out);
  return hipGetLastError();
}

hipError_t launch_decode_gemv(const GemmArgs& g, bool gate_up, hipStream_t stream) {
  const int nslice = gate_up ? g.I / 16 : g.N / 32;
  const dim3 grid(g.max_tiles * nslice);
  // waves: enough for at most kGvGroupsPerWave quant groups each (the
  // reduction is at most 2048 columns, 32 groups)
  const bool small = g.Kdim / 64 <= 4 * kGvGroupsPerWave;
  static_assert(MOE_MAX_REDUCTION / 64 <= 8 * kGvGroupsPerWave, "eight waves cover the longest reduction");
  if (gate_up) {
    if (small) hipLaunchKernelGGL((decode_gemv_kernel<true, 4>), grid, dim3(256), 0, stream, g);
    else hipLaunchKernelGGL((decode_gemv_kernel<true, 8>), grid, dim3(512), 0, stream, g);
  } else {
    if (small) hipLaunchKernelGGL((decode_gemv_kernel<false, 4>), grid, dim3(256), 0, stream, g);
    else hipLaunchKernelGGL((decode_gemv_kernel<false, 8>), grid, dim3(512), 0, stream, g);
  }
  return hipGetLastError();
}

}  // namespace moeq4
