// Gated DeltaNet prefill scan (gfx950 / CDNA4).
//
// Per value head the state S (DV x DK, fp32) follows the gated delta rule
//   S_t = alpha_t S_{t-1} + beta_t (v_t - alpha_t S_{t-1} k_t) k_t^T,
//   o_t = S_t q_t
// (the Gated DeltaNet layer the pages pair with the MoE layers: "Perplexity
// Lily 오픈소스 공개", alltoptrend.co.kr, section 4; "Apple silicon용 Lily,
// Qwen 추론 최적화", aitrends.kr, glossary entry on Gated DeltaNet).
//
// Row i of S only needs k_t, q_t, v_t[i], alpha_t and beta_t: rows evolve
// independently, so every row is its own sequential scan.  The pages give
// one state column per SIMD group and keep it in registers for the whole
// scan, writing the fp32 state once at the end (aitrends.kr, section
// "GPU 상주와 메모리 절감").  Here:
//  * a row is held by 16 lanes (one DPP row), DK/16 fp32 entries each (in
//    groups of 4, so that LDS reads of k and q are conflict-free), in
//    registers from the first token to the last; a wave holds 4 rows and a
//    workgroup of 4 waves 16 rows of one head, so a 32-head, 128-row layer
//    runs 256 workgroups, one per CU;
//  * a step is: the row's recall S k (DK/16 fma per lane, then a 4-step DPP
//    butterfly over the 16 lanes that leaves the same sum in each), the
//    delta coefficient c = beta (v_i - alpha recall), the update
//    S = c k + alpha S, and the output S q (another butterfly, off the
//    recurrence's critical path);
//  * k and q of 32 tokens are staged in LDS as fp32, converted once per
//    workgroup instead of once per row, double-buffered: the next chunk's
//    global loads are issued at the start of a chunk and land in the other
//    buffer at its end;
//  * a chunk's outputs collect in LDS and leave as 64-byte row pieces.
#include "common.hpp"
#include "gdn_scan.h"

namespace moeq4 {
namespace {

constexpr int kGdnRows = 16;    // state rows per workgroup (4 per wave)
constexpr int kGdnThreads = 256;
constexpr int kChunk = 32;      // tokens staged in LDS at a time

struct GdnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const float* alpha;
  const float* beta;
  const float* state_in;
  float* o;
  float* state_out;
  int T, HK, HV, DV;
};

template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xf, 0xf, false));
}

// Sum over the 16 lanes of a DPP row.  Each step adds a lane's value to its
// partner's in either order, so all 16 lanes end with the same bits.
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_f32<0xB1>(x);   // quad_perm [1,0,3,2]: pairs
  x += dpp_f32<0x4E>(x);   // quad_perm [2,3,0,1]: quads
  x += dpp_f32<0x141>(x);  // row_half_mirror: halves of 8
  x += dpp_f32<0x140>(x);  // row_mirror: the row of 16
  return x;
}

__device__ __forceinline__ void bf16x8_to_f32(const u32x4& w, float* out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

template <int kE>  // key entries per lane: DK / 16
__global__ __launch_bounds__(kGdnThreads, 1) void gdn_scan_kernel(GdnArgs a) {
  constexpr int DK = 16 * kE;
  constexpr int kPieces = kChunk * DK / 8;               // 16-byte pieces of k (and of q) per chunk
  constexpr int kPerThread = kPieces / kGdnThreads;      // 1 (DK = 64) or 2 (DK = 128)
  static_assert(kPerThread * kGdnThreads == kPieces, "staging split");
  __shared__ __attribute__((aligned(16))) float kf[2][kChunk][DK];
  __shared__ __attribute__((aligned(16))) float qf[2][kChunk][DK];
  __shared__ __attribute__((aligned(16))) float vf[2][kChunk][kGdnRows];
  __shared__ __attribute__((aligned(16))) float gb[2][kChunk][2];  // alpha, beta
  __shared__ __attribute__((aligned(16))) float ob[kChunk][kGdnRows];

  const int T = a.T;
  // workgroup b takes head b % HV: with HV a multiple of 8 all row blocks of
  // a head share an XCD (workgroups go round-robin over the 8), so the
  // head's k and q are fetched into one L2 instead of eight
  const int hv = blockIdx.x % a.HV;
  const int blk = blockIdx.x / a.HV;
  const int hk = hv / (a.HV / a.HK);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rl = 4 * wave + (lane >> 4);  // row within the workgroup
  const int l16 = lane & 15;

  // this lane's part of the state: row 16*blk + rl of head hv, entries
  // 64*(e/4) + 4*l16 + e%4 for e < kE.  Groups of 4 consecutive entries per
  // lane, 64 apart, so each 16-byte LDS read of k or q by the 16 lanes of a
  // row covers 256 consecutive bytes: every bank once, no conflict (8
  // consecutive entries per lane would put two lanes on each bank group).
  float S[kE];
  auto entry = [&](int e) { return 64 * (e / 4) + 4 * l16; };  // first of the 4 entries of group e/4
  const size_t srow = ((size_t)hv * a.DV + kGdnRows * blk + rl) * DK;
  if (a.state_in) {
#pragma unroll
    for (int e = 0; e < kE; e += 4) {
      const f32x4 s4 = *reinterpret_cast<const f32x4*>(a.state_in + srow + entry(e));
#pragma unroll
      for (int i = 0; i < 4; ++i) S[e + i] = s4[i];
    }
  } else {
#pragma unroll
    for (int e = 0; e < kE; ++e) S[e] = 0.0f;
  }

  // ---- staging of one chunk: global loads into registers, then LDS ------
  struct Staged {
    u32x4 k[kPerThread], q[kPerThread];
    u32x4 v;
    float g;
  };
  auto fetch = [&](int t0, Staged& st) {
#pragma unroll
    for (int p = 0; p < kPerThread; ++p) {
      const int piece = tid + kGdnThreads * p;
      const int s = piece / (DK / 8), c = piece % (DK / 8);
      const int t = t0 + s;
      st.k[p] = st.q[p] = u32x4{0u, 0u, 0u, 0u};
      if (t < T) {
        const size_t off = ((size_t)t * a.HK + hk) * DK + 8 * c;
        st.k[p] = *reinterpret_cast<const u32x4*>(a.k + off);
        st.q[p] = *reinterpret_cast<const u32x4*>(a.q + off);
      }
    }
    st.v = u32x4{0u, 0u, 0u, 0u};
    st.g = 0.0f;
    if (tid < 2 * kChunk) {  // v: 16 rows of one token = two 16-byte pieces
      const int t = t0 + tid / 2;
      if (t < T)
        st.v = *reinterpret_cast<const u32x4*>(a.v + ((size_t)t * a.HV + hv) * a.DV + kGdnRows * blk + 8 * (tid & 1));
    } else if (tid < 4 * kChunk) {  // alpha, then beta
      const int s = (tid - 2 * kChunk) % kChunk;
      const int t = t0 + s;
      if (t < T) st.g = (tid < 3 * kChunk ? a.alpha : a.beta)[(size_t)t * a.HV + hv];
    }
  };
  auto stash = [&](int b, const Staged& st) {
#pragma unroll
    for (int p = 0; p < kPerThread; ++p) {
      const int piece = tid + kGdnThreads * p;
      const int s = piece / (DK / 8), c = piece % (DK / 8);
      float f[8];
      bf16x8_to_f32(st.k[p], f);
      *reinterpret_cast<f32x4*>(&kf[b][s][8 * c]) = f32x4{f[0], f[1], f[2], f[3]};
      *reinterpret_cast<f32x4*>(&kf[b][s][8 * c + 4]) = f32x4{f[4], f[5], f[6], f[7]};
      bf16x8_to_f32(st.q[p], f);
      *reinterpret_cast<f32x4*>(&qf[b][s][8 * c]) = f32x4{f[0], f[1], f[2], f[3]};
      *reinterpret_cast<f32x4*>(&qf[b][s][8 * c + 4]) = f32x4{f[4], f[5], f[6], f[7]};
    }
    if (tid < 2 * kChunk) {
      float f[8];
      bf16x8_to_f32(st.v, f);
      const int s = tid / 2, h = 8 * (tid & 1);
      *reinterpret_cast<f32x4*>(&vf[b][s][h]) = f32x4{f[0], f[1], f[2], f[3]};
      *reinterpret_cast<f32x4*>(&vf[b][s][h + 4]) = f32x4{f[4], f[5], f[6], f[7]};
    } else if (tid < 4 * kChunk) {
      const int s = (tid - 2 * kChunk) % kChunk;
      gb[b][s][tid < 3 * kChunk ? 0 : 1] = st.g;
    }
  };

  const int nchunks = (T + kChunk - 1) / kChunk;
  Staged st;
  if (nchunks > 0) {
    fetch(0, st);
    stash(0, st);
  }
  __syncthreads();
  for (int ch = 0; ch < nchunks; ++ch) {
    const int b = ch & 1;
    const int t0 = ch * kChunk;
    const bool more = ch + 1 < nchunks;
    if (more) fetch(t0 + kChunk, st);  // lands in the other buffer after this chunk
    const int n = min(kChunk, T - t0);
    // one token's inputs, read from LDS a step before they are used
    struct StepIn {
      float k[kE], q[kE];
      float v, al, be;
    };
    static_assert(kChunk == 32, "each lane keeps the outputs of two tokens of a chunk");
    float keep0 = 0.0f, keep1 = 0.0f;  // outputs of tokens l16 and 16 + l16 of the chunk
    auto load_step = [&](int s, StepIn& in) {
#pragma unroll
      for (int e = 0; e < kE; e += 4) {
        const f32x4 k4 = *reinterpret_cast<const f32x4*>(&kf[b][s][entry(e)]);
        const f32x4 q4 = *reinterpret_cast<const f32x4*>(&qf[b][s][entry(e)]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          in.k[e + i] = k4[i];
          in.q[e + i] = q4[i];
        }
      }
      in.v = vf[b][s][rl];
      in.al = gb[b][s][0];
      in.be = gb[b][s][1];
    };
    auto step = [&](int s, const StepIn& in) {
      // recall of the decayed state for k_t
      float d0 = 0.0f, d1 = 0.0f;
#pragma unroll
      for (int e = 0; e < kE; e += 2) {
        d0 = __builtin_fmaf(S[e], in.k[e], d0);
        d1 = __builtin_fmaf(S[e + 1], in.k[e + 1], d1);
      }
      const float recall = in.al * row16_sum(d0 + d1);
      const float c = in.be * (in.v - recall);
      float o0 = 0.0f, o1 = 0.0f;
#pragma unroll
      for (int e = 0; e < kE; ++e) {
        S[e] = __builtin_fmaf(c, in.k[e], in.al * S[e]);
        if (e & 1) o1 = __builtin_fmaf(S[e], in.q[e], o1);
        else o0 = __builtin_fmaf(S[e], in.q[e], o0);
      }
      // the 16 lanes of the row hold the same sum; lane s % 16 keeps it, so
      // a chunk's outputs leave through two LDS writes per lane, not one
      // masked write per token
      const float ov = row16_sum(o0 + o1);
      const bool mine = l16 == (s & 15);
      keep0 = mine && s < 16 ? ov : keep0;
      keep1 = mine && s >= 16 ? ov : keep1;
    };
    // two tokens per iteration, each one's inputs loaded during the previous
    // token, so the output sum of one token overlaps the next one's recall;
    // a full chunk runs as straight-line code (LDS offsets become
    // immediates), the last, partial one as a loop
    StepIn x0, x1;
    load_step(0, x0);
    if (n == kChunk) {
#pragma unroll
      for (int s = 0; s < kChunk; s += 2) {
        load_step(s + 1, x1);
        step(s, x0);
        if (s + 2 < kChunk) load_step(s + 2, x0);
        step(s + 1, x1);
      }
    } else {
      int s = 0;
      for (; s + 2 <= n; s += 2) {
        load_step(s + 1, x1);
        step(s, x0);
        if (s + 2 < n) load_step(s + 2, x0);
        step(s + 1, x1);
      }
      if (s < n) step(s, x0);
    }
    ob[l16][rl] = keep0;
    ob[16 + l16][rl] = keep1;
    __syncthreads();  // the chunk's outputs are in ob and buffer b is no longer read
    {
      const int s = tid / (kGdnRows / 2), part = tid % (kGdnRows / 2);
      if (s < n) {
        const float2 w = *reinterpret_cast<const float2*>(&ob[s][2 * part]);
        *reinterpret_cast<float2*>(a.o + ((size_t)(t0 + s) * a.HV + hv) * a.DV + kGdnRows * blk + 2 * part) = w;
      }
    }
    if (more) stash(b ^ 1, st);
    __syncthreads();
  }

  // the state leaves once, after the last token
#pragma unroll
  for (int e = 0; e < kE; e += 4)
    *reinterpret_cast<f32x4*>(a.state_out + srow + entry(e)) = f32x4{S[e], S[e + 1], S[e + 2], S[e + 3]};
}

inline bool misaligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

}  // namespace
}  // namespace moeq4

extern "C" int gdn_prefill_scan(const gdn_scan_desc* d, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                const float* alpha, const float* beta, const float* state_in, float* o,
                                float* state_out, void* stream) {
  using namespace moeq4;
  if (!d || !state_out) return MOE_ERR_INVALID_ARGUMENT;
  if (d->T < 0 || d->HK <= 0 || d->HV <= 0 || d->DK <= 0 || d->DV <= 0) return MOE_ERR_INVALID_ARGUMENT;
  if (d->T > 0 && (!q || !k || !v || !alpha || !beta || !o)) return MOE_ERR_INVALID_ARGUMENT;
  if (state_in && state_in == state_out) return MOE_ERR_INVALID_ARGUMENT;
  if ((d->DK != 64 && d->DK != 128) || d->DV % kGdnRows != 0 || d->HV % d->HK != 0)
    return MOE_ERR_UNSUPPORTED_SHAPE;
  if (misaligned16(state_out) || (state_in && misaligned16(state_in)) ||
      (d->T > 0 && (misaligned16(q) || misaligned16(k) || misaligned16(v) || misaligned16(alpha) ||
                    misaligned16(beta) || misaligned16(o))))
    return MOE_ERR_MISALIGNED;
  GdnArgs a{q, k, v, alpha, beta, state_in, o, state_out, d->T, d->HK, d->HV, d->DV};
  const dim3 grid((unsigned)(d->HV * (d->DV / kGdnRows)));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (d->DK == 128) hipLaunchKernelGGL((gdn_scan_kernel<8>), grid, dim3(kGdnThreads), 0, s, a);
  else hipLaunchKernelGGL((gdn_scan_kernel<4>), grid, dim3(kGdnThreads), 0, s, a);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}
