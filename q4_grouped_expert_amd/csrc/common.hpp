// Shared device-side helpers of libmoeq4 (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_q4.h"

namespace moeq4 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Rows per GEMM tile in the block map.
constexpr int kTileRows = 256;
// Prompts of at most kSmallPromptTokens tokens run the grouped GEMMs over
// pieces of at most kSmallRows rows (routing lists them), all in the
// short-tile form of a smaller-LDS kernel, so more workgroups share a CU.
constexpr int kSmallRows = 64;
constexpr int kSmallPromptTokens = 1536;
// Quant groups per weight row the GEMM keeps in LDS (reduction dim <= 2048).
constexpr int kMaxGroupsPerRow = 32;
// Tokens per expert-histogram group of the router (the scan runs over groups).
constexpr int kHistTokens = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Pack two fp32 values into two bf16 (round to nearest even) in one dword.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}

// Device-side launchers (defined in the .hip files, called by api.hip).
struct RouteArgs {
  const uint16_t* x;
  const uint16_t* w_router;
  const float* router_bias;
  int T, H, E, K, norm_topk, has_shared;
  moe_route_out out;
  // null, or where the grouping also lists the GEMMs' tiles in launch order
  // (n_launch entries): launch_rows == kTileRows: the block map's tiles, most
  // 16-row subtiles first; launch_rows == kSmallRows: every expert's rows in
  // pieces of at most kSmallRows rows, in the same order (full pieces first,
  // then the partial ones by subtile count)
  int32_t* launch_map;
  int32_t* n_launch;
  int launch_rows;
};
// Routing scratch (expert histograms per 64-token group, router-row norms, a
// piece-major copy of the router matrix, approximate logits) and launcher.
size_t route_workspace_bytes(int T, int H, int E);
hipError_t launch_route(const RouteArgs& a, void* ws, hipStream_t stream);

struct GemmArgs {
  const uint16_t* a;        // activations, bf16 [*, Kdim]
  const uint8_t* codes;     // routed experts [E][N][Kdim/2]
  const uint16_t* scales;   // [E][N][Kdim/64]
  const uint16_t* biases;
  const uint8_t* s_codes;   // shared expert [N][Kdim/2] (or null)
  const uint16_t* s_scales;
  const uint16_t* s_biases;
  const uint16_t* wbf;      // unfused variant: bf16 weights [E][N][Kdim] (codes unused), else null
  const uint16_t* s_wbf;    // and the shared expert's [N][Kdim]
  const int32_t* sorted_idx;
  const int32_t* block_map;
  const int32_t* launch_map;  // null, or the tiles in launch order
  const int32_t* n_launch;    // with small: the list's entry count (else n_tiles bounds it)
  int small;                  // the list holds pieces of at most kSmallRows rows: the small kernel
  const int32_t* n_tiles;
  void* c;                  // output
  int out_mode;             // down: kOutF32, kOutBf16 or kOutCombine
  const float* topk_w;      // kOutCombine: weight of each (t, k)
  float* zero_out;          // gate/up: if set, the launch zeroes zero_n floats here
  size_t zero_n;
  int T, E, topk, R;
  int N, Kdim;              // weight matrix [N][Kdim]
  int I;                    // gate/up: intermediate size (h width)
  int max_tiles;
};
// Down-GEMM epilogues: y fp32, y bf16, or the weighted rows added into out.
constexpr int kOutF32 = 0;
constexpr int kOutBf16 = 1;
constexpr int kOutCombine = 2;
hipError_t launch_gemm_gate_up(const GemmArgs& g, hipStream_t stream);
hipError_t launch_gemm_down(const GemmArgs& g, hipStream_t stream);

// Unfused variant, step 1: w_bf16[e] = bf16(fma(q, scale, bias)) for every
// expert e < n_exp with counts[e] > 0 (all of them when counts is null).
struct DequantArgs {
  const uint8_t* codes;
  const uint16_t* scales;
  const uint16_t* biases;
  const int32_t* counts;
  uint16_t* out;
  int n_exp, N, K;
};
hipError_t launch_dequant(const DequantArgs& d, hipStream_t stream);

// Decode-shape layer (at most 16 tokens): fp32 piece-major router copy
// (once per model), router + grouping, split-reduction expert GEMVs.
struct DecodeRouteArgs {
  const uint16_t* x;
  const uint16_t* wt;  // [H/8][E][8] bf16, piece-major
  const float* router_bias;
  float* logits;  // workspace [T][E] fp32
  int T, H, E, K, norm_topk, has_shared;
  moe_route_out out;
};
hipError_t launch_decode_prep(const uint16_t* wr, int H, int E, uint16_t* wt, hipStream_t stream);
hipError_t launch_decode_route(const DecodeRouteArgs& a, hipStream_t stream);
hipError_t launch_decode_gemv(const GemmArgs& g, bool gate_up, hipStream_t stream);

struct CombineArgs {
  const void* y;            // fp32 or bf16 [R(+T)][H]
  int y_bf16;
  const float* topk_w;
  const int32_t* inv_pos;
  float* out;
  int T, H, K, R, has_shared;
};
hipError_t launch_combine(const CombineArgs& c, hipStream_t stream);

}  // namespace moeq4
