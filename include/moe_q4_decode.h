/* libmoeq4: the decode-shape MoE layer, at most 16 tokens per call.
 *
 * Decode produces one token per sequence at a time, so its cost is the
 * weight bytes moved per token ("Perplexity Lily 오픈소스 공개",
 * alltoptrend.co.kr, section 6; "Apple silicon용 Lily, Qwen 추론 최적화",
 * aitrends.kr, section "Decode의 토큰 단위 최적화").  This path computes
 * exactly what moe_layer_forward computes for the same tokens (the same
 * routing rule and sequential fp32 logits, the same bf16 weights, fp32
 * accumulation) with kernels sized for a handful of rows: an exact router
 * over all experts and a one-workgroup grouping step; the expert FFN runs
 * as GEMVs that split the reduction over the waves of a workgroup (every
 * tile has at most 16 rows).  Only the weights of the chosen experts (plus
 * the shared expert) are read.
 *
 * Conventions are those of moe_q4.h.
 */
#ifndef MOE_Q4_DECODE_H
#define MOE_Q4_DECODE_H

#include "moe_q4.h"

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_DECODE_MAX_TOKENS 16
/* Size of the scratch array behind moe_decode_forward_noalloc: enough for
 * every shape the decode path takes (T <= 16, H and I <= 2048, E <= 256,
 * top_k <= 16). */
#define MOE_DECODE_NOALLOC_SCRATCH_BYTES (4u << 20)

/* Write the router matrix once per model in the layout the decode router
 * reads, piece-major: w_router_pm[p][e][i] = w_router[e][8*p + i] for
 * p < H/8, i < 8 (E * H bf16, device, caller-owned), so that piece p of 64
 * consecutive experts is 1 KB of consecutive memory.  desc supplies H and E
 * (T unused). */
int moe_decode_router_prepare(const moe_layer_desc* desc, const uint16_t* w_router, uint16_t* w_router_pm,
                              void* stream);

/* The layer for 1 <= T <= MOE_DECODE_MAX_TOKENS tokens (T == 0: no-op):
 * routing (every expert's logit as one fp32 chain over h, top_k by (logit
 * descending, expert ascending), weights as in moe_layer_forward), grouping
 * (counts, offsets, stable sorted_idx / inv_pos, a block map with one tile per
 * expert with rows and then the shared expert's), gate/up + SwiGLU, down and
 * the combine, all on `stream`.  w_router_pm: from
 * moe_decode_router_prepare.  Other arguments, the workspace
 * (moe_layer_workspace_size bytes) and the combine mode as for
 * moe_layer_forward. */
int moe_decode_forward(const moe_layer_desc* desc, const uint16_t* x, const uint16_t* w_router_pm,
                       const float* router_bias, const moe_q4_tensor* w_gate_up, const moe_q4_tensor* w_down,
                       const moe_q4_tensor* shared_gate_up, const moe_q4_tensor* shared_down, float* out,
                       const moe_route_out* route_or_null, void* ws, size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * moe_decode_forward with no workspace argument.  Its scratch is a
 * library-owned device array of MOE_DECODE_NOALLOC_SCRATCH_BYTES bytes,
 * one per GPU, held until the process ends; the call allocates and frees
 * nothing.  Arguments otherwise as for moe_decode_forward.  Calls on one GPU
 * share that array, so calls that overlap on one GPU (different streams, or
 * different host threads) race and give unspecified results; calls in order
 * on one stream are safe.  Nothing in the array needs to start at zero.
 * Errors: as moe_decode_forward; MOE_ERR_WORKSPACE_TOO_SMALL if the shape's
 * scratch exceeds the array; MOE_ERR_HIP if the array's device address
 * cannot be taken. */
int moe_decode_forward_noalloc(const moe_layer_desc* desc, const uint16_t* x, const uint16_t* w_router_pm,
                               const float* router_bias, const moe_q4_tensor* w_gate_up,
                               const moe_q4_tensor* w_down, const moe_q4_tensor* shared_gate_up,
                               const moe_q4_tensor* shared_down, float* out, const moe_route_out* route_or_null,
                               void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_Q4_DECODE_H */
