/* libmoeq4: the two prefill alternatives the fused, GPU-resident layer is
 * measured against.
 *
 * The pages credit two changes with most of the prefill gain at 512 tokens:
 *  - dequantizing the 4-bit weights tile by tile inside the grouped GEMM
 *    instead of writing the whole bf16 weight array to memory and reading it
 *    back ("Perplexity Lily 오픈소스 공개", alltoptrend.co.kr, section 5-1;
 *    "Apple silicon용 Lily, Qwen 추론 최적화", aitrends.kr, section
 *    "Qwen 구조와 Prefill 경로");
 *  - keeping histogram, scan, scatter and block map in one GPU submission
 *    instead of letting the host read the routing result before it submits
 *    the expert GEMMs (alltoptrend.co.kr, section 5-2; aitrends.kr, section
 *    "GPU 상주와 메모리 절감").
 * These entry points rebuild each alternative on the same kernels so that
 * the two gains can be measured on this hardware.  They compute the same
 * results as moe_layer_forward: the same bf16 weights (w = bf16_rne(fma(q,
 * scale, bias)) in fp32), the same routing, fp32 accumulation.
 *
 * Conventions are those of moe_q4.h (device pointers, caller-owned buffers,
 * 16-byte alignment, checks before any HIP call, T == 0 a no-op), except
 * where an entry point says it synchronizes.
 */
#ifndef MOE_Q4_ABLATION_H
#define MOE_Q4_ABLATION_H

#include "moe_q4.h"

#ifdef __cplusplus
extern "C" {
#endif

/* bf16 weights of n_exp experts, each an [N, K] matrix, bf16 bits
 * [n_exp][N][K] (device). */
typedef struct {
  const uint16_t* w;
  int32_t n_exp, N, K;
} moe_bf16_tensor;

/* Write out[e][n][k] = bf16_rne(fma(q, scale, bias)) (bf16 bits, device,
 * [n_exp][N][K]) for every expert e of w with counts[e] > 0; counts (device,
 * int32 [n_exp], e.g. moe_route_out.counts) may be NULL to write every
 * expert.  Experts with no rows are skipped and their part of `out` is left
 * as it was.  K must be a multiple of 64. */
int moe_dequant_q4_to_bf16(const moe_q4_tensor* w, const int32_t* counts_or_null, uint16_t* out, void* stream);

/* moe_grouped_gemm_q4 with bf16 weights read from memory instead of 4-bit
 * codes dequantized in the kernel: same modes, tiles, row order and
 * epilogues (ws, ws_bytes as there: unused, may be NULL).  w: the E routed
 * experts; w_shared: the shared expert (n_exp = 1), required iff
 * desc->has_shared. */
int moe_grouped_gemm_bf16(const moe_layer_desc* desc, int mode, const void* a, const moe_bf16_tensor* w,
                          const moe_bf16_tensor* w_shared, const moe_route_out* route, void* c, void* ws,
                          size_t ws_bytes, void* stream);

/* moe_layer_forward with a host round trip after routing: the routing
 * kernels run, then the host copies n_tiles back, waits for the stream and
 * launches the GEMMs with exactly n_tiles tiles instead of the host-known
 * bound.  This entry point SYNCHRONIZES `stream` once and therefore cannot
 * be captured into a HIP graph.  Arguments, workspace and combine mode as
 * for moe_layer_forward. */
int moe_layer_forward_host_sync(const moe_layer_desc* desc, const uint16_t* x, const uint16_t* w_router,
                                const float* router_bias, const moe_q4_tensor* w_gate_up,
                                const moe_q4_tensor* w_down, const moe_q4_tensor* shared_gate_up,
                                const moe_q4_tensor* shared_down, float* out,
                                const moe_route_out* route_or_null, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_Q4_ABLATION_H */
