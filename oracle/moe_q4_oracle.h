/*
 * CPU oracle for the prefill sparse-MoE layer with groupwise-affine 4-bit
 * expert weights.  TEST INFRASTRUCTURE ONLY: the test suite, the smoke check
 * and the benchmark's CPU-baseline leg may call it; the GPU library never
 * does, and the two share no code.
 *
 * All pointers are HOST pointers.  Layouts are row-major and contiguous:
 *   x         bf16 bits [T][H]
 *   wr        bf16 bits [E][H]           router weight
 *   rb        fp32 [E] or NULL           router bias (added after the sum)
 *   codes     u8   [N][K/2]              element k in bits 4*(k&1) of byte k/2
 *   scales    bf16 bits [N][K/64]        w = q*scale + bias per 64-group
 *   biases    bf16 bits [N][K/64]
 * Expert tensors are stacked over experts: [E][N][...].
 * Return value: 0 on success, -1 on a bad argument.
 */
#ifndef MOE_Q4_ORACLE_H
#define MOE_Q4_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int moe_ref_logits(int T, int H, int E, const uint16_t* x, const uint16_t* wr,
                   const float* rb, float* logits, int nthreads);
int moe_ref_topk(int T, int E, int K, int norm_topk, const float* logits,
                 int32_t* ids, float* w);
int moe_ref_histogram(int R, int E, const int32_t* ids, int32_t* counts);
int moe_ref_scan(int E, const int32_t* counts, int32_t* offsets);
int moe_ref_scatter(int T, int K, const int32_t* ids, const int32_t* offsets,
                    int E, int32_t* sorted_idx, int32_t* inv_pos);
int moe_ref_block_map(int E, int T, int K, int has_shared, int BM,
                      const int32_t* counts, const int32_t* offsets,
                      int max_tiles, int32_t* block_map, int32_t* n_tiles);
int moe_ref_dequant(int N, int K, const uint8_t* codes, const uint16_t* scales,
                    const uint16_t* biases, uint16_t* w);
int moe_ref_route(int T, int H, int E, int K, int norm_topk, const uint16_t* x,
                  const uint16_t* wr, const float* rb, float* logits_or_null,
                  int32_t* ids, float* w, int32_t* counts, int32_t* offsets,
                  int32_t* sorted_idx, int32_t* inv_pos, int nthreads);
int moe_ref_layer_forward(
    int T, int H, int I, int E, int K, int norm_topk, int has_shared,
    const uint16_t* x, const uint16_t* wr, const float* rb,
    const uint8_t* gu_codes, const uint16_t* gu_scales, const uint16_t* gu_biases,
    const uint8_t* d_codes, const uint16_t* d_scales, const uint16_t* d_biases,
    const uint8_t* sgu_codes, const uint16_t* sgu_scales, const uint16_t* sgu_biases,
    const uint8_t* sd_codes, const uint16_t* sd_scales, const uint16_t* sd_biases,
    float* out, int32_t* ids, float* w, int32_t* counts, int32_t* offsets,
    int32_t* sorted_idx, int32_t* inv_pos, uint16_t* h_or_null, float* y_or_null,
    int nthreads);
double moe_ref_bf16_from_f64(double v);   /* RNE rounding helper, exposed for pins */
uint16_t moe_ref_bf16_bits_from_f64(double v);

#ifdef __cplusplus
}
#endif
#endif
