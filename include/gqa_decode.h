/* libmoeq4: batch-1 decode attention with grouped KV heads.
 *
 * The pages' model has full-attention layers with 16 query heads over 2 KV
 * heads (grouped-query attention); a decode step attends one new token over
 * the whole KV cache, so its cost is reading the cache.  Their decode kernel
 * lets the query heads that share a KV head share one load of each KV row
 * (GQA packing: 8 separate KV requests become 2 shared loads), reads the
 * cache coalesced, and uses a fixed block layout for long contexts
 * ("Perplexity Lily 오픈소스 공개", alltoptrend.co.kr, sections 4 and 6-2;
 * "Apple silicon용 Lily, Qwen 추론 최적화", aitrends.kr, section
 * "Decode의 토큰 단위 최적화").
 *
 * For query head h, with G = HQ / HKV query heads per KV head and g = h / G:
 *   s_j = scale * (q_h . K_g[j]),  p = softmax(s) over j < L,
 *   out_h = sum_j p_j V_g[j].
 *
 * KV cache layout (fixed blocks of GQA_BLOCK = 32 tokens per KV head; token
 * j is entry j % 32 of block j / 32; entries past L in the last block are
 * never used, whatever they hold):
 *   k_cache  bf16 [nblocks][HKV][32][D]   token-major inside a block
 *   v_cache  bf16 [nblocks][HKV][D][32]   dimension-major inside a block
 * with nblocks >= ceil(L / 32).
 *
 * Conventions are those of moe_q4.h: device pointers, caller-owned buffers,
 * every pointer 16-byte aligned, arguments checked before any HIP call (the
 * MOE_ERR_* codes), asynchronous on `stream` (NULL = the default stream).
 */
#ifndef GQA_DECODE_H
#define GQA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#include "moe_q4.h"

#ifdef __cplusplus
extern "C" {
#endif

#define GQA_BLOCK 32

typedef struct {
  int32_t L;    /* context length (tokens in the cache), >= 0 */
  int32_t HQ;   /* query heads */
  int32_t HKV;  /* KV heads; HQ must be a multiple, with HQ / HKV <= 16 */
  int32_t D;    /* head dimension: 128 or 256 */
  float scale;  /* score scale, usually 1 / sqrt(D) */
} gqa_decode_desc;

/* Bytes of workspace gqa_decode_attention needs for this descriptor
 * (partial softmax sums of the context splits).  Returns MOE_OK or
 * MOE_ERR_INVALID_ARGUMENT / MOE_ERR_UNSUPPORTED_SHAPE. */
int gqa_decode_workspace_size(const gqa_decode_desc* desc, size_t* bytes);

/* One decode step of attention.
 *   q     bf16 [HQ][D], the new token's queries
 *   k_cache, v_cache as above (may be NULL when L == 0)
 *   out   fp32 [HQ][D] (written; zeros when L == 0)
 *   ws    device workspace of at least gqa_decode_workspace_size() bytes
 * Returns MOE_OK, MOE_ERR_INVALID_ARGUMENT, MOE_ERR_UNSUPPORTED_SHAPE,
 * MOE_ERR_WORKSPACE_TOO_SMALL, MOE_ERR_MISALIGNED or MOE_ERR_HIP. */
int gqa_decode_attention(const gqa_decode_desc* desc, const uint16_t* q, const uint16_t* k_cache,
                         const uint16_t* v_cache, float* out, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* GQA_DECODE_H */
