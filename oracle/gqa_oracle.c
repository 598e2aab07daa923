/* CPU oracle of batch-1 GQA decode attention -- TEST INFRASTRUCTURE ONLY.
 *
 * The pages' model has full-attention layers in which 16 query heads share
 * 2 KV heads (grouped-query attention), and a decode step attends the new
 * token's queries over the whole KV cache, so the step reads the cache once
 * per token ("Perplexity Lily 오픈소스 공개", alltoptrend.co.kr, sections 4
 * and 6-2; "Apple silicon용 Lily, Qwen 추론 최적화", aitrends.kr, section
 * "Decode의 토큰 단위 최적화").  For query head h of G = HQ / HKV heads per
 * KV head, g = h / G:
 *
 *   s_j = scale * (q_h . K_g[j]),  p = softmax(s) over j < L,
 *   out_h = sum_j p_j V_g[j]
 *
 * The cache uses the fixed block layout the kernel reads (blocks of 32
 * tokens, per KV head): K[b][g][t][d] (token-major inside the block) and
 * V[b][g][d][t] (dimension-major inside the block), token j = 32 b + t.
 * Everything is fp64; q, K and V are bf16 bit patterns (converted exactly).
 */
#include <math.h>
#include <stddef.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GQA_BLOCK 32

static double bf16_bits_to_f64(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* K element (token j, KV head g, dim d) of the block layout */
static size_t k_index(int j, int g, int d, int HKV, int D) {
  return (((size_t)(j / GQA_BLOCK) * HKV + g) * GQA_BLOCK + (size_t)(j % GQA_BLOCK)) * D + d;
}
/* V element (token j, KV head g, dim d) of the block layout */
static size_t v_index(int j, int g, int d, int HKV, int D) {
  return (((size_t)(j / GQA_BLOCK) * HKV + g) * D + d) * GQA_BLOCK + (size_t)(j % GQA_BLOCK);
}

/* q: [HQ][D] bf16; k, v: the block layout above with ceil(L/32) blocks;
 * out: [HQ][D] (fp64).  L == 0 gives zeros.  Returns 0 or -1. */
int gqa_ref_decode(int L, int HQ, int HKV, int D, double scale, const uint16_t* q, const uint16_t* k,
                   const uint16_t* v, double* out) {
  if (L < 0 || HQ <= 0 || HKV <= 0 || D <= 0 || HQ % HKV != 0) return -1;
  const int G = HQ / HKV;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int h = 0; h < HQ; ++h) {
    const int g = h / G;
    double* s = (double*)malloc((size_t)(L > 0 ? L : 1) * sizeof(double));
    if (!s) {
#pragma omp atomic write
      bad = 1;
      continue;
    }
    double m = -INFINITY;
    for (int j = 0; j < L; ++j) {
      double dot = 0.0;
      for (int d = 0; d < D; ++d)
        dot += bf16_bits_to_f64(q[(size_t)h * D + d]) * bf16_bits_to_f64(k[k_index(j, g, d, HKV, D)]);
      s[j] = scale * dot;
      if (s[j] > m) m = s[j];
    }
    double den = 0.0;
    for (int j = 0; j < L; ++j) {
      s[j] = exp(s[j] - m);
      den += s[j];
    }
    for (int d = 0; d < D; ++d) {
      double acc = 0.0;
      for (int j = 0; j < L; ++j) acc += s[j] * bf16_bits_to_f64(v[v_index(j, g, d, HKV, D)]);
      out[(size_t)h * D + d] = L > 0 ? acc / den : 0.0;
    }
    free(s);
  }
  return bad ? -1 : 0;
}

/* OpenMP threads of the next calls (n <= 0 leaves the default).  Threading
 * only: the arithmetic and its order per output are the same for any n. */
void gqa_ref_set_threads(int n) {
  if (n > 0) omp_set_num_threads(n);
}
