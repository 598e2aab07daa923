/* CPU oracle of the Gated DeltaNet prefill scan -- TEST INFRASTRUCTURE ONLY.
 *
 * The pages describe the Gated DeltaNet layer as a linear-attention layer
 * (proposed by NVIDIA) that keeps a fixed-size recurrent state in place of
 * a growing KV cache and updates it, token after token, with a gate and a
 * delta update from the current token ("Perplexity Lily 오픈소스 공개",
 * alltoptrend.co.kr, section 4; "Apple silicon용 Lily, Qwen 추론 최적화",
 * aitrends.kr, glossary entry on Gated DeltaNet).  Their prefill kernel keeps
 * the fp32 state in registers for the whole scan and writes it once at the
 * end (aitrends.kr, section "GPU 상주와 메모리 절감").
 *
 * The pages give no formula.  This oracle takes the published gated delta
 * rule of that layer: per value head, with the state S a DV x DK matrix
 * mapping keys to values,
 *
 *   S_t = alpha_t * S_{t-1} + beta_t * (v_t - alpha_t * S_{t-1} k_t) k_t^T
 *   o_t = S_t q_t
 *
 * (the same as S_t = S_{t-1} alpha_t (I - beta_t k_t k_t^T) + beta_t v_t k_t^T),
 * where alpha_t in (0, 1] is the gate (decay) and beta_t in [0, 1] the write
 * strength of token t.  q and k belong to key heads; value head hv reads key
 * head hv / (HV / HK).  Normalisation of q and k, the gate and beta
 * activations and the output projection are outside the scan: they arrive
 * as inputs.
 *
 * Everything is fp64, the rows of S in order, each sum over the key index
 * in ascending order.  q, k and v are bf16 bit patterns (converted exactly);
 * alpha, beta and the initial state are fp32.
 */
#include <stddef.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double bf16_bits_to_f64(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* q, k: [T][HK][DK] bf16 bits; v: [T][HV][DV] bf16 bits; alpha, beta: [T][HV];
 * state_in: [HV][DV][DK] or NULL (zeros); o: [T][HV][DV]; state_out:
 * [HV][DV][DK].  Returns 0, or -1 on bad sizes. */
int gdn_ref_scan(int T, int HK, int HV, int DK, int DV, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                 const float* alpha, const float* beta, const float* state_in, double* o, double* state_out) {
  if (T < 0 || HK <= 0 || HV <= 0 || DK <= 0 || DV <= 0 || HV % HK != 0) return -1;
  const int group = HV / HK;  /* value heads per key head */
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int hv = 0; hv < HV; ++hv) {
    const int hk = hv / group;
    double* S = (double*)malloc((size_t)DV * DK * sizeof(double));
    double* kk = (double*)malloc((size_t)DK * sizeof(double));
    double* qq = (double*)malloc((size_t)DK * sizeof(double));
    if (!S || !kk || !qq) {
#pragma omp atomic write
      bad = 1;
      free(S);
      free(kk);
      free(qq);
      continue;
    }
    for (size_t i = 0; i < (size_t)DV * DK; ++i)
      S[i] = state_in ? (double)state_in[(size_t)hv * DV * DK + i] : 0.0;
    for (int t = 0; t < T; ++t) {
      const double a = (double)alpha[(size_t)t * HV + hv];
      const double b = (double)beta[(size_t)t * HV + hv];
      for (int j = 0; j < DK; ++j) {
        kk[j] = bf16_bits_to_f64(k[((size_t)t * HK + hk) * DK + j]);
        qq[j] = bf16_bits_to_f64(q[((size_t)t * HK + hk) * DK + j]);
      }
      for (int i = 0; i < DV; ++i) {
        double* row = S + (size_t)i * DK;
        /* what the decayed state recalls for k_t */
        double recall = 0.0;
        for (int j = 0; j < DK; ++j) recall += row[j] * kk[j];
        recall *= a;
        /* delta update: move the recall for k_t towards v_t by beta_t */
        const double vi = bf16_bits_to_f64(v[((size_t)t * HV + hv) * DV + i]);
        const double c = b * (vi - recall);
        for (int j = 0; j < DK; ++j) row[j] = a * row[j] + c * kk[j];
        double out = 0.0;
        for (int j = 0; j < DK; ++j) out += row[j] * qq[j];
        o[((size_t)t * HV + hv) * DV + i] = out;
      }
    }
    memcpy(state_out + (size_t)hv * DV * DK, S, (size_t)DV * DK * sizeof(double));
    free(S);
    free(kk);
    free(qq);
  }
  return bad ? -1 : 0;
}

/* OpenMP threads of the next calls (n <= 0 leaves the default).  Threading
 * only: the arithmetic and its order per output are the same for any n. */
void gdn_ref_set_threads(int n) {
  if (n > 0) omp_set_num_threads(n);
}
