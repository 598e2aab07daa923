/* libmoeq4: the Gated DeltaNet prefill scan.
 *
 * The pages pair the MoE layers with Gated DeltaNet layers: linear attention
 * that replaces the growing KV cache by a fixed-size recurrent state, updated
 * token by token with a gate and the current token's delta update, so that
 * each token depends on the state the previous ones left ("Perplexity Lily
 * 오픈소스 공개", alltoptrend.co.kr, section 4; "Apple silicon용 Lily, Qwen
 * 추론 최적화", aitrends.kr, glossary entry on Gated DeltaNet).  Their prefill
 * kernel gives each state column to one SIMD group, keeps the fp32 state in
 * registers for the whole scan and writes it once at the end (aitrends.kr,
 * section "GPU 상주와 메모리 절감").
 *
 * The update is the published gated delta rule of that layer.  Per value
 * head, with the state S a DV x DK matrix (row i maps keys to value i):
 *
 *   S_t = alpha_t * S_{t-1} + beta_t * (v_t - alpha_t * S_{t-1} k_t) k_t^T
 *   o_t = S_t q_t
 *
 * Value head hv reads key head hv / (HV / HK).  Normalising q and k, the
 * gate and write-strength activations and the projections around the scan
 * are the caller's: they arrive as inputs.  Arithmetic is fp32; the state
 * stays on chip from the first token to the last.
 *
 * Conventions are those of moe_q4.h: device pointers, caller-owned buffers,
 * every pointer 16-byte aligned, arguments checked before any HIP call (the
 * MOE_ERR_* codes), asynchronous on `stream` (NULL = the default stream).
 */
#ifndef GDN_SCAN_H
#define GDN_SCAN_H

#include <stdint.h>

#include "moe_q4.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t T;   /* tokens, >= 0; T == 0 copies state_in (or zeros) to state_out */
  int32_t HK;  /* key heads (q and k), >= 1 */
  int32_t HV;  /* value heads, a multiple of HK */
  int32_t DK;  /* key dimension: 64 or 128 */
  int32_t DV;  /* value dimension: a positive multiple of 16 */
} gdn_scan_desc;

/* One prefill scan over T tokens.
 *   q, k      bf16 bits [T][HK][DK]
 *   v         bf16 bits [T][HV][DV]
 *   alpha     fp32 [T][HV], the gate in (0, 1]
 *   beta      fp32 [T][HV], the write strength in [0, 1]
 *   state_in  fp32 [HV][DV][DK], or NULL for a zero state
 *   o         fp32 [T][HV][DV]   (written)
 *   state_out fp32 [HV][DV][DK]  (written; may not alias state_in)
 * Returns MOE_OK, MOE_ERR_INVALID_ARGUMENT (NULL pointer, negative size,
 * state_out == state_in), MOE_ERR_UNSUPPORTED_SHAPE (DK, DV or HV/HK not as
 * above), MOE_ERR_MISALIGNED or MOE_ERR_HIP. */
int gdn_prefill_scan(const gdn_scan_desc* desc, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                     const float* alpha, const float* beta, const float* state_in, float* o, float* state_out,
                     void* stream);

#ifdef __cplusplus
}
#endif
#endif /* GDN_SCAN_H */
