/*
 * CPU oracle for the prefill sparse-MoE layer (TEST INFRASTRUCTURE ONLY).
 *
 * Plain, slow, obviously correct loops.  Only the test suite, the smoke check
 * and the benchmark's CPU-baseline leg use it; the GPU library never links,
 * loads or calls it, and it includes nothing from the GPU library.
 *
 * Sources, cited by page and section:
 *  [P1] "Perplexity Lily 오픈소스 공개 — Apple Silicon에서 Qwen3.6-35B-A3B를 더
 *       빠르게 돌리는 Rust + Metal 추론 엔진" (alltoptrend.co.kr):
 *       §4 (256 experts, 8 chosen per token; uneven expert groups),
 *       §5-1 (groupwise affine 4-bit weights, 64 weights per bf16 scale+bias
 *       pair, dequant to bf16 inside the grouped GEMM, FP32 accumulation),
 *       §5-2 (histogram, prefix scan, scatter and block map on the GPU;
 *       bounded prefill chunks).
 *  [P3] "Apple silicon용 Lily, Qwen 추론 최적화" (aitrends.kr):
 *       section "Qwen 구조와 Prefill 경로" (8 of 256 experts plus 1 shared
 *       expert; Q4 weights restored to bf16 tile by tile),
 *       section "GPU 상주와 메모리 절감" (histogram -> prefix scan for start
 *       offsets -> scatter of rows into expert groups),
 *       glossary "그룹 단위 Affine 4비트 양자화" (4-bit codes, bf16 scale and
 *       bias per 64-weight group).
 * The router rule (softmax over logits, top-k, ties to the lower expert), the
 * SwiGLU expert FFN, the gate/up row split and the top-k weighted combine are
 * not on the pages; they are the layer's definition as taken for this build.
 *
 * Precision: router logits in fp32, summed over the hidden axis one column
 * at a time in ascending order (the plain loop); this decides integer expert
 * ids, so both implementations take that decision in the same precision and
 * order.  The pages fix no summation order; the plain sequential one is the
 * reading taken.  Dequantized weights are
 * bf16 (the pages' matrix-op input format); the expert h activation is
 * rounded to bf16 before the down projection (same reason); every other sum
 * is accumulated in fp64 and rounded once.
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -fopenmp -shared -fPIC.
 */
#include "moe_q4_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- bf16 helpers (own implementation, RNE, no flush-to-zero) ---------- */

static float bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* Round a double to the nearest bfloat16 (ties to even) in one step, so no
 * double rounding through fp32 happens.  bf16 keeps 8 significant bits and
 * fp32's exponent range (subnormal quantum 2^-133). */
double moe_ref_bf16_from_f64(double v) {
  if (isnan(v) || isinf(v) || v == 0.0) return v;
  double a = fabs(v);
  int ex;
  (void)frexp(a, &ex);          /* a = f * 2^ex, 0.5 <= f < 1 */
  int q = ex - 8;               /* quantum of an 8-bit significand */
  if (q < -133) q = -133;
  double m = nearbyint(ldexp(a, -q)); /* default rounding mode: ties to even */
  double r = ldexp(m, q);
  if (r >= ldexp(1.0, 128)) r = INFINITY;
  return v < 0 ? -r : r;
}

uint16_t moe_ref_bf16_bits_from_f64(double v) {
  if (isnan(v)) return 0x7FC0;
  float f = (float)moe_ref_bf16_from_f64(v); /* exact: already a bf16 value */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

static void set_threads(int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
}

/* ---- step 1: router logits ------------------------------------------------
 * l[t,e] = sum_h x[t,h] * Wr[e,h] (+ rb[e]) in fp32: acc starts at 0, adds
 * the products for h = 0, 1, ..., H-1 in that order, then adds rb[e].
 * Each bf16*bf16 product is exact in fp32, so contraction cannot change it. */
int moe_ref_logits(int T, int H, int E, const uint16_t* x, const uint16_t* wr,
                   const float* rb, float* logits, int nthreads) {
  if (T < 0 || H <= 0 || E <= 0 || (T > 0 && (!x || !wr || !logits))) return -1;
  set_threads(nthreads);
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    for (int e = 0; e < E; ++e) {
      float acc = 0.0f;
      for (int h = 0; h < H; ++h) {
        float p = bf16_to_f32(x[(size_t)t * H + h]) * bf16_to_f32(wr[(size_t)e * H + h]);
        acc = acc + p;
      }
      if (rb) acc = acc + rb[e];
      logits[(size_t)t * E + e] = acc;
    }
  }
  return 0;
}

/* ---- step 2: top-k and combine weights ------------------------------------
 * [P1 §4], [P3 "Qwen 구조와 Prefill 경로"]: each token picks K of E experts.
 * Order: logit descending, ties to the lower expert index; that order is also
 * the slot order.  Weights: softmax over the K selected logits
 * (norm_topk=1), which equals a softmax over all E renormalized over the
 * chosen K; norm_topk=0 keeps the softmax over all E.  fp64, rounded once. */
int moe_ref_topk(int T, int E, int K, int norm_topk, const float* logits,
                 int32_t* ids, float* w) {
  if (T < 0 || E <= 0 || K <= 0 || K > E) return -1;
  char* taken = (char*)malloc((size_t)E);
  if (!taken) return -1;
  for (int t = 0; t < T; ++t) {
    const float* l = logits + (size_t)t * E;
    memset(taken, 0, (size_t)E);
    for (int k = 0; k < K; ++k) {
      int best = -1;
      for (int e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || l[e] > l[best]) best = e; /* strict '>' keeps the lower e on ties */
      }
      taken[best] = 1;
      ids[(size_t)t * K + k] = best;
    }
    double m = (double)l[ids[(size_t)t * K]];
    double den = 0.0;
    if (norm_topk) {
      for (int k = 0; k < K; ++k) den += exp((double)l[ids[(size_t)t * K + k]] - m);
    } else {
      for (int e = 0; e < E; ++e) den += exp((double)l[e] - m);
    }
    for (int k = 0; k < K; ++k)
      w[(size_t)t * K + k] = (float)(exp((double)l[ids[(size_t)t * K + k]] - m) / den);
  }
  free(taken);
  return 0;
}

/* ---- step 3: histogram ([P1 §5-2], [P3 "GPU 상주와 메모리 절감"]) -------- */
int moe_ref_histogram(int R, int E, const int32_t* ids, int32_t* counts) {
  if (R < 0 || E <= 0) return -1;
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int r = 0; r < R; ++r) {
    if (ids[r] < 0 || ids[r] >= E) return -1;
    counts[ids[r]] += 1;
  }
  return 0;
}

/* ---- step 4: exclusive prefix scan -> group start offsets --------------- */
int moe_ref_scan(int E, const int32_t* counts, int32_t* offsets) {
  if (E <= 0) return -1;
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  return 0;
}

/* ---- step 5: scatter rows into expert groups -----------------------------
 * The scattered "rows" are indices (t*K + k); the GEMM gathers activations.
 * Stable: within a group, rows keep ascending (t, k) order. */
int moe_ref_scatter(int T, int K, const int32_t* ids, const int32_t* offsets,
                    int E, int32_t* sorted_idx, int32_t* inv_pos) {
  if (T < 0 || K <= 0 || E <= 0) return -1;
  int32_t* cursor = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
  if (!cursor) return -1;
  for (int e = 0; e < E; ++e) cursor[e] = offsets[e];
  for (int t = 0; t < T; ++t) {
    for (int k = 0; k < K; ++k) {
      int r = t * K + k;
      int p = cursor[ids[r]]++;
      sorted_idx[p] = r;
      inv_pos[r] = p;
    }
  }
  free(cursor);
  return 0;
}

/* ---- step 6: tile block map ([P1 §5-2]) -----------------------------------
 * For e = 0..E-1, then the shared expert (index E, rows R..R+T-1):
 * tiles of at most BM rows, (expert, first row, row count, 0).  Returns -1 if
 * max_tiles is too small. */
int moe_ref_block_map(int E, int T, int K, int has_shared, int BM,
                      const int32_t* counts, const int32_t* offsets,
                      int max_tiles, int32_t* block_map, int32_t* n_tiles) {
  if (E <= 0 || T < 0 || K <= 0 || BM <= 0) return -1;
  int n = 0;
  int R = T * K;
  for (int e = 0; e <= E; ++e) {
    int c, base;
    if (e < E) {
      c = counts[e];
      base = offsets[e];
    } else {
      if (!has_shared) break;
      c = T;
      base = R;
    }
    for (int r = 0; r < c; r += BM) {
      if (n >= max_tiles) return -1;
      block_map[4 * n + 0] = e;
      block_map[4 * n + 1] = base + r;
      block_map[4 * n + 2] = (c - r < BM) ? (c - r) : BM;
      block_map[4 * n + 3] = 0;
      ++n;
    }
  }
  *n_tiles = n;
  return 0;
}

/* ---- step 7: dequant ([P1 §5-1], [P3 glossary]) ---------------------------
 * q = 4-bit code (element k in the low nibble of byte k/2 when k is even),
 * W[n][k] = bf16_rne(fma(q, scale[n][k/64], bias[n][k/64])). */
int moe_ref_dequant(int N, int K, const uint8_t* codes, const uint16_t* scales,
                    const uint16_t* biases, uint16_t* w) {
  if (N <= 0 || K <= 0 || K % 64) return -1;
#pragma omp parallel for schedule(static)
  for (int n = 0; n < N; ++n) {
    for (int k = 0; k < K; ++k) {
      uint8_t byte = codes[(size_t)n * (K / 2) + k / 2];
      int q = (k & 1) ? (byte >> 4) : (byte & 15);
      float s = bf16_to_f32(scales[(size_t)n * (K / 64) + k / 64]);
      float b = bf16_to_f32(biases[(size_t)n * (K / 64) + k / 64]);
      float v = fmaf((float)q, s, b);
      w[(size_t)n * K + k] = moe_ref_bf16_bits_from_f64((double)v);
    }
  }
  return 0;
}

int moe_ref_route(int T, int H, int E, int K, int norm_topk, const uint16_t* x,
                  const uint16_t* wr, const float* rb, float* logits_or_null,
                  int32_t* ids, float* w, int32_t* counts, int32_t* offsets,
                  int32_t* sorted_idx, int32_t* inv_pos, int nthreads) {
  if (T < 0 || H <= 0 || E <= 0 || K <= 0 || K > E) return -1;
  float* logits = logits_or_null;
  if (!logits) {
    logits = (float*)malloc(sizeof(float) * ((size_t)T * E + 1));
    if (!logits) return -1;
  }
  int rc = moe_ref_logits(T, H, E, x, wr, rb, logits, nthreads);
  if (!rc) rc = moe_ref_topk(T, E, K, norm_topk, logits, ids, w);
  if (!rc) rc = moe_ref_histogram(T * K, E, ids, counts);
  if (!rc) rc = moe_ref_scan(E, counts, offsets);
  if (!rc) rc = moe_ref_scatter(T, K, ids, offsets, E, sorted_idx, inv_pos);
  if (!logits_or_null) free(logits);
  return rc;
}

/* ---- steps 8-9: one expert's SwiGLU FFN over its group of rows ------------
 * g_j = sum_h x[t,h] Wg[j,h], u_j = sum_h x[t,h] Wu[j,h] (fp64, rounded to
 * fp32); h_j = bf16(silu(g_j) * u_j) from those fp32 values in fp64;
 * y_n = fp32(sum_j h_j Wd[n,j]) in fp64. */
static int expert_ffn(int H, int I, int nrows, const int32_t* row_token,
                      const int32_t* row_pos, const uint16_t* x,
                      const uint8_t* gu_c, const uint16_t* gu_s, const uint16_t* gu_b,
                      const uint8_t* d_c, const uint16_t* d_s, const uint16_t* d_b,
                      uint16_t* hbuf, float* y) {
  size_t ngu = (size_t)2 * I * H, nd = (size_t)H * I;
  uint16_t* wgu_bits = (uint16_t*)malloc(ngu * sizeof(uint16_t));
  uint16_t* wd_bits = (uint16_t*)malloc(nd * sizeof(uint16_t));
  float* wgu = (float*)malloc(ngu * sizeof(float));
  float* wd = (float*)malloc(nd * sizeof(float));
  if (!wgu_bits || !wd_bits || !wgu || !wd) {
    free(wgu_bits); free(wd_bits); free(wgu); free(wd);
    return -1;
  }
  moe_ref_dequant(2 * I, H, gu_c, gu_s, gu_b, wgu_bits);
  moe_ref_dequant(H, I, d_c, d_s, d_b, wd_bits);
  for (size_t i = 0; i < ngu; ++i) wgu[i] = bf16_to_f32(wgu_bits[i]);
  for (size_t i = 0; i < nd; ++i) wd[i] = bf16_to_f32(wd_bits[i]);
  free(wgu_bits);
  free(wd_bits);

#pragma omp parallel for schedule(dynamic, 1)
  for (int r = 0; r < nrows; ++r) {
    const int t = row_token[r];
    const size_t p = (size_t)row_pos[r];
    const uint16_t* xt = x + (size_t)t * H;
    uint16_t* hp = hbuf + p * I;
    for (int j = 0; j < I; ++j) {
      const float* wg = wgu + (size_t)j * H;
      const float* wu = wgu + (size_t)(I + j) * H;
      double g = 0.0, u = 0.0;
      for (int h = 0; h < H; ++h) {
        double xv = (double)bf16_to_f32(xt[h]);
        g += xv * (double)wg[h];
        u += xv * (double)wu[h];
      }
      float gf = (float)g, uf = (float)u;
      double silu = (double)gf / (1.0 + exp(-(double)gf));
      hp[j] = moe_ref_bf16_bits_from_f64(silu * (double)uf);
    }
    float* yp = y + p * H;
    for (int n = 0; n < H; ++n) {
      const float* wrow = wd + (size_t)n * I;
      double acc = 0.0;
      for (int j = 0; j < I; ++j) acc += (double)bf16_to_f32(hp[j]) * (double)wrow[j];
      yp[n] = (float)acc;
    }
  }
  free(wgu);
  free(wd);
  return 0;
}

/* ---- the whole layer, steps 1-10 -------------------------------------------
 * Row numbering: routed rows are the sorted positions 0..R-1 (R = T*K); the
 * shared expert's rows are R..R+T-1 in token order.
 * Step 10 (combine): out[t] = y[R+t] + sum_k w[t,k] * y[inv_pos[t*K+k]],
 * fp64 in exactly that order, rounded once to fp32. */
int moe_ref_layer_forward(
    int T, int H, int I, int E, int K, int norm_topk, int has_shared,
    const uint16_t* x, const uint16_t* wr, const float* rb,
    const uint8_t* gu_codes, const uint16_t* gu_scales, const uint16_t* gu_biases,
    const uint8_t* d_codes, const uint16_t* d_scales, const uint16_t* d_biases,
    const uint8_t* sgu_codes, const uint16_t* sgu_scales, const uint16_t* sgu_biases,
    const uint8_t* sd_codes, const uint16_t* sd_scales, const uint16_t* sd_biases,
    float* out, int32_t* ids, float* w, int32_t* counts, int32_t* offsets,
    int32_t* sorted_idx, int32_t* inv_pos, uint16_t* h_or_null, float* y_or_null,
    int nthreads) {
  if (T < 0 || H <= 0 || I <= 0 || E <= 0 || K <= 0 || K > E || H % 64 || I % 64) return -1;
  if (T == 0) return 0;
  if (has_shared && (!sgu_codes || !sd_codes)) return -1;
  set_threads(nthreads);
  int rc = moe_ref_route(T, H, E, K, norm_topk, x, wr, rb, NULL, ids, w, counts,
                         offsets, sorted_idx, inv_pos, nthreads);
  if (rc) return rc;

  const size_t R = (size_t)T * K;
  const size_t rows = R + (has_shared ? (size_t)T : 0);
  uint16_t* hbuf = h_or_null ? h_or_null : (uint16_t*)malloc(rows * I * sizeof(uint16_t));
  float* y = y_or_null ? y_or_null : (float*)malloc(rows * H * sizeof(float));
  int32_t* row_token = (int32_t*)malloc(sizeof(int32_t) * (R > (size_t)T ? R : (size_t)T));
  int32_t* row_pos = (int32_t*)malloc(sizeof(int32_t) * (R > (size_t)T ? R : (size_t)T));
  if (!hbuf || !y || !row_token || !row_pos) { rc = -1; goto done; }

  const size_t gu_codes_e = (size_t)2 * I * (H / 2), gu_grp_e = (size_t)2 * I * (H / 64);
  const size_t d_codes_e = (size_t)H * (I / 2), d_grp_e = (size_t)H * (I / 64);
  for (int e = 0; e < E && !rc; ++e) {
    int c = counts[e];
    if (c == 0) continue; /* an empty group touches no weights */
    for (int r = 0; r < c; ++r) {
      row_pos[r] = offsets[e] + r;
      row_token[r] = sorted_idx[offsets[e] + r] / K;
    }
    rc = expert_ffn(H, I, c, row_token, row_pos, x,
                    gu_codes + e * gu_codes_e, gu_scales + e * gu_grp_e, gu_biases + e * gu_grp_e,
                    d_codes + e * d_codes_e, d_scales + e * d_grp_e, d_biases + e * d_grp_e,
                    hbuf, y);
  }
  if (!rc && has_shared) {
    for (int t = 0; t < T; ++t) {
      row_pos[t] = (int32_t)(R + t);
      row_token[t] = t;
    }
    rc = expert_ffn(H, I, T, row_token, row_pos, x, sgu_codes, sgu_scales, sgu_biases,
                    sd_codes, sd_scales, sd_biases, hbuf, y);
  }
  if (!rc) {
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
      for (int n = 0; n < H; ++n) {
        double acc = has_shared ? (double)y[(R + t) * H + n] : 0.0;
        for (int k = 0; k < K; ++k) {
          size_t p = (size_t)inv_pos[(size_t)t * K + k];
          acc += (double)w[(size_t)t * K + k] * (double)y[p * H + n];
        }
        out[(size_t)t * H + n] = (float)acc;
      }
    }
  }
done:
  if (!h_or_null) free(hbuf);
  if (!y_or_null) free(y);
  free(row_token);
  free(row_pos);
  return rc;
}
