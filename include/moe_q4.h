/*
 * moe_q4.h -- C ABI of libmoeq4.so: the prefill sparse-MoE layer with
 * groupwise-affine 4-bit expert weights, for AMD Instinct MI355X (gfx950).
 *
 * What the layer computes (sources cited by page and section):
 *  - Routing: every token picks top_k of E routed experts plus one always-on
 *    shared expert ("Apple silicon용 Lily, Qwen 추론 최적화", aitrends.kr,
 *    section "Qwen 구조와 Prefill 경로"; "Perplexity Lily 오픈소스 공개",
 *    alltoptrend.co.kr, section 4).  The rule is: router logits
 *    l[t,e] = sum_h x[t,h]*Wr[e,h] (+ bias[e]) in fp32, one sequential
 *    chain in ascending h from zero with the bias added last, top_k by
 *    (logit descending, expert ascending), weights =
 *    softmax of the chosen logits (norm_topk=1) or the full softmax
 *    probability (norm_topk=0).
 *  - Grouping without a host round trip: histogram of expert choices,
 *    exclusive prefix scan into group start offsets, scatter of rows into the
 *    expert groups and a tile block map, all enqueued on the caller's stream
 *    (alltoptrend.co.kr section 5-2; aitrends.kr section "GPU 상주와 메모리
 *    절감").
 *  - Grouped GEMM over the uneven expert groups on 4-bit codes that share
 *    one bf16 scale and one bf16 bias per 64 weights; the weights are
 *    dequantized tile by tile inside the GEMM (q*scale+bias in fp32, rounded
 *    to bf16), never written out, and the products accumulate in fp32
 *    (alltoptrend.co.kr section 5-1; aitrends.kr glossary entry on groupwise
 *    affine 4-bit quantization).  The expert FFN is SwiGLU:
 *    h = bf16(silu(x Wg^T) * (x Wu^T)), y = h Wd^T.
 *  - Combine: out[t] = y_shared[t] + sum_k w[t,k] * y[(t,k)] in fp32.
 *  - Long prompts run as bounded chunks through the same workspace
 *    (alltoptrend.co.kr section 5-2).
 *
 * Conventions for every entry point:
 *  - Tensors are row-major and contiguous.  Pointers named in a struct or
 *    argument are DEVICE pointers unless said otherwise; the descriptor
 *    structs themselves are host memory, read during the call only.
 *  - bf16 tensors are passed as their 16-bit patterns (uint16_t).
 *  - The caller owns every buffer, including the workspace.  The library
 *    allocates nothing, frees nothing and keeps no pointer after returning.
 *  - Calls only enqueue work on `stream` (a hipStream_t; NULL = the null
 *    stream) and never synchronize or read device memory on the host, so
 *    moe_layer_forward can be captured into a HIP graph.  Errors found on
 *    the device surface at the caller's next synchronization.
 *  - Argument checks look only at scalars and pointers, before any HIP call,
 *    so they behave the same on a machine without a GPU.
 *  - Calls are reentrant; concurrent calls need distinct workspaces/outputs.
 *  - Device tensors must be 16-byte aligned (MOE_ERR_MISALIGNED otherwise).
 *  - T == 0 is a successful no-op.
 */
#ifndef MOE_Q4_H
#define MOE_Q4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1,   /* required pointer NULL, dimension < 0 or == 0 where not allowed */
  MOE_ERR_UNSUPPORTED_SHAPE = 2,  /* H or I not a multiple of 64 or above MOE_MAX_REDUCTION, top_k > E,
                                     top_k or E above maximum, tensor shape not matching the descriptor */
  MOE_ERR_WORKSPACE_TOO_SMALL = 3,
  MOE_ERR_MISALIGNED = 4,         /* a device tensor not 16-byte aligned */
  MOE_ERR_HIP = 5                 /* a kernel launch failed */
};

#define MOE_MAX_EXPERTS 256   /* routed experts per layer */
#define MOE_MAX_TOPK 16       /* experts chosen per token */
#define MOE_GROUP_SIZE 64     /* weights per (scale, bias) pair */
#define MOE_MAX_REDUCTION 2048 /* H and I: a GEMM keeps a tile's scales/biases on chip */

/* Groupwise-affine 4-bit weights of n_exp experts, each an [N, K] matrix
 * (N output rows, K reduction columns), stored as
 *   codes  u8        [n_exp][N][K/2]  element k in bits 4*(k&1)..+3 of byte k/2
 *   scales bf16 bits [n_exp][N][K/64]
 *   biases bf16 bits [n_exp][N][K/64]
 * and decoded as w[n][k] = bf16_rne(fma(q, scale[n][k/64], bias[n][k/64])). */
typedef struct {
  const uint8_t* codes;
  const uint16_t* scales;
  const uint16_t* biases;
  int32_t n_exp, N, K;
} moe_q4_tensor;

/* Layer shape.  T tokens in this call (one chunk), hidden size H, expert
 * intermediate size I, E routed experts, top_k chosen per token.
 * group_size: weights per (scale, bias) pair along the reduction axis; the
 * pages give 64 ("Perplexity Lily 오픈소스 공개", section 5-1), the only
 * value the kernels take (MOE_ERR_UNSUPPORTED_SHAPE otherwise).
 * norm_topk: 1 = renormalize the weights over the chosen experts.
 * has_shared: 1 = one shared expert with weight 1 for every token. */
typedef struct {
  int32_t T, H, I, E, top_k;
  int32_t group_size;
  int32_t norm_topk;
  int32_t has_shared;
} moe_layer_desc;

/* Routing results, all device buffers owned by the caller (R = T*top_k):
 *   topk_ids   int32 [T][top_k]  chosen experts, slot order = logit descending
 *   topk_w     fp32  [T][top_k]  combine weights
 *   counts     int32 [E]         rows per expert
 *   offsets    int32 [E+1]       exclusive scan of counts, offsets[E] = R
 *   sorted_idx int32 [R]         row p of the grouped order holds t*top_k+k;
 *                                ascending (t,k) inside each expert group
 *   inv_pos    int32 [R]         inverse permutation: inv_pos[sorted_idx[p]] = p
 *   block_map  int32 [max_tiles][4]  GEMM tiles (expert, first row, rows, 0),
 *                                experts in order then the shared expert
 *                                (expert index E, rows R..R+T-1); at most
 *                                moe_route_block_rows() rows per tile
 *   n_tiles    int32 [1]         number of valid block_map entries
 * Row numbering used by the GEMMs: routed rows are grouped positions
 * 0..R-1, shared-expert rows are R..R+T-1 in token order. */
typedef struct {
  int32_t* topk_ids;
  float* topk_w;
  int32_t* counts;
  int32_t* offsets;
  int32_t* sorted_idx;
  int32_t* inv_pos;
  int32_t* block_map;
  int32_t* n_tiles;
} moe_route_out;

enum moe_gemm_mode {
  MOE_GEMM_GATE_UP_SWIGLU = 0, /* a = x [T][H] bf16 (routed rows gathered through
                                  sorted_idx), w: N=2I (rows [0,I) gate, [I,2I) up),
                                  K=H; c = h bf16 [R(+T)][I] */
  MOE_GEMM_DOWN = 1,           /* a = h bf16 [R(+T)][I]; w: N=H, K=I;
                                  c = y fp32 [R(+T)][H] */
  MOE_GEMM_DOWN_BF16 = 2,      /* as MOE_GEMM_DOWN, c = y rounded to bf16 (RNE) */
  MOE_GEMM_DOWN_COMBINE = 3    /* as MOE_GEMM_DOWN, but each row's result is
                                  weighted (topk_w of its (t,k); 1 for a shared
                                  row) and ADDED into c = out fp32 [T][H] with
                                  fp32 atomics: the combine fused into the
                                  epilogue.  c must hold zeros (or values to add
                                  to) before the call.  The order of the adds is
                                  not fixed, so results may differ in the last
                                  bits from run to run. */
};

/* Element type of the staged expert outputs y handed to moe_combine. */
enum moe_dtype {
  MOE_DTYPE_F32 = 0,
  MOE_DTYPE_BF16 = 1
};

/* How moe_layer_forward_ex hands the down GEMM's rows to the combine. */
enum moe_combine_mode {
  MOE_COMBINE_Y_F32 = 0,    /* y fp32 in the workspace, then moe_combine */
  MOE_COMBINE_Y_BF16 = 1,   /* y bf16 in the workspace, then moe_combine */
  MOE_COMBINE_FUSED = 2     /* MOE_GEMM_DOWN_COMBINE into out (zeroed by the
                               gate/up launch); no y, not bitwise reproducible */
};

/* Human-readable name of a status code (static string). */
const char* moe_status_string(int status);

/* Rows per GEMM tile used in the block map (host-only, pure).  The pages
 * group rows into fixed-height tiles per expert ("Apple silicon용 Lily, Qwen
 * 추론 최적화", section "GPU 상주와 메모리 절감"); this library's tiles hold
 * up to this many rows. */
int moe_route_block_rows(void);

/* Upper bound on block-map entries for `desc`:
 * floor(R/BM) + min(E, R) + (has_shared ? ceil(T/BM) : 0).  Host-only, pure.
 * The GEMM grids are sized from it, so no host round trip is needed to
 * launch them ("Perplexity Lily 오픈소스 공개", section 5-2). */
int moe_route_max_tiles(const moe_layer_desc* desc, int32_t* max_tiles);

/* Workspace bytes of moe_layer_forward for `desc` (host-only, pure): the
 * routing scratch, the routing results (used when route_or_null is NULL),
 * the GEMMs' launch list (the block map's tiles again, in the order the
 * GEMMs start them: max_tiles entries of 16 bytes; for T <= 1536 instead
 * every expert's rows in pieces of at most 64 rows: up to R/64 + min(R, E)
 * (+ ceil(T/64)) entries, and their count), h bf16 [R(+T)][I] and
 * y bf16 [R(+T)][H], each piece 256-byte aligned.  The
 * same buffer also serves moe_route and moe_grouped_gemm_q4.  The pages keep
 * temporary activations of a prompt bounded by running it in chunks through
 * one workspace ("Perplexity Lily 오픈소스 공개", section 5-2; "Apple
 * silicon용 Lily, Qwen 추론 최적화", section "GPU 상주와 메모리 절감").
 * Workspace contents need no initialization and are overwritten.
 * Errors: MOE_ERR_INVALID_ARGUMENT (NULL pointer, bad descriptor),
 * MOE_ERR_UNSUPPORTED_SHAPE. */
int moe_layer_workspace_size(const moe_layer_desc* desc, size_t* bytes);

/* Workspace bytes of moe_layer_forward_ex in `combine_mode` (a
 * moe_combine_mode): y fp32, y bf16, or no y at all (MOE_COMBINE_FUSED). */
int moe_layer_workspace_size_ex(const moe_layer_desc* desc, int combine_mode, size_t* bytes);

/* Workspace bytes moe_route alone needs (host-only, pure): expert histograms
 * per 64-token group, E * (ceil(T/64) rounded up to 4) int32; 256 fp32
 * router-row norms; a piece-major copy of the router matrix, E * H bf16; the
 * approximate router logits as ns partial sums, ns * T * E fp32, with ns = 1,
 * 2, 4 or 8 splits of the hidden axis (the most that keep the logit grid at
 * or below 256 workgroups of 64 tokens x 64 experts); each piece 256-byte
 * aligned.  moe_layer_workspace_size is at least this. */
int moe_route_workspace_size(const moe_layer_desc* desc, size_t* bytes);

/* Routing, steps histogram -> scan -> scatter -> block map included, all on
 * `stream` with no host round trip: per-token selection of top_k of E
 * experts, then a histogram of the choices, an exclusive prefix scan into
 * group offsets, a stable scatter into expert groups and the tile block map
 * ("Perplexity Lily 오픈소스 공개", sections 4 and 5-2; "Apple silicon용 Lily,
 * Qwen 추론 최적화", sections "Qwen 구조와 Prefill 경로" and "GPU 상주와
 * 메모리 절감").
 * x bf16 [T][H], w_router bf16 [E][H], router_bias fp32 [E] or NULL.
 * Writes every field of *out (all required; block_map entries past n_tiles
 * are left unspecified).  ws: at least moe_route_workspace_size bytes.
 * Errors: MOE_ERR_INVALID_ARGUMENT, MOE_ERR_UNSUPPORTED_SHAPE,
 * MOE_ERR_MISALIGNED, MOE_ERR_WORKSPACE_TOO_SMALL, MOE_ERR_HIP. */
int moe_route(const moe_layer_desc* desc, const uint16_t* x, const uint16_t* w_router,
              const float* router_bias, const moe_route_out* out, void* ws, size_t ws_bytes,
              void* stream);

/* One grouped GEMM over the tiles of route->block_map (see moe_gemm_mode),
 * on 4-bit groupwise-affine weights that are dequantized tile by tile inside
 * the GEMM and never written out ("Perplexity Lily 오픈소스 공개", section 5-1;
 * "Apple silicon용 Lily, Qwen 추론 최적화", section "Qwen 구조와 Prefill 경로").
 * w: the E routed experts; w_shared: the shared expert (n_exp = 1), required
 * iff desc->has_shared.  Reads route->sorted_idx, block_map and n_tiles
 * (MOE_GEMM_DOWN_COMBINE also topk_w).  ws, ws_bytes: GEMM scratch; the
 * kernels of this version need none, so ws may be NULL (any ws_bytes is
 * accepted).  Errors: MOE_ERR_INVALID_ARGUMENT (NULL pointer, unknown mode),
 * MOE_ERR_UNSUPPORTED_SHAPE (a weight tensor not matching desc and mode),
 * MOE_ERR_MISALIGNED, MOE_ERR_HIP. */
int moe_grouped_gemm_q4(const moe_layer_desc* desc, int mode, const void* a,
                        const moe_q4_tensor* w, const moe_q4_tensor* w_shared,
                        const moe_route_out* route, void* c, void* ws, size_t ws_bytes,
                        void* stream);

/* The top-k weighted combine back to token order, fp32:
 * out[t] = y[R+t] (if has_shared) + sum_k topk_w[t][k] * y[inv_pos[t*top_k+k]],
 * added in that order.  y [R(+T)][H] from MOE_GEMM_DOWN (y_dtype
 * MOE_DTYPE_F32) or MOE_GEMM_DOWN_BF16 (MOE_DTYPE_BF16).  The pages' layer
 * sums the chosen experts' outputs with the router weights plus the shared
 * expert's ("Apple silicon용 Lily, Qwen 추론 최적화", section "Qwen 구조와
 * Prefill 경로").  Errors: MOE_ERR_INVALID_ARGUMENT (NULL pointer, unknown
 * y_dtype), MOE_ERR_MISALIGNED, MOE_ERR_HIP. */
int moe_combine(const moe_layer_desc* desc, const void* y, int y_dtype, const moe_route_out* route,
                float* out, void* stream);

/* The whole layer for one chunk of T tokens: moe_route, the two grouped GEMMs
 * and the combine, all on `stream`, in the default combine mode
 * (MOE_COMBINE_Y_BF16: deterministic).  Long prompts call it once per bounded
 * chunk with the same workspace ("Perplexity Lily 오픈소스 공개", section 5-2).
 * route_or_null: if non-NULL, routing results are written there; otherwise
 * they live in the workspace.  ws: moe_layer_workspace_size bytes.
 * Errors: as moe_route and moe_grouped_gemm_q4. */
int moe_layer_forward(const moe_layer_desc* desc, const uint16_t* x, const uint16_t* w_router,
                      const float* router_bias, const moe_q4_tensor* w_gate_up,
                      const moe_q4_tensor* w_down, const moe_q4_tensor* shared_gate_up,
                      const moe_q4_tensor* shared_down, float* out,
                      const moe_route_out* route_or_null, void* ws, size_t ws_bytes,
                      void* stream);

/* moe_layer_forward in an explicit moe_combine_mode; ws:
 * moe_layer_workspace_size_ex(desc, combine_mode) bytes.  MOE_COMBINE_FUSED
 * zeroes `out` in the gate/up launch and adds into it in the down launch, so
 * its outputs may differ in the last bits between runs. */
int moe_layer_forward_ex(const moe_layer_desc* desc, int combine_mode, const uint16_t* x,
                         const uint16_t* w_router, const float* router_bias,
                         const moe_q4_tensor* w_gate_up, const moe_q4_tensor* w_down,
                         const moe_q4_tensor* shared_gate_up, const moe_q4_tensor* shared_down,
                         float* out, const moe_route_out* route_or_null, void* ws, size_t ws_bytes,
                         void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_Q4_H */
