// Host side of libmoeq4: argument checks, workspace layout and launches.
// Every check runs before the first HIP call, so a machine without a GPU
// sees the same status codes.
#include <stddef.h>
#include <stdint.h>

#include <mutex>

#include "common.hpp"
#include "moe_q4_ablation.h"
#include "moe_q4_decode.h"

using namespace moeq4;

// Scratch of moe_decode_forward_noalloc: a file-scope device array, one copy
// per GPU for the life of the process.  Host code never uses its name as an
// address (that is a host-side stand-in); it takes each device's address
// once with hipGetSymbolAddress and uses that.
constexpr size_t kScratchBytes = MOE_DECODE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, once taken

// The current device's copy of `scratch` (taken on its first use there).
int device_scratch(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

namespace {

constexpr size_t kAlign = 256;  // workspace sub-buffer alignment

inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

inline bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

int check_desc(const moe_layer_desc* d) {
  if (!d) return MOE_ERR_INVALID_ARGUMENT;
  if (d->T < 0 || d->H <= 0 || d->I <= 0 || d->E <= 0 || d->top_k <= 0) return MOE_ERR_INVALID_ARGUMENT;
  if ((d->norm_topk != 0 && d->norm_topk != 1) || (d->has_shared != 0 && d->has_shared != 1))
    return MOE_ERR_INVALID_ARGUMENT;
  if (d->group_size <= 0) return MOE_ERR_INVALID_ARGUMENT;
  if (d->group_size != MOE_GROUP_SIZE) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (d->H % MOE_GROUP_SIZE || d->I % MOE_GROUP_SIZE) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (d->H > MOE_MAX_REDUCTION || d->I > MOE_MAX_REDUCTION) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (d->E > MOE_MAX_EXPERTS || d->top_k > MOE_MAX_TOPK || d->top_k > d->E) return MOE_ERR_UNSUPPORTED_SHAPE;
  // row indices (T*(top_k+1)) stay well inside int32, and every activation
  // tensor the kernels address through 32-bit buffer offsets stays below 2 GiB
  if ((int64_t)d->T * (d->top_k + 1) > (int64_t(1) << 30)) return MOE_ERR_UNSUPPORTED_SHAPE;
  if ((int64_t)d->T * d->H * 2 >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED_SHAPE;
  if ((int64_t)d->T * (d->top_k + 1) * d->I * 2 >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED_SHAPE;
  return MOE_OK;
}

int64_t max_tiles_of(const moe_layer_desc* d) {
  const int64_t R = (int64_t)d->T * d->top_k;
  const int64_t bm = kTileRows;
  int64_t n = R / bm + (R < d->E ? R : d->E);
  if (d->has_shared) n += (d->T + bm - 1) / bm;
  return n;
}

// Prompts of at most kSmallPromptTokens tokens run the GEMMs over pieces of
// at most kSmallRows rows (the small-prompt kernel).
bool small_prompt(const moe_layer_desc* d) { return d->T <= kSmallPromptTokens; }

// Entries of the launch list: the tiles again, or the small prompt's pieces.
int64_t max_launch_of(const moe_layer_desc* d) {
  if (!small_prompt(d)) return max_tiles_of(d);
  const int64_t R = (int64_t)d->T * d->top_k;
  const int64_t bm = kSmallRows;
  int64_t n = R / bm + (R < d->E ? R : d->E);
  if (d->has_shared) n += (d->T + bm - 1) / bm;
  return n;
}

struct Layout {
  size_t hist, ids, w, counts, offsets, sorted, inv, bmap, lmap, ntiles, route_end;
  size_t h, y, total;
};

// The default combine mode of moe_layer_forward and its variants.
constexpr int kDefaultCombine = MOE_COMBINE_Y_BF16;

Layout layout_of(const moe_layer_desc* d, int combine_mode = kDefaultCombine) {
  const size_t R = (size_t)d->T * d->top_k;
  const size_t rows = R + (d->has_shared ? (size_t)d->T : 0);
  Layout L;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = round_up(o + bytes, kAlign);
    return at;
  };
  L.hist = take(route_workspace_bytes(d->T, d->H, d->E));
  L.ids = take(R * 4);
  L.w = take(R * 4);
  L.counts = take((size_t)d->E * 4);
  L.offsets = take((size_t)(d->E + 1) * 4);
  L.sorted = take(R * 4);
  L.inv = take(R * 4);
  L.bmap = take((size_t)max_tiles_of(d) * 16);
  L.lmap = take((size_t)max_launch_of(d) * 16);
  L.ntiles = take(8);  // n_tiles, then the launch list's entry count
  L.route_end = o;
  L.h = take(rows * (size_t)d->I * 2);
  const size_t y_elem = combine_mode == MOE_COMBINE_Y_F32 ? 4 : combine_mode == MOE_COMBINE_Y_BF16 ? 2 : 0;
  L.y = take(rows * (size_t)d->H * y_elem);
  L.total = o;
  return L;
}

int check_q4(const moe_q4_tensor* t, int n_exp, int N, int K) {
  if (!t || !t->codes || !t->scales || !t->biases) return MOE_ERR_INVALID_ARGUMENT;
  if (t->n_exp != n_exp || t->N != N || t->K != K) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (misaligned(t->codes) || misaligned(t->scales) || misaligned(t->biases)) return MOE_ERR_MISALIGNED;
  return MOE_OK;
}

int check_route_out(const moe_route_out* r) {
  if (!r || !r->topk_ids || !r->topk_w || !r->counts || !r->offsets || !r->sorted_idx || !r->inv_pos ||
      !r->block_map || !r->n_tiles)
    return MOE_ERR_INVALID_ARGUMENT;
  if (misaligned(r->topk_ids) || misaligned(r->topk_w) || misaligned(r->counts) || misaligned(r->offsets) ||
      misaligned(r->sorted_idx) || misaligned(r->inv_pos) || misaligned(r->block_map) || misaligned(r->n_tiles))
    return MOE_ERR_MISALIGNED;
  return MOE_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// launch_map: null, or where routing also writes the tiles in launch order
// (the layer's own workspace; the GEMMs of the same call read it).
// n_launch: where its entry count goes; small: the list holds the small
// prompt's pieces instead of the block map's tiles.
int do_route(const moe_layer_desc* d, const uint16_t* x, const uint16_t* wr, const float* rb,
             const moe_route_out* out, void* ws, hipStream_t s, int32_t* launch_map = nullptr,
             int32_t* n_launch = nullptr, bool small = false) {
  RouteArgs a;
  a.launch_map = launch_map;
  a.n_launch = n_launch;
  a.launch_rows = small ? kSmallRows : kTileRows;
  a.x = x;
  a.w_router = wr;
  a.router_bias = rb;
  a.T = d->T;
  a.H = d->H;
  a.E = d->E;
  a.K = d->top_k;
  a.norm_topk = d->norm_topk;
  a.has_shared = d->has_shared;
  a.out = *out;
  return hip_status(launch_route(a, ws, s));
}

// Weights of one grouped GEMM: 4-bit (q, qs) or, for the unfused variant,
// bf16 in memory (bf, bfs).  The shared expert's are null without one.
struct GemmWeights {
  const moe_q4_tensor* q = nullptr;
  const moe_q4_tensor* qs = nullptr;
  const uint16_t* bf = nullptr;
  const uint16_t* bfs = nullptr;
};

// The down GEMM's epilogue for a moe_gemm_mode (gate/up: unused).
int out_mode_of(int mode) {
  return mode == MOE_GEMM_DOWN_BF16 ? kOutBf16 : mode == MOE_GEMM_DOWN_COMBINE ? kOutCombine : kOutF32;
}

// tiles > 0: launch exactly that many tiles (known on the host) instead of
// the bound max_tiles_of(d).  zero_out: a gate/up launch also clears T*H
// floats there (the fused combine's output).  n_launch (with launch_map): the
// small prompt's piece list and its entry count, for the small-prompt kernel.
int do_gemm(const moe_layer_desc* d, int mode, const void* a, const GemmWeights& w, const moe_route_out* r, void* c,
            hipStream_t s, int tiles = 0, bool decode = false, float* zero_out = nullptr,
            const int32_t* launch_map = nullptr, const int32_t* n_launch = nullptr) {
  GemmArgs g;
  g.launch_map = launch_map;
  g.n_launch = n_launch;
  g.small = launch_map && n_launch;
  g.a = reinterpret_cast<const uint16_t*>(a);
  g.codes = w.q ? w.q->codes : nullptr;
  g.scales = w.q ? w.q->scales : nullptr;
  g.biases = w.q ? w.q->biases : nullptr;
  g.s_codes = w.qs ? w.qs->codes : nullptr;
  g.s_scales = w.qs ? w.qs->scales : nullptr;
  g.s_biases = w.qs ? w.qs->biases : nullptr;
  g.wbf = w.bf;
  g.s_wbf = w.bfs;
  g.sorted_idx = r->sorted_idx;
  g.block_map = r->block_map;
  g.n_tiles = r->n_tiles;
  g.c = c;
  g.out_mode = out_mode_of(mode);
  g.topk_w = r->topk_w;
  g.zero_out = zero_out;
  g.zero_n = zero_out ? (size_t)d->T * d->H : 0;
  g.T = d->T;
  g.E = d->E;
  g.topk = d->top_k;
  g.R = d->T * d->top_k;
  g.I = d->I;
  g.max_tiles = tiles > 0 ? tiles : (int)(g.small ? max_launch_of(d) : max_tiles_of(d));
  if (mode == MOE_GEMM_GATE_UP_SWIGLU) {
    g.N = 2 * d->I;
    g.Kdim = d->H;
    return hip_status(decode ? launch_decode_gemv(g, true, s) : launch_gemm_gate_up(g, s));
  }
  g.N = d->H;
  g.Kdim = d->I;
  return hip_status(decode ? launch_decode_gemv(g, false, s) : launch_gemm_down(g, s));
}

int do_combine(const moe_layer_desc* d, const void* y, int y_dtype, const moe_route_out* r, float* out,
               hipStream_t s) {
  CombineArgs c;
  c.y = y;
  c.y_bf16 = y_dtype == MOE_DTYPE_BF16;
  c.topk_w = r->topk_w;
  c.inv_pos = r->inv_pos;
  c.out = out;
  c.T = d->T;
  c.H = d->H;
  c.K = d->top_k;
  c.R = d->T * d->top_k;
  c.has_shared = d->has_shared;
  return hip_status(launch_combine(c, s));
}

int check_bf16(const moe_bf16_tensor* t, int n_exp, int N, int K) {
  if (!t || !t->w) return MOE_ERR_INVALID_ARGUMENT;
  if (t->n_exp != n_exp || t->N != N || t->K != K) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (misaligned(t->w)) return MOE_ERR_MISALIGNED;
  // one expert's bf16 matrix is addressed through 32-bit buffer offsets
  if ((int64_t)N * K * 2 >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED_SHAPE;
  return MOE_OK;
}

// The layer for one chunk.  host_sync: after routing, copy n_tiles to the
// host, wait for the stream and size the GEMM grids from it.
// decode_wt: the decode path (T <= 16) with the prepared piece-major router copy;
// w_router is then unused.
int layer_forward(const moe_layer_desc* desc, const uint16_t* x, const uint16_t* w_router, const float* router_bias,
                  const moe_q4_tensor* w_gate_up, const moe_q4_tensor* w_down, const moe_q4_tensor* shared_gate_up,
                  const moe_q4_tensor* shared_down, float* out, const moe_route_out* route_or_null, void* ws,
                  size_t ws_bytes, void* stream, bool host_sync, const uint16_t* decode_wt = nullptr,
                  int combine_mode = kDefaultCombine, bool use_scratch = false) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (combine_mode != MOE_COMBINE_Y_F32 && combine_mode != MOE_COMBINE_Y_BF16 && combine_mode != MOE_COMBINE_FUSED)
    return MOE_ERR_INVALID_ARGUMENT;
  const bool decode = decode_wt != nullptr;
  if (decode && desc->T > MOE_DECODE_MAX_TOKENS) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (desc->T == 0) return MOE_OK;
  if (!x || !w_router || !out || (!ws && !use_scratch)) return MOE_ERR_INVALID_ARGUMENT;
  if ((rc = check_q4(w_gate_up, desc->E, 2 * desc->I, desc->H))) return rc;
  if ((rc = check_q4(w_down, desc->E, desc->H, desc->I))) return rc;
  if (desc->has_shared) {
    if ((rc = check_q4(shared_gate_up, 1, 2 * desc->I, desc->H))) return rc;
    if ((rc = check_q4(shared_down, 1, desc->H, desc->I))) return rc;
  } else {
    shared_gate_up = shared_down = nullptr;
  }
  if (route_or_null && (rc = check_route_out(route_or_null))) return rc;
  if (misaligned(x) || misaligned(w_router) || misaligned(out) || (!use_scratch && misaligned(ws)) ||
      (router_bias && misaligned(router_bias)))
    return MOE_ERR_MISALIGNED;
  const Layout L = layout_of(desc, combine_mode);
  if (use_scratch) {
    // the library's own scratch instead of a caller workspace
    if (L.total > kScratchBytes) return MOE_ERR_WORKSPACE_TOO_SMALL;
    if ((rc = device_scratch(&ws))) return rc;
    ws_bytes = kScratchBytes;
  }
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE_TOO_SMALL;

  char* base = reinterpret_cast<char*>(ws);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  moe_route_out r;
  if (route_or_null) {
    r = *route_or_null;
  } else {
    r.topk_ids = reinterpret_cast<int32_t*>(base + L.ids);
    r.topk_w = reinterpret_cast<float*>(base + L.w);
    r.counts = reinterpret_cast<int32_t*>(base + L.counts);
    r.offsets = reinterpret_cast<int32_t*>(base + L.offsets);
    r.sorted_idx = reinterpret_cast<int32_t*>(base + L.sorted);
    r.inv_pos = reinterpret_cast<int32_t*>(base + L.inv);
    r.block_map = reinterpret_cast<int32_t*>(base + L.bmap);
    r.n_tiles = reinterpret_cast<int32_t*>(base + L.ntiles);
  }
  void* h = base + L.h;
  void* y = base + L.y;
  // the prefill routing also lists the tiles in launch order (a small
  // prompt: its pieces, and their count); the decode routing does not, and
  // its GEMMs walk the block map
  int32_t* lmap = decode ? nullptr : reinterpret_cast<int32_t*>(base + L.lmap);
  const bool small = !decode && small_prompt(desc);
  int32_t* nlaunch = small ? reinterpret_cast<int32_t*>(base + L.ntiles) + 1 : nullptr;
  if (decode) {
    DecodeRouteArgs a;
    a.x = x;
    a.wt = decode_wt;
    a.router_bias = router_bias;
    a.logits = reinterpret_cast<float*>(base + L.hist);  // the routing scratch holds T*E fp32 and more
    a.T = desc->T;
    a.H = desc->H;
    a.E = desc->E;
    a.K = desc->top_k;
    a.norm_topk = desc->norm_topk;
    a.has_shared = desc->has_shared;
    a.out = r;
    if ((rc = hip_status(launch_decode_route(a, s)))) return rc;
  } else if ((rc = do_route(desc, x, w_router, router_bias, &r, base + L.hist, s, lmap, nlaunch, small))) {
    return rc;
  }
  int tiles = 0;
  if (host_sync) {
    int32_t nt = 0;
    // the GEMMs' grid: the block map's tiles, or the small prompt's pieces
    if (hipMemcpyAsync(&nt, small ? nlaunch : r.n_tiles, sizeof(nt), hipMemcpyDeviceToHost, s) != hipSuccess)
      return MOE_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return MOE_ERR_HIP;
    // routing produced no valid block map
    if (nt <= 0 || nt > (small ? max_launch_of(desc) : max_tiles_of(desc))) return MOE_ERR_HIP;
    tiles = nt;
  }
  GemmWeights gu, dn;
  gu.q = w_gate_up;
  gu.qs = shared_gate_up;
  dn.q = w_down;
  dn.qs = shared_down;
  // decode (at most 16 tokens, so every tile has at most 16 rows): the
  // split-reduction GEMVs (measured faster than the tiled GEMM at 1-16 tokens)
  const bool gemv = decode;
  if (combine_mode == MOE_COMBINE_FUSED) {
    // gate/up clears out, down adds every weighted row into it
    if ((rc = do_gemm(desc, MOE_GEMM_GATE_UP_SWIGLU, x, gu, &r, h, s, tiles, gemv, out, lmap, nlaunch))) return rc;
    return do_gemm(desc, MOE_GEMM_DOWN_COMBINE, h, dn, &r, out, s, tiles, gemv, nullptr, lmap, nlaunch);
  }
  const bool bf = combine_mode == MOE_COMBINE_Y_BF16;
  if ((rc = do_gemm(desc, MOE_GEMM_GATE_UP_SWIGLU, x, gu, &r, h, s, tiles, gemv, nullptr, lmap, nlaunch))) return rc;
  if ((rc = do_gemm(desc, bf ? MOE_GEMM_DOWN_BF16 : MOE_GEMM_DOWN, h, dn, &r, y, s, tiles, gemv, nullptr, lmap,
                    nlaunch)))
    return rc;
  return do_combine(desc, y, bf ? MOE_DTYPE_BF16 : MOE_DTYPE_F32, &r, out, s);
}

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARGUMENT: return "MOE_ERR_INVALID_ARGUMENT: a required pointer is NULL or a size is invalid";
    case MOE_ERR_UNSUPPORTED_SHAPE: return "MOE_ERR_UNSUPPORTED_SHAPE: shape outside what the kernels support";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
    case MOE_ERR_MISALIGNED: return "MOE_ERR_MISALIGNED: device tensors must be 16-byte aligned";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: a HIP launch failed";
    default: return "unknown moe status";
  }
}

int moe_route_block_rows(void) { return kTileRows; }

int moe_route_max_tiles(const moe_layer_desc* desc, int32_t* max_tiles) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!max_tiles) return MOE_ERR_INVALID_ARGUMENT;
  *max_tiles = (int32_t)max_tiles_of(desc);
  return MOE_OK;
}

int moe_layer_workspace_size(const moe_layer_desc* desc, size_t* bytes) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!bytes) return MOE_ERR_INVALID_ARGUMENT;
  *bytes = layout_of(desc).total;
  return MOE_OK;
}

int moe_layer_workspace_size_ex(const moe_layer_desc* desc, int combine_mode, size_t* bytes) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!bytes) return MOE_ERR_INVALID_ARGUMENT;
  if (combine_mode != MOE_COMBINE_Y_F32 && combine_mode != MOE_COMBINE_Y_BF16 && combine_mode != MOE_COMBINE_FUSED)
    return MOE_ERR_INVALID_ARGUMENT;
  *bytes = layout_of(desc, combine_mode).total;
  return MOE_OK;
}

int moe_route_workspace_size(const moe_layer_desc* desc, size_t* bytes) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!bytes) return MOE_ERR_INVALID_ARGUMENT;
  *bytes = route_workspace_bytes(desc->T, desc->H, desc->E);
  return MOE_OK;
}

int moe_route(const moe_layer_desc* desc, const uint16_t* x, const uint16_t* w_router, const float* router_bias,
              const moe_route_out* out, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (desc->T == 0) return MOE_OK;
  if (!x || !w_router || !ws) return MOE_ERR_INVALID_ARGUMENT;
  if ((rc = check_route_out(out))) return rc;
  if (misaligned(x) || misaligned(w_router) || misaligned(ws) || (router_bias && misaligned(router_bias)))
    return MOE_ERR_MISALIGNED;
  if (ws_bytes < route_workspace_bytes(desc->T, desc->H, desc->E)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  return do_route(desc, x, w_router, router_bias, out, ws, reinterpret_cast<hipStream_t>(stream));
}

int moe_grouped_gemm_q4(const moe_layer_desc* desc, int mode, const void* a, const moe_q4_tensor* w,
                        const moe_q4_tensor* w_shared, const moe_route_out* route, void* c, void* ws,
                        size_t ws_bytes, void* stream) {
  (void)ws;  // no GEMM scratch in this version
  (void)ws_bytes;
  int rc = check_desc(desc);
  if (rc) return rc;
  if (mode < MOE_GEMM_GATE_UP_SWIGLU || mode > MOE_GEMM_DOWN_COMBINE) return MOE_ERR_INVALID_ARGUMENT;
  if (desc->T == 0) return MOE_OK;
  if (!a || !c || !route || !route->sorted_idx || !route->block_map || !route->n_tiles)
    return MOE_ERR_INVALID_ARGUMENT;
  if (mode == MOE_GEMM_DOWN_COMBINE && !route->topk_w) return MOE_ERR_INVALID_ARGUMENT;
  const int N = mode == MOE_GEMM_GATE_UP_SWIGLU ? 2 * desc->I : desc->H;
  const int K = mode == MOE_GEMM_GATE_UP_SWIGLU ? desc->H : desc->I;
  if ((rc = check_q4(w, desc->E, N, K))) return rc;
  if (desc->has_shared) {
    if ((rc = check_q4(w_shared, 1, N, K))) return rc;
  } else {
    w_shared = nullptr;
  }
  if (misaligned(a) || misaligned(c) || misaligned(route->sorted_idx) || misaligned(route->block_map) ||
      misaligned(route->n_tiles) || (mode == MOE_GEMM_DOWN_COMBINE && misaligned(route->topk_w)))
    return MOE_ERR_MISALIGNED;
  GemmWeights gw;
  gw.q = w;
  gw.qs = w_shared;
  return do_gemm(desc, mode, a, gw, route, c, reinterpret_cast<hipStream_t>(stream));
}

int moe_combine(const moe_layer_desc* desc, const void* y, int y_dtype, const moe_route_out* route, float* out,
                void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (y_dtype != MOE_DTYPE_F32 && y_dtype != MOE_DTYPE_BF16) return MOE_ERR_INVALID_ARGUMENT;
  if (desc->T == 0) return MOE_OK;
  if (!y || !out || !route || !route->topk_w || !route->inv_pos) return MOE_ERR_INVALID_ARGUMENT;
  if (misaligned(y) || misaligned(out) || misaligned(route->topk_w) || misaligned(route->inv_pos))
    return MOE_ERR_MISALIGNED;
  return do_combine(desc, y, y_dtype, route, out, reinterpret_cast<hipStream_t>(stream));
}

int moe_layer_forward(const moe_layer_desc* desc, const uint16_t* x, const uint16_t* w_router,
                      const float* router_bias, const moe_q4_tensor* w_gate_up, const moe_q4_tensor* w_down,
                      const moe_q4_tensor* shared_gate_up, const moe_q4_tensor* shared_down, float* out,
                      const moe_route_out* route_or_null, void* ws, size_t ws_bytes, void* stream) {
  return layer_forward(desc, x, w_router, router_bias, w_gate_up, w_down, shared_gate_up, shared_down, out,
                       route_or_null, ws, ws_bytes, stream, false);
}

int moe_layer_forward_ex(const moe_layer_desc* desc, int combine_mode, const uint16_t* x, const uint16_t* w_router,
                         const float* router_bias, const moe_q4_tensor* w_gate_up, const moe_q4_tensor* w_down,
                         const moe_q4_tensor* shared_gate_up, const moe_q4_tensor* shared_down, float* out,
                         const moe_route_out* route_or_null, void* ws, size_t ws_bytes, void* stream) {
  return layer_forward(desc, x, w_router, router_bias, w_gate_up, w_down, shared_gate_up, shared_down, out,
                       route_or_null, ws, ws_bytes, stream, false, nullptr, combine_mode);
}

int moe_layer_forward_host_sync(const moe_layer_desc* desc, const uint16_t* x, const uint16_t* w_router,
                                const float* router_bias, const moe_q4_tensor* w_gate_up,
                                const moe_q4_tensor* w_down, const moe_q4_tensor* shared_gate_up,
                                const moe_q4_tensor* shared_down, float* out, const moe_route_out* route_or_null,
                                void* ws, size_t ws_bytes, void* stream) {
  return layer_forward(desc, x, w_router, router_bias, w_gate_up, w_down, shared_gate_up, shared_down, out,
                       route_or_null, ws, ws_bytes, stream, true);
}

int moe_decode_router_prepare(const moe_layer_desc* desc, const uint16_t* w_router, uint16_t* w_router_pm,
                              void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!w_router || !w_router_pm) return MOE_ERR_INVALID_ARGUMENT;
  if (misaligned(w_router) || misaligned(w_router_pm)) return MOE_ERR_MISALIGNED;
  return hip_status(launch_decode_prep(w_router, desc->H, desc->E, w_router_pm, reinterpret_cast<hipStream_t>(stream)));
}

int moe_decode_forward(const moe_layer_desc* desc, const uint16_t* x, const uint16_t* w_router_pm,
                       const float* router_bias, const moe_q4_tensor* w_gate_up, const moe_q4_tensor* w_down,
                       const moe_q4_tensor* shared_gate_up, const moe_q4_tensor* shared_down, float* out,
                       const moe_route_out* route_or_null, void* ws, size_t ws_bytes, void* stream) {
  if (!w_router_pm) return MOE_ERR_INVALID_ARGUMENT;
  if (misaligned(w_router_pm)) return MOE_ERR_MISALIGNED;
  // the bf16 router matrix is not read on this path; the prepared copy stands
  // in for it in the shared argument checks
  return layer_forward(desc, x, w_router_pm, router_bias, w_gate_up, w_down, shared_gate_up, shared_down, out,
                       route_or_null, ws, ws_bytes, stream, false, w_router_pm);
}

int moe_decode_forward_noalloc(const moe_layer_desc* desc, const uint16_t* x, const uint16_t* w_router_pm,
                               const float* router_bias, const moe_q4_tensor* w_gate_up,
                               const moe_q4_tensor* w_down, const moe_q4_tensor* shared_gate_up,
                               const moe_q4_tensor* shared_down, float* out, const moe_route_out* route_or_null,
                               void* stream) {
  if (!w_router_pm) return MOE_ERR_INVALID_ARGUMENT;
  if (misaligned(w_router_pm)) return MOE_ERR_MISALIGNED;
  return layer_forward(desc, x, w_router_pm, router_bias, w_gate_up, w_down, shared_gate_up, shared_down, out,
                       route_or_null, nullptr, 0, stream, false, w_router_pm, kDefaultCombine, true);
}

int moe_dequant_q4_to_bf16(const moe_q4_tensor* w, const int32_t* counts_or_null, uint16_t* out, void* stream) {
  if (!w || !w->codes || !w->scales || !w->biases || !out) return MOE_ERR_INVALID_ARGUMENT;
  if (w->n_exp < 0 || w->N < 0 || w->K < 0) return MOE_ERR_INVALID_ARGUMENT;
  if (w->K % MOE_GROUP_SIZE) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (misaligned(w->codes) || misaligned(w->scales) || misaligned(w->biases) || misaligned(out) ||
      (counts_or_null && misaligned(counts_or_null)))
    return MOE_ERR_MISALIGNED;
  if (w->n_exp == 0 || w->N == 0 || w->K == 0) return MOE_OK;
  // one expert's weights and its grid stay inside 32-bit indexing
  if ((int64_t)w->N * w->K >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED_SHAPE;
  DequantArgs d;
  d.codes = w->codes;
  d.scales = w->scales;
  d.biases = w->biases;
  d.counts = counts_or_null;
  d.out = out;
  d.n_exp = w->n_exp;
  d.N = w->N;
  d.K = w->K;
  return hip_status(launch_dequant(d, reinterpret_cast<hipStream_t>(stream)));
}

int moe_grouped_gemm_bf16(const moe_layer_desc* desc, int mode, const void* a, const moe_bf16_tensor* w,
                          const moe_bf16_tensor* w_shared, const moe_route_out* route, void* c, void* ws,
                          size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  int rc = check_desc(desc);
  if (rc) return rc;
  if (mode < MOE_GEMM_GATE_UP_SWIGLU || mode > MOE_GEMM_DOWN_COMBINE) return MOE_ERR_INVALID_ARGUMENT;
  if (desc->T == 0) return MOE_OK;
  if (!a || !c || !route || !route->sorted_idx || !route->block_map || !route->n_tiles)
    return MOE_ERR_INVALID_ARGUMENT;
  const int N = mode == MOE_GEMM_GATE_UP_SWIGLU ? 2 * desc->I : desc->H;
  const int K = mode == MOE_GEMM_GATE_UP_SWIGLU ? desc->H : desc->I;
  if (mode == MOE_GEMM_DOWN_COMBINE && !route->topk_w) return MOE_ERR_INVALID_ARGUMENT;
  if ((rc = check_bf16(w, desc->E, N, K))) return rc;
  if (desc->has_shared) {
    if ((rc = check_bf16(w_shared, 1, N, K))) return rc;
  } else {
    w_shared = nullptr;
  }
  if (misaligned(a) || misaligned(c) || misaligned(route->sorted_idx) || misaligned(route->block_map) ||
      misaligned(route->n_tiles))
    return MOE_ERR_MISALIGNED;
  GemmWeights gw;
  gw.bf = w->w;
  gw.bfs = w_shared ? w_shared->w : nullptr;
  return do_gemm(desc, mode, a, gw, route, c, reinterpret_cast<hipStream_t>(stream));
}

}  // extern "C"
