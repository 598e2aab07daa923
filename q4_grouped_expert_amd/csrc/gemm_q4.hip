// Grouped GEMM over uneven expert groups on groupwise-affine 4-bit weights,
// dequantized tile by tile inside the GEMM and never written out
// ("Perplexity Lily 오픈소스 공개", alltoptrend.co.kr, section 5-1;
// "Apple silicon용 Lily, Qwen 추론 최적화", aitrends.kr, section
// "Qwen 구조와 Prefill 경로").
//
// gfx950 mapping
//  * One workgroup = 4 waves, one per SIMD, and two workgroups share a CU
//    (80 KB of LDS and at most 256 registers per wave each), so every SIMD
//    runs two independent waves: while one issues MFMAs the other dequantizes,
//    waits at its barrier or runs its prologue/epilogue.
//  * A workgroup computes one block-map tile (<= 256 rows of one expert
//    group) against a 128-column slice of that expert's weights (gate/up:
//    64 gate + the matching 64 up columns).  Each wave owns every row of the
//    tile and 32 weight columns (two 16-column MFMA subtiles): every weight
//    of the slice is dequantized by exactly one lane per tile, and a tile
//    holds a whole expert group of up to 256 rows, so an expert's weights
//    are streamed and dequantized once per column slice whatever its row
//    count; the accumulators (<= 128 per lane) stay in registers.
//  * The number of live 16-row subtiles (1..16) is a template parameter,
//    picked once per workgroup: a 150-row group runs a 10-subtile body with
//    straight-line code and no MFMAs beyond the last partial subtile.
//  * Activations (x rows gathered through sorted_idx, or h rows) reach LDS by
//    direct-to-LDS buffer loads into a 2-slot ring of 64-column stages (one
//    quant group each), issued one stage ahead and spread over the MFMA
//    regions, with a 16-byte-chunk XOR swizzle that keeps MFMA fragment
//    reads conflict-free.
//  * Weights go from global memory straight to VGPRs through buffer loads
//    (per-lane row offset in a VGPR, stage offset in an SGPR), two stages
//    ahead of use: a lane loads 8 bytes = 16 codes of one weight row, turns
//    codes into floats two at a time (packed fp8 conversion of the masked
//    nibbles), forms q*scale+bias with one fma per weight in fp32, rounds to
//    bf16 and feeds the result as the A operand of v_mfma_f32_16x16x32_bf16
//    (activations are the B operand, so each lane ends with 4 consecutive
//    output columns of one row); accumulation is fp32.  The tile's scales and
//    biases for the whole reduction are loaded once per tile into LDS tables.
//  * Tiles of at most 4 row subtiles (64 rows) have too little matrix work
//    per stage to cover memory latency with that pipeline; they run a 4-slot
//    LDS ring that holds both the activations and the codes of a stage, each
//    loaded direct-to-LDS three stages ahead.  Both forms issue the same
//    MFMA sequence per output, so results do not depend on the form.
//  * The reduction index is permuted identically for A and B inside each
//    64-wide group (lane group g, MFMA step s -> columns 16g+8s..16g+8s+7),
//    which lets one 8-byte code load serve both MFMA steps.
//  * Gate/up mode gives each wave gate rows j and up rows I+j for the same
//    16 j, so the SwiGLU epilogue h = bf16(silu(g)*u) happens in registers
//    and leaves as one 8-byte store per row and subtile; down writes fp32 y
//    with one 16-byte store per row and subtile.
//  * Block order: tiles are visited in the routing's launch order, most
//    16-row subtiles first, so the grid ends on its shortest workgroups
//    (without that list the block map is walked backwards: the shared
//    expert's full tiles first), and the N-slices of one tile get workgroup
//    ids that are equal modulo 8, which puts them on the same XCD so the
//    tile's activations are shared in that XCD's L2.
#include <math.h>

#include <type_traits>
#include <utility>

#include "common.hpp"
#include "gemm_common.hpp"

namespace moeq4 {

namespace {
using namespace gemm;

constexpr int BK = 64;           // reduction columns per stage (= quant group)
constexpr int NWAVES = 4;        // one wave per SIMD
constexpr int NT = 64 * NWAVES;  // lanes per workgroup
constexpr int NS = 2;            // 16-column subtiles per wave
constexpr int WN = 16 * NS;      // columns per wave
constexpr int BN = NWAVES * WN;  // weight columns per workgroup
constexpr int kXcds = 8;
constexpr int kMaxGroups = kMaxGroupsPerRow;  // scale/bias groups per weight row kept in LDS
// 16-byte-chunk swizzle of a 128-byte LDS row: conflict-free for the 16 rows
// an MFMA fragment read touches, whether LDS serves 8 lanes over 32 banks or
// 16 lanes over 64 banks per cycle.  An involution: swz(r, swz(r, c)) == c.
__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ (row & 7) ^ ((row >> 3) & 1); }

// The 64 KB activation space as four separate LDS arrays of 16 KB (128 rows
// of one 64-column stage each).  Every access below names its array by a
// compile-time index, so the compiler can tell that a direct-to-LDS load
// into one array does not alias reads of another and need not wait for the
// load before those reads (with one array it would, and the pipeline
// would drain at every LDS read).
constexpr int kQElems = 128 * BK;
struct LdsQ {
  uint16_t* q0;
  uint16_t* q1;
  uint16_t* q2;
  uint16_t* q3;
};
__device__ __forceinline__ uint16_t* lds_q(const LdsQ& L, int i) {
  return i == 0 ? L.q0 : i == 1 ? L.q1 : i == 2 ? L.q2 : L.q3;
}

// Weight registers of one stage and lane: 16 codes per subtile (8 bytes), or
// with bf16 weights in memory the 16 bf16 values themselves (two 16-byte
// loads per subtile).
template <bool kBf16W>
struct BRegs {
  u32x2 c[NS];
};
template <>
struct BRegs<true> {
  u32x4 c[NS][2];
};

// Per-workgroup state shared by every subtile-count instantiation.
struct TileCtx {
  rsrc_t a_rs, c_rs, s_rs, b_rs;
  uint32_t c_off[NS];   // byte offset of this lane's code row + 8*lg
  int sb_row[NS];       // this lane's rows in the LDS scale/bias tables
  uint32_t sb_src[2];   // byte offsets of the (up to two) contiguous row ranges
  int sb_half;          // 16-byte chunks per range
  int sb_mask;          // chunk rotation mask of a table row (0: none)
  int sb_f[NS];         // rotation of this lane's table rows
  int nk;               // stages
  int row0, nrows;
  int ocol[NS];
  bool jval[NS];
  int col0;             // first output column of the workgroup's slice (h or y)
  uint32_t wd_off[1];   // per-lane offset of the direct-to-LDS code load (short-tile form)
};

// The tile's scales and biases for the whole reduction: one or two
// contiguous row ranges per table, fetched once as whole cache lines with
// 16-byte direct-to-LDS loads (chunk q of range r lands at LDS byte
// 16*(r*half + q)).  Chunks past a range read zeros into the slack of the
// table.  Inside a table row the 16-byte chunks are rotated by
// f(row) = (row * gpr / 128) & mask, so that the 16 consecutive rows one
// dequant read touches fall on 16 different bank groups (without it, 32
// groups per row put them on 4).
__device__ __forceinline__ void load_sb_tables(const TileCtx& t, int gpr, uint16_t* __restrict__ Ssh,
                                               uint16_t* __restrict__ Bsh) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int chunks = 2 * t.sb_half;  // both ranges
#pragma unroll
  for (int round = 0; round < (32 * kMaxGroups + NT - 1) / NT; ++round) {  // <= 32*gpr chunks
    const int q0 = NT * round + 64 * wave;  // first chunk of this wave's DMA
    if (q0 < chunks) {
      const int q = q0 + lane;
      const int r = q >= t.sb_half;
      int qi = q - r * t.sb_half;
      if (t.sb_mask) {
        const int cp = q & t.sb_mask;        // physical chunk in its table row
        const int row = q / (t.sb_mask + 1);  // table row
        qi += (cp ^ (((row * gpr) >> 7) & t.sb_mask)) - cp;
      }
      const uint32_t off = (q < chunks) ? t.sb_src[r] + 16u * qi : kOob;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(t.s_rs, (__attribute__((address_space(3))) void*)(Ssh + 8 * q0), 16, off,
                                               0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(t.b_rs, (__attribute__((address_space(3))) void*)(Bsh + 8 * q0), 16, off,
                                               0, 0, 0);
    }
  }
}

// Per-lane source offsets of a tile's activation loads.  Per stage, DMA i of
// wave w fills tile rows 32i + 8w .. +7 (1 KB, 16 B per lane).  Lane l lands
// at row 32i + 8w + l/8, physical chunk l%8, so it fetches the logical chunk
// that the swizzle maps there.  Rows past the group read zeros (the DMAs past
// the live subtiles stay inside the slot and are never read).
template <bool kGateUp, int MSUB>
__device__ __forceinline__ void activation_offsets(const GemmArgs& g, const TileCtx& t,
                                                   uint32_t (&adoff)[(MSUB * 16 + 8 * NWAVES - 1) / (8 * NWAVES)]) {
  constexpr int ROWS_PER_DMA = 8 * NWAVES;
  constexpr int ADMA = (MSUB * 16 + ROWS_PER_DMA - 1) / ROWS_PER_DMA;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int Kd = g.Kdim;
#pragma unroll
  for (int i = 0; i < ADMA; ++i) {
    const int r = ROWS_PER_DMA * i + 8 * wave + (lane >> 3);
    const int c = swz(r, lane & 7);  // swz is an involution
    adoff[i] = kOob;
    if (r < t.nrows) {
      const int p = t.row0 + r;
      int src;
      if (kGateUp) src = (p < g.R) ? g.sorted_idx[p] / g.topk : p - g.R;
      else src = p;
      adoff[i] = ((uint32_t)src * (uint32_t)Kd + 8u * c) * 2u;
    }
  }
}

// Epilogue: the lane holds output row 16m + ln, columns 4*lg..4*lg+3 of each
// subtile, written as one vector store per subtile.
template <bool kGateUp, int MSUB>
__device__ __forceinline__ void store_tile_direct(const GemmArgs& g, const TileCtx& t, const f32x4 (&acc)[MSUB][NS]) {
  const int lane = threadIdx.x & 63;
  const int ln = lane & 15, lg = lane >> 4;
  const int r_in = ln;
  if (kGateUp) {
    // subtile 0: gate columns; 1: the matching up columns
    uint16_t* h = reinterpret_cast<uint16_t*>(g.c);
    if (t.jval[0]) {
      const int c0 = t.ocol[0] - ln + 4 * lg;
#pragma unroll
      for (int m = 0; m < MSUB; ++m) {
        const int r = m * 16 + r_in;
        if (r < t.nrows) {
          uint32_t hv[2];
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            float o[2];
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              const float gv = acc[m][0][2 * i + q], uv = acc[m][1][2 * i + q];
              o[q] = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * uv;
            }
            hv[i] = pack_bf16x2(o[0], o[1]);
          }
          *reinterpret_cast<u32x2*>(&h[(size_t)(t.row0 + r) * g.I + c0]) = u32x2{hv[0], hv[1]};
        }
      }
    }
  } else {
#pragma unroll
    for (int m = 0; m < MSUB; ++m) {
      const int r = m * 16 + r_in;
      if (r < t.nrows) {
        const DownRow dr = down_row(g, t.row0 + r);
#pragma unroll
        for (int j = 0; j < NS; ++j)
          if (t.jval[j]) store_down4(g, dr, t.ocol[j] - ln + 4 * lg, acc[m][j]);
      }
    }
  }
}

// SwiGLU of four gate/up accumulator pairs, as two dwords of bf16 h.
__device__ __forceinline__ u32x2 swiglu4(const f32x4& gt, const f32x4& up) {
  uint32_t hv[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    float o[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const float gv = gt[2 * i + q], uv = up[2 * i + q];
      o[q] = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * uv;
    }
    hv[i] = pack_bf16x2(o[0], o[1]);
  }
  return u32x2{hv[0], hv[1]};
}

// Epilogue for bf16 outputs (gate/up h, down y in bf16).  A lane holds four
// consecutive columns of 16 rows per subtile, so direct stores are 8 bytes
// spread over 16 rows; instead the tile goes through LDS (free once the last
// stage has been read) and leaves as 16-byte stores that cover the slice's
// whole row segment: 128 B of h or 256 B of y per row, full cache lines.
// y is written with non-temporal stores: it is far larger than L2 and is
// read back only by the combine, while h is read by the down GEMM next.
// LDS layout: row r of the slice in array r / RPA, its 16-byte chunk c at
// chunk c ^ (r % CH), so the 16 rows one write instruction touches fall on
// different banks.
template <bool kGateUp, int MSUB, int QE = kQElems>  // QE: bf16 elements per LDS array
__device__ __forceinline__ void store_tile(const GemmArgs& g, const TileCtx& t, const LdsQ& L,
                                           const f32x4 (&acc)[MSUB][NS]) {
  if (!kGateUp && g.out_mode != kOutBf16) {
    store_tile_direct<kGateUp, MSUB>(g, t, acc);
    return;
  }
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 15, lg = lane >> 4;
  constexpr int OC = kGateUp ? BN / 2 : BN;  // bf16 output columns of the slice
  constexpr int CH = OC / 8;                 // 16-byte chunks per row
  constexpr int RPA = QE / OC;               // slice rows per LDS array
  static_assert(MSUB * 16 <= 3 * RPA || (QE == kQElems && MSUB * 16 <= 4 * RPA), "the staged tile fits the arrays");
  auto at = [&](int r, int c) { return lds_q(L, r / RPA) + (r % RPA) * OC + ((c ^ (r % CH)) * 8); };
  wait_vmcnt<0>();
  __syncthreads();  // every wave's ring DMAs landed and every wave is past its last LDS read
#pragma unroll
  for (int m = 0; m < MSUB; ++m) {
    const int r = m * 16 + ln;
    if constexpr (kGateUp) {
      const int col = wave * (WN / 2) + 4 * lg;  // h column in the slice
      *reinterpret_cast<u32x2*>(at(r, col / 8) + (col & 4)) = swiglu4(acc[m][0], acc[m][1]);
    } else {
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        const int col = wave * WN + 16 * j + 4 * lg;
        const f32x4 v = acc[m][j];
        *reinterpret_cast<u32x2*>(at(r, col / 8) + (col & 4)) =
            u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      }
    }
  }
  __syncthreads();
  uint16_t* out = reinterpret_cast<uint16_t*>(g.c);
  const int ld = kGateUp ? g.I : g.N;  // row pitch of h or y
  const int ncol = ld - t.col0;        // columns of the slice inside the matrix
#pragma unroll
  for (int it = 0; it < (MSUB * 16 * CH + NT - 1) / NT; ++it) {
    const int idx = tid + NT * it;
    const int r = idx / CH, c = idx % CH;
    if (r < t.nrows && 8 * c < ncol) {
      u32x4* dst = reinterpret_cast<u32x4*>(out + (size_t)(t.row0 + r) * ld + t.col0 + 8 * c);
      const u32x4 v = *reinterpret_cast<const u32x4*>(at(r, c));
      if constexpr (kGateUp) *dst = v;
      else __builtin_nontemporal_store(v, dst);
    }
  }
}

template <bool kGateUp, bool kBf16W, int MSUB>
__device__ __forceinline__ void tile_body(const GemmArgs& g, const TileCtx& t, const LdsQ& L,
                                          uint16_t* __restrict__ Ssh, uint16_t* __restrict__ Bsh) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: LDS bases stay scalar
  const int ln = lane & 15, lg = lane >> 4;
  const int Kd = g.Kdim;
  const int gpr = Kd / 64;  // quant groups per weight row
  constexpr int AROWS = MSUB * 16;
  constexpr int ROWS_PER_DMA = 8 * NWAVES;                         // one 1-KB write per wave covers 8 rows
  constexpr int ADMA = (AROWS + ROWS_PER_DMA - 1) / ROWS_PER_DMA;  // LDS-DMA writes per wave per stage

  uint32_t adoff[ADMA];
  activation_offsets<kGateUp, MSUB>(g, t, adoff);

  f32x4 acc[MSUB][NS];  // first written by the k-step-0 MFMAs of stage 0
  BRegs<kBf16W> bq[2];  // weights of two consecutive stages
  constexpr int kLoadsB = kBf16W ? 2 * NS : NS;  // weight loads per wave per stage
  bf16x8 bf[NS][2];     // dequantized B fragments of the current stage

  // ring slot p is arrays 2p (tile rows 0..127) and 2p+1 (rows 128..255);
  // DMA i writes rows 32i.. and lands in array 2p + i/4
  auto a_dst = [&](int p, int i) {
    return lds_q(L, 2 * p + i / 4) + (ROWS_PER_DMA * (i % 4) + 8 * wave) * BK;
  };
  auto dma_a = [&](int p, int kt) {
#pragma unroll
    for (int i = 0; i < ADMA; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(t.a_rs, (__attribute__((address_space(3))) void*)a_dst(p, i), 16,
                                               adoff[i], kt * BK * 2, 0, 0);
  };
  auto load_b = [&](BRegs<kBf16W>& q, int kt) {
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      if constexpr (kBf16W) {
        q.c[j][0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(t.c_rs, t.c_off[j], kt * 128, 0));
        q.c[j][1] =
            __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(t.c_rs, t.c_off[j], kt * 128 + 16, 0));
      } else {
        q.c[j] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(t.c_rs, t.c_off[j], kt * 32, 0));
      }
    }
  };
  // Dequantize stage kt's codes into bf, with each subtile's scale and bias
  // from the tile's LDS tables.
  auto dequant = [&](const BRegs<kBf16W>& q, int kt) {
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      if constexpr (kBf16W) {
        bf[j][0] = __builtin_bit_cast(bf16x8, q.c[j][0]);
        bf[j][1] = __builtin_bit_cast(bf16x8, q.c[j][1]);
      } else {
        const int idx = t.sb_row[j] * gpr + 8 * ((kt >> 3) ^ t.sb_f[j]) + (kt & 7);
        const float sv = bf16_bits_to_f32(Ssh[idx]), bv = bf16_bits_to_f32(Bsh[idx]);
        bf[j][0] = dequant8(q.c[j][0], sv, bv);
        bf[j][1] = dequant8(q.c[j][1], sv, bv);
      }
    }
  };
  auto dma_sb = [&]() { load_sb_tables(t, gpr, Ssh, Bsh); };
  // A fragment of subtile m in slot p (row 16m + ln; the swizzle only
  // depends on the row's low 4 bits, the same in the array)
  auto a_frag = [&](int p, int m, int st) {
    const uint16_t* Ab = lds_q(L, 2 * p + m / 8);
    const int r = (m % 8) * 16 + ln;
    return *reinterpret_cast<const bf16x8*>(&Ab[r * BK + swz(r, 2 * lg + st) * 8]);
  };

  // Every wave issues the same, unconditional sequence of loads (stage
  // indices clamped at the end, rows past the group reading zeros): per
  // stage ADMA direct-to-LDS loads then NS code loads, and no other vector
  // memory access, so the wait before each barrier can count them.
  const int nk = t.nk;
  const int last = nk - 1;
  if constexpr (!kBf16W) dma_sb();
  dma_a(0, 0);
  load_b(bq[0], 0);
  load_b(bq[1], min(1, last));
  __syncthreads();  // every wave's DMAs of the tables and of stage 0 landed
  dequant(bq[0], 0);

  // Stage kt (ring slot kt%2, codes bq[kt%2]):
  //  - DMA stage kt+1 into the other slot (read in stage kt-1, free since the
  //    last barrier) and load the codes of stage kt+2 into bq[kt%2]
  //    (dequantized at the end of stage kt-1);
  //  - per 16-row subtile m, one scheduling region with the LDS reads of
  //    subtile m+2's A fragments and subtile m's 2*NS MFMAs;
  //  - dequantize stage kt+1's codes into bf in place (the MFMAs have read
  //    their operands), wait until only this stage's NS code loads are in
  //    flight (so the DMA of stage kt+1 has landed) and meet at the barrier
  //    (a plain s_barrier: a fenced one would drain every outstanding load).
  auto stage = [&](auto first, auto slot, int kt, BRegs<kBf16W>& qown, const BRegs<kBf16W>& qnext) {
    constexpr int P = decltype(slot)::value;  // this stage's ring slot; the next stage's is 1 - P
    // The loads for later stages are spread over the subtile regions (DMA i
    // in region i, the code loads in the region after the last DMA), so
    // their issue overlaps this wave's MFMAs; the DMAs still come first.
    const int ka = min(kt + 1, last);
    auto dma_one = [&](int i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(t.a_rs, (__attribute__((address_space(3))) void*)a_dst(1 - P, i), 16,
                                               adoff[i], ka * BK * 2, 0, 0);
    };
    // A fragments are read two subtiles ahead of their MFMAs (a subtile's
    // 2*NS MFMAs alone are shorter than an LDS read)
    bf16x8 af[3][2];
#pragma unroll
    for (int m = 0; m < 2 && m < MSUB; ++m) {
      af[m][0] = a_frag(P, m, 0);
      af[m][1] = a_frag(P, m, 1);
    }
#pragma unroll
    for (int m = 0; m < MSUB; ++m) {
      if (m + 2 < MSUB) {
        af[(m + 2) % 3][0] = a_frag(P, m + 2, 0);
        af[(m + 2) % 3][1] = a_frag(P, m + 2, 1);
      }
      if (m < ADMA) dma_one(m);
      if (m == ADMA) load_b(qown, min(kt + 2, last));
      // weights as the A operand, activations as B: the 16x16 result holds
      // output row 16m + ln, columns 4*lg..4*lg+3 of subtile j in each lane
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        if constexpr (decltype(first)::value) mfma_first(acc[m][j], bf[j][0], af[m % 3][0]);
        else mfma_acc(acc[m][j], bf[j][0], af[m % 3][0]);
      }
#pragma unroll
      for (int j = 0; j < NS; ++j) mfma_acc(acc[m][j], bf[j][1], af[m % 3][1]);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (ADMA >= MSUB) load_b(qown, min(kt + 2, last));
    // the last stage dequantizes its own codes again (clamped), unused
    dequant(qnext, min(kt + 1, last));
    wait_vmcnt<kLoadsB>();
    __builtin_amdgcn_s_barrier();
  };
  const std::integral_constant<bool, true> kFirst;
  const std::integral_constant<bool, false> kNext;

  // Stage 0 starts the accumulators; then two stages per iteration with no
  // conditions inside; the last (nk - 1) % 2 stage follows the loop.
  const std::integral_constant<int, 0> kSlot0;
  const std::integral_constant<int, 1> kSlot1;
  stage(kFirst, kSlot0, 0, bq[0], bq[1]);
  int kt = 1;
  for (; kt + 2 <= nk; kt += 2) {
    stage(kNext, kSlot1, kt, bq[1], bq[0]);
    stage(kNext, kSlot0, kt + 1, bq[0], bq[1]);
  }
  if (kt < nk) stage(kNext, kSlot1, kt, bq[1], bq[0]);
  wait_vmcnt<0>();  // no direct-to-LDS write outlives the tile

  store_tile<kGateUp, MSUB, kQElems>(g, t, L, acc);
}

// Short tiles (<= 4 row subtiles) have little matrix work per stage, so the
// 2-stage pipeline leaves them waiting on memory latency.  Their form runs a
// 4-slot ring over the four LDS arrays: slot s (array s) holds one stage's
// activations (direct-to-LDS, rows 0..63) and the workgroup's codes for it
// (direct-to-LDS from byte 8192: 32 weight rows x 32 bytes per wave), and
// stage kt issues the loads of stage kt + 3, so every load has three stages
// to land.  Loads for stages past the end read zeros.  The accumulators
// start at zero and every stage accumulates: the same MFMA sequence as the
// 2-stage form, so both give bit-identical results.
constexpr int kRingMaxSub = 4;  // row subtiles up to which a tile takes the ring form
constexpr int kRingW = 4096;  // bf16-element offset of a slot's codes
// The small-prompt kernel's LDS arrays: one ring slot each (activations of 64
// rows, then the codes), 12 KB instead of 16 KB, and three of them.
constexpr int kSmallQElems = kRingW + NWAVES * 512;

// kRing: slots (4: loads three stages ahead; the small-prompt kernel's 3: two
// stages ahead, in less LDS)
// kTbl: the kernel instance's table capacity (only tells instances apart: the
// host compile pass accepts a body instance from one kernel instance only)
template <bool kGateUp, int MSUB, int kRing, int QE, int kTbl>
__device__ __forceinline__ void tile_body_ring(const GemmArgs& g, const TileCtx& t, const LdsQ& L,
                                               uint16_t* __restrict__ Ssh, uint16_t* __restrict__ Bsh) {
  static_assert(kRing == 3 || kRing == 4, "ring slots");
  static_assert(kRingW + NWAVES * 512 <= QE, "a slot fits its array");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: LDS bases stay scalar
  const int ln = lane & 15, lg = lane >> 4;
  const int gpr = g.Kdim / 64;
  constexpr int ROWS_PER_DMA = 8 * NWAVES;
  constexpr int ADMA = (MSUB * 16 + ROWS_PER_DMA - 1) / ROWS_PER_DMA;
  constexpr int kPerStage = ADMA + 1;  // vector-memory loads per wave per stage
  static_assert(ADMA * ROWS_PER_DMA * BK <= kRingW, "activations overlap the codes");
  static_assert(kRingW + NWAVES * 512 <= kSmallQElems, "slot overflow");

  uint32_t adoff[ADMA];
  activation_offsets<kGateUp, MSUB>(g, t, adoff);
  f32x4 acc[MSUB][NS];
#pragma unroll
  for (int m = 0; m < MSUB; ++m)
#pragma unroll
    for (int j = 0; j < NS; ++j) acc[m][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  bf16x8 bf[NS][2];

  const int nk = t.nk;
  const int last = nk - 1;
  // the loads of stage kl into slot s (zeros past the last stage)
  auto issue_a = [&](int kl, int s, int i) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        t.a_rs, (__attribute__((address_space(3))) void*)(lds_q(L, s) + (ROWS_PER_DMA * i + 8 * wave) * BK), 16,
        kl <= last ? adoff[i] : kOob, min(kl, last) * BK * 2, 0, 0);
  };
  auto issue_w = [&](int kl, int s) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        t.c_rs, (__attribute__((address_space(3))) void*)(lds_q(L, s) + kRingW + wave * 512), 16,
        kl <= last ? t.wd_off[0] : kOob, min(kl, last) * 32, 0, 0);
  };
  // this lane's codes of stage kt (row 16j + ln of the wave's part, bytes
  // 8*lg..), dequantized with the tile's scales and biases
  auto weights = [&](int kt, int s) {
    const uint16_t* wp = lds_q(L, s) + kRingW + wave * 512;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const u32x2 c = *reinterpret_cast<const u32x2*>(wp + (16 * j + ln) * 16 + 4 * lg);
      const int idx = t.sb_row[j] * gpr + 8 * ((kt >> 3) ^ t.sb_f[j]) + (kt & 7);
      const float sv = bf16_bits_to_f32(Ssh[idx]), bv = bf16_bits_to_f32(Bsh[idx]);
      bf[j][0] = dequant8(c[0], sv, bv);
      bf[j][1] = dequant8(c[1], sv, bv);
    }
  };
  auto a_frag = [&](int s, int m, int st) {
    const uint16_t* Ab = lds_q(L, s);
    const int r = m * 16 + ln;
    return *reinterpret_cast<const bf16x8*>(&Ab[r * BK + swz(r, 2 * lg + st) * 8]);
  };

  // Every wave issues the same unconditional sequence of loads: the tables,
  // then per stage ADMA activation loads and one code load.
  load_sb_tables(t, gpr, Ssh, Bsh);
#pragma unroll
  for (int s = 0; s < kRing - 1; ++s) {
#pragma unroll
    for (int i = 0; i < ADMA; ++i) issue_a(s, s, i);
    issue_w(s, s);
  }
  wait_vmcnt<(kRing - 2) * kPerStage>();  // the tables and stage 0 landed
  __builtin_amdgcn_s_barrier();

  // Stage kt in slot S: load stage kt + kRing - 1 into slot S - 1 (read in
  // stage kt - 1, free since the last barrier), dequantize this stage's
  // codes, run the MFMA regions, wait until stage kt + 1 has landed, barrier.
  auto stage = [&](auto slot, int kt) {
    constexpr int S = decltype(slot)::value;
    constexpr int LS = (S + kRing - 1) % kRing;
    const int kl = kt + kRing - 1;
    weights(kt, S);
    bf16x8 af[3][2];
#pragma unroll
    for (int m = 0; m < 2 && m < MSUB; ++m) {
      af[m][0] = a_frag(S, m, 0);
      af[m][1] = a_frag(S, m, 1);
    }
#pragma unroll
    for (int m = 0; m < MSUB; ++m) {
      if (m + 2 < MSUB) {
        af[(m + 2) % 3][0] = a_frag(S, m + 2, 0);
        af[(m + 2) % 3][1] = a_frag(S, m + 2, 1);
      }
      if (m < ADMA) issue_a(kl, LS, m);
      if (m == ADMA) issue_w(kl, LS);
#pragma unroll
      for (int j = 0; j < NS; ++j) mfma_acc(acc[m][j], bf[j][0], af[m % 3][0]);
#pragma unroll
      for (int j = 0; j < NS; ++j) mfma_acc(acc[m][j], bf[j][1], af[m % 3][1]);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (ADMA >= MSUB) issue_w(kl, LS);
    wait_vmcnt<(kRing - 2) * kPerStage>();
    __builtin_amdgcn_s_barrier();
  };
  const std::integral_constant<int, 0> kS0;
  const std::integral_constant<int, 1> kS1;
  const std::integral_constant<int, 2> kS2;
  const std::integral_constant<int, 3> kS3;
  int kt = 0;
  if constexpr (kRing == 4) {
    for (; kt + kRing <= nk; kt += kRing) {
      stage(kS0, kt);
      stage(kS1, kt + 1);
      stage(kS2, kt + 2);
      stage(kS3, kt + 3);
    }
    if (kt < nk) stage(kS0, kt);
    if (kt + 1 < nk) stage(kS1, kt + 1);
    if (kt + 2 < nk) stage(kS2, kt + 2);
  } else {
    for (; kt + kRing <= nk; kt += kRing) {
      stage(kS0, kt);
      stage(kS1, kt + 1);
      stage(kS2, kt + 2);
    }
    if (kt < nk) stage(kS0, kt);
    if (kt + 1 < nk) stage(kS1, kt + 1);
  }
  wait_vmcnt<0>();  // no direct-to-LDS write outlives the tile
  store_tile<kGateUp, MSUB, QE>(g, t, L, acc);
}

// kSmall: the small-prompt kernel, over a list of pieces of at most
// kSmallRows rows, all in the short-tile form with a 3-slot ring: 52 KB of
// LDS (gate/up) and three workgroups per CU instead of two.
// kTblGroups: quant groups per weight row the LDS tables hold; the small
// kernel's down GEMM with at most 8 (a reduction of at most 512) keeps 40 KB of
// LDS and four workgroups per CU.
template <bool kGateUp, bool kBf16W, bool kSmall, int kTblGroups>
__global__ __launch_bounds__(NT, kSmall ? (kTblGroups <= 8 ? 4 : 3) : 2) void gemm_q4_kernel(GemmArgs g) {
  // activation ring: two stages of [256 rows][64] bf16, as four arrays of
  // 128 rows (short tiles: a 4-slot ring of activations and codes); the
  // small kernel: three arrays of one 3-slot ring's slot each
  constexpr int QE = kSmall ? kSmallQElems : kQElems;
  __shared__ __attribute__((aligned(16))) uint16_t Lq0[QE];
  __shared__ __attribute__((aligned(16))) uint16_t Lq1[QE];
  __shared__ __attribute__((aligned(16))) uint16_t Lq2[QE];
  __shared__ __attribute__((aligned(16))) uint16_t Lq3[kSmall ? 8 : kQElems];  // not used by the small kernel
  const LdsQ L{Lq0, Lq1, Lq2, kSmall ? Lq2 : Lq3};
  // the tile's scales and biases: [128 weight rows][<= 32 groups] bf16 each
  __shared__ __attribute__((aligned(16))) uint16_t Ssh[BN * kTblGroups];
  __shared__ __attribute__((aligned(16))) uint16_t Bsh[BN * kTblGroups];

  // ---- which tile / column slice -------------------------------------------
  const int nN = kGateUp ? (g.I + BN / 2 - 1) / (BN / 2) : (g.N + BN - 1) / BN;
  const int b = blockIdx.x;
  const int grp = b / (kXcds * nN);
  const int rem = b % (kXcds * nN);
  const int nb = rem / kXcds;
  const int lin = grp * kXcds + rem % kXcds;  // tile rank in launch order
  if (kGateUp) zero_share(g);
  const int n_tiles = kSmall ? *g.n_launch : *g.n_tiles;
  if (lin >= n_tiles) return;
  // launch order: the routing's list (most subtiles first, or the small
  // kernel's pieces), else the block map backwards (the shared expert's full
  // tiles first)
  const int32_t* bmap = g.launch_map ? g.launch_map + 4 * lin : g.block_map + 4 * (n_tiles - 1 - lin);
  const int e = bmap[0];
  {
    // an entry that routing did not produce (out of range) is skipped, never read through
    const int r0 = bmap[1], nr = bmap[2];
    const bool shared_ok = g.s_codes || g.s_wbf;
    if (e < 0 || e > g.E || (e == g.E && !shared_ok) || nr <= 0 || nr > (kSmall ? kSmallRows : kTileRows) ||
        r0 < 0 || r0 + nr > g.R + (shared_ok ? g.T : 0))
      return;
  }

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 15, lg = lane >> 4;
  const int Kd = g.Kdim;
  const uint32_t cpr = Kd / 2;   // code bytes per weight row
  const uint32_t gpr = Kd / 64;  // quant groups per weight row

  TileCtx t;
  t.row0 = bmap[1];
  t.nrows = bmap[2];
  t.nk = Kd / BK;
  const uint8_t* codes;
  const uint16_t* scl;
  const uint16_t* bia;
  if (e < g.E) {
    codes = g.codes + (size_t)e * g.N * cpr;
    scl = g.scales + (size_t)e * g.N * gpr;
    bia = g.biases + (size_t)e * g.N * gpr;
  } else {
    codes = g.s_codes;
    scl = g.s_scales;
    bia = g.s_biases;
  }
  // bf16 weights in memory (the unfused variant): one row is Kd * 2 bytes
  const uint32_t wrow = kBf16W ? (uint32_t)Kd * 2u : cpr;
  if (kBf16W) t.c_rs = make_rsrc(e < g.E ? g.wbf + (size_t)e * g.N * Kd : g.s_wbf, (uint32_t)g.N * wrow);
  else t.c_rs = make_rsrc(codes, (uint32_t)g.N * cpr);
  t.s_rs = make_rsrc(scl, (uint32_t)g.N * gpr * 2u);
  t.b_rs = make_rsrc(bia, (uint32_t)g.N * gpr * 2u);
  const uint32_t a_rows = kGateUp ? (uint32_t)g.T : (uint32_t)(g.R + g.T);
  t.a_rs = make_rsrc(g.a, a_rows * (uint32_t)Kd * 2u);

  // Weight row of subtile j, lane row l16 of this wave, or -1 past the
  // matrix edge.  Gate/up: subtile 0 holds gate rows hc..hc+15, subtile 1
  // the matching up rows I + hc.. (hc = this wave's first gate row).
  auto weight_row = [&](int j, int l16) -> int {
    if (kGateUp) {
      const int row = nb * (BN / 2) + wave * (WN / 2) + 16 * (j % (NS / 2));
      return row < g.I ? (j < NS / 2 ? 0 : g.I) + row + l16 : -1;
    }
    const int c = nb * BN + wave * WN + 16 * j;
    return c < g.N ? c + l16 : -1;
  };
  // This lane's weight rows (one per 16-column subtile).  Subtiles past the
  // matrix edge read row 0 and are never stored.
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const int r = weight_row(j, ln);
    t.jval[j] = r >= 0;
    t.c_off[j] = (uint32_t)max(r, 0) * wrow + (kBf16W ? 32u : 8u) * lg;
  }
  // Direct-to-LDS code load of the short-tile form: the wave's 32 weight
  // rows as [row][32 stage bytes], two lanes per row, 16 B each; rows past
  // the edge read zeros.
  {
    const int rr = lane >> 1;
    const int r = weight_row(rr >> 4, rr & 15);
    t.wd_off[0] = r >= 0 ? (uint32_t)r * cpr + 16u * (lane & 1) : kOob;
  }
  if (kGateUp) {
    const int hc = nb * (BN / 2) + wave * (WN / 2);
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int jj = j % (NS / 2);
      t.ocol[j] = hc + 16 * jj + ln;
      // scale/bias tables: rows 0..63 = gate rows nb*64.., 64..127 = up rows
      t.sb_row[j] = (j < NS / 2 ? 0 : BN / 2) + wave * (WN / 2) + 16 * jj + ln;
    }
    t.sb_half = (BN / 2) * gpr * 2 / 16;
    t.sb_src[0] = (uint32_t)(nb * (BN / 2)) * gpr * 2u;
    t.sb_src[1] = (uint32_t)(g.I + nb * (BN / 2)) * gpr * 2u;
    t.col0 = nb * (BN / 2);
  } else {
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      t.ocol[j] = nb * BN + wave * WN + 16 * j + ln;
      t.sb_row[j] = wave * WN + 16 * j + ln;
    }
    t.col0 = nb * BN;
    // one contiguous range of 128 rows, split in two halves of 64
    t.sb_half = (BN / 2) * gpr * 2 / 16;
    t.sb_src[0] = (uint32_t)(nb * BN) * gpr * 2u;
    t.sb_src[1] = (uint32_t)(nb * BN + BN / 2) * gpr * 2u;
  }

  {
    const int cpr8 = (int)gpr / 8;  // 16-byte chunks per table row
    t.sb_mask = (cpr8 >= 2 && (cpr8 & (cpr8 - 1)) == 0) ? cpr8 - 1 : 0;
#pragma unroll
    for (int j = 0; j < NS; ++j) t.sb_f[j] = ((t.sb_row[j] * (int)gpr) >> 7) & t.sb_mask;
  }

  const int msub = (t.nrows + 15) >> 4;
  if constexpr (kSmall) {
    static_assert(!kBf16W && kSmallRows == 16 * kRingMaxSub, "the small kernel runs 4-bit pieces of the ring form");
    switch (msub) {
      case 1: tile_body_ring<kGateUp, 1, 3, QE, kTblGroups>(g, t, L, Ssh, Bsh); break;
      case 2: tile_body_ring<kGateUp, 2, 3, QE, kTblGroups>(g, t, L, Ssh, Bsh); break;
      case 3: tile_body_ring<kGateUp, 3, 3, QE, kTblGroups>(g, t, L, Ssh, Bsh); break;
      default: tile_body_ring<kGateUp, 4, 3, QE, kTblGroups>(g, t, L, Ssh, Bsh); break;
    }
  } else {
    // (not instantiated in the small kernel, so no tile-body instance is
    // shared by two kernel instances)
    switch (msub) {
      case 1:
        if constexpr (!kBf16W) tile_body_ring<kGateUp, 1, 4, QE, kTblGroups>(g, t, L, Ssh, Bsh);
        else tile_body<kGateUp, kBf16W, 1>(g, t, L, Ssh, Bsh);
        break;
      case 2:
        if constexpr (!kBf16W && kRingMaxSub >= 2) tile_body_ring<kGateUp, 2, 4, QE, kTblGroups>(g, t, L, Ssh, Bsh);
        else tile_body<kGateUp, kBf16W, 2>(g, t, L, Ssh, Bsh);
        break;
      case 3:
        if constexpr (!kBf16W && kRingMaxSub >= 3) tile_body_ring<kGateUp, 3, 4, QE, kTblGroups>(g, t, L, Ssh, Bsh);
        else tile_body<kGateUp, kBf16W, 3>(g, t, L, Ssh, Bsh);
        break;
      case 4:
        if constexpr (!kBf16W && kRingMaxSub >= 4) tile_body_ring<kGateUp, 4, 4, QE, kTblGroups>(g, t, L, Ssh, Bsh);
        else tile_body<kGateUp, kBf16W, 4>(g, t, L, Ssh, Bsh);
        break;
      case 5: tile_body<kGateUp, kBf16W, 5>(g, t, L, Ssh, Bsh); break;
      case 6: tile_body<kGateUp, kBf16W, 6>(g, t, L, Ssh, Bsh); break;
      case 7: tile_body<kGateUp, kBf16W, 7>(g, t, L, Ssh, Bsh); break;
      case 8: tile_body<kGateUp, kBf16W, 8>(g, t, L, Ssh, Bsh); break;
      case 9: tile_body<kGateUp, kBf16W, 9>(g, t, L, Ssh, Bsh); break;
      case 10: tile_body<kGateUp, kBf16W, 10>(g, t, L, Ssh, Bsh); break;
      case 11: tile_body<kGateUp, kBf16W, 11>(g, t, L, Ssh, Bsh); break;
      case 12: tile_body<kGateUp, kBf16W, 12>(g, t, L, Ssh, Bsh); break;
      case 13: tile_body<kGateUp, kBf16W, 13>(g, t, L, Ssh, Bsh); break;
      case 14: tile_body<kGateUp, kBf16W, 14>(g, t, L, Ssh, Bsh); break;
      case 15: tile_body<kGateUp, kBf16W, 15>(g, t, L, Ssh, Bsh); break;
      default: tile_body<kGateUp, kBf16W, 16>(g, t, L, Ssh, Bsh); break;
    }
  }
}

int grid_blocks(int max_tiles, int nN) { return (max_tiles + kXcds - 1) / kXcds * kXcds * nN; }

}  // namespace

hipError_t launch_gemm_down(const GemmArgs& g, hipStream_t stream) {
  const int nN = (g.N + BN - 1) / BN;
  const dim3 grid(grid_blocks(g.max_tiles, nN));
  constexpr int G = kMaxGroups;
  if (g.wbf) hipLaunchKernelGGL((gemm_q4_kernel<false, true, false, G>), grid, dim3(NT), 0, stream, g);
  else if (g.small && g.Kdim <= 8 * 64)
    hipLaunchKernelGGL((gemm_q4_kernel<false, false, true, 8>), grid, dim3(NT), 0, stream, g);
  else if (g.small) hipLaunchKernelGGL((gemm_q4_kernel<false, false, true, G>), grid, dim3(NT), 0, stream, g);
  else hipLaunchKernelGGL((gemm_q4_kernel<false, false, false, G>), grid, dim3(NT), 0, stream, g);
  return hipGetLastError();
}

hipError_t launch_gemm_gate_up(const GemmArgs& g, hipStream_t stream) {
  const int nN = (g.I + BN / 2 - 1) / (BN / 2);
  const dim3 grid(grid_blocks(g.max_tiles, nN));
  constexpr int G = kMaxGroups;
  if (g.wbf) hipLaunchKernelGGL((gemm_q4_kernel<true, true, false, G>), grid, dim3(NT), 0, stream, g);
  else if (g.small) hipLaunchKernelGGL((gemm_q4_kernel<true, false, true, G>), grid, dim3(NT), 0, stream, g);
  else hipLaunchKernelGGL((gemm_q4_kernel<true, false, false, G>), grid, dim3(NT), 0, stream, g);
  return hipGetLastError();
}

}  // namespace moeq4
