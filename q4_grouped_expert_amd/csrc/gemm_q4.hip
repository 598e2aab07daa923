// Grouped GEMM over uneven expert groups on groupwise-affine 4-bit weights,
// dequantized tile by tile inside the GEMM and never written out
// ("Perplexity Lily 오픈소스 공개", alltoptrend.co.kr, section 5-1;
// "Apple silicon용 Lily, Qwen 추론 최적화", aitrends.kr, section
// "Qwen 구조와 Prefill 경로").
//
// gfx950 mapping
//  * A workgroup = 4 waves computes one block-map tile (<= 128 rows of one
//    expert group) against a 128-column slice of the expert's weight matrix.
//    Each wave owns all the tile's rows and 32 weight rows (two 16-column
//    MFMA subtiles), so every weight of the slice is dequantized by exactly
//    one lane of the workgroup.
//  * Activations (x rows gathered through sorted_idx, or h rows) are staged
//    in LDS as bf16, 64 reduction columns per stage (one quant group),
//    double-buffered, with a 16-byte-chunk XOR swizzle so the 16 rows a wave
//    reads per MFMA hit distinct banks.
//  * Weights go straight from global memory to VGPRs: a lane loads 8 bytes
//    = 16 codes of one weight row, applies q*scale+bias in fp32 (fma),
//    rounds to bf16 (v_cvt_pk_bf16_f32) and feeds the result as the B
//    operand of v_mfma_f32_16x16x32_bf16; accumulation is fp32.
//  * The reduction index is permuted identically for A and B inside each
//    64-wide group (lane group g, MFMA step s -> columns 16g+8s..16g+8s+7),
//    which lets one 8-byte code load serve both MFMA steps.
//  * Gate/up mode pairs gate row j and up row I+j in the same wave so the
//    SwiGLU epilogue h = bf16(silu(g)*u) happens in registers.
#include <math.h>

#include "common.hpp"

namespace moeq4 {

namespace {

constexpr int BM = kTileRows;  // rows per tile
constexpr int BK = 64;         // reduction columns per stage (= quant group)
constexpr int MS = BM / 16;    // 16-row MFMA subtiles per tile

__device__ __forceinline__ bf16x8 dequant8(uint32_t d, float s, float b) {
  // d holds 8 codes: element 2i in the low nibble of byte i, 2i+1 in the high
  const uint32_t lo = d & 0x0F0F0F0Fu;
  const uint32_t hi = (d >> 4) & 0x0F0F0F0Fu;
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float q0 = (float)((lo >> (8 * i)) & 0xFFu);
    const float q1 = (float)((hi >> (8 * i)) & 0xFFu);
    r[i] = pack_bf16x2(__builtin_fmaf(q0, s, b), __builtin_fmaf(q1, s, b));
  }
  return __builtin_bit_cast(bf16x8, r);
}

template <bool kGateUp>
__global__ __launch_bounds__(256) void gemm_q4_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * BK];

  const int tile = blockIdx.x;
  if (tile >= *g.n_tiles) return;  // grid is sized from an upper bound
  const int32_t* bmap = g.block_map + 4 * tile;
  const int e = bmap[0], row0 = bmap[1], nrows = bmap[2];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 15, lg = lane >> 4;
  const int Kd = g.Kdim;
  const int cpr = Kd / 2;   // code bytes per weight row
  const int gpr = Kd / 64;  // quant groups per weight row

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

  // This wave's two weight rows (one per 16-column subtile) for column ln.
  int wrow[2];
  bool jval[2];
  int ocol[2];
  if (kGateUp) {
    const int j0 = blockIdx.y * 64 + wave * 16;
    wrow[0] = j0 + ln;
    wrow[1] = g.I + j0 + ln;
    jval[0] = jval[1] = true;
    ocol[0] = ocol[1] = j0 + ln;
  } else {
    const int c0 = blockIdx.y * 128 + wave * 32;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      jval[j] = (c0 + 16 * j) < g.N;
      ocol[j] = c0 + 16 * j + ln;
      wrow[j] = jval[j] ? ocol[j] : 0;
    }
  }

  // Activation rows this lane stages: chunk q = tid + 256*i -> row q/8, 16-byte chunk q%8.
  const int ac = tid & 7;
  const uint16_t* arow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (tid >> 3) + 32 * i;
    arow[i] = nullptr;
    if (r < nrows) {
      const int p = row0 + r;
      if (kGateUp) {
        const int t = (p < g.R) ? g.sorted_idx[p] / g.topk : p - g.R;
        arow[i] = g.a + (size_t)t * Kd;
      } else {
        arow[i] = g.a + (size_t)p * Kd;
      }
    }
  }

  f32x4 acc[MS][2];
#pragma unroll
  for (int m = 0; m < MS; ++m)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[m][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 areg[4];
  u32x2 creg[2];
  uint32_t sreg[2], breg[2];

  auto load_a = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      areg[i] = u32x4{0u, 0u, 0u, 0u};
      if (arow[i]) areg[i] = *reinterpret_cast<const u32x4*>(arow[i] + kt * BK + 8 * ac);
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (tid >> 3) + 32 * i;
      const int phys = ac ^ (r & 7);
      *reinterpret_cast<u32x4*>(&As[buf][r * BK + phys * 8]) = areg[i];
    }
  };
  auto load_w = [&](int kt) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      creg[j] = *reinterpret_cast<const u32x2*>(codes + (size_t)wrow[j] * cpr + kt * 32 + 8 * lg);
      sreg[j] = scl[(size_t)wrow[j] * gpr + kt];
      breg[j] = bia[(size_t)wrow[j] * gpr + kt];
    }
  };

  const int nk = Kd / BK;
  load_a(0);
  store_a(0);
  load_w(0);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    bf16x8 bfrag[2][2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float s = bf16_bits_to_f32(sreg[j]);
      const float b = bf16_bits_to_f32(breg[j]);
      bfrag[j][0] = dequant8(creg[j][0], s, b);
      bfrag[j][1] = dequant8(creg[j][1], s, b);
    }
    if (kt + 1 < nk) {
      load_a(kt + 1);
      load_w(kt + 1);
    }
    const uint16_t* Ab = As[kt & 1];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
#pragma unroll
      for (int m = 0; m < MS; ++m) {
        if (m * 16 < nrows) {
          const int r = m * 16 + ln;
          const int phys = (2 * lg + st) ^ (r & 7);
          const bf16x8 av = *reinterpret_cast<const bf16x8*>(&Ab[r * BK + phys * 8]);
#pragma unroll
          for (int j = 0; j < 2; ++j)
            if (jval[j]) acc[m][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bfrag[j][st], acc[m][j], 0, 0, 0);
        }
      }
    }
    if (kt + 1 < nk) store_a((kt + 1) & 1);
    __syncthreads();
  }

  // Epilogue.  MFMA 16x16 output layout: lane holds rows 4*lg+i, column ln.
  if (kGateUp) {
    uint16_t* h = reinterpret_cast<uint16_t*>(g.c);
#pragma unroll
    for (int m = 0; m < MS; ++m) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = m * 16 + 4 * lg + i;
        if (r < nrows) {
          const float gv = acc[m][0][i], uv = acc[m][1][i];
          const float hv = gv / (1.0f + expf(-gv)) * uv;
          h[(size_t)(row0 + r) * g.I + ocol[0]] = f32_to_bf16_bits(hv);
        }
      }
    }
  } else {
    float* y = reinterpret_cast<float*>(g.c);
#pragma unroll
    for (int m = 0; m < MS; ++m) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = m * 16 + 4 * lg + i;
        if (r < nrows) {
#pragma unroll
          for (int j = 0; j < 2; ++j)
            if (jval[j]) y[(size_t)(row0 + r) * g.N + ocol[j]] = acc[m][j][i];
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_gate_up(const GemmArgs& g, hipStream_t stream) {
  dim3 grid(g.max_tiles, g.I / 64);
  hipLaunchKernelGGL(gemm_q4_kernel<true>, grid, dim3(256), 0, stream, g);
  return hipGetLastError();
}

hipError_t launch_gemm_down(const GemmArgs& g, hipStream_t stream) {
  dim3 grid(g.max_tiles, (g.N + 127) / 128);
  hipLaunchKernelGGL(gemm_q4_kernel<false>, grid, dim3(256), 0, stream, g);
  return hipGetLastError();
}

}  // namespace moeq4
