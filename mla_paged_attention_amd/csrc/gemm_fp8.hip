// gemm_fp8.hip -- the block-scaled E4M3 projection beside MLA decode, for
// small decode batches (issue #28427 "DeepSeek-R1 KV Proj is Too Slow for TP":
// the fused q/kv down-projection runs a block-FP8 GEMM at a handful of
// tokens, where swapping the operands so that the weight rows fill the
// matrix instruction's 16-row side pays off).
//
//   c[i][j] = sum_k e4m3(a[i][k]) a_scale[i][k / 128] * e4m3(b[j][k]) b_scale[j / 128][k / 128]
//
//  1. quant_fp8_groups_kernel: bf16 activations -> E4M3 codes with one fp32
//     scale per token and 128-wide group (scale = max(amax, 1e-10) / 448,
//     codes rounded to nearest even from clamp(x / scale, +-448)).
//  2. gemm_fp8_kernel<MT>: one workgroup per 16 weight rows and 16 MT tokens.
//     The weight tile is the A operand of v_mfma_scale_f32_16x16x128_f8f6f4
//     (rows = output features), the tokens the B operand (columns), so a
//     single token wastes only the unused columns. Wave w of eight takes the
//     128-wide k blocks w, w + 8, ..., loading two blocks ahead; each block's
//     product is scaled in fp32 by its token's group scale times the block's
//     weight scale (the op's power-of-two scales cannot hold fp32 scales), and
//     the eight partial tiles are summed through LDS.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_internal.h"

namespace mla {
namespace {

typedef float g_f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int g_u32x4_t __attribute__((ext_vector_type(4)));
typedef int g_i32x8_t __attribute__((ext_vector_type(8)));

constexpr int kGemmWaves = 8;
constexpr int kGemmThreads = 64 * kGemmWaves;
constexpr int kGroup = 128;  // k per scale group = k per matrix op

__device__ __forceinline__ float bf16_to_f32(unsigned bits16) {
  return __builtin_bit_cast(float, bits16 << 16);
}

// One wave per (token, group); lane l holds elements 2 l and 2 l + 1.
__global__ void __launch_bounds__(256) quant_fp8_groups_kernel(const uint16_t* x, uint8_t* q,
                                                               float* scale, int32_t m,
                                                               int32_t k) {
  const int groups = k / kGroup;
  const int64_t gid = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (gid >= int64_t(m) * groups) return;
  const int lane = threadIdx.x & 63;
  const int64_t row = gid / groups;
  const int grp = int(gid - row * groups);
  const size_t off = size_t(row) * k + size_t(grp) * kGroup + 2 * lane;
  const unsigned two = *reinterpret_cast<const unsigned*>(x + off);
  const float v0 = bf16_to_f32(two & 0xffffu), v1 = bf16_to_f32(two >> 16);
  float amax = fmaxf(fabsf(v0), fabsf(v1));
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) amax = fmaxf(amax, __shfl_xor(amax, d));
  const float s = fmaxf(amax, 1e-10f) / 448.f;  // correctly rounded division
  const float y0 = fminf(fmaxf(v0 / s, -448.f), 448.f);
  const float y1 = fminf(fmaxf(v1 / s, -448.f), 448.f);
  const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
  *reinterpret_cast<uint16_t*>(q + off) = uint16_t(pk & 0xffff);
  if (lane == 0) scale[row * groups + grp] = s;
}

// 32 bytes (k = 32 g .. 32 g + 31 of one 128-wide block) of one row.
__device__ __forceinline__ g_i32x8_t load32(const uint8_t* p) {
  const g_u32x4_t lo = *reinterpret_cast<const g_u32x4_t*>(p);
  const g_u32x4_t hi = *reinterpret_cast<const g_u32x4_t*>(p + 16);
  return __builtin_bit_cast(g_i32x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

template <int MT>
__global__ void __launch_bounds__(kGemmThreads) gemm_fp8_kernel(
    const uint8_t* a, const float* a_scale, const uint8_t* b, const float* b_scale, uint16_t* c,
    int32_t m, int32_t n, int32_t k) {
  __shared__ g_f32x4_t red[kGemmWaves][MT][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int cc = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const int m0 = blockIdx.y * 16 * MT;
  const int kb_n = k / kGroup;

  // A operand: weight row n0 + cc; B operand of tile t: token m0 + 16 t + cc
  // (a token past m reads token 0 and is dropped at the store).
  const uint8_t* brow = b + size_t(n0 + cc) * k + 32 * g;
  const float* bs_row = b_scale + size_t(n0 / kGroup) * kb_n;
  const uint8_t* arow[MT];
  const float* as_row[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int tok = m0 + 16 * t + cc;
    const int tk = tok < m ? tok : 0;
    arow[t] = a + size_t(tk) * k + 32 * g;
    as_row[t] = a_scale + size_t(tk) * kb_n;
  }

  g_f32x4_t acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = g_f32x4_t{0.f, 0.f, 0.f, 0.f};

  struct Stage {
    g_i32x8_t w;
    g_i32x8_t x[MT];
    float s[MT];
  };
  auto load = [&](int kb, Stage& st) {
    st.w = load32(brow + size_t(kb) * kGroup);
    const float bs = bs_row[kb];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      st.x[t] = load32(arow[t] + size_t(kb) * kGroup);
      st.s[t] = as_row[t][kb] * bs;
    }
  };
  auto compute = [&](const Stage& st) {
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      // Format 0 = E4M3 for both operands; E8M0 scales 127 = 2^0.
      const g_f32x4_t d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
          st.w, st.x[t], g_f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
      acc[t] += d * st.s[t];
    }
  };

  // k blocks of this wave: wave, wave + 8, ...; two stages in flight.
  Stage s0, s1;
  int kb = wave;
  if (kb < kb_n) load(kb, s0);
  if (kb + kGemmWaves < kb_n) load(kb + kGemmWaves, s1);
  for (; kb < kb_n; kb += 2 * kGemmWaves) {
    compute(s0);
    if (kb + 2 * kGemmWaves < kb_n) load(kb + 2 * kGemmWaves, s0);
    if (kb + kGemmWaves < kb_n) {
      compute(s1);
      if (kb + 3 * kGemmWaves < kb_n) load(kb + 3 * kGemmWaves, s1);
    }
  }

#pragma unroll
  for (int t = 0; t < MT; ++t) red[wave][t][lane] = acc[t];
  __syncthreads();
  // Thread (t, lane) sums the eight partial tiles: rows n0 + 4 g + r of
  // token m0 + 16 t + cc.
  if (threadIdx.x < MT * 64) {
    const int t = threadIdx.x >> 6;
    g_f32x4_t sum = red[0][t][lane];
#pragma unroll
    for (int w = 1; w < kGemmWaves; ++w) sum += red[w][t][lane];
    const int tok = m0 + 16 * t + cc;
    if (tok < m) {
      unsigned short h[4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        h[r] = __builtin_bit_cast(unsigned short, (__bf16)sum[r]);  // nearest even
      const unsigned lo = unsigned(h[0]) | (unsigned(h[1]) << 16);
      const unsigned hi = unsigned(h[2]) | (unsigned(h[3]) << 16);
      *reinterpret_cast<unsigned long long*>(c + size_t(tok) * n + n0 + 4 * g) =
          (unsigned long long)lo | ((unsigned long long)hi << 32);
    }
  }
}

}  // namespace

hipError_t launch_quant_fp8_groups(const uint16_t* x, uint8_t* q, float* scale, int32_t m,
                                   int32_t k, hipStream_t stream) {
  const int64_t pairs = int64_t(m) * (k / kGroup);
  hipLaunchKernelGGL(quant_fp8_groups_kernel, dim3(unsigned((pairs + 3) / 4)), dim3(256), 0,
                     stream, x, q, scale, m, k);
  return hipGetLastError();
}

hipError_t launch_gemm_fp8(const uint8_t* a, const float* a_scale, const uint8_t* b,
                           const float* b_scale, uint16_t* c, int32_t m, int32_t n, int32_t k,
                           hipStream_t stream) {
  const int mt = m <= 16 ? 1 : (m <= 32 ? 2 : 4);
  const dim3 grid(unsigned(n / 16), unsigned((m + 16 * mt - 1) / (16 * mt)));
  if (mt == 1)
    hipLaunchKernelGGL(gemm_fp8_kernel<1>, grid, dim3(kGemmThreads), 0, stream, a, a_scale, b,
                       b_scale, c, m, n, k);
  else if (mt == 2)
    hipLaunchKernelGGL(gemm_fp8_kernel<2>, grid, dim3(kGemmThreads), 0, stream, a, a_scale, b,
                       b_scale, c, m, n, k);
  else
    hipLaunchKernelGGL(gemm_fp8_kernel<4>, grid, dim3(kGemmThreads), 0, stream, a, a_scale, b,
                       b_scale, c, m, n, k);
  return hipGetLastError();
}

}  // namespace mla
