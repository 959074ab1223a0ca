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
//  2. gemm_fp8_kernel<NT, MT, G>: one workgroup per 16 NT weight rows and
//     16 MT tokens. Weight tiles are the A operand of
//     v_mfma_scale_f32_16x16x128_f8f6f4 (rows = output features), tokens the B
//     operand (columns), so a single token wastes only the unused columns.
//     Wave w of eight takes the 128-wide k blocks w, w + 8, ..., with two
//     groups of G blocks in flight (all seven of a wave's blocks at k = 7168
//     and the smallest tiles); each block's
//     product is scaled in fp32 by its token's group scale times the block's
//     weight scale (the op's power-of-two scales cannot hold fp32 scales), and
//     the eight partial tiles are summed through LDS.
//  3. gemm_fp8_lds_kernel<XM>: the same tiles for up to 16 tokens and
//     k <= 8192, with each workgroup's weight rows (and, up to 4 tokens, the
//     activations) streamed into LDS as 1 KB chunks before the matrix ops.
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

// The 32 k-bytes of lane group g within one 128-wide block of a row: bytes
// 16 g .. 16 g + 15 and 64 + 16 g .. 64 + 16 g + 15. Both operands use the same
// assignment (a dot product does not depend on the order of k), and each of
// the two loads of a wave reads one contiguous 64-byte half of every row.
__device__ __forceinline__ g_i32x8_t load32(const uint8_t* p) {
  const g_u32x4_t lo = *reinterpret_cast<const g_u32x4_t*>(p);
  const g_u32x4_t hi = *reinterpret_cast<const g_u32x4_t*>(p + 64);
  return __builtin_bit_cast(g_i32x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// One workgroup per RT NT weight rows x 16 MT tokens (RT = 16, or 8: lanes
// 8..15 of the op's 16-row side repeat rows 0..7 and their results are
// dropped, which doubles the workgroups streaming the weights). Wave w takes
// the k blocks w, w + 8, ..., loading G blocks per group, two groups in flight.
template <int RT, int NT, int MT, int G>
__global__ void __launch_bounds__(kGemmThreads) gemm_fp8_kernel(
    const uint8_t* a, const float* a_scale, const uint8_t* b, const float* b_scale, uint16_t* c,
    int32_t m, int32_t n, int32_t k) {
  __shared__ g_f32x4_t red[kGemmWaves][NT * MT][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int cc = lane & 15, g = lane >> 4;
  static_assert(RT == 16 || RT == 8, "rows per tile");
  const int n0 = blockIdx.x * RT * NT;
  const int m0 = blockIdx.y * 16 * MT;
  const int kb_n = k / kGroup;

  // A operands: weight rows n0 + 16 u + cc (a tile past n reads the last
  // tile and is dropped at the store). B operands: token m0 + 16 t + cc (a
  // token past m reads token 0 and is dropped).
  const uint8_t* brow[NT];
  const float* bs_row[NT];
#pragma unroll
  for (int u = 0; u < NT; ++u) {
    const int tile = min(n0 + RT * u, n - RT);
    brow[u] = b + size_t(tile + (cc & (RT - 1))) * k + 16 * g;
    bs_row[u] = b_scale + size_t(tile / kGroup) * kb_n;
  }
  const uint8_t* arow[MT];
  const float* as_row[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int tok = m0 + 16 * t + cc;
    const int tk = tok < m ? tok : 0;
    arow[t] = a + size_t(tk) * k + 16 * g;
    as_row[t] = a_scale + size_t(tk) * kb_n;
  }

  g_f32x4_t acc[NT][MT];
#pragma unroll
  for (int u = 0; u < NT; ++u)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[u][t] = g_f32x4_t{0.f, 0.f, 0.f, 0.f};

  struct Stage {
    g_i32x8_t w[NT];
    g_i32x8_t x[MT];
    float sb[NT];
    float sa[MT];
  };
  auto load_stage = [&](int kb, Stage& st) {
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      st.w[u] = load32(brow[u] + size_t(kb) * kGroup);
      st.sb[u] = bs_row[u][kb];
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      st.x[t] = load32(arow[t] + size_t(kb) * kGroup);
      st.sa[t] = as_row[t][kb];
    }
  };
  auto compute_stage = [&](const Stage& st) {
#pragma unroll
    for (int u = 0; u < NT; ++u)
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        // Format 0 = E4M3 for both operands; E8M0 scales 127 = 2^0.
        const g_f32x4_t d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            st.w[u], st.x[t], g_f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
        acc[u][t] += d * (st.sa[t] * st.sb[u]);
      }
  };

  // This wave's k blocks: wave + 8 i, i < cnt, in groups of G.
  const int cnt = kb_n > wave ? (kb_n - wave + kGemmWaves - 1) / kGemmWaves : 0;
  const int ng = (cnt + G - 1) / G;
  Stage s0[G], s1[G];
  auto load_group = [&](int gi, Stage (&st)[G]) {
#pragma unroll
    for (int j = 0; j < G; ++j)
      if (gi * G + j < cnt) load_stage(wave + kGemmWaves * (gi * G + j), st[j]);
  };
  auto compute_group = [&](int gi, const Stage (&st)[G]) {
#pragma unroll
    for (int j = 0; j < G; ++j)
      if (gi * G + j < cnt) compute_stage(st[j]);
  };
  load_group(0, s0);
  load_group(1, s1);
  for (int gi = 0; gi < ng; gi += 2) {
    compute_group(gi, s0);
    if (gi + 2 < ng) load_group(gi + 2, s0);
    if (gi + 1 < ng) {
      compute_group(gi + 1, s1);
      if (gi + 3 < ng) load_group(gi + 3, s1);
    }
  }

#pragma unroll
  for (int u = 0; u < NT; ++u)
#pragma unroll
    for (int t = 0; t < MT; ++t) red[wave][u * MT + t][lane] = acc[u][t];
  __syncthreads();
  // (tile, lane) pairs: rows n0 + RT u + 4 (lane / 16) + r of token
  // m0 + 16 t + lane % 16, summed over the eight waves.
  for (int idx = threadIdx.x; idx < NT * MT * 64; idx += kGemmThreads) {
    const int tile = idx >> 6, ln = idx & 63;
    if (4 * (ln >> 4) >= RT) continue;  // repeated rows of an 8-row tile
    const int u = tile / MT, t = tile - (tile / MT) * MT;
    g_f32x4_t sum = red[0][tile][ln];
#pragma unroll
    for (int w = 1; w < kGemmWaves; ++w) sum += red[w][tile][ln];
    const int tok = m0 + 16 * t + (ln & 15);
    const int row = n0 + RT * u + 4 * (ln >> 4);
    if (tok < m && n0 + RT * u < n) {
      unsigned short h[4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        h[r] = __builtin_bit_cast(unsigned short, (__bf16)sum[r]);  // nearest even
      const unsigned lo = unsigned(h[0]) | (unsigned(h[1]) << 16);
      const unsigned hi = unsigned(h[2]) | (unsigned(h[3]) << 16);
      *reinterpret_cast<unsigned long long*>(c + size_t(tok) * n + row) =
          (unsigned long long)lo | ((unsigned long long)hi << 32);
    }
  }
}

// The same product for up to 16 tokens and k <= 8192 with the weights staged
// in LDS. A workgroup's 16 weight rows are one contiguous run of 16 k bytes;
// it streams in whole 1 KB chunks with 16-byte direct-to-LDS loads, every
// chunk in flight at once (each CU keeps its whole share of the weights
// pending, and each load instruction reads 1 KB of consecutive bytes rather
// than 64 bytes of 16 rows). Lane l of the load of chunk ch fetches the chunk's
// 16-byte slot l ^ (ch % 16) into LDS slot l, so that the 16 rows a matrix
// operand gathers (k bytes apart) fall in distinct bank groups when k is an
// odd multiple of 1 KB. Wave w then multiplies the k blocks w, w + 8, ... out
// of LDS.
//
// Activations, XM = 4 (up to 4 tokens): their m k bytes are one contiguous
// run as well and stream into LDS the same way, a few chunks per workgroup.
// XM = 0 (up to 16 tokens): each lane loads its token's operand bytes itself.
constexpr int kLdsMaxK = 8192;
// Word 3 of a raw buffer resource (no swizzle, no stride, 32-bit format): loads
// at or past the record count return zeros.
constexpr int kBufferWord3 = 0x00020000;

__device__ __forceinline__ uint32_t swz_offset(uint32_t o) {
  const uint32_t ch = o >> 10, slot = (o >> 4) & 63;
  return (ch << 10) | ((slot ^ (ch & 15)) << 4);
}

// Streams bytes 0 .. bytes - 1 of run into dst (swizzled 1 KB chunks; a lane
// past the end reloads the run's last 16 bytes, into a slot nobody reads).
__device__ __forceinline__ void stream_run_to_lds(const uint8_t* run, uint32_t bytes,
                                                  uint8_t* dst, int wave, int lane) {
  const int nch = int((bytes + 1023) >> 10);
  for (int ch = wave; ch < nch; ch += kGemmWaves) {
    const uint32_t o = min((uint32_t(ch) << 10) + ((uint32_t(lane) ^ uint32_t(ch & 15)) << 4),
                           bytes - 16u);
    __builtin_amdgcn_global_load_lds(run + o,
                                     (void __attribute__((address_space(3)))*)(dst + (ch << 10)),
                                     16, 0, 0);
  }
}

__device__ __forceinline__ g_i32x8_t lds_operand(const uint8_t* buf, uint32_t o) {
  const g_u32x4_t lo = *reinterpret_cast<const g_u32x4_t*>(buf + swz_offset(o));
  const g_u32x4_t hi = *reinterpret_cast<const g_u32x4_t*>(buf + swz_offset(o + 64));
  return __builtin_bit_cast(g_i32x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

template <int XM>
__global__ void __launch_bounds__(kGemmThreads) gemm_fp8_lds_kernel(
    const uint8_t* a, const float* a_scale, const uint8_t* b, const float* b_scale, uint16_t* c,
    int32_t m, int32_t n, int32_t k) {
  // Weights, then (XM > 0) activations; the partial tiles reuse the front.
  __shared__ __attribute__((aligned(1024))) uint8_t lds[(16 + XM) * kLdsMaxK];
  uint8_t* const wbuf = lds;
  uint8_t* const xbuf = lds + 16 * kLdsMaxK;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int cc = lane & 15, g = lane >> 4;
  const int n0 = min(int(blockIdx.x) * 16, n - 16);
  const int kb_n = k / kGroup;

  // Weights: rows n0 .. n0 + 15 = bytes 0 .. 16 k - 1 of this run.
  stream_run_to_lds(b + size_t(n0) * k, 16u * uint32_t(k), wbuf, wave, lane);
  if constexpr (XM > 0) stream_run_to_lds(a, uint32_t(m) * uint32_t(k), xbuf, wave, lane);

  // Scales (and, XM = 0, activations of token cc) for this wave's k blocks,
  // while the weights stream. Buffer loads bounded by the m tokens' bytes
  // return zeros to the lanes of tokens past m, with no branch: a branch that
  // zeroed them would write registers that loads in flight also write, which
  // makes the compiler wait for every load, the weights' included. Nothing
  // here uses a loaded value before the wait below, for the same reason.
  constexpr int kMaxBlocks = kLdsMaxK / kGroup / kGemmWaves;  // 8
  const int cnt = kb_n > wave ? (kb_n - wave + kGemmWaves - 1) / kGemmWaves : 0;
  const __amdgpu_buffer_rsrc_t a_rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a), 0, m * k, kBufferWord3);
  const __amdgpu_buffer_rsrc_t as_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(a_scale), 0, m * kb_n * 4, kBufferWord3);
  const uint32_t a_off = uint32_t(cc) * uint32_t(k) + 16u * uint32_t(g);
  const uint32_t as_off = uint32_t(cc) * uint32_t(kb_n) * 4u;
  const float* bs_row = b_scale + size_t(n0 / kGroup) * kb_n;
  g_i32x8_t x[kMaxBlocks];
  float sa[kMaxBlocks], sb[kMaxBlocks];
#pragma unroll
  for (int j = 0; j < kMaxBlocks; ++j) {
    if (j < cnt) {
      const int kb = wave + kGemmWaves * j;
      if constexpr (XM == 0) {
        const uint32_t o = a_off + uint32_t(kb) * kGroup;
        const g_u32x4_t lo = __builtin_bit_cast(
            g_u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, o, 0, 0));
        const g_u32x4_t hi = __builtin_bit_cast(
            g_u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, o + 64, 0, 0));
        x[j] =
            __builtin_bit_cast(g_i32x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
      sa[j] = __builtin_bit_cast(
          float, __builtin_amdgcn_raw_buffer_load_b32(as_rsrc, as_off + 4u * uint32_t(kb), 0, 0));
      sb[j] = bs_row[kb];
    }
  }
  // Every chunk has landed (each wave waits for its own loads, the barrier
  // for everyone's).
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();

  g_f32x4_t acc = g_f32x4_t{0.f, 0.f, 0.f, 0.f};
  const bool tok_live = cc < m;
#pragma unroll
  for (int j = 0; j < kMaxBlocks; ++j) {
    if (j < cnt) {
      const uint32_t kofs = uint32_t(wave + kGemmWaves * j) * kGroup;
      const g_i32x8_t w = lds_operand(wbuf, a_off + kofs);
      if constexpr (XM > 0) {
        // Token cc's bytes (token 0's for a lane past m, then zeros).
        const g_i32x8_t xv = lds_operand(xbuf, (tok_live ? a_off : 16u * uint32_t(g)) + kofs);
        x[j] = tok_live ? xv : g_i32x8_t{0, 0, 0, 0, 0, 0, 0, 0};
      }
      const g_f32x4_t d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
          w, x[j], g_f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
      acc += d * (sa[j] * sb[j]);
    }
  }

  __syncthreads();  // every wave is done with the weights
  g_f32x4_t* red = reinterpret_cast<g_f32x4_t*>(lds);  // [kGemmWaves][64]
  red[wave * 64 + lane] = acc;
  __syncthreads();
  // Lane ln of the tile: rows n0 + 4 (ln / 16) + r of token ln % 16.
  if (threadIdx.x < 64) {
    const int ln = threadIdx.x;
    g_f32x4_t sum = red[ln];
#pragma unroll
    for (int w = 1; w < kGemmWaves; ++w) sum += red[w * 64 + ln];
    const int tok = ln & 15;
    const int row = n0 + 4 * (ln >> 4);
    if (tok < m) {
      unsigned short h[4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        h[r] = __builtin_bit_cast(unsigned short, (__bf16)sum[r]);  // nearest even
      const unsigned lo = unsigned(h[0]) | (unsigned(h[1]) << 16);
      const unsigned hi = unsigned(h[2]) | (unsigned(h[3]) << 16);
      *reinterpret_cast<unsigned long long*>(c + size_t(tok) * n + row) =
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
  // Tile shape by token count: 16-row weight tiles (132 workgroups at
  // n = 2112) up to 128 tokens; above, 32-row tiles cut the activations'
  // re-reads (a 64-row tile would spill). Measured: 8-row tiles, whose
  // upper lanes repeat rows, are slower at every m. Up to 16 tokens the
  // LDS-staged kernel (8.1 -> 6.9 us at m = 4, n = 2112, k = 7168).
  auto go = [&](auto kern, int rows, int mt) {
    const dim3 grid(unsigned((n + rows - 1) / rows), unsigned((m + 16 * mt - 1) / (16 * mt)));
    hipLaunchKernelGGL(kern, grid, dim3(kGemmThreads), 0, stream, a, a_scale, b, b_scale, c, m, n,
                       k);
  };
  if (m <= 4 && k <= kLdsMaxK)
    hipLaunchKernelGGL(gemm_fp8_lds_kernel<4>, dim3(unsigned(n / 16)), dim3(kGemmThreads), 0,
                       stream, a, a_scale, b, b_scale, c, m, n, k);
  else if (m <= 16 && k <= kLdsMaxK)
    hipLaunchKernelGGL(gemm_fp8_lds_kernel<0>, dim3(unsigned(n / 16)), dim3(kGemmThreads), 0,
                       stream, a, a_scale, b, b_scale, c, m, n, k);
  else if (m <= 16)
    go(gemm_fp8_kernel<16, 1, 1, 4>, 16, 1);
  else if (m <= 32)
    go(gemm_fp8_kernel<16, 1, 2, 3>, 16, 2);
  else if (m <= 128)
    go(gemm_fp8_kernel<16, 1, 4, 2>, 16, 4);
  else
    go(gemm_fp8_kernel<16, 2, 4, 1>, 32, 4);
  return hipGetLastError();
}

}  // namespace mla
