// absorb.hip -- the per-head bf16 products on either side of absorbed MLA
// decode. The decode kernels take a 576-wide query whose first 512 columns
// are the no-rope query absorbed into the 512-wide latent space, and return
// a 512-wide latent output that the value up-projection maps back to the
// head's value dimension (DeepSeek's shapes: 128 no-rope and 64 rope query
// dims, 512 latent dims, 128 value dims):
//
//   q[b][h][0:512]   = sum_d q_nope[b][h][d] W_UK[h][d][0:512]     (d < 128)
//   q[b][h][512:576] = q_rope[b][h][0:64]
//   o[b][h][v]       = sum_c o_latent[b][h][c] W_UV[h][v][c]       (c < 512)
//
// Both weights are 128 x 512 bf16 per head (W_UV stored one 512-wide row per
// value dim, the up-projection's own layout). The products are skinny (a
// decode batch of rows against a 128 KB weight per head), so the work is cut
// to spread the bytes over all CUs rather than to maximise reuse: a single
// CU streams only a small share of HBM bandwidth, and every extra split is
// an L2 re-read, not an HBM one. One workgroup takes (head, a slice of NS
// output columns, 64 batch rows): it copies the weight slice into LDS (rows
// padded by 16 bytes), with all of its loads issued before the first store,
// and its four waves take one 16-row batch tile each. The products run on
// v_mfma_f32_16x16x32_bf16 with the weight as the A operand (16 output
// columns) and the activations as the B operand (16 batch rows, 16 bytes of
// consecutive k per lane straight from memory), so each lane ends with four
// consecutive output columns of one batch row and stores them as 8 bytes.
// W_UK's A operand is read with gfx950's transposing LDS read
// ds_read_b64_tr_b16 (k runs down its rows); W_UV's with 16-byte reads along
// its rows. With a head count that is a multiple of 8, each XCD keeps whole
// heads (absorb_task), so a head's activations and weight slices are fetched
// into one L2 only.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_internal.h"

namespace mla {
namespace {

typedef float a_f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int a_u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int a_u32x2_t __attribute__((ext_vector_type(2)));
typedef short a_s16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 a_bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int kAbsorbThreads = 256;
constexpr int kAbsorbRows = 64;   // batch rows per workgroup: one 16-row tile per wave
constexpr int kRope = 64;
constexpr int kNope = 128;        // no-rope query dims = value dims
constexpr int kLatent = 512;

__device__ __forceinline__ a_u32x2_t pack4(a_f32x4_t v) {
  const uint32_t lo = __builtin_bit_cast(uint16_t, (__bf16)v[0]) |
                      (uint32_t(__builtin_bit_cast(uint16_t, (__bf16)v[1])) << 16);
  const uint32_t hi = __builtin_bit_cast(uint16_t, (__bf16)v[2]) |
                      (uint32_t(__builtin_bit_cast(uint16_t, (__bf16)v[3])) << 16);
  return a_u32x2_t{lo, hi};  // nearest even
}

// Workgroup -> (head, column slice, batch group) of a one-dimensional launch
// of heads * slices * groups workgroups. Workgroups are dispatched round-robin
// over the eight XCDs (each with its own L2), so with a head count that is a
// multiple of 8 the XCD of launch index L (L mod 8) keeps the heads h = L mod 8
// (mod 8): the slices of one batch group (which read the same activation rows)
// and the groups of one slice (which read the same weight slice) then share
// one L2. Other head counts keep the plain order (head and slice fastest).
struct AbsorbTask {
  int h, slice, group;
};

__device__ __forceinline__ AbsorbTask absorb_task(int L, int heads, int slices, int groups) {
  (void)groups;
  if ((heads & 7) == 0) {
    const int x = L & 7, local = L >> 3;
    const int per_head = slices * groups;
    const int hh = local / per_head, rem = local - hh * per_head;
    return AbsorbTask{8 * hh + x, rem % slices, rem / slices};
  }
  const int hs = heads * slices;
  const int g = L / hs, r = L - g * hs;
  return AbsorbTask{r / slices, r % slices, g};
}

// Copy a ROWS x COLS bf16 block (source row stride `stride` elements) into
// LDS rows of COLS + 8: every load of the thread is issued before its first
// LDS store.
template <int ROWS, int COLS>
__device__ __forceinline__ void stage(const uint16_t* src, size_t stride, uint16_t* dst,
                                      int tid) {
  constexpr int kChunks = ROWS * COLS / 8, kPer = kChunks / kAbsorbThreads;
  static_assert(kChunks % kAbsorbThreads == 0, "slice must split evenly");
  a_u32x4_t v[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int ch = tid + i * kAbsorbThreads, r = ch / (COLS / 8), q = ch % (COLS / 8);
    v[i] = *reinterpret_cast<const a_u32x4_t*>(src + r * stride + 8 * q);
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int ch = tid + i * kAbsorbThreads, r = ch / (COLS / 8), q = ch % (COLS / 8);
    *reinterpret_cast<a_u32x4_t*>(dst + r * (COLS + 8) + 8 * q) = v[i];
  }
}

// q[b][h] = [q_nope[b][h] . W_UK[h], q_rope[b][h]] for the (head, slice of NS
// columns, group of 64 TW batch rows) of absorb_task, TW 16-row tiles per
// wave. Slice 0 also copies the rope part of its rows.
template <int NS, int TW>
__global__ void __launch_bounds__(kAbsorbThreads) absorb_q_kernel(const uint16_t* x,
                                                                  const uint16_t* w,
                                                                  const uint16_t* rope,
                                                                  uint16_t* c, int32_t batch,
                                                                  int32_t heads) {
  constexpr int K = kNope, kOut = kLatent + kRope, kJ = NS / 16, kSplit = kLatent / NS;
  constexpr int kPitch = NS + 8, kRows = kAbsorbRows * TW;
  __shared__ __attribute__((aligned(16))) uint16_t sw[K * kPitch];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int cc = lane & 15, g = lane >> 4;
  const AbsorbTask task =
      absorb_task(blockIdx.x, heads, kSplit, (batch + kRows - 1) / kRows);
  const int h = task.h, n0 = task.slice * NS;
  const int b0 = task.group * kRows;
  const int bt = b0 + 16 * TW * wave;  // this wave's first batch row

  // B operand: batch row bt + 16 t + cc, k = 32 s + 8 g .. + 7 (a row past
  // the batch reads the last row and is dropped at the store).
  a_u32x4_t xf[TW][K / 32];
#pragma unroll
  for (int t = 0; t < TW; ++t) {
    const int b = min(bt + 16 * t + cc, batch - 1);
    const uint16_t* p = x + (size_t(b) * heads + h) * K + 8 * g;
#pragma unroll
    for (int s = 0; s < K / 32; ++s) xf[t][s] = *reinterpret_cast<const a_u32x4_t*>(p + 32 * s);
  }
  // The rope columns (slice 0 only) are requested with the other operands and
  // stored after the barrier, so their round trip overlaps the weights'.
  constexpr int kRopeIters = (kRows * kRope / 8 + kAbsorbThreads - 1) / kAbsorbThreads;
  a_u32x4_t rv[kRopeIters];
  if (n0 == 0) {
#pragma unroll
    for (int it = 0; it < kRopeIters; ++it) {
      const int i = tid + it * kAbsorbThreads;
      const int b = b0 + i / (kRope / 8), q = i % (kRope / 8);
      if (i < kRows * kRope / 8 && b < batch)
        rv[it] = *reinterpret_cast<const a_u32x4_t*>(rope + (size_t(b) * heads + h) * kRope + 8 * q);
    }
  }
  stage<K, NS>(w + size_t(h) * K * kLatent + n0, kLatent, sw, tid);
  __syncthreads();

  if (n0 == 0) {
#pragma unroll
    for (int it = 0; it < kRopeIters; ++it) {
      const int i = tid + it * kAbsorbThreads;
      const int b = b0 + i / (kRope / 8), q = i % (kRope / 8);
      if (i < kRows * kRope / 8 && b < batch)
        *reinterpret_cast<a_u32x4_t*>(c + (size_t(b) * heads + h) * kOut + kLatent + 8 * q) =
            rv[it];
    }
  }
  if (bt >= batch) return;  // no rows in this wave's tiles

  a_f32x4_t acc[kJ][TW];
#pragma unroll
  for (int j = 0; j < kJ; ++j)
#pragma unroll
    for (int t = 0; t < TW; ++t) acc[j][t] = a_f32x4_t{0.f, 0.f, 0.f, 0.f};

  // A operand by transposing reads: lane 4a + e of a 16-lane group gets
  // element e of the 8-byte words of lanes a, a + 4, a + 8, a + 12; lane l
  // addresses row k0 + 8 g + (l % 16) / 4 (+ 4 for the second read), columns
  // 4 (l % 4) .. of its 16-column block, so lane (cc, g) receives
  // W[k0 + 8 g + i][block + cc], i = 0..7.
  const int lr = (lane & 15) >> 2, lc = 4 * (lane & 3);
#pragma unroll
  for (int s = 0; s < K / 32; ++s) {
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      const uint16_t* p0 = sw + (32 * s + 8 * g + lr) * kPitch + 16 * j + lc;
      const a_s16x4_t t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) a_s16x4_t*)(p0));
      const a_s16x4_t t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) a_s16x4_t*)(p0 + 4 * kPitch));
      const a_bf16x8_t av = __builtin_bit_cast(
          a_bf16x8_t, __builtin_shufflevector(t0, t1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int t = 0; t < TW; ++t)
        acc[j][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            av, __builtin_bit_cast(a_bf16x8_t, xf[t][s]), acc[j][t], 0, 0, 0);
    }
  }

  // D[4 g + r][cc] of (j, t) = q[bt + 16 t + cc][h][n0 + 16 j + 4 g + r].
#pragma unroll
  for (int t = 0; t < TW; ++t) {
    const int b = bt + 16 * t + cc;
    if (b < batch) {
      uint16_t* dst = c + (size_t(b) * heads + h) * kOut + n0 + 4 * g;
#pragma unroll
      for (int j = 0; j < kJ; ++j)
        *reinterpret_cast<a_u32x2_t*>(dst + 16 * j) = pack4(acc[j][t]);
    }
  }
}

// o[b][h] = o_latent[b][h] . W_UV[h]^T for the (head, slice of NS value
// columns, 64-row batch group) of absorb_task.
template <int NS>
__global__ void __launch_bounds__(kAbsorbThreads) absorb_out_kernel(const uint16_t* x,
                                                                    const uint16_t* w,
                                                                    uint16_t* c, int32_t batch,
                                                                    int32_t heads) {
  constexpr int K = kLatent, kOut = kNope, kJ = NS / 16, kSplit = kNope / NS;
  constexpr int kPitch = K + 8;
  __shared__ __attribute__((aligned(16))) uint16_t sw[NS * kPitch];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int cc = lane & 15, g = lane >> 4;
  const AbsorbTask task =
      absorb_task(blockIdx.x, heads, kSplit, (batch + kAbsorbRows - 1) / kAbsorbRows);
  const int h = task.h, n0 = task.slice * NS;
  const int bt = task.group * kAbsorbRows + 16 * wave;

  a_u32x4_t xf[K / 32];
  {
    const int b = min(bt + cc, batch - 1);
    const uint16_t* p = x + (size_t(b) * heads + h) * K + 8 * g;
#pragma unroll
    for (int s = 0; s < K / 32; ++s) xf[s] = *reinterpret_cast<const a_u32x4_t*>(p + 32 * s);
  }
  stage<NS, K>(w + (size_t(h) * kNope + n0) * K, K, sw, tid);
  __syncthreads();
  if (bt >= batch) return;

  a_f32x4_t acc[kJ];
#pragma unroll
  for (int j = 0; j < kJ; ++j) acc[j] = a_f32x4_t{0.f, 0.f, 0.f, 0.f};

  // A operand: lane (cc, g) reads W_UV[h][n0 + 16 j + cc][32 s + 8 g .. + 7].
#pragma unroll
  for (int s = 0; s < K / 32; ++s) {
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      const a_u32x4_t av =
          *reinterpret_cast<const a_u32x4_t*>(sw + (16 * j + cc) * kPitch + 32 * s + 8 * g);
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          __builtin_bit_cast(a_bf16x8_t, av), __builtin_bit_cast(a_bf16x8_t, xf[s]), acc[j], 0,
          0, 0);
    }
  }

  const int b = bt + cc;
  if (b < batch) {
    uint16_t* dst = c + (size_t(b) * heads + h) * kOut + n0 + 4 * g;
#pragma unroll
    for (int j = 0; j < kJ; ++j) *reinterpret_cast<a_u32x2_t*>(dst + 16 * j) = pack4(acc[j]);
  }
}

// Bytes one CU moves for an absorb_q launch with slices of NS columns and
// `rows` batch rows per workgroup: the launch's workgroup bytes (activations,
// weight slice, output, rope share) spread over min(workgroups, 256) CUs.
// Re-reads of a slice or a row by another workgroup are L2 hits, but they
// still pass through a CU, and a CU's own stream rate is what bounds these
// small products.
inline double absorb_q_cu_bytes(int32_t batch, int32_t heads, int ns, int rows) {
  const long groups = long(heads) * (kLatent / ns) * ((batch + rows - 1) / rows);
  const double r = double(batch < rows ? batch : rows);
  const double per = r * kNope * 2 + double(kNope) * ns * 2 + r * ns * 2 +
                     r * kRope * 2 * ns / kLatent;
  return per * groups / double(groups < 256 ? groups : 256);
}

}  // namespace

// absorb_q: the slice width and rows per workgroup that move the fewest
// bytes per CU (absorb_q_cu_bytes) among four shapes.
hipError_t launch_absorb_q(const uint16_t* q_nope, const uint16_t* w_uk, const uint16_t* q_rope,
                           uint16_t* q, int32_t batch, int32_t heads, hipStream_t stream) {
  struct Shape { int ns, tw; };
  constexpr Shape kShapes[] = {{32, 1}, {128, 1}, {128, 2}, {256, 2}};
  int best = 0;
  double best_bytes = 0;
  for (int i = 0; i < 4; ++i) {
    const double v = absorb_q_cu_bytes(batch, heads, kShapes[i].ns, kAbsorbRows * kShapes[i].tw);
    if (i == 0 || v < best_bytes) best = i, best_bytes = v;
  }
  const int ns = kShapes[best].ns, rows = kAbsorbRows * kShapes[best].tw;
  const dim3 grid(unsigned(heads) * unsigned(kLatent / ns) * unsigned((batch + rows - 1) / rows));
  const dim3 block(kAbsorbThreads);
  switch (best) {
    case 0:
      hipLaunchKernelGGL((absorb_q_kernel<32, 1>), grid, block, 0, stream, q_nope, w_uk, q_rope,
                         q, batch, heads);
      break;
    case 1:
      hipLaunchKernelGGL((absorb_q_kernel<128, 1>), grid, block, 0, stream, q_nope, w_uk, q_rope,
                         q, batch, heads);
      break;
    case 2:
      hipLaunchKernelGGL((absorb_q_kernel<128, 2>), grid, block, 0, stream, q_nope, w_uk, q_rope,
                         q, batch, heads);
      break;
    default:
      hipLaunchKernelGGL((absorb_q_kernel<256, 2>), grid, block, 0, stream, q_nope, w_uk, q_rope,
                         q, batch, heads);
      break;
  }
  return hipGetLastError();
}

// absorb_out: 32 value columns per workgroup, or 16 where that leaves fewer
// than 256 workgroups.
hipError_t launch_absorb_out(const uint16_t* o_latent, const uint16_t* w_uv, uint16_t* o,
                             int32_t batch, int32_t heads, hipStream_t stream) {
  const unsigned groups = unsigned((batch + kAbsorbRows - 1) / kAbsorbRows);
  if (long(heads) * (kNope / 32) * groups >= 256)
    hipLaunchKernelGGL(absorb_out_kernel<32>, dim3(unsigned(heads) * (kNope / 32) * groups),
                       dim3(kAbsorbThreads), 0, stream, o_latent, w_uv, o, batch, heads);
  else
    hipLaunchKernelGGL(absorb_out_kernel<16>, dim3(unsigned(heads) * (kNope / 16) * groups),
                       dim3(kAbsorbThreads), 0, stream, o_latent, w_uv, o, batch, heads);
  return hipGetLastError();
}

}  // namespace mla
