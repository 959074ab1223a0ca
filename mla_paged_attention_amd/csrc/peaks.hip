// peaks.hip -- calibration kernels that measure what this MI355X actually
// delivers, as denominators beside the vendor peaks: HBM read bandwidth
// (a direct-to-LDS stream of 36 KB tiles shaped like the attention kernels'
// KV ring, in order and in scattered order as a paged cache places its
// blocks, a gather of single rows as sparse decode reads them, and a plain
// vector read) and dense matrix-core throughput
// (v_mfma_f32_16x16x32_bf16 and v_mfma_scale_f32_16x16x128_f8f6f4 in E4M3).
// Measurement only: built into libmla_peaks.so, never into the decode
// library. The caller times the launches with events on `stream`.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kTileBytes = 36864;              // one ring stage of the attention kernels
constexpr int kStreamThreads = 256;
constexpr int kLoadsPerTile = kTileBytes / (16 * kStreamThreads);  // 9
constexpr int kStages = 4;

template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Workgroup w streams tiles w, w + G, w + 2G, ... (G = grid size) into a
// four-stage LDS ring with IN_FLIGHT tiles pending, as the attention
// kernels' ring does (16-byte direct-to-LDS loads, cache policy `policy`).
template <int IN_FLIGHT, int POLICY>
__global__ void __launch_bounds__(kStreamThreads) stream_lds_kernel(const uint8_t* src,
                                                                    int64_t ntiles) {
  __shared__ uint8_t ring[kStages][kTileBytes];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int64_t issued = 0;
  for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    if (issued >= IN_FLIGHT) wait_vmem<(IN_FLIGHT - 1) * kLoadsPerTile>();
    const uint8_t* base = src + t * kTileBytes + tid * 16;
    uint8_t* dst = &ring[issued % kStages][0] + wave * 64 * 16;
#pragma unroll
    for (int i = 0; i < kLoadsPerTile; ++i)
      __builtin_amdgcn_global_load_lds(
          base + i * kStreamThreads * 16,
          (void __attribute__((address_space(3)))*)(dst + i * kStreamThreads * 16), 16, 0, POLICY);
    ++issued;
  }
  wait_vmem<0>();
}

// The same ring over tiles in scattered order, as a paged cache reads its
// blocks: workgroup w's k-th tile is tile ((w * per_wg + k) * stride) % ntiles
// (stride coprime to ntiles, so every tile is read once), two tiles in
// flight, non-temporal loads.
__global__ void __launch_bounds__(kStreamThreads) stream_perm_kernel(const uint8_t* src,
                                                                   int64_t ntiles, int64_t stride,
                                                                   int per_wg) {
  __shared__ uint8_t ring[kStages][kTileBytes];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  auto issue = [&](int k) {
    const int64_t t = ((int64_t(blockIdx.x) * per_wg + k) * stride) % ntiles;
    const uint8_t* base = src + t * kTileBytes + tid * 16;
    uint8_t* dst = &ring[k % kStages][0] + wave * 64 * 16;
#pragma unroll
    for (int i = 0; i < kLoadsPerTile; ++i)
      __builtin_amdgcn_global_load_lds(
          base + i * kStreamThreads * 16,
          (void __attribute__((address_space(3)))*)(dst + i * kStreamThreads * 16), 16, 0, 2);
  };
  issue(0);
  if (per_wg > 1) issue(1);
  for (int k = 0; k < per_wg; ++k) {
    if (k + 1 < per_wg) wait_vmem<kLoadsPerTile>(); else wait_vmem<0>();
    __syncthreads();
    if (k + 2 < per_wg) issue(k + 2);
  }
}

// Row gather, as sparse decode reads its listed tokens: every 36 KB tile is
// 36864 / row_bytes rows taken from hashed positions among nrows rows of
// row_bytes bytes, two tiles in flight, non-temporal loads.
__global__ void __launch_bounds__(kStreamThreads) gather_rows_kernel(const uint8_t* src,
                                                                   int64_t nrows, int row_bytes,
                                                                   int per_wg) {
  __shared__ uint8_t ring[kStages][kTileBytes];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int chunks = row_bytes / 16;
  auto issue = [&](int k) {
    uint8_t* dst = &ring[k % kStages][0] + wave * 64 * 16;
#pragma unroll
    for (int i = 0; i < kLoadsPerTile; ++i) {
      const int pos = i * kStreamThreads + tid;
      const int t = pos / chunks, ch = pos - (pos / chunks) * chunks;
      uint32_t h = uint32_t(blockIdx.x) * 2654435761u ^ uint32_t(k) * 40503u ^
                   uint32_t(t) * 2246822519u;
      h ^= h >> 15;
      h *= 2654435761u;
      h ^= h >> 13;
      const int64_t row = int64_t(h % uint64_t(nrows));
      __builtin_amdgcn_global_load_lds(
          src + row * row_bytes + ch * 16,
          (void __attribute__((address_space(3)))*)(dst + i * kStreamThreads * 16), 16, 0, 2);
    }
  };
  issue(0);
  if (per_wg > 1) issue(1);
  for (int k = 0; k < per_wg; ++k) {
    if (k + 1 < per_wg) wait_vmem<kLoadsPerTile>(); else wait_vmem<0>();
    __syncthreads();
    if (k + 2 < per_wg) issue(k + 2);
  }
}

// Plain read: 16-byte vector loads, eight in flight per thread, folded into
// one word per thread so that nothing is optimised away.
__global__ void __launch_bounds__(256) read_kernel(const u32x4_t* src, int64_t n16,
                                                   unsigned* sink) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  unsigned acc = 0;
  int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  for (; i + 7 * stride < n16; i += 8 * stride) {
    u32x4_t v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = __builtin_nontemporal_load(src + i + k * stride);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc ^= v[k][0] ^ v[k][1] ^ v[k][2] ^ v[k][3];
  }
  for (; i < n16; i += stride) {
    const u32x4_t v = src[i];
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;  // practically never: keeps the loads live
}

// Matrix cores: each wave runs `iters` rounds of four independent
// accumulation chains on register operands.
__global__ void __launch_bounds__(256) mfma_bf16_kernel(int iters, float* sink) {
  const int lane = threadIdx.x & 63;
  bf16x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * float((lane * 8 + i) % 17));
    b[i] = (__bf16)(0.001f * float((lane * 5 + i) % 13));
  }
  f32x4_t c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0, c2 = c0, c3 = c0;
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c3, 0, 0, 0);
  }
  const f32x4_t s = c0 + c1 + c2 + c3;
  if (s[0] == -1.f) sink[blockIdx.x] = s[1];  // keeps the chains live
}

__global__ void __launch_bounds__(256) mfma_fp8_kernel(int iters, float* sink) {
  const int lane = threadIdx.x & 63;
  i32x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = 0x38302820 + ((lane + i) & 7);   // small E4M3 codes
    b[i] = 0x30282018 + ((lane * 3 + i) & 7);
  }
  f32x4_t c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0, c2 = c0, c3 = c0;
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c0, 0, 0, 0, 127, 0, 127);
    c1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c1, 0, 0, 0, 127, 0, 127);
    c2 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c2, 0, 0, 0, 127, 0, 127);
    c3 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c3, 0, 0, 0, 127, 0, 127);
  }
  const f32x4_t s = c0 + c1 + c2 + c3;
  if (s[0] == -1.f) sink[blockIdx.x] = s[1];
}

}  // namespace

extern "C" {

// Streams ntiles 36,864-byte tiles of src (ntiles * 36864 bytes must lie in
// the buffer) through LDS with `in_flight` (1..3) tiles pending per
// workgroup; nontemporal != 0 sets the ring loads' non-temporal bit.
int peaks_stream_lds(const void* src, int64_t ntiles, int grid, int in_flight, int nontemporal,
                     void* stream) {
  if (!src || ntiles <= 0 || grid <= 0 || in_flight < 1 || in_flight > 3) return -1;
  const uint8_t* p = static_cast<const uint8_t*>(src);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 g(grid), b(kStreamThreads);
  if (nontemporal) {  // the non-temporal cache-policy bit, as the attention ring uses
    if (in_flight == 1) hipLaunchKernelGGL((stream_lds_kernel<1, 2>), g, b, 0, s, p, ntiles);
    else if (in_flight == 2) hipLaunchKernelGGL((stream_lds_kernel<2, 2>), g, b, 0, s, p, ntiles);
    else hipLaunchKernelGGL((stream_lds_kernel<3, 2>), g, b, 0, s, p, ntiles);
  } else {
    if (in_flight == 1) hipLaunchKernelGGL((stream_lds_kernel<1, 0>), g, b, 0, s, p, ntiles);
    else if (in_flight == 2) hipLaunchKernelGGL((stream_lds_kernel<2, 0>), g, b, 0, s, p, ntiles);
    else hipLaunchKernelGGL((stream_lds_kernel<3, 0>), g, b, 0, s, p, ntiles);
  }
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

// Streams grid * per_wg 36,864-byte tiles of src in scattered order (tile k
// of workgroup w is ((w * per_wg + k) * stride) % ntiles; grid * per_wg <=
// ntiles; ntiles * 36864 bytes must lie in the buffer).
int peaks_stream_perm(const void* src, int64_t ntiles, int64_t stride, int grid, int per_wg,
                      void* stream) {
  if (!src || ntiles <= 0 || stride <= 0 || grid <= 0 || per_wg <= 0 ||
      int64_t(grid) * per_wg > ntiles)
    return -1;
  hipLaunchKernelGGL(stream_perm_kernel, dim3(grid), dim3(kStreamThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint8_t*>(src), ntiles,
                     stride, per_wg);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

// Gathers grid * per_wg tiles of rows of row_bytes (1152 or 576) bytes from
// hashed rows among the nrows rows of src (nrows * row_bytes bytes).
int peaks_gather_rows(const void* src, int64_t nrows, int row_bytes, int grid, int per_wg,
                      void* stream) {
  if (!src || nrows <= 0 || (row_bytes != 1152 && row_bytes != 576) || grid <= 0 || per_wg <= 0)
    return -1;
  hipLaunchKernelGGL(gather_rows_kernel, dim3(grid), dim3(kStreamThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint8_t*>(src), nrows,
                     row_bytes, per_wg);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

// Reads n16 16-byte words of src (16-byte aligned) with `grid` workgroups.
int peaks_read(const void* src, int64_t n16, int grid, unsigned* sink, void* stream) {
  if (!src || !sink || n16 <= 0 || grid <= 0 || (reinterpret_cast<uintptr_t>(src) & 15)) return -1;
  hipLaunchKernelGGL(read_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4_t*>(src), n16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

// grid workgroups of four waves, each wave 4 * iters matrix ops; sink holds
// grid floats. Flops: grid * 4 * 4 * iters * (16384 bf16 | 65536 fp8).
int peaks_mfma(int fp8, int grid, int iters, float* sink, void* stream) {
  if (!sink || grid <= 0 || iters <= 0) return -1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (fp8)
    hipLaunchKernelGGL(mfma_fp8_kernel, dim3(grid), dim3(256), 0, s, iters, sink);
  else
    hipLaunchKernelGGL(mfma_bf16_kernel, dim3(grid), dim3(256), 0, s, iters, sink);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

}  // extern "C"
