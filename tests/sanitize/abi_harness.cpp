// abi_harness.cpp -- drives every entry point of include/mla.h through its
// host-side validation, for a build of mla_api.hip's host code under
// AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_sanitizers.py).
// The kernel launchers are stubs: on a machine without a GPU no call may get
// past the device query, and the harness fails if one does.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdio.h>

#include "../../include/mla.h"
#include "../../mla_paged_attention_amd/csrc/mla_internal.h"

static int g_launches = 0;

namespace mla {
hipError_t launch_plan(const int32_t*, int32_t, int32_t, int32_t, int32_t, const WorkspaceLayout&,
                       void*,
                       hipStream_t) { ++g_launches; return hipErrorUnknown; }
hipError_t launch_attention(const AttnArgs&, int, int32_t, hipStream_t) {
  ++g_launches; return hipErrorUnknown;
}
hipError_t launch_combine(const float*, const float*, const int32_t*, uint16_t*, float*, int32_t,
                          int32_t, int, int32_t, hipStream_t) { ++g_launches; return hipErrorUnknown; }
hipError_t launch_sparse_rows(const int32_t*, int32_t, const int32_t*, const int32_t*, int32_t,
                              int32_t, int32_t, int32_t, int32_t, int32_t, int32_t*, int32_t*,
                              void*, int32_t*, hipStream_t) { ++g_launches; return hipErrorUnknown; }
hipError_t launch_clear_word(int32_t*, hipStream_t) { ++g_launches; return hipErrorUnknown; }
hipError_t launch_quant_fp8_groups(const uint16_t*, uint8_t*, float*, int32_t, int32_t,
                                   hipStream_t) { ++g_launches; return hipErrorUnknown; }
hipError_t launch_gemm_fp8(const uint8_t*, const float*, const uint8_t*, const float*, uint16_t*,
                           int32_t, int32_t, int32_t, hipStream_t) { ++g_launches; return hipErrorUnknown; }
hipError_t launch_absorb_q(const uint16_t*, const uint16_t*, const uint16_t*, uint16_t*, int32_t,
                           int32_t, hipStream_t) { ++g_launches; return hipErrorUnknown; }
hipError_t launch_absorb_out(const uint16_t*, const uint16_t*, uint16_t*, int32_t, int32_t,
                             hipStream_t) { ++g_launches; return hipErrorUnknown; }
hipError_t launch_combine_split(const float*, const float*, const int4*, const int32_t*,
                                uint16_t*, float*, int32_t, int32_t, hipStream_t) {
  ++g_launches; return hipErrorUnknown;
}
}  // namespace mla

static int g_fail = 0;
#define EXPECT(cond, what)                                        \
  do {                                                            \
    if (!(cond)) {                                                \
      fprintf(stderr, "FAIL %s:%d %s\n", __FILE__, __LINE__, what); \
      ++g_fail;                                                   \
    }                                                             \
  } while (0)

// 256-byte aligned addresses that are never dereferenced (validation and the
// device query come first).
static void* P(uintptr_t k = 1) { return reinterpret_cast<void*>(k << 20); }

static mla_status_t dec(void* q, void* kv, void* bt, void* sl, void* out, void* lse, float scale,
                        int heads, int bs, int splits, int batch, int max_blocks, int nblocks,
                        int kvd, float kvs, void* ws, size_t wsb) {
  return mla_decode(q, kv, static_cast<const int32_t*>(bt), static_cast<const int32_t*>(sl), out,
                    static_cast<float*>(lse), scale, heads, bs, splits, batch, max_blocks, nblocks,
                    kvd, kvs, ws, wsb, nullptr);
}

int main() {
  const int32_t big = INT32_MAX;
  // Workspace-size queries: every argument at and beyond its limits (the size
  // arithmetic must neither overflow nor read out of bounds).
  const int64_t vals[] = {-1, 0, 1, 15, 16, 17, 128, 129, 4096, INT32_MAX / 2, INT32_MAX,
                          (int64_t(1) << 40), INT64_MAX};
  for (int64_t b : vals)
    for (int64_t h : vals)
      for (int64_t n : vals)
        for (int64_t s : {int64_t(-1), int64_t(0), int64_t(1), int64_t(16), int64_t(17)}) {
          (void)mla_get_workspace_size(b, h, n, s, 0);
          (void)mla_get_workspace_size_multi_token(b, h, 16, n, s, 256);
          (void)mla_get_workspace_size_sparse(b, h, n, s, -5);
        }
  EXPECT(mla_get_workspace_size(-1, 16, 100, 0, 0) == 0, "negative batch");
  EXPECT(mla_get_workspace_size(8, 0, 100, 0, 0) == 0, "zero heads");
  EXPECT(mla_get_workspace_size(8, 16, 100, 17, 0) == 0, "17 splits");
  EXPECT(mla_get_workspace_size(8, 16, 100, 0, 0) > 0, "valid size");

  // Decode: invalid arguments are refused before any HIP call.
  const float nan = __builtin_nanf("");
  EXPECT(dec(nullptr, P(), P(), P(), P(), nullptr, 0.07f, 16, 32, 0, 2, 4, 8, 0, 1.f, P(), 1 << 30) ==
             MLA_ERR_INVALID_ARG, "null q");
  EXPECT(dec(P(), P(), P(), P(), P(), nullptr, nan, 16, 32, 0, 2, 4, 8, 0, 1.f, P(), 1 << 30) ==
             MLA_ERR_INVALID_ARG, "nan scale");
  EXPECT(dec(P(), P(), P(), P(), P(), nullptr, 0.07f, 16, 48, 0, 2, 4, 8, 0, 1.f, P(), 1 << 30) ==
             MLA_ERR_INVALID_ARG, "block size 48");
  EXPECT(dec(P(), P(), P(), P(), P(), nullptr, 0.07f, 16, 32, 0, 2, big, 8, 0, 1.f, P(), 1 << 30) ==
             MLA_ERR_INVALID_ARG, "max blocks overflow");
  EXPECT(dec(P(), P(), P(), P(), P(), nullptr, 0.07f, 16, 128, 0, big, big / 128, big, 0, 1.f, P(),
             SIZE_MAX) == MLA_ERR_INVALID_ARG, "cost total overflow");
  EXPECT(dec(P(), P(), P(), P(), P(), nullptr, 0.07f, 16, 32, 0, 2, 4, 8, 0, 1.f, P(), 64) ==
             MLA_ERR_WORKSPACE_TOO_SMALL, "workspace too small");
  EXPECT(dec(P(), P(), P(), P(), P(), nullptr, 0.07f, 16, 32, 0, 2, 4, 8, 1, 0.f, P(), 1 << 30) ==
             MLA_ERR_INVALID_ARG, "fp8 scale 0");
  int dev_count = 0;
  const bool no_dev = hipGetDeviceCount(&dev_count) != hipSuccess || dev_count == 0;
  if (no_dev) {
    EXPECT(dec(P(), P(), P(), P(), P(), nullptr, 0.07f, 16, 32, 0, 2, 4, 8, 0, 1.f, P(), 1 << 30) ==
               MLA_ERR_NO_DEVICE, "no device");
    EXPECT(mla_decode_noalloc(P(), P(), static_cast<const int32_t*>(P()),
                              static_cast<const int32_t*>(P()), P(), nullptr, 0.07f, 128, 16, 64,
                              16, 300, 4, 8, 0, 1.f, nullptr) == MLA_ERR_NO_DEVICE,
           "noalloc without device");
    EXPECT(mla_decode_sparse(P(), P(), static_cast<const int32_t*>(P()),
                             static_cast<const int32_t*>(P()), static_cast<const int32_t*>(P()),
                             2048, P(), nullptr, 0.07f, 16, 32, 0, 2, 4, 8, 0, 1.f, P(),
                             1 << 30, nullptr) == MLA_ERR_NO_DEVICE, "sparse without device");
  }
  EXPECT(mla_decode_multi_token(P(), P(), static_cast<const int32_t*>(P()),
                                static_cast<const int32_t*>(P()), P(), nullptr, 0.07f, 16, 17, 32,
                                0, 2, 4, 8, 0, 1.f, P(), 1 << 30, nullptr) == MLA_ERR_INVALID_ARG,
         "q_len 17");
  EXPECT(mla_decode_sparse(P(), P(), static_cast<const int32_t*>(P()),
                           static_cast<const int32_t*>(P()), nullptr, 16, P(), nullptr, 0.07f, 16,
                           32, 0, 2, 4, 8, 0, 1.f, P(), 1 << 30, nullptr) == MLA_ERR_INVALID_ARG,
         "sparse null indices");
  EXPECT(mla_decode_sparse(P(), P(), static_cast<const int32_t*>(P()),
                           static_cast<const int32_t*>(P()), static_cast<const int32_t*>(P()),
                           MLA_MAX_TOPK + 1, P(), nullptr, 0.07f, 16, 32, 0, 2, 4, 8, 0, 1.f, P(),
                           1 << 30, nullptr) == MLA_ERR_INVALID_ARG, "topk too large");
  EXPECT(mla_decode_profiled(P(), P(), static_cast<const int32_t*>(P()),
                             static_cast<const int32_t*>(P()), P(), nullptr, 0.07f, 16, 1, 32, 0,
                             2, 4, 8, 0, 1.f, P(), 1 << 30, nullptr, nullptr) ==
             MLA_ERR_INVALID_ARG, "profiled without events");
  EXPECT(mla_decode_noalloc(P(), P(), static_cast<const int32_t*>(P()),
                            static_cast<const int32_t*>(P()), P(), nullptr, 0.07f, 0, 1, 32, 0, 2,
                            4, 8, 0, 1.f, nullptr) == MLA_ERR_INVALID_ARG, "noalloc zero heads");
  EXPECT(mla_combine(nullptr, nullptr, nullptr, nullptr, nullptr, -1, 16, nullptr) ==
             MLA_ERR_INVALID_ARG, "combine negative batch");
  EXPECT(mla_combine(static_cast<const float*>(P()), static_cast<const float*>(P()),
                     static_cast<const int32_t*>(P()), P(), nullptr, big, 2048, nullptr) ==
             MLA_ERR_INVALID_ARG, "combine grid overflow");
  EXPECT(mla_gemm_fp8_blockscale(P(), static_cast<const float*>(P()), P(),
                                 static_cast<const float*>(P()), P(), 4, 2112, 7100, nullptr) ==
             MLA_ERR_INVALID_ARG, "gemm k not a multiple of 128");
  EXPECT(mla_quant_fp8_groups(P(), P(), static_cast<float*>(P()), MLA_GEMM_MAX_M + 1, 128,
                              nullptr) == MLA_ERR_INVALID_ARG, "quant m too large");
  EXPECT(mla_absorb_q(P(), P(), nullptr, P(), 4, 16, nullptr) == MLA_ERR_INVALID_ARG,
         "absorb_q null rope");
  EXPECT(mla_absorb_out(P(), P(), P(), 4, 129, nullptr) == MLA_ERR_INVALID_ARG,
         "absorb_out 129 heads");
  for (int st = -8; st <= 2; ++st) EXPECT(mla_status_string(st) != nullptr, "status string");
  EXPECT(mla_abi_version() >= 2, "abi version");
  if (no_dev) EXPECT(g_launches == 0, "a launcher was reached without a device");
  printf("abi harness: %d failures, %d launches\n", g_fail, g_launches);
  return g_fail ? 1 : 0;
}
