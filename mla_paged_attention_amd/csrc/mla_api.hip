// mla_api.hip -- the C ABI declared in include/mla.h: argument validation,
// workspace sizing, device checks and kernel dispatch. No allocation, no
// host synchronisation, no exceptions across the boundary.
#include <hip/hip_runtime.h>

#include <algorithm>

#include <math.h>
#include <mutex>
#include <string.h>

#include "../../include/mla.h"
#include "mla_internal.h"

namespace {

using mla::WorkspaceLayout;

constexpr int64_t kDefaultCus = 256;  // MI355X
constexpr int kMaxDevices = 64;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int bs_log2_of(int32_t bs) {
  switch (bs) {
    case 16: return 4;
    case 32: return 5;
    case 64: return 6;
    case 128: return 7;
    default: return -1;
  }
}

// Partial rows the automatic plan may need with at most `parts` partitions.
// Contiguous plan: every cut inside a request adds one piece, and a split
// request of p pieces holds p rows, so at most 2 * (parts - 1) rows. Snake
// plan: only requests costing more than the per-partition target P are cut,
// into ceil(cost / P) <= 2 cost / P pieces, so at most 2 * parts rows.
// Never more than batch * min(parts, units of the longest request).
int64_t auto_rows(int64_t batch, int64_t parts, int64_t max_seq_len) {
  if (parts <= 1 || batch <= 0) return 0;
  int64_t units = (max_seq_len + mla::kUnit - 1) / mla::kUnit;
  if (units < 1) units = 1;
  int64_t per_req = parts < units ? parts : units;
  if (per_req <= 1) return 0;
  int64_t a = 2 * parts, b = batch * per_req;
  return a < b ? a : b;
}

int64_t forced_rows(int64_t batch, int64_t splits) { return splits > 1 ? batch * splits : 0; }

struct DeviceInfo {
  bool valid = false;
  bool gfx950 = false;
  int cus = 0;
};

std::mutex g_dev_mutex;
DeviceInfo g_dev[kMaxDevices];  // immutable device properties, filled once per device

mla_status_t query_device(DeviceInfo* info, int* dev_index = nullptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MLA_ERR_NO_DEVICE;
  if (dev_index) *dev_index = dev;
  if (dev >= kMaxDevices) return MLA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_dev_mutex);
  if (!g_dev[dev].valid) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MLA_ERR_NO_DEVICE;
    DeviceInfo d;
    d.valid = true;
    d.gfx950 = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    d.cus = prop.multiProcessorCount;
    g_dev[dev] = d;
  }
  *info = g_dev[dev];
  return MLA_OK;
}

// Workspace bytes of a dense decode call (one or several query tokens).
size_t dense_workspace_need(int64_t batch, int64_t rows, int64_t max_seq_len,
                            int64_t num_splits, int64_t num_cus);

}  // namespace

// Device scratch of mla_decode_noalloc: the workspace of calls that cannot
// allocate. Every GPU the library runs on holds its own copy of this array
// (set up by the code object's loader) until the process ends. In host code
// the name is only a stand-in: its device address comes from
// hipGetSymbolAddress, once per device.
static __device__ __align__(256) uint8_t scratch[MLA_NOALLOC_SCRATCH_BYTES];

namespace {

void* g_scratch[kMaxDevices];  // device address of `scratch` per device (g_dev_mutex)

// Address of `scratch` on device `dev`, which must be the current device.
mla_status_t scratch_address(int dev, void** ptr) {
  std::lock_guard<std::mutex> lock(g_dev_mutex);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MLA_ERR_HIP;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return MLA_OK;
}

struct DecodeArgs {
  const void* q;
  const void* kv_cache;
  const int32_t* block_table;
  const int32_t* seq_lens;
  void* out;
  float* lse;
  float scale;
  int32_t num_heads, q_len, block_size, num_splits, batch, max_blocks, num_blocks, kv_dtype;
  float kv_scale;
  void* workspace;
  size_t workspace_bytes;
  hipStream_t stream;
  const int32_t* indices = nullptr;  // sparse decode: [batch][topk] token positions
  int32_t topk = 0;                  // > 0: sparse decode
  bool scratch = false;              // workspace = the library's device scratch array

  int32_t rows() const { return num_heads * q_len; }  // query rows per request
};

mla_status_t validate_decode(const DecodeArgs& a) {
  if (a.batch < 0) return MLA_ERR_INVALID_ARG;
  if (a.num_heads < 1 || a.num_heads > MLA_MAX_HEADS) return MLA_ERR_INVALID_ARG;
  if (a.q_len < 1 || a.q_len > MLA_MAX_QUERY_LEN) return MLA_ERR_INVALID_ARG;
  if (bs_log2_of(a.block_size) < 0) return MLA_ERR_INVALID_ARG;
  if (a.num_splits < 0 || a.num_splits > MLA_MAX_FORCED_SPLITS) return MLA_ERR_INVALID_ARG;
  if (a.max_blocks < 1 || a.num_blocks < 1) return MLA_ERR_INVALID_ARG;
  if (int64_t(a.max_blocks) * a.block_size > INT32_MAX / 2) return MLA_ERR_INVALID_ARG;
  if (int64_t(a.num_blocks) * a.block_size * MLA_HEAD_DIM_K > (int64_t(1) << 46))
    return MLA_ERR_INVALID_ARG;
  if (!isfinite(a.scale)) return MLA_ERR_INVALID_ARG;
  if (a.kv_dtype == MLA_KV_BF16) {
    if (a.kv_scale != 1.0f) return MLA_ERR_INVALID_ARG;
  } else if (a.kv_dtype == MLA_KV_FP8_E4M3) {
    if (!(isfinite(a.kv_scale) && a.kv_scale > 0.f)) return MLA_ERR_INVALID_ARG;
  } else {
    return MLA_ERR_INVALID_ARG;
  }
  if (a.topk < 0 || a.topk > MLA_MAX_TOPK) return MLA_ERR_INVALID_ARG;
  if (a.topk > 0) {
    if (a.q_len != 1) return MLA_ERR_INVALID_ARG;
    // Row ids are int32; the prepass indexes batch * stride entries.
    if (int64_t(a.num_blocks) * a.block_size > INT32_MAX) return MLA_ERR_INVALID_ARG;
    if (int64_t(a.batch) * mla::sparse_stride(a.topk) > INT32_MAX) return MLA_ERR_INVALID_ARG;
  }
  if (a.batch == 0) return MLA_OK;
  {
    // The split plan sums per-request costs (overhead + 16-token units, at
    // most the cap) in int32: the largest total, plus a partition of slack,
    // must fit.
    const int64_t cap_tokens = a.topk > 0 ? a.topk : int64_t(a.max_blocks) * a.block_size;
    const int64_t max_cost = std::max(mla::kOverheadUnitsWs, mla::kOverheadUnitsMh) +
                             (cap_tokens + mla::kUnit - 1) / mla::kUnit;
    if (int64_t(a.batch) * max_cost > INT32_MAX / 2) return MLA_ERR_INVALID_ARG;
  }
  if (!a.q || !a.kv_cache || !a.block_table || !a.seq_lens || !a.out)
    return MLA_ERR_INVALID_ARG;
  if (!a.scratch && !a.workspace) return MLA_ERR_INVALID_ARG;
  if (a.topk > 0 && (!a.indices || !aligned(a.indices, 4))) return MLA_ERR_INVALID_ARG;
  if (!aligned(a.q, 16) || !aligned(a.kv_cache, 16) || !aligned(a.out, 16) ||
      !aligned(a.block_table, 4) || !aligned(a.seq_lens, 4) ||
      (!a.scratch && !aligned(a.workspace, 256)))
    return MLA_ERR_INVALID_ARG;
  if (a.lse && !aligned(a.lse, 4)) return MLA_ERR_INVALID_ARG;
  // The scratch array's size is checked against the whole need once the
  // device (its CU count) is known.
  if (a.scratch) {
    if (a.num_splits > 0) {
      const int64_t tiles = mla::head_tiles(a.rows());
      if (int64_t(a.batch) * a.num_splits * tiles > INT32_MAX ||
          int64_t(a.batch) * tiles * (MLA_HEAD_DIM_V / 64) > INT32_MAX)
        return MLA_ERR_INVALID_ARG;
    }
    return MLA_OK;
  }
  // Metadata alone must fit whatever the mode.
  if (a.workspace_bytes < mla::workspace_layout(a.batch, a.rows(), 0, 1, a.topk).total)
    return MLA_ERR_WORKSPACE_TOO_SMALL;
  if (a.num_splits > 0) {
    // One workgroup per (request, split, 16-row tile) and per (request, tile,
    // 64-feature chunk) of the combine: grids stay within 2^31 - 1.
    const int64_t tiles = mla::head_tiles(a.rows());
    if (int64_t(a.batch) * a.num_splits * tiles > INT32_MAX ||
        int64_t(a.batch) * tiles * (MLA_HEAD_DIM_V / 64) > INT32_MAX)
      return MLA_ERR_INVALID_ARG;
    WorkspaceLayout w =
        mla::workspace_layout(a.batch, a.rows(), forced_rows(a.batch, a.num_splits), 1, a.topk);
    if (a.workspace_bytes < w.total) return MLA_ERR_WORKSPACE_TOO_SMALL;
  }
  return MLA_OK;
}

mla_status_t run_decode(const DecodeArgs& call, void* const* events) {
  mla_status_t st = validate_decode(call);
  if (st != MLA_OK) return st;
  if (events && (!events[0] || !events[1] || !events[2] || !events[3]))
    return MLA_ERR_INVALID_ARG;
  DeviceInfo dev;
  int dev_index = -1;
  st = query_device(&dev, &dev_index);
  if (st != MLA_OK) return st;
  if (!dev.gfx950) return MLA_ERR_UNSUPPORTED;
  DecodeArgs a = call;
  if (a.scratch) {
    // The whole workspace this call needs must fit the fixed array; nothing
    // is shrunk to fit, so the call computes exactly what mla_decode would
    // with a workspace of mla_get_workspace_size bytes.
    const size_t need = dense_workspace_need(a.batch, a.rows(),
                                             int64_t(a.max_blocks) * a.block_size, a.num_splits,
                                             dev.cus);
    if (need == 0 || need > MLA_NOALLOC_SCRATCH_BYTES) return MLA_ERR_WORKSPACE_TOO_SMALL;
    st = scratch_address(dev_index, &a.workspace);
    if (st != MLA_OK) return st;
    a.workspace_bytes = MLA_NOALLOC_SCRATCH_BYTES;
  }
  if (a.batch == 0) return MLA_OK;

  // Tokens per request the kernels walk: the cache (dense) or the list (sparse).
  const int64_t cache_cap = int64_t(a.max_blocks) * a.block_size;
  const bool sparse = a.topk > 0;
  const int64_t cap = sparse ? a.topk : cache_cap;
  WorkspaceLayout w;
  int64_t max_parts = 0;
  const int32_t rows = a.rows();
  if (a.num_splits > 0) {
    w = mla::workspace_layout(a.batch, rows, forced_rows(a.batch, a.num_splits), 1, a.topk);
  } else {
    // Largest partition count whose plan and partial rows fit the workspace.
    max_parts = mla::max_partitions(dev.cus, rows, a.kv_dtype == MLA_KV_FP8_E4M3);
    auto layout = [&](int64_t parts) {
      return mla::workspace_layout(a.batch, rows, auto_rows(a.batch, parts, cap), parts, a.topk);
    };
    while (max_parts > 1 && layout(max_parts).total > a.workspace_bytes)
      max_parts = max_parts * 3 / 4;
    w = layout(max_parts);
    if (w.total > a.workspace_bytes) return MLA_ERR_WORKSPACE_TOO_SMALL;
  }
  const int32_t plan_ovh =
      mla::plan_overhead_units(rows, a.kv_dtype == MLA_KV_FP8_E4M3 ? 1 : 0, sparse);
  uint8_t* ws = static_cast<uint8_t*>(a.workspace);
  int32_t* header = reinterpret_cast<int32_t*>(ws + w.header);
  int32_t* part_ptr = reinterpret_cast<int32_t*>(ws + w.part_ptr);
  int4* work = reinterpret_cast<int4*>(ws + w.work);
  int4* split = reinterpret_cast<int4*>(ws + w.split);
  float* part_lse = reinterpret_cast<float*>(ws + w.part_lse);
  float* part_out = reinterpret_cast<float*>(ws + w.part_out);

  hipStream_t s = a.stream;
  auto rec = [&](int i) -> bool {
    return !events || hipEventRecord(static_cast<hipEvent_t>(events[i]), s) == hipSuccess;
  };

  if (!rec(0)) return MLA_ERR_HIP;
  // Bounds-check build: this call's error word, zeroed first.
  int32_t* err_word = nullptr;
  if (MLA_BOUNDS_CHECK) {
    err_word = header + mla::kBoundsWordIndex;
    if (mla::launch_clear_word(err_word, s) != hipSuccess) return MLA_ERR_HIP;
  }
  // The plan sees every sparse request as topk tokens long.
  const int32_t* lens = a.seq_lens;
  if (sparse) {
    int32_t* sp_len = reinterpret_cast<int32_t*>(ws + w.sp_len);
    if (mla::launch_sparse_rows(a.indices, a.topk, a.block_table, a.seq_lens, a.batch,
                                a.max_blocks, a.num_blocks, bs_log2_of(a.block_size),
                                int32_t(cache_cap), int32_t(mla::sparse_stride(a.topk)),
                                reinterpret_cast<int32_t*>(ws + w.sp_rows), sp_len,
                                ws + w.zero_row, err_word, s) != hipSuccess)
      return MLA_ERR_HIP;
    lens = sp_len;
  }
  // The attention kernel works the automatic plan out itself (one launch
  // fewer): the contiguous plan by one wave for small batches or by every
  // workgroup up to kInlineContigBatch requests, and the snake plan (at
  // least two requests per partition) up to kInlineSnakeBatch requests whose
  // pieces fill at most 64 rounds of the deal. Forced splits need no plan:
  // piece k of request b is partition b * S + k, its partial row too.
  int inline_plan = mla::kInlineNone;
  if (a.num_splits == 0) {
    if (a.batch <= mla::kInlinePlanBatch && a.batch < 2 * max_parts)
      inline_plan = mla::kInlineContiguous;
    else if (a.batch >= 2 * max_parts && a.batch <= mla::kInlineSnakeBatch &&
             a.batch + max_parts <= 64 * max_parts)
      inline_plan = mla::kInlineSnake;
    else if (a.batch < 2 * max_parts && a.batch <= mla::kInlineContigBatch)
      inline_plan = mla::kInlineContiguousWide;
  }
  if (inline_plan == mla::kInlineNone && a.num_splits == 0 &&
      mla::launch_plan(lens, a.batch, int32_t(cap), int32_t(max_parts), plan_ovh, w, a.workspace,
                       s) !=
          hipSuccess)
    return MLA_ERR_HIP;
  if (!rec(1)) return MLA_ERR_HIP;

  mla::AttnArgs args;
  args.q = static_cast<const uint16_t*>(a.q);
  args.kv = static_cast<const uint8_t*>(a.kv_cache);
  args.block_table = a.block_table;
  args.seq_lens = lens;
  args.out = static_cast<uint16_t*>(a.out);
  args.lse = a.lse;
  args.part_out = part_out;
  args.part_lse = part_lse;
  args.header = header;
  args.part_ptr = part_ptr;
  args.work = work;
  args.scale_log2 = a.scale * 1.4426950408889634f;
  args.kv_scale = a.kv_scale;
  args.rows = rows;
  args.heads = a.num_heads;
  args.q_len = a.q_len;
  args.batch = a.batch;
  args.max_blocks = a.max_blocks;
  args.num_blocks = a.num_blocks;
  args.bs_log2 = bs_log2_of(a.block_size);
  args.cap_tokens = int32_t(cap);
  args.num_splits = a.num_splits;
  args.parts_cap = int32_t(max_parts);
  args.items_cap = int32_t(a.batch + max_parts);
  args.rows_cap = int32_t(w.rows);
  args.head_tiles = mla::head_tiles(rows);
  args.head_groups = (args.head_tiles + 3) / 4;
  args.sparse_rows = sparse ? reinterpret_cast<const int32_t*>(ws + w.sp_rows) : nullptr;
  args.sparse_stride = sparse ? int32_t(mla::sparse_stride(a.topk)) : 0;
  args.zero_row = sparse ? ws + w.zero_row : nullptr;
  args.inline_plan = inline_plan;
  args.wr_split = split;
  args.wr_header = header;
  args.err_word = err_word;
  args.plan_ovh = plan_ovh;
  int64_t parts = a.num_splits > 0 ? int64_t(a.batch) * a.num_splits : max_parts;
  int64_t parts_launched = (parts + 7) / 8 * 8;
  if (parts_launched * args.head_tiles > INT32_MAX) return MLA_ERR_INVALID_ARG;
  hipError_t e = mla::launch_attention(args, a.kv_dtype == MLA_KV_FP8_E4M3, int32_t(parts_launched), s);
  if (e == hipErrorNotSupported) return MLA_ERR_UNSUPPORTED;
  if (e != hipSuccess) return MLA_ERR_HIP;
  if (!rec(2)) return MLA_ERR_HIP;

  if (a.num_splits > 1) {
    if (mla::launch_combine(part_out, part_lse, nullptr, static_cast<uint16_t*>(a.out), a.lse,
                            a.batch, rows, 0, a.num_splits, s) != hipSuccess)
      return MLA_ERR_HIP;
  } else if (a.num_splits == 0 && max_parts > 1 && w.rows > 0) {
    // Split requests are fewer than the partitions (each is costlier than
    // a partition's share, or straddles one of the parts - 1 cuts).
    const int64_t max_split = a.batch < max_parts ? a.batch : max_parts;
    if (mla::launch_combine_split(part_out, part_lse, split, header,
                                  static_cast<uint16_t*>(a.out), a.lse, int32_t(max_split),
                                  rows, s) != hipSuccess)
      return MLA_ERR_HIP;
  }
  if (!rec(3)) return MLA_ERR_HIP;
  return MLA_OK;
}

size_t dense_workspace_need(int64_t batch, int64_t rows, int64_t max_seq_len,
                            int64_t num_splits, int64_t num_cus) {
  if (num_cus <= 0) num_cus = kDefaultCus;
  if (num_splits > 0)
    return mla::workspace_layout(batch, rows, forced_rows(batch, num_splits), 1).total;
  const int64_t parts = mla::max_partitions(num_cus, rows, 0);
  return mla::workspace_layout(batch, rows, auto_rows(batch, parts, max_seq_len), parts).total;
}

}  // namespace

extern "C" {

size_t mla_get_workspace_size_multi_token(int64_t batch, int64_t num_heads, int64_t q_len,
                                          int64_t max_seq_len, int64_t num_splits,
                                          int64_t num_cus) {
  if (batch < 0 || batch > INT32_MAX / 2) return 0;
  if (num_heads < 1 || num_heads > MLA_MAX_HEADS) return 0;
  if (q_len < 1 || q_len > MLA_MAX_QUERY_LEN) return 0;
  if (max_seq_len < 0 || max_seq_len > INT32_MAX / 2) return 0;
  if (num_splits < 0 || num_splits > MLA_MAX_FORCED_SPLITS) return 0;
  return dense_workspace_need(batch, num_heads * q_len, max_seq_len, num_splits, num_cus);
}

size_t mla_get_workspace_size(int64_t batch, int64_t num_heads, int64_t max_seq_len,
                              int64_t num_splits, int64_t num_cus) {
  return mla_get_workspace_size_multi_token(batch, num_heads, 1, max_seq_len, num_splits,
                                            num_cus);
}

mla_status_t mla_decode_multi_token(const void* q, const void* kv_cache,
                                    const int32_t* block_table, const int32_t* seq_lens,
                                    void* out, float* lse, float scale, int32_t num_heads,
                                    int32_t q_len, int32_t block_size, int32_t num_splits,
                                    int32_t batch, int32_t max_blocks_per_seq,
                                    int32_t num_blocks, int32_t kv_dtype, float kv_scale,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  DecodeArgs a{q, kv_cache, block_table, seq_lens, out, lse, scale, num_heads, q_len,
               block_size, num_splits, batch, max_blocks_per_seq, num_blocks, kv_dtype,
               kv_scale, workspace, workspace_bytes, static_cast<hipStream_t>(stream)};
  return run_decode(a, nullptr);
}

mla_status_t mla_decode(const void* q, const void* kv_cache, const int32_t* block_table,
                        const int32_t* seq_lens, void* out, float* lse, float scale,
                        int32_t num_heads, int32_t block_size, int32_t num_splits,
                        int32_t batch, int32_t max_blocks_per_seq, int32_t num_blocks,
                        int32_t kv_dtype, float kv_scale, void* workspace,
                        size_t workspace_bytes, void* stream) {
  return mla_decode_multi_token(q, kv_cache, block_table, seq_lens, out, lse, scale, num_heads,
                                1, block_size, num_splits, batch, max_blocks_per_seq,
                                num_blocks, kv_dtype, kv_scale, workspace, workspace_bytes,
                                stream);
}

mla_status_t mla_decode_noalloc(const void* q, const void* kv_cache, const int32_t* block_table,
                                const int32_t* seq_lens, void* out, float* lse, float scale,
                                int32_t num_heads, int32_t q_len, int32_t block_size,
                                int32_t num_splits, int32_t batch, int32_t max_blocks_per_seq,
                                int32_t num_blocks, int32_t kv_dtype, float kv_scale,
                                void* stream) {
  DecodeArgs a{q, kv_cache, block_table, seq_lens, out, lse, scale, num_heads, q_len,
               block_size, num_splits, batch, max_blocks_per_seq, num_blocks, kv_dtype,
               kv_scale, nullptr, 0, static_cast<hipStream_t>(stream)};
  a.scratch = true;
  return run_decode(a, nullptr);
}

mla_status_t mla_decode_profiled(const void* q, const void* kv_cache,
                                 const int32_t* block_table, const int32_t* seq_lens,
                                 void* out, float* lse, float scale, int32_t num_heads,
                                 int32_t q_len, int32_t block_size, int32_t num_splits,
                                 int32_t batch, int32_t max_blocks_per_seq, int32_t num_blocks,
                                 int32_t kv_dtype, float kv_scale, void* workspace,
                                 size_t workspace_bytes, void* stream, void* const* events) {
  if (!events) return MLA_ERR_INVALID_ARG;
  DecodeArgs a{q, kv_cache, block_table, seq_lens, out, lse, scale, num_heads, q_len,
               block_size, num_splits, batch, max_blocks_per_seq, num_blocks, kv_dtype,
               kv_scale, workspace, workspace_bytes, static_cast<hipStream_t>(stream)};
  return run_decode(a, events);
}

size_t mla_get_workspace_size_sparse(int64_t batch, int64_t num_heads, int64_t topk,
                                     int64_t num_splits, int64_t num_cus) {
  if (batch < 0 || batch > INT32_MAX / 2) return 0;
  if (num_heads < 1 || num_heads > MLA_MAX_HEADS) return 0;
  if (topk < 1 || topk > MLA_MAX_TOPK) return 0;
  if (num_splits < 0 || num_splits > MLA_MAX_FORCED_SPLITS) return 0;
  if (num_cus <= 0) num_cus = kDefaultCus;
  if (num_splits > 0)
    return mla::workspace_layout(batch, num_heads, forced_rows(batch, num_splits), 1, topk).total;
  const int64_t parts = mla::max_partitions(num_cus, num_heads, 0);
  return mla::workspace_layout(batch, num_heads, auto_rows(batch, parts, topk), parts, topk)
      .total;
}

mla_status_t mla_decode_sparse(const void* q, const void* kv_cache, const int32_t* block_table,
                               const int32_t* seq_lens, const int32_t* indices, int32_t topk,
                               void* out, float* lse, float scale, int32_t num_heads,
                               int32_t block_size, int32_t num_splits, int32_t batch,
                               int32_t max_blocks_per_seq, int32_t num_blocks, int32_t kv_dtype,
                               float kv_scale, void* workspace, size_t workspace_bytes,
                               void* stream) {
  if (topk < 1) return MLA_ERR_INVALID_ARG;
  DecodeArgs a{q, kv_cache, block_table, seq_lens, out, lse, scale, num_heads, 1, block_size,
               num_splits, batch, max_blocks_per_seq, num_blocks, kv_dtype, kv_scale,
               workspace, workspace_bytes, static_cast<hipStream_t>(stream), indices, topk};
  return run_decode(a, nullptr);
}

mla_status_t mla_decode_sparse_profiled(const void* q, const void* kv_cache,
                                        const int32_t* block_table, const int32_t* seq_lens,
                                        const int32_t* indices, int32_t topk, void* out,
                                        float* lse, float scale, int32_t num_heads,
                                        int32_t block_size, int32_t num_splits, int32_t batch,
                                        int32_t max_blocks_per_seq, int32_t num_blocks,
                                        int32_t kv_dtype, float kv_scale, void* workspace,
                                        size_t workspace_bytes, void* stream,
                                        void* const* events) {
  if (topk < 1 || !events) return MLA_ERR_INVALID_ARG;
  DecodeArgs a{q, kv_cache, block_table, seq_lens, out, lse, scale, num_heads, 1, block_size,
               num_splits, batch, max_blocks_per_seq, num_blocks, kv_dtype, kv_scale,
               workspace, workspace_bytes, static_cast<hipStream_t>(stream), indices, topk};
  return run_decode(a, events);
}

mla_status_t mla_combine(const float* partial_out, const float* partial_lse,
                         const int32_t* split_indptr, void* out, float* lse, int32_t batch,
                         int32_t num_heads, void* stream) {
  if (batch < 0 || num_heads < 1 || num_heads > MLA_MAX_HEADS * MLA_MAX_QUERY_LEN)
    return MLA_ERR_INVALID_ARG;
  if (int64_t(batch) * mla::head_tiles(num_heads) * (MLA_HEAD_DIM_V / 64) > INT32_MAX)
    return MLA_ERR_INVALID_ARG;
  if (batch > 0) {
    if (!partial_out || !partial_lse || !split_indptr || !out) return MLA_ERR_INVALID_ARG;
    if (!aligned(partial_out, 16) || !aligned(partial_lse, 4) || !aligned(split_indptr, 4) ||
        !aligned(out, 16) || (lse && !aligned(lse, 4)))
      return MLA_ERR_INVALID_ARG;
  }
  DeviceInfo dev;
  mla_status_t st = query_device(&dev);
  if (st != MLA_OK) return st;
  if (!dev.gfx950) return MLA_ERR_UNSUPPORTED;
  if (batch == 0) return MLA_OK;
  if (mla::launch_combine(partial_out, partial_lse, split_indptr, static_cast<uint16_t*>(out),
                          lse, batch, num_heads, 1, 0, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return MLA_ERR_HIP;
  return MLA_OK;
}

mla_status_t mla_quant_fp8_groups(const void* x, void* x_fp8, float* x_scale, int32_t m,
                                  int32_t k, void* stream) {
  if (m < 0 || m > MLA_GEMM_MAX_M || k < MLA_FP8_GROUP || k % MLA_FP8_GROUP ||
      k > MLA_GEMM_MAX_K)
    return MLA_ERR_INVALID_ARG;
  if (m > 0 && (!x || !x_fp8 || !x_scale || !aligned(x, 4) || !aligned(x_fp8, 2) ||
                !aligned(x_scale, 4)))
    return MLA_ERR_INVALID_ARG;
  DeviceInfo dev;
  mla_status_t st = query_device(&dev);
  if (st != MLA_OK) return st;
  if (!dev.gfx950) return MLA_ERR_UNSUPPORTED;
  if (m == 0) return MLA_OK;
  if (mla::launch_quant_fp8_groups(static_cast<const uint16_t*>(x), static_cast<uint8_t*>(x_fp8),
                                   x_scale, m, k, static_cast<hipStream_t>(stream)) != hipSuccess)
    return MLA_ERR_HIP;
  return MLA_OK;
}

mla_status_t mla_gemm_fp8_blockscale(const void* a, const float* a_scale, const void* b,
                                     const float* b_scale, void* c, int32_t m, int32_t n,
                                     int32_t k, void* stream) {
  if (m < 0 || m > MLA_GEMM_MAX_M || n < 16 || n % 16 || n > MLA_GEMM_MAX_N ||
      k < MLA_FP8_GROUP || k % MLA_FP8_GROUP || k > MLA_GEMM_MAX_K)
    return MLA_ERR_INVALID_ARG;
  if (m > 0 && (!a || !a_scale || !b || !b_scale || !c || !aligned(a, 16) || !aligned(b, 16) ||
                !aligned(c, 8) || !aligned(a_scale, 4) || !aligned(b_scale, 4)))
    return MLA_ERR_INVALID_ARG;
  DeviceInfo dev;
  mla_status_t st = query_device(&dev);
  if (st != MLA_OK) return st;
  if (!dev.gfx950) return MLA_ERR_UNSUPPORTED;
  if (m == 0) return MLA_OK;
  if (mla::launch_gemm_fp8(static_cast<const uint8_t*>(a), a_scale,
                           static_cast<const uint8_t*>(b), b_scale, static_cast<uint16_t*>(c), m,
                           n, k, static_cast<hipStream_t>(stream)) != hipSuccess)
    return MLA_ERR_HIP;
  return MLA_OK;
}

namespace {
mla_status_t absorb_checks(const void* x, const void* w, const void* out, int32_t batch,
                           int32_t heads) {
  if (batch < 0 || batch > MLA_GEMM_MAX_M || heads < 1 || heads > MLA_MAX_HEADS)
    return MLA_ERR_INVALID_ARG;
  if (batch > 0 && (!x || !w || !out || !aligned(x, 16) || !aligned(w, 16) || !aligned(out, 16)))
    return MLA_ERR_INVALID_ARG;
  DeviceInfo dev;
  mla_status_t st = query_device(&dev);
  if (st != MLA_OK) return st;
  return dev.gfx950 ? MLA_OK : MLA_ERR_UNSUPPORTED;
}
}  // namespace

mla_status_t mla_absorb_q(const void* q_nope, const void* w_uk, const void* q_rope, void* q,
                          int32_t batch, int32_t num_heads, void* stream) {
  if (batch > 0 && (!q_rope || !aligned(q_rope, 16))) return MLA_ERR_INVALID_ARG;
  mla_status_t st = absorb_checks(q_nope, w_uk, q, batch, num_heads);
  if (st != MLA_OK || batch == 0) return st;
  if (mla::launch_absorb_q(static_cast<const uint16_t*>(q_nope), static_cast<const uint16_t*>(w_uk),
                           static_cast<const uint16_t*>(q_rope), static_cast<uint16_t*>(q), batch,
                           num_heads, static_cast<hipStream_t>(stream)) != hipSuccess)
    return MLA_ERR_HIP;
  return MLA_OK;
}

mla_status_t mla_absorb_out(const void* o_latent, const void* w_uv, void* o, int32_t batch,
                            int32_t num_heads, void* stream) {
  mla_status_t st = absorb_checks(o_latent, w_uv, o, batch, num_heads);
  if (st != MLA_OK || batch == 0) return st;
  if (mla::launch_absorb_out(static_cast<const uint16_t*>(o_latent),
                             static_cast<const uint16_t*>(w_uv), static_cast<uint16_t*>(o), batch,
                             num_heads, static_cast<hipStream_t>(stream)) != hipSuccess)
    return MLA_ERR_HIP;
  return MLA_OK;
}

const char* mla_status_string(int32_t status) {
  switch (status) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED";
    case MLA_ERR_WORKSPACE_TOO_SMALL: return "MLA_ERR_WORKSPACE_TOO_SMALL";
    case MLA_ERR_NO_DEVICE: return "MLA_ERR_NO_DEVICE";
    case MLA_ERR_HIP: return "MLA_ERR_HIP";
    default: return "MLA_ERR_UNKNOWN";
  }
}

int32_t mla_abi_version(void) { return 2; }

}  // extern "C"
