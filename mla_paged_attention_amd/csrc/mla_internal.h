// mla_internal.h -- launch interface between the C-ABI layer (mla_api.hip) and
// the gfx950 kernels (mla_kernels.hip). Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

// Bounds-check build (-DMLA_BOUNDS_CHECK=1, libmla_mi355x_checked.so): every
// clamp of a corrupt input is also reported in an error word of the
// workspace. The release build compiles the reports away.
#ifndef MLA_BOUNDS_CHECK
#define MLA_BOUNDS_CHECK 0
#endif

namespace mla {

constexpr int kBoundsBadBlock = 1;   // a block-table entry outside [0, num_blocks)
constexpr int kBoundsBadSeqLen = 2;  // a seq_lens entry outside [0, max_blocks * block_size]
constexpr int kBoundsWordIndex = 8;  // int32 index of the error word in the workspace header

constexpr int kDK = 576;        // key width (512 kv_c + 64 rope)
constexpr int kDV = 512;        // value width (kv_c)
constexpr int kUnit = 16;       // tokens per scheduling unit = MFMA tile rows
constexpr int kHeadTile = 16;   // heads per workgroup (MFMA tile columns)
constexpr int kWaves = 4;       // waves per attention workgroup
constexpr int kThreads = 64 * kWaves;
// Per-request fixed cost of the balanced plan, in 16-token units: what
// starting a piece costs the attention kernel (the first tile's latency, q,
// the epilogue). Chosen by measurement, per kernel: the value that balanced
// the partitions best (v2lite-64 for the 16-head kernel, fullhead for the
// many-head kernel; 1, 4, 6, 8, 12 and 16 were tried).
constexpr int kOverheadUnitsWs = 8;
constexpr int kOverheadUnitsMh = 16;
constexpr int kMinPartUnits = 8;    // smallest partition (128 tokens): fewer, cheaper merges
// Smallest partition when the one-wave plan finds few units in all (batch 1
// and 2 of short requests): 64 tokens. Measured against 8: v2lite-1 call
// 15.4 -> 14.0 us; batch 8 was slower at 4 (20.2 against 19.3 us).
constexpr int kMinPartUnitsFew = 4;
constexpr int kPlanThreads = 1024;
constexpr int kPlanThreadsSmall = 256;
constexpr int kMaxPlanParts = 2048;  // partitions of the automatic plan (work list bound)

// Workspace layout. Offsets are 256-byte aligned. `parts` bounds the
// partitions of the automatic plan (1 in forced-split mode, which needs no
// work list).
struct WorkspaceLayout {
  size_t header;    // int32[64]: [0] partitions, [1] cost units per partition,
                    // [2] split requests, [3] plan mode
  size_t cum;       // int32[batch + 1]: exclusive prefix of per-request costs
  size_t part_ptr;  // int32[parts + 1]: first work item of each partition
  size_t work;      // int32x4[batch + parts]: (request, unit begin, unit end, row or -1)
  size_t split;     // int4[parts]: (request, first partial row, rows, 0) per split request
  size_t part_lse;  // float[rows][num_heads]
  size_t part_out;  // float[rows][num_heads][512]
  size_t sp_rows;   // sparse: int32[batch][sparse_stride] physical row ids
  size_t sp_len;    // sparse: int32[batch] list length per request
  size_t zero_row;  // sparse: 1152 zero bytes
  size_t total;
  int64_t rows;
  int64_t parts;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Row-id entries per request of the sparse prepass: the list rounded up to
// whole units plus one 64-token tile, so every tile's id load stays inside.
inline int64_t sparse_stride(int64_t topk) { return (topk + kUnit - 1) / kUnit * kUnit + 64; }

inline WorkspaceLayout workspace_layout(int64_t batch, int64_t num_heads, int64_t rows,
                                        int64_t parts, int64_t topk = 0) {
  WorkspaceLayout w;
  if (parts < 1) parts = 1;
  size_t off = 0;
  w.header = off;
  off += 256;
  w.cum = off;
  off += align256(size_t(batch + 1) * 4);
  w.part_ptr = off;
  off += align256(size_t(parts + 1) * 4);
  w.work = off;
  off += align256(size_t(batch + parts) * 16);
  w.split = off;
  off += align256(size_t(parts) * 16);
  w.part_lse = off;
  off += align256(size_t(rows) * size_t(num_heads) * 4);
  w.part_out = off;
  off += align256(size_t(rows) * size_t(num_heads) * kDV * 4);
  w.sp_rows = w.sp_len = w.zero_row = off;
  if (topk > 0) {
    w.sp_rows = off;
    off += align256(size_t(batch) * size_t(sparse_stride(topk)) * 4);
    w.sp_len = off;
    off += align256(size_t(batch) * 4);
    w.zero_row = off;
    off += align256(size_t(kDK) * 2);
  }
  w.total = off;
  w.rows = rows;
  w.parts = parts;
  return w;
}

inline int head_tiles(int num_heads) { return (num_heads + kHeadTile - 1) / kHeadTile; }

// The attention kernel a call runs (launch_attention): the 16-head bf16
// kernel for one head tile of a dense bf16 cache, the many-head kernel
// otherwise. Its per-piece cost sets the plan's overhead units.
inline bool uses_16_head_kernel(int rows, int kv_fp8, bool sparse) {
  return !sparse && !kv_fp8 && head_tiles(rows) == 1;
}
inline int plan_overhead_units(int rows, int kv_fp8, bool sparse) {
  return uses_16_head_kernel(rows, kv_fp8, sparse) ? kOverheadUnitsWs : kOverheadUnitsMh;
}

// Workgroups per partition: the many-head kernels (and the E4M3 kernel) put
// four 16-head tiles in one workgroup; the 16-head bf16 kernel uses one.
inline int workgroups_per_partition(int num_heads, int kv_fp8) {
  (void)kv_fp8;
  return (head_tiles(num_heads) + 3) / 4;
}

// Upper bound on balanced partitions for a device with `num_cus` CUs: one
// attention workgroup per CU at a time.
inline int64_t max_partitions(int64_t num_cus, int64_t num_heads, int kv_fp8) {
  int64_t g = num_cus / workgroups_per_partition(int(num_heads), kv_fp8);
  if (g > kMaxPlanParts) g = kMaxPlanParts;
  return g < 8 ? 8 : g;
}

// Query rows: a request's q holds q_len query tokens of `heads` heads each,
// row r = token (r / heads), head (r % heads); the kernels work on
// rows = q_len * heads rows per request, and query token i sees the first
// seq_len - (q_len - 1 - i) cache tokens.
struct AttnArgs {
  const uint16_t* q;         // [B][rows][576] bf16 bits
  const uint8_t* kv;         // [NB][bs][576] bf16 or e4m3 bytes
  const int32_t* block_table;
  const int32_t* seq_lens;
  uint16_t* out;             // [B][rows][512] bf16 bits
  float* lse;                // [B][rows] or null
  float* part_out;
  float* part_lse;
  const int32_t* header;
  const int32_t* part_ptr;   // automatic plan: work items of each partition
  const int4* work;
  float scale_log2;          // logit scale * log2(e)
  float kv_scale;            // fp8 dequantisation scale (1 for bf16)
  int32_t rows;              // q_len * heads
  int32_t heads;             // heads per query token
  int32_t q_len;             // query tokens per request
  int32_t batch;
  int32_t max_blocks;
  int32_t num_blocks;
  int32_t bs_log2;
  int32_t cap_tokens;        // max_blocks * block_size
  int32_t num_splits;        // 0 = automatic plan
  int32_t parts_cap;         // automatic plan: partitions in part_ptr
  int32_t items_cap;         // automatic plan: entries of work
  int32_t rows_cap;          // partial rows in part_out / part_lse
  int32_t head_tiles;        // ceil(rows / 16)
  int32_t head_groups;       // workgroups per partition of the many-head kernel
  // Sparse decode (null otherwise): physical row id (-1: none) of each listed
  // position, sparse_stride ids per request, and a zeroed row to read instead.
  const int32_t* sparse_rows;
  int32_t sparse_stride;
  const uint8_t* zero_row;
  // Automatic plan worked out inside the attention kernel (batches of at
  // most kInlinePlanBatch requests with a contiguous plan): no plan launch;
  // the partition-0 workgroups write split and header for the combine.
  int32_t inline_plan;
  int4* wr_split;
  int32_t* wr_header;
  // Bounds-check build: the error word (null otherwise).
  int32_t* err_word;
  // Per-request fixed cost of the automatic plan, in units (plan_overhead_units).
  int32_t plan_ovh;
};

constexpr int kInlinePlanBatch = 64;  // one request per lane of a wave
// inline_plan modes: none (plan kernel, or forced splits), the contiguous
// plan worked out by one wave (at most kInlinePlanBatch requests), or the
// snake plan worked out by every workgroup (at most kInlineSnakeBatch).
constexpr int kInlineNone = 0;
constexpr int kInlineContiguous = 1;
constexpr int kInlineSnake = 2;
constexpr int kInlineContiguousWide = 3;  // the contiguous plan, worked out by every workgroup
constexpr int kInlineSnakeBatch = 1024;
constexpr int kInlineContigBatch = 4096;

// Split plan (one workgroup) for the automatic plan when the attention kernel
// does not work it out itself: fills header, cum, part_ptr, work and split.
hipError_t launch_plan(const int32_t* seq_lens, int32_t batch, int32_t cap_tokens,
                       int32_t max_parts, int32_t ovh, const WorkspaceLayout& w, void* workspace,
                       hipStream_t stream);

// kv_fp8: 0 = bf16 cache, 1 = E4M3 cache. `parts_launched` is a multiple of 8.
hipError_t launch_attention(const AttnArgs& args, int kv_fp8, int32_t parts_launched,
                            hipStream_t stream);

hipError_t launch_combine(const float* part_out, const float* part_lse,
                          const int32_t* row_ptr, uint16_t* out, float* lse, int32_t batch,
                          int32_t num_heads, int zero_empty, int32_t uniform,
                          hipStream_t stream);

// Sparse decode prepass: rows[b * stride + k] = physical row of listed
// position k of request b, or -1; eff_len[b] = topk; zero_row = 1152 zero bytes.
hipError_t launch_sparse_rows(const int32_t* indices, int32_t topk, const int32_t* block_table,
                              const int32_t* seq_lens, int32_t batch, int32_t max_blocks,
                              int32_t num_blocks, int32_t bs_log2, int32_t cap_tokens,
                              int32_t stride, int32_t* rows, int32_t* eff_len, void* zero_row,
                              int32_t* err_word, hipStream_t stream);

// Bounds-check build: zeroes the error word at the start of a call.
hipError_t launch_clear_word(int32_t* word, hipStream_t stream);

// Block-scaled E4M3 projection (gemm_fp8.hip): bf16 -> E4M3 codes with one
// scale per token and 128-wide group, and c[m][n] = A[m][k] B[n][k]^T with
// per-group activation and per-128x128-block weight scales.
hipError_t launch_quant_fp8_groups(const uint16_t* x, uint8_t* q, float* scale, int32_t m,
                                   int32_t k, hipStream_t stream);
hipError_t launch_gemm_fp8(const uint8_t* a, const float* a_scale, const uint8_t* b,
                           const float* b_scale, uint16_t* c, int32_t m, int32_t n, int32_t k,
                           hipStream_t stream);

// Per-head absorption products (absorb.hip): q = [q_nope . W_UK[h], q_rope]
// and o[v] = sum_c o_latent[c] W_UV[h][v][c], bf16 with fp32 accumulation.
hipError_t launch_absorb_q(const uint16_t* q_nope, const uint16_t* w_uk, const uint16_t* q_rope,
                           uint16_t* q, int32_t batch, int32_t heads, hipStream_t stream);
hipError_t launch_absorb_out(const uint16_t* o_latent, const uint16_t* w_uv, uint16_t* o,
                             int32_t batch, int32_t heads, hipStream_t stream);

// Combine of the automatic plan: only the requests listed in `split`
// (header[2] of them, at most `max_split`).
hipError_t launch_combine_split(const float* part_out, const float* part_lse,
                                const int4* split,
                                const int32_t* header, uint16_t* out, float* lse,
                                int32_t max_split, int32_t num_heads, hipStream_t stream);

}  // namespace mla
