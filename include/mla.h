/*
 * mla.h -- C ABI of libmla_mi355x.so: absorbed Multi-head Latent Attention
 * (MLA) decode over a paged latent KV cache, for AMD Instinct MI355X (gfx950).
 *
 * What is computed. One query token per request (PR #20769 "SM100 Cutlass
 * MLA decode with unrestricted num_heads (< 128) for DeepSeek TP", review of
 * ensure_size: max_query_len = 1, batch_size = num_decodes). Every cached
 * token is a 576-wide latent row: columns 0..511 are kv_c, 512..575 the rope
 * part. For request b with N = seq_lens[b] tokens and head h:
 *
 *     x_t      = scale * <q[b][h][0:576], K_t[0:576]>         t < N
 *     out[b][h] = sum_t exp(x_t) K_t[0:512] / sum_t exp(x_t)   (V = kv_c)
 *     lse[b][h] = ln(sum_t exp(x_t))                           (natural log)
 *
 * where K_t is row (t mod block_size) of physical block
 * block_table[b][t / block_size] (paged cache: PR #21078 "Flashinfer MLA
 * (trtllm-gen) decode kernel integration", E2E command --block-size 32).
 * The KV length is split across workgroups and the normalised partials are
 * merged by log-sum-exp (PR #20769, summary of changes: split KV across
 * multiple blocks/SMs plus a reduction kernel that combines the results).
 * Any head count 1..128 is accepted (PR #20769: num_heads below 128 is what
 * lets tensor parallelism shard heads); no padding to 128 is required.
 * mla_decode_multi_token takes several query tokens per request under a
 * causal mask (speculative decoding; see its comment), and mla_decode_sparse
 * attends to a listed subset of each request's tokens.
 *
 * Conventions shared by every entry point:
 *  - All data pointers are caller-owned DEVICE memory on the current HIP
 *    device. The library never allocates, frees, or retains pointers. Every
 *    call's plan, partial rows and counters live in the caller's workspace
 *    (PR #20769 review: a module-global workspace is not thread-safe; the
 *    workspace is per caller). The only global state is a mutex-guarded
 *    cache of immutable device properties (architecture, CU count), filled
 *    on a device's first call.
 *  - Every call enqueues on `stream` (a hipStream_t; NULL = the null stream)
 *    and returns without synchronising. A returned MLA_OK covers argument
 *    validation and launch only.
 *  - Arguments are validated before any HIP call, so every MLA_ERR_INVALID_ARG
 *    path is observable on a machine without a GPU. Then: no usable device ->
 *    MLA_ERR_NO_DEVICE; a device other than gfx950 -> MLA_ERR_UNSUPPORTED
 *    (every symbol is always exported; PR #20769 timeline: an undefined
 *    workspace-size symbol broke import on other GPUs).
 *  - Unsupported configurations are reported, never silently changed.
 *  - No C++ exception crosses this boundary.
 *  - Device-side inputs are clamped, never trusted: a block-table entry outside
 *    [0, num_blocks) is read as block 0 and a seq_lens entry outside
 *    [0, max_blocks_per_seq * block_size] is clamped into that range (no
 *    out-of-bounds access; the result is not meaningful). The bounds-check
 *    build of this library (libmla_mi355x_checked.so, compiled with
 *    MLA_BOUNDS_CHECK=1) also reports each clamp: every decode call with a
 *    workspace first zeroes the 32-bit word at byte offset
 *    MLA_BOUNDS_WORD_OFFSET of the workspace, then ORs MLA_BOUNDS_BAD_BLOCK
 *    and/or MLA_BOUNDS_BAD_SEQ_LEN into it; the host reads it after the call
 *    has run (e.g. after a stream sync). A sparse list entry outside
 *    [0, seq_len) is not an error (it is skipped by definition), but its
 *    request's seq_len and the block ids it maps through are checked.
 *    mla_decode_noalloc reports nothing.
 */
#ifndef MLA_MI355X_H
#define MLA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_HEAD_DIM_K 576   /* key width: 512 kv_c + 64 rope */
#define MLA_HEAD_DIM_V 512   /* value width: kv_c */
#define MLA_MAX_HEADS 128
#define MLA_MAX_QUERY_LEN 16   /* query tokens per request (mla_decode_multi_token) */
#define MLA_MAX_FORCED_SPLITS 16
#define MLA_MAX_TOPK 65536     /* listed positions per request (mla_decode_sparse) */
#define MLA_FP8_GROUP 128      /* k per scale group of the block-scaled E4M3 GEMM */
#define MLA_GEMM_MAX_M 65536   /* tokens per mla_gemm_fp8_blockscale call */
#define MLA_GEMM_MAX_N 65536
#define MLA_GEMM_MAX_K 65536
/* Bounds-check build: the error word's byte offset in the workspace, and its bits. */
#define MLA_BOUNDS_WORD_OFFSET 32
#define MLA_BOUNDS_BAD_BLOCK 1
#define MLA_BOUNDS_BAD_SEQ_LEN 2
/* Bytes of the device scratch array behind mla_decode_noalloc (one per GPU). */
#define MLA_NOALLOC_SCRATCH_BYTES (96ull << 20)

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = -1,        /* null/misaligned pointer, out-of-range size */
  MLA_ERR_UNSUPPORTED = -2,        /* valid request the library does not serve (device not gfx950) */
  MLA_ERR_WORKSPACE_TOO_SMALL = -3,
  MLA_ERR_NO_DEVICE = -4,
  MLA_ERR_HIP = -5                 /* a HIP runtime call or launch failed */
} mla_status_t;

typedef enum {
  MLA_KV_BF16 = 0,
  MLA_KV_FP8_E4M3 = 1  /* OCP E4M3FN codes times one per-tensor fp32 scale */
} mla_kv_dtype_t;

/*
 * Workspace bytes that mla_decode needs (the analogue of the workspace-size
 * query with four 64-bit arguments in PR #20769, workspace sizing snippet).
 * Pure host arithmetic: no HIP call, works without a GPU.
 *
 *  batch        number of decode requests (>= 0)
 *  num_heads    1..128
 *  max_seq_len  upper bound on any seq_len; mla_decode itself checks against
 *               max_blocks_per_seq * block_size, so pass that product
 *  num_splits   0 = automatic scheduling; 1..16 = that many splits per request
 *  num_cus      compute units to plan for; <= 0 means 256 (MI355X)
 *
 * Returns 0 when an argument is out of range.
 */
size_t mla_get_workspace_size(int64_t batch, int64_t num_heads, int64_t max_seq_len,
                              int64_t num_splits, int64_t num_cus);

/*
 * Workspace bytes that mla_decode_multi_token needs: as mla_get_workspace_size
 * with q_len (1..16) query tokens per request. q_len = 1 gives the same value
 * as mla_get_workspace_size.
 */
size_t mla_get_workspace_size_multi_token(int64_t batch, int64_t num_heads, int64_t q_len,
                                          int64_t max_seq_len, int64_t num_splits,
                                          int64_t num_cus);

/*
 * mla_decode: out, lse <- attention of q over the paged cache (formula above).
 *
 *  q            [batch][num_heads][576] bf16, contiguous, 16-byte aligned
 *  kv_cache     [num_blocks][block_size][576] bf16 (MLA_KV_BF16) or uint8
 *               E4M3FN codes (MLA_KV_FP8_E4M3), contiguous, 16-byte aligned
 *  block_table  [batch][max_blocks_per_seq] int32 physical block ids; entries
 *               past ceil(seq_lens[b] / block_size) are never read
 *  seq_lens     [batch] int32, 0 <= seq_lens[b] <= max_blocks_per_seq *
 *               block_size. A request with seq_len 0 gets out = 0,
 *               lse = -inf. Lengths beyond the table capacity are clamped to
 *               it, and a block id outside [0, num_blocks) is read as block 0:
 *               the result of such a request is then not meaningful, but
 *               nothing outside the cache is ever read.
 *  out          [batch][num_heads][512] bf16 (fp32 accumulation, round to
 *               nearest even), 16-byte aligned, fully overwritten
 *  lse          [batch][num_heads] fp32 natural-log LSE of the scaled logits,
 *               or NULL if not wanted
 *  scale        logit scale applied to q.k (finite)
 *  num_heads    1..128
 *  block_size   16, 32, 64 or 128 tokens per physical block
 *  num_splits   0 = automatic: the KV of all requests is cut into balanced
 *               contiguous ranges, one per workgroup slot on the device, so
 *               every CU is busy even at batch 1; a request cut into several
 *               ranges is merged by the LSE combine. 1..16 = every request is
 *               cut into exactly that many near-equal token ranges (some may
 *               be empty), merged the same way.
 *  batch        number of requests (0 is a no-op); batch * (1 + ceil(
 *               max_blocks_per_seq * block_size / 16)) must not exceed
 *               2^30 - 1 (the split plan sums per-request costs in int32;
 *               with sparse decode topk stands for the product)
 *  max_blocks_per_seq  row length of block_table (>= 1)
 *  num_blocks   number of physical blocks in kv_cache (>= 1)
 *  kv_dtype     mla_kv_dtype_t
 *  kv_scale     per-tensor dequantisation scale: exactly 1.0 for MLA_KV_BF16,
 *               finite and > 0 for MLA_KV_FP8_E4M3. In the fp8 path q is
 *               quantised inside the kernel into two E4M3 rows per (request,
 *               head): the rounded row and its rounding residual, both in
 *               the row's one scale amax / 448; P * 2^8 is carried the same
 *               way as two E4M3 terms, and both products run on fp8 matrix
 *               cores.
 *  workspace    caller-owned device scratch of at least workspace_bytes,
 *               256-byte aligned, needing no initialisation; distinct
 *               concurrent calls need distinct workspaces
 *  workspace_bytes  >= mla_get_workspace_size(batch, num_heads,
 *               max_blocks_per_seq * block_size, num_splits, <device CUs>)
 *               in forced mode; in automatic mode a smaller workspace is
 *               accepted down to what one partition per CU needs, and fewer
 *               partitions are used (results are unchanged)
 *  stream       hipStream_t to enqueue on
 */
mla_status_t mla_decode(const void* q, const void* kv_cache, const int32_t* block_table,
                        const int32_t* seq_lens, void* out, float* lse, float scale,
                        int32_t num_heads, int32_t block_size, int32_t num_splits,
                        int32_t batch, int32_t max_blocks_per_seq, int32_t num_blocks,
                        int32_t kv_dtype, float kv_scale, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * mla_decode_multi_token: q_len query tokens per request, as speculative
 * decoding verifies draft tokens (PR #57428, measurement notes: speculative
 * decoding named as not measured; PR #20769, review of ensure_size: the
 * decode workspace follows max_query_len). The pages leave the mask open;
 * this library takes the causal reading: the q_len new tokens are the last
 * q_len positions of the request, already in the cache and counted in
 * seq_lens[b] = N, and query token i (0-based) attends to cache tokens
 * 0 .. N - q_len + i. A query token that sees no token (N - q_len + i < 0)
 * gets out = 0, lse = -inf.
 *
 *  q            [batch][q_len][num_heads][576] bf16, contiguous, 16-byte aligned
 *  out          [batch][q_len][num_heads][512] bf16, 16-byte aligned
 *  lse          [batch][q_len][num_heads] fp32, or NULL
 *  q_len        1..16; num_heads 1..128 as for mla_decode
 *  workspace_bytes  >= mla_get_workspace_size_multi_token(batch, num_heads,
 *               q_len, max_blocks_per_seq * block_size, num_splits, <CUs>)
 *               (automatic mode again accepts less, with fewer partitions)
 *
 * Every other argument, the error behaviour and the ownership rules are
 * those of mla_decode; q_len = 1 is exactly mla_decode. All q_len * num_heads
 * query rows of a request share each cached token read.
 */
mla_status_t mla_decode_multi_token(const void* q, const void* kv_cache,
                                    const int32_t* block_table, const int32_t* seq_lens,
                                    void* out, float* lse, float scale, int32_t num_heads,
                                    int32_t q_len, int32_t block_size, int32_t num_splits,
                                    int32_t batch, int32_t max_blocks_per_seq,
                                    int32_t num_blocks, int32_t kv_dtype, float kv_scale,
                                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * mla_decode_noalloc: mla_decode_multi_token for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). It takes no workspace: the plan, partial rows and
 * counters live in a static device array of MLA_NOALLOC_SCRATCH_BYTES
 * (96 MiB) that every GPU the library runs on holds until the process ends;
 * the call itself allocates nothing (no hipMalloc, hipFree or allocating
 * library routine). The caller still passes inputs and outputs, with the
 * layouts, limits and error behaviour of mla_decode_multi_token.
 *
 *  - A call whose workspace need, mla_get_workspace_size_multi_token(batch,
 *    num_heads, q_len, max_blocks_per_seq * block_size, num_splits, <CUs>),
 *    exceeds the array is rejected with MLA_ERR_WORKSPACE_TOO_SMALL before
 *    anything is enqueued. Automatic mode fits any head count and query
 *    length at batches up to tens of thousands of requests; forced splits
 *    need batch * num_splits * num_heads * q_len * 2052 bytes and more.
 *  - Nothing in the array needs to start at zero: each call writes what it
 *    reads, and the array keeps the last call's contents.
 *  - Every call on one GPU shares that GPU's array: calls that overlap on one
 *    GPU (concurrent streams, or several host threads) race and may corrupt
 *    each other's results. Serialise them, e.g. on one stream.
 *  - The array's device address is looked up once per device, on that
 *    device's first call (hipGetSymbolAddress), with the device current.
 */
mla_status_t mla_decode_noalloc(const void* q, const void* kv_cache, const int32_t* block_table,
                                const int32_t* seq_lens, void* out, float* lse, float scale,
                                int32_t num_heads, int32_t q_len, int32_t block_size,
                                int32_t num_splits, int32_t batch, int32_t max_blocks_per_seq,
                                int32_t num_blocks, int32_t kv_dtype, float kv_scale,
                                void* stream);

/*
 * mla_decode_profiled: exactly mla_decode_multi_token, and additionally
 * records the four caller-created hipEvent_t handles in events[0..3] on
 * `stream`: before the split-plan kernel, before the attention kernel, after
 * the attention kernel and after the combine kernel. Used to time the
 * attention kernel alone. events must be non-NULL with four non-NULL entries.
 */
mla_status_t mla_decode_profiled(const void* q, const void* kv_cache,
                                 const int32_t* block_table, const int32_t* seq_lens,
                                 void* out, float* lse, float scale, int32_t num_heads,
                                 int32_t q_len, int32_t block_size, int32_t num_splits,
                                 int32_t batch, int32_t max_blocks_per_seq, int32_t num_blocks,
                                 int32_t kv_dtype, float kv_scale, void* workspace,
                                 size_t workspace_bytes, void* stream, void* const* events);

/*
 * mla_decode_sparse: each request attends to a listed subset of its cached
 * tokens (sparse MLA decode; PR #57428 deploys a sparse MLA attention
 * backend with the fp8 cache, deployment command and test result). The
 * pages do not define the operation; this library takes the plain reading:
 *
 *   request b attends to the tokens at positions indices[b][0..topk), each
 *   entry counted once per appearance (a repeated position weighs twice);
 *   entries outside [0, seq_lens[b]) are skipped, so short lists are padded
 *   with -1; a list with no valid entry gives out = 0, lse = -inf.
 *
 *  indices      [batch][topk] int32 token positions within each request
 *               (device, 4-byte aligned); the order is free
 *  topk         1..65536 entries per request
 *  q, out, lse  as for mla_decode (one query token per request)
 *  workspace_bytes  >= mla_get_workspace_size_sparse(batch, num_heads, topk,
 *               num_splits, <CUs>) (automatic mode accepts less, as above)
 *
 * Every other argument, the error behaviour and the ownership rules are
 * those of mla_decode. Also MLA_ERR_INVALID_ARG if num_blocks * block_size
 * exceeds 2^31 - 1. A prepass turns each entry into a physical row id through
 * block_table; the attention kernel then gathers the listed rows.
 */
mla_status_t mla_decode_sparse(const void* q, const void* kv_cache, const int32_t* block_table,
                               const int32_t* seq_lens, const int32_t* indices, int32_t topk,
                               void* out, float* lse, float scale, int32_t num_heads,
                               int32_t block_size, int32_t num_splits, int32_t batch,
                               int32_t max_blocks_per_seq, int32_t num_blocks, int32_t kv_dtype,
                               float kv_scale, void* workspace, size_t workspace_bytes,
                               void* stream);

/* Workspace bytes that mla_decode_sparse needs (pure host arithmetic; 0 when
 * an argument is out of range). */
size_t mla_get_workspace_size_sparse(int64_t batch, int64_t num_heads, int64_t topk,
                                     int64_t num_splits, int64_t num_cus);

/* mla_decode_sparse, recording events[0..3] as mla_decode_profiled does
 * (events[0] precedes the sparse prepass). */
mla_status_t mla_decode_sparse_profiled(const void* q, const void* kv_cache,
                                        const int32_t* block_table, const int32_t* seq_lens,
                                        const int32_t* indices, int32_t topk, void* out,
                                        float* lse, float scale, int32_t num_heads,
                                        int32_t block_size, int32_t num_splits, int32_t batch,
                                        int32_t max_blocks_per_seq, int32_t num_blocks,
                                        int32_t kv_dtype, float kv_scale, void* workspace,
                                        size_t workspace_bytes, void* stream,
                                        void* const* events);

/*
 * mla_combine: merge normalised split partials by log-sum-exp (PR #20769,
 * summary of changes: the reduction kernel that combines split-KV results).
 * num_heads counts the rows of one request: the heads, or q_len * heads for
 * partials of several query tokens (1..2048).
 *
 *  partial_out  [total_rows][num_heads][512] fp32, each row already divided
 *               by its own softmax denominator, 16-byte aligned
 *  partial_lse  [total_rows][num_heads] fp32 natural-log LSE; -inf marks an
 *               empty split (weight 0; its partial_out values are ignored)
 *  split_indptr [batch + 1] int32, non-decreasing, split_indptr[0] = 0:
 *               request b owns rows split_indptr[b] .. split_indptr[b+1]-1
 *  out          [batch][num_heads][512] bf16: sum_s w_s o_s / sum_s w_s with
 *               w_s = exp(lse_s - max_s lse_s); a request with no row or only
 *               empty rows gets out = 0, lse = -inf
 *  lse          [batch][num_heads] fp32 = max + ln(sum_s w_s), or NULL
 */
mla_status_t mla_combine(const float* partial_out, const float* partial_lse,
                         const int32_t* split_indptr, void* out, float* lse, int32_t batch,
                         int32_t num_heads, void* stream);

/*
 * The projection beside the decode path: the block-scaled E4M3 GEMM of the
 * DeepSeek-R1 fused q/kv down-projection (issue #28427, "DeepSeek-R1 KV Proj
 * is Too Slow for TP": block FP8 weights at a handful of decode tokens,
 * where a swapped-operand kernel wins). The pages name the format (block
 * FP8) but not its block shape; this library takes DeepSeek's: one fp32 scale
 * per token and 128-wide group of k for activations, one per 128 x 128
 * block for weights.
 *
 * mla_quant_fp8_groups: x [m][k] bf16 -> x_fp8 [m][k] E4M3FN codes and
 * x_scale [m][k / 128] fp32, per token and group:
 *     scale = max(amax, 1e-10) / 448,  code = E4M3(clamp(x / scale, +-448))
 * with a correctly rounded fp32 division and round-to-nearest-even codes.
 *  m 0..65536 (0 is a no-op); k a multiple of 128 up to 65536; x 4-byte,
 *  x_fp8 2-byte, x_scale 4-byte aligned. Finite inputs.
 *
 * mla_gemm_fp8_blockscale: c [m][n] bf16 (fp32 accumulation, round to nearest
 * even) =
 *     sum_k e4m3(a[i][k]) a_scale[i][k / 128] * e4m3(b[j][k]) b_scale[j / 128][k / 128]
 *  a        [m][k] E4M3FN codes, 16-byte aligned; a_scale [m][k / 128] fp32
 *  b        [n][k] E4M3FN codes (one row per output feature), 16-byte
 *           aligned; b_scale [ceil(n / 128)][k / 128] fp32
 *  c        [m][n] bf16, 8-byte aligned, fully overwritten
 *  m 0..65536, n a multiple of 16 up to 65536, k a multiple of 128 up to 65536.
 * Ownership, asynchrony and error behaviour as for mla_decode; no workspace.
 */
mla_status_t mla_quant_fp8_groups(const void* x, void* x_fp8, float* x_scale, int32_t m,
                                  int32_t k, void* stream);
mla_status_t mla_gemm_fp8_blockscale(const void* a, const float* a_scale, const void* b,
                                     const float* b_scale, void* c, int32_t m, int32_t n,
                                     int32_t k, void* stream);

/*
 * The per-head products on either side of absorbed decode (the pages show
 * only the absorbed, 576-wide query; DeepSeek's shapes are taken: 128
 * no-rope and 64 rope query dims per head, 512 latent dims, 128 value dims).
 *
 * mla_absorb_q: q [batch][num_heads][576] bf16 =
 *     [ q_nope[b][h][0:128] . w_uk[h] (128 x 512), q_rope[b][h][0:64] ]
 * the query mla_decode takes.
 *  q_nope [batch][num_heads][128], w_uk [num_heads][128][512],
 *  q_rope [batch][num_heads][64]: bf16, 16-byte aligned.
 *
 * mla_absorb_out: o [batch][num_heads][128] bf16,
 *     o[b][h][v] = sum over c < 512 of o_latent[b][h][c] * w_uv[h][v][c]
 * mapping mla_decode's output back to the value dimension. w_uv holds one
 * 512-wide row per value dim (the value up-projection's own layout).
 *  o_latent [batch][num_heads][512], w_uv [num_heads][128][512]: bf16,
 *  16-byte aligned.
 *
 * fp32 accumulation, bf16 rounding to nearest even. batch 0..65536 (0 is a
 * no-op), num_heads 1..128. Ownership and errors as for mla_decode.
 */
mla_status_t mla_absorb_q(const void* q_nope, const void* w_uk, const void* q_rope, void* q,
                          int32_t batch, int32_t num_heads, void* stream);
mla_status_t mla_absorb_out(const void* o_latent, const void* w_uv, void* o, int32_t batch,
                            int32_t num_heads, void* stream);

/* Static, human-readable name of a status code. */
const char* mla_status_string(int32_t status);

/* ABI revision of this header; bumped on any signature change. */
int32_t mla_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_MI355X_H */
