/*
 * mla_oracle.c -- plain, slow, fp64 CPU reference for absorbed MLA decode over a
 * paged latent KV cache.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this file's library. It shares no
 * code, header, table or constant with the GPU path, and it includes no HIP.
 *
 * What it computes (written from the sources, not from any listing):
 *
 *  - One query token per request, batch = number of decode requests
 *    (PR #20769 "SM100 Cutlass MLA decode with unrestricted num_heads (< 128)
 *    for DeepSeek TP", review of ensure_size: max_query_len = 1,
 *    batch_size = num_decodes).
 *  - Or q_len > 1 query tokens per request, as speculative decoding verifies
 *    draft tokens (PR #57428, measurement notes: speculative decoding named
 *    as untested; PR #20769, the same review: the workspace follows
 *    max_query_len). The pages do not define the mask, so the oracle takes
 *    the usual causal reading: the q_len new tokens are the last q_len
 *    positions of the request, already counted in seq_len, and query token
 *    i (0-based) sees cache tokens 0 .. N - q_len + i. A query token with no
 *    visible token gets out = 0, lse = -inf.
 *  - The cache is paged: a request's token t lives in physical block
 *    block_table[b][t / block_size], slot t % block_size
 *    (PR #21078 "Flashinfer MLA (trtllm-gen) decode kernel integration",
 *    E2E benchmark command: --block-size 32; PR #20769, workspace sizing
 *    snippet: PAGE_SIZE).
 *  - Each cached token is a 576-wide latent: columns 0..511 are the compressed
 *    kv_c, columns 512..575 the rope part. Keys are the full 576 columns and
 *    values are the first 512 (the absorbed-MLA shape of DeepSeek-V2/R1).
 *  - Per (request, head): x_t = scale * <q, k_t>, out = sum_t softmax(x)_t v_t,
 *    lse = log(sum_t exp(x_t)) in natural log. This is exact softmax
 *    attention, so the oracle is that definition written out in fp64.
 *  - Split-KV: a request's tokens may be cut into contiguous ranges whose
 *    normalised partial outputs and LSEs are merged by log-sum-exp weights
 *    (PR #20769, summary of changes: split KV across multiple blocks/SMs and a
 *    reduction kernel that combines the results). oracle_lse_merge is that
 *    merge written out.
 *  - fp8 cache: OCP E4M3FN codes (sign, 4 exponent bits with bias 7, 3
 *    mantissa bits; exponent 15 with mantissa 7 is NaN; no infinities) times
 *    a per-tensor fp32 scale (PR #57428, deployment command:
 *    --kv-cache-dtype fp8). oracle_e4m3_to_double decodes one code from that
 *    definition.
 *
 * Readings taken where the sources are silent: an empty token range yields
 * out = 0 and lse = -inf; tokens at or past seq_len are never read; table
 * entries past ceil(seq_len / block_size) are never read.
 *
 * Every floating-point step is fp64 on inputs that are exact in fp64 (bf16
 * values, e4m3 codes times an fp32 scale, the fp32 softmax scale), so the
 * result carries only fp64 rounding.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_D 576   /* latent + rope width: key width */
#define ORACLE_DV 512  /* kv_c width: value width */

/* Status codes returned by the oracle entry points. */
#define ORACLE_OK 0
#define ORACLE_BAD_ARG -1
#define ORACLE_BAD_BLOCK -2

static double bf16_bits_to_double(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* OCP 8-bit floating point, E4M3FN variant: value of one code. */
double oracle_e4m3_to_double(uint8_t code) {
  int sign = (code >> 7) & 1;
  int exponent = (code >> 3) & 0xF;
  int mantissa = code & 0x7;
  double v;
  if (exponent == 0xF && mantissa == 0x7) return NAN;
  if (exponent == 0)
    v = ldexp((double)mantissa / 8.0, -6); /* subnormal: 0.m * 2^(1-7) */
  else
    v = ldexp(1.0 + (double)mantissa / 8.0, exponent - 7);
  return sign ? -v : v;
}

double oracle_bf16_to_double(uint16_t bits) { return bf16_bits_to_double(bits); }

/* The value of every E4M3 code, from oracle_e4m3_to_double (filled before any
 * parallel region; a lookup gives exactly the decoded value, only faster). */
static double e4m3[256];

static void fill_e4m3_table(void) {
  for (int c = 0; c < 256; ++c) e4m3[c] = oracle_e4m3_to_double((uint8_t)c);
}

/* Key/value row of one cached token, widened to fp64. */
static void load_token(const void* kv_cache, int kv_fp8, double kv_scale, int64_t row,
                       double* k) {
  if (kv_fp8) {
    const uint8_t* p = (const uint8_t*)kv_cache + row * ORACLE_D;
    for (int d = 0; d < ORACLE_D; ++d) k[d] = e4m3[p[d]] * kv_scale;
  } else {
    const uint16_t* p = (const uint16_t*)kv_cache + row * ORACLE_D;
    for (int d = 0; d < ORACLE_D; ++d) k[d] = bf16_bits_to_double(p[d]);
  }
}

/*
 * oracle_mla_attend: exact attention of selected (request, token range) items.
 *
 *  q           [batch][q_len][num_heads][576] bf16 bits
 *  kv_cache    [num_blocks][block_size][576] bf16 bits (kv_fp8 = 0) or
 *              E4M3FN codes (kv_fp8 = 1)
 *  kv_scale    per-tensor dequantisation scale for E4M3 (ignored for bf16)
 *  block_table [batch][max_blocks] physical block ids
 *  seq_lens    [batch]
 *  scale       the fp32 logit scale, widened exactly to fp64
 *  q_len       query tokens per request (>= 1)
 *  items       n_items entries; item i covers request req[i], tokens
 *              [tok_begin[i], tok_end[i]) clipped to [0, seq_lens[req[i]]);
 *              query token qi additionally sees only tokens
 *              t < seq_lens[req[i]] - (q_len - 1 - qi)
 *  out         [n_items][q_len][num_heads][512] fp64: sum_t w_t v_t / sum_t w_t
 *  lse         [n_items][q_len][num_heads] fp64: natural log of sum_t exp(x_t)
 *
 * The work is spread over (item, query token, head) with OpenMP; each is a
 * plain sequential loop, so results do not depend on the thread count.
 */
int oracle_mla_attend(const uint16_t* q, const void* kv_cache, int kv_fp8, float kv_scale,
                      const int32_t* block_table, const int32_t* seq_lens, int64_t batch,
                      int64_t num_heads, int64_t q_len, int64_t block_size,
                      int64_t max_blocks, int64_t num_blocks, float scale, const int32_t* req,
                      const int64_t* tok_begin, const int64_t* tok_end, int64_t n_items,
                      double* out, double* lse) {
  if (!q || !kv_cache || !block_table || !seq_lens || !req || !tok_begin || !tok_end ||
      !out || !lse)
    return ORACLE_BAD_ARG;
  if (batch < 0 || num_heads < 1 || q_len < 1 || block_size < 1 || max_blocks < 0 ||
      num_blocks < 0 || n_items < 0)
    return ORACLE_BAD_ARG;

  /* Validate every block id that will be read, before any arithmetic. */
  for (int64_t i = 0; i < n_items; ++i) {
    int64_t b = req[i];
    if (b < 0 || b >= batch) return ORACLE_BAD_ARG;
    int64_t n = seq_lens[b];
    if (n < 0 || n > max_blocks * block_size) return ORACLE_BAD_ARG;
    int64_t t0 = tok_begin[i] < 0 ? 0 : tok_begin[i];
    int64_t t1 = tok_end[i] > n ? n : tok_end[i];
    for (int64_t t = t0; t < t1; ++t) {
      int64_t blk = block_table[b * max_blocks + t / block_size];
      if (blk < 0 || blk >= num_blocks) return ORACLE_BAD_BLOCK;
    }
  }

  const double s = (double)scale;
  const double kvs = (double)kv_scale;
  int64_t n_work = n_items * q_len * num_heads;
  fill_e4m3_table();

#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t w = 0; w < n_work; ++w) {
    int64_t i = w / (q_len * num_heads);
    int64_t qi = (w / num_heads) % q_len, h = w % num_heads;
    int64_t b = req[i];
    int64_t n = seq_lens[b];
    int64_t visible = n - (q_len - 1 - qi); /* causal: tokens up to query qi's own */
    int64_t t0 = tok_begin[i] < 0 ? 0 : tok_begin[i];
    int64_t t1 = tok_end[i] > n ? n : tok_end[i];
    if (t1 > visible) t1 = visible;
    int64_t row_out = (i * q_len + qi) * num_heads + h;
    double* o = out + row_out * ORACLE_DV;
    double qv[ORACLE_D], k[ORACLE_D];
    for (int d = 0; d < ORACLE_DV; ++d) o[d] = 0.0;
    if (t1 <= t0) {
      lse[row_out] = -INFINITY;
      continue;
    }
    for (int d = 0; d < ORACLE_D; ++d)
      qv[d] = bf16_bits_to_double(q[((b * q_len + qi) * num_heads + h) * ORACLE_D + d]);

    /* Pass 1: every logit x_t and their maximum. */
    int64_t len = t1 - t0;
    double* x = (double*)malloc((size_t)len * sizeof(double));
    double m = -INFINITY;
    for (int64_t t = t0; t < t1; ++t) {
      int64_t row = (int64_t)block_table[b * max_blocks + t / block_size] * block_size +
                    t % block_size;
      load_token(kv_cache, kv_fp8, kvs, row, k);
      double dot = 0.0;
      for (int d = 0; d < ORACLE_D; ++d) dot += qv[d] * k[d];
      x[t - t0] = s * dot;
      if (x[t - t0] > m) m = x[t - t0];
    }
    /* Pass 2: weights w_t = exp(x_t - m), their sum, and sum_t w_t v_t. */
    double l = 0.0;
    for (int64_t t = t0; t < t1; ++t) {
      int64_t row = (int64_t)block_table[b * max_blocks + t / block_size] * block_size +
                    t % block_size;
      load_token(kv_cache, kv_fp8, kvs, row, k);
      double wt = exp(x[t - t0] - m);
      l += wt;
      for (int d = 0; d < ORACLE_DV; ++d) o[d] += wt * k[d];
    }
    free(x);
    for (int d = 0; d < ORACLE_DV; ++d) o[d] /= l;
    lse[row_out] = m + log(l);
  }
  return ORACLE_OK;
}

/*
 * oracle_mla_attend_sparse: attention of each request over a listed subset of
 * its cached tokens (sparse MLA decode). The pages name a sparse MLA backend
 * next to the fp8 cache (PR #57428, deployment command and test result:
 * FLASHINFER_MLA_SPARSE_DSV41 with --kv-cache-dtype fp8) without defining
 * it; the oracle takes the plain reading: request b attends to the tokens
 * whose positions indices[b][0..topk) lists, each listed entry counted once
 * per appearance, and entries outside [0, seq_lens[b]) are skipped (they
 * pad short lists). With no listed token: out = 0, lse = -inf.
 *
 *  q        [batch][num_heads][576] bf16 bits (one query token per request)
 *  indices  [batch][topk] token positions within each request
 *  out      [batch][num_heads][512] fp64; lse [batch][num_heads] fp64
 * Other arguments as for oracle_mla_attend.
 */
int oracle_mla_attend_sparse(const uint16_t* q, const void* kv_cache, int kv_fp8,
                             float kv_scale, const int32_t* block_table,
                             const int32_t* seq_lens, int64_t batch, int64_t num_heads,
                             int64_t block_size, int64_t max_blocks, int64_t num_blocks,
                             float scale, const int32_t* indices, int64_t topk, double* out,
                             double* lse) {
  if (!q || !kv_cache || !block_table || !seq_lens || !indices || !out || !lse)
    return ORACLE_BAD_ARG;
  if (batch < 0 || num_heads < 1 || block_size < 1 || max_blocks < 0 || num_blocks < 0 ||
      topk < 0)
    return ORACLE_BAD_ARG;
  for (int64_t b = 0; b < batch; ++b) {
    int64_t n = seq_lens[b];
    if (n < 0 || n > max_blocks * block_size) return ORACLE_BAD_ARG;
    for (int64_t j = 0; j < topk; ++j) {
      int64_t t = indices[b * topk + j];
      if (t < 0 || t >= n) continue;
      int64_t blk = block_table[b * max_blocks + t / block_size];
      if (blk < 0 || blk >= num_blocks) return ORACLE_BAD_BLOCK;
    }
  }
  const double s = (double)scale;
  const double kvs = (double)kv_scale;
  fill_e4m3_table();

#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t w = 0; w < batch * num_heads; ++w) {
    int64_t b = w / num_heads, h = w % num_heads;
    int64_t n = seq_lens[b];
    double* o = out + w * ORACLE_DV;
    double qv[ORACLE_D], k[ORACLE_D];
    for (int d = 0; d < ORACLE_DV; ++d) o[d] = 0.0;
    for (int d = 0; d < ORACLE_D; ++d)
      qv[d] = bf16_bits_to_double(q[(b * num_heads + h) * ORACLE_D + d]);
    double* x = (double*)malloc((size_t)(topk > 0 ? topk : 1) * sizeof(double));
    /* Pass 1: the logit of every listed token and their maximum. */
    double m = -INFINITY;
    int64_t listed = 0;
    for (int64_t j = 0; j < topk; ++j) {
      int64_t t = indices[b * topk + j];
      if (t < 0 || t >= n) continue;
      int64_t row = (int64_t)block_table[b * max_blocks + t / block_size] * block_size +
                    t % block_size;
      load_token(kv_cache, kv_fp8, kvs, row, k);
      double dot = 0.0;
      for (int d = 0; d < ORACLE_D; ++d) dot += qv[d] * k[d];
      x[j] = s * dot;
      if (x[j] > m) m = x[j];
      ++listed;
    }
    if (listed == 0) {
      free(x);
      lse[w] = -INFINITY;
      continue;
    }
    /* Pass 2: weights, their sum and the weighted value rows. */
    double l = 0.0;
    for (int64_t j = 0; j < topk; ++j) {
      int64_t t = indices[b * topk + j];
      if (t < 0 || t >= n) continue;
      int64_t row = (int64_t)block_table[b * max_blocks + t / block_size] * block_size +
                    t % block_size;
      load_token(kv_cache, kv_fp8, kvs, row, k);
      double wt = exp(x[j] - m);
      l += wt;
      for (int d = 0; d < ORACLE_DV; ++d) o[d] += wt * k[d];
    }
    free(x);
    for (int d = 0; d < ORACLE_DV; ++d) o[d] /= l;
    lse[w] = m + log(l);
  }
  return ORACLE_OK;
}

/*
 * oracle_lse_merge: merge n_parts normalised partial results of one request.
 *
 *  part_out [n_parts][num_heads][512], part_lse [n_parts][num_heads]
 *  out      [num_heads][512], lse [num_heads]
 *
 * Per head: M = max_s lse_s; w_s = exp(lse_s - M); lse = M + log(sum_s w_s);
 * out = sum_s w_s out_s / sum_s w_s. A part with lse = -inf has weight 0 and
 * its out is not read; if every part is -inf the result is out = 0,
 * lse = -inf.
 */
int oracle_lse_merge(const double* part_out, const double* part_lse, int64_t n_parts,
                     int64_t num_heads, double* out, double* lse) {
  if (!part_out || !part_lse || !out || !lse || n_parts < 0 || num_heads < 1)
    return ORACLE_BAD_ARG;
  for (int64_t h = 0; h < num_heads; ++h) {
    double* o = out + h * ORACLE_DV;
    double M = -INFINITY;
    for (int64_t p = 0; p < n_parts; ++p)
      if (part_lse[p * num_heads + h] > M) M = part_lse[p * num_heads + h];
    for (int d = 0; d < ORACLE_DV; ++d) o[d] = 0.0;
    if (M == -INFINITY) {
      lse[h] = -INFINITY;
      continue;
    }
    double wsum = 0.0;
    for (int64_t p = 0; p < n_parts; ++p) {
      double ls = part_lse[p * num_heads + h];
      if (ls == -INFINITY) continue;
      double w = exp(ls - M);
      wsum += w;
      const double* po = part_out + (p * num_heads + h) * ORACLE_DV;
      for (int d = 0; d < ORACLE_DV; ++d) o[d] += w * po[d];
    }
    for (int d = 0; d < ORACLE_DV; ++d) o[d] /= wsum;
    lse[h] = M + log(wsum);
  }
  return ORACLE_OK;
}

/*
 * oracle_gemm_fp8_blockscale: the block-scaled E4M3 projection that sits beside
 * MLA decode (the DeepSeek-R1 fused q/kv down-projection of issue #28427
 * "DeepSeek-R1 KV Proj is Too Slow for TP": block FP8 weights, small decode M).
 * The plain definition, dequantising every element:
 *
 *   c[i][j] = sum_k (e4m3(a[i][k]) * a_scale[i][k / 128]) *
 *                   (e4m3(b[j][k]) * b_scale[j / 128][k / 128])
 *
 *  a        [m][k] E4M3FN codes (activations); a_scale [m][k / 128] fp32, one
 *           per token and 128-wide group of k
 *  b        [n][k] E4M3FN codes (weights, one row per output feature);
 *           b_scale [ceil(n / 128)][k / 128] fp32, one per 128 x 128 block
 *  c        [m][n] fp64
 * k must be a multiple of 128. OpenMP over rows of c.
 */
int oracle_gemm_fp8_blockscale(const uint8_t* a, const float* a_scale, const uint8_t* b,
                               const float* b_scale, int64_t m, int64_t n, int64_t k,
                               double* c) {
  if (!a || !a_scale || !b || !b_scale || !c || m < 0 || n < 0 || k < 0 || k % 128)
    return ORACLE_BAD_ARG;
  const int64_t kg = k / 128;
  fill_e4m3_table();
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < m; ++i) {
    for (int64_t j = 0; j < n; ++j) {
      double sum = 0.0;
      for (int64_t t = 0; t < k; ++t) {
        double x = e4m3[a[i * k + t]] * (double)a_scale[i * kg + t / 128];
        double w = e4m3[b[j * k + t]] * (double)b_scale[(j / 128) * kg + t / 128];
        sum += x * w;
      }
      c[i * n + j] = sum;
    }
  }
  return ORACLE_OK;
}

/*
 * oracle_absorb: the per-head products on either side of absorbed MLA decode
 * (the decode path takes a 576-wide q whose first 512 columns are the no-rope
 * query absorbed into the latent space, and returns a 512-wide latent output
 * that the value up-projection maps back to the head dimension; DeepSeek's
 * shapes: 128 no-rope dims, 64 rope dims, 512 latent dims, 128 value dims).
 * Written out per element in fp64:
 *
 *   c[b][h][j] = sum_i x[b][h][i] * w[h][i][j]       j < n_out
 *
 *  x  [batch][heads][k_in] bf16 bits;  w [heads][k_in][n_out] bf16 bits
 *  c  [batch][heads][n_out] fp64
 * q absorption: k_in = 128, n_out = 512 (w = W_UK per head); output
 * absorption: k_in = 512, n_out = 128 (w = W_UV per head).
 */
int oracle_absorb(const uint16_t* x, const uint16_t* w, int64_t batch, int64_t heads,
                  int64_t k_in, int64_t n_out, double* c) {
  if (!x || !w || !c || batch < 0 || heads < 1 || k_in < 1 || n_out < 1) return ORACLE_BAD_ARG;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t bh = 0; bh < batch * heads; ++bh) {
    int64_t h = bh % heads;
    for (int64_t j = 0; j < n_out; ++j) {
      double sum = 0.0;
      for (int64_t i = 0; i < k_in; ++i)
        sum += bf16_bits_to_double(x[bh * k_in + i]) *
               bf16_bits_to_double(w[(h * k_in + i) * n_out + j]);
      c[bh * n_out + j] = sum;
    }
  }
  return ORACLE_OK;
}

int oracle_abi_version(void) { return 4; }
