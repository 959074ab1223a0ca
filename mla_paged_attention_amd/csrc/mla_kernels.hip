// mla_kernels.hip -- gfx950 (CDNA4) kernels for absorbed MLA decode over a
// paged latent KV cache.
//
// Three kernels run per decode call, all on the caller's stream:
//
//  1. plan_kernel: from device seq_lens, the split plan. In balanced mode the
//     KV of all requests is laid end to end in 16-token units (plus a fixed
//     per-request overhead) and cut into equal contiguous partitions, one per
//     attention workgroup slot on the device; a request that straddles a cut
//     becomes several pieces. In forced mode every request is cut into
//     num_splits near-equal pieces. The plan stays on the device, so the host
//     never synchronises. (PR #20769 "SM100 Cutlass MLA decode with
//     unrestricted num_heads (< 128) for DeepSeek TP", summary of changes: a
//     tile scheduler and splitting KV across multiple blocks/SMs.)
//
//  2. attention: one workgroup per partition (and group of up to four
//     16-head tiles). The KV of each piece streams HBM -> LDS in tiles with
//     coalesced direct-to-LDS loads through a four-stage ring; the logits
//     (q from registers, K from LDS) and P.V (V through LDS transpose reads)
//     run on matrix cores with an fp32 online softmax in the log2 domain. A
//     one-piece request is written as the final bf16 output and LSE, a piece
//     of a split request as a normalised fp32 partial plus its LSE. Three
//     variants: attn_ws_kernel (bf16, up to 16 heads: a logit wave feeds four
//     P.V waves), attn_mh_kernel<0> (bf16, more heads) and
//     attn_mh_kernel<1> (E4M3 cache, any head count): four logit waves of
//     16 heads each feed four P.V waves of 128 output features each.
//
//  3. combine_kernel: log-sum-exp merge of the partial rows of each split
//     request (PR #20769, summary of changes: the reduction kernel that
//     combines split-KV results).
//
// Operand layouts of v_mfma_f32_16x16x32_bf16 / v_mfma_f32_16x16x16_bf16
// used below (lane l, c = l % 16, g = l / 16): A[i][k] lives in lane with
// i = c and k in the g-th group of k slots; B[k][j] in lane with j = c and
// the same k slots; D[i][j] in lane with j = c, i = 4g + r, r = 0..3. Only
// the symmetry between the k-slot maps of A and B is relied on.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "mla_internal.h"

namespace mla {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kRowBytes = kDK * 2;       // one bf16 cache row: 1152 bytes
constexpr int kQChunks = kDK / 32;       // 18 k-steps of 32 features
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ unsigned short bf16_bits(float x) {
  __bf16 h = (__bf16)x;  // round to nearest even
  return __builtin_bit_cast(unsigned short, h);
}

// ----------------------------------------------------------------------------
// Wave-level scan and maximum on DPP row shifts (rows of 16 lanes: shifts 1,
// 2, 4, 8 with zero fill), then the row totals through v_readlane. All 64
// lanes must be active.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);  // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31),
            r2 = __builtin_amdgcn_readlane(v, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return v + (row > 0 ? r0 : 0) + (row > 1 ? r1 : 0) + (row > 2 ? r2 : 0);
}

__device__ __forceinline__ int wave_max(int v) {
  v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x111, 0xf, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x112, 0xf, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x114, 0xf, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x118, 0xf, 0xf, false));
  return max(max(__builtin_amdgcn_readlane(v, 15), __builtin_amdgcn_readlane(v, 31)),
             max(__builtin_amdgcn_readlane(v, 47), __builtin_amdgcn_readlane(v, 63)));
}

// Block-wide exclusive scan over NT threads: wave scans, then every thread
// adds the totals of the waves before its own.
template <int NT = kPlanThreads>
__device__ int block_exclusive_scan(int v, int* s_wave, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int inc = wave_inclusive_scan(v);
  if (lane == 63) s_wave[wave] = inc;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int t = s_wave[w];
    base += w < wave ? t : 0;
    tot += t;
  }
  *total = tot;
  __syncthreads();
  return base + inc - v;
}

// Block-wide exclusive scans of three values at once (same barriers).
template <int NT>
__device__ int3 block_exclusive_scan3(int3 v, int* s_wave, int3* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int3 inc = make_int3(wave_inclusive_scan(v.x), wave_inclusive_scan(v.y),
                             wave_inclusive_scan(v.z));
  if (lane == 63) {
    s_wave[wave] = inc.x;
    s_wave[16 + wave] = inc.y;
    s_wave[32 + wave] = inc.z;
  }
  __syncthreads();
  int3 base = make_int3(0, 0, 0), tot = make_int3(0, 0, 0);
  for (int w = 0; w < NT / 64; ++w) {
    const int3 sw = make_int3(s_wave[w], s_wave[16 + w], s_wave[32 + w]);
    if (w < wave) {
      base.x += sw.x;
      base.y += sw.y;
      base.z += sw.z;
    }
    tot.x += sw.x;
    tot.y += sw.y;
    tot.z += sw.z;
  }
  __syncthreads();
  *total = tot;
  return make_int3(base.x + inc.x - v.x, base.y + inc.y - v.y, base.z + inc.z - v.z);
}

// Start of piece j when `units` are cut into k near-equal pieces (the first
// units % k pieces one unit longer).
__device__ __forceinline__ int piece_start(int j, int units, int k) {
  const int q = units / k, r = units - q * k;
  return j * q + min(j, r);
}

__device__ __forceinline__ int clamp_len(int n, int cap) { return n < 0 ? 0 : (n > cap ? cap : n); }

// Bounds-check build: reports a clamped input in the call's error word.
__device__ __forceinline__ void report_bounds(int32_t* word, int bit) {
#if MLA_BOUNDS_CHECK
  if (word) atomicOr(word, bit);
#else
  (void)word;
  (void)bit;
#endif
}

// seq_lens[b] clamped to [0, cap]; a value outside is reported.
__device__ __forceinline__ int checked_len(int n, int cap, int32_t* word) {
  if (n < 0 || n > cap) report_bounds(word, kBoundsBadSeqLen);
  return clamp_len(n, cap);
}

__device__ __forceinline__ int units_of(int n) {
  int u = (n + kUnit - 1) / kUnit;
  return u < 1 ? 1 : u;  // an empty request still owns one (empty) unit
}

// Wave-uniform load through the scalar unit (counted by lgkmcnt, not vmcnt,
// so it does not disturb the vector-memory pipeline of the KV ring).
__device__ __forceinline__ int32_t scalar_load_i32(const int32_t* p) {
  int32_t v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
  return v;
}

// Automatic plan modes (header[3]).
constexpr int kPlanContiguous = 0;
constexpr int kPlanSnake = 1;
constexpr int kSnakeMaxBatch = 4096;   // largest batch the snake plan sorts
// Counting-sort buckets of piece costs: 4 per plan thread.

template <int NT>
__device__ __forceinline__ int block_max(int v, int* s_wave) {
  v = wave_max(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) s_wave[wave] = v;
  __syncthreads();
  int r = s_wave[0];
  for (int i = 1; i < NT / 64; ++i) r = max(r, s_wave[i]);
  __syncthreads();
  return r;
}

// Block-wide total and maximum in one exchange (two barriers).
template <int NT>
__device__ __forceinline__ int2 block_sum_max(int sum, int mx, int* s_wave) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ws = __builtin_amdgcn_readlane(wave_inclusive_scan(sum), 63);
  const int wm = wave_max(mx);
  if (lane == 0) {
    s_wave[wave] = ws;
    s_wave[16 + wave] = wm;
  }
  __syncthreads();
  int t = 0, m = s_wave[16];
  for (int i = 0; i < NT / 64; ++i) {
    t += s_wave[i];
    m = max(m, s_wave[16 + i]);
  }
  __syncthreads();
  return make_int2(t, m);
}

// Exclusive scan of s[0..n) in place (n <= NT * 4), returns the total.
template <int NT>
__device__ int block_scan_lds(int* s, int n, int* s_wave) {
  const int tid = threadIdx.x;
  int v[4], sum = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = 4 * tid + k;
    v[k] = i < n ? s[i] : 0;
    sum += v[k];
  }
  int tot;
  int ex = block_exclusive_scan<NT>(sum, s_wave, &tot);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = 4 * tid + k;
    if (i < n) s[i] = ex;
    ex += v[k];
  }
  __syncthreads();
  return tot;
}

// One workgroup, automatic splits only (forced splits need no plan: piece k
// of request b is partition and partial row b * S + k). A list of work items
// (request, unit begin, unit end, partial row or -1 when the item is the
// whole request) per partition, at most max_parts partitions, with costs
// balanced in units of 16 tokens plus a fixed per-request overhead:
//  - snake (batch >= 2 * max_parts, batch <= kSnakeMaxBatch): requests above
//    the per-partition target are cut into near-equal pieces, all pieces are
//    ranked by cost (counting sort, largest first) and dealt to partitions
//    in alternating direction, so large batches need no partial rows;
//  - contiguous otherwise: the requests' costs laid end to end and cut into
//    equal partitions; a request straddling a cut becomes several pieces.
template <int NT>
__global__ void __launch_bounds__(NT) plan_kernel(
    const int32_t* seq_lens, int32_t batch, int32_t cap_tokens, int32_t max_parts, int32_t ovh,
    int32_t* header, int32_t* cum, int32_t* part_ptr, int4* work,
    int4* split) {
  __shared__ int s_wave[48];
  __shared__ int s_cnt[kMaxPlanParts + 1];
  __shared__ int s_bucket[4 * NT];
  __shared__ short s_pq[kSnakeMaxBatch + kMaxPlanParts];
  const int tid = threadIdx.x;
  if (batch <= 4 * NT) {
    // Fast path: thread t owns requests 4 t .. 4 t + 3, kept in registers.
    int units[4], cost[4], c0[4];
    int csum = 0, cmax = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int b = 4 * tid + i;
      units[i] = b < batch ? units_of(clamp_len(seq_lens[b], cap_tokens)) : 0;
      cost[i] = b < batch ? ovh + units[i] : 0;
      c0[i] = csum;
      csum += cost[i];
      cmax = max(cmax, cost[i]);
    }
    int total;
    const int cex = block_exclusive_scan<NT>(csum, s_wave, &total);
    cmax = block_max<NT>(cmax, s_wave);
    int P = (total + max_parts - 1) / max_parts;
    if (P < kMinPartUnits) P = kMinPartUnits;
    const bool snake = batch >= 2 * max_parts && batch <= kSnakeMaxBatch;
    int k[4];
    int3 mine = make_int3(0, 0, 0);  // items, rows, split requests
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c0[i] += cex;
      const int b = 4 * tid + i;
      if (b < batch) {
        k[i] = snake ? (cost[i] > P ? (cost[i] + P - 1) / P : 1)
                     : (c0[i] + cost[i] - 1) / P - (c0[i] + ovh) / P + 1;
      } else {
        k[i] = 0;
      }
      mine.x += k[i];
      mine.y += k[i] > 1 ? k[i] : 0;
      mine.z += k[i] > 1 ? 1 : 0;
    }
    for (int q = tid; q <= max_parts; q += NT) s_cnt[q] = 0;
    if (snake)
      for (int i = tid; i < (4 * NT); i += NT) s_bucket[i] = 0;
    int3 tot3;
    const int3 ex3 = block_exclusive_scan3<NT>(mine, s_wave, &tot3);  // also orders the zeroing
    const int nitems = tot3.x;
    const int parts = snake ? min(max_parts, nitems) : (total + P - 1) / P;
    int shift = 0;
    while ((cmax >> shift) >= (4 * NT)) ++shift;
    int ib = ex3.x, rb = ex3.y, sb = ex3.z;
    int ibase[4], rbase[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int b = 4 * tid + i;
      ibase[i] = ib;
      rbase[i] = rb;
      if (b < batch) {
        cum[b] = c0[i];
        if (k[i] > 1) split[sb++] = make_int4(b, rb, k[i], 0);
        if (!snake) {
          const int ub = c0[i] + ovh, ue = c0[i] + cost[i];
          const int first = ub / P;
          for (int j = 0; j < k[i]; ++j) {
            const int q = first + j;
            const int p0 = max(ub, q * P), p1 = min(ue, (q + 1) * P);
            work[ib + j] = make_int4(b, p0 - ub, p1 - ub, k[i] > 1 ? rb + j : -1);
            atomicAdd(&s_cnt[q], 1);
          }
        } else {
          // Piece lengths: q + 1 (first r pieces) and q.
          const int q = units[i] / k[i], r = units[i] - q * k[i];
          if (r > 0) atomicAdd(&s_bucket[(ovh + q + 1) >> shift], r);
          if (k[i] > r) atomicAdd(&s_bucket[(ovh + q) >> shift], k[i] - r);
        }
      }
      ib += k[i];
      rb += k[i] > 1 ? k[i] : 0;
    }
    __syncthreads();
    if (snake) {
      // Rank base of each cost bucket, largest first.
      {
        int v[4], sum = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[i] = s_bucket[(4 * NT) - 1 - (4 * tid + i)];
          sum += v[i];
        }
        int tot;
        int ex = block_exclusive_scan<NT>(sum, s_wave, &tot);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          s_bucket[(4 * NT) - 1 - (4 * tid + i)] = ex;
          ex += v[i];
        }
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (k[i] == 0) continue;  // slot past the batch
        const int q = units[i] / k[i], r = units[i] - q * k[i];
        for (int j = 0; j < k[i]; ++j) {
          const int len = q + (j < r ? 1 : 0);
          const int rank = atomicAdd(&s_bucket[(ovh + len) >> shift], 1);
          const int round = rank / parts, pos = rank - round * parts;
          const int q = (round & 1) ? parts - 1 - pos : pos;
          s_pq[ibase[i] + j] = short(q);
          atomicAdd(&s_cnt[q], 1);
        }
      }
      __syncthreads();
    }
    block_scan_lds<NT>(s_cnt, max_parts + 1, s_wave);
    for (int q = tid; q <= max_parts; q += NT) part_ptr[q] = s_cnt[q];
    __syncthreads();
    if (snake) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int b = 4 * tid + i;
        for (int j = 0; j < k[i]; ++j) {
          const int pos = atomicAdd(&s_cnt[s_pq[ibase[i] + j]], 1);
          work[pos] = make_int4(b, piece_start(j, units[i], k[i]),
                                piece_start(j + 1, units[i], k[i]), k[i] > 1 ? rbase[i] + j : -1);
        }
      }
    }
    if (tid == 0) {
      cum[batch] = total;
      header[0] = parts;
      header[1] = P;
      header[2] = tot3.z;
      header[3] = snake ? kPlanSnake : kPlanContiguous;
    }
    return;
  }
  // Large batches: contiguous plan over the requests in chunks of
  // NT (costs re-read per pass).
  auto cost_of = [&](int b) {
    return ovh + units_of(clamp_len(seq_lens[b], cap_tokens));
  };
  int carry = 0;
  for (int base = 0; base < batch; base += NT) {
    const int b = base + tid;
    const int cost = b < batch ? cost_of(b) : 0;
    int tot;
    const int ex = block_exclusive_scan<NT>(cost, s_wave, &tot);
    if (b < batch) cum[b] = carry + ex;
    carry += tot;
  }
  const int total = carry;
  int P = (total + max_parts - 1) / max_parts;
  if (P < kMinPartUnits) P = kMinPartUnits;
  const int parts = (total + P - 1) / P;
  for (int q = tid; q <= max_parts; q += NT) s_cnt[q] = 0;
  __syncthreads();
  int3 carry3 = make_int3(0, 0, 0);
  for (int base = 0; base < batch; base += NT) {
    const int b = base + tid;
    int k = 0, c0 = 0, cost = 0;
    if (b < batch) {
      cost = cost_of(b);
      c0 = cum[b];
      k = (c0 + cost - 1) / P - (c0 + ovh) / P + 1;
    }
    int3 tot3;
    const int3 ex3 = block_exclusive_scan3<NT>(make_int3(k, k > 1 ? k : 0, k > 1 ? 1 : 0), s_wave,
                                           &tot3);
    if (b < batch) {
      const int ibase = carry3.x + ex3.x, rbase = carry3.y + ex3.y;
      if (k > 1) split[carry3.z + ex3.z] = make_int4(b, rbase, k, 0);
      const int ub = c0 + ovh, ue = c0 + cost;
      const int first = ub / P;
      for (int j = 0; j < k; ++j) {
        const int q = first + j;
        const int p0 = max(ub, q * P), p1 = min(ue, (q + 1) * P);
        work[ibase + j] = make_int4(b, p0 - ub, p1 - ub, k > 1 ? rbase + j : -1);
        atomicAdd(&s_cnt[q], 1);
      }
    }
    carry3.x += tot3.x;
    carry3.y += tot3.y;
    carry3.z += tot3.z;
  }
  __syncthreads();
  block_scan_lds<NT>(s_cnt, max_parts + 1, s_wave);
  for (int q = tid; q <= max_parts; q += NT) part_ptr[q] = s_cnt[q];
  if (tid == 0) {
    cum[batch] = total;
    header[0] = parts;
    header[1] = P;
    header[2] = carry3.z;
    header[3] = kPlanContiguous;
  }
}

// The snake plan of plan_kernel, worked out by every workgroup of the
// attention kernel itself (batches of at most kInlineSnakeBatch requests),
// so that no plan kernel runs. Every workgroup must derive the same plan, so
// the ranking is deterministic: pieces are ordered by an 8-bit cost bucket,
// largest first, ties in piece order (a stable LSD radix sort of one bit per
// pass), where plan_kernel ranks equal costs in atomic order. Scratch lives
// in `scr` (the attention kernel's still-empty LDS ring). The partition-0
// workgroups write split and header for the combine. This
// partition's items (in rank order) land in items[0..*n_items).
// Ints of LDS the plans may use before the ring fills: the four-stage ring
// of 36,864-byte tiles (checked where the ring is declared).
constexpr int kPlanScratchInts = 4 * 36864 / 4;

template <int NT>
__device__ void inline_snake_plan(const AttnArgs& a, int part, int* scr, int4* items,
                                  int* n_items) {
  const int ovh = a.plan_ovh;
  __shared__ int s_wave[48];
  constexpr int kMaxPieces = kInlineSnakeBatch + kMaxPlanParts;
  const int tid = threadIdx.x;
  const int B = a.batch;
  int* units = scr;                           // [B]
  int* kb = units + B;                        // [B] pieces per request
  int* pk = kb + B;                           // [B + 1] first piece of each request
  int* rb = pk + B + 1;                       // [B + 1] first partial row
  int* preq = rb + B + 1;                     // [N] request of each piece
  int* keyA = preq + kMaxPieces;              // [N] sort key of each piece
  int* keyB = keyA + kMaxPieces;              // per-wave key histograms
  int* idxB = keyB + kMaxPieces;              // [N] pieces by rank
  // Units and costs; their total and maximum. Every length this thread needs
  // is requested before the first is used (one round trip, not one per
  // request).
  constexpr int kLensPerThread = (kInlineSnakeBatch + NT - 1) / NT;
  int lens[kLensPerThread];
#pragma unroll
  for (int i = 0; i < kLensPerThread; ++i) {
    const int b = tid + i * NT;
    lens[i] = b < B ? a.seq_lens[b] : 0;
  }
  int csum = 0, cmax = 0;
#pragma unroll
  for (int i = 0; i < kLensPerThread; ++i) {
    const int b = tid + i * NT;
    if (b < B) {
      const int u = units_of(clamp_len(lens[i], a.cap_tokens));
      units[b] = u;
      csum += ovh + u;
      cmax = max(cmax, ovh + u);
    }
  }
  const int2 sm = block_sum_max<NT>(csum, cmax, s_wave);  // also orders the units[] stores
  const int tot = sm.x;
  cmax = sm.y;
  int P = (tot + a.parts_cap - 1) / a.parts_cap;
  if (P < kMinPartUnits) P = kMinPartUnits;
  int shift = 0;
  while ((cmax >> shift) > 255) ++shift;
  int N, n_split = 0;
  if (cmax <= P) {
    // No request costs more than the target, so none is cut: piece b is
    // request b and no partial row exists.
    N = B;
#pragma unroll
    for (int i = 0; i < kLensPerThread; ++i) {
      const int b = tid + i * NT;
      if (b < B) {
        const int u = units_of(clamp_len(lens[i], a.cap_tokens));
        kb[b] = 1;
        pk[b] = b;
        rb[b] = 0;
        keyA[b] = 255 - min(255, (ovh + u) >> shift);
        preq[b] = b;
      }
    }
  } else {
    // Pieces per request (requests above the target are cut) and the bases
    // of pieces, partial rows and split requests, over contiguous chunks.
    const int C = (B + NT - 1) / NT;
    const int b0 = min(B, tid * C), b1 = min(B, b0 + C);
    int3 mine = make_int3(0, 0, 0);
    for (int b = b0; b < b1; ++b) {
      const int cost = ovh + units[b];
      const int k = cost > P ? (cost + P - 1) / P : 1;
      kb[b] = k;
      mine.x += k;
      mine.y += k > 1 ? k : 0;
      mine.z += k > 1 ? 1 : 0;
    }
    int3 tot3;
    int3 ex3 = block_exclusive_scan3<NT>(mine, s_wave, &tot3);
    N = tot3.x;
    n_split = tot3.z;
    for (int b = b0; b < b1; ++b) {
      const int k = kb[b];
      pk[b] = ex3.x;
      rb[b] = ex3.y;
      if (part == 0 && k > 1) a.wr_split[ex3.z] = make_int4(b, ex3.y, k, 0);
      const int q = units[b] / k, r = units[b] - q * k;
      for (int j = 0; j < k; ++j) {
        const int len = q + (j < r ? 1 : 0);
        keyA[ex3.x + j] = 255 - min(255, (ovh + len) >> shift);
        preq[ex3.x + j] = b;
      }
      ex3.x += k;
      ex3.y += k > 1 ? k : 0;
      ex3.z += k > 1 ? 1 : 0;
    }
  }
  const int parts = min(a.parts_cap, N);
  if (part == 0 && tid == 0) {
    a.wr_header[0] = parts;
    a.wr_header[1] = P;
    a.wr_header[2] = n_split;
    a.wr_header[3] = kPlanSnake;
  }
  __syncthreads();
  // Stable counting sort of the pieces by their 8-bit keys, in one pass.
  // Wave w owns a contiguous chunk of pieces and counts its keys into
  // hist[w][key]; one scan over keys and waves turns the counts into the
  // first output slot of each (wave, key). A second walk, 64 pieces at a
  // time, scatters: the lanes holding equal keys in a batch find each other
  // with eight ballots (one per key bit), which ranks them among themselves
  // in lane order. Every workgroup reaches the same permutation (the stable
  // order is unique).
  constexpr int kW = NT / 64;
  int* hist = keyB;        // [kW][256]
  int* order = idxB;       // [N] pieces by rank
  static_assert(4 * kInlineSnakeBatch + 2 + 4 * kMaxPieces <= kPlanScratchInts,
                "snake plan scratch exceeds the ring");
  static_assert(kW * 256 <= kMaxPieces && NT >= 256, "histogram layout");
  const int lane = tid & 63, wave = tid >> 6;
  const int chunk = (N + kW - 1) / kW;
  const int c0 = min(N, wave * chunk), c1 = min(N, c0 + chunk);
  for (int k = lane; k < 256; k += 64) hist[wave * 256 + k] = 0;
  // Lanes of the batch with this lane's key (all 64 lanes take part in the
  // ballots; lanes past the chunk are masked out).
  auto peers = [&](int key, bool live) -> uint64_t {
    uint64_t m = __ballot(live);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      const uint64_t ones = __ballot(live && ((key >> bit) & 1));
      m &= ((key >> bit) & 1) ? ones : ~ones;
    }
    return m;
  };
  const uint64_t below = (uint64_t(1) << lane) - 1;
  // Counts only: LDS atomic adds (the totals do not depend on their order).
  for (int e = c0 + lane; e < c1; e += 64) atomicAdd(&hist[wave * 256 + keyA[e]], 1);
  __syncthreads();
  // Slot bases: keys in ascending order, waves in order within a key.
  {
    int tot = 0;
    int h[kW];
    if (tid < 256) {
#pragma unroll
      for (int w = 0; w < kW; ++w) {
        h[w] = hist[w * 256 + tid];
        tot += h[w];
      }
    }
    int all;
    int base = block_exclusive_scan<NT>(tid < 256 ? tot : 0, s_wave, &all);
    if (tid < 256) {
#pragma unroll
      for (int w = 0; w < kW; ++w) {
        hist[w * 256 + tid] = base;
        base += h[w];
      }
    }
  }
  __syncthreads();
  for (int e = c0; e < c1; e += 64) {
    const bool live = e + lane < c1;
    const int key = live ? keyA[e + lane] : 0;
    const uint64_t m = peers(key, live);
    if (live) order[hist[wave * 256 + key] + __popcll(m & below)] = e + lane;
    // The key's first lane moves the base past this batch (after every lane
    // of the wave has read it: a wave's LDS operations run in order).
    if (live && (m & below) == 0) hist[wave * 256 + key] += __popcll(m);
  }
  __syncthreads();
  const int* iin = order;
  // This partition's pieces: ranks r * parts + (r odd ? parts - 1 - part : part).
  if (tid < 64) {
    const int r = tid;
    const int i = r * parts + ((r & 1) ? parts - 1 - part : part);
    const bool live = part < parts && i < N;
    const uint64_t m = __ballot(live);
    if (live) {
      const int p = iin[i];
      const int b = preq[p];
      const int j = p - pk[b];
      const int k = kb[b];
      items[r] = make_int4(b, piece_start(j, units[b], k), piece_start(j + 1, units[b], k),
                           k > 1 ? rb[b] + j : -1);
    }
    if (tid == 0) *n_items = __popcll(m);
  }
  __syncthreads();
}

// The contiguous plan of plan_kernel, worked out by every workgroup of the
// attention kernel (kInlinePlanBatch < batch <= kInlineContigBatch): costs
// laid end to end, cut into partitions of P units. A partition's pieces are
// one run of consecutive requests, so the workgroup keeps only where its run
// starts (request, its cost prefix and its first partial row) and walks it.
// Partition 0 writes split and header for the combine. `scr` is the
// still-empty LDS ring.
struct ContigWalk {
  int b, cum, rb, P, parts;
};

template <int NT>
__device__ void inline_contiguous_plan(const AttnArgs& a, int part, int* scr, ContigWalk* walk) {
  const int ovh = a.plan_ovh;
  __shared__ int s_wave[48];
  const int tid = threadIdx.x;
  const int B = a.batch;
  int* cost = scr;  // [B]
  const int C = (B + NT - 1) / NT;
  const int b0 = min(B, tid * C), b1 = min(B, b0 + C);
  int csum = 0;
  for (int b = b0; b < b1; ++b) {
    cost[b] = ovh + units_of(clamp_len(a.seq_lens[b], a.cap_tokens));
    csum += cost[b];
  }
  int total;
  const int cex = block_exclusive_scan<NT>(csum, s_wave, &total);
  int P = (total + a.parts_cap - 1) / a.parts_cap;
  if (P < kMinPartUnits) P = kMinPartUnits;
  const int parts = (total + P - 1) / P;
  // Pieces per request and the bases of partial rows and split requests.
  int c0 = cex;
  int3 mine = make_int3(0, 0, 0);
  for (int b = b0; b < b1; ++b) {
    const int ub = c0 + ovh, ue = c0 + cost[b];
    const int k = (ue - 1) / P - ub / P + 1;
    mine.y += k > 1 ? k : 0;
    mine.z += k > 1 ? 1 : 0;
    c0 = ue;
  }
  int3 tot3;
  const int3 ex3 = block_exclusive_scan3<NT>(mine, s_wave, &tot3);
  c0 = cex;
  int rb = ex3.y, sb = ex3.z;
  const int lo = part * P;
  for (int b = b0; b < b1; ++b) {
    const int ub = c0 + ovh, ue = c0 + cost[b];
    const int k = (ue - 1) / P - ub / P + 1;
    // The first request reaching into this partition starts the walk.
    if (part < parts && ue > lo && c0 <= lo) *walk = ContigWalk{b, c0, rb, P, parts};
    if (part == 0 && k > 1) a.wr_split[sb] = make_int4(b, rb, k, 0);
    rb += k > 1 ? k : 0;
    sb += k > 1 ? 1 : 0;
    c0 = ue;
  }
  if (part == 0 && tid == 0) {
    a.wr_header[0] = parts;
    a.wr_header[1] = P;
    a.wr_header[2] = tot3.z;
    a.wr_header[3] = kPlanContiguous;
  }
  if (tid == 0 && part >= parts) *walk = ContigWalk{B, 0, 0, P, parts};
  __syncthreads();
}

// Partition -> work items. Calls fn(b, u0, u1, row) for every piece of
// partition `part`: units [u0, u1) of request b, written as the final output
// when row < 0, else as partial row `row`. Uniform across the workgroup.
template <int NT, typename Fn>
__device__ __forceinline__ void for_each_piece(const AttnArgs& a, int part, int* scratch,
                                               Fn&& fn) {
  const int ovh = a.plan_ovh;
  // The item list of the four modes, then one loop with the only call of
  // fn (the whole attention body is inlined there).
  __shared__ int4 s_items[kInlinePlanBatch];
  __shared__ int s_nitems;
  __shared__ ContigWalk s_walk;
  int n = 0, i0 = 0;
  // Wide contiguous plan: this partition's run of requests (uniform across
  // the workgroup), walked from its first request.
  const bool walk = a.inline_plan == kInlineContiguousWide;
  int wb = 0, wcum = 0, wrb = 0, wP = 1;
  if (walk) {
    inline_contiguous_plan<NT>(a, part, scratch, &s_walk);
    wb = __builtin_amdgcn_readfirstlane(s_walk.b);
    wcum = __builtin_amdgcn_readfirstlane(s_walk.cum);
    wrb = __builtin_amdgcn_readfirstlane(s_walk.rb);
    wP = __builtin_amdgcn_readfirstlane(s_walk.P);
    n = a.batch;  // at most one piece per request of the run
  } else if (a.inline_plan == kInlineSnake) {
    inline_snake_plan<NT>(a, part, scratch, s_items, &s_nitems);
    n = __builtin_amdgcn_readfirstlane(s_nitems);
  } else if (a.num_splits > 0) {
    // Forced split k of request b; an empty split still writes its
    // (zero, -inf) partial because the combine reads every row.
    n = part < a.batch * a.num_splits ? 1 : 0;
  } else if (a.inline_plan == kInlineContiguous) {
    // The contiguous plan of plan_kernel, worked out by the first wave from
    // seq_lens (request = lane): costs, their prefix, the per-partition
    // target P, the pieces k of each request and the partial rows of split
    // requests. This partition's pieces go to LDS in request order.
    if (threadIdx.x < 64) {
      const int lane = threadIdx.x;
      const bool live = lane < a.batch;
      const int units = live ? units_of(clamp_len(a.seq_lens[lane], a.cap_tokens)) : 0;
      const int cost = live ? ovh + units : 0;
      const int cinc = wave_inclusive_scan(cost);
      const int total = __builtin_amdgcn_readlane(cinc, 63);
      int P = (total + a.parts_cap - 1) / a.parts_cap;
      // Few and short requests (pieces of kMinPartUnits would keep under a
      // quarter of the partitions busy) take smaller pieces: such a call is
      // bound by each piece's latency, not by its bytes.
      const int pmin =
          4 * total < a.parts_cap * kMinPartUnits ? kMinPartUnitsFew : kMinPartUnits;
      if (P < pmin) P = pmin;
      const int ub = cinc - cost + ovh, ue = cinc;
      // Requests of equal length whose count divides the partitions: each is
      // cut into S = partitions / batch equal pieces, one partition each, so
      // that the cuts fall on request boundaries. (The cut at multiples of P
      // would give most of them a third, small piece: one more partial row
      // and one more piece start per workgroup.)
      const int c0 = __builtin_amdgcn_readlane(cost, 0);
      const int cv = live ? cost : c0;
      const int S = a.parts_cap / a.batch;
      const bool aligned = wave_max(cv) == -wave_max(-cv) && a.parts_cap % a.batch == 0 &&
                           S >= 2 && c0 - ovh >= S * kMinPartUnits;
      const int first = aligned ? lane * S : ub / P;
      const int k = live ? (aligned ? S : (ue - 1) / P - first + 1) : 0;
      const int nrows = k > 1 ? k : 0;
      const int rinc = wave_inclusive_scan(nrows);
      const int sinc = wave_inclusive_scan(k > 1 ? 1 : 0);
      if (part == 0) {
        // Same values from every partition-0 workgroup (one per head tile).
        if (live && k > 1) a.wr_split[sinc - 1] = make_int4(lane, rinc - nrows, k, 0);
        if (lane == 0) {
          a.wr_header[0] = aligned ? a.batch * S : (total + P - 1) / P;
          a.wr_header[1] = aligned ? (c0 - ovh + S - 1) / S : P;
          a.wr_header[2] = __builtin_amdgcn_readlane(sinc, 63);
          a.wr_header[3] = kPlanContiguous;
        }
      }
      const bool mine = part < a.parts_cap && live && first <= part && part < first + k;
      const uint64_t m = __ballot(mine);
      if (mine) {
        const int idx = __builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32),
                                                  __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0));
        int u0, u1;
        if (aligned) {
          const int j = part - first;
          u0 = int((long long)j * units / S);
          u1 = int((long long)(j + 1) * units / S);
        } else {
          u0 = max(ub, part * P) - ub;
          u1 = min(ue, (part + 1) * P) - ub;
        }
        s_items[idx] = make_int4(lane, u0, u1, k > 1 ? rinc - nrows + part - first : -1);
      }
      if (lane == 0) s_nitems = __popcll(m);
    }
    __syncthreads();
    n = __builtin_amdgcn_readfirstlane(s_nitems);
  } else if (part < a.parts_cap) {
    i0 = max(a.part_ptr[part], 0);
    n = min(a.part_ptr[part + 1], a.items_cap) - i0;
  }
  for (int i = 0; i < n; ++i) {
    int b, u0, u1, row;
    if (walk) {
      const int lo = part * wP, hi = lo + wP;
      const int ub = wcum + ovh;
      if (wb >= a.batch || ub >= hi) break;
      const int ue = wcum + ovh +
                     units_of(clamp_len(scalar_load_i32(a.seq_lens + wb), a.cap_tokens));
      const int first = ub / wP;
      const int k = (ue - 1) / wP - first + 1;
      b = wb;
      u0 = max(ub, lo) - ub;
      u1 = min(ue, hi) - ub;
      row = k > 1 ? wrb + (part - first) : -1;
      wrb += k > 1 ? k : 0;
      wcum = ue;
      ++wb;
    } else if (a.num_splits > 0) {
      const int S = a.num_splits;
      b = part / S;
      const int k = part - b * S;
      const int nu = (clamp_len(a.seq_lens[b], a.cap_tokens) + kUnit - 1) / kUnit;
      u0 = int((long long)k * nu / S);
      u1 = int((long long)(k + 1) * nu / S);
      row = S > 1 ? part : -1;
    } else {
      const int4 it = a.inline_plan ? s_items[i] : a.work[i0 + i];
      b = __builtin_amdgcn_readfirstlane(it.x);
      u0 = __builtin_amdgcn_readfirstlane(it.y);
      u1 = __builtin_amdgcn_readfirstlane(it.z);
      row = __builtin_amdgcn_readfirstlane(it.w);
    }
    // Items that would address outside the buffers are skipped (never
    // produced by a plan; a guard against a corrupted workspace).
    if (unsigned(b) >= unsigned(a.batch) || u0 < 0 || u1 < u0 || row >= a.rows_cap) continue;
    fn(b, u0, u1, row);
  }
}

// ----------------------------------------------------------------------------
// Tile-streaming attention (bf16 cache, one 16-head tile per workgroup).
//
// The four waves share every KV tile: 32 tokens (two 16-token units, each in
// one page) are copied HBM -> LDS with coalesced direct-to-LDS loads into a
// ring of kStages stages, kept kStages - 2 tiles ahead of the tile being
// consumed, so that the bytes in flight live in LDS rather than registers.
// Every wave computes the same 16 x 32 logit tile and softmax (q in
// registers, K from LDS) and owns 128 of the 512 output features for P.V, so
// no cross-wave merge is needed. The ring's waits are explicit: each thread
// issues kDmaPerThread loads per tile and no other vector-memory operation
// inside the loop, so "tile j landed" is vmcnt <= kDmaPerThread * (tiles
// issued after j). LDS reads are issued as ds_read_b128 statements followed
// by an explicit lgkmcnt wait that the results pass through.
//
// LDS tile layout: row t (token) holds 72 sixteen-byte chunks; chunk ch of
// row t sits in slot ch ^ (t & 7), so that 8 rows read at the same chunk, or
// 8 consecutive chunks of one row, hit 8 different 4-bank groups.

constexpr int kTile = 2 * kUnit;                      // tokens per LDS tile
constexpr int kStages = 4;                            // LDS ring depth
constexpr int kRowChunks = kRowBytes / 16;            // 72 chunks per cached row
constexpr int kTileBytesBf16 = kTile * kRowBytes;     // 36864
static_assert(kStages * kTileBytesBf16 == 4 * kPlanScratchInts, "plan scratch is the ring");
constexpr int kDmaPerThread = kTile * kRowChunks / kThreads;  // 9
static_assert(kTile * kRowChunks == kDmaPerThread * kThreads, "tile must split evenly");

// Cache policy of the ring's loads: the non-temporal (nt) bit. A cache row is
// read once per call (one head group) or twice within microseconds (two head
// groups on the same XCD), so it is streamed rather than kept. Measured at
// batch 512 x 16 heads: 219.6 -> 197.3 us per attention launch (6.2 TB/s of
// algorithmic bytes); 128 heads gain 1-3 %.
constexpr int kRingLoadPolicy = 2;

template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Wait until at most `after` (clamped to MAX) later tiles' loads are pending.
template <int MAX>
__device__ __forceinline__ void wait_ring(int after) {
  if constexpr (MAX == 0) {
    wait_vmem<0>();
  } else {
    if (after >= MAX)
      wait_vmem<MAX * kDmaPerThread>();
    else
      wait_ring<MAX - 1>(after);
  }
}

__device__ __forceinline__ void wave_barrier_all() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// LDS reads of one operand set, issued and completed inside one asm
// statement (no copy of a destination register can be scheduled between the
// read and its wait).
#define MLA_DSR(i, base, off) "ds_read_b128 %" #i ", %" #base " offset:" #off "\n\t"

// K operand of one 16-token unit: chunk 2k of row t at a_even + 128 k, chunk
// 2k + 1 at a_odd + 128 k (the XOR swizzle folded into the two bases).
__device__ __forceinline__ void lds_read_k(uint32_t a_even, uint32_t a_odd,
                                           u32x4_t (&kf)[kQChunks]) {
  asm volatile(
      MLA_DSR(0, 18, 0) MLA_DSR(1, 19, 0) MLA_DSR(2, 18, 128) MLA_DSR(3, 19, 128)
      MLA_DSR(4, 18, 256) MLA_DSR(5, 19, 256) MLA_DSR(6, 18, 384) MLA_DSR(7, 19, 384)
      MLA_DSR(8, 18, 512) MLA_DSR(9, 19, 512) MLA_DSR(10, 18, 640) MLA_DSR(11, 19, 640)
      MLA_DSR(12, 18, 768) MLA_DSR(13, 19, 768) MLA_DSR(14, 18, 896) MLA_DSR(15, 19, 896)
      MLA_DSR(16, 18, 1024) MLA_DSR(17, 19, 1024) "s_waitcnt lgkmcnt(0)"
      : "=&v"(kf[0]), "=&v"(kf[1]), "=&v"(kf[2]), "=&v"(kf[3]), "=&v"(kf[4]), "=&v"(kf[5]),
        "=&v"(kf[6]), "=&v"(kf[7]), "=&v"(kf[8]), "=&v"(kf[9]), "=&v"(kf[10]), "=&v"(kf[11]),
        "=&v"(kf[12]), "=&v"(kf[13]), "=&v"(kf[14]), "=&v"(kf[15]), "=&v"(kf[16]),
        "=&v"(kf[17])
      : "v"(a_even), "v"(a_odd)
      : "memory");
}

// Eight V rows (16 bytes each) at eight addresses.
__device__ __forceinline__ void lds_read_v8(const uint32_t (&ad)[8], u32x4_t (&v)[8]) {
  asm volatile(
      MLA_DSR(0, 8, 0) MLA_DSR(1, 9, 0) MLA_DSR(2, 10, 0) MLA_DSR(3, 11, 0) MLA_DSR(4, 12, 0)
      MLA_DSR(5, 13, 0) MLA_DSR(6, 14, 0) MLA_DSR(7, 15, 0) "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]),
        "=&v"(v[6]), "=&v"(v[7])
      : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]),
        "v"(ad[7])
      : "memory");
}

// Eight transposing LDS reads (ds_read_b64_tr_b16): for n' = 0..3 and token
// halves h = 0, 1, read n' at vb[n'] + 128 M + 18432 h (one 16-token unit is
// 16 rows of 1152 bytes). Within each 16-lane group, lane 4 a + b receives
// element b of the 8-byte words addressed by lanes a, a + 4, a + 8, a + 12.
#define MLA_DSTR(i, base, off) "ds_read_b64_tr_b16 %" #i ", %" #base " offset:" #off "\n\t"
#define MLA_TR8(o0, o1)                                                                  \
  asm volatile(MLA_DSTR(0, 8, o0) MLA_DSTR(1, 8, o1) MLA_DSTR(2, 9, o0) MLA_DSTR(3, 9, o1) \
               MLA_DSTR(4, 10, o0) MLA_DSTR(5, 10, o1) MLA_DSTR(6, 11, o0)               \
               MLA_DSTR(7, 11, o1) "s_waitcnt lgkmcnt(0)"                                 \
               : "=&v"(t[0][0]), "=&v"(t[0][1]), "=&v"(t[1][0]), "=&v"(t[1][1]),          \
                 "=&v"(t[2][0]), "=&v"(t[2][1]), "=&v"(t[3][0]), "=&v"(t[3][1])           \
               : "v"(vb[0]), "v"(vb[1]), "v"(vb[2]), "v"(vb[3])                           \
               : "memory")

template <int M>
__device__ __forceinline__ void lds_read_tr8(const uint32_t (&vb)[4], u32x2_t (&t)[4][2]) {
  static_assert(M >= 0 && M < 8, "feature group");
  if constexpr (M == 0) MLA_TR8(0, 18432);
  else if constexpr (M == 1) MLA_TR8(128, 18560);
  else if constexpr (M == 2) MLA_TR8(256, 18688);
  else if constexpr (M == 3) MLA_TR8(384, 18816);
  else if constexpr (M == 4) MLA_TR8(512, 18944);
  else if constexpr (M == 5) MLA_TR8(640, 19072);
  else if constexpr (M == 6) MLA_TR8(768, 19200);
  else MLA_TR8(896, 19328);
}
#undef MLA_TR8
#undef MLA_DSTR


// Wave-specialised variant of the tile stream. Waves 0..3 issue the ring's
// loads and own 128 output features each for P.V; wave 4 (the logit wave)
// computes the 16 x 32 logit tile, the online softmax and P for tile s while
// the P.V waves consume tile s - 1. P (already in the A-operand layout), the
// frame-rescale factors and a rescale flag pass through double-buffered LDS
// slots; one barrier per step. Ring: at step s the P.V waves read tile
// s - 1, the logit wave tile s, tiles s + 1 and s + 2 are in flight.
constexpr int kPvWaves = 4;
constexpr int kWsThreads = 64 * (kPvWaves + 1);

__device__ __forceinline__ void wave_barrier_lds() {
  // LDS writes of this wave complete before anyone passes the barrier.
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  wave_barrier_all();
}

__global__ void __launch_bounds__(kWsThreads, 1) attn_ws_kernel(AttnArgs a) {
  __shared__ uint8_t ring[kStages][kTileBytesBf16];
  __shared__ u32x4_t pbuf[2][64];          // P of the step's tile, one A operand per lane
  __shared__ float abuf[2][kHeadTile];     // frame rescale factor per head
  __shared__ int fbuf[2];                  // 1: rescale the accumulators first
  __shared__ float lbuf[kHeadTile];        // final softmax denominators

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int c = lane & 15, g = lane >> 4;
  const bool logit_wave = wave == kPvWaves;
  const int H = a.rows;

  const int lin = blockIdx.x;
  const int xcd = lin & 7, slot = lin >> 3;
  const int ht = slot % a.head_tiles;
  const int part = (slot / a.head_tiles) * 8 + xcd;
  const int h0 = ht * kHeadTile;
  // Logit wave: row h0 + c belongs to query token (h0 + c) / heads, which sees
  // all but the last `back` tokens of the request.
  const int back = a.q_len - 1 - min(h0 + c, H - 1) / a.heads;

  // Per-thread DMA map of the P.V waves: load i fills ring slot i * 256 + tid.
  uint32_t dma_off[kDmaPerThread];
  uint32_t dma_hi = 0;
#pragma unroll
  for (int i = 0; i < kDmaPerThread; ++i) {
    const int pos = i * kThreads + (tid & (kThreads - 1));
    const int t = pos / kRowChunks, sl = pos - (pos / kRowChunks) * kRowChunks;
    const int ch = sl ^ (t & 7);
    dma_off[i] = uint32_t((t & 15) * kRowBytes + ch * 16);
    dma_hi |= uint32_t(t >> 4) << i;
  }
  const uint32_t ring_lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (void __attribute__((address_space(3)))*)(&ring[0][0])));
  const int bs_mask = (1 << a.bs_log2) - 1;

  for_each_piece<kWsThreads>(a, part, reinterpret_cast<int*>(&ring[0][0]),
                             [&](int b, int u0, int u1, int out_row) {
    const int n = checked_len(a.seq_lens[b], a.cap_tokens, a.err_word);
    const int u_end = min(u1, (n + kUnit - 1) / kUnit);
    const int ntiles = u_end > u0 ? (u_end - u0 + 1) / 2 : 0;
    const int32_t* bt_row = a.block_table + size_t(b) * a.max_blocks;
    // Tokens of tile k's two units.
    auto tile_nv = [&](int k, int (&nv)[2]) {
      const int t0 = (u0 + 2 * k) * kUnit;
      nv[0] = min(kUnit, n - t0);
      nv[1] = u0 + 2 * k + 1 < u_end ? min(kUnit, n - t0 - kUnit) : 0;
    };
    // Rows of unit u; a block id outside the cache is replaced by block 0.
    auto unit_rows = [&](int u, bool valid) -> const uint8_t* {
      const int t0 = u * kUnit;
      int blk = valid ? scalar_load_i32(bt_row + (t0 >> a.bs_log2)) : 0;
      if (blk < 0 || blk >= a.num_blocks) {
        report_bounds(a.err_word, kBoundsBadBlock);
        blk = 0;
      }
      return a.kv + (size_t(blk) * (size_t(1) << a.bs_log2) + size_t(t0 & bs_mask)) * kRowBytes;
    };
    auto issue_tile = [&](int k) {
      int nv[2];
      tile_nv(k, nv);
      // A second unit in the same page continues the first unit's rows:
      // no second block-table lookup (a scalar-load round trip).
      const int t0 = (u0 + 2 * k) * kUnit;
      const uint8_t* r0 = unit_rows(u0 + 2 * k, true);
      const uint8_t* r1 = r0;
      if (nv[1] > 0)
        r1 = ((t0 + kUnit) >> a.bs_log2) == (t0 >> a.bs_log2)
                 ? r0 + kUnit * kRowBytes
                 : unit_rows(u0 + 2 * k + 1, true);
      uint8_t* dst = &ring[k % kStages][0] + wave * 64 * 16;
#pragma unroll
      for (int i = 0; i < kDmaPerThread; ++i) {
        const uint8_t* src = ((dma_hi >> i) & 1 ? r1 : r0) + dma_off[i];
        __builtin_amdgcn_global_load_lds(
            src, (void __attribute__((address_space(3)))*)(dst + i * kThreads * 16), 16, 0,
            kRingLoadPolicy);
      }
    };

    wave_barrier_all();  // the ring and slots of the previous piece are free
    u32x4_t qf[kQChunks];
    if (logit_wave) {
      // q fragment: head h0 + c (padded heads repeat head H - 1), features
      // 32 s + 8 g .. + 7.
      const u32x4_t* qp =
          reinterpret_cast<const u32x4_t*>(a.q + (size_t(b) * H + min(h0 + c, H - 1)) * kDK) + g;
#pragma unroll
      for (int s2 = 0; s2 < kQChunks; ++s2) qf[s2] = qp[4 * s2];
      wait_vmem<0>();
    } else {
      for (int k = 0; k < 2 && k < ntiles; ++k) issue_tile(k);
    }

    f32x4_t acc[8];  // P.V waves: heads 4 g + r, features 128 wave + 8 c + i
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m_ref = -INFINITY;  // logit wave: accumulation frame of head c (log2 domain)
    float l_run = 0.f;        // logit wave: lane's share of head c's denominator

    for (int s = 0; s <= ntiles; ++s) {
      if (!logit_wave && s < ntiles) wait_ring<1>(ntiles - 1 - s);  // tile s landed
      wave_barrier_lds();
      if (logit_wave) {
        if (s < ntiles) {
          const uint32_t st = ring_lds + uint32_t(s % kStages) * kTileBytesBf16;
          int nv[2];
          tile_nv(s, nv);
          const int vis = n - back - (u0 + 2 * s) * kUnit;  // visible tokens of row c from here
          float x[2][4];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int nvh = min(nv[h], vis - h * kUnit);
            const int t = h * kUnit + c;
            const uint32_t y = uint32_t(g ^ (c & 7));
            const uint32_t row = st + uint32_t(t * kRowBytes);
            u32x4_t kf[kQChunks];
            lds_read_k(row + 16 * y, row + 16 * (y ^ 4), kf);
            f32x4_t sc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s2 = 0; s2 < kQChunks; ++s2)
              sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  __builtin_bit_cast(bf16x8_t, kf[s2]), __builtin_bit_cast(bf16x8_t, qf[s2]), sc,
                  0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r)
              x[h][r] = (4 * g + r < nvh) ? sc[r] * a.scale_log2 : -INFINITY;
          }
          float mt = fmaxf(fmaxf(fmaxf(x[0][0], x[0][1]), fmaxf(x[0][2], x[0][3])),
                           fmaxf(fmaxf(x[1][0], x[1][1]), fmaxf(x[1][2], x[1][3])));
          mt = fmaxf(mt, __shfl_xor(mt, 16));
          mt = fmaxf(mt, __shfl_xor(mt, 32));
          const bool move = __ballot(mt > m_ref + 8.f) != 0ull;  // wave-uniform
          if (move) {
            const float m_new = fmaxf(m_ref, mt);
            const float alpha = m_ref == -INFINITY ? 0.f : fast_exp2(m_ref - m_new);
            l_run *= alpha;
            m_ref = m_new;
            if (g == 0) abuf[s & 1][c] = alpha;
          }
          if (lane == 0) fbuf[s & 1] = move ? 1 : 0;
          const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
          float p[2][4];
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int r = 0; r < 4; ++r) p[h][r] = fast_exp2(x[h][r] - m_use);
          l_run += ((p[0][0] + p[0][1]) + (p[0][2] + p[0][3])) +
                   ((p[1][0] + p[1][1]) + (p[1][2] + p[1][3]));
          // A operand of P.V: k slots 8 g .. + 3 = unit 0 tokens 4 g + r,
          // 8 g + 4 .. + 7 = unit 1 tokens 4 g + r.
          bf16x8_t pa;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            pa[r] = (__bf16)p[0][r];
            pa[4 + r] = (__bf16)p[1][r];
          }
          pbuf[s & 1][lane] = __builtin_bit_cast(u32x4_t, pa);
        }
        if (s == ntiles - 1 || ntiles == 0) {
          float l_c = l_run + __shfl_xor(l_run, 16);
          l_c += __shfl_xor(l_c, 32);
          if (g == 0) {
            lbuf[c] = l_c;
            if (h0 + c < H) {
              const float lse_v = l_c > 0.f ? (m_ref + __log2f(l_c)) * kLn2 : -INFINITY;
              if (out_row < 0) {
                if (a.lse) a.lse[size_t(b) * H + h0 + c] = lse_v;
              } else {
                a.part_lse[size_t(out_row) * H + h0 + c] = lse_v;
              }
            }
          }
        }
      } else {
        if (s + 2 < ntiles) issue_tile(s + 2);
        if (s >= 1) {
          const int k = s - 1;
          if (fbuf[k & 1]) {
            // acc <- diag(alpha) acc on the matrix cores: 4 fp32 MFMAs per
            // 16 x 16 block, k slot g of MFMA m carrying row 4 g + m.
            const float alpha = abuf[k & 1][c];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              f32x4_t z = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int m = 0; m < 4; ++m)
                z = __builtin_amdgcn_mfma_f32_16x16x4f32(c == 4 * g + m ? alpha : 0.f,
                                                          acc[i][m], z, 0, 0, 0);
              acc[i] = z;
            }
          }
          const bf16x8_t pa = __builtin_bit_cast(bf16x8_t, pbuf[k & 1][lane]);
          const uint32_t st = ring_lds + uint32_t(k % kStages) * kTileBytesBf16;
          int nv[2];
          tile_nv(k, nv);
          // V rows: tokens 16 h + 4 g + r, features 128 wave + 8 c .. + 7.
          u32x4_t vf[2][4];
          {
            uint32_t ad[8];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int t = h * kUnit + 4 * g + r;
                ad[4 * h + r] =
                    st + uint32_t(t * kRowBytes) + 16u * uint32_t(16 * wave + (c ^ (t & 7)));
              }
            }
            u32x4_t v8[8];
            lds_read_v8(ad, v8);
#pragma unroll
            for (int i = 0; i < 8; ++i) vf[i >> 2][i & 3] = v8[i];
          }
          // Masked tokens contribute exactly 0 even if their bytes are NaN.
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            if (nv[h] < kUnit) {
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const unsigned keep = (4 * g + r < nv[h]) ? 0xffffffffu : 0u;
                vf[h][r] &= keep;
              }
            }
          }
          // Feature 128 wave + 8 c + e of the 8 tokens as one B operand.
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const unsigned a0 = vf[0][0][i], a1 = vf[0][1][i], a2 = vf[0][2][i],
                           a3 = vf[0][3][i];
            const unsigned b0 = vf[1][0][i], b1 = vf[1][1][i], b2 = vf[1][2][i],
                           b3 = vf[1][3][i];
            const u32x4_t ve =
                u32x4_t{(a0 & 0xffffu) | (a1 << 16), (a2 & 0xffffu) | (a3 << 16),
                        (b0 & 0xffffu) | (b1 << 16), (b2 & 0xffffu) | (b3 << 16)};
            const u32x4_t vo =
                u32x4_t{(a0 >> 16) | (a1 & 0xffff0000u), (a2 >> 16) | (a3 & 0xffff0000u),
                        (b0 >> 16) | (b1 & 0xffff0000u), (b2 >> 16) | (b3 & 0xffff0000u)};
            acc[2 * i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                pa, __builtin_bit_cast(bf16x8_t, ve), acc[2 * i], 0, 0, 0);
            acc[2 * i + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                pa, __builtin_bit_cast(bf16x8_t, vo), acc[2 * i + 1], 0, 0, 0);
          }
        }
      }
    }
    wave_barrier_lds();  // lbuf is complete

    if (!logit_wave) {
      // Epilogue: heads 4 g + r, features 128 wave + 8 c .. + 7 in acc[0..7][r].
      const bool final_out = out_row < 0;
      const int row = final_out ? 0 : out_row;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int hh = 4 * g + r;
        const int h = h0 + hh;
        const float lh = lbuf[hh];
        const float inv = lh > 0.f ? 1.f / lh : 0.f;
        if (h < H) {
          const int d = 128 * wave + 8 * c;
          if (final_out) {
            u32x4_t pk;
#pragma unroll
            for (int e = 0; e < 4; ++e)
              pk[e] = unsigned(bf16_bits(acc[2 * e][r] * inv)) |
                      (unsigned(bf16_bits(acc[2 * e + 1][r] * inv)) << 16);
            *reinterpret_cast<u32x4_t*>(a.out + (size_t(b) * H + h) * kDV + d) = pk;
          } else {
            float* dst = a.part_out + (size_t(row) * H + h) * kDV + d;
            *reinterpret_cast<f32x4_t*>(dst) =
                f32x4_t{acc[0][r], acc[1][r], acc[2][r], acc[3][r]} * inv;
            *reinterpret_cast<f32x4_t*>(dst + 4) =
                f32x4_t{acc[4][r], acc[5][r], acc[6][r], acc[7][r]} * inv;
          }
        }
      }
    }
  });
}

// ----------------------------------------------------------------------------
// Frame of the many-head kernel: set from each head's first-tile maximum and
// never moved while weights 2^(x - frame) stay below 2^kHeadsSlack, so fp32
// accumulators cannot overflow. A head whose logits ever rise further makes
// the workgroup stream the piece a second time with the frame preset to the
// true maximum observed in the first pass (the first pass's sums of that
// head tile are discarded), so the accumulators are only ever cleared or
// updated by matrix ops.
constexpr float kHeadsSlack = 64.f;

// ----------------------------------------------------------------------------
// E4M3 cache: scaled 16x16x128 E4M3 matrix ops (used by attn_mh_kernel<1>).
//
// A tile is 64 tokens (four 16-token units) of 576-byte rows, 36,864 bytes as
// in the bf16 kernels, so ring, DMA map and waits are theirs. Chunk ch (16
// bytes) of row t sits in slot ch ^ fp8_swizzle(t), a permutation inside each
// aligned group of four chunks that keeps both read patterns below free of
// LDS bank conflicts.
//
// Logits: q is carried as its rounded E4M3 term and the term's residual,
// both in q's per-head scale amax / 448 (about 2^-8 relative error, as with
// bf16). One op covers 128 dimensions against q_hi and a second the same
// K bytes against q_lo; the last 64 dimensions fill one op with K's bytes
// twice against (q_hi, q_lo).
// P.V: one op covers the tile's 64 tokens twice. A holds P_hi and P_lo (the
// rounded weight times 2^8 and its E4M3 residual) of 16 tokens per lane
// group, B the same V bytes twice, read with ds_read_b64_tr_b8.
// Weights: each head keeps the frame m of its first tile for the whole piece.
// Per tile and head, e = ceil(tile max - m) (at least 0) moves into the op's
// per-lane E8M0 scale of A, so the stored weights 2^(x - m - e) never exceed
// 1 while the products carry 2^(x - m); the frame never has to move. As in
// the bf16 kernel, a head whose logits rise more than 64 above its frame
// makes the workgroup stream the piece again with the frame preset.
constexpr int kTileFp8 = 4 * kUnit;          // tokens per E4M3 tile
constexpr int kRowChunksFp8 = kDK / 16;      // 36
constexpr int kKChunksFp8 = kDK / 64;        // 9 logit ops per unit
static_assert(kTileFp8 * kDK == kTileBytesBf16, "E4M3 tile matches the bf16 tile size");
static_assert(kTileFp8 * kRowChunksFp8 == kDmaPerThread * kThreads, "tile must split evenly");

typedef int i32x8_t __attribute__((ext_vector_type(8)));

// Slot permutation of row t (measured free of bank conflicts for both the
// K reads and the transposing V reads; depends on bits 1, 2 and 4 of t only,
// so rows 32 apart and units of equal parity share it).
__device__ __forceinline__ int fp8_swizzle(int t) {
  return ((t >> 1) ^ ((t >> 4) & 1)) & 3;
}

// E4M3 encoding without range clamp (callers guarantee |x| <= 448).
__device__ __forceinline__ unsigned pack_e4m3x4_inrange(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return unsigned(w);
}

// The nine K chunks of one unit: base + OFF + 64 m, m = 0..8.
template <int OFF>
__device__ __forceinline__ void lds_read_k9(uint32_t base, u32x4_t (&kf)[kKChunksFp8]) {
  asm volatile(
      "ds_read_b128 %0, %9 offset:%10\n\t"
      "ds_read_b128 %1, %9 offset:%11\n\t"
      "ds_read_b128 %2, %9 offset:%12\n\t"
      "ds_read_b128 %3, %9 offset:%13\n\t"
      "ds_read_b128 %4, %9 offset:%14\n\t"
      "ds_read_b128 %5, %9 offset:%15\n\t"
      "ds_read_b128 %6, %9 offset:%16\n\t"
      "ds_read_b128 %7, %9 offset:%17\n\t"
      "ds_read_b128 %8, %9 offset:%18\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(kf[0]), "=&v"(kf[1]), "=&v"(kf[2]), "=&v"(kf[3]), "=&v"(kf[4]), "=&v"(kf[5]),
        "=&v"(kf[6]), "=&v"(kf[7]), "=&v"(kf[8])
      : "v"(base), "i"(OFF), "i"(OFF + 64), "i"(OFF + 128), "i"(OFF + 192), "i"(OFF + 256),
        "i"(OFF + 320), "i"(OFF + 384), "i"(OFF + 448), "i"(OFF + 512)
      : "memory");
}

// Eight transposing byte reads (ds_read_b64_tr_b8): for n' = 0..3 and row
// halves h = 0, 1, read (n', h) at vb[n'] + OFF + 18432 h (32 rows of 576
// bytes). Within each 16-lane group, lane 8 a + b receives byte b of the
// 8-byte words addressed by lanes a, a + 2, ..., a + 14.
template <int OFF>
__device__ __forceinline__ void lds_read_trb8(const uint32_t (&vb)[4], u32x2_t (&t)[4][2]) {
  asm volatile(
      "ds_read_b64_tr_b8 %0, %8 offset:%12\n\t"
      "ds_read_b64_tr_b8 %1, %8 offset:%13\n\t"
      "ds_read_b64_tr_b8 %2, %9 offset:%12\n\t"
      "ds_read_b64_tr_b8 %3, %9 offset:%13\n\t"
      "ds_read_b64_tr_b8 %4, %10 offset:%12\n\t"
      "ds_read_b64_tr_b8 %5, %10 offset:%13\n\t"
      "ds_read_b64_tr_b8 %6, %11 offset:%12\n\t"
      "ds_read_b64_tr_b8 %7, %11 offset:%13\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(t[0][0]), "=&v"(t[0][1]), "=&v"(t[1][0]), "=&v"(t[1][1]), "=&v"(t[2][0]),
        "=&v"(t[2][1]), "=&v"(t[3][0]), "=&v"(t[3][1])
      : "v"(vb[0]), "v"(vb[1]), "v"(vb[2]), "v"(vb[3]), "i"(OFF), "i"(OFF + 18432)
      : "memory");
}

// The four head tiles' E4M3 P operands (two 16-byte halves each, 2048
// bytes apart per tile) and E8M0 scales (64 bytes apart per tile) of one
// lane, read with an explicit wait (no wait on the ring's loads).
__device__ __forceinline__ void lds_read_p4(uint32_t p_addr, uint32_t e_addr, u32x4_t (&p)[4][2],
                                            int (&e)[4]) {
  asm volatile(
      "ds_read_b128 %0, %12 offset:0\n\t"
      "ds_read_b128 %1, %12 offset:16\n\t"
      "ds_read_b128 %2, %12 offset:2048\n\t"
      "ds_read_b128 %3, %12 offset:2064\n\t"
      "ds_read_b128 %4, %12 offset:4096\n\t"
      "ds_read_b128 %5, %12 offset:4112\n\t"
      "ds_read_b128 %6, %12 offset:6144\n\t"
      "ds_read_b128 %7, %12 offset:6160\n\t"
      "ds_read_b32 %8, %13 offset:0\n\t"
      "ds_read_b32 %9, %13 offset:64\n\t"
      "ds_read_b32 %10, %13 offset:128\n\t"
      "ds_read_b32 %11, %13 offset:192\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(p[0][0]), "=&v"(p[0][1]), "=&v"(p[1][0]), "=&v"(p[1][1]), "=&v"(p[2][0]),
        "=&v"(p[2][1]), "=&v"(p[3][0]), "=&v"(p[3][1]), "=&v"(e[0]), "=&v"(e[1]), "=&v"(e[2]),
        "=&v"(e[3])
      : "v"(p_addr), "v"(e_addr)
      : "memory");
}

// Nine LDS dword reads at per-lane addresses, with an explicit wait (no wait
// on the ring's loads in flight).
__device__ __forceinline__ void lds_read_ids9(const uint32_t (&ad)[9], int (&v)[9]) {
  asm volatile(
      "ds_read_b32 %0, %9\n\t"
      "ds_read_b32 %1, %10\n\t"
      "ds_read_b32 %2, %11\n\t"
      "ds_read_b32 %3, %12\n\t"
      "ds_read_b32 %4, %13\n\t"
      "ds_read_b32 %5, %14\n\t"
      "ds_read_b32 %6, %15\n\t"
      "ds_read_b32 %7, %16\n\t"
      "ds_read_b32 %8, %17\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]),
        "=&v"(v[6]), "=&v"(v[7]), "=&v"(v[8])
      : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]),
        "v"(ad[7]), "v"(ad[8])
      : "memory");
}

// Maximum over lanes c, c + 16, c + 32 and c + 48 (the four lane groups of
// a 16-column fragment) with gfx950's lane-swap moves, which stay in
// registers (no round trip through the LDS crossbar). One asm statement:
// the compiler folds max(swap results) of the builtins to the first result.
// Each swap reads a VGPR written by the instruction before it, so two wait
// states (s_nop 1) separate them, as the compiler places them itself.
__device__ __forceinline__ float max_over_lane_groups(float v) {
  float t;
  asm volatile(
      "v_mov_b32 %1, %0\n\t"
      "s_nop 1\n\t"
      "v_permlane32_swap_b32 %0, %1\n\t"
      "v_max_f32 %0, %0, %1\n\t"
      "v_mov_b32 %1, %0\n\t"
      "s_nop 1\n\t"
      "v_permlane16_swap_b32 %0, %1\n\t"
      "v_max_f32 %0, %0, %1"
      : "+v"(v), "=&v"(t));
  return v;
}

__device__ __forceinline__ f32x4_t mfma_e4m3_128(const i32x8_t& a, const i32x8_t& b,
                                                 const f32x4_t& c, int scale_a) {
  // Format code 0 = E4M3 for both operands; E8M0 scales (127 = 2^0).
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, scale_a, 0, 127);
}

// ----------------------------------------------------------------------------
// Many-head wave-specialised tile stream (more than 16 heads, or an E4M3
// cache): eight waves per workgroup, up to four 16-head tiles.
//
// Waves 4..7 are logit waves: wave 4 + t computes the logits and softmax of
// head tile t (q in registers, K from LDS) for tile s of the stream and
// leaves P, already in the A-operand layout, in LDS. Waves 0..3 are P.V
// waves: wave f owns output features 128 f .. 128 f + 127 of all four head
// tiles, reads its quarter of V once per tile and multiplies it against the
// four tiles' P (four matrix ops per V fragment), and issues the ring's
// direct-to-LDS loads. Waves f and 4 + f share a SIMD, so one wave's softmax,
// LDS waits and barriers overlap the other's matrix ops. At step s the logit
// waves work on tile s and the P.V waves on tile s - 1; P is handed over
// through a single LDS buffer between two barriers per step.
//
// Frames as in the per-tile kernels: each head's frame is its first tile's
// maximum; bf16 weights up to 2^64 are accumulated as they are, E4M3 weights
// carry the tile's exponent rise in the op's E8M0 scale. A head tile whose
// logits rise more than 64 above its frame is recomputed in a second pass
// with the frame preset (the other tiles then contribute zero weights).
//
// SPARSE: a request's tokens are the positions of its top-k list, already
// turned into physical row ids (-1: no token) by sparse_rows_kernel. Each
// P.V wave fetches a quarter of tile k's ids into an eight-slot LDS ring two
// tiles ahead of tile k's rows (one extra ring load per tile and wave; the
// order per step is rows of tile s + 2, then ids of tile s + 4) and reads
// its nine row ids back when it issues the tile. A missing token is read
// from a zero row in the workspace and its logit is masked.
constexpr int kMhWaves = 8;
constexpr int kMhThreads = 64 * kMhWaves;

template <int KV_FP8, int SPARSE>
__global__ void __launch_bounds__(kMhThreads, 1) attn_mh_kernel(AttnArgs a) {
  constexpr int kTok = KV_FP8 ? 4 * kUnit : 2 * kUnit;   // tokens per tile
  constexpr int kUnits = kTok / kUnit;
  constexpr int kRowB = KV_FP8 ? kDK : 2 * kDK;          // bytes per cached row
  constexpr int kRowCh = kRowB / 16;
  constexpr int kPWords = KV_FP8 ? 2 : 1;                 // u32x4 per lane of P
  static_assert(kTok * kRowB == kTileBytesBf16, "tile size");
  static_assert(kTok * kRowCh == kDmaPerThread * kThreads, "tile must split evenly");

  __shared__ uint8_t ring[kStages][kTileBytesBf16];
  __shared__ __attribute__((aligned(32))) u32x4_t pbuf[4][64][kPWords];  // P per head tile, lane
  __shared__ int ebuf[4][kHeadTile];        // E4M3: E8M0 scale of P per head
  __shared__ float lbuf[4][kHeadTile];      // final softmax denominators
  __shared__ int redo_tile[4];
  __shared__ int redo_any;
  __shared__ __attribute__((aligned(16))) int32_t sp_ids[SPARSE ? 8 : 1][kTok];  // row ids

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int c = lane & 15, g = lane >> 4;
  const bool logit_wave = wave >= 4;
  const int wq = wave & 3;  // logit waves: head tile; P.V waves: feature quarter
  const int H = a.rows;

  const int lin = blockIdx.x;
  const int xcd = lin & 7, slot = lin >> 3;
  const int hg = slot % a.head_groups;
  const int part = (slot / a.head_groups) * 8 + xcd;
  const int ht0 = 4 * hg;                                 // first head tile of the group
  const bool lw_active = logit_wave && ht0 + wq < a.head_tiles;
  const int h0 = (ht0 + wq) * kHeadTile;                  // logit wave's first head
  // Logit waves: row h0 + c belongs to query token (h0 + c) / heads, which
  // sees all but the last `back` tokens of the request.
  const int back = a.q_len - 1 - min(h0 + c, H - 1) / a.heads;

  // DMA map of the P.V waves (thread tid < 256): load i fills LDS slot
  // i * 256 + tid of the stage.
  uint32_t dma_off[kDmaPerThread];
  uint32_t dma_unit = 0;  // two bits per load
#pragma unroll
  for (int i = 0; i < kDmaPerThread; ++i) {
    const int pos = i * kThreads + (tid & (kThreads - 1));
    const int t = pos / kRowCh, sl = pos - (pos / kRowCh) * kRowCh;
    const int ch = KV_FP8 ? (sl ^ fp8_swizzle(t)) : (sl ^ (t & 7));
    // Sparse: (token of the tile << 16) | byte offset in its row.
    dma_off[i] = SPARSE ? (uint32_t(t) << 16) | uint32_t(ch * 16)
                        : uint32_t((t & 15) * kRowB + ch * 16);
    dma_unit |= uint32_t(t >> 4) << (2 * i);
  }
  const uint32_t ids_lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (void __attribute__((address_space(3)))*)(&sp_ids[0][0])));
  const uint32_t ring_lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (void __attribute__((address_space(3)))*)(&ring[0][0])));
  const int bs_mask = (1 << a.bs_log2) - 1;

  // Stage-independent LDS offsets.
  // Logit waves, K: bf16 row c of each unit at chunk pairs (g ^ (c & 7)) and
  // its partner; E4M3 row c, chunk 4 m + (g ^ swizzle) (units of equal parity
  // share the swizzle).
  uint32_t k_off0, k_off1;
  if constexpr (KV_FP8) {
    k_off0 = uint32_t(c * kDK + 16 * (g ^ fp8_swizzle(c)));
    k_off1 = uint32_t(c * kDK + 16 * (g ^ fp8_swizzle(16 + c)));
  } else {
    const uint32_t y = uint32_t(g ^ (c & 7));
    k_off0 = uint32_t(c * kRowB) + 16 * y;
    k_off1 = uint32_t(c * kRowB) + 16 * (y ^ 4);
  }
  // P.V waves, V: transposing reads of features 128 wq + 16 n' + ..,
  // n' = 4 M + j; v_off[j] is the lane's address for j (M in the immediate).
  uint32_t v_off[4];
  if constexpr (KV_FP8) {
    const int s4 = lane & 15, av = s4 & 1, ev = s4 >> 1;
    const int t = 16 * (ev >> 2) + 4 * g + (ev & 3);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      v_off[j] = uint32_t(t * kDK + 16 * (8 * wq + (j ^ fp8_swizzle(t))) + 8 * av);
  } else {
    const int s4 = lane & 15, av = s4 & 3, ev = s4 >> 2;
    const int t0 = 4 * g + ev;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      v_off[j] = uint32_t(t0 * kRowB) +
                 16u * uint32_t(16 * wq + ((2 * j + (av >> 1)) ^ (t0 & 7))) + 8u * uint32_t(av & 1);
  }

  // P.V waves (E4M3): LDS addresses of this lane's P operands and scales.
  const uint32_t p_lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (void __attribute__((address_space(3)))*)(&pbuf[0][lane][0])));
  const uint32_t e_lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (void __attribute__((address_space(3)))*)(&ebuf[0][c])));
  static_assert(!KV_FP8 || sizeof(pbuf[0]) == 2048, "P operand stride");
  static_assert(sizeof(ebuf[0]) == 64, "scale stride");

  for_each_piece<kMhThreads>(a, part, reinterpret_cast<int*>(&ring[0][0]),
                             [&](int b, int u0, int u1, int out_row) {
    const int n = checked_len(a.seq_lens[b], a.cap_tokens, a.err_word);
    const int u_end = min(u1, (n + kUnit - 1) / kUnit);
    const int ntiles = u_end > u0 ? (u_end - u0 + kUnits - 1) / kUnits : 0;
    const int32_t* bt_row = a.block_table + size_t(b) * a.max_blocks;
    auto tile_nv = [&](int k, int (&nv)[kUnits]) {
#pragma unroll
      for (int u = 0; u < kUnits; ++u) {
        const int uu = u0 + kUnits * k + u;
        nv[u] = uu < u_end ? min(kUnit, n - uu * kUnit) : 0;
      }
    };
    auto unit_rows = [&](int u) -> const uint8_t* {
      const int t0 = u * kUnit;
      int blk = scalar_load_i32(bt_row + (t0 >> a.bs_log2));
      if (blk < 0 || blk >= a.num_blocks) {
        report_bounds(a.err_word, kBoundsBadBlock);
        blk = 0;
      }
      return a.kv + (size_t(blk) * (size_t(1) << a.bs_log2) + size_t(t0 & bs_mask)) * kRowB;
    };
    auto issue_tile = [&](int k) {
      const int uk = u0 + kUnits * k;
      const uint8_t* r[4];
      r[0] = unit_rows(uk);
      // Units in the page of the unit before continue its rows: one
      // block-table lookup (a scalar-load round trip) per page, not per unit.
#pragma unroll
      for (int u = 1; u < 4; ++u) {
        const int tu = (uk + u) * kUnit;
        r[u] = !(u < kUnits && uk + u < u_end)           ? r[0]
               : (tu >> a.bs_log2) == ((tu - kUnit) >> a.bs_log2) ? r[u - 1] + kUnit * kRowB
                                                                  : unit_rows(uk + u);
      }
      uint8_t* dst = &ring[k % kStages][0] + wave * 64 * 16;
#pragma unroll
      for (int i = 0; i < kDmaPerThread; ++i) {
        const uint32_t us = (dma_unit >> (2 * i)) & 3u;
        const uint8_t* base = (us & 2) ? ((us & 1) ? r[3] : r[2]) : ((us & 1) ? r[1] : r[0]);
        __builtin_amdgcn_global_load_lds(
            base + dma_off[i], (void __attribute__((address_space(3)))*)(dst + i * kThreads * 16),
            16, 0, kRingLoadPolicy);
      }
    };
    // Sparse: ids of tile k (a quarter per P.V wave) into slot k % 8.
    auto issue_ids = [&](int k) {
      constexpr int kPer = kTok / 4;
      if (lane < kPer) {
        const int32_t* src = a.sparse_rows + size_t(b) * a.sparse_stride + size_t(u0) * kUnit +
                             size_t(k) * kTok + wave * kPer + lane;
        __builtin_amdgcn_global_load_lds(
            src, (void __attribute__((address_space(3)))*)(&sp_ids[k & 7][wave * kPer]), 4, 0, 0);
      }
    };
    // Sparse: rows of tile k from its ids (already in LDS).
    auto issue_tile_sparse = [&](int k) {
      uint32_t ad[kDmaPerThread];
      int rid[kDmaPerThread];
      const uint32_t slot = ids_lds + uint32_t((k & 7) * kTok * 4);
#pragma unroll
      for (int i = 0; i < kDmaPerThread; ++i) ad[i] = slot + ((dma_off[i] >> 16) << 2);
      lds_read_ids9(ad, rid);
      uint8_t* dst = &ring[k % kStages][0] + wave * 64 * 16;
#pragma unroll
      for (int i = 0; i < kDmaPerThread; ++i) {
        const uint32_t ch16 = dma_off[i] & 0xffffu;
        const uint8_t* src = rid[i] >= 0 ? a.kv + size_t(rid[i]) * kRowB + ch16 : a.zero_row + ch16;
        __builtin_amdgcn_global_load_lds(
            src, (void __attribute__((address_space(3)))*)(dst + i * kThreads * 16), 16, 0,
            kRingLoadPolicy);
      }
    };

    const bool final_out = out_row < 0;
    const int row = final_out ? 0 : out_row;
    // Both roles pass the same barriers in the same order: per pass one
    // opening barrier, two per step, two closing ones; then one before the
    // epilogue's output stores.
    if (logit_wave) {
      // q of head h0 + c (padded heads repeat H - 1).
      u32x4_t qf[kQChunks];                 // bf16: features 32 s + 8 g .. + 7
      i32x8_t qb_hi[4], qb_lo[4], qb_last;  // E4M3: pairs of 64-dim blocks, hi / lo
      float xscale = a.scale_log2;
      {
        const int hq = min(h0 + c, H - 1);
        if constexpr (!KV_FP8) {
          const u32x4_t* qp =
              reinterpret_cast<const u32x4_t*>(a.q + (size_t(b) * H + hq) * kDK) + g;
#pragma unroll
          for (int s2 = 0; s2 < kQChunks; ++s2) qf[s2] = qp[4 * s2];
        } else {
          const u32x4_t* qp =
              reinterpret_cast<const u32x4_t*>(a.q + (size_t(b) * H + hq) * kDK + 16 * g);
          u32x4_t raw[kKChunksFp8][2];
#pragma unroll
          for (int m = 0; m < kKChunksFp8; ++m) {
            raw[m][0] = qp[8 * m];
            raw[m][1] = qp[8 * m + 1];
          }
          float amax = 0.f;
#pragma unroll
          for (int m = 0; m < kKChunksFp8; ++m)
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
              for (int w = 0; w < 4; ++w) {
                const unsigned x = raw[m][h][w];
                amax = fmaxf(amax, fmaxf(fabsf(__builtin_bit_cast(float, x << 16)),
                                         fabsf(__builtin_bit_cast(float, x & 0xffff0000u))));
              }
          amax = fmaxf(amax, __shfl_xor(amax, 16));
          amax = fmaxf(amax, __shfl_xor(amax, 32));
          // The floor keeps 448 / amax finite for rows of tiny magnitude (bf16
          // reaches 1e-38, where 448 / amax would overflow fp32); such rows'
          // logits are far below any resolution of the softmax anyway.
          amax = fmaxf(amax, 0x1p-100f);
          const float inv = 448.f / amax;
          xscale = (amax / 448.f) * a.kv_scale * a.scale_log2;
#pragma unroll
          for (int m = 0; m < kKChunksFp8; ++m) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
              for (int w2 = 0; w2 < 2; ++w2) {
                const unsigned x0 = raw[m][h][2 * w2], x1 = raw[m][h][2 * w2 + 1];
                const float f0 = __builtin_bit_cast(float, x0 << 16) * inv;
                const float f1 = __builtin_bit_cast(float, x0 & 0xffff0000u) * inv;
                const float f2 = __builtin_bit_cast(float, x1 << 16) * inv;
                const float f3 = __builtin_bit_cast(float, x1 & 0xffff0000u) * inv;
                const unsigned hi = pack_e4m3x4_inrange(f0, f1, f2, f3);
                const unsigned lo = pack_e4m3x4_inrange(
                    f0 - __builtin_amdgcn_cvt_f32_fp8(int(hi), 0),
                    f1 - __builtin_amdgcn_cvt_f32_fp8(int(hi), 1),
                    f2 - __builtin_amdgcn_cvt_f32_fp8(int(hi), 2),
                    f3 - __builtin_amdgcn_cvt_f32_fp8(int(hi), 3));
                const int w = 2 * h + w2;
                if (m < 8) {
                  qb_hi[m >> 1][4 * (m & 1) + w] = int(hi);
                  qb_lo[m >> 1][4 * (m & 1) + w] = int(lo);
                } else {
                  qb_last[w] = int(hi);
                  qb_last[4 + w] = int(lo);
                }
              }
            }
          }
        }
      }
      float m_ref = -INFINITY;   // frame of head c (log2 domain)
      float m_seen = -INFINITY;  // largest logit of head c (first pass)
      float l_run = 0.f;         // lane's share of head c's denominator
      bool redo = false;         // frame exceeded in the first pass

      for (int pass = 0; pass < 2; ++pass) {
        // First pass: every active tile; second: only those that asked.
        const bool work = lw_active && (pass == 0 || redo);
        if (pass == 1 && work) {
          m_ref = m_seen;
          l_run = 0.f;
        }
        redo = false;
        wave_barrier_all();  // ring and P buffer of the previous pass or piece are free
        wait_vmem<0>();      // q
        if constexpr (SPARSE) wave_barrier_all();  // the P.V waves' first ids are in LDS
        for (int s = 0; s <= ntiles; ++s) {
          wave_barrier_lds();  // barrier 1: tile s is in the ring
          wave_barrier_lds();  // barrier 2: the P.V waves hold P of tile s - 1
          if (s == ntiles) continue;
          u32x4_t pw[kPWords];
          int e_scale = 127;
          // The logit wave is the step's critical path: its K reads and
          // matrix ops take precedence over the P.V wave sharing the SIMD,
          // whose matrix ops then fill the gaps and the softmax below.
          __builtin_amdgcn_s_setprio(3);
          if (work) {
            int nv[kUnits];
            tile_nv(s, nv);
            // Row c's visible tokens per unit (none once past its query token).
            const int vis = n - back - (u0 + kUnits * s) * kUnit;
#pragma unroll
            for (int u = 0; u < kUnits; ++u) nv[u] = min(nv[u], vis - u * kUnit);
            float x[kUnits][4];
            // K through ordinary LDS loads: logit waves issue no ring loads,
            // so the compiler's own waits cost nothing and it may overlap the
            // reads with the matrix ops.
            const uint8_t* stp = &ring[s % kStages][0];
            if constexpr (!KV_FP8) {
#pragma unroll
              for (int h = 0; h < 2; ++h) {
                const uint8_t* rowp = stp + h * kUnit * kRowB;
                u32x4_t kf[kQChunks];
#pragma unroll
                for (int k2 = 0; k2 < kQChunks / 2; ++k2) {
                  kf[2 * k2] = *reinterpret_cast<const u32x4_t*>(rowp + k_off0 + 128 * k2);
                  kf[2 * k2 + 1] = *reinterpret_cast<const u32x4_t*>(rowp + k_off1 + 128 * k2);
                }
                f32x4_t sc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s2 = 0; s2 < kQChunks; ++s2)
                  sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                      __builtin_bit_cast(bf16x8_t, kf[s2]), __builtin_bit_cast(bf16x8_t, qf[s2]),
                      sc, 0, 0, 0);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                  x[h][r] = (4 * g + r < nv[h]) ? sc[r] * xscale : -INFINITY;
              }
            } else {
              auto logits = [&](auto uc) {
                constexpr int U = decltype(uc)::value;
                u32x4_t kf[kKChunksFp8];
                const uint8_t* up = stp + U * kUnit * kDK + ((U & 1) ? k_off1 : k_off0);
#pragma unroll
                for (int m = 0; m < kKChunksFp8; ++m)
                  kf[m] = *reinterpret_cast<const u32x4_t*>(up + 64 * m);
                f32x4_t sc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int p2 = 0; p2 < 4; ++p2) {
                  const i32x8_t ka = __builtin_bit_cast(
                      i32x8_t,
                      __builtin_shufflevector(kf[2 * p2], kf[2 * p2 + 1], 0, 1, 2, 3, 4, 5, 6, 7));
                  sc = mfma_e4m3_128(ka, qb_hi[p2], sc, 127);
                  sc = mfma_e4m3_128(ka, qb_lo[p2], sc, 127);
                }
                {
                  const i32x8_t ka = __builtin_bit_cast(
                      i32x8_t, __builtin_shufflevector(kf[8], kf[8], 0, 1, 2, 3, 4, 5, 6, 7));
                  sc = mfma_e4m3_128(ka, qb_last, sc, 127);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r)
                  x[U][r] = (4 * g + r < nv[U]) ? sc[r] * xscale : -INFINITY;
              };
              logits(std::integral_constant<int, 0>{});
              logits(std::integral_constant<int, 1>{});
              logits(std::integral_constant<int, 2>{});
              logits(std::integral_constant<int, 3>{});
            }
            // Keep nine K reads in flight ahead of the matrix ops: 9 reads,
            // then (1 op, 1 read) x 27, then the last 9 ops.
            __builtin_amdgcn_sched_group_barrier(0x100, 9, 0);
#pragma unroll
            for (int i = 0; i < 27; ++i) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 9, 0);
            if constexpr (SPARSE) {
              // Listed positions that name no token get no weight.
#pragma unroll
              for (int u = 0; u < kUnits; ++u) {
                const int4 id = *reinterpret_cast<const int4*>(&sp_ids[s & 7][16 * u + 4 * g]);
                if (id.x < 0) x[u][0] = -INFINITY;
                if (id.y < 0) x[u][1] = -INFINITY;
                if (id.z < 0) x[u][2] = -INFINITY;
                if (id.w < 0) x[u][3] = -INFINITY;
              }
            }
            __builtin_amdgcn_s_setprio(0);
            float mt = -INFINITY;
#pragma unroll
            for (int u = 0; u < kUnits; ++u)
              mt = fmaxf(mt, fmaxf(fmaxf(x[u][0], x[u][1]), fmaxf(x[u][2], x[u][3])));
            mt = max_over_lane_groups(mt);
            m_seen = fmaxf(m_seen, mt);
            if (m_ref == -INFINITY) m_ref = mt;  // first tile (per head): the frame
            if (__ballot(mt > m_ref + kHeadsSlack) != 0ull) redo = true;  // wave-uniform
            // A row that has seen no token yet (all masked) keeps weight 0.
            const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
            if constexpr (!KV_FP8) {
              float p[2][4];
#pragma unroll
              for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int r = 0; r < 4; ++r) p[h][r] = fast_exp2(x[h][r] - m_use);
              l_run += ((p[0][0] + p[0][1]) + (p[0][2] + p[0][3])) +
                       ((p[1][0] + p[1][1]) + (p[1][2] + p[1][3]));
              bf16x8_t pa;
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                pa[r] = (__bf16)p[0][r];
                pa[4 + r] = (__bf16)p[1][r];
              }
              pw[0] = __builtin_bit_cast(u32x4_t, pa);
            } else {
              const float rise = mt - m_use;
              const int e = rise > 0.f ? min(int(ceilf(rise)), int(kHeadsSlack)) : 0;
              const float fe = m_use + float(e);
              unsigned ph[4], pl[4];
              float lt = 0.f;   // sum of the stored weights 2^(x - fe + 8)
              const float fe8 = fe - 8.f;
#pragma unroll
              for (int u = 0; u < 4; ++u) {
                float ps[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                  ps[r] = fast_exp2(x[u][r] - fe8);
                  lt += ps[r];
                }
                ph[u] = pack_e4m3x4_inrange(ps[0], ps[1], ps[2], ps[3]);
                // Residuals against the rounded bytes 0-1 and 2-3, decoded in pairs.
                const f32x2_t h01 = __builtin_amdgcn_cvt_pk_f32_fp8(int(ph[u]), false);
                const f32x2_t h23 = __builtin_amdgcn_cvt_pk_f32_fp8(int(ph[u]), true);
                pl[u] = pack_e4m3x4_inrange(ps[0] - h01[0], ps[1] - h01[1], ps[2] - h23[0],
                                            ps[3] - h23[1]);
              }
              l_run += __builtin_amdgcn_ldexpf(lt, e - 8);
              pw[0] = u32x4_t{ph[0], ph[1], ph[2], ph[3]};
              pw[kPWords - 1] = u32x4_t{pl[0], pl[1], pl[2], pl[3]};
              e_scale = 127 + e;
            }
          } else {
#pragma unroll
            for (int w = 0; w < kPWords; ++w) pw[w] = u32x4_t{0u, 0u, 0u, 0u};
          }
          // (Scalar: executes on both sides of the branch above, so the
          // priority is dropped here rather than in its else side.)
          __builtin_amdgcn_s_setprio(0);
#pragma unroll
          for (int w = 0; w < kPWords; ++w) pbuf[wq][lane][w] = pw[w];
          if (KV_FP8 && g == 0) ebuf[wq][c] = e_scale;
        }
        wave_barrier_lds();  // closing barrier 1: redo_any cleared
        if (lane == 0) {
          redo_tile[wq] = (work && redo) ? 1 : 0;
          if (work && redo) redo_any = 1;
        }
        wave_barrier_lds();  // closing barrier 2: redo flags complete
        if (redo_any == 0) break;
      }
      float l_c = l_run + __shfl_xor(l_run, 16);
      l_c += __shfl_xor(l_c, 32);
      if (g == 0) {
        lbuf[wq][c] = l_c;
        if (lw_active && h0 + c < H) {
          const float lse_v = l_c > 0.f ? (m_ref + __log2f(l_c)) * kLn2 : -INFINITY;
          if (final_out) {
            if (a.lse) a.lse[size_t(b) * H + h0 + c] = lse_v;
          } else {
            a.part_lse[size_t(row) * H + h0 + c] = lse_v;
          }
        }
      }
      wave_barrier_lds();  // lbuf complete
    } else {
      // acc[t][j]: head 16 t + 4 g + r of the group, feature 128 wq + 16 j + c.
      f32x4_t acc[4][8];
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[t][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      for (int pass = 0; pass < 2; ++pass) {
        if (pass == 1) {
          // Clear the accumulators of recomputed head tiles (by selection:
          // their first-pass sums may hold non-finite values).
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const bool clear = redo_tile[t] != 0;
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
              for (int r = 0; r < 4; ++r) acc[t][j][r] = clear ? 0.f : acc[t][j][r];
          }
        }
        wave_barrier_all();  // ring and P buffer of the previous pass or piece are free
        if constexpr (SPARSE) {
          for (int k = 0; k < 2 && k < ntiles; ++k) issue_ids(k);
          wait_vmem<0>();
          wave_barrier_all();  // ids of tiles 0 and 1 from every P.V wave
          for (int k = 0; k < 2 && k < ntiles; ++k) {
            issue_tile_sparse(k);
            if (k + 2 < ntiles) issue_ids(k + 2);
          }
        } else {
          for (int k = 0; k < 2 && k < ntiles; ++k) issue_tile(k);
        }
        for (int s = 0; s <= ntiles; ++s) {
          if constexpr (SPARSE) {
            // Tile s and the ids of tile s + 2 landed: loads issued after
            // them are the rows of tile s + 1 and the ids of tile s + 3.
            if (s + 3 < ntiles)
              wait_vmem<kDmaPerThread + 1>();
            else if (s + 1 < ntiles)
              wait_vmem<kDmaPerThread>();
            else if (s < ntiles)
              wait_vmem<0>();
          } else {
            if (s < ntiles) wait_ring<1>(ntiles - 1 - s);  // tile s landed
          }
          wave_barrier_lds();  // barrier 1: P of tile s - 1 is in pbuf
          u32x4_t pv_p[4];   // bf16 A operands
          i32x8_t pv_pa[4];  // E4M3 A operands
          int pv_e[4];
          if (s >= 1) {
            if constexpr (KV_FP8) {
              // Ordinary loads here would make the compiler wait for every
              // ring load in flight first (it cannot tell them apart).
              u32x4_t ph[4][2];
              lds_read_p4(p_lds, e_lds, ph, pv_e);
#pragma unroll
              for (int t = 0; t < 4; ++t)
                pv_pa[t] = __builtin_bit_cast(
                    i32x8_t, __builtin_shufflevector(ph[t][0], ph[t][1], 0, 1, 2, 3, 4, 5, 6, 7));
            } else {
#pragma unroll
              for (int t = 0; t < 4; ++t) pv_p[t] = pbuf[t][lane][0];
            }
          }
          wave_barrier_lds();  // barrier 2: P taken, pbuf may be overwritten
          if constexpr (SPARSE) {
            if (s + 2 < ntiles) issue_tile_sparse(s + 2);
            if (s + 4 < ntiles) issue_ids(s + 4);
          } else {
            if (s + 2 < ntiles) issue_tile(s + 2);
          }
          if (s == 0) continue;
          const int k = s - 1;
          const uint32_t st = ring_lds + uint32_t(k % kStages) * kTileBytesBf16;
          int nv[kUnits];
          tile_nv(k, nv);
          bool vmask = false;
#pragma unroll
          for (int u = 0; u < kUnits; ++u) vmask |= nv[u] < kUnit;
          // Per read half h: which of the lane's 8-byte elements are tokens.
          uint64_t vkeep[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            if constexpr (KV_FP8) {
              uint64_t k2 = 0;
#pragma unroll
              for (int q2 = 0; q2 < 2; ++q2) {
                const int kc = min(max(nv[2 * h + q2] - 4 * g, 0), 4);
                const uint64_t m4 = kc >= 4 ? 0xffffffffull : ((1ull << (8 * kc)) - 1ull);
                k2 |= m4 << (32 * q2);
              }
              vkeep[h] = k2;
            } else {
              const int kc = min(max(nv[h] - 4 * g, 0), 4);
              vkeep[h] = kc >= 4 ? ~0ull : ((1ull << (16 * kc)) - 1ull);
            }
          }
          uint32_t vb[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) vb[j] = st + v_off[j];
          auto pv_group = [&](auto mc) {
            constexpr int M = decltype(mc)::value;
            u32x2_t tv[4][2];
            if constexpr (KV_FP8)
              lds_read_trb8<64 * M>(vb, tv);
            else
              lds_read_tr8<M>(vb, tv);
            if (vmask) {
#pragma unroll
              for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                  tv[j][h] = __builtin_bit_cast(
                      u32x2_t, __builtin_bit_cast(uint64_t, tv[j][h]) & vkeep[h]);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              if constexpr (KV_FP8) {
                // One doubled V operand at a time keeps the copies' registers
                // short-lived.
                __builtin_amdgcn_sched_barrier(0);
                const i32x8_t bv = i32x8_t{int(tv[j][0][0]), int(tv[j][0][1]), int(tv[j][1][0]),
                                           int(tv[j][1][1]), int(tv[j][0][0]), int(tv[j][0][1]),
                                           int(tv[j][1][0]), int(tv[j][1][1])};
#pragma unroll
                for (int t = 0; t < 4; ++t)
                  acc[t][4 * M + j] = mfma_e4m3_128(pv_pa[t], bv, acc[t][4 * M + j], pv_e[t]);
              } else {
                const u32x4_t bv = u32x4_t{tv[j][0][0], tv[j][0][1], tv[j][1][0], tv[j][1][1]};
#pragma unroll
                for (int t = 0; t < 4; ++t)
                  acc[t][4 * M + j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                      __builtin_bit_cast(bf16x8_t, pv_p[t]), __builtin_bit_cast(bf16x8_t, bv),
                      acc[t][4 * M + j], 0, 0, 0);
              }
            }
          };
          pv_group(std::integral_constant<int, 0>{});
          pv_group(std::integral_constant<int, 1>{});
        }
        if (tid == 0) redo_any = 0;
        wave_barrier_lds();  // closing barrier 1
        wave_barrier_lds();  // closing barrier 2: redo flags complete
        if (redo_any == 0) break;
      }
      wave_barrier_lds();  // lbuf complete
      const float out_scale = KV_FP8 ? a.kv_scale * (1.f / 256.f) : 1.f;
      // The output rows' addresses are formed here from values the compiler
      // cannot see through, not hoisted to the kernel start (where sixteen
      // per-lane 64-bit head offsets would stay live across the step loops
      // and spill).
      int row_base = final_out ? b : row;
      int ge = g, ce = c;
      asm volatile("" : "+s"(row_base), "+v"(ge), "+v"(ce));
#pragma unroll
      for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int hh = 4 * ge + r;
          const int h = (ht0 + t) * kHeadTile + hh;
          const float lh = lbuf[t][hh];
          const float inv = lh > 0.f ? out_scale / lh : 0.f;
          if (h < H) {
            if (final_out) {
              uint16_t* dst = a.out + (size_t(row_base) * H + h) * kDV + 128 * wq + ce;
#pragma unroll
              for (int j = 0; j < 8; ++j) dst[16 * j] = bf16_bits(acc[t][j][r] * inv);
            } else {
              float* dst = a.part_out + (size_t(row_base) * H + h) * kDV + 128 * wq + ce;
#pragma unroll
              for (int j = 0; j < 8; ++j) dst[16 * j] = acc[t][j][r] * inv;
            }
          }
        }
      }
    }
  });
}

// ----------------------------------------------------------------------------
// LSE combine: one workgroup per (request, 16-head tile, feature chunk);
// thread (head hh, sub) merges F features of the chunk from 64 / F partial
// rows in flight. F = 8 (four 128-feature chunks per head tile) when there
// are many (request, tile) pairs; fewer features per thread, and so more
// workgroups, when there are few: each workgroup then reads a smaller share
// of a request's rows, which bounds small batches (a request split into many
// pieces at batch 8 gives 32 workgroups at F = 8, 128 at F = 2).
constexpr int kCombineGrid = 1 << 30;  // no cap: one workgroup per (request, tile, chunk)

template <int F>
__device__ __forceinline__ void load_features(const float* src, float (&v)[F]) {
  if constexpr (F == 2) {
    const f32x2_t x = *reinterpret_cast<const f32x2_t*>(src);
    v[0] = x[0];
    v[1] = x[1];
  } else {
#pragma unroll
    for (int i = 0; i < F / 4; ++i) {
      const f32x4_t x = reinterpret_cast<const f32x4_t*>(src)[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * i + e] = x[e];
    }
  }
}

// Merge rows r0 .. r0 + nr - 1 of request b for head tile ht and feature
// chunk `chunk` (16 F features): thread (head tid / 16, features F (tid % 16)
// ..) of 256.
template <int F>
__device__ __forceinline__ void combine_rows(const float* part_out, const float* part_lse, int r0,
                                             int nr, uint16_t* out, float* lse, int b, int H,
                                             int ht, int chunk) {
  constexpr int U = 64 / F;  // rows per batch of loads
  const int tid = threadIdx.x;
  const int h = ht * kHeadTile + (tid >> 4);
  if (h >= H) return;
  const int d = chunk * 16 * F + F * (tid & 15);
  // One pass with a running maximum, U rows in flight: acc and W are kept
  // relative to M and rescaled when M rises.
  float M = -INFINITY;
  float acc[F];
#pragma unroll
  for (int i = 0; i < F; ++i) acc[i] = 0.f;
  float W = 0.f;
  for (int s0 = 0; s0 < nr; s0 += U) {
    // Rows past the request's last are not loaded (the count is uniform
    // across the workgroup, so the skipped loads are branched over).
    const int cnt = min(nr - s0, U);
    float v[U][F];
    float ls[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      if (k < cnt) {
        ls[k] = part_lse[size_t(r0 + s0 + k) * H + h];
        load_features<F>(part_out + (size_t(r0 + s0 + k) * H + h) * kDV + d, v[k]);
      } else {
        ls[k] = -INFINITY;
#pragma unroll
        for (int i = 0; i < F; ++i) v[k][i] = 0.f;
      }
    }
    float mb = ls[0];
#pragma unroll
    for (int k = 1; k < U; ++k) mb = fmaxf(mb, ls[k]);
    if (mb == -INFINITY) continue;  // only empty rows in this batch
    const float Mn = fmaxf(M, mb);
    const float a = M == -INFINITY ? 0.f : fast_exp2((M - Mn) * kLog2e);
#pragma unroll
    for (int i = 0; i < F; ++i) acc[i] *= a;
    W *= a;
    M = Mn;
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const float w = ls[k] != -INFINITY ? fast_exp2((ls[k] - M) * kLog2e) : 0.f;
      if (w != 0.f) {  // an empty row's values are never used
#pragma unroll
        for (int i = 0; i < F; ++i) acc[i] += w * v[k][i];
      }
      W += w;
    }
  }
  const float inv = W > 0.f ? 1.f / W : 0.f;
  unsigned pk[F / 2];
#pragma unroll
  for (int i = 0; i < F / 2; ++i)
    pk[i] = unsigned(bf16_bits(acc[2 * i] * inv)) | (unsigned(bf16_bits(acc[2 * i + 1] * inv)) << 16);
  uint16_t* dst = out + (size_t(b) * H + h) * kDV + d;
  if constexpr (F == 8) {
    *reinterpret_cast<u32x4_t*>(dst) = u32x4_t{pk[0], pk[1], pk[2], pk[3]};
  } else if constexpr (F == 4) {
    *reinterpret_cast<u32x2_t*>(dst) = u32x2_t{pk[0], pk[1]};
  } else {
    *reinterpret_cast<unsigned*>(dst) = pk[0];
  }
  if (chunk == 0 && (tid & 15) == 0 && lse) lse[size_t(b) * H + h] = W > 0.f ? M + __logf(W) : -INFINITY;
}

// Rows of request b: row_ptr[b] .. row_ptr[b + 1] - 1, or with uniform > 0
// (forced splits, no plan launched) b * uniform .. b * uniform + uniform - 1.
template <int F>
__global__ void __launch_bounds__(256) combine_kernel(const float* part_out, const float* part_lse,
                                                      const int32_t* row_ptr, uint16_t* out,
                                                      float* lse, int32_t batch, int32_t H,
                                                      int32_t tiles, int zero_empty,
                                                      int32_t uniform) {
  constexpr int kChunks = kDV / (16 * F);
  const int blk = blockIdx.x;
  const int chunk = blk % kChunks;
  const int bt = blk / kChunks;
  const int b = bt / tiles, ht = bt - (bt / tiles) * tiles;
  const int r0 = uniform > 0 ? b * uniform : row_ptr[b];
  const int nr = uniform > 0 ? uniform : row_ptr[b + 1] - r0;
  if (nr <= 0 && !zero_empty) return;
  combine_rows<F>(part_out, part_lse, r0, nr, out, lse, b, H, ht, chunk);
}

// The automatic plan's combine: block k merges the split request of record
// split[k] = (request, first partial row, rows), header[2] such records; the
// rest exit at once. The first record a block needs is requested together
// with header[2] (one round trip before the rows, not two).
template <int F>
__global__ void __launch_bounds__(256) combine_split_kernel(
    const float* part_out, const float* part_lse, const int4* split, const int32_t* header,
    uint16_t* out, float* lse, int32_t H, int32_t tiles, int32_t max_split) {
  // Grid-stride over (split request, head tile, chunk): a plan without
  // split requests costs one small launch.
  constexpr int kChunks = kDV / (16 * F);
  const int per = tiles * kChunks;
  const int k0 = blockIdx.x / per;
  const int4 rec0 = k0 < max_split ? split[k0] : make_int4(0, 0, 0, 0);
  const int n = header[2] * per;
  for (int w = blockIdx.x; w < n; w += gridDim.x) {
    const int k = w / per;
    const int4 rec = w == int(blockIdx.x) ? rec0 : split[k];
    const int rest = w - k * per;
    const int chunk = rest % kChunks, ht = rest / kChunks;
    combine_rows<F>(part_out, part_lse, rec.y, rec.z, out, lse, rec.x, H, ht, chunk);
  }
}

// Features per combine thread for `pairs` (request, head tile) pairs.
int combine_features(int64_t pairs) { return pairs >= 128 ? 8 : pairs >= 32 ? 4 : 2; }

// ----------------------------------------------------------------------------
// Host-side launchers.

hipError_t launch_plan(const int32_t* seq_lens, int32_t batch, int32_t cap_tokens,
                       int32_t max_parts, int32_t ovh, const WorkspaceLayout& w, void* workspace,
                       hipStream_t stream) {
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  // Small batches and partition counts: a quarter of the threads (cheaper barriers).
  const bool small = batch <= 4 * kPlanThreadsSmall && max_parts < 4 * kPlanThreadsSmall;
  auto kern = small ? plan_kernel<kPlanThreadsSmall> : plan_kernel<kPlanThreads>;
  hipLaunchKernelGGL(kern, dim3(1), dim3(small ? kPlanThreadsSmall : kPlanThreads), 0, stream,
                     seq_lens, batch, cap_tokens, max_parts, ovh,
                     reinterpret_cast<int32_t*>(ws + w.header), reinterpret_cast<int32_t*>(ws + w.cum),
                     reinterpret_cast<int32_t*>(ws + w.part_ptr),
                     reinterpret_cast<int4*>(ws + w.work), reinterpret_cast<int4*>(ws + w.split));
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& args, int kv_fp8, int32_t parts_launched,
                            hipStream_t stream) {
  dim3 grid(unsigned(parts_launched) * unsigned(args.head_tiles));
  const dim3 grid_mh(unsigned(parts_launched) * unsigned(args.head_groups));
  if (args.sparse_rows) {
    if (kv_fp8)
      hipLaunchKernelGGL((attn_mh_kernel<1, 1>), grid_mh, dim3(kMhThreads), 0, stream, args);
    else
      hipLaunchKernelGGL((attn_mh_kernel<0, 1>), grid_mh, dim3(kMhThreads), 0, stream, args);
  } else if (kv_fp8) {
    hipLaunchKernelGGL((attn_mh_kernel<1, 0>), grid_mh, dim3(kMhThreads), 0, stream, args);
  } else if (uses_16_head_kernel(args.rows, kv_fp8, false)) {
    hipLaunchKernelGGL(attn_ws_kernel, grid, dim3(kWsThreads), 0, stream, args);
  } else {
    hipLaunchKernelGGL((attn_mh_kernel<0, 0>), grid_mh, dim3(kMhThreads), 0, stream, args);
  }
  return hipGetLastError();
}

// Sparse decode: physical row id of every listed position (-1 where the
// entry is outside [0, seq_len) or its block id is outside the cache), the
// list length as every request's token count, and a zero row.
__global__ void __launch_bounds__(256) sparse_rows_kernel(
    const int32_t* indices, int32_t topk, const int32_t* block_table, const int32_t* seq_lens,
    int32_t batch, int32_t max_blocks, int32_t num_blocks, int32_t bs_log2, int32_t cap_tokens,
    int32_t stride, int32_t* rows, int32_t* eff_len, uint32_t* zero_row, int32_t* err_word) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < kDK * 2 / 4) zero_row[i] = 0u;
  if (i >= int64_t(batch) * stride) return;
  const int b = int(i / stride), k = int(i - int64_t(b) * stride);
  if (k == 0) eff_len[b] = topk;
  int row = -1;
  if (k < topk) {
    const int t = indices[size_t(b) * topk + k];
    const int n = checked_len(seq_lens[b], cap_tokens, err_word);
    if (t >= 0 && t < n) {
      const int blk = block_table[size_t(b) * max_blocks + (t >> bs_log2)];
      if (blk >= 0 && blk < num_blocks)
        row = (blk << bs_log2) + (t & ((1 << bs_log2) - 1));
      else
        report_bounds(err_word, kBoundsBadBlock);
    }
  }
  rows[i] = row;
}

hipError_t launch_sparse_rows(const int32_t* indices, int32_t topk, const int32_t* block_table,
                              const int32_t* seq_lens, int32_t batch, int32_t max_blocks,
                              int32_t num_blocks, int32_t bs_log2, int32_t cap_tokens,
                              int32_t stride, int32_t* rows, int32_t* eff_len, void* zero_row,
                              int32_t* err_word, hipStream_t stream) {
  const int64_t n = int64_t(batch) * stride;
  const int64_t nb = (n > kDK * 2 / 4 ? n : kDK * 2 / 4) + 255;
  hipLaunchKernelGGL(sparse_rows_kernel, dim3(unsigned(nb / 256)), dim3(256), 0, stream, indices,
                     topk, block_table, seq_lens, batch, max_blocks, num_blocks, bs_log2,
                     cap_tokens, stride, rows, eff_len, static_cast<uint32_t*>(zero_row), err_word);
  return hipGetLastError();
}

__global__ void clear_word_kernel(int32_t* word) { *word = 0; }

hipError_t launch_clear_word(int32_t* word, hipStream_t stream) {
  hipLaunchKernelGGL(clear_word_kernel, dim3(1), dim3(1), 0, stream, word);
  return hipGetLastError();
}

hipError_t launch_combine(const float* part_out, const float* part_lse,
                          const int32_t* row_ptr, uint16_t* out, float* lse, int32_t batch,
                          int32_t num_heads, int zero_empty, int32_t uniform,
                          hipStream_t stream) {
  const int tiles = head_tiles(num_heads);
  const int64_t pairs = int64_t(batch) * tiles;
  auto go = [&](auto kern, int f) {
    hipLaunchKernelGGL(kern, dim3(unsigned(pairs * (kDV / (16 * f)))), dim3(256), 0, stream,
                       part_out, part_lse, row_ptr, out, lse, batch, num_heads, tiles, zero_empty,
                       uniform);
  };
  switch (combine_features(pairs)) {
    case 8: go(combine_kernel<8>, 8); break;
    case 4: go(combine_kernel<4>, 4); break;
    default: go(combine_kernel<2>, 2); break;
  }
  return hipGetLastError();
}

hipError_t launch_combine_split(const float* part_out, const float* part_lse,
                                const int4* split,
                                const int32_t* header, uint16_t* out, float* lse,
                                int32_t max_split, int32_t num_heads, hipStream_t stream) {
  const int tiles = head_tiles(num_heads);
  if (max_split <= 0) return hipSuccess;
  const int64_t pairs = int64_t(max_split) * tiles;
  auto go = [&](auto kern, int f) {
    const int64_t tuples = pairs * (kDV / (16 * f));
    const unsigned grid = unsigned(tuples < kCombineGrid ? tuples : kCombineGrid);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(256), 0, stream, part_out, part_lse, split, header,
                       out, lse, num_heads, tiles, max_split);
  };
  switch (combine_features(pairs)) {
    case 8: go(combine_split_kernel<8>, 8); break;
    case 4: go(combine_split_kernel<4>, 4); break;
    default: go(combine_split_kernel<2>, 2); break;
  }
  return hipGetLastError();
}

}  // namespace mla
