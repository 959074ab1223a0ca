"""Seeded synthetic inputs for MLA paged-KV decode.

This module only draws inputs. It holds none of the attention arithmetic, and
both the fp64 oracle and the HIP path consume what it returns. Everything is
drawn on the CPU from ``torch.Generator('cpu').manual_seed(seed)`` in a fixed
order: sequence lengths, then the physical block permutation, then q, then the
KV pool.

Shapes follow the decode workloads described by the pages:
  * one query token per request (PR #20769, review of ensure_size), or q_len
    tokens per request as in speculative decoding (q [B, q_len, H, 576]; the
    new tokens are the last q_len positions counted in seq_lens);
  * a paged cache addressed through a per-request block table with block sizes
    of 16 to 128 tokens (PR #21078 E2E command uses --block-size 32);
  * 576-wide latent rows (512 kv_c + 64 rope) shared by all heads;
  * bf16 q and cache drawn from N(0, 1), or an fp8 E4M3 cache with one fp32
    per-tensor scale (PR #57428 deployment command, --kv-cache-dtype fp8).

Named configurations:
  tiny      B=2,   H=16,  seq_lens {37, 130}, bs=16, 16-block pool (4 unused)
  v2lite-N  B=N,   H=16,  seq_lens U[1024, 4096], bs=64      (N = 1, 8, 64)
  r1tp8     B=512, H=16,  seq_lens U[1024, 3072], bs=32
  fullhead  B=128, H=128, seq_lens log-uniform [512, 32768], bs=64
  fp8       B=64,  H=128, seq_lens 8192, bs=64, E4M3 cache + per-tensor scale
  sparse-r1tp8  B=512, H=16, seq_lens U[4096, 16384], bs=32, 2048 listed tokens each
  sparse-fp8    B=64, H=128, seq_lens 16384, bs=64, E4M3, 2048 listed tokens each
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

D_K = 576
D_V = 512
SCALE = float(np.float32(1.0 / math.sqrt(192.0)))  # fp32 value passed to both sides
E4M3_MAX = 448.0

CONFIGS = {
    "tiny": dict(batch=2, num_heads=16, seq=("fixed", [37, 130]), block_size=16,
                 pool_blocks=16, seed=0, kv_dtype="bf16"),
    "v2lite-1": dict(batch=1, num_heads=16, seq=("uniform", 1024, 4096), block_size=64,
                     seed=1, kv_dtype="bf16"),
    "v2lite-8": dict(batch=8, num_heads=16, seq=("uniform", 1024, 4096), block_size=64,
                     seed=2, kv_dtype="bf16"),
    "v2lite-64": dict(batch=64, num_heads=16, seq=("uniform", 1024, 4096), block_size=64,
                      seed=3, kv_dtype="bf16"),
    "r1tp8": dict(batch=512, num_heads=16, seq=("uniform", 1024, 3072), block_size=32,
                  seed=4, kv_dtype="bf16"),
    "fullhead": dict(batch=128, num_heads=128, seq=("loguniform", 512, 32768), block_size=64,
                     seed=5, kv_dtype="bf16"),
    "fp8": dict(batch=64, num_heads=128, seq=("fixed", [8192] * 64), block_size=64,
                seed=6, kv_dtype="fp8"),
    # Sparse decode: each request attends to 2048 listed positions of a longer
    # context (synthetic top-k lists).
    "sparse-r1tp8": dict(batch=512, num_heads=16, seq=("uniform", 4096, 16384), block_size=32,
                         seed=7, kv_dtype="bf16", topk=2048),
    "sparse-fp8": dict(batch=64, num_heads=128, seq=("fixed", [16384] * 64), block_size=64,
                       seed=8, kv_dtype="fp8", topk=2048),
}


@dataclasses.dataclass
class Workload:
    name: str
    q: torch.Tensor            # [B, H, 576] bf16, or [B, q_len, H, 576]
    kv: torch.Tensor           # [NB, bs, 576] bf16, or uint8 E4M3FN codes
    block_table: torch.Tensor  # [B, max_blocks] int32, -1 past each request's blocks
    seq_lens: torch.Tensor     # [B] int32
    block_size: int
    kv_dtype: str              # "bf16" | "fp8"
    kv_scale: float            # per-tensor E4M3 scale (1.0 for bf16)
    scale: float = SCALE
    indices: torch.Tensor | None = None  # sparse decode: [B, topk] int32 token positions

    @property
    def batch(self) -> int:
        return self.q.shape[0]

    @property
    def num_heads(self) -> int:
        return self.q.shape[-2]

    @property
    def q_len(self) -> int:
        return 1 if self.q.dim() == 3 else self.q.shape[1]

    @property
    def num_blocks(self) -> int:
        return self.kv.shape[0]

    @property
    def max_blocks(self) -> int:
        return self.block_table.shape[1]

    @property
    def total_tokens(self) -> int:
        return int(self.seq_lens.sum())

    # Views handed to the oracle (bit patterns, numpy).
    def q_bits(self) -> np.ndarray:
        return self.q.view(torch.int16).numpy().view(np.uint16)

    def kv_bits(self) -> np.ndarray:
        if self.kv_dtype == "fp8":
            return self.kv.numpy()
        return self.kv.view(torch.int16).numpy().view(np.uint16)


def draw_seq_lens(gen: torch.Generator, batch: int, spec) -> torch.Tensor:
    kind = spec[0]
    if kind == "fixed":
        vals = torch.tensor(spec[1], dtype=torch.int32)
        if vals.numel() != batch:
            raise ValueError("fixed seq_lens must have one entry per request")
        return vals
    if kind == "uniform":  # integers, inclusive bounds
        lo, hi = spec[1], spec[2]
        return torch.randint(lo, hi + 1, (batch,), generator=gen, dtype=torch.int64).to(
            torch.int32)
    if kind == "loguniform":  # round(exp(U(ln lo, ln hi))), clamped to [lo, hi]
        lo, hi = spec[1], spec[2]
        u = torch.rand(batch, generator=gen, dtype=torch.float64)
        v = torch.exp(math.log(lo) + u * (math.log(hi) - math.log(lo)))
        return v.round().clamp(lo, hi).to(torch.int32)
    raise ValueError(f"unknown seq_len spec {spec}")


def _randn_bf16(gen: torch.Generator, n_rows: int, chunk_rows: int = 1 << 15) -> torch.Tensor:
    """N(0,1) drawn in fp32, rounded to bf16 (round to nearest even), chunked."""
    out = torch.empty((n_rows, D_K), dtype=torch.bfloat16)
    for r0 in range(0, n_rows, chunk_rows):
        r1 = min(n_rows, r0 + chunk_rows)
        out[r0:r1] = torch.randn((r1 - r0, D_K), generator=gen, dtype=torch.float32).to(
            torch.bfloat16)
    return out


def make_workload(name: str = "custom", *, batch: int, num_heads: int, seq, block_size: int,
                  seed: int, kv_dtype: str = "bf16", pool_blocks: int | None = None,
                  poison: bool = False, q_len: int = 1, topk: int | None = None) -> Workload:
    """Draw one workload.

    seq          ("fixed", list) | ("uniform", lo, hi) | ("loguniform", lo, hi)
    q_len        query tokens per request; q is [B, H, 576] for 1, else
                 [B, q_len, H, 576] (the same draw order either way)
    pool_blocks  physical pool size (default: exactly the blocks the requests use)
    poison       put NaN in unused blocks and in tail slots past each seq_len
    topk         sparse decode: draw indices [B, topk], per request a sorted
                 sample without replacement of min(topk, N) positions of [0, N),
                 padded with -1 (drawn last, after the KV pool)
    """
    gen = torch.Generator("cpu").manual_seed(seed)
    seq_lens = draw_seq_lens(gen, batch, seq)
    nblk = [(int(n) + block_size - 1) // block_size for n in seq_lens]
    used = sum(nblk)
    pool = used if pool_blocks is None else pool_blocks
    if pool < used:
        raise ValueError("pool smaller than the blocks in use")
    perm = torch.randperm(pool, generator=gen).to(torch.int32)
    max_blocks = max(1, max(nblk) if nblk else 1)
    table = torch.full((batch, max_blocks), -1, dtype=torch.int32)
    off = 0
    for b, k in enumerate(nblk):
        table[b, :k] = perm[off:off + k]
        off += k
    q_shape = (batch, num_heads, D_K) if q_len == 1 else (batch, q_len, num_heads, D_K)
    q = torch.randn(q_shape, generator=gen, dtype=torch.float32).to(torch.bfloat16)
    if kv_dtype == "bf16":
        kv = _randn_bf16(gen, pool * block_size).view(pool, block_size, D_K)
        kv_scale = 1.0
    elif kv_dtype == "fp8":
        kv32 = torch.randn((pool * block_size, D_K), generator=gen, dtype=torch.float32)
        kv, kv_scale = quantize_e4m3(kv32)
        del kv32
        kv = kv.view(pool, block_size, D_K)
    else:
        raise ValueError(f"unknown kv dtype {kv_dtype}")
    wl = Workload(name=name, q=q, kv=kv, block_table=table, seq_lens=seq_lens,
                  block_size=block_size, kv_dtype=kv_dtype, kv_scale=kv_scale)
    if topk is not None:
        wl.indices = draw_indices(gen, seq_lens, topk)
    if poison:
        poison_unused(wl)
    return wl


def draw_indices(gen: torch.Generator, seq_lens: torch.Tensor, topk: int) -> torch.Tensor:
    """Synthetic top-k lists: per request a sorted sample without replacement
    of min(topk, N) positions of [0, N), padded with -1."""
    out = torch.full((seq_lens.numel(), topk), -1, dtype=torch.int32)
    for b, n in enumerate(seq_lens.tolist()):
        k = min(topk, n)
        if k:
            pick = torch.randperm(n, generator=gen)[:k].sort().values
            out[b, :k] = pick.to(torch.int32)
    return out


def make_gemm(m: int, n: int, k: int, seed: int):
    """Operands of the block-scaled E4M3 projection: codes of N(0,1) * 64 cast to
    E4M3FN (the two NaN codes cannot occur), and scales log-uniform in
    [2^-10, 2^-4], drawn in that order (a, a_scale, b, b_scale). Returns uint8
    codes a [m, k], b [n, k] and fp32 scales a_scale [m, k/128], b_scale
    [ceil(n/128), k/128]. The default projection shape is DeepSeek-R1's fused
    q/kv down-projection: n = 1536 + 576 = 2112, k = 7168."""
    gen = torch.Generator("cpu").manual_seed(seed)

    def codes(rows):
        x = torch.randn((rows, k), generator=gen, dtype=torch.float32) * 64.0
        return x.clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn).view(torch.uint8)

    def scales(rows):
        u = torch.rand((rows, k // 128), generator=gen, dtype=torch.float64)
        return torch.exp2(-10.0 + 6.0 * u).to(torch.float32)

    a = codes(m)
    a_scale = scales(m)
    b = codes(n)
    b_scale = scales((n + 127) // 128)
    return a, a_scale, b, b_scale


def make_absorb(batch: int, heads: int, seed: int):
    """Operands of the per-head absorption products, all bf16 from fp32 normals
    rounded to nearest even, drawn in order: q_nope [B, H, 128], q_rope
    [B, H, 64], W_UK [H, 128, 512] * 0.05, o_latent [B, H, 512], W_UV
    [H, 128, 512] * 0.05 (one 512-wide row per value dim; weights scaled so
    that outputs stay near N(0, 1))."""
    gen = torch.Generator("cpu").manual_seed(seed)

    def draw(shape, s=1.0):
        return (torch.randn(shape, generator=gen, dtype=torch.float32) * s).to(torch.bfloat16)

    q_nope = draw((batch, heads, 128))
    q_rope = draw((batch, heads, 64))
    w_uk = draw((heads, 128, 512), 0.05)
    o_latent = draw((batch, heads, 512))
    w_uv = draw((heads, 128, 512), 0.05)
    return q_nope, q_rope, w_uk, o_latent, w_uv


def quantize_e4m3(kv32: torch.Tensor):
    """Per-tensor E4M3 codes (uint8) and fp32 scale: amax maps to 448."""
    amax = float(kv32.abs().max())
    kv_scale = float(np.float32(amax / E4M3_MAX)) if amax > 0 else 1.0
    codes = (kv32 / kv_scale).clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
    return codes.view(torch.uint8), kv_scale


def make_rising(num_heads: int, kv_dtype: str, seed: int, block_size: int = 64,
                q_len: int = 1) -> Workload:
    """Logits that climb far above the first tile's: past the first third of
    each request, key row t is alpha_t * q[b, 0] plus small noise, alpha_t
    ramping from 0.5 to 3.0, so head 0's logits rise from about 20 to about
    125 (natural log units) while the other heads stay near N(0, 3). With
    q_len > 1 the direction is head 0 of the last query token."""
    lens = [200, 900, 2100]
    wl = make_workload("rising", batch=len(lens), num_heads=num_heads, seq=("fixed", lens),
                       block_size=block_size, seed=seed, kv_dtype="bf16", q_len=q_len)
    gen = torch.Generator("cpu").manual_seed(seed + 1)
    kv32 = wl.kv.float().reshape(-1, D_K).clone()
    for b, n in enumerate(lens):
        t0 = n // 3
        t = torch.arange(t0, n)
        rows = wl.block_table[b, t // block_size].long() * block_size + t % block_size
        alpha = 0.5 + 2.5 * (t - t0).float() / max(n - 1 - t0, 1)
        noise = 0.2 * torch.randn((len(t), D_K), generator=gen)
        qdir = wl.q[b, 0] if wl.q_len == 1 else wl.q[b, -1, 0]
        kv32[rows] = alpha[:, None] * qdir.float()[None, :] + noise
    if kv_dtype == "bf16":
        wl.kv = kv32.to(torch.bfloat16).view(wl.kv.shape)
    else:
        codes, wl.kv_scale = quantize_e4m3(kv32)
        wl.kv = codes.view(wl.kv.shape)
        wl.kv_dtype = "fp8"
    wl.name = f"rising-{kv_dtype}-H{num_heads}-q{q_len}"
    return wl


def nan_code(kv_dtype: str) -> int:
    return 0x7F if kv_dtype == "fp8" else 0x7FC0


def poison_unused(wl: Workload) -> None:
    """NaN in every slot no request may read: unused blocks and tail slots."""
    raw = wl.kv.view(torch.uint8) if wl.kv_dtype == "fp8" else wl.kv.view(torch.int16)
    code = nan_code(wl.kv_dtype)
    referenced = torch.zeros(wl.num_blocks, dtype=torch.bool)
    bs = wl.block_size
    for b in range(wl.batch):
        n = int(wl.seq_lens[b])
        k = (n + bs - 1) // bs
        if k:
            referenced[wl.block_table[b, :k].long()] = True
            last = int(wl.block_table[b, k - 1])
            tail = n - (k - 1) * bs
            raw[last, tail:, :] = code
    raw[~referenced] = code


def make_config(name: str, **overrides) -> Workload:
    cfg = dict(CONFIGS[name])
    cfg.update(overrides)
    return make_workload(name, **cfg)

