"""fp64 CPU oracle for absorbed MLA decode over a paged latent KV cache.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the CPU-baseline
leg of the benchmark are the only callers. The product path (the HIP library
and its binding) never imports this package, and this package imports nothing
from the product path.

The arithmetic lives in ``mla_oracle.c`` (plain C, fp64, one sequential loop
per (request, query token, head), OpenMP across them). This module builds it with gcc and
marshals numpy arrays through ctypes. See the C file's header for what is
computed and which passage of each page it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "mla_oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle_mla.so")

D_K = 576   # key width: 512 kv_c + 64 rope
D_V = 512   # value width: kv_c

_lib_cache: dict[str, ctypes.CDLL] = {}


def build(source: str = SOURCE, output: str = LIBRARY) -> str:
    """Compile the oracle with gcc (-O2, no fast-math) into a shared library."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
           "-o", output, source, "-lm"]
    subprocess.run(cmd, check=True)
    return output


def _bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.oracle_mla_attend.argtypes = [vp, vp, i32, ctypes.c_float, vp, vp, i64, i64, i64,
                                      i64, i64, i64, ctypes.c_float, vp, vp, vp, i64, vp, vp]
    lib.oracle_mla_attend.restype = i32
    lib.oracle_mla_attend_sparse.argtypes = [vp, vp, i32, ctypes.c_float, vp, vp, i64, i64,
                                             i64, i64, i64, ctypes.c_float, vp, i64, vp, vp]
    lib.oracle_mla_attend_sparse.restype = i32
    lib.oracle_gemm_fp8_blockscale.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp]
    lib.oracle_gemm_fp8_blockscale.restype = i32
    lib.oracle_absorb.argtypes = [vp, vp, i64, i64, i64, i64, vp]
    lib.oracle_absorb.restype = i32
    lib.oracle_lse_merge.argtypes = [vp, vp, i64, i64, vp, vp]
    lib.oracle_lse_merge.restype = i32
    lib.oracle_e4m3_to_double.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_to_double.restype = ctypes.c_double
    lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_double.restype = ctypes.c_double
    return lib


def load(path: str = LIBRARY) -> "Oracle":
    """Load (building first if absent) the oracle library at ``path``."""
    if path not in _lib_cache:
        if not os.path.exists(path):
            if path != LIBRARY:
                raise FileNotFoundError(path)
            build()
        _lib_cache[path] = _bind(ctypes.CDLL(path))
    return Oracle(_lib_cache[path])


def _ptr(a: np.ndarray) -> ctypes.c_void_p:
    return ctypes.c_void_p(a.ctypes.data)


class Oracle:
    """Thin numpy front end over one loaded copy of the C oracle."""

    def __init__(self, lib: ctypes.CDLL):
        self.lib = lib

    def attend(self, q_bits, kv, block_table, seq_lens, block_size, scale,
               kv_fp8=False, kv_scale=1.0, req=None, tok_begin=None, tok_end=None):
        """Exact attention of (request, token range) items.

        q_bits      uint16 [B, H, 576] (one query token per request) or
                    [B, q_len, H, 576] (q_len query tokens, causal): bf16 bits
        kv          uint16 [NB, bs, 576] bf16 bits, or uint8 E4M3FN codes if kv_fp8
        block_table int32 [B, max_blocks]; seq_lens int32 [B]
        req         int32 [n] request of each item (default: every request)
        tok_begin/end int64 [n] token range per item (default: whole request)
        Returns (out float64 [n, H, 512], lse float64 [n, H]), with a q_len
        axis after n when q_bits has one.
        """
        q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
        kv = np.ascontiguousarray(kv, dtype=np.uint8 if kv_fp8 else np.uint16)
        block_table = np.ascontiguousarray(block_table, dtype=np.int32)
        seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
        multi = q_bits.ndim == 4
        if multi:
            batch, q_len, num_heads, dk = q_bits.shape
        else:
            (batch, num_heads, dk), q_len = q_bits.shape, 1
        if dk != D_K or kv.shape[-1] != D_K or kv.shape[1] != block_size:
            raise ValueError("shape mismatch")
        if req is None:
            req = np.arange(batch, dtype=np.int32)
        req = np.ascontiguousarray(req, dtype=np.int32)
        n = req.shape[0]
        if tok_begin is None:
            tok_begin = np.zeros(n, dtype=np.int64)
        if tok_end is None:
            tok_end = seq_lens[req].astype(np.int64)
        tok_begin = np.ascontiguousarray(tok_begin, dtype=np.int64)
        tok_end = np.ascontiguousarray(tok_end, dtype=np.int64)
        out = np.empty((n, q_len, num_heads, D_V), dtype=np.float64)
        lse = np.empty((n, q_len, num_heads), dtype=np.float64)
        rc = self.lib.oracle_mla_attend(
            _ptr(q_bits), _ptr(kv), int(bool(kv_fp8)), float(kv_scale), _ptr(block_table),
            _ptr(seq_lens), batch, num_heads, q_len, block_size, block_table.shape[1],
            kv.shape[0], float(scale), _ptr(req), _ptr(tok_begin), _ptr(tok_end), n, _ptr(out),
            _ptr(lse))
        if rc != 0:
            raise ValueError(f"oracle_mla_attend failed with status {rc}")
        if not multi:
            return out[:, 0], lse[:, 0]
        return out, lse

    def attend_sparse(self, q_bits, kv, block_table, seq_lens, block_size, scale, indices,
                      kv_fp8=False, kv_scale=1.0):
        """Attention of each request over the token positions it lists.

        q_bits   uint16 [B, H, 576] bf16 bits; indices int32 [B, topk] token
                 positions (entries outside [0, seq_len) are skipped)
        Returns (out float64 [B, H, 512], lse float64 [B, H]).
        """
        q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
        kv = np.ascontiguousarray(kv, dtype=np.uint8 if kv_fp8 else np.uint16)
        block_table = np.ascontiguousarray(block_table, dtype=np.int32)
        seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
        indices = np.ascontiguousarray(indices, dtype=np.int32)
        batch, num_heads, dk = q_bits.shape
        if dk != D_K or kv.shape[-1] != D_K or kv.shape[1] != block_size or \
                indices.ndim != 2 or indices.shape[0] != batch:
            raise ValueError("shape mismatch")
        out = np.empty((batch, num_heads, D_V), dtype=np.float64)
        lse = np.empty((batch, num_heads), dtype=np.float64)
        rc = self.lib.oracle_mla_attend_sparse(
            _ptr(q_bits), _ptr(kv), int(bool(kv_fp8)), float(kv_scale), _ptr(block_table),
            _ptr(seq_lens), batch, num_heads, block_size, block_table.shape[1], kv.shape[0],
            float(scale), _ptr(indices), indices.shape[1], _ptr(out), _ptr(lse))
        if rc != 0:
            raise ValueError(f"oracle_mla_attend_sparse failed with status {rc}")
        return out, lse

    def lse_merge(self, part_out, part_lse):
        """Merge normalised partials [S, H, 512] / [S, H] of one request."""
        part_out = np.ascontiguousarray(part_out, dtype=np.float64)
        part_lse = np.ascontiguousarray(part_lse, dtype=np.float64)
        n_parts, num_heads = part_lse.shape
        out = np.empty((num_heads, D_V), dtype=np.float64)
        lse = np.empty((num_heads,), dtype=np.float64)
        rc = self.lib.oracle_lse_merge(_ptr(part_out), _ptr(part_lse), n_parts, num_heads,
                                       _ptr(out), _ptr(lse))
        if rc != 0:
            raise ValueError(f"oracle_lse_merge failed with status {rc}")
        return out, lse

    def gemm_fp8_blockscale(self, a, a_scale, b, b_scale):
        """c [m, n] float64 of the block-scaled E4M3 projection (see the C source):
        a uint8 [m, k], a_scale float32 [m, k/128], b uint8 [n, k],
        b_scale float32 [ceil(n/128), k/128]."""
        a = np.ascontiguousarray(a, dtype=np.uint8)
        b = np.ascontiguousarray(b, dtype=np.uint8)
        a_scale = np.ascontiguousarray(a_scale, dtype=np.float32)
        b_scale = np.ascontiguousarray(b_scale, dtype=np.float32)
        m, k = a.shape
        n = b.shape[0]
        if b.shape[1] != k or k % 128 or a_scale.shape != (m, k // 128) or \
                b_scale.shape != ((n + 127) // 128, k // 128):
            raise ValueError("shape mismatch")
        c = np.empty((m, n), dtype=np.float64)
        rc = self.lib.oracle_gemm_fp8_blockscale(_ptr(a), _ptr(a_scale), _ptr(b), _ptr(b_scale),
                                                 m, n, k, _ptr(c))
        if rc != 0:
            raise ValueError(f"oracle_gemm_fp8_blockscale failed with status {rc}")
        return c

    def absorb(self, x_bits, w_bits):
        """Per-head product c [B, H, n] float64 of x bf16 bits [B, H, k] and
        w bf16 bits [H, k, n] (see the C source)."""
        x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
        w_bits = np.ascontiguousarray(w_bits, dtype=np.uint16)
        batch, heads, k = x_bits.shape
        if w_bits.shape[:2] != (heads, k):
            raise ValueError("shape mismatch")
        n = w_bits.shape[2]
        c = np.empty((batch, heads, n), dtype=np.float64)
        rc = self.lib.oracle_absorb(_ptr(x_bits), _ptr(w_bits), batch, heads, k, n, _ptr(c))
        if rc != 0:
            raise ValueError(f"oracle_absorb failed with status {rc}")
        return c

    @staticmethod
    def quant_fp8_groups(x):
        """Per token and 128-wide group: scale = max(amax, 1e-10) / 448 and
        code = E4M3FN(round to nearest even of clamp(x / scale, +-448)), every
        step in fp32 (numpy's IEEE division; torch's E4M3FN cast rounds to
        nearest even). x: bf16 [m, k] as a torch tensor. Returns (codes uint8
        [m, k], scales float32 [m, k/128])."""
        import torch
        m, k = x.shape
        if k % 128:
            raise ValueError("k must be a multiple of 128")
        xf = x.float().numpy().reshape(m, k // 128, 128)
        amax = np.abs(xf).max(axis=2)
        scale = np.maximum(amax, np.float32(1e-10)).astype(np.float32) / np.float32(448.0)
        y = (xf / scale[:, :, None]).astype(np.float32)
        y = np.clip(y, np.float32(-448.0), np.float32(448.0))
        codes = torch.from_numpy(y.reshape(m, k)).to(torch.float8_e4m3fn).view(torch.uint8)
        return codes.numpy(), scale.astype(np.float32)

    def e4m3_to_double(self, codes):
        codes = np.asarray(codes, dtype=np.uint8)
        return np.array([self.lib.oracle_e4m3_to_double(int(c)) for c in codes.ravel()],
                        dtype=np.float64).reshape(codes.shape)

    def bf16_to_double(self, bits):
        bits = np.asarray(bits, dtype=np.uint16)
        return np.array([self.lib.oracle_bf16_to_double(int(c)) for c in bits.ravel()],
                        dtype=np.float64).reshape(bits.shape)
