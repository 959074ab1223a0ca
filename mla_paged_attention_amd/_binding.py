"""ctypes binding of libmla_mi355x.so (the C ABI in include/mla.h).

Argument marshalling only: shapes and dtypes are checked against the same
constants the header defines, torch supplies device memory and the current
HIP stream, and every step of the computation runs in the library's kernels.
There is no fallback: if the library is missing or the device is not gfx950
the call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY_PATH = os.path.join(HERE, "libmla_mi355x.so")

HEAD_DIM_K = 576
HEAD_DIM_V = 512
MAX_HEADS = 128
MAX_QUERY_LEN = 16
MAX_FORCED_SPLITS = 16
MAX_TOPK = 65536
FP8_GROUP = 128
GEMM_MAX_M = GEMM_MAX_N = GEMM_MAX_K = 65536
BLOCK_SIZES = (16, 32, 64, 128)

MLA_OK = 0
MLA_ERR_INVALID_ARG = -1
MLA_ERR_UNSUPPORTED = -2
MLA_ERR_WORKSPACE_TOO_SMALL = -3
MLA_ERR_NO_DEVICE = -4
MLA_ERR_HIP = -5

MLA_KV_BF16 = 0
MLA_KV_FP8_E4M3 = 1

EXPORTED_SYMBOLS = ("mla_get_workspace_size", "mla_get_workspace_size_multi_token",
                    "mla_get_workspace_size_sparse", "mla_decode", "mla_decode_multi_token",
                    "mla_decode_profiled", "mla_decode_sparse", "mla_decode_sparse_profiled",
                    "mla_combine", "mla_quant_fp8_groups", "mla_gemm_fp8_blockscale",
                    "mla_absorb_q", "mla_absorb_out", "mla_decode_noalloc",
                    "mla_status_string", "mla_abi_version")
NOALLOC_SCRATCH_BYTES = 96 << 20

_lib = None
_lock = threading.Lock()


class MLAError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what} failed: {status_string(status)} ({status})")


def _bind(lib: ctypes.CDLL) -> None:
    vp, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                             ctypes.c_size_t)
    lib.mla_get_workspace_size.argtypes = [i64, i64, i64, i64, i64]
    lib.mla_get_workspace_size.restype = sz
    lib.mla_get_workspace_size_multi_token.argtypes = [i64, i64, i64, i64, i64, i64]
    lib.mla_get_workspace_size_multi_token.restype = sz
    decode_args = [vp, vp, vp, vp, vp, vp, f32, i32, i32, i32, i32, i32, i32, i32, f32, vp, sz,
                   vp]
    lib.mla_decode.argtypes = decode_args
    lib.mla_decode.restype = i32
    multi_args = decode_args[:8] + [i32] + decode_args[8:]   # q_len after num_heads
    lib.mla_decode_multi_token.argtypes = multi_args
    lib.mla_decode_multi_token.restype = i32
    lib.mla_decode_profiled.argtypes = multi_args + [ctypes.POINTER(vp)]
    lib.mla_decode_profiled.restype = i32
    lib.mla_decode_noalloc.argtypes = multi_args[:16] + [vp]  # no workspace arguments
    lib.mla_decode_noalloc.restype = i32
    sparse_args = decode_args[:4] + [vp, i32] + decode_args[4:]  # indices, topk after seq_lens
    lib.mla_decode_sparse.argtypes = sparse_args
    lib.mla_decode_sparse.restype = i32
    lib.mla_decode_sparse_profiled.argtypes = sparse_args + [ctypes.POINTER(vp)]
    lib.mla_decode_sparse_profiled.restype = i32
    lib.mla_get_workspace_size_sparse.argtypes = [i64, i64, i64, i64, i64]
    lib.mla_get_workspace_size_sparse.restype = sz
    lib.mla_combine.argtypes = [vp, vp, vp, vp, vp, i32, i32, vp]
    lib.mla_combine.restype = i32
    lib.mla_quant_fp8_groups.argtypes = [vp, vp, vp, i32, i32, vp]
    lib.mla_quant_fp8_groups.restype = i32
    lib.mla_gemm_fp8_blockscale.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, vp]
    lib.mla_gemm_fp8_blockscale.restype = i32
    lib.mla_absorb_q.argtypes = [vp, vp, vp, vp, i32, i32, vp]
    lib.mla_absorb_q.restype = i32
    lib.mla_absorb_out.argtypes = [vp, vp, vp, i32, i32, vp]
    lib.mla_absorb_out.restype = i32
    lib.mla_status_string.argtypes = [i32]
    lib.mla_status_string.restype = ctypes.c_char_p
    lib.mla_abi_version.argtypes = []
    lib.mla_abi_version.restype = i32


def library() -> ctypes.CDLL:
    """Load the in-tree library once (torch is imported first so that both
    share the one HIP runtime already mapped under the same soname)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIBRARY_PATH):
                raise RuntimeError(
                    f"{LIBRARY_PATH} is not built; run `python -m mla_paged_attention_amd.build`")
            lib = ctypes.CDLL(LIBRARY_PATH)
            _bind(lib)
            _lib = lib
    return _lib


def status_string(status: int) -> str:
    return library().mla_status_string(int(status)).decode()


def abi_version() -> int:
    return int(library().mla_abi_version())


def get_workspace_size(batch: int, num_heads: int, max_seq_len: int, num_splits: int = 0,
                       num_cus: int = 0, q_len: int = 1) -> int:
    if q_len == 1:
        return int(library().mla_get_workspace_size(batch, num_heads, max_seq_len, num_splits,
                                                    num_cus))
    return int(library().mla_get_workspace_size_multi_token(batch, num_heads, q_len,
                                                            max_seq_len, num_splits, num_cus))


def get_workspace_size_sparse(batch: int, num_heads: int, topk: int, num_splits: int = 0,
                              num_cus: int = 0) -> int:
    return int(library().mla_get_workspace_size_sparse(batch, num_heads, topk, num_splits,
                                                       num_cus))


def _ptr(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _stream_handle(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


_workspaces: dict = {}


def _launch_stream(device: torch.device, stream):
    return stream if stream is not None else torch.cuda.current_stream(device)


def workspace_for(device: torch.device, stream, nbytes: int) -> torch.Tensor:
    """Per (device, stream) uninitialised workspace, grown on demand.

    Calls on one stream are ordered, so reusing the buffer between them is
    safe. The buffer is allocated on the launch stream itself, so when a
    larger call replaces it, torch's allocator hands the old block out again
    only to later work on that same stream. A graph capture must bring its
    own workspace: a replayed graph keeps using the buffer it captured, which
    this cache may free or replace in the meantime."""
    if torch.cuda.is_current_stream_capturing():
        raise RuntimeError("pass workspace= when capturing a graph: the binding's cached "
                           "workspace may be replaced while the graph still uses it")
    s = _launch_stream(device, stream)
    key = (device.index, s.cuda_stream)
    buf = _workspaces.get(key)
    if buf is None or buf.numel() < nbytes:
        with torch.cuda.stream(s):
            buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        _workspaces[key] = buf
    return buf


def release_workspaces() -> None:
    """Drop the cached per-stream workspaces (their memory returns to torch's
    allocator once the work queued on their streams has run)."""
    _workspaces.clear()


def _empty_on(stream, shape, dtype, device):
    """An output buffer allocated on the launch stream (so that torch's
    allocator orders its reuse after the kernels that write it)."""
    with torch.cuda.stream(_launch_stream(device, stream)):
        return torch.empty(shape, dtype=dtype, device=device)


def _kv_dtype(kv: torch.Tensor) -> int:
    if kv.dtype == torch.bfloat16:
        return MLA_KV_BF16
    if kv.dtype in (torch.uint8, torch.float8_e4m3fn):
        return MLA_KV_FP8_E4M3
    raise TypeError(f"kv_cache dtype {kv.dtype} is not bf16 or E4M3 (uint8/float8_e4m3fn)")


def decode(q: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor,
           seq_lens: torch.Tensor, *, scale: float, num_splits: int = 0, kv_scale: float = 1.0,
           out: torch.Tensor | None = None, lse: torch.Tensor | bool | None = True,
           workspace: torch.Tensor | None = None, stream=None, events=None):
    """Absorbed MLA decode over a paged cache (see include/mla.h, mla_decode).

    q [B, H, 576] bf16, or [B, q_len, H, 576] for q_len query tokens per request
    under the causal mask of mla_decode_multi_token; kv_cache [num_blocks,
    block_size, 576] bf16 or E4M3 (uint8 / float8_e4m3fn) with per-tensor
    kv_scale; block_table [B, max_blocks] int32; seq_lens [B] int32. Returns
    (out [B, (q_len,) H, 512] bf16, lse [B, (q_len,) H] fp32 or None).
    `events`: four torch.cuda.Event(enable_timing=True) to record around the
    split plan, attention and combine kernels (mla_decode_profiled).
    """
    if q.dim() not in (3, 4) or q.shape[-1] != HEAD_DIM_K or q.dtype != torch.bfloat16:
        raise ValueError("q must be [batch, num_heads, 576] or [batch, q_len, num_heads, 576] "
                         "bf16")
    if kv_cache.dim() != 3 or kv_cache.shape[2] != HEAD_DIM_K:
        raise ValueError("kv_cache must be [num_blocks, block_size, 576]")
    kv_dtype = _kv_dtype(kv_cache)
    batch, num_heads = q.shape[0], q.shape[-2]
    q_len = q.shape[1] if q.dim() == 4 else 1
    num_blocks, block_size, _ = kv_cache.shape
    if block_table.dim() != 2 or block_table.shape[0] != batch or block_table.dtype != torch.int32:
        raise ValueError("block_table must be [batch, max_blocks] int32")
    if seq_lens.shape != (batch,) or seq_lens.dtype != torch.int32:
        raise ValueError("seq_lens must be [batch] int32")
    dev = q.device
    for name, t in (("q", q), ("kv_cache", kv_cache), ("block_table", block_table),
                    ("seq_lens", seq_lens)):
        if t.device != dev or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous on {dev}")
    lead = tuple(q.shape[:-1])                     # (B, H) or (B, q_len, H)
    if out is None:
        out = _empty_on(stream, lead + (HEAD_DIM_V,), torch.bfloat16, dev)
    elif tuple(out.shape) != lead + (HEAD_DIM_V,) or out.dtype != torch.bfloat16 or \
            out.device != dev or not out.is_contiguous():
        raise ValueError(f"out must be contiguous {lead + (HEAD_DIM_V,)} bf16 on {dev}")
    if lse is True:
        lse = _empty_on(stream, lead, torch.float32, dev)
    elif lse is False:
        lse = None
    elif lse is not None and (tuple(lse.shape) != lead or lse.dtype != torch.float32 or
                              lse.device != dev or not lse.is_contiguous()):
        raise ValueError(f"lse must be contiguous {lead} fp32 on {dev}")
    max_blocks = block_table.shape[1]
    need = get_workspace_size(batch, num_heads, max_blocks * block_size, num_splits, 0, q_len)
    if workspace is None:
        workspace = workspace_for(dev, stream, need)
    head = (_ptr(q), _ptr(kv_cache), _ptr(block_table), _ptr(seq_lens), _ptr(out), _ptr(lse),
            float(scale), num_heads)
    tail = (block_size, num_splits, batch, max_blocks, num_blocks, kv_dtype, float(kv_scale),
            _ptr(workspace), workspace.numel() * workspace.element_size(),
            _stream_handle(stream))
    lib = library()
    if events is not None:
        arr = (ctypes.c_void_p * 4)(*[ctypes.c_void_p(e.cuda_event) for e in events])
        st = lib.mla_decode_profiled(*head, q_len, *tail, arr)
        what = "mla_decode_profiled"
    elif q_len == 1 and q.dim() == 3:
        st = lib.mla_decode(*head, *tail)
        what = "mla_decode"
    else:
        st = lib.mla_decode_multi_token(*head, q_len, *tail)
        what = "mla_decode_multi_token"
    if st != MLA_OK:
        raise MLAError(st, what)
    return out, lse


def decode_noalloc(q: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor,
                   seq_lens: torch.Tensor, *, scale: float, out: torch.Tensor,
                   lse: torch.Tensor | None, num_splits: int = 0, kv_scale: float = 1.0,
                   stream=None):
    """decode() through mla_decode_noalloc: no workspace, and the library
    allocates nothing (see include/mla.h). The caller passes out (and lse, or
    None); calls that overlap on one GPU race on its scratch array."""
    if q.dim() not in (3, 4) or q.shape[-1] != HEAD_DIM_K or q.dtype != torch.bfloat16:
        raise ValueError("q must be [batch, num_heads, 576] or [batch, q_len, num_heads, 576] "
                         "bf16")
    if kv_cache.dim() != 3 or kv_cache.shape[2] != HEAD_DIM_K:
        raise ValueError("kv_cache must be [num_blocks, block_size, 576]")
    kv_dtype = _kv_dtype(kv_cache)
    batch, num_heads = q.shape[0], q.shape[-2]
    q_len = q.shape[1] if q.dim() == 4 else 1
    num_blocks, block_size, _ = kv_cache.shape
    if block_table.dim() != 2 or block_table.shape[0] != batch or block_table.dtype != torch.int32:
        raise ValueError("block_table must be [batch, max_blocks] int32")
    if seq_lens.shape != (batch,) or seq_lens.dtype != torch.int32:
        raise ValueError("seq_lens must be [batch] int32")
    lead = tuple(q.shape[:-1])
    dev = q.device
    for name, t in (("q", q), ("kv_cache", kv_cache), ("block_table", block_table),
                    ("seq_lens", seq_lens)):
        if t.device != dev or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous on {dev}")
    if tuple(out.shape) != lead + (HEAD_DIM_V,) or out.dtype != torch.bfloat16 or \
            out.device != dev or not out.is_contiguous():
        raise ValueError(f"out must be contiguous {lead + (HEAD_DIM_V,)} bf16 on {dev}")
    if lse is not None and (tuple(lse.shape) != lead or lse.dtype != torch.float32 or
                            lse.device != dev or not lse.is_contiguous()):
        raise ValueError(f"lse must be contiguous {lead} fp32 on {dev}")
    st = library().mla_decode_noalloc(
        _ptr(q), _ptr(kv_cache), _ptr(block_table), _ptr(seq_lens), _ptr(out), _ptr(lse),
        float(scale), num_heads, q_len, block_size, num_splits, batch, block_table.shape[1],
        num_blocks, kv_dtype, float(kv_scale), _stream_handle(stream))
    if st != MLA_OK:
        raise MLAError(st, "mla_decode_noalloc")
    return out, lse


def decode_sparse(q: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor,
                  seq_lens: torch.Tensor, indices: torch.Tensor, *, scale: float,
                  num_splits: int = 0, kv_scale: float = 1.0, out: torch.Tensor | None = None,
                  lse: torch.Tensor | bool | None = True, workspace: torch.Tensor | None = None,
                  stream=None, events=None):
    """Sparse MLA decode (see include/mla.h, mla_decode_sparse): request b attends
    to the token positions indices[b] lists ([B, topk] int32; entries outside
    [0, seq_len) are skipped). Other arguments and results as for decode()
    with one query token per request."""
    if q.dim() != 3 or q.shape[2] != HEAD_DIM_K or q.dtype != torch.bfloat16:
        raise ValueError("q must be [batch, num_heads, 576] bf16")
    if kv_cache.dim() != 3 or kv_cache.shape[2] != HEAD_DIM_K:
        raise ValueError("kv_cache must be [num_blocks, block_size, 576]")
    kv_dtype = _kv_dtype(kv_cache)
    batch, num_heads, _ = q.shape
    num_blocks, block_size, _ = kv_cache.shape
    if block_table.dim() != 2 or block_table.shape[0] != batch or block_table.dtype != torch.int32:
        raise ValueError("block_table must be [batch, max_blocks] int32")
    if seq_lens.shape != (batch,) or seq_lens.dtype != torch.int32:
        raise ValueError("seq_lens must be [batch] int32")
    if indices.dim() != 2 or indices.shape[0] != batch or indices.dtype != torch.int32:
        raise ValueError("indices must be [batch, topk] int32")
    topk = indices.shape[1]
    dev = q.device
    for name, t in (("q", q), ("kv_cache", kv_cache), ("block_table", block_table),
                    ("seq_lens", seq_lens), ("indices", indices)):
        if t.device != dev or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous on {dev}")
    if out is None:
        out = _empty_on(stream, (batch, num_heads, HEAD_DIM_V), torch.bfloat16, dev)
    elif tuple(out.shape) != (batch, num_heads, HEAD_DIM_V) or out.dtype != torch.bfloat16 or \
            out.device != dev or not out.is_contiguous():
        raise ValueError(f"out must be contiguous [{batch}, {num_heads}, 512] bf16 on {dev}")
    if lse is True:
        lse = _empty_on(stream, (batch, num_heads), torch.float32, dev)
    elif lse is False:
        lse = None
    elif lse is not None and (tuple(lse.shape) != (batch, num_heads) or
                              lse.dtype != torch.float32 or lse.device != dev or
                              not lse.is_contiguous()):
        raise ValueError(f"lse must be contiguous [{batch}, {num_heads}] fp32 on {dev}")
    if workspace is None:
        need = get_workspace_size_sparse(batch, num_heads, max(topk, 1), num_splits, 0)
        workspace = workspace_for(dev, stream, need)
    args = (_ptr(q), _ptr(kv_cache), _ptr(block_table), _ptr(seq_lens), _ptr(indices), topk,
            _ptr(out), _ptr(lse), float(scale), num_heads, block_size, num_splits, batch,
            block_table.shape[1], num_blocks, kv_dtype, float(kv_scale), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream_handle(stream))
    lib = library()
    if events is None:
        st = lib.mla_decode_sparse(*args)
    else:
        arr = (ctypes.c_void_p * 4)(*[ctypes.c_void_p(e.cuda_event) for e in events])
        st = lib.mla_decode_sparse_profiled(*args, arr)
    if st != MLA_OK:
        raise MLAError(st, "mla_decode_sparse")
    return out, lse


def _fp8_codes(t: torch.Tensor) -> bool:
    return t.dtype in (torch.uint8, torch.float8_e4m3fn)


def quant_fp8_groups(x: torch.Tensor, *, out: torch.Tensor | None = None,
                     scale: torch.Tensor | None = None, stream=None):
    """Per token and 128-wide group E4M3 quantisation of bf16 x [m, k] (see
    include/mla.h, mla_quant_fp8_groups). Returns (codes uint8 [m, k],
    scales fp32 [m, k/128])."""
    if x.dim() != 2 or x.dtype != torch.bfloat16 or not x.is_contiguous():
        raise ValueError("x must be contiguous [m, k] bf16")
    m, k = x.shape
    dev = x.device
    if out is None:
        out = torch.empty((m, k), dtype=torch.uint8, device=dev)
    if scale is None:
        scale = torch.empty((m, k // FP8_GROUP), dtype=torch.float32, device=dev)
    if tuple(out.shape) != (m, k) or not _fp8_codes(out) or not out.is_contiguous() or \
            tuple(scale.shape) != (m, k // FP8_GROUP) or scale.dtype != torch.float32 or \
            not scale.is_contiguous():
        raise ValueError("out must be contiguous [m, k] uint8, scale [m, k/128] fp32")
    st = library().mla_quant_fp8_groups(_ptr(x), _ptr(out), _ptr(scale), m, k,
                                        _stream_handle(stream))
    if st != MLA_OK:
        raise MLAError(st, "mla_quant_fp8_groups")
    return out, scale


def gemm_fp8_blockscale(a: torch.Tensor, a_scale: torch.Tensor, b: torch.Tensor,
                        b_scale: torch.Tensor, *, out: torch.Tensor | None = None, stream=None):
    """c [m, n] bf16 = dequant(a) @ dequant(b)^T with per-group activation scales
    a_scale [m, k/128] and per-128x128-block weight scales b_scale
    [ceil(n/128), k/128] (see include/mla.h, mla_gemm_fp8_blockscale)."""
    for name, t in (("a", a), ("b", b)):
        if t.dim() != 2 or not _fp8_codes(t) or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous 2-D E4M3 codes (uint8/float8_e4m3fn)")
    m, k = a.shape
    n = b.shape[0]
    if b.shape[1] != k:
        raise ValueError("a and b must share k")
    if tuple(a_scale.shape) != (m, k // FP8_GROUP) or a_scale.dtype != torch.float32 or \
            tuple(b_scale.shape) != ((n + FP8_GROUP - 1) // FP8_GROUP, k // FP8_GROUP) or \
            b_scale.dtype != torch.float32 or not a_scale.is_contiguous() or \
            not b_scale.is_contiguous():
        raise ValueError("a_scale must be [m, k/128] and b_scale [ceil(n/128), k/128] fp32")
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=a.device)
    elif tuple(out.shape) != (m, n) or out.dtype != torch.bfloat16 or not out.is_contiguous():
        raise ValueError(f"out must be contiguous [{m}, {n}] bf16")
    st = library().mla_gemm_fp8_blockscale(_ptr(a), _ptr(a_scale), _ptr(b), _ptr(b_scale),
                                           _ptr(out), m, n, k, _stream_handle(stream))
    if st != MLA_OK:
        raise MLAError(st, "mla_gemm_fp8_blockscale")
    return out


def _check_bf16(name, t, shape):
    if tuple(t.shape) != tuple(shape) or t.dtype != torch.bfloat16 or not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous {tuple(shape)} bf16")


def absorb_q(q_nope: torch.Tensor, w_uk: torch.Tensor, q_rope: torch.Tensor, *,
             out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """q [B, H, 576] = [q_nope [B, H, 128] . w_uk [H, 128, 512], q_rope [B, H, 64]]
    (see include/mla.h, mla_absorb_q)."""
    batch, heads = q_nope.shape[0], q_nope.shape[1]
    _check_bf16("q_nope", q_nope, (batch, heads, 128))
    _check_bf16("w_uk", w_uk, (heads, 128, 512))
    _check_bf16("q_rope", q_rope, (batch, heads, 64))
    if out is None:
        out = torch.empty((batch, heads, HEAD_DIM_K), dtype=torch.bfloat16, device=q_nope.device)
    _check_bf16("out", out, (batch, heads, HEAD_DIM_K))
    st = library().mla_absorb_q(_ptr(q_nope), _ptr(w_uk), _ptr(q_rope), _ptr(out), batch, heads,
                                _stream_handle(stream))
    if st != MLA_OK:
        raise MLAError(st, "mla_absorb_q")
    return out


def absorb_out(o_latent: torch.Tensor, w_uv: torch.Tensor, *, out: torch.Tensor | None = None,
               stream=None) -> torch.Tensor:
    """o [B, H, 128], o[b, h, v] = sum_c o_latent[b, h, c] w_uv[h, v, c], with
    o_latent [B, H, 512] and w_uv [H, 128, 512] (see include/mla.h, mla_absorb_out)."""
    batch, heads = o_latent.shape[0], o_latent.shape[1]
    _check_bf16("o_latent", o_latent, (batch, heads, HEAD_DIM_V))
    _check_bf16("w_uv", w_uv, (heads, 128, HEAD_DIM_V))
    if out is None:
        out = torch.empty((batch, heads, 128), dtype=torch.bfloat16, device=o_latent.device)
    _check_bf16("out", out, (batch, heads, 128))
    st = library().mla_absorb_out(_ptr(o_latent), _ptr(w_uv), _ptr(out), batch, heads,
                                  _stream_handle(stream))
    if st != MLA_OK:
        raise MLAError(st, "mla_absorb_out")
    return out


def combine(partial_out: torch.Tensor, partial_lse: torch.Tensor, split_indptr: torch.Tensor,
            *, out: torch.Tensor | None = None, lse: torch.Tensor | bool | None = True,
            stream=None):
    """LSE merge of split partials (see include/mla.h, mla_combine).

    partial_out [rows, H, 512] fp32; partial_lse [rows, H] fp32 (-inf = empty);
    split_indptr [B + 1] int32. Returns (out [B, H, 512] bf16, lse [B, H] or None).
    """
    if partial_out.dim() != 3 or partial_out.shape[2] != HEAD_DIM_V or \
            partial_out.dtype != torch.float32:
        raise ValueError("partial_out must be [rows, num_heads, 512] fp32")
    rows, num_heads, _ = partial_out.shape
    if partial_lse.shape != (rows, num_heads) or partial_lse.dtype != torch.float32:
        raise ValueError("partial_lse must be [rows, num_heads] fp32")
    if split_indptr.dim() != 1 or split_indptr.dtype != torch.int32:
        raise ValueError("split_indptr must be [batch + 1] int32")
    batch = split_indptr.shape[0] - 1
    dev = partial_out.device
    for name, t in (("partial_out", partial_out), ("partial_lse", partial_lse),
                    ("split_indptr", split_indptr)):
        if t.device != dev or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous on {dev}")
    if out is None:
        out = torch.empty((batch, num_heads, HEAD_DIM_V), dtype=torch.bfloat16, device=dev)
    if lse is True:
        lse = torch.empty((batch, num_heads), dtype=torch.float32, device=dev)
    elif lse is False:
        lse = None
    st = library().mla_combine(_ptr(partial_out), _ptr(partial_lse), _ptr(split_indptr),
                               _ptr(out), _ptr(lse), batch, num_heads, _stream_handle(stream))
    if st != MLA_OK:
        raise MLAError(st, "mla_combine")
    return out, lse
