"""C-ABI boundary checks that need no GPU.

The library must load on a machine without a GPU, export every entry point
include/mla.h declares, agree with the Python binding on every constant, and
reject bad arguments before making any HIP call (so these paths are testable
here). With valid arguments and no device it reports MLA_ERR_NO_DEVICE.
No kernel is ever launched from this file: on a machine with a GPU the
checks that would reach the device are skipped.
"""
import ctypes
import os
import re
import subprocess

import pytest
import torch

import mla_paged_attention_amd as mla
from mla_paged_attention_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")
HAS_GPU = torch.cuda.is_available()

FAKE = 0x100000  # 256-byte aligned, never dereferenced (validation or no device)


def header_text():
    with open(HEADER) as f:
        return f.read()


def declared_functions():
    return sorted(set(re.findall(r"^\s*[\w\s\*]*?\b(mla_\w+)\s*\(", header_text(), re.M)))


def test_header_declares_the_abi():
    assert declared_functions() == sorted(B.EXPORTED_SYMBOLS)


def test_every_declared_symbol_is_exported():
    lib = mla.library()
    out = subprocess.run(["nm", "-D", "--defined-only", mla.LIBRARY_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (mla_\w+)", out))
    for name in declared_functions():
        assert name in exported, f"{name} declared in mla.h but not exported"
        assert getattr(lib, name) is not None


def test_constants_match_header():
    text = header_text()
    defines = dict(re.findall(r"#define (MLA_\w+) (\d+)", text))
    assert int(defines["MLA_HEAD_DIM_K"]) == mla.HEAD_DIM_K == 576
    assert int(defines["MLA_HEAD_DIM_V"]) == mla.HEAD_DIM_V == 512
    assert int(defines["MLA_MAX_HEADS"]) == mla.MAX_HEADS == 128
    assert int(defines["MLA_MAX_FORCED_SPLITS"]) == mla.MAX_FORCED_SPLITS == 16
    assert int(defines["MLA_MAX_QUERY_LEN"]) == mla.MAX_QUERY_LEN == 16
    assert int(defines["MLA_MAX_TOPK"]) == mla.MAX_TOPK == 65536
    enums = dict((k, int(v)) for k, v in re.findall(r"(MLA_\w+) = (-?\d+)", text))
    for name in ("MLA_OK", "MLA_ERR_INVALID_ARG", "MLA_ERR_UNSUPPORTED",
                 "MLA_ERR_WORKSPACE_TOO_SMALL", "MLA_ERR_NO_DEVICE", "MLA_ERR_HIP",
                 "MLA_KV_BF16", "MLA_KV_FP8_E4M3"):
        assert enums[name] == getattr(mla, name), name


def test_status_strings_and_version():
    for code in (0, -1, -2, -3, -4, -5):
        s = mla.status_string(code)
        assert s.startswith("MLA_") and "UNKNOWN" not in s
    assert mla.status_string(7) == "MLA_ERR_UNKNOWN"
    assert mla.abi_version() == 2


# ------------------------------------------------------------------ workspace size

def _layout(batch, heads, rows, parts=1):
    a = lambda x: (x + 255) // 256 * 256  # noqa: E731
    return (256 + a((batch + 1) * 4) + a((parts + 1) * 4) + a((batch + parts) * 16)
            + a(parts * 16) + a(rows * heads * 4) + a(rows * heads * 512 * 4))


def test_workspace_size_forced_mode():
    for batch, heads, splits in ((1, 16, 1), (7, 20, 2), (512, 16, 16), (128, 128, 16)):
        rows = batch * splits if splits > 1 else 0
        assert mla.get_workspace_size(batch, heads, 4096, splits, 0) == _layout(batch, heads, rows)


def test_workspace_size_auto_mode():
    # 256 CUs, 16 heads: up to 256 partitions -> at most 2 * 256 partial rows.
    assert mla.get_workspace_size(512, 16, 3072, 0, 0) == _layout(512, 16, 512, 256)
    assert mla.get_workspace_size(512, 16, 3072, 0, 256) == _layout(512, 16, 512, 256)
    # 128 heads: two workgroups (four 16-head tiles each) per partition -> 128.
    assert mla.get_workspace_size(128, 128, 32768, 0, 0) == _layout(128, 128, 256, 128)
    # 64 heads fit one workgroup per partition.
    assert mla.get_workspace_size(128, 64, 32768, 0, 0) == _layout(128, 64, 512, 256)
    # Never more rows than every request split into one piece per 16-token unit.
    assert mla.get_workspace_size(2, 16, 32, 0, 0) == _layout(2, 16, 4, 256)
    assert mla.get_workspace_size(2, 16, 16, 0, 0) == _layout(2, 16, 0, 256)


def test_workspace_size_multi_token():
    # q_len = 1 is the one-token query; rows are q_len * heads.
    for args in ((512, 16, 3072, 0, 0), (7, 20, 4096, 2, 0), (128, 128, 32768, 0, 0)):
        assert mla.get_workspace_size(*args, q_len=1) == mla.get_workspace_size(*args)
    # 16 heads x 4 tokens = 64 rows: one workgroup per partition, 256 partitions.
    assert mla.get_workspace_size(512, 16, 3072, 0, 0, q_len=4) == _layout(512, 64, 512, 256)
    # 128 heads x 2 tokens = 256 rows: four workgroups per partition -> 64.
    assert mla.get_workspace_size(128, 128, 32768, 0, 0, q_len=2) == _layout(128, 256, 128, 64)
    # Forced splits: batch * splits partial rows of q_len * heads.
    assert mla.get_workspace_size(3, 8, 100, 4, 0, q_len=3) == _layout(3, 24, 12)
    # 16 tokens x 128 heads = 2048 rows: 32 workgroups per partition -> 8 partitions.
    assert mla.get_workspace_size(4, 128, 1024, 0, 0, q_len=16) == _layout(4, 2048, 16, 8)
    for bad in (0, 17, -1):
        assert mla.get_workspace_size(2, 16, 100, 0, 0, q_len=bad) == 0


@pytest.mark.parametrize("args", [(-1, 16, 10, 0, 0), (1, 0, 10, 0, 0), (1, 129, 10, 0, 0),
                                  (1, 16, -1, 0, 0), (1, 16, 10, -1, 0), (1, 16, 10, 17, 0)])
def test_workspace_size_rejects(args):
    assert mla.get_workspace_size(*args) == 0


# ------------------------------------------------------------------ validation

def _decode(**over):
    a = dict(q=FAKE, kv=FAKE, bt=FAKE, sl=FAKE, out=FAKE, lse=None, scale=0.07, heads=16,
             bs=32, splits=0, batch=2, max_blocks=4, num_blocks=8, kv_dtype=0, kv_scale=1.0,
             ws=FAKE, ws_bytes=1 << 30)
    a.update(over)
    lib = mla.library()
    vp = lambda x: ctypes.c_void_p(x) if x is not None else None  # noqa: E731
    return lib.mla_decode(vp(a["q"]), vp(a["kv"]), vp(a["bt"]), vp(a["sl"]), vp(a["out"]),
                          vp(a["lse"]), a["scale"], a["heads"], a["bs"], a["splits"], a["batch"],
                          a["max_blocks"], a["num_blocks"], a["kv_dtype"], a["kv_scale"],
                          vp(a["ws"]), a["ws_bytes"], None)


INVALID = [
    dict(q=None), dict(kv=None), dict(bt=None), dict(sl=None), dict(out=None), dict(ws=None),
    dict(q=FAKE + 8), dict(kv=FAKE + 4), dict(out=FAKE + 2), dict(bt=FAKE + 2),
    dict(sl=FAKE + 1), dict(lse=FAKE + 2), dict(ws=FAKE + 16),
    dict(heads=0), dict(heads=129), dict(bs=8), dict(bs=48), dict(bs=256), dict(splits=-1),
    dict(splits=17), dict(batch=-1), dict(max_blocks=0), dict(num_blocks=0),
    dict(kv_dtype=2), dict(kv_dtype=0, kv_scale=0.5), dict(kv_dtype=1, kv_scale=0.0),
    dict(kv_dtype=1, kv_scale=float("inf")), dict(scale=float("nan")),
    dict(max_blocks=1 << 30),
]


@pytest.mark.parametrize("over", INVALID, ids=[str(d) for d in INVALID])
def test_decode_rejects_before_any_hip_call(over):
    assert _decode(**over) == mla.MLA_ERR_INVALID_ARG


def _decode_multi(q_len, **over):
    a = dict(q=FAKE, kv=FAKE, bt=FAKE, sl=FAKE, out=FAKE, lse=None, scale=0.07, heads=16,
             bs=32, splits=0, batch=2, max_blocks=4, num_blocks=8, kv_dtype=0, kv_scale=1.0,
             ws=FAKE, ws_bytes=1 << 30)
    a.update(over)
    vp = lambda x: ctypes.c_void_p(x) if x is not None else None  # noqa: E731
    return mla.library().mla_decode_multi_token(
        vp(a["q"]), vp(a["kv"]), vp(a["bt"]), vp(a["sl"]), vp(a["out"]), vp(a["lse"]),
        a["scale"], a["heads"], q_len, a["bs"], a["splits"], a["batch"], a["max_blocks"],
        a["num_blocks"], a["kv_dtype"], a["kv_scale"], vp(a["ws"]), a["ws_bytes"], None)


@pytest.mark.parametrize("q_len", [0, -1, 17])
def test_decode_multi_token_rejects_q_len(q_len):
    assert _decode_multi(q_len) == mla.MLA_ERR_INVALID_ARG


@pytest.mark.parametrize("over", INVALID[:8] + [dict(heads=129), dict(splits=17)],
                         ids=lambda d: str(d))
def test_decode_multi_token_rejects_like_decode(over):
    assert _decode_multi(2, **over) == mla.MLA_ERR_INVALID_ARG


def test_decode_multi_token_workspace_too_small():
    need = mla.get_workspace_size(2, 16, 4 * 32, 4, 0, q_len=3)
    assert need > mla.get_workspace_size(2, 16, 4 * 32, 4, 0)
    assert _decode_multi(3, splits=4, ws_bytes=need - 1) == mla.MLA_ERR_WORKSPACE_TOO_SMALL
    if not HAS_GPU:
        assert _decode_multi(3, splits=4, ws_bytes=need) == mla.MLA_ERR_NO_DEVICE


def test_decode_workspace_too_small():
    assert _decode(ws_bytes=128) == mla.MLA_ERR_WORKSPACE_TOO_SMALL
    need = mla.get_workspace_size(2, 16, 4 * 32, 4, 0)
    assert _decode(splits=4, ws_bytes=need - 1) == mla.MLA_ERR_WORKSPACE_TOO_SMALL


@pytest.mark.skipif(HAS_GPU, reason="would reach the device")
def test_decode_without_device():
    assert _decode() == mla.MLA_ERR_NO_DEVICE
    assert _decode(kv_dtype=1, kv_scale=0.01) == mla.MLA_ERR_NO_DEVICE
    assert _decode(batch=0, q=None, kv=None, bt=None, sl=None, out=None, ws=None) == \
        mla.MLA_ERR_NO_DEVICE


def test_decode_profiled_requires_events():
    lib = mla.library()
    args = [ctypes.c_void_p(FAKE)] * 5 + [None, 0.07, 16, 1, 32, 0, 2, 4, 8, 0, 1.0,
                                          ctypes.c_void_p(FAKE), 1 << 30, None]
    assert lib.mla_decode_profiled(*args, None) == mla.MLA_ERR_INVALID_ARG
    null_events = (ctypes.c_void_p * 4)(None, None, None, None)
    assert lib.mla_decode_profiled(*args, null_events) == mla.MLA_ERR_INVALID_ARG


def test_combine_rejects():
    lib = mla.library()
    f = ctypes.c_void_p(FAKE)
    assert lib.mla_combine(None, f, f, f, None, 2, 16, None) == mla.MLA_ERR_INVALID_ARG
    assert lib.mla_combine(f, f, f, f, None, -1, 16, None) == mla.MLA_ERR_INVALID_ARG
    assert lib.mla_combine(f, f, f, f, None, 2, 0, None) == mla.MLA_ERR_INVALID_ARG
    assert lib.mla_combine(ctypes.c_void_p(FAKE + 4), f, f, f, None, 2, 16, None) == \
        mla.MLA_ERR_INVALID_ARG
    if not HAS_GPU:
        assert lib.mla_combine(f, f, f, f, None, 2, 16, None) == mla.MLA_ERR_NO_DEVICE


def _layout_sparse(batch, heads, rows, parts, topk):
    a = lambda x: (x + 255) // 256 * 256  # noqa: E731
    stride = (topk + 15) // 16 * 16 + 64
    return _layout(batch, heads, rows, parts) + a(batch * stride * 4) + a(batch * 4) + a(1152)


def test_workspace_size_sparse():
    # The plan sees every request as topk tokens long.
    assert mla.get_workspace_size_sparse(512, 16, 2048, 0, 0) == \
        _layout_sparse(512, 16, 512, 256, 2048)
    assert mla.get_workspace_size_sparse(64, 128, 2048, 0, 0) == \
        _layout_sparse(64, 128, 256, 128, 2048)
    assert mla.get_workspace_size_sparse(3, 16, 100, 4, 0) == _layout_sparse(3, 16, 12, 1, 100)
    for bad in ((1, 16, 0, 0, 0), (1, 16, 65537, 0, 0), (1, 0, 10, 0, 0), (1, 16, 10, 17, 0),
                (-1, 16, 10, 0, 0)):
        assert mla.get_workspace_size_sparse(*bad) == 0


def _decode_sparse(**over):
    a = dict(q=FAKE, kv=FAKE, bt=FAKE, sl=FAKE, idx=FAKE, topk=64, out=FAKE, lse=None, scale=0.07,
             heads=16, bs=32, splits=0, batch=2, max_blocks=4, num_blocks=8, kv_dtype=0,
             kv_scale=1.0, ws=FAKE, ws_bytes=1 << 30)
    a.update(over)
    vp = lambda x: ctypes.c_void_p(x) if x is not None else None  # noqa: E731
    return mla.library().mla_decode_sparse(
        vp(a["q"]), vp(a["kv"]), vp(a["bt"]), vp(a["sl"]), vp(a["idx"]), a["topk"], vp(a["out"]),
        vp(a["lse"]), a["scale"], a["heads"], a["bs"], a["splits"], a["batch"], a["max_blocks"],
        a["num_blocks"], a["kv_dtype"], a["kv_scale"], vp(a["ws"]), a["ws_bytes"], None)


SPARSE_INVALID = [dict(idx=None), dict(idx=FAKE + 2), dict(topk=0), dict(topk=65537),
                  dict(topk=-1), dict(heads=129), dict(q=None), dict(bs=48),
                  dict(num_blocks=1 << 26, bs=64)]


@pytest.mark.parametrize("over", SPARSE_INVALID, ids=[str(d) for d in SPARSE_INVALID])
def test_decode_sparse_rejects(over):
    assert _decode_sparse(**over) == mla.MLA_ERR_INVALID_ARG


def test_decode_sparse_workspace_and_device():
    need = mla.get_workspace_size_sparse(2, 16, 64, 3, 0)
    assert _decode_sparse(splits=3, ws_bytes=need - 1) == mla.MLA_ERR_WORKSPACE_TOO_SMALL
    if not HAS_GPU:
        assert _decode_sparse(splits=3, ws_bytes=need) == mla.MLA_ERR_NO_DEVICE
        assert _decode_sparse() == mla.MLA_ERR_NO_DEVICE


def test_decode_sparse_profiled_requires_events():
    lib = mla.library()
    f = ctypes.c_void_p(FAKE)
    args = [f, f, f, f, f, 64, f, None, 0.07, 16, 32, 0, 2, 4, 8, 0, 1.0, f, 1 << 30, None]
    assert lib.mla_decode_sparse_profiled(*args, None) == mla.MLA_ERR_INVALID_ARG


def test_gemm_constants():
    text = header_text()
    defines = dict(re.findall(r"#define (MLA_\w+) (\d+)", text))
    assert int(defines["MLA_FP8_GROUP"]) == mla.FP8_GROUP == 128
    for name in ("MLA_GEMM_MAX_M", "MLA_GEMM_MAX_N", "MLA_GEMM_MAX_K"):
        assert int(defines[name]) == 65536


GEMM_INVALID = [(-1, 16, 128), (65537, 16, 128), (4, 0, 128), (4, 24, 128), (4, 16, 0),
                (4, 16, 64), (4, 16, 200), (4, 65552, 128), (4, 16, 65664)]


@pytest.mark.parametrize("mnk", GEMM_INVALID, ids=str)
def test_gemm_rejects_shapes(mnk):
    f = ctypes.c_void_p(FAKE)
    assert mla.library().mla_gemm_fp8_blockscale(f, f, f, f, f, *mnk, None) == \
        mla.MLA_ERR_INVALID_ARG


def test_gemm_rejects_pointers():
    lib = mla.library()
    f = ctypes.c_void_p(FAKE)
    bad = [(None, f, f, f, f), (f, None, f, f, f), (f, f, None, f, f), (f, f, f, None, f),
           (f, f, f, f, None), (ctypes.c_void_p(FAKE + 8), f, f, f, f),
           (f, f, ctypes.c_void_p(FAKE + 8), f, f), (f, f, f, f, ctypes.c_void_p(FAKE + 4)),
           (f, ctypes.c_void_p(FAKE + 2), f, f, f)]
    for ptrs in bad:
        assert lib.mla_gemm_fp8_blockscale(*ptrs, 4, 32, 256, None) == mla.MLA_ERR_INVALID_ARG
    if not HAS_GPU:
        assert lib.mla_gemm_fp8_blockscale(f, f, f, f, f, 4, 32, 256, None) == \
            mla.MLA_ERR_NO_DEVICE
        assert lib.mla_gemm_fp8_blockscale(None, None, None, None, None, 0, 32, 256, None) == \
            mla.MLA_ERR_NO_DEVICE


def test_quant_rejects():
    lib = mla.library()
    f = ctypes.c_void_p(FAKE)
    for args in ((f, f, f, -1, 128), (f, f, f, 4, 64), (f, f, f, 4, 0), (None, f, f, 4, 128),
                 (f, None, f, 4, 128), (f, f, None, 4, 128), (ctypes.c_void_p(FAKE + 2), f, f, 4, 128),
                 (f, ctypes.c_void_p(FAKE + 1), f, 4, 128)):
        assert lib.mla_quant_fp8_groups(*args, None) == mla.MLA_ERR_INVALID_ARG
    if not HAS_GPU:
        assert lib.mla_quant_fp8_groups(f, f, f, 4, 256, None) == mla.MLA_ERR_NO_DEVICE


def test_gemm_binding_rejects():
    a = torch.zeros((4, 256), dtype=torch.uint8)
    with pytest.raises(ValueError):
        mla.gemm_fp8_blockscale(a, torch.zeros((4, 1)), torch.zeros((32, 256), dtype=torch.uint8),
                                torch.zeros((1, 2)))
    with pytest.raises(ValueError):
        mla.gemm_fp8_blockscale(a.float(), torch.zeros((4, 2)), a, torch.zeros((1, 2)))


def test_plan_cost_total_bound():
    # batch * (1 + ceil(max_blocks * block_size / 16)) must stay within
    # 2^30 - 1: at block 64 and 2^20 blocks per row (2^22 + 1 units), 255
    # requests fit and 256 do not. A too-small workspace stops the accepted
    # case before any HIP call.
    big = dict(max_blocks=1 << 20, bs=64, num_blocks=1 << 20, ws_bytes=128)
    assert _decode(batch=256, **big) == mla.MLA_ERR_INVALID_ARG
    assert _decode(batch=255, **big) == mla.MLA_ERR_WORKSPACE_TOO_SMALL


def test_absorb_rejects():
    lib = mla.library()
    f = ctypes.c_void_p(FAKE)
    m = ctypes.c_void_p(FAKE + 8)
    for args in ((f, f, f, f, -1, 16), (f, f, f, f, 4, 0), (f, f, f, f, 4, 129),
                 (None, f, f, f, 4, 16), (f, None, f, f, 4, 16), (f, f, None, f, 4, 16),
                 (f, f, f, None, 4, 16), (m, f, f, f, 4, 16), (f, f, m, f, 4, 16)):
        assert lib.mla_absorb_q(*args, None) == mla.MLA_ERR_INVALID_ARG
    for args in ((f, f, f, -1, 16), (f, f, f, 4, 0), (None, f, f, 4, 16), (f, m, f, 4, 16)):
        assert lib.mla_absorb_out(*args, None) == mla.MLA_ERR_INVALID_ARG
    if not HAS_GPU:
        assert lib.mla_absorb_q(f, f, f, f, 4, 16, None) == mla.MLA_ERR_NO_DEVICE
        assert lib.mla_absorb_out(f, f, f, 4, 16, None) == mla.MLA_ERR_NO_DEVICE


def test_combine_accepts_multi_token_rows():
    lib = mla.library()
    f = ctypes.c_void_p(FAKE)
    assert lib.mla_combine(f, f, f, f, None, 2, 2049, None) == mla.MLA_ERR_INVALID_ARG
    if not HAS_GPU:
        assert lib.mla_combine(f, f, f, f, None, 2, 2048, None) == mla.MLA_ERR_NO_DEVICE


def test_binding_rejects_bad_tensors():
    q = torch.zeros((2, 16, 512), dtype=torch.bfloat16)
    kv = torch.zeros((4, 32, 576), dtype=torch.bfloat16)
    bt = torch.zeros((2, 2), dtype=torch.int32)
    sl = torch.zeros((2,), dtype=torch.int32)
    with pytest.raises(ValueError):
        mla.decode(q, kv, bt, sl, scale=0.1)
    with pytest.raises(TypeError):
        mla.decode(torch.zeros((2, 16, 576), dtype=torch.bfloat16),
                   kv.float(), bt, sl, scale=0.1)
    with pytest.raises(ValueError):
        mla.decode(torch.zeros((2, 16, 576), dtype=torch.bfloat16), kv, bt.long(), sl,
                   scale=0.1)


def test_cached_workspace_refused_under_graph_capture(monkeypatch):
    # A graph keeps using the buffer it captured, so the binding's cached
    # workspace is refused while a capture is under way (checked before any
    # allocation or HIP call).
    import torch

    import mla_paged_attention_amd as mla
    monkeypatch.setattr(torch.cuda, "is_current_stream_capturing", lambda: True)
    with pytest.raises(RuntimeError, match="capturing"):
        mla.workspace_for(torch.device("cuda", 0), None, 1024)


def _decode_noalloc(q_len=1, **over):
    a = dict(q=FAKE, kv=FAKE, bt=FAKE, sl=FAKE, out=FAKE, lse=None, scale=0.07, heads=16,
             bs=32, splits=0, batch=2, max_blocks=4, num_blocks=8, kv_dtype=0, kv_scale=1.0)
    a.update(over)
    vp = lambda x: ctypes.c_void_p(x) if x is not None else None  # noqa: E731
    return mla.library().mla_decode_noalloc(
        vp(a["q"]), vp(a["kv"]), vp(a["bt"]), vp(a["sl"]), vp(a["out"]), vp(a["lse"]),
        a["scale"], a["heads"], q_len, a["bs"], a["splits"], a["batch"], a["max_blocks"],
        a["num_blocks"], a["kv_dtype"], a["kv_scale"], None)


@pytest.mark.parametrize("over", [d for d in INVALID if "ws" not in d],
                         ids=lambda d: str(d))
def test_decode_noalloc_rejects_like_decode(over):
    assert _decode_noalloc(**over) == mla.MLA_ERR_INVALID_ARG


def test_decode_noalloc_scratch_size_in_header():
    text = open(HEADER).read()
    assert "#define MLA_NOALLOC_SCRATCH_BYTES (96ull << 20)" in text
    assert mla.NOALLOC_SCRATCH_BYTES == 96 << 20


@pytest.mark.skipif(HAS_GPU, reason="would reach the device")
def test_decode_noalloc_without_device():
    assert _decode_noalloc() == mla.MLA_ERR_NO_DEVICE
    assert _decode_noalloc(q_len=3, splits=16, batch=300, heads=128) == mla.MLA_ERR_NO_DEVICE


def test_bounds_check_build_matches_header():
    # The checked build exports the same ABI, and its error-word location and
    # bits in the internal launch header agree with include/mla.h.
    from mla_paged_attention_amd import build as hip_build
    text = open(HEADER).read()
    internal = open(os.path.join(ROOT, "mla_paged_attention_amd", "csrc",
                                 "mla_internal.h")).read()
    off = int(re.search(r"#define MLA_BOUNDS_WORD_OFFSET (\d+)", text).group(1))
    idx = int(re.search(r"kBoundsWordIndex = (\d+);", internal).group(1))
    assert off == 4 * idx
    assert int(re.search(r"#define MLA_BOUNDS_BAD_BLOCK (\d+)", text).group(1)) == \
        int(re.search(r"kBoundsBadBlock = (\d+);", internal).group(1))
    assert int(re.search(r"#define MLA_BOUNDS_BAD_SEQ_LEN (\d+)", text).group(1)) == \
        int(re.search(r"kBoundsBadSeqLen = (\d+);", internal).group(1))
    out = subprocess.run(["nm", "-D", "--defined-only", hip_build.CHECKED_LIBRARY],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (mla_\w+)", out))
    assert set(declared_functions()) <= exported


def test_peaks_library_exports_what_the_bench_binds():
    # The calibration library is separate from the decode library; the bench
    # binds these five entry points by name.
    from mla_paged_attention_amd import build as hip_build
    out = subprocess.run(["nm", "-D", "--defined-only", hip_build.PEAKS_LIBRARY],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (peaks_\w+)", out))
    assert exported == {"peaks_stream_lds", "peaks_stream_perm", "peaks_gather_rows",
                        "peaks_read", "peaks_mfma"}
