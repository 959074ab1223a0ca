"""The bounds-check build reports corrupt device-side inputs.

libmla_mi355x_checked.so is the decode library compiled with
MLA_BOUNDS_CHECK=1. It clamps exactly as the release build does (a block id
outside the cache is read as block 0, a seq_len outside [0, capacity] is
clamped), so every access stays in bounds and nothing faults, and it also ORs
MLA_BOUNDS_BAD_BLOCK / MLA_BOUNDS_BAD_SEQ_LEN into the error word at byte 32 of
the workspace, which each call zeroes first. Requests with clean inputs must
still match the oracle.
"""
import ctypes

import numpy as np
import pytest
import torch

import workloads
from gpu_helpers import DEV, compare, run_oracle, to_device, to_np
from mla_paged_attention_amd import _binding as B
from mla_paged_attention_amd import build as hip_build

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

BAD_BLOCK, BAD_SEQ_LEN, WORD_OFFSET = 1, 2, 32


@pytest.fixture(scope="module")
def checked():
    lib = ctypes.CDLL(hip_build.CHECKED_LIBRARY)
    B._bind(lib)
    return lib


def _decode(lib, wl, q, kv, bt, sl, num_splits=0, indices=None):
    lead = tuple(q.shape[:-1])
    out = torch.empty(lead + (512,), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(lead, dtype=torch.float32, device=DEV)
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    kvd = B.MLA_KV_FP8_E4M3 if wl.kv_dtype == "fp8" else B.MLA_KV_BF16
    h = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if indices is None:
        n = B.get_workspace_size(wl.batch, wl.num_heads, bt.shape[1] * wl.block_size,
                                 num_splits, 0)
        ws = torch.full((n,), 0x5A, dtype=torch.uint8, device=DEV)  # a stale error word
        st = lib.mla_decode(p(q), p(kv), p(bt), p(sl), p(out), p(lse), wl.scale, wl.num_heads,
                            wl.block_size, num_splits, wl.batch, bt.shape[1], kv.shape[0], kvd,
                            wl.kv_scale, p(ws), n, h)
    else:
        n = B.get_workspace_size_sparse(wl.batch, wl.num_heads, indices.shape[1], num_splits, 0)
        ws = torch.full((n,), 0x5A, dtype=torch.uint8, device=DEV)
        st = lib.mla_decode_sparse(p(q), p(kv), p(bt), p(sl), p(indices), indices.shape[1],
                                   p(out), p(lse), wl.scale, wl.num_heads, wl.block_size,
                                   num_splits, wl.batch, bt.shape[1], kv.shape[0], kvd,
                                   wl.kv_scale, p(ws), n, h)
    assert st == B.MLA_OK
    torch.cuda.synchronize()
    word = int(ws[WORD_OFFSET:WORD_OFFSET + 4].cpu().view(torch.int32)[0])
    return out, lse, word


@pytest.mark.parametrize("kv_dtype,num_heads", [("bf16", 16), ("bf16", 64), ("fp8", 32)])
@pytest.mark.parametrize("num_splits", [0, 3])
def test_clean_inputs_report_nothing(orc, checked, kv_dtype, num_heads, num_splits):
    wl = workloads.make_workload(batch=5, num_heads=num_heads, seq=("fixed", [1, 40, 300, 0, 2000]),
                                 block_size=32, seed=111, kv_dtype=kv_dtype, poison=True)
    out, lse, word = _decode(checked, wl, *to_device(wl), num_splits=num_splits)
    assert word == 0
    compare(*to_np(out, lse), *run_oracle(orc, wl), kv_dtype, "checked build, clean inputs")


@pytest.mark.parametrize("kv_dtype,num_heads", [("bf16", 16), ("bf16", 64), ("fp8", 32)])
def test_corrupt_block_ids_and_lengths_are_reported(orc, checked, kv_dtype, num_heads):
    wl = workloads.make_workload(batch=4, num_heads=num_heads, seq=("fixed", [100, 300, 64, 500]),
                                 block_size=32, seed=112, kv_dtype=kv_dtype, poison=True)
    ref_out, ref_lse = run_oracle(orc, wl)
    q, kv, bt, sl = to_device(wl)
    # Request 1: one block id past the cache, one negative.
    bad_bt = bt.clone()
    bad_bt[1, 2] = wl.num_blocks + 7
    bad_bt[1, 5] = -3
    out, lse, word = _decode(checked, wl, q, kv, bad_bt, sl)
    assert word == BAD_BLOCK
    o, l_ = to_np(out, lse)
    assert np.isfinite(o).all()
    keep = [0, 2, 3]
    compare(o[keep], l_[keep], ref_out[keep], ref_lse[keep], kv_dtype, "untouched requests")
    # Request 3 (its table row is full): a length beyond the table's
    # capacity, clamped to it; request 2: negative, clamped to empty.
    bad_sl = sl.clone()
    bad_sl[3] = bt.shape[1] * wl.block_size + 50
    bad_sl[2] = -9
    out, lse, word = _decode(checked, wl, q, kv, bt, bad_sl)
    assert word == BAD_SEQ_LEN
    o, l_ = to_np(out, lse)
    compare(o[:2], l_[:2], ref_out[:2], ref_lse[:2], kv_dtype, "untouched requests")
    assert (o[2] == 0).all() and np.isneginf(l_[2]).all()   # clamped to an empty request
    # Both at once, through forced splits as well.
    for s in (0, 2):
        _, _, word = _decode(checked, wl, q, kv, bad_bt, bad_sl, num_splits=s)
        assert word == BAD_BLOCK | BAD_SEQ_LEN


def test_sparse_reports_corrupt_block_ids(orc, checked):
    wl = workloads.make_workload(batch=3, num_heads=16, seq=("fixed", [90, 400, 33]),
                                 block_size=16, seed=113)
    q, kv, bt, sl = to_device(wl)
    idx = torch.full((3, 64), -1, dtype=torch.int32)
    for b, n in enumerate(wl.seq_lens.tolist()):
        idx[b, :min(n, 64)] = torch.arange(min(n, 64), dtype=torch.int32)
    idx = idx.to(DEV)
    _, _, word = _decode(checked, wl, q, kv, bt, sl, indices=idx)
    assert word == 0
    bad_bt = bt.clone()
    bad_bt[0, 1] = wl.num_blocks       # positions 16..31 of request 0 map through it
    out, lse, word = _decode(checked, wl, q, kv, bad_bt, sl, indices=idx)
    assert word == BAD_BLOCK
    assert torch.isfinite(out.float()).all()
