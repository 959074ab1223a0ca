"""GPU parity of multi-token decode (q_len query tokens per request, causal).

The HIP path (mla_decode_multi_token through the C ABI) against the fp64
oracle on the same seeded inputs, element by element, at the tolerances of
one-token decode. The cases cover query rows that fill one 16-row tile or
several, rows of different query tokens inside one tile (heads not a
multiple of 16), requests shorter than q_len (query tokens that see
nothing), lengths around the 16/32/64-token boundaries, forced and
automatic splits, both cache types, rising logits (second passes with
partly masked rows), and every request of a full-size batch.
"""
import numpy as np
import pytest
import torch

import mla_paged_attention_amd as mla
import workloads
from gpu_helpers import compare, run_gpu, run_oracle, to_device, to_np

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

LENS = [0, 1, 2, 3, 15, 16, 17, 31, 33, 63, 64, 65, 130, 700]


def _check(orc, wl, num_splits=0, req=None, what=""):
    out, lse = to_np(*run_gpu(wl, num_splits))
    ref_out, ref_lse = run_oracle(orc, wl, req)
    if req is not None:
        out, lse = out[req], lse[req]
    return compare(out, lse, ref_out, ref_lse, wl.kv_dtype, what or wl.name)


@pytest.mark.parametrize("num_heads,q_len,block_size", [
    (16, 2, 32),    # 32 rows: two tiles of one token each
    (16, 4, 64),    # 64 rows: one workgroup's four tiles
    (8, 2, 16),     # 16 rows: both tokens in one tile
    (5, 3, 32),     # 15 rows: tokens change inside a tile
    (20, 3, 64),    # 60 rows: tokens change inside tiles
    (1, 16, 16),    # 16 rows: one head, sixteen tokens
    (128, 2, 64),   # 256 rows: four workgroups per partition
    (64, 3, 128),   # 192 rows
])
def test_multi_token_bf16(orc, num_heads, q_len, block_size):
    wl = workloads.make_workload(batch=len(LENS), num_heads=num_heads, seq=("fixed", LENS),
                                 block_size=block_size, seed=300 + num_heads + q_len,
                                 poison=True, q_len=q_len)
    for s in (0, 1, 3):
        _check(orc, wl, s, what=f"bf16 H={num_heads} q_len={q_len} bs={block_size} splits={s}")


@pytest.mark.parametrize("num_heads,q_len", [(16, 2), (48, 3), (128, 2), (7, 4)])
def test_multi_token_fp8(orc, num_heads, q_len):
    wl = workloads.make_workload(batch=len(LENS), num_heads=num_heads, seq=("fixed", LENS),
                                 block_size=64, seed=400 + num_heads + q_len, kv_dtype="fp8",
                                 poison=True, q_len=q_len)
    for s in (0, 2):
        _check(orc, wl, s, what=f"fp8 H={num_heads} q_len={q_len} splits={s}")


def test_max_rows(orc):
    # 16 query tokens x 128 heads = 2048 rows per request.
    wl = workloads.make_workload(batch=2, num_heads=128, seq=("fixed", [9, 300]),
                                 block_size=32, seed=501, poison=True, q_len=16)
    for s in (0, 2):
        _check(orc, wl, s, what=f"2048 rows splits={s}")


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("num_heads", [16, 20])
def test_multi_token_rising_logits(orc, num_heads, kv_dtype):
    wl = workloads.make_rising(num_heads, kv_dtype, seed=61 + num_heads, q_len=3)
    for s in (0, 1):
        _check(orc, wl, s, what=f"{wl.name} splits={s}")


def test_q_len_one_equals_decode_bitwise():
    wl = workloads.make_config("v2lite-8")
    dev = to_device(wl)
    out1, lse1 = run_gpu(wl, 0, dev_tensors=dev)
    q4 = dev[0][:, None].contiguous()
    out4, lse4 = mla.decode(q4, *dev[1:], scale=wl.scale)
    torch.cuda.synchronize()
    assert torch.equal(out4[:, 0], out1) and torch.equal(lse4[:, 0], lse1)


def test_query_tokens_equal_cut_one_token_decodes():
    # Query token i of a multi-token call sees the first N - q_len + 1 + i
    # tokens; with forced single-split partitions its row must equal a
    # one-token call on that prefix in value (different tiles may differ in
    # the last bit, so compare to the bf16 tolerance, and lse closely).
    q_len = 4
    wl = workloads.make_workload(batch=6, num_heads=16, seq=("fixed", [5, 40, 77, 129, 300, 1000]),
                                 block_size=32, seed=77, q_len=q_len)
    q, kv, bt, sl = to_device(wl)
    out, lse = mla.decode(q, kv, bt, sl, scale=wl.scale, num_splits=1)
    for i in range(q_len):
        cut = (sl - (q_len - 1 - i)).clamp(min=0).to(torch.int32).contiguous()
        o1, l1 = mla.decode(q[:, i].contiguous(), kv, bt, cut, scale=wl.scale, num_splits=1)
        torch.cuda.synchronize()
        assert (out[:, i].float() - o1.float()).abs().max().item() <= 2e-2
        assert (lse[:, i] - l1).abs().max().item() <= 1e-4


@pytest.mark.parametrize("q_len", [2, 4])
def test_r1tp8_multi_token_full(orc, q_len):
    # The full 512-request batch at 16 heads, q_len query tokens per request,
    # in the automatic plan the benchmark times; every request against the
    # oracle.
    wl = workloads.make_config("r1tp8", q_len=q_len)
    out, lse = to_np(*run_gpu(wl, 0))
    ref_out, ref_lse = run_oracle(orc, wl)
    compare(out, lse, ref_out, ref_lse, "bf16", f"r1tp8 q_len={q_len} (whole batch)")


def test_fp8_multi_token_full(orc):
    # The fp8 configuration (64 requests of 8192 tokens, 128 heads, E4M3
    # cache) with two query tokens per request: 256 query rows per request in
    # the many-head E4M3 kernel, in the automatic plan the benchmark times;
    # every request against the oracle fed the dequantised cache.
    wl = workloads.make_config("fp8", q_len=2)
    out, lse = to_np(*run_gpu(wl, 0))
    ref_out, ref_lse = run_oracle(orc, wl)
    compare(out, lse, ref_out, ref_lse, "fp8", "fp8 q_len=2 (whole batch)")
