"""The allocation-free entry point against the workspace entry point.

mla_decode_noalloc takes no workspace (the library's static device scratch
array holds the plan and partial rows). On the same inputs it must give what
mla_decode_multi_token gives with a workspace of mla_get_workspace_size bytes,
bit for bit, and match the oracle at the stated tolerances, on two calls in a
row with the second smaller than the first (the array keeps the first call's
contents). A call whose workspace need exceeds the array is refused before
anything is enqueued.
"""
import pytest
import torch

import mla_paged_attention_amd as mla
import workloads
from gpu_helpers import DEV, compare, run_oracle, to_device, to_np

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _both(orc, wl, num_splits):
    q, kv, bt, sl = to_device(wl)
    lead = tuple(q.shape[:-1])
    out_n = torch.empty(lead + (512,), dtype=torch.bfloat16, device=DEV)
    lse_n = torch.empty(lead, dtype=torch.float32, device=DEV)
    mla.decode_noalloc(q, kv, bt, sl, scale=wl.scale, out=out_n, lse=lse_n,
                       num_splits=num_splits, kv_scale=wl.kv_scale)
    need = mla.get_workspace_size(wl.batch, wl.num_heads, wl.max_blocks * wl.block_size,
                                  num_splits, 0, q_len=wl.q_len)
    assert need <= mla.NOALLOC_SCRATCH_BYTES
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    out_w, lse_w = mla.decode(q, kv, bt, sl, scale=wl.scale, num_splits=num_splits,
                              kv_scale=wl.kv_scale, workspace=ws)
    torch.cuda.synchronize()
    what = f"noalloc {wl.kv_dtype} B={wl.batch} H={wl.num_heads} q_len={wl.q_len} s={num_splits}"
    assert torch.equal(out_n, out_w) and torch.equal(lse_n, lse_w), what
    compare(*to_np(out_n, lse_n), *run_oracle(orc, wl), wl.kv_dtype, what)


def test_noalloc_equals_workspace_call_automatic_plan(orc):
    big = workloads.make_workload(batch=24, num_heads=128, seq=("uniform", 500, 6000),
                                  block_size=64, seed=95, poison=True)
    small = workloads.make_workload(batch=3, num_heads=16, seq=("fixed", [1, 70, 900]),
                                    block_size=32, seed=96, poison=True)
    _both(orc, big, 0)
    _both(orc, small, 0)


def test_noalloc_equals_workspace_call_forced_splits(orc):
    big = workloads.make_workload(batch=10, num_heads=32, seq=("uniform", 100, 3000),
                                  block_size=64, seed=97, kv_dtype="fp8", poison=True, q_len=2)
    small = workloads.make_workload(batch=4, num_heads=16, seq=("fixed", [0, 17, 64, 500]),
                                    block_size=16, seed=98, poison=True)
    _both(orc, big, 3)
    _both(orc, small, 2)


def test_noalloc_refuses_calls_beyond_its_array():
    # 300 requests x 16 forced splits x 128 heads of partial rows need far
    # more than the array holds.
    wl = workloads.make_workload(batch=300, num_heads=128, seq=("fixed", [16] * 300),
                                 block_size=16, seed=99)
    need = mla.get_workspace_size(wl.batch, wl.num_heads, wl.max_blocks * wl.block_size, 16, 0)
    assert need > mla.NOALLOC_SCRATCH_BYTES
    q, kv, bt, sl = to_device(wl)
    out = torch.empty((300, 128, 512), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(mla.MLAError) as e:
        mla.decode_noalloc(q, kv, bt, sl, scale=wl.scale, out=out, lse=None, num_splits=16)
    assert e.value.status == mla.MLA_ERR_WORKSPACE_TOO_SMALL
