"""GPU parity of sparse decode (each request attends to listed token positions).

mla_decode_sparse through the C ABI against the fp64 oracle's
attend_sparse on the same seeded inputs, element by element, at the
tolerances of dense decode. Lists cover: sorted and shuffled positions,
repeats, entries outside [0, seq_len) (skipped), -1 padding, lists with no
valid entry, lengths that are not multiples of the 16/32/64-token tiles,
forced and automatic splits, both cache types and 1 to 128 heads, the
longest list the ABI accepts; rising
logits (second passes over gathered rows); a list of every position
against dense decode; and every request of the full-size sparse
workloads.
"""
import numpy as np
import pytest
import torch

import mla_paged_attention_amd as mla
import workloads
from gpu_helpers import DEV, compare, run_gpu, run_oracle, to_device, to_np

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def run_sparse(wl, indices, num_splits=0, **kw):
    q, kv, bt, sl = to_device(wl)
    out, lse = mla.decode_sparse(q, kv, bt, sl, indices.to(DEV).contiguous(), scale=wl.scale,
                                 num_splits=num_splits, kv_scale=wl.kv_scale, **kw)
    torch.cuda.synchronize()
    return to_np(out, lse)


def oracle_sparse(orc, wl, indices, req=None):
    idx = indices.numpy()
    q = wl.q_bits()
    bt, sl = wl.block_table.numpy(), wl.seq_lens.numpy()
    if req is not None:
        q, idx, bt, sl = q[req], idx[req], bt[req], sl[req]
    return orc.attend_sparse(q, wl.kv_bits(), bt, sl, wl.block_size, wl.scale, idx,
                             kv_fp8=wl.kv_dtype == "fp8", kv_scale=wl.kv_scale)


def messy_lists(wl, topk, seed):
    """Shuffled positions with repeats, out-of-range entries and -1 padding."""
    rng = np.random.default_rng(seed)
    out = np.full((wl.batch, topk), -1, np.int32)
    for b, n in enumerate(wl.seq_lens.tolist()):
        k = rng.integers(0, topk + 1)
        row = rng.integers(0, max(n, 1), size=k) if n > 0 else np.full(k, -1)
        if k >= 4:
            row[rng.choice(k, size=3, replace=False)] = [n, n + 100, -7]
        out[b, :k] = row
        rng.shuffle(out[b])
    return torch.from_numpy(out)


LENS = [0, 1, 15, 16, 17, 33, 64, 65, 130, 700, 2000]


@pytest.mark.parametrize("kv_dtype,num_heads,block_size", [
    ("bf16", 16, 32), ("bf16", 1, 16), ("bf16", 20, 64), ("bf16", 128, 128),
    ("fp8", 16, 64), ("fp8", 48, 16), ("fp8", 128, 64)])
@pytest.mark.parametrize("topk", [1, 7, 64, 100, 513])
def test_sparse_messy_lists(orc, kv_dtype, num_heads, block_size, topk):
    wl = workloads.make_workload(batch=len(LENS), num_heads=num_heads, seq=("fixed", LENS),
                                 block_size=block_size, seed=600 + num_heads + topk,
                                 kv_dtype=kv_dtype, poison=True)
    idx = messy_lists(wl, topk, seed=topk + num_heads)
    ref = oracle_sparse(orc, wl, idx)
    for s in (0, 1, 3):
        out, lse = run_sparse(wl, idx, s)
        compare(out, lse, *ref, kv_dtype,
                f"sparse {kv_dtype} H={num_heads} bs={block_size} topk={topk} splits={s}")


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_sparse_sampled_lists(orc, kv_dtype):
    # Sorted samples without replacement (the generator's lists), -1 padded.
    wl = workloads.make_workload(batch=6, num_heads=32, seq=("fixed", [3, 100, 900, 2048, 3000, 5000]),
                                 block_size=64, seed=71, kv_dtype=kv_dtype, poison=True,
                                 topk=2048)
    out, lse = run_sparse(wl, wl.indices)
    compare(out, lse, *oracle_sparse(orc, wl, wl.indices), kv_dtype, f"sparse sampled {kv_dtype}")


@pytest.mark.parametrize("kv_dtype,num_heads", [("bf16", 16), ("bf16", 64), ("fp8", 128)])
def test_sparse_all_positions_is_dense(orc, kv_dtype, num_heads):
    wl = workloads.make_workload(batch=5, num_heads=num_heads, seq=("fixed", [1, 31, 64, 250, 777]),
                                 block_size=32, seed=72, kv_dtype=kv_dtype, poison=True)
    idx = torch.full((5, 800), -1, dtype=torch.int32)
    for b, n in enumerate(wl.seq_lens.tolist()):
        idx[b, :n] = torch.arange(n, dtype=torch.int32)
    out, lse = run_sparse(wl, idx)
    compare(out, lse, *run_oracle(orc, wl), kv_dtype, f"sparse all positions {kv_dtype}")


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_sparse_rising_logits(orc, kv_dtype):
    wl = workloads.make_rising(20, kv_dtype, seed=73)
    rng = np.random.default_rng(73)
    idx = np.full((wl.batch, 1024), -1, np.int32)
    for b, n in enumerate(wl.seq_lens.tolist()):
        k = min(n, 1024)
        idx[b, :k] = np.sort(rng.choice(n, size=k, replace=False))
    idx = torch.from_numpy(idx)
    for s in (0, 1):
        out, lse = run_sparse(wl, idx, s)
        compare(out, lse, *oracle_sparse(orc, wl, idx), kv_dtype, f"sparse rising {kv_dtype} s={s}")


@pytest.mark.parametrize("kv_dtype,num_heads", [("bf16", 16), ("fp8", 32)])
def test_sparse_max_topk(orc, kv_dtype, num_heads):
    # The longest list the ABI accepts, drawn from a 128K-token context,
    # beside a short request whose list is mostly -1 padding.
    topk = mla.MAX_TOPK
    wl = workloads.make_workload(batch=2, num_heads=num_heads, seq=("fixed", [131072, 300]),
                                 block_size=64, seed=76, kv_dtype=kv_dtype)
    rng = np.random.default_rng(76)
    idx = np.full((2, topk), -1, np.int32)
    idx[0] = np.sort(rng.choice(131072, size=topk, replace=False))
    idx[1, :300] = rng.permutation(300)
    idx = torch.from_numpy(idx)
    ref = oracle_sparse(orc, wl, idx)
    for s in (0, 1):
        out, lse = run_sparse(wl, idx, s)
        compare(out, lse, *ref, kv_dtype, f"sparse max topk {kv_dtype} H={num_heads} splits={s}")


def test_sparse_empty_lists():
    wl = workloads.make_workload(batch=3, num_heads=16, seq=("fixed", [0, 10, 40]), block_size=16,
                                 seed=74)
    idx = torch.tensor([[-1, -1, 5, 0], [-1, 10, 11, -2], [39, 39, -1, 40]], dtype=torch.int32)
    out, lse = run_sparse(wl, idx)
    assert (out[:2] == 0).all() and np.isneginf(lse[:2]).all()
    assert np.isfinite(lse[2]).all()


@pytest.mark.parametrize("name", ["sparse-r1tp8", "sparse-fp8"])
def test_sparse_full_size(orc, name):
    # Every request and head of the full-size sparse workloads.
    wl = workloads.make_config(name)
    out, lse = run_sparse(wl, wl.indices)
    compare(out, lse, *oracle_sparse(orc, wl, wl.indices), wl.kv_dtype, f"{name} (whole batch)")
