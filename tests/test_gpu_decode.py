"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Every case draws seeded inputs from workloads.py, runs mla_decode on cuda:0
and the oracle on the host, and compares element by element at the stated
tolerances (bf16 cache: out 1e-2 + 1e-2|ref|, lse 1e-3 absolute; fp8 cache:
2e-2 + 2e-2|ref| for both, against the oracle fed the dequantised cache and
the unquantised bf16 q). Full-size configurations compare every request and
every head, in the launch configuration the benchmark times (automatic plan).
"""
import numpy as np
import pytest
import torch

import mla_paged_attention_amd as mla
import workloads
from gpu_helpers import compare, run_gpu, run_oracle, to_device, to_np

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _check(orc, wl, num_splits=0, req=None, what=""):
    out, lse = to_np(*run_gpu(wl, num_splits))
    ref_out, ref_lse = run_oracle(orc, wl, req)
    if req is not None:
        out, lse = out[req], lse[req]
    return compare(out, lse, ref_out, ref_lse, wl.kv_dtype, what or wl.name)


@pytest.mark.parametrize("num_splits", [1, 2, 0, 3, 7, 16])
@pytest.mark.parametrize("poison", [False, True])
def test_tiny(orc, num_splits, poison):
    wl = workloads.make_config("tiny", poison=poison)
    _check(orc, wl, num_splits, what=f"tiny splits={num_splits} poison={poison}")


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("block_size", [16, 32, 64, 128])
@pytest.mark.parametrize("num_heads", [1, 5, 16, 20, 128])
def test_ragged_edges(orc, block_size, num_heads, kv_dtype):
    # lengths around unit (16), bf16 tile (32) and fp8 tile (64) boundaries
    lens = [0, 1, 15, 16, 17, 31, 33, 63, 64, 65, 129, 700]
    wl = workloads.make_workload(batch=len(lens), num_heads=num_heads, seq=("fixed", lens),
                                 block_size=block_size, seed=100 + block_size + num_heads,
                                 kv_dtype=kv_dtype, pool_blocks=None, poison=True)
    for s in (0, 1, 4):
        _check(orc, wl, s, what=f"edges {kv_dtype} bs={block_size} H={num_heads} splits={s}")


@pytest.mark.parametrize("name", ["v2lite-1", "v2lite-8", "v2lite-64"])
def test_v2lite(orc, name):
    wl = workloads.make_config(name)
    _check(orc, wl, 0)


def test_v2lite8_poisoned(orc):
    wl = workloads.make_config("v2lite-8", poison=True)
    _check(orc, wl, 0, what="v2lite-8 poisoned")


@pytest.mark.parametrize("name", ["r1tp8", "fullhead", "fp8"])
def test_full_size(orc, name):
    # Every request and head of the full-size configuration (512 x 16,
    # 128 x 128, 64 x 128 E4M3) against the oracle, element by element.
    wl = workloads.make_config(name)
    _check(orc, wl, 0, what=f"{name} (whole batch)")


@pytest.mark.parametrize("kv_dtype,num_heads,batch,length",
                         [("bf16", 16, 8, 4096), ("bf16", 16, 64, 1000), ("bf16", 128, 4, 4111),
                          ("fp8", 128, 2, 8192), ("fp8", 16, 32, 2048)])
def test_equal_lengths_cut_on_request_boundaries(orc, kv_dtype, num_heads, batch, length):
    # Equal requests whose count divides the partitions are each cut into
    # equal pieces, one partition apiece (the automatic plan computed in the
    # attention kernel); poisoned tails and unused blocks must not leak.
    wl = workloads.make_workload(batch=batch, num_heads=num_heads, seq=("fixed", [length] * batch),
                                 block_size=64, seed=300 + batch, kv_dtype=kv_dtype, poison=True)
    _check(orc, wl, 0, what=f"equal {kv_dtype} H={num_heads} B={batch} N={length}")


@pytest.mark.parametrize("num_splits", [0, 1, 5])
def test_fp8_small(orc, num_splits):
    wl = workloads.make_workload(batch=5, num_heads=20, seq=("fixed", [1, 17, 100, 513, 2000]),
                                 block_size=64, seed=61, kv_dtype="fp8", poison=True)
    _check(orc, wl, num_splits, what=f"fp8 small splits={num_splits}")


@pytest.mark.parametrize("num_heads", [16, 128])
def test_fp8_tiny_q_rows(orc, num_heads):
    # q rows of tiny magnitude (down to 1e-38, where 448 / amax overflows
    # fp32) and an all-zero row beside ordinary ones.
    wl = workloads.make_workload(batch=3, num_heads=num_heads, seq=("fixed", [40, 300, 1500]),
                                 block_size=64, seed=63, kv_dtype="fp8", poison=True)
    wl.q[0, 1] = (wl.q[0, 1].float() * 1e-37).to(torch.bfloat16)
    wl.q[1, 2] = (wl.q[1, 2].float() * 1e-38).to(torch.bfloat16)
    wl.q[2, 3] = 0
    for s in (0, 1, 2):
        _check(orc, wl, s, what=f"fp8 tiny q rows H={num_heads} splits={s}")


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("num_heads", [16, 20, 128])
def test_rising_logits(orc, num_heads, kv_dtype):
    # Head 0's logits climb by ~100 after the first tiles: the kernels' frame
    # handling (moves, or a second pass) must keep every sum finite and exact.
    wl = workloads.make_rising(num_heads, kv_dtype, seed=71 + num_heads)
    for s in (0, 1, 3):
        _check(orc, wl, s, what=f"{wl.name} splits={s}")


def test_large_batch_with_long_requests(orc):
    # Large batch (more than twice the partitions): long requests are cut
    # into pieces and merged, short ones run whole; all rows are checked.
    lens = [37, 130, 700] * 172 + [30000, 25000, 9000, 4097]
    wl = workloads.make_workload(batch=len(lens), num_heads=16, seq=("fixed", lens),
                                 block_size=64, seed=41, poison=True)
    _check(orc, wl, 0, what="large batch with long requests")


@pytest.mark.parametrize("num_heads", [16, 128])
def test_snake_plan_largest_batch(orc, num_heads):
    # The in-kernel snake plan at its largest batch (1024 requests): every
    # workgroup ranks the pieces itself, so the ranking must agree across
    # workgroups. A few very long requests are cut into many pieces, and
    # many short ones share a cost (equal sort keys); all rows are checked.
    gen = np.random.default_rng(71)
    lens = gen.integers(1, 400, size=1016).tolist() + [0, 1, 16, 17, 12000, 20000, 7000, 33]
    wl = workloads.make_workload(batch=len(lens), num_heads=num_heads, seq=("fixed", lens),
                                 block_size=32, seed=72, poison=True)
    _check(orc, wl, 0, what=f"snake plan, 1024 requests, {num_heads} heads")


@pytest.mark.parametrize("num_heads,kv_dtype,splits",
                         [(16, "bf16", (0, 1)), (128, "bf16", (0, 1)), (32, "fp8", (0, 1))])
def test_long_context(orc, num_heads, kv_dtype, splits):
    # A 128K-token context beside a 1-token and a 64K + 1-token request:
    # unit, tile and piece counts far beyond the benchmark lengths. With one
    # forced split a single workgroup streams the whole 128K context.
    lens = [131072, 1, 65537]
    wl = workloads.make_workload(batch=len(lens), num_heads=num_heads, seq=("fixed", lens),
                                 block_size=64, seed=47, kv_dtype=kv_dtype)
    ref_out, ref_lse = run_oracle(orc, wl)
    for s in splits:
        out, lse = to_np(*run_gpu(wl, s))
        compare(out, lse, ref_out, ref_lse, kv_dtype,
                f"long context, {num_heads} heads, {kv_dtype}, splits={s}")


def test_very_large_batch(orc):
    # Beyond the register-resident plan's batch limit.
    gen = np.random.default_rng(42)
    lens = gen.integers(0, 80, size=5000).tolist()
    wl = workloads.make_workload(batch=len(lens), num_heads=16, seq=("fixed", lens),
                                 block_size=16, seed=42)
    _check(orc, wl, 0, what="5000 short requests")


# ---------------------------------------------------------------- invariants

def test_block_permutation_bitwise():
    wl = workloads.make_workload(batch=6, num_heads=16, seq=("fixed", [5, 64, 100, 333, 1000, 47]),
                                 block_size=32, seed=21, pool_blocks=70)
    out_a, lse_a = run_gpu(wl, 0)
    perm = torch.randperm(wl.num_blocks, generator=torch.Generator().manual_seed(3))
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(wl.num_blocks)
    wl.kv = wl.kv[perm].contiguous()
    valid = wl.block_table >= 0
    wl.block_table[valid] = inv[wl.block_table[valid].long()].to(torch.int32)
    out_b, lse_b = run_gpu(wl, 0)
    assert torch.equal(out_a, out_b) and torch.equal(lse_a, lse_b)


def test_batch_independence_bitwise():
    # Request 0 keeps its piece boundaries when the others change only in content.
    wl = workloads.make_workload(batch=4, num_heads=16, seq=("fixed", [700, 300, 900, 50]),
                                 block_size=64, seed=22)
    out_a, lse_a = run_gpu(wl, 1)
    wl.q[1:] = torch.randn(wl.q[1:].shape, generator=torch.Generator().manual_seed(9)).to(
        torch.bfloat16)
    wl.seq_lens[1:] = torch.tensor([3, 17, 640], dtype=torch.int32)
    out_b, lse_b = run_gpu(wl, 1)
    assert torch.equal(out_a[0], out_b[0]) and torch.equal(lse_a[0], lse_b[0])


@pytest.mark.parametrize("num_splits", [0, 3])
def test_determinism_bitwise(num_splits):
    wl = workloads.make_config("v2lite-8")
    dev = to_device(wl)
    out_a, lse_a = run_gpu(wl, num_splits, dev)
    out_a, lse_a = out_a.clone(), lse_a.clone()
    for _ in range(3):
        out_b, lse_b = run_gpu(wl, num_splits, dev)
        assert torch.equal(out_a, out_b) and torch.equal(lse_a, lse_b)


def test_head_padding_to_128_fp8(orc):
    wl = workloads.make_workload(batch=3, num_heads=16, seq=("fixed", [37, 130, 1000]),
                                 block_size=64, seed=24, kv_dtype="fp8", poison=True)
    out16, lse16 = to_np(*run_gpu(wl, 0))
    q128 = torch.zeros((wl.batch, 128, 576), dtype=torch.bfloat16)
    q128[:, :16] = wl.q
    wl128 = workloads.Workload(name="fp8-pad128", q=q128, kv=wl.kv,
                               block_table=wl.block_table, seq_lens=wl.seq_lens,
                               block_size=wl.block_size, kv_dtype=wl.kv_dtype,
                               kv_scale=wl.kv_scale)
    out128, lse128 = to_np(*run_gpu(wl128, 0))
    ref_out, ref_lse = run_oracle(orc, wl128)
    compare(out128, lse128, ref_out, ref_lse, "fp8", what="fp8 padded to 128 heads")
    compare(out16, lse16, ref_out[:, :16], ref_lse[:, :16], "fp8", what="fp8 16 heads")
    for b in range(wl.batch):
        np.testing.assert_allclose(lse128[b, 16:], np.log(int(wl.seq_lens[b])), atol=1e-3)


def test_head_padding_to_128(orc):
    wl = workloads.make_config("tiny")
    out16, lse16 = to_np(*run_gpu(wl, 0))
    q128 = torch.zeros((wl.batch, 128, 576), dtype=torch.bfloat16)
    q128[:, :16] = wl.q
    wl128 = workloads.Workload(name="tiny-pad128", q=q128, kv=wl.kv,
                               block_table=wl.block_table, seq_lens=wl.seq_lens,
                               block_size=wl.block_size, kv_dtype=wl.kv_dtype,
                               kv_scale=wl.kv_scale)
    out128, lse128 = to_np(*run_gpu(wl128, 0))
    ref_out, ref_lse = run_oracle(orc, wl128)
    compare(out128, lse128, ref_out, ref_lse, what="tiny padded to 128 heads")
    # Real heads: the same per-head arithmetic, so bitwise equal to the 16-head run.
    assert np.array_equal(out128[:, :16], out16) and np.array_equal(lse128[:, :16], lse16)
    # Padded heads (q = 0): the mean of the value rows and ln N.
    for b in range(wl.batch):
        n = int(wl.seq_lens[b])
        np.testing.assert_allclose(lse128[b, 16:], np.log(n), atol=1e-3)


@pytest.mark.parametrize("batch", [40, 160])
def test_forced_splits_larger_batches(orc, batch):
    # Forced splits merge every request: 40 and 160 (request, head tile)
    # pairs run the merge with 4 and 8 features per thread.
    gen = np.random.default_rng(batch)
    lens = [0, 1, 17] + gen.integers(1, 700, size=batch - 3).tolist()
    wl = workloads.make_workload(batch=batch, num_heads=16, seq=("fixed", lens), block_size=32,
                                 seed=batch + 5, poison=True)
    _check(orc, wl, 3, what=f"forced 3 splits, batch {batch}")


@pytest.mark.parametrize("kv_dtype,num_heads", [("bf16", 16), ("bf16", 64), ("fp8", 48)])
def test_split_counts_agree(orc, kv_dtype, num_heads):
    wl = workloads.make_workload(batch=3, num_heads=num_heads, seq=("fixed", [2000, 37, 4097]),
                                 block_size=64, seed=23, kv_dtype=kv_dtype, poison=True)
    ref_out, ref_lse = run_oracle(orc, wl)
    for s in range(0, 17):
        out, lse = to_np(*run_gpu(wl, s))
        compare(out, lse, ref_out, ref_lse, kv_dtype, what=f"{kv_dtype} H={num_heads} splits={s}")


def test_small_workspace_auto_mode(orc):
    wl = workloads.make_config("v2lite-8")
    meta = mla.get_workspace_size(wl.batch, wl.num_heads, 0, 1, 0)
    full = mla.get_workspace_size(wl.batch, wl.num_heads, wl.max_blocks * wl.block_size, 0, 0)
    ref_out, ref_lse = run_oracle(orc, wl)
    for nbytes in (meta, (meta + full) // 2, full):
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
        out, lse = to_np(*run_gpu(wl, 0, workspace=ws))
        compare(out, lse, ref_out, ref_lse, what=f"auto with {nbytes} B workspace")


def test_plan_modes_agree(orc):
    # 64 requests: the attention kernel works the contiguous plan out itself;
    # 65: plan_kernel's contiguous plan; 64 with a workspace too small for
    # partial rows: plan_kernel's snake plan. Lengths include empty, single
    # token and long requests cut into many pieces.
    gen = np.random.default_rng(61)
    lens = [0, 1, 15, 16, 17, 20000, 9000] + gen.integers(0, 3000, size=58).tolist()
    for batch in (64, 65):
        wl = workloads.make_workload(batch=batch, num_heads=16, seq=("fixed", lens[:batch]),
                                     block_size=32, seed=62, poison=True)
        ref_out, ref_lse = run_oracle(orc, wl)
        out, lse = to_np(*run_gpu(wl, 0))
        compare(out, lse, ref_out, ref_lse, what=f"automatic plan, batch {batch}")
        if batch == 64:
            meta = mla.get_workspace_size(wl.batch, wl.num_heads, 0, 1, 0)
            ws = torch.empty(meta, dtype=torch.uint8, device="cuda:0")
            out, lse = to_np(*run_gpu(wl, 0, workspace=ws))
            compare(out, lse, ref_out, ref_lse, what="batch 64, no partial rows (snake plan)")


def test_dirty_workspace(orc):
    # The workspace needs no initialisation: one buffer, filled with 0xFF bytes
    # (int32 -1, fp32 NaN) and then reused dirty, serves every mode in turn:
    # forced splits (no plan launch), the in-kernel plan (5 requests),
    # plan_kernel's contiguous plan (65, 300) and its snake plan (600 requests
    # of 16 heads), for both cache types and both attention kernels.
    gen = np.random.default_rng(63)
    cases = []
    for kv_dtype, heads, batches in (("bf16", 16, (5, 65, 600)), ("fp8", 32, (5, 65, 300)),
                                     ("bf16", 40, (5, 65, 300))):
        for batch in batches:
            lens = gen.integers(0, 1200, size=batch).tolist()
            lens[0] = 7000
            wl = workloads.make_workload(batch=batch, num_heads=heads, seq=("fixed", lens),
                                         block_size=64, seed=64 + batch, kv_dtype=kv_dtype,
                                         poison=True)
            cases.append(wl)
    nbytes = max(mla.get_workspace_size(wl.batch, wl.num_heads, wl.max_blocks * wl.block_size,
                                        s, 0) for wl in cases for s in (0, 1, 3))
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda:0")
    for wl in cases:
        ref_out, ref_lse = run_oracle(orc, wl)
        for s in (3, 0, 1):
            out, lse = to_np(*run_gpu(wl, s, workspace=ws))
            compare(out, lse, ref_out, ref_lse, wl.kv_dtype,
                    what=f"dirty workspace {wl.kv_dtype} H={wl.num_heads} B={wl.batch} splits={s}")


def test_forced_workspace_too_small():
    wl = workloads.make_config("tiny")
    ws = torch.empty(mla.get_workspace_size(wl.batch, wl.num_heads, 0, 1, 0), dtype=torch.uint8,
                     device="cuda:0")
    with pytest.raises(mla.MLAError) as e:
        run_gpu(wl, 4, workspace=ws)
    assert e.value.status == mla.MLA_ERR_WORKSPACE_TOO_SMALL


def test_batch_zero():
    q = torch.empty((0, 16, 576), dtype=torch.bfloat16, device="cuda:0")
    kv = torch.zeros((1, 16, 576), dtype=torch.bfloat16, device="cuda:0")
    bt = torch.zeros((0, 1), dtype=torch.int32, device="cuda:0")
    sl = torch.zeros((0,), dtype=torch.int32, device="cuda:0")
    out, lse = mla.decode(q, kv, bt, sl, scale=0.1)
    torch.cuda.synchronize()
    assert out.shape == (0, 16, 512)


# ---------------------------------------------------------------- combine

@pytest.mark.parametrize("nreq,H", [(6, 20), (40, 16), (70, 32)])
def test_combine_matches_oracle_merge(orc, nreq, H):
    # (request, 16-head tile) pairs: 12, 40 and 140, so the merge runs with
    # 2, 4 and 8 features per thread.
    gen = torch.Generator().manual_seed(31 + nreq)
    counts = ([0, 1, 2, 5, 16, 3] * ((nreq + 5) // 6))[:nreq]
    indptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rows = int(indptr[-1])
    part_out = torch.randn((rows, H, 512), generator=gen, dtype=torch.float32)
    part_lse = (torch.randn((rows, H), generator=gen, dtype=torch.float32) * 5)
    part_lse[3, :4] = -float("inf")           # some empty splits
    part_lse[indptr[3]:indptr[4], 7] = -float("inf")  # a request-head with only empty splits
    out, lse = mla.combine(part_out.cuda(), part_lse.cuda(), torch.from_numpy(indptr).cuda())
    torch.cuda.synchronize()
    out, lse = to_np(out, lse)
    for b in range(len(counts)):
        r0, r1 = indptr[b], indptr[b + 1]
        ref_out, ref_lse = orc.lse_merge(part_out[r0:r1].double().numpy(),
                                         part_lse[r0:r1].double().numpy())
        if r1 == r0:
            ref_out = np.zeros((H, 512))
            ref_lse = np.full(H, -np.inf)
        compare(out[b], lse[b], ref_out, ref_lse, what=f"combine request {b}")
