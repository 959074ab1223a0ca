"""Decode captured in a HIP graph (torch.cuda.CUDAGraph on ROCm).

mla_decode allocates nothing and never synchronises the host, so a caller
may capture it. The captured call is replayed several times, with new
seq_lens and eager decode calls between the replays, and every replay must
equal an eager call on the same inputs bit for bit (the kernels are
deterministic). Covered: the in-kernel small-batch plan with split requests,
the plan kernel with the combine of split requests, an E4M3 cache, several
query tokens per request, and sparse decode with its list prepass.
"""
import pytest
import torch

import mla_paged_attention_amd as mla
import workloads
from gpu_helpers import DEV, to_device

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.mark.parametrize("batch,num_heads,kv_dtype", [(6, 16, "bf16"), (100, 16, "bf16"),
                                                      (5, 128, "fp8")])
def test_graph_replays_match_eager(batch, num_heads, kv_dtype):
    gen = torch.Generator().manual_seed(batch)
    lens0 = torch.randint(1, 3000, (batch,), generator=gen).tolist()
    lens0[0] = 6000  # a request long enough to be cut into pieces
    wl = workloads.make_workload(batch=batch, num_heads=num_heads, seq=("fixed", lens0),
                                 block_size=64, seed=90 + batch, kv_dtype=kv_dtype)
    q, kv, bt, sl = to_device(wl)
    ws = torch.empty(mla.get_workspace_size(batch, num_heads, wl.max_blocks * wl.block_size, 0, 0),
                     dtype=torch.uint8, device=DEV)
    out = torch.empty((batch, num_heads, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((batch, num_heads), dtype=torch.float32, device=DEV)

    def call():
        mla.decode(q, kv, bt, sl, scale=wl.scale, kv_scale=wl.kv_scale, out=out, lse=lse,
                   workspace=ws)

    call()  # load the library and warm up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for rep in range(4):
        # New lengths within the same block tables: the plan is recomputed on
        # the device at every replay.
        new = [max(1, n - 97 * rep) for n in lens0]
        sl.copy_(torch.tensor(new, dtype=torch.int32))
        graph.replay()
        torch.cuda.synchronize()
        g_out, g_lse = out.clone(), lse.clone()
        eager_out, eager_lse = mla.decode(q, kv, bt, sl, scale=wl.scale, kv_scale=wl.kv_scale)
        torch.cuda.synchronize()
        assert torch.equal(g_out, eager_out), f"replay {rep}: out differs from eager"
        assert torch.equal(g_lse.view(torch.int32), eager_lse.view(torch.int32)), \
            f"replay {rep}: lse differs from eager"


def _replay_against_eager(graph, call_eager, out, lse, update, reps=4):
    for rep in range(reps):
        update(rep)
        graph.replay()
        torch.cuda.synchronize()
        g_out, g_lse = out.clone(), lse.clone()
        eager_out, eager_lse = call_eager()
        torch.cuda.synchronize()
        assert torch.equal(g_out, eager_out), f"replay {rep}: out differs from eager"
        assert torch.equal(g_lse.view(torch.int32), eager_lse.view(torch.int32)), \
            f"replay {rep}: lse differs from eager"


@pytest.mark.parametrize("q_len,num_heads,kv_dtype", [(3, 16, "bf16"), (2, 128, "fp8")])
def test_graph_multi_token(q_len, num_heads, kv_dtype):
    lens0 = [5000, 40, 700, 3, 1999, 64]
    wl = workloads.make_workload(batch=len(lens0), num_heads=num_heads, seq=("fixed", lens0),
                                 block_size=64, seed=95 + q_len, kv_dtype=kv_dtype, q_len=q_len)
    q, kv, bt, sl = to_device(wl)
    ws = torch.empty(mla.get_workspace_size(wl.batch, num_heads, wl.max_blocks * wl.block_size,
                                            0, 0, q_len=q_len), dtype=torch.uint8, device=DEV)
    o0, l0 = mla.decode(q, kv, bt, sl, scale=wl.scale, kv_scale=wl.kv_scale)
    out, lse = torch.empty_like(o0), torch.empty_like(l0)

    def call():
        mla.decode(q, kv, bt, sl, scale=wl.scale, kv_scale=wl.kv_scale, out=out, lse=lse,
                   workspace=ws)

    call()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    gen = torch.Generator().manual_seed(7)

    def update(rep):
        sl.copy_(torch.tensor([max(q_len, n - 113 * rep) for n in lens0], dtype=torch.int32))
        q.copy_(torch.randn(q.shape, generator=gen).to(q.dtype))

    _replay_against_eager(
        graph, lambda: mla.decode(q, kv, bt, sl, scale=wl.scale, kv_scale=wl.kv_scale),
        out, lse, update)


@pytest.mark.parametrize("kv_dtype,num_heads", [("bf16", 16), ("fp8", 32)])
def test_graph_sparse(kv_dtype, num_heads):
    lens0 = [3000, 17, 900, 64, 2500]
    topk = 1024
    wl = workloads.make_workload(batch=len(lens0), num_heads=num_heads, seq=("fixed", lens0),
                                 block_size=32, seed=97, kv_dtype=kv_dtype)
    q, kv, bt, sl = to_device(wl)
    gen = torch.Generator().manual_seed(11)

    def lists():
        idx = torch.full((wl.batch, topk), -1, dtype=torch.int32)
        for b, n in enumerate(sl.tolist()):
            k = min(n, topk)
            idx[b, :k] = torch.randperm(n, generator=gen)[:k].to(torch.int32)
        return idx

    idx = lists().to(DEV)
    ws = torch.empty(mla.get_workspace_size_sparse(wl.batch, num_heads, topk, 0, 0),
                     dtype=torch.uint8, device=DEV)
    out = torch.empty((wl.batch, num_heads, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((wl.batch, num_heads), dtype=torch.float32, device=DEV)

    def call():
        mla.decode_sparse(q, kv, bt, sl, idx, scale=wl.scale, kv_scale=wl.kv_scale, out=out,
                          lse=lse, workspace=ws)

    call()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()

    def update(rep):
        sl.copy_(torch.tensor([max(1, n - 211 * rep) for n in lens0], dtype=torch.int32))
        idx.copy_(lists().to(DEV))

    _replay_against_eager(
        graph, lambda: mla.decode_sparse(q, kv, bt, sl, idx, scale=wl.scale, kv_scale=wl.kv_scale),
        out, lse, update)
