"""Decode captured in a HIP graph (torch.cuda.CUDAGraph on ROCm).

mla_decode allocates nothing and never synchronises the host, so a caller
may capture it. The captured call is replayed several times, with new
seq_lens and eager decode calls between the replays, and every replay must
equal an eager call on the same inputs bit for bit (the kernels are
deterministic). Covered: the in-kernel small-batch plan with split requests,
the plan kernel with the combine of split requests, and an E4M3 cache.
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
