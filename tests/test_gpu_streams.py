"""Calls in flight at once on separate streams.

The library keeps no state between calls: each call's plan, partial rows and
combine live in the caller's workspace, and every kernel is enqueued on the
caller's stream. Two decodes of different shapes and cache types, each with
its own stream and workspace, therefore overlap freely, and each must equal
the same call run alone, bit for bit, on every repetition.
"""
import pytest
import torch

import mla_paged_attention_amd as mla
import workloads
from gpu_helpers import DEV, to_device

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def test_concurrent_streams_with_own_workspaces():
    wa = workloads.make_workload(batch=40, num_heads=16, seq=("uniform", 100, 5000),
                                 block_size=64, seed=81)
    wb = workloads.make_workload(batch=7, num_heads=128, seq=("uniform", 1000, 9000),
                                 block_size=32, seed=82, kv_dtype="fp8")
    da, db = to_device(wa), to_device(wb)
    ref_a = mla.decode(*da, scale=wa.scale)
    ref_b = mla.decode(*db, scale=wb.scale, kv_scale=wb.kv_scale)
    torch.cuda.synchronize()

    def workspace(wl):
        n = mla.get_workspace_size(wl.batch, wl.num_heads, wl.max_blocks * wl.block_size, 0, 0)
        return torch.empty(n, dtype=torch.uint8, device=DEV)

    wsa, wsb = workspace(wa), workspace(wb)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()  # default priority
    for rep in range(4):
        with torch.cuda.stream(sa):
            out_a, lse_a = mla.decode(*da, scale=wa.scale, workspace=wsa, stream=sa)
        with torch.cuda.stream(sb):
            out_b, lse_b = mla.decode(*db, scale=wb.scale, kv_scale=wb.kv_scale, workspace=wsb,
                                      stream=sb)
        torch.cuda.synchronize()
        assert torch.equal(out_a, ref_a[0]) and torch.equal(lse_a, ref_a[1]), f"stream a, rep {rep}"
        assert torch.equal(out_b, ref_b[0]) and torch.equal(lse_b, ref_b[1]), f"stream b, rep {rep}"


def test_cached_workspace_on_a_side_stream_grows(orc):
    # No workspace passed: the binding's cached buffer for the side stream is
    # replaced by a larger one at each call, and the outputs are allocated on
    # that stream too. Every result must still match the oracle after the
    # stream has drained (nothing freed and reused while a kernel used it).
    from gpu_helpers import compare, run_oracle, to_np

    mla.release_workspaces()
    side = torch.cuda.Stream()  # default priority
    runs = []
    for i, (batch, hi) in enumerate(((2, 300), (9, 4000), (40, 20000), (300, 3000))):
        wl = workloads.make_workload(batch=batch, num_heads=16, seq=("uniform", 1, hi),
                                     block_size=32, seed=90 + i)
        dev = to_device(wl)
        side.wait_stream(torch.cuda.current_stream())
        out, lse = mla.decode(*dev, scale=wl.scale, stream=side)
        runs.append((wl, dev, out, lse))
    torch.cuda.synchronize()
    for wl, _, out, lse in runs:
        o, l = to_np(out, lse)
        compare(o, l, *run_oracle(orc, wl), what=f"side stream, batch {wl.batch}")
    mla.release_workspaces()
