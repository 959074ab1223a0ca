"""GPU parity of the per-head absorption products around the decode path.

mla_absorb_q and mla_absorb_out against the oracle's fp64 per-head
products on seeded bf16 operands. The error is the fp32 accumulation
(about 2^-24 of the sum of |terms| per add, 128 or 512 adds) plus the bf16
rounding of the result (at most 2^-9 relative): the tests allow
4e-3 |ref| + 1e-4 sum|terms|. The rope part of the query is copied and must
match bit for bit. A chained case runs absorption, decode and output
absorption and compares with the oracle's chain (bf16 between the steps,
as the tensors the steps exchange are bf16).
"""
import numpy as np
import pytest
import torch

import mla_paged_attention_amd as mla
import workloads
from gpu_helpers import DEV

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def bits(x):
    return x.contiguous().view(torch.int16).numpy().view(np.uint16)


def within(got, ref, mag, what):
    err = np.abs(got - ref)
    bound = 4e-3 * np.abs(ref) + 1e-4 * mag
    if (err > bound).any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: at {i} got {got[i]} ref {ref[i]} "
                             f"({int((err > bound).sum())} out of tolerance)")


def magnitude(x, w):
    return torch.matmul(x.double().abs().permute(1, 0, 2), w.double().abs()).permute(1, 0, 2).numpy()


# Shapes chosen so that each launch shape of mla_absorb_q runs, with ragged
# last row groups: 32-column slices (1, 17, 64 rows), 128-column slices with
# one tile per wave (100 x 20) or two (512 x 16, 250 x 32), 256-column slices
# (3 x 128, 130 x 128).
@pytest.mark.parametrize("batch,heads", [(1, 16), (17, 16), (64, 1), (100, 20), (512, 16),
                                         (250, 32), (3, 128), (130, 128)])
def test_absorb_q(orc, batch, heads):
    q_nope, q_rope, w_uk, _, _ = workloads.make_absorb(batch, heads, seed=batch + heads)
    q = mla.absorb_q(q_nope.to(DEV), w_uk.to(DEV), q_rope.to(DEV))
    torch.cuda.synchronize()
    q = q.cpu()
    ref = orc.absorb(bits(q_nope), bits(w_uk))
    within(q[..., :512].double().numpy(), ref, magnitude(q_nope, w_uk), f"absorb_q B={batch} H={heads}")
    assert torch.equal(q[..., 512:], q_rope), "rope part must be copied exactly"


@pytest.mark.parametrize("batch,heads", [(1, 16), (33, 16), (64, 5), (512, 16), (2, 128)])
def test_absorb_out(orc, batch, heads):
    _, _, _, o_lat, w_uv = workloads.make_absorb(batch, heads, seed=7 * batch + heads)
    o = mla.absorb_out(o_lat.to(DEV), w_uv.to(DEV))
    torch.cuda.synchronize()
    w_kn = w_uv.transpose(1, 2).contiguous()  # [H, 512, 128]: the oracle's [H, k, n]
    ref = orc.absorb(bits(o_lat), bits(w_kn))
    within(o.cpu().double().numpy(), ref, magnitude(o_lat, w_kn), f"absorb_out B={batch} H={heads}")


def test_absorb_decode_absorb_chain(orc):
    # q_nope, q_rope -> absorbed q -> paged decode -> absorbed output.
    wl = workloads.make_workload(batch=6, num_heads=16, seq=("fixed", [1, 40, 129, 500, 700, 2000]),
                                 block_size=32, seed=81, poison=True)
    q_nope, q_rope, w_uk, _, w_uv = workloads.make_absorb(6, 16, seed=82)
    q = mla.absorb_q(q_nope.to(DEV), w_uk.to(DEV), q_rope.to(DEV))
    out, _ = mla.decode(q, wl.kv.to(DEV), wl.block_table.to(DEV), wl.seq_lens.to(DEV),
                        scale=wl.scale)
    o = mla.absorb_out(out, w_uv.to(DEV))
    torch.cuda.synchronize()
    # Oracle chain, bf16 between the steps.
    q_ref = torch.cat([torch.from_numpy(orc.absorb(bits(q_nope), bits(w_uk))).to(torch.bfloat16),
                       q_rope], dim=-1)
    lat, _ = orc.attend(bits(q_ref), wl.kv_bits(), wl.block_table.numpy(), wl.seq_lens.numpy(),
                        wl.block_size, wl.scale)
    lat_bf = torch.from_numpy(lat).to(torch.bfloat16)
    o_ref = orc.absorb(bits(lat_bf), bits(w_uv.transpose(1, 2).contiguous()))
    got = o.cpu().double().numpy()
    # Each step's bf16 rounding can move the next; allow 2e-2 of the row scale.
    scale = np.abs(o_ref).max(axis=-1, keepdims=True)
    assert np.all(np.abs(got - o_ref) <= 2e-2 * np.abs(o_ref) + 2e-2 * scale), "absorb-decode-absorb chain"
