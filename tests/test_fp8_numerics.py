"""Why the fp8 path carries q and P as two E4M3 terms (host-side emulation).

The fp8 cache path quantises q in-kernel and feeds P to fp8 matrix cores.
This emulation (fp64 arithmetic with torch's float8_e4m3fn rounding) shows
that one E4M3 term for q, or for P, can exceed the 2e-2 + 2e-2|ref| bound,
while the two-term form (rounded value + rounded residual, both E4M3 codes
in the same scale, so that one matrix instruction can take the pair as
a doubled contraction depth) stays well inside it. It tests the numerical design, not the
kernel; the GPU parity tests check the kernel against the oracle.
"""
import torch

import workloads

BOUND_ATOL = BOUND_RTOL = 2e-2


def e4m3(x):
    return x.clamp(-448, 448).to(torch.float8_e4m3fn).to(torch.float64)


def quantise_rows(q, two_terms):
    s1 = q.abs().amax(-1, keepdim=True) / 448
    hi = e4m3(q / s1) * s1
    if not two_terms:
        return hi
    # the residual is at most half an E4M3 step of 448 (16 codes), so it
    # fits the same scale without saturating
    return hi + e4m3((q - hi) / s1) * s1


def quantise_p(p, two_terms):
    ps = p * 256
    hi = e4m3(ps)
    return (hi + e4m3(ps - hi)) / 256 if two_terms else hi / 256


def worst_ratio(wl, two_q, two_p):
    deq = wl.kv.view(torch.float8_e4m3fn).to(torch.float64) * wl.kv_scale
    worst = 0.0
    for b in range(wl.batch):
        n = int(wl.seq_lens[b])
        rows = torch.stack([deq[int(wl.block_table[b, t // wl.block_size]), t % wl.block_size]
                            for t in range(n)])
        q = wl.q[b].to(torch.float64)
        x = wl.scale * q @ rows.T
        m = x.amax(1, keepdim=True)
        p = torch.exp(x - m)
        ref = (p @ rows[:, :512]) / p.sum(1, keepdim=True)
        xq = wl.scale * quantise_rows(q, two_q) @ rows.T
        pq = torch.exp(xq - m)
        out = (quantise_p(pq, two_p) @ rows[:, :512]) / pq.sum(1, keepdim=True)
        ratio = (out - ref).abs() / (BOUND_ATOL + BOUND_RTOL * ref.abs())
        worst = max(worst, float(ratio.max()))
    return worst


def test_two_term_q_and_p_fit_the_bound():
    short = workloads.make_workload(batch=5, num_heads=20, seq=("fixed", [1, 17, 100, 513, 2000]),
                                    block_size=64, seed=61, kv_dtype="fp8")
    long_rows = workloads.make_workload(batch=2, num_heads=128, seq=("fixed", [8192, 8192]),
                                        block_size=64, seed=6, kv_dtype="fp8")
    assert worst_ratio(short, True, True) < 0.5
    assert worst_ratio(long_rows, True, True) < 0.5
    # One E4M3 term for P is not enough on short rows, nor one for q on long ones.
    assert worst_ratio(short, True, False) > 1.0
    assert worst_ratio(long_rows, False, True) > 1.0


def test_tiny_q_rows_need_a_scale_floor():
    # A bf16 q row can be as small as 1e-38. Its E4M3 scale 448 / amax then
    # overflows fp32 (codes inf or NaN), so the kernel floors amax at 2^-100:
    # codes stay finite and such a row's logits (about 1e-37) still give the
    # uniform softmax the oracle computes.
    wl = workloads.make_workload(batch=2, num_heads=16, seq=("fixed", [40, 300]), block_size=64,
                                 seed=62, kv_dtype="fp8")
    q = wl.q.to(torch.float32) * 1e-37
    amax = q.abs().amax(-1, keepdim=True)
    assert not torch.isfinite(torch.tensor(448.0, dtype=torch.float32) / amax).all()
    floored = amax.clamp(min=2.0 ** -100)
    inv = torch.tensor(448.0, dtype=torch.float32) / floored
    codes = (q * inv).clamp(-448, 448).to(torch.float8_e4m3fn).to(torch.float64)
    assert torch.isfinite(codes).all() and codes.abs().max() <= 448
    deq = wl.kv.view(torch.float8_e4m3fn).to(torch.float64) * wl.kv_scale
    for b in range(wl.batch):
        n = int(wl.seq_lens[b])
        rows = torch.stack([deq[int(wl.block_table[b, t // wl.block_size]), t % wl.block_size]
                            for t in range(n)])
        x_ref = wl.scale * q[b].to(torch.float64) @ rows.T
        x_emu = wl.scale * (codes[b] * (floored[b].to(torch.float64) / 448)) @ rows.T
        assert float((x_ref - x_emu).abs().max()) < 1e-30
        ref = torch.softmax(x_ref, 1) @ rows[:, :512]
        emu = torch.softmax(x_emu, 1) @ rows[:, :512]
        assert float(((emu - ref).abs() / (BOUND_ATOL + BOUND_RTOL * ref.abs())).max()) < 0.01
