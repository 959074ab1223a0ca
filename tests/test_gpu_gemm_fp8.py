"""GPU parity of the block-scaled E4M3 projection beside the decode path.

mla_quant_fp8_groups against the oracle's group quantisation: codes and
scales bit-exact (an integer decision taken in fp32 on both sides).
mla_gemm_fp8_blockscale against the oracle's fp64 definition on seeded
synthetic codes and scales. Each 128-wide block's products of E4M3 values
are exact in fp32, so the error is the fp32 scaling and accumulation (about
2^-24 of the sum of |terms| per step, 56 steps at k = 7168) plus the final
bf16 rounding (at most 2^-9 relative): the test allows
4e-3 |ref| + 1e-5 sum|terms|.
"""
import numpy as np
import pytest
import torch

import mla_paged_attention_amd as mla
import workloads

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda:0"


def deq_abs(codes, scale_expanded):
    return codes.view(torch.float8_e4m3fn).double().abs() * scale_expanded.double()


def check_gemm(orc, m, n, k, seed, rows=None):
    a, sa, b, sb = workloads.make_gemm(m, n, k, seed)
    c = mla.gemm_fp8_blockscale(a.to(DEV), sa.to(DEV), b.to(DEV), sb.to(DEV))
    torch.cuda.synchronize()
    c = c.float().cpu().double().numpy()
    assert np.isfinite(c).all()
    rows = np.arange(m) if rows is None else np.asarray(rows)
    ref = orc.gemm_fp8_blockscale(a.numpy()[rows], sa.numpy()[rows], b.numpy(), sb.numpy())
    sa_e = sa[rows].repeat_interleave(128, dim=1)
    sb_e = sb.repeat_interleave(128, dim=0)[:n].repeat_interleave(128, dim=1)
    mag = (deq_abs(a[rows], sa_e) @ deq_abs(b, sb_e).T).numpy()
    err = np.abs(c[rows] - ref)
    bound = 4e-3 * np.abs(ref) + 1e-5 * mag
    if (err > bound).any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"gemm m={m} n={n} k={k}: c{i} = {c[rows][i]} ref {ref[i]} "
                             f"({int((err > bound).sum())} out of tolerance)")


@pytest.mark.parametrize("m,n,k", [(1, 2112, 7168), (4, 2112, 7168), (16, 576, 7168),
                                   (17, 576, 1024), (33, 16, 128), (64, 2112, 2048),
                                   (100, 576, 1152), (2, 48, 384), (1, 16, 128),
                                   (3, 32, 16384), (16, 2112, 9088), (4, 32, 8192),
                                   (5, 64, 8192)])
def test_gemm_matches_oracle(orc, m, n, k):
    check_gemm(orc, m, n, k, seed=m + n + k)


@pytest.mark.parametrize("m", [64, 256])
def test_gemm_full_shape(orc, m):
    # DeepSeek-R1's fused q/kv down-projection at decode batch m; every row.
    check_gemm(orc, m, 2112, 7168, seed=900 + m)


@pytest.mark.parametrize("m,k", [(1, 128), (5, 7168), (64, 1024), (300, 256)])
def test_quant_bit_exact(orc, m, k):
    gen = torch.Generator().manual_seed(m * 7 + k)
    mag = torch.exp2(torch.randint(-12, 12, (m, 1), generator=gen).float())
    x = (torch.randn((m, k), generator=gen) * mag).to(torch.bfloat16)
    x[0, :128] = 0.0                       # one all-zero group
    if m > 1:
        x[1, 5] = -0.0
    codes, scale = mla.quant_fp8_groups(x.to(DEV))
    torch.cuda.synchronize()
    ref_codes, ref_scale = orc.quant_fp8_groups(x)
    got_c = codes.cpu().numpy()
    bad = np.flatnonzero(got_c.ravel() != ref_codes.ravel())
    assert bad.size == 0, f"{bad.size} codes differ, first at {np.unravel_index(bad[0], got_c.shape)}"
    assert np.array_equal(scale.cpu().numpy(), ref_scale), "scales differ"


def test_quant_then_gemm_matches_oracle(orc):
    # The projection as used: bf16 activations quantised on the GPU, then the
    # GEMM; the oracle quantises the same activations itself.
    gen = torch.Generator().manual_seed(31)
    x = torch.randn((8, 7168), generator=gen).to(torch.bfloat16)
    _, _, b, sb = workloads.make_gemm(1, 2112, 7168, 32)
    codes, scale = mla.quant_fp8_groups(x.to(DEV))
    c = mla.gemm_fp8_blockscale(codes, scale, b.to(DEV), sb.to(DEV))
    torch.cuda.synchronize()
    ra, rsa = orc.quant_fp8_groups(x)
    ref = orc.gemm_fp8_blockscale(ra, rsa, b.numpy(), sb.numpy())
    got = c.float().cpu().double().numpy()
    assert np.all(np.abs(got - ref) <= 4e-3 * np.abs(ref) + 1e-3 * np.abs(ref).max())
