"""Shared helpers of the GPU parity tests: run the HIP path and the oracle on
the same seeded inputs and compare element by element."""
from __future__ import annotations

import numpy as np
import torch

import mla_paged_attention_amd as mla

# Tolerances (|gpu - ref| <= atol + rtol * |ref|, ref = fp64 oracle).
BF16_OUT_ATOL, BF16_OUT_RTOL, BF16_LSE_ATOL = 1e-2, 1e-2, 1e-3
FP8_ATOL, FP8_RTOL = 2e-2, 2e-2

DEV = "cuda:0"


def to_device(wl):
    return (wl.q.to(DEV), wl.kv.to(DEV), wl.block_table.to(DEV), wl.seq_lens.to(DEV))


def run_gpu(wl, num_splits=0, dev_tensors=None, **kw):
    q, kv, bt, sl = dev_tensors if dev_tensors is not None else to_device(wl)
    out, lse = mla.decode(q, kv, bt, sl, scale=wl.scale, num_splits=num_splits,
                          kv_scale=wl.kv_scale, **kw)
    torch.cuda.synchronize()
    return out, lse


def to_np(out, lse):
    return out.float().cpu().double().numpy(), lse.cpu().double().numpy()


def run_oracle(orc, wl, req=None):
    return orc.attend(wl.q_bits(), wl.kv_bits(), wl.block_table.numpy(), wl.seq_lens.numpy(),
                      wl.block_size, wl.scale, kv_fp8=wl.kv_dtype == "fp8",
                      kv_scale=wl.kv_scale, req=req)


def compare(out, lse, ref_out, ref_lse, kv_dtype="bf16", what=""):
    """Assert the HIP result matches the oracle within the stated tolerances."""
    out = np.asarray(out, np.float64)
    lse = np.asarray(lse, np.float64)
    if kv_dtype == "fp8":
        o_atol, o_rtol, l_atol, l_rtol = FP8_ATOL, FP8_RTOL, FP8_ATOL, FP8_RTOL
    else:
        o_atol, o_rtol, l_atol, l_rtol = BF16_OUT_ATOL, BF16_OUT_RTOL, BF16_LSE_ATOL, 0.0
    assert out.shape == ref_out.shape and lse.shape == ref_lse.shape
    assert np.isfinite(out).all(), f"{what}: non-finite output"
    err = np.abs(out - ref_out)
    bound = o_atol + o_rtol * np.abs(ref_out)
    bad = err > bound
    if bad.any():
        idx = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: out mismatch at {idx}: gpu {out[idx]} ref {ref_out[idx]} "
                             f"({int(bad.sum())} elements out of tolerance, max abs err "
                             f"{err.max():.3e})")
    ninf = np.isneginf(ref_lse)
    assert (np.isneginf(lse) == ninf).all(), f"{what}: -inf lse pattern differs"
    lerr = np.abs(lse[~ninf] - ref_lse[~ninf])
    lbound = l_atol + l_rtol * np.abs(ref_lse[~ninf])
    if (lerr > lbound).any():
        i = int(np.argmax(lerr - lbound))
        raise AssertionError(f"{what}: lse mismatch: gpu {lse[~ninf][i]} ref {ref_lse[~ninf][i]} "
                             f"(max abs err {lerr.max():.3e})")
    return float(err.max()) if err.size else 0.0, float(lerr.max()) if lerr.size else 0.0
