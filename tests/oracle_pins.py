"""Pins that tie the fp64 oracle to facts outside itself.

Each pin checks the oracle against something it does not share code with:
a library routine (torch's float64 scaled_dot_product_attention, with its own
causal mask for several query tokens, and logsumexp,
torch's float8_e4m3fn and bfloat16 decoders, numpy's logaddexp), a closed form
of softmax attention, or an invariant the pages fix (split-then-merge equals
unsplit; zero-padding heads to 128 leaves the real heads alone; a physical
block permutation under a matching table changes nothing).

The same pins run against deliberately broken copies of the oracle source in
``test_oracle_mutants.py``; every plausible mistake must trip at least one.

Run as a script (``python tests/oracle_pins.py --lib PATH``) to check one
library build: exit status 0 if every pin holds, 1 otherwise.
"""
from __future__ import annotations

import argparse
import math
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads  # noqa: E402

TOL = 1e-12
S = workloads.SCALE


def _bf16(x: torch.Tensor) -> torch.Tensor:
    return x.to(torch.bfloat16)


def _bits(x: torch.Tensor) -> np.ndarray:
    return x.contiguous().view(torch.int16).numpy().view(np.uint16)


def _paged_from_dense(dense_list, block_size, gen, extra_blocks=0, poison=True):
    """Scatter dense per-request [N_b, 576] bf16 rows into a shuffled page pool."""
    nblk = [(d.shape[0] + block_size - 1) // block_size for d in dense_list]
    pool = sum(nblk) + extra_blocks
    perm = torch.randperm(pool, generator=gen)
    max_blocks = max(1, max(nblk))
    table = torch.full((len(dense_list), max_blocks), -1, dtype=torch.int32)
    kv = torch.full((pool, block_size, 576), float("nan"), dtype=torch.bfloat16)
    if not poison:
        kv = _bf16(torch.randn((pool, block_size, 576), generator=gen))
    off = 0
    for b, d in enumerate(dense_list):
        for j in range(nblk[b]):
            blk = int(perm[off + j])
            table[b, j] = blk
            rows = d[j * block_size:(j + 1) * block_size]
            kv[blk, :rows.shape[0]] = rows
        off += nblk[b]
    seq = torch.tensor([d.shape[0] for d in dense_list], dtype=torch.int32)
    return kv, table, seq


def _sdpa64(q_bf16: torch.Tensor, k_bf16: torch.Tensor, scale: float):
    """Library reference for one request: q [H, 576], k [N, 576] -> out [H, 512], lse [H]."""
    q = q_bf16.to(torch.float64)[None, :, None, :]            # [1, H, 1, 576]
    k = k_bf16.to(torch.float64)[None, None, :, :].expand(1, q.shape[1], -1, -1)
    v = k[..., :512]
    out = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=scale)[0, :, 0, :]
    logits = scale * (q_bf16.to(torch.float64) @ k_bf16.to(torch.float64).T)
    return out.numpy(), torch.logsumexp(logits, dim=-1).numpy()


def _close(a, b, tol=TOL):
    a, b = np.asarray(a), np.asarray(b)
    return a.shape == b.shape and bool(np.all(np.abs(a - b) <= tol * (1 + np.abs(b))))


# --------------------------------------------------------------------------- pins

def pin_e4m3_decode(orc):
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = orc.e4m3_to_double(codes)
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all(), "E4M3 NaN codes differ"
    assert (got[~nan] == ref[~nan]).all(), "E4M3 decode differs from torch float8_e4m3fn"


def pin_bf16_widen(orc):
    gen = torch.Generator().manual_seed(11)
    x = _bf16(torch.randn(4096, generator=gen) * 100)
    got = orc.bf16_to_double(_bits(x))
    assert (got == x.to(torch.float64).numpy()).all(), "bf16 widening differs from torch"


def pin_sdpa_identity_table(orc):
    """One request, pages in order: equals float64 SDPA with Eq=576, Ev=512."""
    gen = torch.Generator().manual_seed(1)
    H, N, bs = 5, 45, 16
    q = _bf16(torch.randn((1, H, 576), generator=gen))
    k = _bf16(torch.randn((N, 576), generator=gen))
    nb = (N + bs - 1) // bs
    kv = _bf16(torch.randn((nb * bs, 576), generator=gen))
    kv[:N] = k
    table = torch.arange(nb, dtype=torch.int32)[None]
    out, lse = orc.attend(_bits(q), _bits(kv.view(nb, bs, 576)), table.numpy(),
                          np.array([N], np.int32), bs, S)
    ref_out, ref_lse = _sdpa64(q[0], k, S)
    assert _close(out[0], ref_out), "out differs from float64 SDPA"
    assert _close(lse[0], ref_lse), "lse differs from float64 logsumexp"


def pin_sdpa_shuffled_pages(orc):
    """Ragged requests scattered over shuffled pages (unused slots NaN) equal dense SDPA."""
    gen = torch.Generator().manual_seed(2)
    H = 3
    for bs in (16, 32, 64):
        lens = [1, 15, 16, 17, 70, 131]
        dense = [_bf16(torch.randn((n, 576), generator=gen)) for n in lens]
        kv, table, seq = _paged_from_dense(dense, bs, gen, extra_blocks=3)
        q = _bf16(torch.randn((len(lens), H, 576), generator=gen))
        out, lse = orc.attend(_bits(q), _bits(kv), table.numpy(), seq.numpy(), bs, S)
        for b in range(len(lens)):
            ref_out, ref_lse = _sdpa64(q[b], dense[b], S)
            assert _close(out[b], ref_out), f"paged out differs (bs={bs}, b={b})"
            assert _close(lse[b], ref_lse), f"paged lse differs (bs={bs}, b={b})"


def pin_closed_forms(orc):
    gen = torch.Generator().manual_seed(3)
    H, bs = 4, 16
    # N = 1: out is the single value row, lse its logit.
    q = _bf16(torch.randn((1, H, 576), generator=gen))
    k = _bf16(torch.randn((1, 576), generator=gen))
    kv, table, seq = _paged_from_dense([k], bs, gen)
    out, lse = orc.attend(_bits(q), _bits(kv), table.numpy(), seq.numpy(), bs, S)
    v0 = k[0, :512].to(torch.float64).numpy()
    x0 = S * (q[0].to(torch.float64) @ k[0].to(torch.float64)).numpy()
    assert (out[0] == v0[None, :]).all(), "N=1: out must equal v_0 exactly"
    assert _close(lse[0], x0), "N=1: lse must equal the logit"
    # q = 0: uniform weights, out = mean of value rows, lse = ln N.
    N = 29
    k = _bf16(torch.randn((N, 576), generator=gen))
    kv, table, seq = _paged_from_dense([k], bs, gen)
    qz = torch.zeros((1, H, 576), dtype=torch.bfloat16)
    out, lse = orc.attend(_bits(qz), _bits(kv), table.numpy(), seq.numpy(), bs, S)
    mean = k[:, :512].to(torch.float64).mean(0).numpy()
    assert _close(out[0], np.broadcast_to(mean, (H, 512))), "q=0: out must be the mean row"
    assert _close(lse[0], np.full(H, math.log(N))), "q=0: lse must be ln N"
    # Equal kv_c rows (rope random): out = that row for any q.
    c = _bf16(torch.randn((576,), generator=gen))
    k = _bf16(torch.randn((N, 576), generator=gen))
    k[:, :512] = c[:512]
    kv, table, seq = _paged_from_dense([k], bs, gen)
    q = _bf16(torch.randn((1, H, 576), generator=gen))
    out, lse = orc.attend(_bits(q), _bits(kv), table.numpy(), seq.numpy(), bs, S)
    assert _close(out[0], np.broadcast_to(c[:512].to(torch.float64).numpy(), (H, 512))), \
        "equal value rows: out must equal that row"
    # All 576-wide rows equal: lse = x + ln N.
    k = c[None, :].expand(N, 576).contiguous()
    kv, table, seq = _paged_from_dense([k], bs, gen)
    out, lse = orc.attend(_bits(q), _bits(kv), table.numpy(), seq.numpy(), bs, S)
    x = S * (q[0].to(torch.float64) @ c.to(torch.float64)).numpy()
    assert _close(lse[0], x + math.log(N)), "equal rows: lse must be x + ln N"
    # N = 2: out = sigmoid(x0 - x1) v0 + sigmoid(x1 - x0) v1.
    k = _bf16(torch.randn((2, 576), generator=gen) * 0.3)
    kv, table, seq = _paged_from_dense([k], bs, gen)
    out, lse = orc.attend(_bits(q), _bits(kv), table.numpy(), seq.numpy(), bs, S)
    k64 = k.to(torch.float64).numpy()
    x = S * (q[0].to(torch.float64).numpy() @ k64.T)            # [H, 2]
    sig = 1.0 / (1.0 + np.exp(-(x[:, 0] - x[:, 1])))
    ref = sig[:, None] * k64[0, :512] + (1 - sig)[:, None] * k64[1, :512]
    assert _close(out[0], ref), "N=2 closed form"
    assert _close(lse[0], np.logaddexp(x[:, 0], x[:, 1])), "N=2 lse = logaddexp(x0, x1)"


def pin_empty_request(orc):
    gen = torch.Generator().manual_seed(4)
    q = _bf16(torch.randn((2, 2, 576), generator=gen))
    k = _bf16(torch.randn((5, 576), generator=gen))
    kv, table, _ = _paged_from_dense([k, k], 16, gen)
    out, lse = orc.attend(_bits(q), _bits(kv), table.numpy(), np.array([0, 5], np.int32),
                          16, S)
    assert (out[0] == 0).all() and np.isneginf(lse[0]).all(), "empty request: out 0, lse -inf"
    assert np.isfinite(lse[1]).all()


def pin_split_merge(orc):
    """Any partition into contiguous ranges, merged by LSE, equals the unsplit result."""
    wl = workloads.make_workload(batch=3, num_heads=4, seq=("fixed", [1, 77, 200]),
                                 block_size=16, seed=5, poison=True)
    args = (wl.q_bits(), wl.kv_bits(), wl.block_table.numpy(), wl.seq_lens.numpy(),
            wl.block_size, wl.scale)
    full_out, full_lse = orc.attend(*args)
    rng = np.random.default_rng(5)
    for b in range(wl.batch):
        n = int(wl.seq_lens[b])
        for n_parts in (1, 2, 3, 7):
            cuts = np.sort(rng.integers(0, n + 1, size=n_parts - 1))
            edges = np.concatenate([[0], cuts, [n]]).astype(np.int64)
            req = np.full(n_parts, b, np.int32)
            po, pl = orc.attend(*args, req=req, tok_begin=edges[:-1], tok_end=edges[1:])
            mo, ml = orc.lse_merge(po, pl)
            assert _close(mo, full_out[b]), f"split-merge out (b={b}, parts={n_parts})"
            assert _close(ml, full_lse[b]), f"split-merge lse (b={b}, parts={n_parts})"


def pin_merge_closed_form(orc):
    rng = np.random.default_rng(6)
    po = rng.standard_normal((3, 2, 512))
    pl = np.array([[0.5, -np.inf], [2.0, -np.inf], [-np.inf, -np.inf]])
    out, lse = orc.lse_merge(po, pl)
    w0, w1 = 1 / (1 + math.exp(1.5)), 1 / (1 + math.exp(-1.5))
    assert _close(lse[0], np.logaddexp(0.5, 2.0)), "merge lse = logaddexp"
    assert _close(out[0], w0 * po[0, 0] + w1 * po[1, 0]), "merge weights = softmax(lse)"
    assert (out[1] == 0).all() and np.isneginf(lse[1]), "all-empty merge: out 0, lse -inf"


def pin_rope_shift(orc):
    """A rope vector shared by every key shifts all logits equally: out unchanged,
    lse moves by scale * <q_rope, r>."""
    gen = torch.Generator().manual_seed(7)
    H, N, bs = 4, 50, 16
    k = _bf16(torch.randn((N, 576), generator=gen))
    r = _bf16(torch.randn((64,), generator=gen))
    k0 = k.clone()
    k0[:, 512:] = 0
    k1 = k.clone()
    k1[:, 512:] = r
    q = _bf16(torch.randn((1, H, 576), generator=gen))
    res = []
    for kk in (k0, k1):
        kv, table, seq = _paged_from_dense([kk], bs, torch.Generator().manual_seed(8))
        res.append(orc.attend(_bits(q), _bits(kv), table.numpy(), seq.numpy(), bs, S))
    shift = S * (q[0, :, 512:].to(torch.float64) @ r.to(torch.float64)).numpy()
    assert _close(res[1][0], res[0][0]), "shared rope vector must not change out"
    assert _close(res[1][1][0], res[0][1][0] + shift), "shared rope vector shifts lse"


def pin_head_padding(orc):
    """Zero-padding heads to 128 leaves the real heads bitwise unchanged; the padded
    heads give the uniform-weight closed form."""
    wl = workloads.make_workload(batch=2, num_heads=16, seq=("fixed", [37, 130]),
                                 block_size=16, seed=9)
    args = (wl.kv_bits(), wl.block_table.numpy(), wl.seq_lens.numpy(), wl.block_size,
            wl.scale)
    out16, lse16 = orc.attend(wl.q_bits(), *args)
    q128 = torch.zeros((2, 128, 576), dtype=torch.bfloat16)
    q128[:, :16] = wl.q
    out128, lse128 = orc.attend(_bits(q128), *args)
    assert (out128[:, :16] == out16).all() and (lse128[:, :16] == lse16).all(), \
        "padding heads changed the real heads"
    for b in range(2):
        n = int(wl.seq_lens[b])
        rows = []
        for t in range(n):
            blk = int(wl.block_table[b, t // 16])
            rows.append(wl.kv[blk, t % 16, :512].to(torch.float64).numpy())
        mean = np.mean(rows, axis=0)
        assert _close(out128[b, 16:], np.broadcast_to(mean, (112, 512))), "padded heads: mean"
        assert _close(lse128[b, 16:], np.full(112, math.log(n))), "padded heads: ln N"


def pin_block_permutation(orc):
    """Permuting the physical pool under a matching table leaves results bitwise equal."""
    wl = workloads.make_workload(batch=3, num_heads=4, seq=("fixed", [5, 64, 100]),
                                 block_size=16, seed=10, pool_blocks=14)
    out_a, lse_a = orc.attend(wl.q_bits(), wl.kv_bits(), wl.block_table.numpy(),
                              wl.seq_lens.numpy(), 16, wl.scale)
    perm = torch.randperm(wl.num_blocks, generator=torch.Generator().manual_seed(10))
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(wl.num_blocks)
    kv_p = wl.kv[perm]                       # new block j holds old block perm[j]
    table = wl.block_table.clone()
    valid = table >= 0
    table[valid] = inv[table[valid].long()].to(torch.int32)
    out_b, lse_b = orc.attend(wl.q_bits(), _bits(kv_p), table.numpy(), wl.seq_lens.numpy(),
                              16, wl.scale)
    assert (out_a == out_b).all() and (lse_a == lse_b).all(), "block permutation changed results"


def pin_batch_independence(orc):
    wl = workloads.make_workload(batch=3, num_heads=4, seq=("fixed", [40, 64, 100]),
                                 block_size=16, seed=12)
    args = (wl.kv_bits(), wl.block_table.numpy(), wl.block_size, wl.scale)
    out_a, lse_a = orc.attend(wl.q_bits(), args[0], args[1], wl.seq_lens.numpy(), *args[2:])
    q2 = wl.q.clone()
    q2[1:] = _bf16(torch.randn(q2[1:].shape, generator=torch.Generator().manual_seed(1)))
    seq2 = wl.seq_lens.clone()
    seq2[1:] = torch.tensor([3, 99], dtype=torch.int32)
    out_b, lse_b = orc.attend(_bits(q2), args[0], args[1], seq2.numpy(), *args[2:])
    assert (out_a[0] == out_b[0]).all() and (lse_a[0] == lse_b[0]).all(), \
        "request 0 depends on other requests"


def pin_fp8_dequant(orc):
    """E4M3 cache with a per-tensor scale equals float64 SDPA on the dequantised rows."""
    wl = workloads.make_workload(batch=2, num_heads=4, seq=("fixed", [20, 90]), block_size=16,
                                 seed=13, kv_dtype="fp8")
    out, lse = orc.attend(wl.q_bits(), wl.kv_bits(), wl.block_table.numpy(),
                          wl.seq_lens.numpy(), 16, wl.scale, kv_fp8=True,
                          kv_scale=wl.kv_scale)
    deq = wl.kv.view(torch.float8_e4m3fn).to(torch.float64) * wl.kv_scale
    for b in range(2):
        n = int(wl.seq_lens[b])
        rows = torch.stack([deq[int(wl.block_table[b, t // 16]), t % 16] for t in range(n)])
        q = wl.q[b].to(torch.float64)[None, :, None, :]
        kk = rows[None, None].expand(1, 4, -1, -1)
        ref = torch.nn.functional.scaled_dot_product_attention(
            q, kk, kk[..., :512], scale=wl.scale)[0, :, 0].numpy()
        ref_lse = torch.logsumexp(wl.scale * (wl.q[b].to(torch.float64) @ rows.T), -1).numpy()
        assert _close(out[b], ref), f"fp8 out differs from SDPA on dequantised rows (b={b})"
        assert _close(lse[b], ref_lse), f"fp8 lse differs (b={b})"


def pin_multi_token_causal_sdpa(orc):
    """q_len query tokens are the last q_len rows of square causal attention over
    the request: torch's float64 SDPA with is_causal=True (the library's own
    causal mask) fixes which cache tokens each query token sees. Query tokens
    with no position in the request (q_len > N) see nothing: out 0, lse -inf."""
    gen = torch.Generator().manual_seed(14)
    H, bs = 3, 16
    for n, q_len in ((1, 1), (5, 2), (40, 4), (77, 7), (3, 5), (33, 33)):
        k = _bf16(torch.randn((n, 576), generator=gen))
        q_all = _bf16(torch.randn((n, H, 576), generator=gen))
        kv, table, seq = _paged_from_dense([k], bs, gen, extra_blocks=1)
        q = torch.zeros((1, q_len, H, 576), dtype=torch.bfloat16)
        first = max(0, n - q_len)           # request position of the first real query
        pad = max(0, q_len - n)             # query tokens before position 0
        q[0, pad:] = q_all[first:]
        if pad:
            q[0, :pad] = _bf16(torch.randn((pad, H, 576), generator=gen))
        out, lse = orc.attend(_bits(q), _bits(kv), table.numpy(), seq.numpy(), bs, S)
        qq = q_all.to(torch.float64).permute(1, 0, 2)[None]          # [1, H, n, 576]
        kk = k.to(torch.float64)[None, None].expand(1, H, -1, -1)
        ref = torch.nn.functional.scaled_dot_product_attention(
            qq, kk, kk[..., :512], is_causal=True, scale=S)[0]       # [H, n, 512]
        logits = S * (qq[0] @ k.to(torch.float64).T)                  # [H, n, n]
        causal = torch.ones((n, n), dtype=torch.bool).tril()
        ref_lse = torch.logsumexp(logits.masked_fill(~causal, float("-inf")), -1)  # [H, n]
        for i in range(q_len):
            pos = i - pad + first
            if i < pad:
                assert (out[0, i] == 0).all() and np.isneginf(lse[0, i]).all(), \
                    f"query before position 0 must be empty (n={n}, q_len={q_len}, i={i})"
                continue
            assert _close(out[0, i], ref[:, pos].numpy()), \
                f"causal out differs (n={n}, q_len={q_len}, i={i})"
            assert _close(lse[0, i], ref_lse[:, pos].numpy()), \
                f"causal lse differs (n={n}, q_len={q_len}, i={i})"


def pin_multi_token_rows_are_single_decodes(orc):
    """Query token i of a paged, ragged, NaN-poisoned batch equals one-token decode
    of the same request cut to its first N - q_len + 1 + i tokens."""
    q_len = 3
    wl = workloads.make_workload(batch=4, num_heads=2, seq=("fixed", [2, 17, 64, 130]),
                                 block_size=16, seed=15, poison=True, q_len=q_len)
    args = (wl.kv_bits(), wl.block_table.numpy())
    out, lse = orc.attend(wl.q_bits(), *args, wl.seq_lens.numpy(), 16, wl.scale)
    for i in range(q_len):
        cut = np.maximum(wl.seq_lens.numpy() - (q_len - 1 - i), 0).astype(np.int32)
        q1 = wl.q[:, i].contiguous()
        o1, l1 = orc.attend(_bits(q1), *args, cut, 16, wl.scale)
        assert (out[:, i] == o1).all() and (lse[:, i] == l1).all(), \
            f"query token {i} differs from a one-token decode of its visible prefix"


def pin_multi_token_split_merge(orc):
    """With q_len query tokens, token ranges merged by LSE equal the unsplit result
    (a range past a query token's position is empty for it)."""
    q_len = 4
    wl = workloads.make_workload(batch=2, num_heads=3, seq=("fixed", [6, 90]), block_size=16,
                                 seed=16, poison=True, q_len=q_len)
    args = (wl.q_bits(), wl.kv_bits(), wl.block_table.numpy(), wl.seq_lens.numpy(),
            wl.block_size, wl.scale)
    full_out, full_lse = orc.attend(*args)
    for b in range(wl.batch):
        n = int(wl.seq_lens[b])
        edges = np.array([0, n // 3, n - 2, n - 1, n], np.int64)
        req = np.full(len(edges) - 1, b, np.int32)
        po, pl = orc.attend(*args, req=req, tok_begin=edges[:-1], tok_end=edges[1:])
        mo, ml = orc.lse_merge(po.reshape(len(req), q_len * 3, 512), pl.reshape(len(req), -1))
        assert _close(mo, full_out[b].reshape(q_len * 3, 512)), f"multi-token split-merge (b={b})"
        assert _close(ml, full_lse[b].reshape(-1)), f"multi-token split-merge lse (b={b})"


def pin_sparse_all_positions_is_dense(orc):
    """Listing every position in order (padded with -1) is exactly dense decode."""
    wl = workloads.make_workload(batch=4, num_heads=3, seq=("fixed", [0, 5, 33, 100]),
                                 block_size=16, seed=17, poison=True)
    idx = np.full((4, 120), -1, np.int32)
    for b, n in enumerate(wl.seq_lens.tolist()):
        idx[b, :n] = np.arange(n)
    args = (wl.q_bits(), wl.kv_bits(), wl.block_table.numpy(), wl.seq_lens.numpy(), 16,
            wl.scale)
    out, lse = orc.attend_sparse(*args, idx)
    ref_out, ref_lse = orc.attend(*args)
    assert (out == ref_out).all() and np.array_equal(lse, ref_lse), "all positions != dense"


def pin_sparse_sdpa_on_gathered_rows(orc):
    """Random lists with repeats, any order, and skipped entries equal float64 SDPA
    over the gathered rows (repeats included), for bf16 and E4M3 caches."""
    rng = np.random.default_rng(18)
    for kv_dtype in ("bf16", "fp8"):
        wl = workloads.make_workload(batch=3, num_heads=4, seq=("fixed", [1, 40, 150]),
                                     block_size=16, seed=18, kv_dtype=kv_dtype, poison=True)
        topk = 24
        idx = np.full((3, topk), -1, np.int32)
        for b, n in enumerate(wl.seq_lens.tolist()):
            pick = rng.integers(0, n, size=topk - 4)
            junk = np.array([-1, n, n + 7, -3])                 # skipped entries
            row = np.concatenate([pick, junk])
            rng.shuffle(row)
            idx[b] = row
        fp8 = kv_dtype == "fp8"
        out, lse = orc.attend_sparse(wl.q_bits(), wl.kv_bits(), wl.block_table.numpy(),
                                     wl.seq_lens.numpy(), 16, wl.scale, idx, kv_fp8=fp8,
                                     kv_scale=wl.kv_scale)
        if fp8:
            deq = wl.kv.view(torch.float8_e4m3fn).to(torch.float64) * wl.kv_scale
        else:
            deq = wl.kv.to(torch.float64)
        for b, n in enumerate(wl.seq_lens.tolist()):
            keep = [int(t) for t in idx[b] if 0 <= t < n]
            rows = torch.stack([deq[int(wl.block_table[b, t // 16]), t % 16] for t in keep])
            q = wl.q[b].to(torch.float64)
            kk = rows[None, None].expand(1, q.shape[0], -1, -1)
            ref = torch.nn.functional.scaled_dot_product_attention(
                q[None, :, None, :], kk, kk[..., :512], scale=wl.scale)[0, :, 0].numpy()
            ref_lse = torch.logsumexp(wl.scale * (q @ rows.T), -1).numpy()
            assert _close(out[b], ref), f"sparse out vs SDPA ({kv_dtype}, b={b})"
            assert _close(lse[b], ref_lse), f"sparse lse vs logsumexp ({kv_dtype}, b={b})"


def pin_sparse_closed_forms(orc):
    """A position listed twice: out is its value row, lse its logit + ln 2; only
    skipped entries: out 0, lse -inf."""
    wl = workloads.make_workload(batch=2, num_heads=2, seq=("fixed", [20, 20]), block_size=16,
                                 seed=19)
    idx = np.array([[7, 7, -1, 25], [-1, 20, 21, -5]], np.int32)
    out, lse = orc.attend_sparse(wl.q_bits(), wl.kv_bits(), wl.block_table.numpy(),
                                 wl.seq_lens.numpy(), 16, wl.scale, idx)
    k7 = wl.kv[int(wl.block_table[0, 0]), 7].to(torch.float64)
    x7 = (wl.scale * (wl.q[0].to(torch.float64) @ k7)).numpy()
    assert (out[0] == k7[:512].numpy()[None]).all(), "repeated position: out = its value row"
    assert _close(lse[0], x7 + math.log(2)), "repeated position: lse = logit + ln 2"
    assert (out[1] == 0).all() and np.isneginf(lse[1]).all(), "no listed token: out 0, lse -inf"


def pin_sparse_split_merge(orc):
    """Cutting each list into consecutive sub-lists and merging by LSE equals the
    whole list."""
    wl = workloads.make_workload(batch=2, num_heads=3, seq=("fixed", [70, 300]), block_size=16,
                                 seed=20, topk=64, poison=True)
    args = (wl.q_bits(), wl.kv_bits(), wl.block_table.numpy(), wl.seq_lens.numpy(), 16,
            wl.scale)
    idx = wl.indices.numpy()
    full_out, full_lse = orc.attend_sparse(*args, idx)
    cuts = [0, 5, 6, 40, 64]
    parts = [orc.attend_sparse(*args, np.ascontiguousarray(idx[:, a:b]))
             for a, b in zip(cuts[:-1], cuts[1:])]
    for b in range(2):
        mo, ml = orc.lse_merge(np.stack([p[0][b] for p in parts]),
                               np.stack([p[1][b] for p in parts]))
        assert _close(mo, full_out[b]) and _close(ml, full_lse[b]), f"sparse split-merge b={b}"


def _rand_codes(rng, shape):
    """Random E4M3FN codes without the two NaN codes."""
    c = rng.integers(0, 256, size=shape, dtype=np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x3F
    return c


def _deq(codes):
    """E4M3FN codes decoded by torch (a library routine, not the oracle)."""
    return torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64)


def pin_gemm_matches_torch_matmul(orc):
    """The block-scaled projection equals torch's float64 matmul of the
    dequantised operands (decoded by torch's float8_e4m3fn, scales broadcast
    per 128-group and per 128 x 128 block)."""
    rng = np.random.default_rng(21)
    for m, n, k in ((3, 300, 384), (17, 128, 256), (1, 16, 128)):
        a = _rand_codes(rng, (m, k))
        b = _rand_codes(rng, (n, k))
        sa = rng.uniform(0.01, 2.0, size=(m, k // 128)).astype(np.float32)
        sb = rng.uniform(0.01, 2.0, size=((n + 127) // 128, k // 128)).astype(np.float32)
        c = orc.gemm_fp8_blockscale(a, sa, b, sb)
        da = _deq(a) * torch.from_numpy(np.repeat(sa, 128, axis=1)).double()
        sbe = np.repeat(np.repeat(sb, 128, axis=0)[:n], 128, axis=1)
        db = _deq(b) * torch.from_numpy(sbe).double()
        ref = (da @ db.T).numpy()
        mag = (da.abs() @ db.abs().T).numpy()
        assert np.all(np.abs(c - ref) <= 1e-12 * (1 + mag)), f"gemm vs matmul (m={m} n={n} k={k})"


def pin_gemm_closed_forms(orc):
    """One-hot activations pick one weight column exactly; scaling one block's
    weight scale scales exactly that block's contribution (linearity)."""
    rng = np.random.default_rng(22)
    n, k, k0 = 200, 384, 257
    b = _rand_codes(rng, (n, k))
    sb = rng.uniform(0.5, 2.0, size=(2, 3)).astype(np.float32)
    a = np.zeros((1, k), np.uint8)
    a[0, k0] = 0x38                                    # E4M3FN code of 1.0
    c = orc.gemm_fp8_blockscale(a, np.ones((1, 3), np.float32), b, sb)
    col = torch.from_numpy(b[:, k0].copy()).view(torch.float8_e4m3fn).double().numpy()
    want = col * sb[np.arange(n) // 128, k0 // 128].astype(np.float64)
    assert (c[0] == want).all(), "one-hot row must select the weight column exactly"
    a = _rand_codes(rng, (4, k))
    sa = rng.uniform(0.5, 2.0, size=(4, 3)).astype(np.float32)
    base = orc.gemm_fp8_blockscale(a, sa, b, sb)
    sb2 = sb.copy()
    sb2[1, 2] *= 2                                     # rows 128..199, k 256..383
    only = np.zeros_like(sa)
    only[:, 2] = sa[:, 2]
    part = orc.gemm_fp8_blockscale(a, only, b, sb)     # contribution of group 2 alone
    got = orc.gemm_fp8_blockscale(a, sa, b, sb2)
    want = base.copy()
    want[:, 128:] += part[:, 128:]
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12), "block scale must act on its block"


def pin_quant_groups(orc):
    """Group quantisation: each group's largest magnitude maps to +-448
    exactly; an all-zero group gives zero codes and scale 1e-10/448; every code is
    the nearest E4M3FN value to x / scale (ties to the even code), found by
    brute force over all codes decoded by the oracle's own decoder."""
    gen = torch.Generator().manual_seed(23)
    x = (torch.randn((5, 384), generator=gen) * torch.tensor([1e-3, 1.0, 30.0, 1e4, 0.0])[:, None])
    x = x.to(torch.bfloat16)
    x[0, 100] = 0.0
    codes, scale = orc.quant_fp8_groups(x)
    xf = x.float().numpy().reshape(5, 3, 128)
    vals = orc.e4m3_to_double(np.arange(256, dtype=np.uint8))
    finite = ~np.isnan(vals)
    for i in range(5):
        for g in range(3):
            grp = xf[i, g]
            cg = codes[i, g * 128:(g + 1) * 128]
            if np.abs(grp).max() == 0:
                # +0 and -0 keep their sign bit: codes 0x00 and 0x80
                assert (vals[cg] == 0).all() and scale[i, g] == np.float32(1e-10) / np.float32(448)
                continue
            j = int(np.argmax(np.abs(grp)))
            assert vals[cg[j]] == np.sign(grp[j]) * 448.0, "group maximum must map to +-448"
            y = np.clip((grp / scale[i, g]).astype(np.float32), -448, 448).astype(np.float64)
            for t in range(128):
                d = np.abs(vals - y[t])
                d[~finite] = np.inf
                best = np.flatnonzero(d == d.min())
                if len(best) > 1:                        # tie: the even code
                    best = best[(best & 1) == 0]
                assert vals[cg[t]] == vals[best[0]], f"code not nearest (row {i}, group {g})"


def pin_absorb(orc):
    """The per-head absorption products equal torch's float64 batched matmul;
    an identity block in W passes x through exactly."""
    gen = torch.Generator().manual_seed(24)
    for b, h, k, n in ((3, 2, 128, 512), (5, 3, 512, 128)):
        x = _bf16(torch.randn((b, h, k), generator=gen))
        w = _bf16(torch.randn((h, k, n), generator=gen) * 0.05)
        c = orc.absorb(_bits(x), _bits(w))
        ref = torch.matmul(x.double().permute(1, 0, 2), w.double()).permute(1, 0, 2).numpy()
        mag = torch.matmul(x.double().abs().permute(1, 0, 2), w.double().abs()).permute(1, 0, 2)
        assert np.all(np.abs(c - ref) <= 1e-12 * (1 + mag.numpy())), f"absorb vs matmul k={k}"
    x = _bf16(torch.randn((2, 2, 128), generator=gen))
    w = torch.zeros((2, 128, 512), dtype=torch.bfloat16)
    w[:, :, :128] = torch.eye(128, dtype=torch.bfloat16)
    c = orc.absorb(_bits(x), _bits(w))
    assert (c[:, :, :128] == x.double().numpy()).all() and (c[:, :, 128:] == 0).all(), \
        "identity block must pass x through"


PINS = [pin_e4m3_decode, pin_bf16_widen, pin_sdpa_identity_table, pin_sdpa_shuffled_pages,
        pin_closed_forms, pin_empty_request, pin_split_merge, pin_merge_closed_form,
        pin_rope_shift, pin_head_padding, pin_block_permutation, pin_batch_independence,
        pin_fp8_dequant, pin_multi_token_causal_sdpa, pin_multi_token_rows_are_single_decodes,
        pin_multi_token_split_merge, pin_sparse_all_positions_is_dense,
        pin_sparse_sdpa_on_gathered_rows, pin_sparse_closed_forms, pin_sparse_split_merge,
        pin_gemm_matches_torch_matmul, pin_gemm_closed_forms, pin_quant_groups, pin_absorb]


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--lib", required=True)
    args = ap.parse_args(argv)
    import oracle
    orc = oracle.load(args.lib)
    failed = []
    for pin in PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError) as e:
            failed.append(f"{pin.__name__}: {e}")
    for f in failed:
        print("FAIL", f)
    print(f"{len(PINS) - len(failed)}/{len(PINS)} pins hold")
    return 1 if failed else 0


if __name__ == "__main__":
    sys.exit(main())
