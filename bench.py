"""Benchmark of absorbed MLA paged-KV decode on one MI355X.

One step = one mla_decode call (split plan + attention + LSE combine) over the
whole synthetic batch, inputs already resident in HBM. Default workload: the
DeepSeek-R1 one-GPU share at 8-way tensor parallelism (batch 512, 16 heads,
seq_lens U[1024, 3072], block 32, bf16 cache), the configuration the headline
metric is quoted on.

Prints ONE JSON line: µs per call (value), the attention kernel's achieved
algorithmic HBM bandwidth against the 8 TB/s peak (roofline), and the fp64
CPU oracle timed on a bounded sample of the same workload (cpu_baseline).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E
PEAK_MFMA_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}
MALL_BYTES = 256 << 20          # memory-side cache; smaller pools are rotated
ROTATE_MIN_BYTES = 1 << 30
KERNEL_SOURCES = [os.path.join(ROOT, "mla_paged_attention_amd", "csrc", f)
                  for f in ("mla_kernels.hip", "mla_internal.h")]
PROFILES = os.path.join(ROOT, "profiles")
D_K, D_V = 576, 512


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(config: str, khash: str):
    """HBM bytes per attention launch from the committed rocprofv3 counter
    summaries (FETCH_SIZE + WRITE_SIZE, calibrated against a plain copy), or
    None if none was taken for this workload with the current kernel source."""
    if not os.path.isdir(PROFILES):
        return None
    for name in sorted(os.listdir(PROFILES)):
        if not name.endswith(".md"):
            continue
        with open(os.path.join(PROFILES, name)) as f:
            for line in f:
                if line.startswith("traffic_line:"):
                    _, cfg, h, nbytes = line.split()
                    if cfg == config and h == khash:
                        return int(nbytes)
    return None


def listed_tokens(wl) -> int:
    """Sparse decode: list entries that name a token of their request."""
    n = wl.seq_lens[:, None].long()
    idx = wl.indices.long()
    return int(((idx >= 0) & (idx < n)).sum())


def algorithmic_bytes(wl) -> int:
    """Bytes a decode call must move at least once: the cache rows of every
    token (sparse: of every listed token), q, out, lse, the block-table
    entries used (sparse: one per listed token, plus the lists) and seq_lens."""
    e_kv = 1 if wl.kv_dtype == "fp8" else 2
    b, h = wl.batch, wl.num_heads * wl.q_len   # query rows per request
    io = b * h * D_K * 2 + b * h * D_V * 2 + b * h * 4 + b * 4
    if wl.indices is not None:
        n_tok = listed_tokens(wl)
        return n_tok * D_K * e_kv + io + n_tok * 4 + wl.indices.numel() * 4
    nblk = sum((int(n) + wl.block_size - 1) // wl.block_size for n in wl.seq_lens)
    return wl.total_tokens * D_K * e_kv + io + nblk * 4


def algorithmic_flops(wl) -> int:
    """Logits (2 * 576) and P.V (2 * 512) multiply-adds per head and visible
    token: query token i of q_len sees N - q_len + 1 + i of a request's N
    (sparse: the listed tokens)."""
    if wl.indices is not None:
        return 2 * (D_K + D_V) * wl.num_heads * listed_tokens(wl)
    visible = sum(max(0, int(n) - wl.q_len + 1 + i) for n in wl.seq_lens
                  for i in range(wl.q_len))
    return 2 * (D_K + D_V) * wl.num_heads * visible


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, target_s: float):
    """Time the fp64 oracle on a bounded prefix of the requests. Returns the
    baseline record and the oracle's (out, lse) for that prefix."""
    import numpy as np

    import oracle
    orc = oracle.load()
    kw = dict(kv_fp8=wl.kv_dtype == "fp8", kv_scale=wl.kv_scale)
    if wl.indices is not None:
        idx = wl.indices.numpy()
        lens = ((idx >= 0) & (idx < wl.seq_lens.numpy()[:, None])).sum(1).astype(np.int64)
        total = int(lens.sum())

        def run(n):
            return orc.attend_sparse(wl.q_bits()[:n], wl.kv_bits(), wl.block_table.numpy()[:n],
                                     wl.seq_lens.numpy()[:n], wl.block_size, wl.scale,
                                     np.ascontiguousarray(idx[:n]), **kw)
    else:
        lens = wl.seq_lens.numpy().astype(np.int64)
        total = wl.total_tokens
        args = (wl.q_bits(), wl.kv_bits(), wl.block_table.numpy(), wl.seq_lens.numpy(),
                wl.block_size, wl.scale)

        def run(n):
            return orc.attend(*args, req=np.arange(n, dtype=np.int32), **kw)
    n_probe = min(wl.batch, 4)
    t0 = time.perf_counter()
    run(n_probe)
    probe = time.perf_counter() - t0
    per_tok = probe / max(1, lens[:n_probe].sum())
    want_tok = target_s / max(per_tok, 1e-12)
    n_req = int(np.searchsorted(np.cumsum(lens), want_tok) + 1)
    n_req = max(n_probe, min(wl.batch, n_req))
    # Runs of the sample until about target_s of work (at most 20): the
    # median run is the figure; a sample shorter than the whole batch is
    # scaled to it.
    times = []
    spent = 0.0
    while True:
        t0 = time.perf_counter()
        ref = run(n_req)
        times.append(time.perf_counter() - t0)
        spent += times[-1]
        if spent + times[-1] > target_s or len(times) == 20:
            break
    dt = statistics.median(times)
    tok = int(lens[:n_req].sum())
    full_s = dt * total / tok
    threads = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
    what = "all" if n_req == wl.batch else f"first {n_req} of {wl.batch}"
    return {"value": round(full_s * 1e6, 1), "unit": "us/call", "cores": threads,
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": (f"{what} requests ({tok} of {total} tokens, all heads), median of "
                       f"{len(times)} runs ({dt:.2f} s each, {spent:.1f} s in all)"
                       + ("" if n_req == wl.batch else ", scaled to the whole batch")),
            "tokens_per_s": round(tok / dt, 1)}, (n_req, ref)


def parity_figures(wl, out, lse, n_req: int, ref) -> dict:
    """Element-wise error of the benchmarked call's output against the oracle
    on the first n_req requests, at the stated tolerances (bf16 cache: out
    1e-2 + 1e-2|ref|, lse 1e-3; E4M3 cache: 2e-2 + 2e-2|ref| for both)."""
    import numpy as np

    ref_out, ref_lse = ref
    got_out = out[:n_req].float().cpu().double().numpy()
    got_lse = lse[:n_req].cpu().double().numpy()
    if wl.kv_dtype == "fp8":
        o_atol, o_rtol, l_atol, l_rtol = 2e-2, 2e-2, 2e-2, 2e-2
    else:
        o_atol, o_rtol, l_atol, l_rtol = 1e-2, 1e-2, 1e-3, 0.0
    err = np.abs(got_out - ref_out)
    ratio = err / (o_atol + o_rtol * np.abs(ref_out))
    fin = np.isfinite(ref_lse)
    lerr = np.where(fin, np.abs(got_lse - np.where(fin, ref_lse, 0.0)), 0.0)
    lratio = lerr / (l_atol + l_rtol * np.abs(np.where(fin, ref_lse, 0.0)))
    worst = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
    lse_pattern_ok = bool((np.isneginf(got_lse) == ~fin).all())
    return {"requests_compared": int(n_req), "elements_compared": int(err.size),
            "max_abs_err_out": float(err.max()), "max_abs_err_lse": float(lerr.max()),
            "max_err_over_bound": round(float(max(ratio.max(), lratio.max())), 4),
            "worst_out_element": {"index": [int(i) for i in worst],
                                  "gpu": float(got_out[worst]), "ref": float(ref_out[worst])},
            "tolerance": {"out": [o_atol, o_rtol], "lse": [l_atol, l_rtol]},
            "pass": bool(ratio.max() <= 1.0 and lratio.max() <= 1.0 and lse_pattern_ok
                         and np.isfinite(got_out).all())}


def calib_copy(torch, dev, nbytes: int, reps: int) -> int:
    """Plain copies (read n + write n bytes per launch) and sums (read n bytes)
    of known size: the reference for scaling FETCH_SIZE / WRITE_SIZE counters
    and the practically reachable HBM bandwidth."""
    src = torch.randn(nbytes // 4, device=dev)
    dst = torch.empty_like(src)
    res = {"calib_bytes_per_launch": nbytes, "reps": reps}
    for name, fn, moved in (("copy", lambda: dst.copy_(src), 2 * nbytes),
                            ("sum", lambda: src.sum(), nbytes)):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        res[f"{name}_us"] = round(ms * 1e3, 2)
        res[f"{name}_GBps"] = round(moved / (ms * 1e-3) / 1e9, 1)
    print(json.dumps(res), flush=True)
    return 0


def _peaks_lib():
    import ctypes

    from mla_paged_attention_amd import build as hip_build
    if not os.path.exists(hip_build.PEAKS_LIBRARY):
        raise RuntimeError(f"{hip_build.PEAKS_LIBRARY} is not built")
    lib = ctypes.CDLL(hip_build.PEAKS_LIBRARY)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.peaks_stream_lds.argtypes = [vp, i64, i32, i32, i32, vp]
    lib.peaks_stream_perm.argtypes = [vp, i64, i64, i32, i32, vp]
    lib.peaks_gather_rows.argtypes = [vp, i64, i32, i32, i32, vp]
    lib.peaks_read.argtypes = [vp, i64, i32, vp, vp]
    lib.peaks_mfma.argtypes = [i32, i32, i32, vp, vp]
    for f in (lib.peaks_stream_lds, lib.peaks_stream_perm, lib.peaks_gather_rows, lib.peaks_read,
              lib.peaks_mfma):
        f.restype = i32
    return lib


def _median_launch_us(torch, launch, reps: int) -> float:
    """Median duration of `reps` back-to-back launches, each between events."""
    stream = torch.cuda.current_stream()
    launch()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for e0, e1 in ev:
        e0.record(stream)
        launch()
        e1.record(stream)
    torch.cuda.synchronize()
    return statistics.median(e0.elapsed_time(e1) * 1e3 for e0, e1 in ev)


TILE_BYTES = 36864          # one ring stage of the attention kernels


PATTERN_KERNELS = {
    "tiles": "the same ring over 36 KB tiles in scattered order (a paged cache's blocks)",
    "rows1152": "the same ring gathering single 1152-byte rows at hashed positions",
    "rows576": "the same ring gathering single 576-byte rows at hashed positions",
}


def measure_peaks(torch, dev, which=("hbm", "bf16", "fp8"), full: bool = False,
                  reps: int = 10, patterns=()) -> dict:
    """What this GPU delivers, measured by libmla_peaks.so's calibration
    kernels (HBM: 2 GiB streamed through LDS as 36 KB direct-to-LDS tiles
    with the non-temporal bit, one workgroup per CU and two tiles in flight
    as in the attention ring; with `patterns` (or `full`) the same ring over
    scattered tiles and over gathered single rows, the access patterns of the
    paged and the sparse decode; matrix cores: dense loops of the bf16
    16x16x32 and scaled E4M3 16x16x128 ops on every SIMD)."""
    import ctypes
    lib = _peaks_lib()
    h = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    res = {}
    if "hbm" in which:
        nbytes = 2 << 30
        buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        ntiles = nbytes // TILE_BYTES
        moved = ntiles * TILE_BYTES
        shapes = [(256, 2, 1)]
        if full:
            shapes += [(256, 1, 1), (256, 3, 1), (1024, 2, 1), (2048, 2, 1), (256, 2, 0),
                       (1024, 2, 0)]
        for grid, inflight, nt in shapes:
            def launch(g=grid, k=inflight, n=nt):
                assert lib.peaks_stream_lds(ctypes.c_void_p(buf.data_ptr()), ntiles, g, k, n,
                                            h) == 0
            us = _median_launch_us(torch, launch, reps)
            key = f"stream_lds_grid{grid}_inflight{inflight}_{'nt' if nt else 'plain'}"
            res[key] = round(moved / (us * 1e-6) / 1e9, 1)
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
        for grid in ((1024, 4096) if full else (4096,)):
            def launch_read(g=grid):
                assert lib.peaks_read(ctypes.c_void_p(buf.data_ptr()), nbytes // 16, g,
                                      ctypes.c_void_p(sink.data_ptr()), h) == 0
            us = _median_launch_us(torch, launch_read, reps)
            res[f"read_grid{grid}"] = round(nbytes / (us * 1e-6) / 1e9, 1)
        res["hbm_GBps"] = res["stream_lds_grid256_inflight2_nt"]
        grid = 256
        per_wg = ntiles // grid
        pattern_bytes = grid * per_wg * TILE_BYTES
        for pat in (tuple(PATTERN_KERNELS) if full else tuple(patterns)):
            if pat == "tiles":
                stride = 7919                      # prime, coprime to the tile count
                while math.gcd(stride, ntiles) != 1:
                    stride += 2

                def launch_pat(st=stride):
                    assert lib.peaks_stream_perm(ctypes.c_void_p(buf.data_ptr()), ntiles, st, grid,
                                                 per_wg, h) == 0
            else:
                row_bytes = int(pat[4:])

                def launch_pat(rb=row_bytes):
                    assert lib.peaks_gather_rows(ctypes.c_void_p(buf.data_ptr()), nbytes // rb, rb,
                                                 grid, per_wg, h) == 0
            us = _median_launch_us(torch, launch_pat, reps)
            res[f"pattern_{pat}_GBps"] = round(pattern_bytes / (us * 1e-6) / 1e9, 1)
        del buf
    for name, fp8, iters, per_op in (("bf16", 0, 8192, 16384), ("fp8", 1, 4096, 65536)):
        if name not in which:
            continue
        grid = 1024   # four workgroups of four waves per CU: four waves per SIMD
        sink = torch.zeros(grid, dtype=torch.float32, device=dev)

        def launch_mfma(f=fp8, it=iters):
            assert lib.peaks_mfma(f, grid, it, ctypes.c_void_p(sink.data_ptr()), h) == 0
        us = _median_launch_us(torch, launch_mfma, reps)
        flops = grid * 4 * 4 * iters * per_op
        res[f"mfma_{name}_TFLOPs"] = round(flops / (us * 1e-6) / 1e12, 1)
    return res


def bench_peaks(torch, dev) -> int:
    res = measure_peaks(torch, dev, full=True)
    res.update({"spec_hbm_GBps": PEAK_HBM_GBPS, "spec_mfma_TFLOPs": PEAK_MFMA_TFLOPS,
                "kernel_source": "mla_paged_attention_amd/csrc/peaks.hip"})
    print(json.dumps(res), flush=True)
    return 0


def time_queued(torch, fn, steps: int, warmup: int):
    """GPU time of calls fn(i) that are shorter than their own host-side
    launch cost. The stream is held by a bounded spin kernel while the host
    queues the calls, so they run back to back on the GPU. Returns (mean us
    per call over `steps` calls between one event pair, sorted per-call us
    from a second pass with an event pair around each call; those include the
    events' own cost, about 2 us)."""
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        fn(i)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    torch.cuda._sleep(100_000 * steps)  # clock ticks; covers the host's queueing
    e0.record(stream)
    for i in range(steps):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    mean = e0.elapsed_time(e1) * 1e3 / steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * steps)]
    torch.cuda._sleep(100_000 * steps)
    for i in range(steps):
        ev[2 * i].record(stream)
        fn(i)
        ev[2 * i + 1].record(stream)
    torch.cuda.synchronize()
    return mean, sorted(ev[2 * i].elapsed_time(ev[2 * i + 1]) * 1e3 for i in range(steps))


def bench_gemm(torch, mla, workloads, dev, m: int, n: int, k: int, steps: int, warmup: int) -> int:
    """Block-scaled E4M3 projection at decode batch m (DeepSeek-R1 fused q/kv
    down-projection by default: n = 2112, k = 7168): one JSON line with us per
    GEMM and its roofline. Weights rotate across copies of >= 1 GB in total so
    that HBM, not the memory-side cache, is measured."""
    a, sa, b, sb = workloads.make_gemm(m, n, k, seed=11)
    copies = max(2, math.ceil(ROTATE_MIN_BYTES / (n * k)))
    bs = [(b.to(dev), sb.to(dev)) for _ in range(copies)]
    a, sa = a.to(dev), sa.to(dev)
    out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    avg, us = time_queued(torch,
                          lambda i: mla.gemm_fp8_blockscale(a, sa, *bs[i % copies], out=out),
                          steps, warmup)
    alg_bytes = m * k + n * k + 4 * m * (k // 128) + 4 * ((n + 127) // 128) * (k // 128) + 2 * m * n
    flops = 2 * m * n * k
    t_hbm = alg_bytes / (PEAK_HBM_GBPS * 1e9)
    t_mfma = flops / (PEAK_MFMA_TFLOPS["fp8"] * 1e12)
    gbps = alg_bytes / (avg * 1e-6) / 1e9
    tflops = flops / (avg * 1e-6) / 1e12
    if t_mfma > t_hbm:
        roof = {"bound": "mfma", "achieved": round(tflops, 1), "peak": PEAK_MFMA_TFLOPS["fp8"],
                "unit": "TFLOP/s", "frac": round(tflops / PEAK_MFMA_TFLOPS["fp8"], 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS,
                "unit": "GB/s", "frac": round(gbps / PEAK_HBM_GBPS, 4)}
    if m <= 16 and k <= 8192:
        kname = f"mla::gemm_fp8_lds_kernel<{4 if m <= 4 else 0}>"
    else:
        kname = "mla::gemm_fp8_kernel"
    roof.update({"kernel": kname, "algorithmic_bytes_per_launch": alg_bytes,
                 "algorithmic_flops_per_launch": flops, "traffic": None})
    print(json.dumps({
        "metric": "block-fp8 projection us/call at decode batch", "value": round(avg, 2),
        "unit": "us/call", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "higher_is_better": False, "dtype": "fp8", "data": "synthetic",
        "config": {"workload": f"gemm-fp8-m{m}", "m": m, "n": n, "k": k,
                   "scales": "activation 1x128, weight 128x128"},
        "us_p10_p90_with_events": [round(us[len(us) // 10], 2),
                                   round(us[(9 * len(us)) // 10], 2)],
        "roofline": roof}), flush=True)
    return 0


def bench_absorb(torch, mla, workloads, dev, batch: int, heads: int, steps: int,
                 warmup: int) -> int:
    """Per-head absorption products at decode batch `batch` and `heads` heads:
    one JSON line with us per call of mla_absorb_q and mla_absorb_out and the
    roofline of the first. Weights rotate across copies of >= 1 GB in total
    so that their reads come from HBM."""
    q_nope, q_rope, w_uk, o_lat, w_uv = workloads.make_absorb(batch, heads, seed=12)
    copies = max(2, math.ceil(ROTATE_MIN_BYTES / (2 * w_uk.numel())))
    wk = [w_uk.to(dev) for _ in range(copies)]
    wv = [w_uv.to(dev) for _ in range(copies)]
    q_nope, q_rope, o_lat = q_nope.to(dev), q_rope.to(dev), o_lat.to(dev)
    q = torch.empty((batch, heads, 576), dtype=torch.bfloat16, device=dev)
    o = torch.empty((batch, heads, 128), dtype=torch.bfloat16, device=dev)
    avg_q, us_q = time_queued(
        torch, lambda i: mla.absorb_q(q_nope, wk[i % copies], q_rope, out=q), steps, warmup)
    avg_o, _ = time_queued(
        torch, lambda i: mla.absorb_out(o_lat, wv[i % copies], out=o), steps, warmup)
    # Algorithmic bytes of mla_absorb_q: q_nope + W_UK + q_rope read, q written.
    bytes_q = 2 * (batch * heads * 128 + heads * 128 * 512 + batch * heads * 64
                   + batch * heads * 576)
    bytes_o = 2 * (batch * heads * 512 + heads * 512 * 128 + batch * heads * 128)
    flops = 2 * batch * heads * 128 * 512
    gbps = bytes_q / (avg_q * 1e-6) / 1e9
    tflops = flops / (avg_q * 1e-6) / 1e12
    if flops / (PEAK_MFMA_TFLOPS["bf16"] * 1e12) > bytes_q / (PEAK_HBM_GBPS * 1e9):
        roof = {"bound": "mfma", "achieved": round(tflops, 1), "peak": PEAK_MFMA_TFLOPS["bf16"],
                "unit": "TFLOP/s", "frac": round(tflops / PEAK_MFMA_TFLOPS["bf16"], 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS,
                "unit": "GB/s", "frac": round(gbps / PEAK_HBM_GBPS, 4)}
    roof.update({"kernel": "mla::absorb_q_kernel",
                 "algorithmic_bytes_per_launch": bytes_q, "algorithmic_flops_per_launch": flops,
                 "traffic": None})
    print(json.dumps({
        "metric": "absorbed query projection us/call at decode batch", "value": round(avg_q, 2),
        "unit": "us/call", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "higher_is_better": False, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"absorb-b{batch}-h{heads}", "batch": batch, "heads": heads},
        "us_p10_p90_with_events": [round(us_q[len(us_q) // 10], 2),
                                   round(us_q[(9 * len(us_q)) // 10], 2)],
        "absorb_out": {"us": round(avg_o, 2), "algorithmic_bytes_per_launch": bytes_o,
                       "GB/s": round(bytes_o / (avg_o * 1e-6) / 1e9, 1)},
        "roofline": roof}), flush=True)
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="r1tp8")
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--q-len", type=int, default=1,
                    help="query tokens per request (speculative decoding, causal)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="also time the call replayed from a captured HIP graph")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-measured-peak", action="store_true",
                    help="skip the calibration kernels (measured peak beside the spec peak)")
    ap.add_argument("--gemm", type=int, default=0, metavar="M",
                    help="instead of decoding, time the block-scaled E4M3 projection at "
                         "decode batch M (n = 2112, k = 7168 unless --gemm-nk)")
    ap.add_argument("--gemm-nk", type=int, nargs=2, default=(2112, 7168), metavar=("N", "K"))
    ap.add_argument("--absorb", type=int, default=0, metavar="B",
                    help="instead of decoding, time the per-head absorption products at "
                         "decode batch B (heads from --absorb-heads)")
    ap.add_argument("--absorb-heads", type=int, default=16)
    ap.add_argument("--peaks", action="store_true",
                    help="instead of decoding, measure this GPU's HBM stream and matrix-core "
                         "peaks with the calibration kernels (libmla_peaks.so)")
    ap.add_argument("--calib-copy", type=int, default=0, metavar="MIB",
                    help="instead of decoding, run plain device copies and reductions of "
                         "MIB MiB (HBM counter calibration and practical bandwidth)")
    args = ap.parse_args(argv)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; the decode path "
                                   "has no multi-GPU mode (heads shard across GPUs with no "
                                   "exchange inside attention)", "n_gpus": args.gpus}))
        return 2

    import torch

    import mla_paged_attention_amd as mla
    import workloads

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        return 1
    dev = torch.device("cuda:0")
    if args.calib_copy:
        return calib_copy(torch, dev, args.calib_copy << 20, max(args.steps, 1))
    if args.peaks:
        return bench_peaks(torch, dev)
    if args.absorb:
        return bench_absorb(torch, mla, workloads, dev, args.absorb, args.absorb_heads,
                            args.steps, args.warmup)
    if args.gemm:
        return bench_gemm(torch, mla, workloads, dev, args.gemm, *args.gemm_nk, args.steps,
                          args.warmup)
    mla.library()  # fail loudly now if the HIP library is missing

    label = args.config if args.q_len == 1 else f"{args.config}-q{args.q_len}"
    log(f"generating workload {label}")
    wl = workloads.make_config(args.config, q_len=args.q_len)
    cfg = workloads.CONFIGS[args.config]
    pool_bytes = wl.kv.numel() * wl.kv.element_size()
    copies = 1 if pool_bytes >= 2 * MALL_BYTES else max(4, math.ceil(ROTATE_MIN_BYTES / pool_bytes))
    q, bt, sl = wl.q.to(dev), wl.block_table.to(dev), wl.seq_lens.to(dev)
    kvs = [wl.kv.to(dev) for _ in range(copies)]
    out = torch.empty(tuple(wl.q.shape[:-1]) + (D_V,), dtype=torch.bfloat16, device=dev)
    lse = torch.empty(tuple(wl.q.shape[:-1]), dtype=torch.float32, device=dev)
    if wl.indices is not None:
        if args.q_len != 1:
            raise SystemExit("sparse workloads take one query token per request")
        nbytes = mla.get_workspace_size_sparse(wl.batch, wl.num_heads, wl.indices.shape[1],
                                               args.num_splits, 0)
        idx = wl.indices.to(dev)
    else:
        nbytes = mla.get_workspace_size(wl.batch, wl.num_heads, wl.max_blocks * wl.block_size,
                                        args.num_splits, 0, q_len=wl.q_len)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    log(f"tokens={wl.total_tokens} pool={pool_bytes / 2**20:.0f} MiB copies={copies} "
        f"workspace={nbytes / 2**20:.1f} MiB")

    def call(i, events=None, on=stream):
        if wl.indices is not None:
            mla.decode_sparse(q, kvs[i % copies], bt, sl, idx, scale=wl.scale,
                              num_splits=args.num_splits, kv_scale=wl.kv_scale, out=out, lse=lse,
                              workspace=ws, stream=on, events=events)
            return
        mla.decode(q, kvs[i % copies], bt, sl, scale=wl.scale, num_splits=args.num_splits,
                   kv_scale=wl.kv_scale, out=out, lse=lse, workspace=ws, stream=on,
                   events=events)

    mp = None
    if not args.no_measured_peak:
        # The HBM calibration (memory-bound, about 50 ms of streaming) runs
        # before the warmup: it is measurement work of its own, and it brings
        # the GPU out of the idle state of the host-side set-up before the
        # timed calls. The matrix-core loops, which heat the chip, run after
        # the timed regions.
        log("measuring this GPU's HBM peak")
        pattern = ("rows576" if wl.kv_dtype == "fp8" else "rows1152") if wl.indices is not None \
            else "tiles"
        mp = measure_peaks(torch, dev, which=("hbm",), reps=150, patterns=(pattern,))
    for i in range(args.warmup):
        call(i)
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} calls)")

    def timed_run():
        """K plain calls back to back between one event pair: us per call."""
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for i in range(args.steps):
            call(i)
        stop.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(stop) / args.steps

    # Timed region: K plain calls (the headline value).
    t0 = time.perf_counter()
    ms_per_step = timed_run()
    wall = time.perf_counter() - t0
    log(f"timed {args.steps} calls: {ms_per_step * 1e3:.1f} us/call (wall {wall * 1e3 / args.steps:.1f})")

    def hold(n_calls):
        # A bounded spin kernel holds the stream while the host queues the
        # calls, so that they run back to back on the GPU (no idle gaps in
        # which the clock could recover between calls).
        torch.cuda._sleep(int(200_000 * n_calls))

    # Per-call spread: an event pair around each call, calls back to back.
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    hold(args.steps)
    for i in range(args.steps):
        ev[i][0].record(stream)
        call(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    call_us = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in ev)

    # Kernel durations: HIP events around each kernel (same stream), the
    # calls again queued back to back.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for row in evs:
        for e in row:
            e.record(stream)  # create the underlying HIP events
    torch.cuda.synchronize()
    hold(args.steps)
    for i in range(args.steps):
        call(i, events=evs[i])
    torch.cuda.synchronize()
    attn_ms = [r[1].elapsed_time(r[2]) for r in evs]
    plan_ms = [r[0].elapsed_time(r[1]) for r in evs]
    comb_ms = [r[2].elapsed_time(r[3]) for r in evs]
    tot_ms = [r[0].elapsed_time(r[3]) for r in evs]
    attn_avg = statistics.fmean(attn_ms)
    log(f"attention kernel {attn_avg * 1e3:.1f} us avg, before it {statistics.fmean(plan_ms) * 1e3:.1f},"
        f" combine {statistics.fmean(comb_ms) * 1e3:.1f}")

    # Second timed run of the same K plain calls, after the other regions.
    ms_second = timed_run()
    log(f"second timed run: {ms_second * 1e3:.1f} us/call")

    if mp is not None:
        log("measuring this GPU's matrix-core peaks")
        mp.update(measure_peaks(torch, dev, which=("bf16", "fp8")))

    graph_us = None
    if args.graph:
        # Optional: one HIP graph holding `copies` calls (one per cache copy),
        # replayed back to back.
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(copies):
                call(i, on=None)  # the capture stream
        torch.cuda.synchronize()
        reps = max(1, args.steps // copies)
        graph.replay()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        g0.record(stream)
        for _ in range(reps):
            graph.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        graph_us = round(g0.elapsed_time(g1) * 1e3 / (reps * copies), 2)
        log(f"graph replays: {graph_us} us/call")

    def pct(v, f):
        return round(v[min(len(v) - 1, int(f * len(v)))], 2)

    alg_bytes = algorithmic_bytes(wl)
    alg_flops = algorithmic_flops(wl)
    achieved = alg_bytes / (attn_avg * 1e-3) / 1e9
    mfma_peak = PEAK_MFMA_TFLOPS["fp8" if wl.kv_dtype == "fp8" else "bf16"]
    traffic = measured_traffic(label, kernel_source_hash())
    sparse = int(wl.indices is not None)
    if wl.kv_dtype == "fp8":
        kernel_name = f"mla::attn_mh_kernel<1, {sparse}>"
    elif wl.num_heads * wl.q_len <= 16 and not sparse:
        kernel_name = "mla::attn_ws_kernel"
    else:
        kernel_name = f"mla::attn_mh_kernel<0, {sparse}>"
    # The roof that bounds the call: whichever of HBM bytes and matrix-core
    # flops needs more time at peak.
    t_hbm = alg_bytes / (PEAK_HBM_GBPS * 1e9)
    t_mfma = alg_flops / (mfma_peak * 1e12)
    achieved_tflops = alg_flops / (attn_avg * 1e-3) / 1e12
    t_floor = max(t_hbm, t_mfma)
    if t_mfma > t_hbm:
        roofline = {"bound": "mfma", "achieved": round(achieved_tflops, 1), "peak": mfma_peak,
                    "unit": "TFLOP/s", "frac": round(achieved_tflops / mfma_peak, 4)}
    else:
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS,
                    "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4)}
    if mp is not None:
        measured = mp["hbm_GBps"] if roofline["bound"] == "hbm" else \
            mp[f"mfma_{'fp8' if wl.kv_dtype == 'fp8' else 'bf16'}_TFLOPs"]
        which = ("bf16",) if wl.kv_dtype != "fp8" else ("fp8",)
        roofline["measured_peak"] = measured
        roofline["frac_of_measured_peak"] = round(roofline["achieved"] / measured, 4)
        roofline["measured_peak_kernel"] = (
            "2 GiB through LDS in 36 KB direct-to-LDS tiles, non-temporal, 256 workgroups, "
            "2 tiles in flight" if roofline["bound"] == "hbm" else
            f"dense {which[0]} matrix-op loop, 4 waves per SIMD")
        pat_keys = [k for k in mp if k.startswith("pattern_")]
        if roofline["bound"] == "hbm" and pat_keys:
            pat = pat_keys[0][len("pattern_"):-len("_GBps")]
            roofline["pattern_peak"] = mp[pat_keys[0]]
            roofline["frac_of_pattern_peak"] = round(roofline["achieved"] / mp[pat_keys[0]], 4)
            roofline["pattern_peak_kernel"] = PATTERN_KERNELS[pat]
    roofline.update({
        "traffic": traffic, "kernel": kernel_name,
        "kernel_us_avg": round(attn_avg * 1e3, 2),
        "timing": "attention kernel between HIP events, calls queued back to back",
        "hbm_time_us_at_peak": round(t_hbm * 1e6, 2),
        "mfma_time_us_at_peak": round(t_mfma * 1e6, 2),
        "algorithmic_bytes_per_launch": alg_bytes,
        "algorithmic_flops_per_launch": alg_flops,
        "hbm_frac": round(achieved / PEAK_HBM_GBPS, 4),
        "mfma_frac": round(achieved_tflops / mfma_peak, 4),
        # The whole call (plan, attention and combine) against the same floor.
        "call_frac": round(t_floor / (ms_per_step * 1e-3), 4)})
    result = {
        "metric": "MLA decode us/call + achieved HBM GB/s & MFMA % at bs=512, 16 heads",
        "value": round(ms_per_step * 1e3, 2),
        "unit": "us/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8" if wl.kv_dtype == "fp8" else "bf16",
        "data": "synthetic",
        "config": {"workload": label, "batch": wl.batch, "num_heads": wl.num_heads,
                   "q_len": wl.q_len,
                   "topk": None if wl.indices is None else wl.indices.shape[1],
                   "seq_lens": list(cfg["seq"]) if cfg["seq"][0] != "fixed" else
                   sorted(set(cfg["seq"][1])), "total_tokens": wl.total_tokens,
                   "block_size": wl.block_size, "kv_dtype": wl.kv_dtype,
                   "num_splits": args.num_splits or "auto", "parallelism": "single-gpu",
                   "kv_pool_copies": copies},
        "tokens_per_s": round((wl.total_tokens if wl.indices is None else listed_tokens(wl))
                              / (ms_per_step * 1e-3), 1),
        "hbm_GBps_algorithmic": round(alg_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "mfma_pct": round(100 * alg_flops / (ms_per_step * 1e-3) / 1e12 / mfma_peak, 2),
        "call_us": {"first_run": round(ms_per_step * 1e3, 2),
                    "second_run": round(ms_second * 1e3, 2),
                    "median_with_events": pct(call_us, 0.5),
                    "p10_p90_with_events": [pct(call_us, 0.1), pct(call_us, 0.9)]},
        # before_attention: from the call's first event to the attention
        # launch, i.e. the plan kernel or the sparse prepass where one runs;
        # with the plan worked out inside the attention kernel only the two
        # event records (a few us).
        "kernels_us": {"before_attention": round(statistics.fmean(plan_ms) * 1e3, 2),
                       "attention": round(attn_avg * 1e3, 2),
                       "combine": round(statistics.fmean(comb_ms) * 1e3, 2),
                       "call_with_events": round(statistics.fmean(tot_ms) * 1e3, 2),
                       "attention_median": pct(sorted(x * 1e3 for x in attn_ms), 0.5),
                       "attention_p10_p90": [pct(sorted(x * 1e3 for x in attn_ms), 0.1),
                                             pct(sorted(x * 1e3 for x in attn_ms), 0.9)]},
        "roofline": roofline,
        "measured_peaks": mp,
        "cpu_baseline": None,
        "parity": None,
    }
    if graph_us is not None:
        result["graph_us_per_call"] = graph_us
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on a sample")
        base, (n_req, ref) = cpu_baseline(wl, args.cpu_seconds)
        result["cpu_baseline"] = base
        result["parity"] = parity_figures(wl, out, lse, n_req, ref)
        log(f"parity on {n_req} requests: max err/bound {result['parity']['max_err_over_bound']}")
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
