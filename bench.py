"""Throughput of the exact tiled attention path on one MI355X.

One step = the whole hot path on one batch of the GQA training workload
(B=2, Hq=32, Hkv=8, N=8192, d=128, causal, bf16): forward (fa_fwd) then the
recompute backward (fa_bwd_stage 0, 1 = dQ with the row statistics D, dK/dV), with inputs
resident in HBM. FLOPs per step follow the method's accounting: 4*B*Hq*Nq*Nk*d for
the forward, 2.5x that for the backward, halved for causal.

Prints one JSON line. Besides the headline value it carries:
  roofline      the dominant kernel's algorithmic FLOP/s (HIP events on the launch
                stream) against the bf16 dense MFMA peak, plus its HBM traffic when a
                counter summary for the current kernel source is in profiles/, and
                the matrix-core rate measured on this GPU (fa_mfma_probe, zeros and
                normal-like bf16 operands) with the kernel's fraction of the latter;
  cpu_baseline  the float64 oracle on this host, timed on a bounded sample;
  phases        per-kernel average milliseconds over the timed steps;
  median_ms, min_ms, step_stats
                the step and each kernel timed one by one over --stat-steps (50)
                further steps: mean, median and minimum;
  extra         forward/decode throughput of the other workloads (50 calls each, an
                event pair per call: mean, median, minimum).

Modes: default; --profile (no oracle/extras, a known-size copy first, for rocprofv3
counter runs that calibrate FETCH_SIZE/WRITE_SIZE; after the step, short runs of the
matrix-core probe, the d=64 forward and both decode shapes).
"""
import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd/bwd TFLOP/s at 1 GPU and % of bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 dense bf16 flop/clk/CU
PEAK_FP8_TFLOPS = 5033.2    # 256 CU x 2.4 GHz x 8192 dense fp8 flop/clk/CU
PEAK_HBM_GBS = 8000.0
WORKLOAD = "c5_bf16_causal_gqa_B2Hq32Hkv8N8192d128"
KERNEL_SOURCES = {
    "fwd_pp_kernel": ["fwd_pp.h", "fwd_bf16.h", "fwd_bf16.hip", "common.h"],
    "bwd_dkdv_kernel": ["bwd_dkdv.h", "bwd_dkdv_d128.hip", "bwd.hip", "common.h"],
    "bwd_dq_kernel": ["bwd_dq.h", "bwd_dq_small.hip", "bwd.hip", "bwd_dkdv.h", "common.h"],
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def fwd_flops(B, Hq, Nq, Nk, d, causal):
    f = 4.0 * B * Hq * Nq * Nk * d
    return f / 2 if (causal and Nq == Nk) else f


def source_sha(kernel):
    """Hash of the kernel's sources and of the build script (its per-file compiler
    options change the binary too)."""
    h = hashlib.sha256()
    with open(os.path.join(ROOT, "exact_tiled_attention_36_amd", "build.py"), "rb") as fh:
        h.update(fh.read())
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "exact_tiled_attention_36_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(kernel, workload):
    """Counter-derived HBM bytes per launch from profiles/counters_*.txt, or None when
    no summary matches the current kernel source."""
    pdir = os.path.join(ROOT, "profiles")
    if not os.path.isdir(pdir):
        return None
    want = source_sha(kernel)
    for fn in sorted(os.listdir(pdir)):
        if not fn.startswith("counters_") or not fn.endswith(".txt"):
            continue
        for line in open(os.path.join(pdir, fn)):
            if not line.startswith("TRAFFIC "):
                continue
            kv = dict(re.findall(r"(\w+)=(\S+)", line))
            if kv.get("kernel") == kernel and kv.get("workload") == workload \
                    and kv.get("source_sha") == want:
                return float(kv["hbm_bytes_per_launch"])
    return None


class Timer:
    """HIP events recorded on the stream the kernels are launched on."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream
        self.pairs = {}

    def mark(self, name, fn):
        t = self.torch
        a, b = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        a.record(self.stream)
        fn()
        b.record(self.stream)
        self.pairs.setdefault(name, []).append((a, b))

    def avg_ms(self):
        return {k: sum(a.elapsed_time(b) for a, b in v) / len(v) for k, v in self.pairs.items()}

    def stats(self):
        return {k: summarize([a.elapsed_time(b) for a, b in v]) for k, v in self.pairs.items()}


def cpu_baseline(inp, min_seconds=10.0):
    """The float64 oracle, as written, on a bounded sample of the workload: whole
    (batch 0, kv-head) groups -- every query head of the group, forward and backward
    over the full sequence -- added one group at a time until at least `min_seconds`
    of CPU work. Reported in the same FLOP accounting as the GPU value."""
    from oracle import attention as A
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = None
    cores = len(os.sched_getaffinity(0))
    g = inp.Hq // inp.Hkv
    qa, ka, va, da = (inp.as_f64(n) for n in ("q", "k", "v", "do"))
    dt, groups = 0.0, 0
    while dt < min_seconds and groups < inp.Hkv:
        hs = slice(groups * g, (groups + 1) * g)
        q, do = qa[:1, hs], da[:1, hs]
        k, v = ka[:1, groups:groups + 1], va[:1, groups:groups + 1]
        t0 = time.perf_counter()
        A.forward(q, k, v, inp.scale, inp.causal)
        A.backward(q, k, v, do, inp.scale, inp.causal)
        dt += time.perf_counter() - t0
        groups += 1
    fl = 3.5 * fwd_flops(1, groups * g, inp.Nq, inp.Nk, inp.d, inp.causal)
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": threads or cores,
            "host_cpus": cores, "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"batch 0, {groups} kv-head group(s) = {groups * g} query heads of "
                      f"{WORKLOAD}: float64 forward + backward over all {inp.Nq} rows, "
                      "S and P materialised"}


def warm(torch, call, warm_ms=50.0, min_calls=10):
    """Warm-up calls until at least warm_ms of GPU time has passed and at least
    min_calls calls were made, so that short kernels are timed at the clock a sustained
    run reaches."""
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    spent, n = 0.0, 0
    while n < min_calls or spent < warm_ms:
        e0.record(st)
        call()
        e1.record(st)
        torch.cuda.synchronize()
        spent += e0.elapsed_time(e1)
        n += 1


def summarize(times):
    """mean, median and min of a list of milliseconds."""
    import statistics
    return {"mean_ms": round(sum(times) / len(times), 4),
            "median_ms": round(statistics.median(times), 4),
            "min_ms": round(min(times), 4), "calls": len(times)}


def timed_stats(torch, call, iters=50, warm_ms=50.0):
    """Per-call milliseconds of iters calls issued back to back on the current stream
    (one pair of HIP events around each call), after warm-up; returns mean, median and
    min."""
    warm(torch, call, warm_ms)
    st = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(iters)]
    for a, b in ev:
        a.record(st)
        call()
        b.record(st)
    torch.cuda.synchronize()
    return summarize([a.elapsed_time(b) for a, b in ev])


def timed_ms(torch, call, iters, warm_ms=50.0):
    """Average milliseconds per call over iters back-to-back calls on the current
    stream (one event pair around all of them), after warm-up."""
    warm(torch, call, warm_ms, min_calls=3)
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(iters):
        call()
    e1.record(st)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters


def with_stats(rec, st, flops=None):
    """Fold timed_stats() output into a result record: ms is the mean; median and min
    are kept beside it (TFLOP/s from the mean)."""
    rec["ms"] = st["mean_ms"]
    rec["median_ms"] = st["median_ms"]
    rec["min_ms"] = st["min_ms"]
    rec["calls"] = st["calls"]
    if flops is not None:
        rec["tflops"] = round(flops / st["mean_ms"] / 1e9, 1)
        rec["tflops_at_median"] = round(flops / st["median_ms"] / 1e9, 1)
        rec["pct_bf16_peak"] = round(flops / st["mean_ms"] / 1e9 / PEAK_BF16_TFLOPS * 100, 2)
    return rec


def mfma_ceiling(torch, fa, blocks=4096, iters=400, reps=5):
    """Measured matrix-core rate (fa_mfma_probe): bf16 32x32x16 products on register
    operands that are zeros or normal-like bf16, in TFLOP/s. The chip's clock under
    matrix load depends on the operand bits, so the normal-like figure is the ceiling
    a dense bf16 product on this workload's data can reach on this GPU."""
    res = {}
    out = torch.empty(blocks * 256, device="cuda", dtype=torch.float32)
    for kind in ("zeros", "normal_bf16"):
        flop = [0.0]

        def call():
            flop[0], _ = fa.mfma_probe(blocks, iters, kind, out=out)
        ms = timed_ms(torch, call, reps)
        res[kind] = round(flop[0] / ms / 1e9, 1)
    del out
    return res


def extras(torch, fa, iters=50):
    """Forward throughput on the other workloads, decode in GB/s (seeded torch.randn);
    each timing is iters calls with an event pair per call (mean, median, min)."""
    from exact_tiled_attention_36_amd import synth
    out = {}
    g = torch.Generator(device="cuda")
    g.manual_seed(1234)
    for name in ("c2_bf16_B2H16N1024d64", "c3a_bf16_causal_B4H32N4096d128",
                 "c3b_bf16_causal_B2H16N4096d256", "c4a_bf16_causal_B1H8N32768d128",
                 "c4b_bf16_decode_B8H8Nq1Nk32768d128"):
        w = synth.WORKLOADS[name]
        B, Hq, Hkv, Nq, Nk, d, causal = (w[x] for x in ("B", "Hq", "Hkv", "Nq", "Nk", "d", "causal"))
        q = torch.randn(B, Hq, Nq, d, device="cuda", dtype=torch.bfloat16, generator=g)
        k = torch.randn(B, Hkv, Nk, d, device="cuda", dtype=torch.bfloat16, generator=g)
        v = torch.randn(B, Hkv, Nk, d, device="cuda", dtype=torch.bfloat16, generator=g)
        decode = Nq == 1
        o = torch.empty_like(q)
        lse = torch.empty(B, Hq, Nq, device="cuda", dtype=torch.float32)
        if decode:
            ws = torch.empty(fa.splitkv_workspace_bytes(B, Hq, Hkv, Nq, Nk, d), device="cuda",
                             dtype=torch.uint8)
            call = lambda: fa.fwd_splitkv(q, k, v, causal=causal, out=o, lse=lse, workspace=ws)
        else:
            call = lambda: fa.fwd(q, k, v, causal=causal, out=o, lse=lse)
        fl = fwd_flops(B, Hq, Nq, Nk, d, causal)
        rec = with_stats({}, timed_stats(torch, call, iters), fl)
        ms = rec["ms"]
        if decode:
            nbytes = 2 * (q.numel() + k.numel() + v.numel() + o.numel()) + 4 * lse.numel()
            rec["gbs"] = round(nbytes / ms / 1e6, 1)
            rec["pct_hbm_peak"] = round(nbytes / ms / 1e6 / PEAK_HBM_GBS * 100, 2)
            rec["kernel"] = "fa_fwd_splitkv (chunk + merge)"
        out[name] = rec
        del q, k, v, o, lse
        torch.cuda.empty_cache()
    out["c3b_bf16_causal_B2H16N4096d256_backward"] = backward_d256(torch, fa, g, iters)
    out["c2_bf16_B2H16N1024d64_rotated"] = rotated_small(torch, fa, g)
    out["decode_gqa_B16Hq32Hkv4Nq1Nk8192d128"] = gqa_decode(torch, fa, g, iters)
    out["v1_vs_v2"] = version_ablation(torch, fa, g)
    out["fp8_forward"] = fp8_forward(torch, fa, g, out)
    return out


def backward_d256(torch, fa, g, iters):
    """Recompute backward at B2 H16 N4096 d256 causal: dQ with D (stage 0), dK/dV
    (stage 1, the split-slot kernel) and both, after one forward for O and LSE. Flops:
    dQ three products, dK/dV four, of the forward's two."""
    B, H, N, d = 2, 16, 4096, 256
    rnd = lambda: torch.randn(B, H, N, d, device="cuda", dtype=torch.bfloat16, generator=g)
    q, k, v, do = rnd(), rnd(), rnd(), rnd()
    o = torch.empty_like(q)
    lse = torch.empty(B, H, N, device="cuda", dtype=torch.float32)
    fa.fwd(q, k, v, causal=True, out=o, lse=lse)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa.bwd_workspace_bytes(B, H, H, N, N, d), device="cuda", dtype=torch.uint8)
    f = fwd_flops(B, H, N, N, d, True)
    out = {}
    for stage, name, mult in ((0, "dq_kernel", 1.5), (1, "dkdv_kernel", 2.0), (-1, "whole", 2.5)):
        call = lambda stage=stage: fa.bwd(q, k, v, o, do, lse, causal=True, dq=dq, dk=dk, dv=dv,
                                          workspace=ws, stage=stage)
        out[name] = with_stats({}, timed_stats(torch, call, iters), mult * f)
    out["kernels"] = "bwd_dq_kernel<256, 32, 4, true>, bwd_dkdv_rs_kernel<true>"
    del q, k, v, do, o, dq, dk, dv, ws
    torch.cuda.empty_cache()
    return out


def fp8_forward(torch, fa, g, bf16_results, iters=50):
    """fa_fwd_fp8 on the shapes of the d=128 causal bf16 forward workloads: E4M3 inputs
    from seeded torch.randn scaled by 32 (per-tensor descale 1/32), FLOPs counted as for
    bf16, against the dense FP8 MFMA peak, with the speedup over fa_fwd on the same
    shape."""
    res = {}
    for name in ("c3a_bf16_causal_B4H32N4096d128", "c4a_bf16_causal_B1H8N32768d128"):
        from exact_tiled_attention_36_amd import synth
        w = synth.WORKLOADS[name]
        B, Hq, Hkv, Nq, Nk, d, causal = (w[x] for x in ("B", "Hq", "Hkv", "Nq", "Nk", "d", "causal"))
        mk = lambda *shape: (torch.randn(*shape, device="cuda", generator=g) * 32).to(torch.float8_e4m3fn)
        q, k, v = mk(B, Hq, Nq, d), mk(B, Hkv, Nk, d), mk(B, Hkv, Nk, d)
        o = torch.empty(B, Hq, Nq, d, device="cuda", dtype=torch.bfloat16)
        lse = torch.empty(B, Hq, Nq, device="cuda", dtype=torch.float32)
        call = lambda: fa.fwd_fp8(q, k, v, 1 / 32, 1 / 32, 1 / 32, causal=causal, out=o, lse=lse)
        fl = fwd_flops(B, Hq, Nq, Nk, d, causal)
        rec = with_stats({"workload": name.replace("bf16", "fp8")},
                         timed_stats(torch, call, iters), fl)
        del rec["pct_bf16_peak"]
        ms = rec["ms"]
        rec["pct_fp8_peak"] = round(fl / ms / 1e9 / PEAK_FP8_TFLOPS * 100, 2)
        if name in bf16_results:
            rec["speedup_over_bf16_fwd"] = round(bf16_results[name]["ms"] / ms, 3)
        res[name.replace("bf16", "fp8")] = rec
        del q, k, v, o, lse
        torch.cuda.empty_cache()
    return res


def rotated_small(torch, fa, g, sets=24, iters=96):
    """The B2 H16 N1024 d64 forward with its inputs and outputs (16.9 MB per call)
    rotated over `sets` copies, about 400 MB in all, more than the 256 MB last-level
    cache: each call finds its operands in HBM, not in cache as when one set is timed
    over and over."""
    B, H, N, d = 2, 16, 1024, 64
    bufs = []
    for _ in range(sets):
        q, k, v = (torch.randn(B, H, N, d, device="cuda", dtype=torch.bfloat16, generator=g)
                   for _ in range(3))
        bufs.append((q, k, v, torch.empty_like(q),
                     torch.empty(B, H, N, device="cuda", dtype=torch.float32)))
    turn = [0]

    def call():
        q, k, v, o, lse = bufs[turn[0] % sets]
        turn[0] += 1
        fa.fwd(q, k, v, causal=False, out=o, lse=lse)

    fl = fwd_flops(B, H, N, N, d, False)
    rec = with_stats({}, timed_stats(torch, call, iters), fl)
    nbytes = 2 * 4 * B * H * N * d + 4 * B * H * N
    del bufs
    torch.cuda.empty_cache()
    rec.update({"gbs": round(nbytes / rec["ms"] / 1e6, 1), "input_sets": sets})
    return rec


def gqa_decode(torch, fa, g, iters):
    """Split-KV decode with eight query heads per kv-head (the chunks run on the matrix
    cores), in GB/s of Q, K, V, O and LSE moved once."""
    B, Hq, Hkv, Nk, d = 16, 32, 4, 8192, 128
    q = torch.randn(B, Hq, 1, d, device="cuda", dtype=torch.bfloat16, generator=g)
    k = torch.randn(B, Hkv, Nk, d, device="cuda", dtype=torch.bfloat16, generator=g)
    v = torch.randn(B, Hkv, Nk, d, device="cuda", dtype=torch.bfloat16, generator=g)
    o = torch.empty_like(q)
    lse = torch.empty(B, Hq, 1, device="cuda", dtype=torch.float32)
    ws = torch.empty(fa.splitkv_workspace_bytes(B, Hq, Hkv, 1, Nk, d), device="cuda",
                     dtype=torch.uint8)
    call = lambda: fa.fwd_splitkv(q, k, v, causal=True, out=o, lse=lse, workspace=ws)
    rec = with_stats({}, timed_stats(torch, call, iters))
    ms = rec["ms"]
    nbytes = 2 * (q.numel() + k.numel() + v.numel() + o.numel()) + 4 * lse.numel()
    del q, k, v, o, lse, ws
    torch.cuda.empty_cache()
    rec.update({"gbs": round(nbytes / ms / 1e6, 1),
                "pct_hbm_peak": round(nbytes / ms / 1e6 / PEAK_HBM_GBS * 100, 2),
                "kernel": "fa_fwd_splitkv (matrix-core chunks + merge)"})
    return rec


def version_ablation(torch, fa, g, iters=5, reps=5):
    """The first version of the method against the second, on MI355X: the same forward
    through fa_fwd_variant 0 (deferred normalisation, (batch, head, row-block) grid),
    1 (renormalise O after every key block, same grid), 2 (first-version loop
    order: K/V blocks outer, Q blocks inner, O/m/l through HBM, (batch, head) grid) and
    3 (fa_fwd with every eighth exponential computed by a polynomial). The variants are
    timed in turn, reps times over, and the median of each is reported."""
    import statistics
    from exact_tiled_attention_36_amd import synth
    names = ("deferred", "renorm_every_block", "v1_loop_order", "poly_exp_1_in_8")
    res = {}
    for name in ("c2_bf16_B2H16N1024d64", "c3a_bf16_causal_B4H32N4096d128"):
        w = synth.WORKLOADS[name]
        B, Hq, Hkv, Nq, Nk, d, causal = (w[x] for x in ("B", "Hq", "Hkv", "Nq", "Nk", "d", "causal"))
        q = torch.randn(B, Hq, Nq, d, device="cuda", dtype=torch.bfloat16, generator=g)
        k = torch.randn(B, Hkv, Nk, d, device="cuda", dtype=torch.bfloat16, generator=g)
        v = torch.randn(B, Hkv, Nk, d, device="cuda", dtype=torch.bfloat16, generator=g)
        o = torch.empty_like(q)
        lse = torch.empty(B, Hq, Nq, device="cuda", dtype=torch.float32)
        ws = torch.empty(max(1, fa.load().fa_fwd_variant_workspace_bytes(B, Hq, Hkv, Nq, Nk, d, 2)),
                         device="cuda", dtype=torch.uint8)
        fl = fwd_flops(B, Hq, Nq, Nk, d, causal)
        times = {var: [] for var in range(4)}
        for _ in range(reps):
            for var in range(4):
                call = lambda: fa.fwd_variant(q, k, v, var, causal=causal, out=o, lse=lse, workspace=ws)
                times[var].append(timed_ms(torch, call, iters, warm_ms=20.0))
        rec = {}
        for var in range(4):
            ms = statistics.median(times[var])
            rec[names[var]] = {"ms": round(ms, 4), "tflops": round(fl / ms / 1e9, 1)}
        rec["v2_speedup_over_v1"] = round(rec["v1_loop_order"]["ms"] / rec["deferred"]["ms"], 2)
        res[name] = rec
        del q, k, v, o, lse, ws
        torch.cuda.empty_cache()
    return res


def profile_tail(torch, fa, calls=3):
    """Counter-run mode only: short runs of the kernels outside the training step, so one
    rocprofv3 pass also covers them: fa_mfma_probe on normal-like bf16 operands (matrix
    cores busy by construction: the reference for the busy-cycle counter), the
    non-causal B2 H16 N1024 d64 forward, split-KV decode at B8 H8 Nk32768 d128 (one row
    per kv-head) and B16 Hq32 Hkv4 Nk8192 d128 (eight rows), and the causal forward at
    B4 H32 N4096 d128, B2 H16 N4096 d256 and B1 H8 N32768 d128, and the d256 backward
    (B2 H16 N4096 causal)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(99)
    out = torch.empty(1024 * 256, device="cuda", dtype=torch.float32)
    for _ in range(calls):
        fa.mfma_probe(1024, 200, "normal_bf16", out=out)
    rnd = lambda *shape: torch.randn(*shape, device="cuda", dtype=torch.bfloat16, generator=g)
    q, k, v = rnd(2, 16, 1024, 64), rnd(2, 16, 1024, 64), rnd(2, 16, 1024, 64)
    for _ in range(calls):
        fa.fwd(q, k, v, causal=False)
    for B, Hq, Hkv, Nk in ((8, 8, 8, 32768), (16, 32, 4, 8192)):
        q, k, v = rnd(B, Hq, 1, 128), rnd(B, Hkv, Nk, 128), rnd(B, Hkv, Nk, 128)
        ws = torch.empty(fa.splitkv_workspace_bytes(B, Hq, Hkv, 1, Nk, 128), device="cuda",
                         dtype=torch.uint8)
        for _ in range(calls):
            fa.fwd_splitkv(q, k, v, causal=True, workspace=ws)
    # the causal forward workloads: B4 H32 N4096 d128, B2 H16 N4096 d256, B1 H8 N32768
    # d128, two calls each (in this order)
    for B, H, N, d in ((4, 32, 4096, 128), (2, 16, 4096, 256), (1, 8, 32768, 128)):
        q, k, v = rnd(B, H, N, d), rnd(B, H, N, d), rnd(B, H, N, d)
        for _ in range(2):
            fa.fwd(q, k, v, causal=True)
        del q, k, v
    # the d = 256 backward at B2 H16 N4096 causal: dQ with D, then dK/dV, twice
    q, k, v, do = (rnd(2, 16, 4096, 256) for _ in range(4))
    o = torch.empty_like(q)
    lse = torch.empty(2, 16, 4096, device="cuda", dtype=torch.float32)
    fa.fwd(q, k, v, causal=True, out=o, lse=lse)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa.bwd_workspace_bytes(2, 16, 16, 4096, 4096, 256), device="cuda",
                     dtype=torch.uint8)
    for _ in range(2):
        for stage in (0, 1):
            fa.bwd(q, k, v, o, do, lse, causal=True, dq=dq, dk=dk, dv=dv, workspace=ws,
                   stage=stage)
    torch.cuda.synchronize()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--stat-steps", type=int, default=50,
                    help="steps timed one by one after the timed region (median, min)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--profile", action="store_true",
                    help="counter-run mode: 1 GiB copy first, then the step; afterwards "
                         "the matrix-core probe, the d=64 forward, the two decode shapes "
                         "and the causal forward workloads; no oracle, no extras")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the method's heads and batch shard with no communication; see the "
              "design notes for how the path would shard)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from exact_tiled_attention_36_amd import fa, synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    fa.load()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)

    if args.profile:
        a = torch.zeros(1 << 28, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        torch.add(a, 1.0, out=b)  # elementwise kernel: exactly 1 GiB read, 1 GiB written
        torch.cuda.synchronize()
        del a, b

    log(f"generating {WORKLOAD}")
    inp = synth.workload(WORKLOAD)
    B, Hq, Hkv, Nq, Nk, d, causal = inp.B, inp.Hq, inp.Hkv, inp.Nq, inp.Nk, inp.d, inp.causal

    def to_dev(name):
        return torch.from_numpy(getattr(inp, name).view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v, do = to_dev("q"), to_dev("k"), to_dev("v"), to_dev("do")
    o = torch.empty_like(q)
    lse = torch.empty(B, Hq, Nq, device=dev, dtype=torch.float32)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa.bwd_workspace_bytes(B, Hq, Hkv, Nq, Nk, d), device=dev, dtype=torch.uint8)

    timer = Timer(torch, stream)

    def step_marks(tm):
        run = tm.mark if tm is not None else (lambda name, fn: fn())
        run("fwd_pp_kernel", lambda: fa.fwd(q, k, v, causal=causal, scale=inp.scale,
                                              out=o, lse=lse))
        for stg, name in ((0, "bwd_dq_kernel"), (1, "bwd_dkdv_kernel")):
            run(name, lambda stg=stg: fa.bwd(q, k, v, o, do, lse, causal=causal,
                                             scale=inp.scale, dq=dq, dk=dk, dv=dv,
                                             workspace=ws, stage=stg))

    def step(record):
        step_marks(timer if record else None)

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    f_fwd = fwd_flops(B, Hq, Nq, Nk, d, causal)
    f_step = 3.5 * f_fwd
    value = args.steps * f_step / elapsed / 1e12
    ms = timer.avg_ms()

    # Statistics pass after the timed region: STAT_STEPS more steps, each bracketed by
    # its own event pair (and each kernel by one), for the median and minimum.
    step_stats, phase_stats = {"median_ms": None, "min_ms": None}, {}
    if args.stat_steps > 0 and not args.profile:
        log(f"statistics over {args.stat_steps} steps")
        stat_timer = Timer(torch, stream)
        for _ in range(args.stat_steps):
            stat_timer.mark("step", lambda: step(False))
        inner = Timer(torch, stream)
        for _ in range(args.stat_steps):
            step_marks(inner)
        torch.cuda.synchronize()
        step_stats = stat_timer.stats()["step"]
        phase_stats = inner.stats()

    # algorithmic flops per launch: dense products each kernel performs (causal halved)
    per_kernel_flops = {"fwd_pp_kernel": f_fwd, "bwd_dkdv_kernel": 2 * f_fwd,
                        "bwd_dq_kernel": 1.5 * f_fwd}
    dom = max(per_kernel_flops, key=lambda kname: ms[kname])
    achieved = per_kernel_flops[dom] / (ms[dom] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 1),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": read_traffic(dom, WORKLOAD),
                "avg_launch_ms": round(ms[dom], 4)}

    rec = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": WORKLOAD, "B": B, "Hq": Hq, "Hkv": Hkv, "N": Nq, "d": d,
                   "causal": causal, "step": "fwd + recompute bwd"},
        "pct_bf16_peak": round(value / PEAK_BF16_TFLOPS * 100, 2),
        "roofline": roofline,
        "phases_ms": {kname: round(t, 4) for kname, t in ms.items()},
        "median_ms": step_stats["median_ms"], "min_ms": step_stats["min_ms"],
        "step_stats": {"step": step_stats, **phase_stats,
                       "note": f"{args.stat_steps} further steps after the timed region, "
                               "one event pair per step (and, in a second pass, per kernel)"},
        "phase_tflops": {"fwd": round(f_fwd / ms["fwd_pp_kernel"] / 1e9, 1),
                         "bwd": round(2.5 * f_fwd / (ms["bwd_dkdv_kernel"] + ms["bwd_dq_kernel"])
                                     / 1e9, 1)},
    }
    if args.profile:
        profile_tail(torch, fa)
    if not args.profile:
        log("matrix-core ceiling")
        ceil = mfma_ceiling(torch, fa)
        roofline["measured_mfma_tflops"] = ceil
        roofline["frac_of_measured_normal_bf16"] = round(achieved / ceil["normal_bf16"], 4)
    if not args.profile and not args.no_extra:
        log("extra workloads")
        rec["extra"] = extras(torch, fa)
    if not args.profile and not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        rec["cpu_baseline"] = cpu_baseline(inp)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
