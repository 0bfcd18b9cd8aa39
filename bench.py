"""Benchmark of the fused SDPA forward on one MI355X.

One step = one call of the fused forward (one kernel) over the long-sequence causal
workload: q, k, v bf16 [B=1, H=32, L=8192, D=128], entries N(0,1)*0.5, each a [B,L,H,D]
buffer viewed as [B,H,L,D] (non-contiguous), scale 1/sqrt(128), causal.  Inputs are
resident in HBM before the timed region.

Throughput is causal-adjusted: the algorithmic work of one step is 4*D flops per visible
(query, key) pair (2*D for q.k, 2*D for p.v), i.e. 2*B*H*D*L*(L+1) flops for a causal
square problem; work the kernel spends on the masked half of diagonal tiles is not
credited.  The roofline peak is MI355X's dense bf16 matrix-core rate,
256 CU x 2.4 GHz x 4096 flop/clk = 2516.6 TFLOP/s.

Prints one JSON line.  `--report PATH` also writes per-workload timings (all five
configurations, rank-3 vs rank-4) to PATH.

`--pass varlen` measures sdpa_fwd_varlen on packed documents: 32768 tokens in documents of
log-uniform lengths in [128, 8192] (seeded), H=32, D=128, bf16, causal per document; work
is 4*D per visible pair summed over the documents.

`--pass decode` measures sdpa_fwd_splitkv on a decode step: B=8 x H=32 heads, one query
each, against a 32768-key cache laid out [B,L,H,D], D=128, bf16, bottom-right causal (the
query sees every key).  It is bound by HBM: `value` is algorithmic bytes (q, k, v, out,
lse, each once) per second, against 8000 GB/s.

`--pass bias` measures sdpa_fwd_bias: q/k/v bf16 [2,8,4096,64], causal, an ALiBi-style
fp32 bias [1,8,4096,4096] (per-head slope times the query-key distance) broadcast over the
batch; 4*D flops per visible pair.

`--pass bwd` measures the gradients instead: one step = one sdpa_bwd call (its dq and dk/dv
kernels) on the same workload, with the forward's out and lse and an upstream gradient
(N(0,1), same [B,L,H,D] layout) resident before the timed region, gradients written in the
inputs' layout.  Its algorithmic work is 10*D flops per visible pair: five products of
2*D (the scores recomputed once, since P is never stored; dP; dV; dQ; dK).  The second
recomputation of S and dP inside the dq kernel is not credited.
"""
import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 256 * 2.4e9 * 4096 / 1e12  # 2516.58
PEAK_F32_TFLOPS = 157.3
HBM_PEAK_GBS = 8000.0
METRIC = "causal SDPA fwd TFLOP/s on 1 MI355X (% of bf16 MFMA peak), L=8192 D=128"
BWD_METRIC = "causal SDPA bwd TFLOP/s on 1 MI355X (% of bf16 MFMA peak), L=8192 D=128"
DECODE_METRIC = ("decode SDPA (split keys) GB/s on 1 MI355X (% of HBM peak), B=8 H=32 Lq=1 "
                 "Lk=32768 D=128")
BIAS_METRIC = ("causal SDPA fwd with an additive mask TFLOP/s on 1 MI355X (% of bf16 MFMA peak), "
               "B=2 H=8 L=4096 D=64")
VARLEN_METRIC = ("causal packed-documents SDPA fwd TFLOP/s on 1 MI355X (% of bf16 MFMA peak), "
                 "32768 tokens H=32 D=128")
# HBM bytes per launch of the fused kernel on the default workload: FETCH_SIZE and
# WRITE_SIZE from two rocprofv3 --pmc passes, each scaled by what the same counter reads
# for an elementwise kernel of known traffic (1 GiB in, 1 GiB out).  Valid only for the
# kernel source they were taken on (sha256 prefix below); reported as null otherwise.
TRAFFIC_BYTES = 544232 * 1024
TRAFFIC_KERNEL_SHA256 = "9a0c4c6655ddfdbb"
KERNEL_SOURCE = os.path.join(ROOT, "scaled_dot_product_11_amd", "csrc", "sdpa_fwd_gfx950.hip")
# The same for one backward call (dq and dk/dv kernels together).
BWD_TRAFFIC_BYTES = 1670917 * 1024
BWD_TRAFFIC_KERNEL_SHA256 = "93054143fcb440f2"
BWD_KERNEL_SOURCE = os.path.join(ROOT, "scaled_dot_product_11_amd", "csrc", "sdpa_bwd_gfx950.hip")


def measured_traffic(source=KERNEL_SOURCE, sha=TRAFFIC_KERNEL_SHA256, nbytes=TRAFFIC_BYTES):
    import hashlib
    with open(source, "rb") as f:
        current = hashlib.sha256(f.read()).hexdigest()
    return nbytes if current.startswith(sha) else None


def visible_pairs(Lq, Lk, causal):
    """(query, key) pairs of one head inside the causal triangle (all pairs otherwise)."""
    if not causal:
        return Lq * Lk
    full = min(Lq, Lk)
    return full * (full + 1) // 2 + max(0, Lq - Lk) * Lk


def step_flops(wl):
    """Algorithmic flops of one forward: 4*D per (query, key) pair the method evaluates.
    A causal problem evaluates only the triangle; a boolean mask is applied to the full
    score matrix, so a masked problem is counted dense."""
    B, H, Lq, Lk, D = wl.shape4()
    return 4 * D * B * H * visible_pairs(Lq, Lk, wl.is_causal)


def bwd_step_flops(wl):
    """Algorithmic flops of one backward: 10*D per visible pair (five products of 2*D)."""
    B, H, Lq, Lk, D = wl.shape4()
    return 10 * D * B * H * visible_pairs(Lq, Lk, wl.is_causal)


def time_kernel(fn, steps, warmup):
    """Warm up, then time `steps` calls: wall clock around all of them (synchronised on
    both sides) and HIP events around each launch on the stream the kernel runs on."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    t0 = time.perf_counter()
    for s, e in ev:
        s.record(stream)
        fn()
        e.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [s.elapsed_time(e) for s, e in ev]  # ms
    return wall, per


def cpu_baseline(wl, target_s=12.0, seed=0):
    """The fp64 oracle on a bounded sample of rows of the same workload, on the host
    cores; flops of the sampled rows / time, in TFLOP/s."""
    import numpy as np
    import oracle
    B, H, Lq, Lk, D = wl.shape4()
    rng = np.random.default_rng(seed)

    def row_flops(rows):
        i = rows % Lq
        vis = np.minimum(i + 1, Lk) if wl.is_causal else np.full_like(i, Lk)
        return int(4 * D * vis.sum())

    def run(n):
        rows = np.sort(rng.choice(B * H * Lq, size=n, replace=False))
        t0 = time.perf_counter()
        oracle.sdpa_oracle(wl.q, wl.k, wl.v, mask=wl.mask, is_causal=wl.is_causal,
                           scale=wl.scale, rows=rows)
        return time.perf_counter() - t0, row_flops(rows), n

    dt, fl, n = run(256)  # calibration
    n2 = int(min(B * H * Lq, max(256, 256 * target_s / max(dt, 1e-3))))
    dt, fl, n = run(n2)
    threads = oracle.default_threads()
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} query rows drawn uniformly from the {B * H * Lq} rows of the same "
                      f"workload, fp64 oracle, {dt:.2f} s for {fl / 1e9:.2f} GFLOP of visible "
                      f"pairs, {threads} OpenMP threads, host cpu: {cpu_model()}"}


def cpu_baseline_bwd(wl, target_s=12.0):
    """The fp64 backward oracle on a bounded sample of the same workload: the causal
    top-left corner [0, T) of the first 8 heads (an exact causal problem of its own, run
    one head per thread), T grown from 512 until about target_s; algorithmic flops of its
    visible pairs / time, in TFLOP/s."""
    import oracle
    import workloads as W
    B, H, Lq, Lk, D = wl.shape4()
    nh = min(8, H)
    dout = W.upstream_grad(41, wl.q, blhd=True)

    def run(T):
        sl = lambda t: t[:1, :nh, :T]
        t0 = time.perf_counter()
        oracle.sdpa_bwd_oracle(sl(wl.q), sl(wl.k), sl(wl.v), sl(dout), is_causal=wl.is_causal,
                               scale=wl.scale)
        return time.perf_counter() - t0, 10 * D * nh * visible_pairs(T, T, wl.is_causal)

    T = 512
    dt, fl = run(T)
    while dt < target_s / 4 and 2 * T <= Lq:  # cost grows ~4x per doubling
        T *= 2
        dt, fl = run(T)
    threads = min(nh, oracle.default_threads())
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"causal top-left corner L={T} of heads 0..{nh - 1} of the same workload, "
                      f"fp64 backward oracle, {dt:.2f} s for {fl / 1e9:.2f} GFLOP of visible "
                      f"pairs, one head per thread, host cpu: {cpu_model()}"}


def cpu_model():
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def to_device(wl, dev):
    import torch

    def mv(t):
        if t is None:
            return None
        d = t.to(dev)
        assert d.stride() == t.stride(), "device copy must keep the layout"
        return d
    return mv(wl.q), mv(wl.k), mv(wl.v), mv(wl.mask)


def bench_workload(wl, steps, warmup):
    import torch
    from scaled_dot_product_11_amd import sdpa_fwd
    q, k, v, m = to_device(wl, "cuda")
    out = torch.empty(q.shape, dtype=q.dtype, device="cuda")
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device="cuda")

    def fn():
        sdpa_fwd(q, k, v, out, lse, mask=m, is_causal=wl.is_causal, scale=wl.scale)
    wall, per = time_kernel(fn, steps, warmup)
    flops = step_flops(wl)
    return {"workload": wl.name, "flops": flops, "wall_s": wall, "steps": steps,
            "kernel_ms_mean": statistics.fmean(per), "kernel_ms_median": statistics.median(per),
            "kernel_ms_min": min(per), "kernel_ms_max": max(per),
            "tflops_median": flops / (statistics.median(per) * 1e-3) / 1e12}


# Vector-unit ceiling of the 16-bit forward.  A wave64 fp32 vector instruction issues in 4
# cycles (16 lanes per clock per SIMD; packed fp32 is not used), v_exp_f32 in ~8.6 cycles
# (device micro-benchmark).  Per workload, the vector instructions per computed score
# (SQ_INSTS_VALU / SQ_INSTS_VALU_TRANS_F32, one exponential per score) and the fraction of
# computed scores that are algorithmic (visible / computed) are counter measurements of the
# current kernels (profiles/sdpa_fwd_vector_work_per_score.md).  The ceiling is the rate at
# which 1024 SIMDs at 2.4 GHz could issue that vector work: 4*D flops per algorithmic score.
VALU_CYCLES_PER_INST = 4.0
EXP_CYCLES_PER_INST = 8.6
VALU_PER_SCORE = {  # workload name prefix: (vector instructions per score, visible / computed)
    "c2_": (6.28, 0.925), "c3_": (6.61, 0.961), "c4_": (5.42, 0.990), "c5_": (8.38, 0.997),
}


def valu_ceiling_tflops(name, D):
    """Vector-issue ceiling (TFLOP/s of algorithmic work) of a measured workload, or None."""
    for prefix, (v, frac) in VALU_PER_SCORE.items():
        if name.startswith(prefix):
            cycles_per_score = ((v - 1) * VALU_CYCLES_PER_INST + EXP_CYCLES_PER_INST) / 64
            return 4 * D * 1024 * 2.4e9 / cycles_per_score * frac / 1e12
    return None


def copy_calibration(mib):
    """One elementwise kernel that reads `mib` MiB and writes `mib` MiB: the HBM counters
    read for it give their scale factor against known traffic."""
    import torch
    n = mib * 2 ** 20 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.neg(src, out=dst)
    torch.cuda.synchronize()


def bench_bwd(wl, steps, warmup):
    import torch
    import workloads as W
    from scaled_dot_product_11_amd import sdpa_bwd, sdpa_fwd
    q, k, v, m = to_device(wl, "cuda")
    dout = W.upstream_grad(41, wl.q, device="cuda", blhd=True)
    out, lse = sdpa_fwd(q, k, v, mask=m, is_causal=wl.is_causal, scale=wl.scale)
    grads = [torch.empty_like(t) for t in (q, k, v)]  # keeps the inputs' strides
    for g, t in zip(grads, (q, k, v)):
        assert g.stride() == t.stride()
    delta = torch.empty_like(lse)

    def fn():
        sdpa_bwd(q, k, v, out, dout, lse, *grads, delta, mask=m, is_causal=wl.is_causal,
                 scale=wl.scale)
    wall, per = time_kernel(fn, steps, warmup)
    flops = bwd_step_flops(wl)
    return {"workload": wl.name, "flops": flops, "wall_s": wall, "steps": steps,
            "kernel_ms_mean": statistics.fmean(per), "kernel_ms_median": statistics.median(per),
            "kernel_ms_min": min(per), "kernel_ms_max": max(per),
            "tflops_median": flops / (statistics.median(per) * 1e-3) / 1e12}


def cpu_baseline_varlen(wl, target_s=12.0, seed=0):
    """The fp64 oracle on a bounded sample of query rows of every document, on the host
    cores; flops of the sampled rows / time, in TFLOP/s."""
    import numpy as np
    import oracle
    H, D = wl.q.shape[1], wl.q.shape[2]
    cq = wl.extra["cu_seqlens_q"].tolist()
    rng = np.random.default_rng(seed)

    def run(per_doc):
        fl, t0 = 0, time.perf_counter()
        for s, L in enumerate(wl.extra["lengths"]):
            view = lambda t: t[cq[s]:cq[s + 1]].transpose(0, 1).unsqueeze(0)
            rows = np.sort(rng.choice(H * L, size=min(per_doc, H * L), replace=False))
            oracle.sdpa_oracle(view(wl.q), view(wl.k), view(wl.v), is_causal=True,
                               scale=wl.scale, rows=rows)
            fl += int(4 * D * ((rows % L) + 1).sum())
        return time.perf_counter() - t0, fl

    n = 16
    dt, fl = run(n)
    n = int(max(16, n * target_s / max(dt, 1e-3)))
    dt, fl = run(n)
    threads = oracle.default_threads()
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} query rows drawn uniformly from each of the "
                      f"{len(wl.extra['lengths'])} documents (all heads), fp64 oracle, "
                      f"{dt:.2f} s for {fl / 1e9:.2f} GFLOP of visible pairs, {threads} OpenMP "
                      f"threads, host cpu: {cpu_model()}"}


def main_varlen(args, props):
    import torch
    import workloads as W
    from scaled_dot_product_11_amd import sdpa_fwd_varlen
    wl = W.config_varlen()
    q, k, v = (t.to("cuda") for t in (wl.q, wl.k, wl.v))
    cq = wl.extra["cu_seqlens_q"].to("cuda")
    lengths = wl.extra["lengths"]
    out = torch.empty_like(q)
    lse = torch.empty((q.shape[1], q.shape[0]), dtype=torch.float32, device="cuda")

    def fn():
        sdpa_fwd_varlen(q, k, v, cq, cq, max(lengths), out, lse, is_causal=True, scale=wl.scale)
    wall, per = time_kernel(fn, args.steps, args.warmup)
    H, D = q.shape[1], q.shape[2]
    flops = 4 * D * H * sum(visible_pairs(L, L, True) for L in lengths)
    ms_per_step = wall / args.steps * 1e3
    value = flops / (ms_per_step * 1e-3) / 1e12
    mean = statistics.fmean(per)
    achieved = flops / (mean * 1e-3) / 1e12
    line = {
        "metric": VARLEN_METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "pass": "varlen", "tokens": int(q.shape[0]), "heads": H,
                   "head_dim": D, "documents": len(lengths), "max_len": max(lengths),
                   "is_causal": True, "scale": wl.scale, "flops_per_step": flops,
                   "flop_convention": "4*D per visible (i,j) pair within each document",
                   "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
                   "device": props.name, "cus": props.multi_processor_count},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3),
                     "peak": round(PEAK_BF16_TFLOPS, 1), "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "kernel_ms_mean": round(mean, 4),
                     "kernel_ms_median": round(statistics.median(per), 4)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_varlen(wl)
    print(json.dumps(line), flush=True)


def decode_workload(device, heads=None):
    """The decode step's inputs, i.i.d. N(0,1) bf16 drawn on `device` from a generator
    seeded with 9: q [8,32,1,128] and the [8,32768,32,128] k and v buffers viewed as
    [B,H,L,D].  heads=n draws a smaller problem of the same distribution, [1,n,1,128]
    queries against [1,n,32768,128] keys, for the CPU sample."""
    import torch
    g = torch.Generator(device=device).manual_seed(9)
    B, H, L, D = (8, 32, 32768, 128) if heads is None else (1, heads, 32768, 128)

    def draw(shape):
        return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
    q = draw((B, 1, H, D)).transpose(1, 2)
    k, v = (draw((B, L, H, D)).transpose(1, 2) for _ in range(2))
    return q, k, v


def cpu_baseline_decode():
    """The fp64 oracle on a bounded sample of the decode step: heads of the same shape and
    distribution (one query row each, all 32768 keys), on the host cores; algorithmic bytes
    of those rows (their q, k, v, out, lse) / time, in GB/s."""
    import oracle
    import torch

    def run(n):
        q, k, v = decode_workload("cpu", heads=n)
        Lq, Lk, D = q.shape[2], k.shape[2], q.shape[3]
        mask = torch.ones(Lq, Lk, dtype=torch.bool).tril(Lk - Lq)
        t0 = time.perf_counter()
        oracle.sdpa_oracle(q, k, v, mask=mask)
        return time.perf_counter() - t0, n * (2 * Lk * D * 2 + 2 * D * 2 + 4)

    # drawing the sample costs more than evaluating it, so its size is fixed
    n = 64
    dt, nb = run(n)
    threads = oracle.default_threads()
    return {"value": nb / dt / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} heads of the decode step's shape (one query against 32768 keys "
                      f"each), fp64 oracle, {dt:.2f} s, {threads} OpenMP threads, host cpu: "
                      f"{cpu_model()}"}


def main_bias(args, props):
    import torch
    import workloads as W
    from scaled_dot_product_11_amd import sdpa_fwd_bias
    g = torch.Generator().manual_seed(960)
    q, k, v = (t.to("cuda") for t in W.draw_qkv(g, (2, 8, 4096, 64)))
    i = torch.arange(4096, device="cuda")
    slopes = 0.5 * 2.0 ** -torch.arange(8, dtype=torch.float32, device="cuda")
    bias = (-slopes[:, None, None] * (i[:, None] - i[None, :]).abs()).unsqueeze(0)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device="cuda")

    def fn():
        sdpa_fwd_bias(q, k, v, bias, out, lse, is_causal=True)
    wall, per = time_kernel(fn, args.steps, args.warmup)
    flops = 4 * 64 * 2 * 8 * visible_pairs(4096, 4096, True)
    # HBM bound (about 64 flop per byte, below the ridge): algorithmic bytes are q, k, v, out
    # (bf16), the lse and the bias entries of the visible pairs, read once (the bias is
    # broadcast over the batch)
    nbytes = 4 * q.numel() * 2 + lse.numel() * 4 + 8 * visible_pairs(4096, 4096, True) * 4
    ms_per_step = wall / args.steps * 1e3
    mean = statistics.fmean(per)
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved_gbs = nbytes / (mean * 1e-3) / 1e9
    line = {
        "metric": BIAS_METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "bias_alibi_bf16_causal_b2_h8_l4096_d64", "pass": "bias",
                   "bias": "fp32 [1,8,4096,4096], slope 0.5*2^-h times |i - j|",
                   "flops_per_step": flops, "flop_convention": "4*D per visible (i,j) pair",
                   "bias_bytes_read_per_step": 2 * 8 * visible_pairs(4096, 4096, True) * 4,
                   "algorithmic_bytes_per_step": nbytes,
                   "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
                   "device": props.name, "cus": props.multi_processor_count},
        "roofline": {"bound": "hbm", "achieved": round(achieved_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved_gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel_ms_mean": round(mean, 4),
                     "kernel_ms_median": round(statistics.median(per), 4)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_bias(q.cpu(), k.cpu(), v.cpu(), bias.cpu())
    print(json.dumps(line), flush=True)


def cpu_baseline_bias(q, k, v, bias, target_s=10.0):
    """The fp64 oracle (bias path) on a bounded sample of query rows of the same workload."""
    import numpy as np
    import oracle
    rng = np.random.default_rng(0)
    B, H, L, D = q.shape

    def run(n):
        rows = np.sort(rng.choice(B * H * L, size=n, replace=False))
        t0 = time.perf_counter()
        oracle.sdpa_oracle(q, k, v, is_causal=True, bias=bias, rows=rows)
        return time.perf_counter() - t0, int(4 * D * ((rows % L) + 1).sum()), n

    dt, fl, n = run(256)
    n = int(min(B * H * L, max(256, 256 * target_s / max(dt, 1e-3))))
    dt, fl, n = run(n)
    threads = oracle.default_threads()
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} query rows of the same workload, fp64 oracle with the bias, "
                      f"{dt:.2f} s, {threads} OpenMP threads, host cpu: {cpu_model()}"}


def main_decode(args, props):
    import torch
    from scaled_dot_product_11_amd import sdpa_fwd, sdpa_fwd_splitkv, sdpa_fwd_splitkv_workspace
    q, k, v = decode_workload("cuda")
    B, H, Lq, D = q.shape
    Lk = k.shape[2]
    out = torch.empty(q.shape, dtype=q.dtype, device="cuda")
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device="cuda")
    need = sdpa_fwd_splitkv_workspace(B, H, Lq, Lk, D, 0, 1)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")

    def fn():
        sdpa_fwd_splitkv(q, k, v, out, lse, is_causal=2, workspace=ws)
    wall, per = time_kernel(fn, args.steps, args.warmup)

    def dense():
        sdpa_fwd(q, k, v, out, lse, is_causal=2)
    _, per_dense = time_kernel(dense, max(5, args.steps // 5), 2)
    # a small batch (one sequence of 8 heads): too few heads to fill the chip without splits
    qs, ks, vs = q[:1, :8], k[:1, :8], v[:1, :8]
    outs, lses = out[:1, :8].clone(), lse[:1, :8].clone()
    ws_s = torch.empty(sdpa_fwd_splitkv_workspace(1, 8, Lq, Lk, D, 0, 1), dtype=torch.uint8,
                       device="cuda")
    _, per_small = time_kernel(lambda: sdpa_fwd_splitkv(qs, ks, vs, outs, lses, is_causal=2,
                                                        workspace=ws_s), 10, 3)
    _, per_small_dense = time_kernel(lambda: sdpa_fwd(qs, ks, vs, outs, lses, is_causal=2), 5, 2)
    small_bytes = 2 * 8 * Lk * D * 2 + 2 * 8 * Lq * D * 2 + 8 * Lq * 4
    nbytes = 2 * B * H * Lk * D * 2 + 2 * B * H * Lq * D * 2 + B * H * Lq * 4
    flops = 4 * D * B * H * visible_pairs(Lq, Lk, False)
    ms_per_step = wall / args.steps * 1e3
    mean = statistics.fmean(per)
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / (mean * 1e-3) / 1e9
    line = {
        "metric": DECODE_METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode_bf16_b8_h32_lq1_lk32768_d128_blhd", "pass": "decode",
                   "shape_q": [B, H, Lq, D], "shape_kv": [B, H, Lk, D],
                   "layout": "[B,L,H,D] buffers viewed as [B,H,L,D]", "is_causal": "bottom-right",
                   "bytes_per_step": nbytes, "tflops": round(flops / (mean * 1e-3) / 1e12, 3),
                   "splits": need // (B * H * Lq * (D + 1) * 4),
                   "dense_single_split_ms_mean": round(statistics.fmean(per_dense), 4),
                   "small_batch_b1_h8": {
                       "splitkv_ms_mean": round(statistics.fmean(per_small), 4),
                       "splitkv_gbs": round(small_bytes / statistics.fmean(per_small) / 1e6, 1),
                       "dense_ms_mean": round(statistics.fmean(per_small_dense), 4),
                       "dense_gbs": round(small_bytes / statistics.fmean(per_small_dense) / 1e6, 1)},
                   "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
                   "device": props.name, "cus": props.multi_processor_count},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernels": "fwd_bf16 (split keys) + splitkv_combine",
                     "kernel_ms_mean": round(mean, 4),
                     "kernel_ms_median": round(statistics.median(per), 4)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_decode()
    if args.copy_calibration_mib:
        copy_calibration(args.copy_calibration_mib)
    print(json.dumps(line), flush=True)


def as_dtype(wl, name):
    """The workload with its q, k, v cast to `name` ("bf16" leaves it as drawn; "f16" casts
    the bf16 draws, exactly, keeping the strides)."""
    import torch
    if name == "f16":
        wl.q, wl.k, wl.v = (t.to(torch.float16) for t in (wl.q, wl.k, wl.v))
        wl.name = wl.name.replace("bf16", "f16")
    return wl


def main_bwd(args, props):
    import workloads as W
    wl = as_dtype(W.config4(), args.dtype)
    r = bench_bwd(wl, args.steps, args.warmup)
    ms_per_step = r["wall_s"] / args.steps * 1e3
    value = r["flops"] / (ms_per_step * 1e-3) / 1e12
    achieved = r["flops"] / (r["kernel_ms_mean"] * 1e-3) / 1e12
    line = {
        "metric": BWD_METRIC if args.dtype == "bf16" else BWD_METRIC.replace("bf16", "fp16"),
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "pass": "bwd", "shape_bhld": [1, 32, 8192, 128],
                   "layout": "[B,L,H,D] buffers viewed as [B,H,L,D], gradients alike",
                   "is_causal": True, "scale": wl.scale, "flops_per_step": r["flops"],
                   "flop_convention": "10*D per visible (i,j) pair, causal-adjusted",
                   "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
                   "device": props.name, "cus": props.multi_processor_count},
        # one step is two kernels (dq, then dk/dv) timed together by events on the stream
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3),
                     "peak": round(PEAK_BF16_TFLOPS, 1), "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(BWD_KERNEL_SOURCE, BWD_TRAFFIC_KERNEL_SHA256,
                                                 BWD_TRAFFIC_BYTES) if args.dtype == "bf16"
                                else None,
                     "kernels": "bwd_dq_bf16 + bwd_dkdv_bf16",
                     "kernel_ms_mean": round(r["kernel_ms_mean"], 4),
                     "kernel_ms_median": round(r["kernel_ms_median"], 4)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_bwd(wl)
    if args.copy_calibration_mib:
        copy_calibration(args.copy_calibration_mib)
    print(json.dumps(line), flush=True)


def main_counters():
    """Three forward launches of each workload the per-score counter summaries cover, in the
    order c2, c5, c3 (rank 4), c4, then [1,32,8192,64] and [1,32,8192,32] causal."""
    import torch
    import workloads as W
    from scaled_dot_product_11_amd import sdpa_fwd
    for wl in (W.config2(), W.config5(), W.config3(rank=4), W.config4(), W.config4(D=64),
               W.config4(D=32)):
        q, k, v, m = to_device(wl, "cuda")
        out = torch.empty(q.shape, dtype=q.dtype, device="cuda")
        lse = torch.empty(q.shape[:-1], dtype=torch.float32, device="cuda")
        for _ in range(3):
            sdpa_fwd(q, k, v, out, lse, mask=m, is_causal=wl.is_causal, scale=wl.scale)
        torch.cuda.synchronize()
        print(wl.name, tuple(q.shape), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--dtype", choices=("bf16", "f16"), default="bf16",
                    help="input type of the fwd and bwd passes (default bf16, the metric's)")
    ap.add_argument("--pass", dest="which",
                    choices=("fwd", "bwd", "varlen", "decode", "bias", "counters"),
                    default="fwd",
                    help="fwd (default): the fused forward; bwd: its gradients; varlen: the "
                         "forward over packed documents; decode: split keys, one query per head; "
                         "counters: three forward launches of each profiled workload, for "
                         "counter passes (prints the workload names, no timing)")
    ap.add_argument("--head-dim", type=int, default=128, choices=(32, 64, 96, 128, 256),
                    help="fwd pass: head dim of the [1,32,8192,D] causal workload (default 128, "
                         "the metric's)")
    ap.add_argument("--report", default=None, help="write per-workload timings here")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one elementwise kernel reading and writing this many MiB "
                         "(scale reference for the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as W
    assert torch.cuda.is_available(), "no GPU visible"
    props = torch.cuda.get_device_properties(0)
    if args.which == "bwd":
        main_bwd(args, props)
        return
    if args.which == "varlen":
        main_varlen(args, props)
        return
    if args.which == "decode":
        main_decode(args, props)
        return
    if args.which == "bias":
        main_bias(args, props)
        return
    if args.which == "counters":
        main_counters()
        return

    D = args.head_dim
    wl = as_dtype(W.config4(D=D), args.dtype)
    r = bench_workload(wl, args.steps, args.warmup)
    ms_per_step = r["wall_s"] / args.steps * 1e3
    value = r["flops"] / (ms_per_step * 1e-3) / 1e12
    achieved = r["flops"] / (r["kernel_ms_mean"] * 1e-3) / 1e12
    line = {
        "metric": (METRIC if args.dtype == "bf16" else METRIC.replace("bf16", "fp16")).replace(
            "D=128", f"D={D}"),
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "shape_bhld": [1, 32, 8192, D],
                   "layout": "[B,L,H,D] buffers viewed as [B,H,L,D]", "is_causal": True,
                   "scale": wl.scale, "flops_per_step": r["flops"],
                   "flop_convention": "4*D per visible (i,j) pair, causal-adjusted",
                   "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
                   "device": props.name, "cus": props.multi_processor_count},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3),
                     "peak": round(PEAK_BF16_TFLOPS, 1), "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic() if args.dtype == "bf16" and D == 128
                     else None,
                     "kernel_ms_mean": round(r["kernel_ms_mean"], 4),
                     "kernel_ms_median": round(r["kernel_ms_median"], 4)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl)

    if args.copy_calibration_mib:
        copy_calibration(args.copy_calibration_mib)

    if args.report:
        rows = [(r, wl)]
        for name, fn in (("c1", W.config1), ("c2", W.config2), ("c5", W.config5)):
            w = fn()
            rows.append((bench_workload(w, args.steps, args.warmup), w))
        for rank in (3, 4):
            w = W.config3(rank=rank)
            rows.append((bench_workload(w, args.steps, args.warmup), w))
        results = []
        for row, w in rows:
            # both ceilings of the 16-bit kernels: the matrix cores and the vector issue
            D = w.shape4()[4]
            vc = valu_ceiling_tflops(w.name, D) if w.q.dtype != torch.float32 else None
            row = dict(row, pct_of_mfma_peak=round(100 * row["tflops_median"] / PEAK_BF16_TFLOPS, 2))
            if vc:
                row.update(valu_ceiling_tflops=round(vc, 1),
                           pct_of_valu_ceiling=round(100 * row["tflops_median"] / vc, 2))
            results.append(row)
        with open(args.report, "w") as f:
            json.dump({"peak_bf16_tflops": PEAK_BF16_TFLOPS, "device": props.name,
                       "results": results}, f, indent=1)

    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
