"""Benchmark of the prefill attention core on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
raw Q, K, V (token-major f32, already resident in HBM) -> per-head QK RMSNorm ->
NeoX RoPE -> causal GQA attention -> O.  ``--path fused`` runs it as the single
``qk_prep_attn`` call; ``--path unfused`` as ``qknorm_rope`` followed by
``gqa_prefill_attn``.  The throughput is causal attention TFLOP/s: 4 * head_dim *
n_head FLOPs per visible (query, key) pair, masked work not counted.

Prints one JSON line.  ``roofline`` describes the attention call (HIP events
around each gqa_prefill_attn / qk_prep_attn launch on the stream it runs on,
inside the timed region; in the bf16 modes that call is the K/V staging kernel
followed by the attention kernel, and the events bracket both);
``cpu_baseline`` is the f64 CPU oracle timed on a bounded sample of query rows
of the same workload on this host.
"""
from __future__ import annotations

import argparse
import hashlib
import glob
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "causal GQA prefill attention TFLOP/s (and % of MFMA peak) at T=512..16384"
PEAK_TFLOPS = {"f32": 157.3, "bf16": 2500.0, "bf16x3": 2500.0, "f16": 2500.0,
               "int8": 5000.0}   # MI355X dense MFMA peaks (int8: TOP/s)
HBM_PEAK_GBS = 8000.0


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "transformer_prefill_attention_amd", "csrc", "*"))):
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def load_traffic(workload: str, kernel: str, precision: str, path: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken
    on the current kernel sources; otherwise None."""
    f = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(f):
        return None
    try:
        rec = json.load(open(f))
    except Exception:
        return None
    key = f"{workload}/{kernel}/{precision}/{path}"
    e = rec.get(key)
    if not e or e.get("source_hash") != kernel_source_hash():
        return None
    return e.get("bytes_per_launch")


def cpu_baseline(w, x, target_s: float):
    """The oracle (as it stands) on evenly spaced query rows of the workload, all heads."""
    import numpy as np
    import oracle
    threads = len(os.sched_getaffinity(0))
    kw = dict(n_head=w.n_head, n_head_kv=w.n_head_kv, head_dim=w.head_dim, rope_dim=w.rope_dim,
              rope_freq_base=float(np.float32(w.rope_freq_base)),
              rms_eps=float(np.float32(w.rms_eps)), scale=w.softmax_scale,
              seq_offsets=w.seq_offsets, n_threads=threads)
    offs = w.seq_offsets

    def flops_of(rows):
        tot = 0
        for r in rows:
            s = int(np.searchsorted(offs, r, side="right") - 1)
            tot += 4 * w.head_dim * w.n_head * (int(r) - int(offs[s]) + 1)
        return tot

    def run(n):
        rows = np.unique(np.linspace(0, w.T - 1, n).round().astype(np.int64))
        t0 = time.perf_counter()
        oracle.qk_prep_attn(x.q, x.k, x.v, x.wq, x.wk, rows=rows, **kw)
        return rows, time.perf_counter() - t0

    # every run also pays the whole sequence's QK-norm + RoPE: fit time = fixed + per-row
    # cost from two small runs (evenly spaced rows cost the same on average), then size the
    # timed sample to the target
    rows_a, dt_a = run(32)
    rows_b, dt_b = run(128)
    per = max((dt_b - dt_a) / max(len(rows_b) - len(rows_a), 1), 1e-9)
    fixed = max(dt_a - per * len(rows_a), 0.0)
    n = int(max(128, min(w.T, (target_s - fixed) / per)))
    rows, dt = run(n)
    fl = flops_of(rows)
    rate = fl / dt
    # a row-sampled measurement: the oracle's rate on the sample; the whole workload's
    # oracle time is that rate's extrapolation to all rows (not run here: minutes)
    return {"value": rate / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"row-sampled: {len(rows)} of {w.T} query rows, evenly spaced, all "
                      f"{w.n_head} heads (QK-norm + RoPE of the whole sequence included); "
                      f"{fl:.3e} causal FLOPs in {dt:.2f} s",
            "sampled_rows": int(len(rows)),
            "full_oracle_s_extrapolated": round(w.attn_flops() / rate, 1)}


def qknorm_hbm(args):
    """qknorm_rope alone, out of place, each run after a 1 GiB read has evicted L2 and the
    MALL, so every input byte comes from HBM.  (Evicting by writing would leave the MALL full
    of dirty lines, whose write-back the timed kernel would then pay for.)  HIP events on the launch stream around each
    launch; median of --steps runs (at least 20).  The same measurement of a torch device copy
    of Q and K gives the rate a plain read + write stream reaches here."""
    import numpy as np
    import torch
    sys.path.insert(0, ROOT)
    import transformer_prefill_attention_amd as pfa
    from transformer_prefill_attention_amd import workloads as wl
    w = wl.CONFIGS[args.workload] if not args.seq_len else wl.sweep_workload(args.seq_len)
    x = wl.make_inputs(w)
    dev = torch.device("cuda:0")
    q, k = torch.from_numpy(x.q).to(dev), torch.from_numpy(x.k).to(dev)
    wq, wk = torch.from_numpy(x.wq).to(dev), torch.from_numpy(x.wk).to(dev)
    qn, kn = torch.empty_like(q), torch.empty_like(k)
    evict = torch.ones(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
    kw = dict(head_dim=w.head_dim, rope_dim=w.rope_dim, rope_freq_base=w.rope_freq_base,
              rms_eps=w.rms_eps, seq_offsets=w.seq_offsets if w.n_seqs > 1 else None)
    nbytes = 2 * (q.numel() + k.numel()) * 4   # read + write of Q and K

    def timed(fn, n):
        ts = []
        for i in range(n + 3):
            evict.max()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            if i >= 3:
                ts.append(a.elapsed_time(b))
        return float(np.median(ts))

    n = max(args.steps, 20)
    t_k = timed(lambda: pfa.qknorm_rope(q, k, wq, wk, q_out=qn, k_out=kn, **kw), n)
    t_c = timed(lambda: (qn.copy_(q), kn.copy_(k)), n)
    print(json.dumps({
        "kernel": "qknorm_rope", "workload": w.name, "bytes": nbytes, "runs": n,
        "evict_bytes": evict.numel() * 4,
        "median_ms": round(t_k, 4), "gbs": round(nbytes / t_k / 1e6, 1),
        "frac_of_8tbs": round(nbytes / t_k / 1e6 / HBM_PEAK_GBS, 4),
        "copy_median_ms": round(t_c, 4), "copy_gbs": round(nbytes / t_c / 1e6, 1)}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--spinup-ms", type=float, default=300.0,
                    help="before the warmup steps, run untimed steps for this long so the GPU "
                         "leaves its idle clock (it needs ~30 ms of load to reach its steady "
                         "shader clock); the timed region is still exactly --steps steps")
    ap.add_argument("--workload", default="prefill_8192")
    ap.add_argument("--seq-len", type=int, default=0, help="override: one sequence of this length "
                                                           "with the 8B-like heads")
    ap.add_argument("--precision", default="f32", choices=["f32", "bf16", "bf16x3", "f16"])
    ap.add_argument("--path", default="unfused", choices=["fused", "unfused", "tiled"],
                    help="unfused (default, currently the faster): qknorm_rope then "
                         "gqa_prefill_attn; fused: the single qk_prep_attn call; tiled (with "
                         "--chunk-base, bf16 modes): qk_prep_chunk_attn_tiled, the cache's bf16 "
                         "tiles kept across calls")
    ap.add_argument("--chunk-base", type=int, default=0, metavar="B",
                    help="time a chunk over a cached prefix instead: the workload's one sequence "
                         "is B cached rows (K normalised and rotated, V) and T - B new rows; "
                         "fused: qk_prep_chunk_attn on the raw new rows, unfused: gqa_chunk_attn "
                         "on prepared ones (no CPU baseline line)")
    ap.add_argument("--window", type=int, default=0, metavar="W",
                    help="with the chunk entry points (any --chunk-base, 0 included): a sliding "
                         "window of W keys per row, its own included")
    ap.add_argument("--gate", default="none", choices=["none", "elem", "head"],
                    help="with the chunk entry points: a gated output, out = O * sigmoid(gate), "
                         "the gate per element or per head (seeded N(0,1))")
    ap.add_argument("--q8", action="store_true",
                    help="time the 8-bit quantised session instead (Q, K, V quantised per "
                         "(token, head) after RoPE, attention through the int8 store): fused: "
                         "qk_prep_attn_q8 on the raw rows, unfused: gqa_attn_q8 on a filled "
                         "store; --chunk-base, --window and --gate apply (no CPU baseline line)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-bars", action="store_true",
                    help="skip the other bars (bf16 at T=8192, T=512 f32/bf16, T=16384 f32)")
    ap.add_argument("--no-profiler", action="store_true",
                    help="do not use the torch profiler for the per-kernel times of the bars")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--qknorm-hbm", action="store_true",
                    help="only time qknorm_rope on the workload's Q and K with L2 and MALL evicted "
                         "between runs (a 1 GiB buffer is read), beside a plain device copy of "
                         "the same bytes; median GB/s against 8 TB/s")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run torch copies of a MIB-sized f32 buffer (reference kernel of "
                         "known traffic for the rocprofv3 FETCH_SIZE / WRITE_SIZE scale factor)")
    args = ap.parse_args()

    if args.calibrate_copy:
        import torch
        n = args.calibrate_copy * (1 << 20) // 4
        a = torch.ones(n, device="cuda:0")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": 4 * n, "dispatches": 3}))
        return

    if args.qknorm_hbm:
        qknorm_hbm(args)
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the path shards by "
              "K/V head with no exchange, so N GPUs would each run the one-GPU kernel on "
              "n_head_kv/N heads.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import transformer_prefill_attention_amd as pfa
    from transformer_prefill_attention_amd import workloads as wl

    w = wl.sweep_workload(args.seq_len) if args.seq_len else wl.CONFIGS[args.workload]
    x = wl.make_inputs(w)
    if args.q8:
        if args.path == "tiled":
            raise SystemExit("--path tiled is a chunk entry (not --q8)")
        run_q8(args, w, x)
        return
    if args.chunk_base or args.window or args.gate != "none" or args.path == "tiled":
        run_chunk(args, w, x)
        return
    k_in = wl.with_outlier_keys(x.k, x.outliers)
    dev = torch.device("cuda:0")
    q = torch.from_numpy(x.q).to(dev)
    k = torch.from_numpy(k_in).to(dev)
    v = torch.from_numpy(x.v).to(dev)
    wq = torch.from_numpy(x.wq).to(dev)
    wk = torch.from_numpy(x.wk).to(dev)
    out = torch.empty_like(q)
    qn = torch.empty_like(q)
    kn = torch.empty_like(k)
    offs = w.seq_offsets if w.n_seqs > 1 else None
    kw_rope = dict(head_dim=w.head_dim, rope_dim=w.rope_dim, rope_freq_base=w.rope_freq_base,
                   rms_eps=w.rms_eps, seq_offsets=offs)
    stream = torch.cuda.current_stream(dev)
    ev = []

    def step(record):
        if args.path == "fused":
            if record:
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
            pfa.qk_prep_attn(q, k, v, wq, wk, scale=w.softmax_scale, precision=args.precision,
                             out=out, **kw_rope)
            if record:
                b.record(stream)
                ev.append((a, b))
        else:
            pfa.qknorm_rope(q, k, wq, wk, q_out=qn, k_out=kn, **kw_rope)
            if record:
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
            pfa.gqa_prefill_attn(qn, kn, v, head_dim=w.head_dim, scale=w.softmax_scale,
                                 precision=args.precision, seq_offsets=offs, out=out)
            if record:
                b.record(stream)
                ev.append((a, b))

    t_spin = time.perf_counter()
    while (time.perf_counter() - t_spin) * 1e3 < args.spinup_ms:
        step(False)
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    flops = w.attn_flops()
    value = flops / (elapsed / args.steps) / 1e12
    kern_ms, kern_med = event_stats(ev)
    achieved = flops / (kern_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[args.precision]
    # the kernels the call enqueues, as the library plans them (the bf16 modes and the f32
    # fused entry are several launches per call; the events bracket all of them)
    kernel = prefill_kernels(pfa, w, args.precision, args.path)
    traffic = load_traffic(w.name, kernel, args.precision, args.path)
    res = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "spinup_ms": args.spinup_ms,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": args.precision, "data": "synthetic (seeded N(0,1) Q/K/V, norm weights 1+N(0,0.1))",
        "config": {"workload": f"{w.name}: causal GQA prefill, T={w.T}, n_head={w.n_head}, "
                               f"n_head_kv={w.n_head_kv}, head_dim={w.head_dim}, "
                               f"rope_dim={w.rope_dim}, seqs={w.n_seqs}",
                   "T": w.T, "n_head": w.n_head, "n_head_kv": w.n_head_kv,
                   "head_dim": w.head_dim, "path": args.path, "causal_flops": flops},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": traffic,
                     "kernel": kernel, "kernel_ms": round(kern_ms, 4),
                     "kernel_ms_median": round(kern_med, 4), "launches": len(ev)},
    }
    if not args.no_bars:
        res["bars"] = measure_bars(pfa, wl, w, x, args)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, wl.Inputs(x.q, k_in, x.v, x.wq, x.wk, x.outliers),
                                           args.cpu_seconds)
    print(json.dumps(res), flush=True)


def event_stats(ev):
    """(mean, median) in ms of HIP event pairs.  The mean is the figure the roofline
    uses (rocprofv3 summaries report averages, and the two must agree); the median is
    reported beside it."""
    import numpy as np
    ts = np.array([a.elapsed_time(b) for a, b in ev], dtype=np.float64)
    return float(ts.mean()), float(np.median(ts))


def prefill_kernels(pfa, w, precision, path):
    entry = pfa.ENTRY_PREP if path == "fused" else pfa.ENTRY_PREFILL
    return pfa.attn_plan(entry, T_q=w.T, n_head=w.n_head, n_head_kv=w.n_head_kv,
                         head_dim=w.head_dim, rope_dim=w.rope_dim, precision=precision,
                         q_offsets=w.seq_offsets if w.n_seqs > 1 else None)["kernels"]


def time_prefill_call(pfa, w, t, precision, path, runs, warmup, profile=False):
    """The attention call alone (unfused: gqa_prefill_attn on prepared Q/K; fused:
    qk_prep_attn on raw rows), HIP events on the launch stream around every launch.
    With ``profile``, also the average device time of each kernel of the call from the
    torch profiler over the same runs (None where that is unavailable)."""
    import torch
    dev = t["q"].device
    stream = torch.cuda.current_stream(dev)
    offs = w.seq_offsets if w.n_seqs > 1 else None
    rope = dict(head_dim=w.head_dim, rope_dim=w.rope_dim, rope_freq_base=w.rope_freq_base,
                rms_eps=w.rms_eps, seq_offsets=offs)
    out = torch.empty_like(t["q"])
    if path == "fused":
        def call():
            pfa.qk_prep_attn(t["q"], t["k"], t["v"], t["wq"], t["wk"], scale=w.softmax_scale,
                             precision=precision, out=out, **rope)
    else:
        qn, kn = pfa.qknorm_rope(t["q"], t["k"], t["wq"], t["wk"], **rope)

        def call():
            pfa.gqa_prefill_attn(qn, kn, t["v"], head_dim=w.head_dim, scale=w.softmax_scale,
                                 precision=precision, seq_offsets=offs, out=out)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    ev = []
    for _ in range(runs):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        call()
        b.record(stream)
        ev.append((a, b))
    torch.cuda.synchronize()
    mean, med = event_stats(ev)
    per_kernel = None
    if profile:
        try:
            from torch.profiler import ProfilerActivity
            from torch.profiler import profile as tprofile
            with tprofile(activities=[ProfilerActivity.CUDA]) as prof:
                for _ in range(runs):
                    call()
                torch.cuda.synchronize()
            per_kernel = {}
            for e in prof.key_averages():
                us = getattr(e, "device_time", None)
                if us is None:
                    us = getattr(e, "cuda_time", None)
                if us and any(n in e.key for n in ("attn_", "stage_kv", "rope_table",
                                                    "qknorm_rope")):
                    per_kernel[e.key] = {"avg_ms": round(us / 1e3, 4), "count": e.count}
        except Exception as exc:  # the profiler is a diagnostic; the events stand alone
            per_kernel = {"unavailable": f"{type(exc).__name__}: {exc}"[:200]}
    return mean, med, per_kernel


def measure_bars(pfa, wl, w_main, x_main, args):
    """The other bars of the metric in the same run: bf16 and f16 at T = 8192 (the call,
    and its attention kernel alone), the 0.6B-like shape (T = 512, 16/8 heads) in f32 and
    bf16, and the long shape (T = 16384, keys with large norms) in f32 and f16.  Each is
    the attention call alone, timed with
    HIP events on its launch stream (20 runs after 5 warmup runs); TFLOP/s and the fraction
    of its own MFMA peak at the median run (a mean of 20 can carry one host stall of the
    process; the mean is reported beside it)."""
    import numpy as np
    import torch
    dev = torch.device("cuda:0")
    bars = []
    specs = [("prefill_8192", "bf16", "unfused", True), ("prefill_8192", "bf16", "fused", True),
             ("prefill_8192", "f16", "unfused", True),
             ("qwen3_0p6b", "f32", "unfused", False), ("qwen3_0p6b", "bf16", "unfused", False),
             ("long", "f32", "unfused", False), ("long", "f16", "unfused", False)]
    cache = {}
    for name, prec, path, prof in specs:
        w = wl.CONFIGS[name]
        if name not in cache:
            x = x_main if w.name == w_main.name else wl.make_inputs(w)
            cache.clear()
            cache[name] = {n: torch.from_numpy(np.ascontiguousarray(
                wl.with_outlier_keys(x.k, x.outliers) if n == "k" else getattr(x, n))).to(dev)
                for n in ("q", "k", "v", "wq", "wk")}
        t = cache[name]
        print(f"bar: {name} {prec} {path}", file=sys.stderr, flush=True)
        mean, med, per_kernel = time_prefill_call(pfa, w, t, prec, path, runs=20, warmup=5,
                                                  profile=prof and not args.no_profiler)
        flops = w.attn_flops()
        peak = PEAK_TFLOPS[prec]
        bar = {"workload": name, "T": w.T, "n_head": w.n_head, "n_head_kv": w.n_head_kv,
               "precision": prec, "path": path,
               "kernel": prefill_kernels(pfa, w, prec, path),
               "call_ms": round(mean, 4), "call_ms_median": round(med, 4),
               "tflops": round(flops / (med * 1e-3) / 1e12, 3),
               "frac": round(flops / (med * 1e-3) / 1e12 / peak, 4), "peak": peak}
        if per_kernel is not None:
            bar["per_kernel"] = per_kernel
            attn = [v for k, v in per_kernel.items() if isinstance(v, dict) and
                    k.split("<")[0].split("::")[-1].startswith("attn_bf16_kernel")]
            if attn:
                ms = attn[0]["avg_ms"]
                bar["attention_kernel_ms"] = ms
                bar["attention_kernel_frac"] = round(flops / (ms * 1e-3) / 1e12 / peak, 4)
        bars.append(bar)
    return bars


def run_chunk(args, w, x):
    """One chunk of new rows over a cached prefix per step (``--chunk-base``)."""
    import torch

    import transformer_prefill_attention_amd as pfa

    if w.n_seqs != 1 or not 0 <= args.chunk_base < w.T:
        raise SystemExit("--chunk-base needs a one-sequence workload longer than the prefix")
    B, T = args.chunk_base, w.T
    T_q = T - B
    dev = torch.device("cuda:0")
    t = {n: torch.from_numpy(getattr(x, n)).to(dev) for n in ("q", "k", "v", "wq", "wk")}
    kw_rope = dict(head_dim=w.head_dim, rope_dim=w.rope_dim, rope_freq_base=w.rope_freq_base,
                   rms_eps=w.rms_eps)
    # the cache a previous call would have left: normalised, rotated K and V of all rows
    # (the fused step rewrites its new rows in place each time)
    qn, kn = pfa.qknorm_rope(t["q"], t["k"], t["wq"], t["wk"], **kw_rope)
    k_cache, v_cache = kn.clone(), t["v"].clone()
    q_new, k_new, v_new = t["q"][B:].contiguous(), t["k"][B:].contiguous(), t["v"][B:].contiguous()
    q_prep = qn[B:].contiguous()
    out = torch.empty_like(q_new)
    kv_tiles = None
    if args.path == "tiled":
        if args.precision == "f32":
            raise SystemExit("--path tiled is for the bf16 modes")
        # the tiles a previous call would have left: the prefix rows appended once
        # (untimed); each step then re-stages the tiles of its new rows
        kv_tiles = torch.empty(pfa.kv_tiles_bytes(1, T, w.n_head_kv, w.head_dim, args.precision),
                               dtype=torch.uint8, device=dev)
        if B:
            kp, vp = k_cache[:B].clone(), v_cache[:B].clone()
            pfa.qk_prep_chunk_attn_tiled(t["q"][:B].contiguous(), t["k"][:B].contiguous(),
                                         t["v"][:B].contiguous(), t["wq"], t["wk"], kp, vp,
                                         kv_tiles, max_rows=T, scale=w.softmax_scale,
                                         precision=args.precision, **kw_rope)
            torch.cuda.synchronize()
    gate = None
    if args.gate != "none":
        g = torch.Generator().manual_seed(w.seed + 1)
        cols = w.n_head * (w.head_dim if args.gate == "elem" else 1)
        gate = torch.randn(T_q, cols, generator=g).to(dev)
    stream = torch.cuda.current_stream(dev)
    ev = []

    def step(record):
        if record:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
        if args.path == "fused":
            pfa.qk_prep_chunk_attn(q_new, k_new, v_new, t["wq"], t["wk"], k_cache, v_cache,
                                   scale=w.softmax_scale, window=args.window, gate=gate,
                                   precision=args.precision, out=out, **kw_rope)
        elif args.path == "tiled":
            pfa.qk_prep_chunk_attn_tiled(q_new, k_new, v_new, t["wq"], t["wk"], k_cache, v_cache,
                                         kv_tiles, max_rows=T, scale=w.softmax_scale,
                                         window=args.window, gate=gate,
                                         precision=args.precision, out=out, **kw_rope)
        else:
            pfa.gqa_chunk_attn(q_prep, k_cache, v_cache, head_dim=w.head_dim,
                               scale=w.softmax_scale, window=args.window, gate=gate,
                               precision=args.precision, out=out)
        if record:
            b.record(stream)
            ev.append((a, b))

    t_spin = time.perf_counter()
    while (time.perf_counter() - t_spin) * 1e3 < args.spinup_ms:
        step(False)
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # visible (query, key) pairs per head: row r sees B + r + 1 keys, or with a window
    # min(W, B + r + 1)
    if args.window:
        Wn = args.window
        pairs = sum(min(Wn, B + r + 1) for r in range(T_q))
    else:
        pairs = T_q * B + T_q * (T_q + 1) // 2
    flops = 4 * w.head_dim * w.n_head * pairs
    kern_ms, kern_med = event_stats(ev)
    achieved = flops / (kern_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[args.precision]
    d = w.head_dim
    entry = {"fused": pfa.ENTRY_CHUNK_PREP, "tiled": pfa.ENTRY_CHUNK_TILED}.get(args.path,
                                                                          pfa.ENTRY_CHUNK)
    kernel = pfa.attn_plan(entry,
                           T_q=T_q, T_kv=T, n_head=w.n_head, n_head_kv=w.n_head_kv, head_dim=d,
                           rope_dim=w.rope_dim, window=args.window, precision=args.precision,
                           q_offsets=[0, T_q], kv_offsets=[0, T])["kernels"]
    res = {
        "metric": METRIC, "value": round(flops / (elapsed / args.steps) / 1e12, 3),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "spinup_ms": args.spinup_ms, "ms_per_step": round(elapsed * 1e3 / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": args.precision, "data": "synthetic (seeded N(0,1) Q/K/V, norm weights 1+N(0,0.1))",
        "config": {"workload": f"{w.name} chunk: {T_q} new rows over {B} cached rows, "
                               f"n_head={w.n_head}, n_head_kv={w.n_head_kv}, head_dim={d}, "
                               f"rope_dim={w.rope_dim}"
                               + (f", window={args.window}" if args.window else "")
                               + (f", gate per {args.gate}" if gate is not None else ""),
                   "T_q": T_q, "T_kv": T, "n_head": w.n_head, "n_head_kv": w.n_head_kv,
                   "head_dim": d, "path": args.path, "causal_flops": flops},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": None,
                     "kernel": kernel, "kernel_ms": round(kern_ms, 4),
                     "kernel_ms_median": round(kern_med, 4)},
    }
    print(json.dumps(res), flush=True)


def run_q8(args, w, x):
    """One step of an 8-bit quantised session (``--q8``): prefill of the workload, or with
    ``--chunk-base B`` its last T - B rows over B stored rows."""
    import torch

    import transformer_prefill_attention_amd as pfa

    if w.n_seqs != 1 or not 0 <= args.chunk_base < w.T:
        raise SystemExit("--q8 needs a one-sequence workload longer than --chunk-base")
    B, T, d = args.chunk_base, w.T, w.head_dim
    T_q = T - B
    dev = torch.device("cuda:0")
    t = {n: torch.from_numpy(getattr(x, n)).to(dev) for n in ("q", "k", "v", "wq", "wk")}
    kw_rope = dict(head_dim=d, rope_dim=w.rope_dim, rope_freq_base=w.rope_freq_base,
                   rms_eps=w.rms_eps)
    offs = dict(q_offsets=[0, T_q], kv_offsets=[0, T]) if B else {}
    # the store a session holds after prefilling all T rows (the fused step rewrites its new
    # rows in place each time); the unfused step also needs the new rows' Q codes
    kc = torch.zeros(T, w.n_head_kv * d, dtype=torch.int8, device=dev)
    vc = torch.zeros_like(kc)
    ks = torch.zeros(T, w.n_head_kv, dtype=torch.float32, device=dev)
    vs = torch.zeros_like(ks)
    pfa.qk_prep_attn_q8(t["q"], t["k"], t["v"], t["wq"], t["wk"], kc, ks, vc, vs,
                        scale=w.softmax_scale, **kw_rope)
    qn, _ = pfa.qknorm_rope(t["q"], t["k"], t["wq"], t["wk"], **kw_rope)
    qc, qs = pfa.quantize_rows(qn[B:].contiguous(), d)
    q_new, k_new, v_new = t["q"][B:].contiguous(), t["k"][B:].contiguous(), t["v"][B:].contiguous()
    out = torch.empty_like(q_new)
    gate = None
    if args.gate != "none":
        g = torch.Generator().manual_seed(w.seed + 1)
        gate = torch.randn(T_q, w.n_head * (d if args.gate == "elem" else 1), generator=g).to(dev)
    stream = torch.cuda.current_stream(dev)
    ev = []

    def step(record):
        if record:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
        if args.path == "fused":
            pfa.qk_prep_attn_q8(q_new, k_new, v_new, t["wq"], t["wk"], kc, ks, vc, vs,
                                scale=w.softmax_scale, window=args.window, gate=gate, out=out,
                                **kw_rope, **offs)
        else:
            pfa.gqa_attn_q8(qc, qs.view(T_q, w.n_head), kc, ks, vc, vs, head_dim=d,
                            scale=w.softmax_scale, window=args.window, gate=gate, out=out,
                            **offs)
        if record:
            b.record(stream)
            ev.append((a, b))

    t_spin = time.perf_counter()
    while (time.perf_counter() - t_spin) * 1e3 < args.spinup_ms:
        step(False)
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    if args.window:
        pairs = sum(min(args.window, B + r + 1) for r in range(T_q))
    else:
        pairs = T_q * B + T_q * (T_q + 1) // 2
    flops = 4 * d * w.n_head * pairs
    kern_ms, kern_med = event_stats(ev)
    achieved = flops / (kern_ms * 1e-3) / 1e12
    # head_dim 128: Q.K^T on int8 matrix cores (5.0 POP/s dense), P.V on bf16 (2.5 PF):
    # half the FLOPs each, so the least time is F/2 (1/5000 + 1/2500) -> a 3333 TFLOP/s
    # peak for the whole; head_dim 64 runs both products on bf16
    peak = (2.0 / (1.0 / PEAK_TFLOPS["int8"] + 1.0 / PEAK_TFLOPS["bf16"]) if d == 128
            else PEAK_TFLOPS["bf16"])
    kernel = pfa.attn_plan(pfa.ENTRY_Q8_PREP if args.path == "fused" else pfa.ENTRY_Q8,
                           T_q=T_q, T_kv=T, n_head=w.n_head, n_head_kv=w.n_head_kv, head_dim=d,
                           rope_dim=w.rope_dim, window=args.window,
                           q_offsets=[0, T_q], kv_offsets=[0, T])["kernels"]
    what = (f"{T_q} new rows over {B} stored rows" if B else f"prefill of {T} rows")
    traffic = None if (B or args.window or gate is not None) else \
        load_traffic(w.name, kernel, "q8", args.path)
    res = {
        "metric": METRIC, "value": round(flops / (elapsed / args.steps) / 1e12, 3),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "spinup_ms": args.spinup_ms, "ms_per_step": round(elapsed * 1e3 / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int8 codes, bf16 MFMA",
        "data": "synthetic (seeded N(0,1) Q/K/V, norm weights 1+N(0,0.1)), quantised per row",
        "config": {"workload": f"{w.name} 8-bit session: {what}, n_head={w.n_head}, "
                               f"n_head_kv={w.n_head_kv}, head_dim={d}, rope_dim={w.rope_dim}"
                               + (f", window={args.window}" if args.window else "")
                               + (f", gate per {args.gate}" if gate is not None else ""),
                   "T_q": T_q, "T_kv": T, "n_head": w.n_head, "n_head_kv": w.n_head_kv,
                   "head_dim": d, "path": args.path, "causal_flops": flops},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": traffic,
                     "kernel": kernel, "kernel_ms": round(kern_ms, 4),
                     "kernel_ms_median": round(kern_med, 4)},
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
