#!/usr/bin/env python
"""Benchmark of exact relative-position attention, forward + backward, on one GPU.

One step = every stage of the path on one batch of seeded synthetic input
already resident in HBM: map tables and relation projection, fused forward,
backward row terms, the query- and key-parallel passes (one launch that
carries the blocks of both), contraction and bucket fold.  The default workload is the 8K layer-benchmark shape of the
setup section of "Fast and Exact Relative-Position Attention via
Structure-Aware Kernels" (nanless.github.io digest) for the Shaw mechanism:
B=1, H=12, N=8192, d=64, fp16, truncation +-128.

Timing: W untimed warmup steps, then exactly K steps between two
synchronisations.  HIP events are recorded between the stage calls, on the
stream the library launches on, so each kernel's average duration is measured
live; the dominant attention kernel gives the roofline figure.
FLOP convention (FlashAttention): forward 4 d per live (query, key) pair,
backward 10 d; the roofline fraction of a kernel counts that useful work, and
the backward launch's executed GEMM work (query pass 6 d plus key pass 8 d
per pair, S and dP computed by both passes) is reported beside it.  Peak
memory is the allocator's high-water mark of one forward and one backward
call beyond what is resident when each starts.  The CPU baseline is the fp64
oracle on a bounded sample (whole (batch, head) slices of the same workload,
about ten seconds of work), forward and backward timed separately on every
host core the process may use.

Prints one JSON line.
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fwd+bwd ms and TFLOP/s (% fp16 MFMA peak), N=8192 H=12 d=64 fp16; peak memory"
PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0, "f32": 157.3}
HBM_PEAK_GBS = 8000.0


def live_pairs(w, key_len):
    """Number of unmasked (query, key) pairs over the whole batch, per head."""
    N = w.N
    total = 0
    for b in range(w.B):
        kl = N if key_len is None else int(key_len[b])
        kl = max(0, min(N, kl))
        if w.causal:
            # query i sees keys j <= min(i, kl - 1)
            m = min(N, kl)
            total += m * (m + 1) // 2 + (N - m) * m
        else:
            total += N * kl
    return total


def describe(w):
    phi = w.phi
    if phi["kind"] == "truncated":
        ps = f"truncated[{phi['lo']},{phi['hi']}]"
    elif phi["kind"] == "t5":
        ps = f"t5[{phi['num_buckets']} buckets, max {phi['max_distance']}]"
    elif phi["kind"] == "log":
        ps = f"log[{phi['num_buckets']} buckets, max {phi['max_distance']}]"
    else:
        ps = "identity"
    terms = "+".join(t for t, f in (("aQ", w.has_aq), ("aK", w.has_ak), ("b", w.has_b)) if f)
    mask = "+".join(m for m, f in (("causal", w.causal), ("key_padding", w.key_padding)) if f)
    out = {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "phi": ps,
           "terms": terms or "none", "mask": mask or "none", "tau": round(w.tau, 6)}
    if w.dropout is not None:
        out["dropout_p"] = w.dropout[0] / 256.0
    if w.zchunk:
        out["zchunk"] = w.zchunk
    if w.relation:
        out["relation"] = w.relation
    return out


def cpu_baseline(w, x, min_seconds=10.0):
    """fp64 oracle, forward then backward of whole (batch, head) slices at the
    full length, taken in order until about `min_seconds` of CPU work is done.
    It runs on every core the process may use, with the BLAS thread pool set
    to that count; the forward and the backward are timed separately, and
    the rate counts the same useful work as the GPU figure (4 d and 10 d
    flops per live pair)."""
    import oracle
    from relpos_synth import as_f64
    cores = len(os.sched_getaffinity(0))
    blas = "unknown"
    limiter = None
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        limiter = threadpool_limits(limits=cores)
        libs = [f"{p.get('internal_api')} {p.get('version')} ({p.get('num_threads')} threads)"
                for p in threadpool_info() if p.get("user_api") == "blas"]
        blas = "; ".join(libs) or blas
    except Exception:  # noqa: BLE001
        pass
    f = {k: as_f64(v) for k, v in x.items() if k != "key_len"}
    kl = None if x["key_len"] is None else x["key_len"].numpy()
    slices = [(b, h) for b in range(w.B) for h in range(w.H)]
    done = []
    pairs = 0
    t_fwd = t_bwd = 0.0
    try:
        for bh in slices:
            t0 = time.perf_counter()
            oracle.forward(f["q"], f["k"], f["v"], f["aq"], f["ak"], f["b"], phi=w.phi,
                           tau=w.tau, causal=w.causal, key_len=kl, bh=[bh], dropout=w.dropout)
            t1 = time.perf_counter()
            oracle.backward(f["q"], f["k"], f["v"], f["aq"], f["ak"], f["b"], dO=f["do"],
                            phi=w.phi, tau=w.tau, causal=w.causal, key_len=kl, bh=[bh],
                            dropout=w.dropout)
            t2 = time.perf_counter()
            t_fwd += t1 - t0
            t_bwd += t2 - t1
            done.append(bh)
            pairs += live_pairs(w.with_(B=1), None if kl is None else kl[bh[0]:bh[0] + 1])
            if t_fwd + t_bwd >= min_seconds:
                break
    finally:
        if limiter is not None:
            limiter.unregister()
    dt = t_fwd + t_bwd
    return {"value": 14.0 * w.d * pairs / dt / 1e12, "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle", "seconds": round(dt, 3),
            "fwd_s": round(t_fwd, 3), "bwd_s": round(t_bwd, 3),
            "fwd_tflops": 4.0 * w.d * pairs / t_fwd / 1e12,
            "bwd_tflops": 10.0 * w.d * pairs / t_bwd / 1e12,
            "blas": blas,
            "sample": f"forward and backward of {len(done)} of {len(slices)} (batch, head) "
                      f"slices at full N={w.N}, fp64 NumPy"}


def window_columns(w, key_side=False):
    """Z entries the projection computes for one (batch, head): each group of
    128 queries (keys) computes the contiguous window of unfolded rows its
    offsets reach, or every row of the unfolded map when that is no wider
    than N + 127 (one group for all); a causal mask keeps offsets <= 0 only.
    This is the algorithmic size of Z^Q (key_side: Z^K), in entries."""
    import exact_relative_position_amd._binding as B_
    N = w.N
    _, lo, hi = B_.phi_info(w.phi, N)
    R = hi - lo + 1

    def row(o):
        return min(max(o, lo), hi) - lo

    G = 128
    groups = [(0, N - 1)] if R <= N + G - 1 else \
        [(g0, min(N - 1, g0 + G - 1)) for g0 in range(0, N, G)]
    total = 0
    for first, last in groups:
        omin, omax = (first - (N - 1), last) if key_side else (-last, N - 1 - first)
        if w.causal:
            omax = min(omax, 0)
        total += (last - first + 1) * (row(omax) - row(omin) + 1)
    return total


_COMMON = ("qside.hpp", "tiles.hpp", "device.hpp", "geometry.hpp", "dropout.hpp")
KERNEL_SOURCES = {
    "fwd_kernel": ("attn_fwd.hip", "inblock.hpp") + _COMMON,
    "bwd_kernel": ("attn_bwd.hpp", "attn_bwd_q.hpp", "attn_bwd_k.hpp", "attn_bwd_f32.hip",
                   "attn_bwd_f16.hip", "attn_bwd_bf16.hip") + _COMMON,
}


def kernel_source_hash(kernel):
    """sha256 over the HIP sources that define one attention kernel."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "exact_relative_position_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    rocprofv3 counter summary, or None when there is none or the kernel's
    source has changed since the counters were taken."""
    try:
        with open(os.path.join(ROOT, "profiles", f"counters_{workload}.md")) as fh:
            lines = fh.read().splitlines()
    except OSError:
        return None
    want = kernel_source_hash(kernel)
    for line in lines:
        f = line.split()
        if len(f) == 5 and f[0] == "traffic" and f[1] == kernel and f[2] == workload:
            kv = dict(x.split("=", 1) for x in f[3:])
            if kv.get("sha256") == want:
                return int(kv["bytes"])
    return None


def copy_probe(torch, dev, mib):
    """One plain device-to-device copy of `mib` MiB, outside the timed region:
    its HBM counter readings calibrate the counters of the other kernels."""
    n = mib * (1 << 20) // 2
    a = torch.empty(n, dtype=torch.float16, device=dev).fill_(1.0)
    c = torch.empty_like(a)
    torch.cuda.synchronize(dev)
    c.copy_(a)
    torch.cuda.synchronize(dev)
    del a, c


def measure_peak_memory(torch, dev, t, w, drop):
    """Peak device memory of one forward and one backward call beyond what is
    allocated when each starts (the pages' measure: extra allocation beyond
    the inputs), by the allocator's high-water mark.  The forward's extra
    memory is O, LSE, the kept projections and its workspace; the backward's
    (with the forward's outputs resident) is dQ, dK, dV, the table gradients
    and its workspace.  Run outside the timed region."""
    import exact_relative_position_amd as rp
    args = (t["q"], t["k"], t["v"], t["aq"], t["ak"], t["b"])
    kw = dict(phi=w.phi, tau=w.tau, causal=w.causal, key_len=t["key_len"], dropout=drop,
              zchunk=w.zchunk, relation=w.relation)
    torch.cuda.synchronize(dev)
    base = torch.cuda.memory_allocated(dev)
    torch.cuda.reset_peak_memory_stats(dev)
    O, lse, zs = rp.forward(*args, keep_z=True, **kw)
    torch.cuda.synchronize(dev)
    fwd = torch.cuda.max_memory_allocated(dev) - base
    base = torch.cuda.memory_allocated(dev)
    torch.cuda.reset_peak_memory_stats(dev)
    grads = rp.backward(*args, O, lse, t["do"], zs, **kw)
    torch.cuda.synchronize(dev)
    bwd = torch.cuda.max_memory_allocated(dev) - base
    del O, lse, zs, grads
    torch.cuda.empty_cache()
    return {"fwd": int(fwd), "bwd": int(bwd)}


def stage_list(B_, run, separate_passes=False):
    """The stages of one step, in order, as (name, call) pairs."""
    stages = [("project", lambda: run.fwd(B_.FWD_PROJECT)),
              ("attend", lambda: run.fwd(B_.FWD_ATTEND)),
              ("prepare", lambda: run.bwd(B_.BWD_PREPARE)),
              ("passes", lambda: run.bwd(B_.BWD_QUERY_PASS | B_.BWD_KEY_PASS)),
              ("contract", lambda: run.bwd(B_.BWD_CONTRACT))]
    if separate_passes:
        # diagnostic: one launch per pass (the default step launches both at once)
        k = [n for n, _ in stages].index("passes")
        stages[k:k + 1] = [("query_pass", lambda: run.bwd(B_.BWD_QUERY_PASS)),
                           ("key_pass", lambda: run.bwd(B_.BWD_KEY_PASS))]
    return stages


def time_stages(torch, dev, stages, warmup, steps):
    """W untimed steps, then K timed steps with HIP events between the stage
    calls on the launch stream.  Returns (average ms per stage, GPU ms per
    step, wall seconds of the timed steps); the per-step stage times are left
    in time_stages.per_step for the median and minimum."""
    for _ in range(warmup):
        for _, fn in stages:
            fn()
    stream = torch.cuda.current_stream(dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
          for _ in range(steps)]
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for s in range(steps):
        ev[s][0].record(stream)
        for k, (_, fn) in enumerate(stages):
            fn()
            ev[s][k + 1].record(stream)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    per_step = [{name: ev[s][k].elapsed_time(ev[s][k + 1]) for k, (name, _) in enumerate(stages)}
                for s in range(steps)]
    time_stages.per_step = per_step
    stage_ms = {name: sum(p[name] for p in per_step) / steps for name, _ in stages}
    gpu_ms = ev[0][0].elapsed_time(ev[steps - 1][len(stages)]) / steps
    return stage_ms, gpu_ms, wall


FWD_STAGES = ("project", "attend")
BWD_STAGES = ("prepare", "passes", "query_pass", "key_pass", "contract")


def spread(per_step):
    """Median and minimum over the timed steps of the step, its forward and
    its backward (ms)."""
    import statistics
    out = {}
    for key, names in (("step", None), ("fwd", FWD_STAGES), ("bwd", BWD_STAGES)):
        v = [sum(t for n, t in p.items() if names is None or n in names) for p in per_step]
        out[key] = {"median": round(statistics.median(v), 4), "min": round(min(v), 4)}
    return out


def run_sweep(args):
    """The layer benchmark's length sweep: for each mechanism, N from 128 to
    8192 at a fixed budget of 16384 tokens per batch (B = 16384 / N), 12
    heads, d = 64, fp16, bidirectional.  One JSON line per (mechanism, N):
    forward and backward ms, their TFLOP/s (4 d and 10 d per live pair) and
    the device memory allocated beyond the inputs."""
    import torch

    import exact_relative_position_amd._binding as B_
    from relpos_synth import make_inputs, sweep_workloads

    dev = torch.device("cuda:0")
    if args.memory_scaling:
        from relpos_synth import memory_scaling_workloads
        todo = memory_scaling_workloads(args.memory_scaling)
        metric = (f"memory scaling in N ({args.memory_scaling}, 1x12xN fp16): fwd and bwd ms, "
                  "extra memory")
    else:
        mechs = None if args.sweep == "all" else set(args.sweep.split(","))
        todo = {n: w for n, w in sweep_workloads().items()
                if mechs is None or n.split("_")[0] in mechs}
        metric = "layer sweep: fwd and bwd ms, TFLOP/s, extra memory"
    for name, w in todo.items():
        if args.relation and not (args.relation == 2 and w.has_ak):
            w = w.with_(relation=args.relation)
        x = make_inputs(w)
        t = {k: (None if v is None else v.to(dev)) for k, v in x.items()}
        torch.cuda.synchronize(dev)
        mem_inputs = torch.cuda.memory_allocated(dev)
        torch.cuda.reset_peak_memory_stats(dev)
        run = B_.Prepared(t["q"], t["k"], t["v"], t["aq"], t["ak"], t["b"], t["do"], phi=w.phi,
                          tau=w.tau, causal=w.causal, key_len=t["key_len"], keep_z=True,
                          zchunk=w.zchunk, relation=w.relation)
        stage_ms, gpu_ms, _ = time_stages(torch, dev, stage_list(B_, run), args.warmup,
                                          args.steps)
        peak_extra = torch.cuda.max_memory_allocated(dev) - mem_inputs
        mem = measure_peak_memory(torch, dev, t, w, None)
        fwd_ms = stage_ms["project"] + stage_ms["attend"]
        bwd_ms = stage_ms["prepare"] + stage_ms["passes"] + stage_ms["contract"]
        kl = None if x["key_len"] is None else x["key_len"].numpy()
        pairs = live_pairs(w, kl) * w.H
        peak = PEAK_TFLOPS[w.dtype]
        out = {"metric": metric, "config":
               describe(w), "dtype": w.dtype, "fwd_ms": round(fwd_ms, 4),
               "bwd_ms": round(bwd_ms, 4), "ms_per_step": round(gpu_ms, 4),
               "ms_spread": spread(time_stages.per_step),
               "fwd_tflops": round(4.0 * w.d * pairs / (fwd_ms * 1e-3) / 1e12, 2),
               "bwd_tflops": round(10.0 * w.d * pairs / (bwd_ms * 1e-3) / 1e12, 2),
               "fwd_pct_peak": round(100.0 * 4.0 * w.d * pairs / (fwd_ms * 1e-3) / 1e12 / peak,
                                     2),
               "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()},
               "peak_extra_bytes": int(peak_extra),
               "peak_extra_bytes_fwd": mem["fwd"], "peak_extra_bytes_bwd": mem["bwd"],
               "steps": args.steps, "warmup": args.warmup}
        print(json.dumps(out), flush=True)
        del run, t, x
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="shaw_n8192_f16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--separate-passes", action="store_true",
                    help="time the query and key passes as two launches (diagnostic)")
    ap.add_argument("--sweep", default=None, metavar="MECHS",
                    help="instead of the one-line step benchmark, run the layer sweep "
                         "(N = 128 .. 8192 at 16384 tokens) for 'all' or a comma list of "
                         "shaw, txl, deberta, t5; one JSON line per point")
    ap.add_argument("--memory-scaling", nargs="?", const="shaw", default=None,
                    metavar="MECH",
                    help="instead of the one-line step benchmark, run the Shaw workload "
                         "(1x12xN fp16; or 'txl': the Transformer-XL identity map at that "
                         "shape with its projection computed 1024 queries at a time) at "
                         "N = 1K .. 16K; one JSON line per N with the memory allocated "
                         "beyond the inputs")
    ap.add_argument("--zchunk", type=int, default=0,
                    help="compute the query-side projection this many queries at a time "
                         "(a multiple of 128; 0 = the whole sequence)")
    ap.add_argument("--relation", type=int, default=0, choices=(0, 1, 2),
                    help="how the forward gets the query-side relation term: 0 by sequence "
                         "length (default), 1 stored projection, 2 computed in each block")
    ap.add_argument("--dropout", type=float, default=0.0, metavar="P",
                    help="attention dropout probability (fp16/bf16; rounded to a multiple "
                         "of 1/256; generator seed 2024, offset 0)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run one plain copy of this many MiB before the warmup "
                         "(calibration of HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path is a "
              "single-device operator and no multi-GPU figure is produced.", file=sys.stderr)
        sys.exit(2)
    if args.sweep or args.memory_scaling:
        run_sweep(args)
        return

    import torch

    import exact_relative_position_amd._binding as B_
    from relpos_synth import WORKLOADS, make_inputs

    if args.workload in WORKLOADS:
        w = WORKLOADS[args.workload]
    else:
        from relpos_synth import sweep_workloads
        sweep = sweep_workloads()
        if args.workload not in sweep:
            sys.exit(f"unknown workload {args.workload!r}")
        w = sweep[args.workload]
    if args.zchunk:
        w = w.with_(name=f"{w.name}_chunk{args.zchunk}", zchunk=args.zchunk)
    if args.relation:
        w = w.with_(name=f"{w.name}_rel{args.relation}", relation=args.relation)
    t_drop = int(round(args.dropout * 256))
    if t_drop > 0:
        w = w.with_(name=f"{w.name}_dropout{t_drop}", dropout=(t_drop, 2024, 0))
    dev = torch.device("cuda:0")
    x = make_inputs(w)
    if args.copy_probe_mib > 0:
        copy_probe(torch, dev, args.copy_probe_mib)
    t = {k: (None if v is None else v.to(dev)) for k, v in x.items()}
    torch.cuda.synchronize(dev)
    mem_inputs = torch.cuda.memory_allocated(dev)
    torch.cuda.reset_peak_memory_stats(dev)

    drop = None if w.dropout is None else (w.dropout[0] / 256.0, w.dropout[1], w.dropout[2])
    run = B_.Prepared(t["q"], t["k"], t["v"], t["aq"], t["ak"], t["b"], t["do"], phi=w.phi,
                      tau=w.tau, causal=w.causal, key_len=t["key_len"], keep_z=True,
                      dropout=drop, zchunk=w.zchunk, relation=w.relation)
    stages = stage_list(B_, run, args.separate_passes)
    stage_ms, gpu_ms, wall = time_stages(torch, dev, stages, args.warmup, args.steps)
    peak_extra = torch.cuda.max_memory_allocated(dev) - mem_inputs
    K = args.steps
    fwd_ms = stage_ms["project"] + stage_ms["attend"]
    bwd_ms = sum(stage_ms[n] for n in ("prepare", "passes", "query_pass", "key_pass", "contract")
                 if n in stage_ms)

    mem = measure_peak_memory(torch, dev, t, w, drop)
    kl = None if x["key_len"] is None else x["key_len"].numpy()
    pairs = live_pairs(w, kl) * w.H
    d = w.d
    useful = 14.0 * d * pairs
    value = useful / (gpu_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    # Useful work per launch (FlashAttention convention, the same count the
    # pages' equal-useful-work comparison implies): forward 4 d flops per live
    # pair (S and P V), backward 10 d (S recomputed once, dP, dV, dQ, dK).
    # The two-pass backward executes 14 d (the key pass recomputes S and dP),
    # reported separately as executed work.
    kern_flops = {"attend": 4.0 * d * pairs, "passes": 10.0 * d * pairs}
    kern_exec = {"attend": 4.0 * d * pairs, "passes": 14.0 * d * pairs,
                 "query_pass": 6.0 * d * pairs, "key_pass": 8.0 * d * pairs}
    kern_name = {"attend": "fwd_kernel", "passes": "bwd_kernel", "query_pass": "bwd_kernel",
                 "key_pass": "bwd_kernel"}
    if "passes" not in stage_ms:
        # --separate-passes: the two launches together are the backward
        stage_ms["passes"] = stage_ms["query_pass"] + stage_ms["key_pass"]
        kern_exec["passes"] = kern_exec["query_pass"] + kern_exec["key_pass"]
    dom = max(("attend", "passes"), key=lambda n: stage_ms[n])
    achieved = kern_flops[dom] / (stage_ms[dom] * 1e-3) / 1e12

    # projection pass: algorithmic bytes = the fp32 window entries written
    # (live columns only, not the row padding of the buffer) + X and the
    # table read once
    zbytes = run.zs.numel() if run.zs is not None else 0
    proj = None
    if zbytes:
        nt = int(w.has_aq) + int(w.has_ak)
        zlive = 4 * w.B * w.H * (window_columns(w) * int(w.has_aq)
                                 + window_columns(w, key_side=True) * int(w.has_ak))
        R = B_.phi_info(w.phi, w.N)[0]
        tab = (1 if w.shared_tables else w.H) * R * d * t["q"].element_size() * nt
        rd = t["q"].numel() * t["q"].element_size() * nt + tab
        proj = {"GB/s": round((zlive + rd) / (stage_ms["project"] * 1e-3) / 1e9, 1),
                "frac_hbm": round((zlive + rd) / (stage_ms["project"] * 1e-3) / 1e9
                                  / HBM_PEAK_GBS, 4),
                "bytes": int(zlive + rd), "z_bytes": int(zlive),
                "ms": round(stage_ms["project"], 4)}

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(gpu_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded normal inputs of the workload's shape and scales)",
        "config": describe(w),
        "fwd_ms": round(fwd_ms, 4),
        "bwd_ms": round(bwd_ms, 4),
        "ms_spread": spread(time_stages.per_step),
        "wall_ms_per_step": round(wall * 1e3 / K, 4),
        "pct_peak": round(100.0 * value / peak, 2),
        "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "projection": proj,
        "peak_extra_bytes": int(peak_extra),
        "peak_extra_bytes_fwd": mem["fwd"],
        "peak_extra_bytes_bwd": mem["bwd"],
        "fwd_pct_peak": round(100.0 * kern_flops["attend"] / (fwd_ms * 1e-3) / 1e12 / peak, 2),
        "attend_pct_peak": round(100.0 * kern_flops["attend"] / (stage_ms["attend"] * 1e-3)
                                 / 1e12 / peak, 2),
        "roofline": {"bound": "mfma", "kernel": kern_name[dom], "achieved": round(achieved, 2),
                     "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": measured_traffic(kern_name[dom], w.name),
                     "flops_per_launch": kern_flops[dom],
                     "flops_executed_per_launch": kern_exec[dom],
                     "frac_executed": round(kern_exec[dom] / (stage_ms[dom] * 1e-3) / 1e12
                                            / peak, 4),
                     "ms_per_launch": round(stage_ms[dom], 4)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, x)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
