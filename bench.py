#!/usr/bin/env python3
"""Benchmark of the gated delta rule hot path on one MI355X.

One step = one forward (saving its context) + one backward over one batch of
the layer shape B=8, H=16, T=4096, d_k=d_v=56, bf16 q/k/v/do, fp32 gates and
state, chunk 64, seeded synthetic inputs (gdn_inputs, workload
"fwdbwd_model"), all resident in HBM before timing starts.

Prints one JSON line with whole-step throughput (tokens/s), the roofline of
the dominant kernel (per-kernel durations measured here with HIP events
around every library launch) and the fp64 CPU oracle timed on a bounded
sample of the same workload on this host's cores.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--no-decode]

The line also carries "forward": the inference forward alone at the same
shape (no context saved; "state_only_*" times the same pass without the
outputs, as a prefill that only needs the final state), and "decode_step": the single-token state update on its own
workload (256 sequences x 16 heads x d 56, 1024 consecutive steps, fp32 state
carried in place, fresh bf16 tokens per step), timed as one captured HIP graph
of the 1024 launches, with the step kernel's HBM roofline; "mtp3_*" runs the
same tokens three per call (the state read and written once per 3 tokens).

Profiling aids (the counter runs behind the committed traffic summaries):
    python bench.py --profile-run N      N untimed steps, then one plain
                                         256 MiB device copy (the calibration
                                         kernel for the HBM byte counters)
    python bench.py --traffic-summary FETCH_DIR WRITE_DIR
                                         turn two rocprofv3 --pmc runs
                                         (FETCH_SIZE, then WRITE_SIZE) of the
                                         above into per-kernel HBM traffic,
                                         written to profiles/
    python bench.py --mfma-summary DIR   per-kernel MFMA busy % and flops from
                                         one --pmc run of MFMA_COUNTERS
    python bench.py --trace-summary KT_DIR KT_LOG BENCH_LOG
                                         kernel-trace tables of the fwd+bwd and
                                         decode workloads from one
                                         rocprofv3 --kernel-trace --stats run
                                         (KT_DIR, its printed line in KT_LOG)
                                         and a bench.py run without the
                                         profiler (BENCH_LOG)
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
WORKLOAD = "fwdbwd_model"
C = 64

# Kernels in launch order within one step (forward with context, backward).
KERNELS = ["fwd_prep", "fwd_chain", "bwd_chain", "bwd_local", "dA_reduce"]


def kernel_bytes_per_token_head(d):
    """Algorithmic HBM bytes per (token, head) of each kernel: the bytes of
    the operation's own inputs it must read and outputs it must write (bf16
    q/k/v/o/do/dq/dk/dv of d elements, fp32 g/beta/dg/dbeta); workspace and
    context traffic is implementation cost and is not counted."""
    e = 2 * d
    return {
        "fwd_prep": 2 * e + 8,          # k, v, g, beta
        "fwd_chain": 2 * e + 4 + e,     # q, k, g -> o
        "bwd_chain": 3 * e + 4,         # q, k, do, g
        "bwd_local": 4 * e + 8 + 3 * e + 8,  # q, k, v, do, g, beta -> dq, dk, dv, dg, dbeta
        "dA_reduce": 0,
    }


def step_model(B, T, H, d):
    """Algorithmic FLOPs and HBM bytes of one forward + backward (chunk-form
    FLOP count per chunk-head: fwd 10C^2d + 6Cd^2 + C^3/3, bwd 20C^2d +
    12Cd^2 + 4C^3; bytes: read q,k,v,do,g,beta,h0 and write o,hT,dq,dk,dv,
    dg,dbeta,dA_log,dh0 once each)."""
    nch = B * H * ((T + C - 1) // C)
    flops = nch * ((10 * C * C * d + 6 * C * d * d + C ** 3 / 3) + (20 * C * C * d + 12 * C * d * d + 4 * C ** 3))
    th = B * T * H
    e = 2 * d
    fwd_bytes = th * (3 * e + 8 + e) + B * H * d * d * 4 * 2  # + h0 read, hT write
    bwd_bytes = th * (4 * e + 8 + 3 * e + 8) + B * H * d * d * 4 * 2 + H * 4
    return flops, fwd_bytes + bwd_bytes


# translation unit of each timed kernel; every kernel also depends on the
# shared headers and on the launch code of the C ABI
KERNEL_SOURCE = {"fwd_prep": "gdn_fwd.hip", "fwd_chain": "gdn_fwd.hip", "bwd_chain": "gdn_bwd.hip",
                 "bwd_local": "gdn_bwd.hip", "dA_reduce": "gdn_bwd.hip"}
SHARED_SOURCES = ("gdn_common.hpp", "gdn_launch.hpp", "gdn_api.cpp")


def source_hash(kernel=None):
    """Hash of the sources a kernel is built from (all library sources when
    kernel is None): a stored counter reading is used only while it matches."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gated_delta_rule_74_amd", "csrc")
    files = sorted(os.listdir(csrc)) if kernel is None else sorted((KERNEL_SOURCE[kernel],) + SHARED_SOURCES)
    for f in files:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel):
    """HBM traffic of a kernel from the committed counter summary, if it was
    taken on the current kernel sources; else None."""
    p = os.path.join(ROOT, "profiles", f"{kernel}_{WORKLOAD}_traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("source_hash") != source_hash(kernel):
        return None
    return t.get("traffic_bytes")


COPY_BYTES = 256 << 20  # calibration copy of --profile-run


def _counter_rows(d):
    """(kernel name, counter, value) of every dispatch in a rocprofv3 csv dir."""
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    out = []
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                out.append((r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"]), r["Dispatch_Id"]))
    return out


def _per_kernel(rows, counter):
    """Per-dispatch values of `counter` (summed over its instances) by kernel."""
    import collections
    per_disp = collections.defaultdict(float)
    name_of = {}
    for name, cn, val, disp in rows:
        if cn.startswith(counter):
            per_disp[disp] += val
            name_of[disp] = name
    by_kernel = collections.defaultdict(list)
    for disp, v in per_disp.items():
        by_kernel[name_of[disp]].append(v)
    return by_kernel


def traffic_summary(fetch_dir, write_dir):
    """HBM bytes per launch of every gdn kernel from FETCH_SIZE / WRITE_SIZE
    (KiB per dispatch), each scaled by the reading of the same counter for the
    plain 256 MiB copy (expected bytes / counted bytes)."""
    fetch_all = _per_kernel(_counter_rows(fetch_dir), "FETCH_SIZE")
    write_all = _per_kernel(_counter_rows(write_dir), "WRITE_SIZE")

    def copy_of(tab):
        # the largest dispatch of the runtime's copy kernel is the 256 MiB copy
        cands = [max(v) for k, v in tab.items() if "copy" in k.lower() and "gdn" not in k]
        if not cands:
            raise SystemExit("calibration copy kernel not found in the counter output")
        return max(cands)

    def avg(tab):
        return {k: sum(v) / len(v) for k, v in tab.items()}

    fetch, write = avg(fetch_all), avg(write_all)

    f_scale = COPY_BYTES / (copy_of(fetch_all) * 1024.0)
    w_scale = COPY_BYTES / (copy_of(write_all) * 1024.0)
    out = {}
    for k in KERNELS:
        src = source_hash(k)
        fk = [v for n, v in fetch.items() if f"gdn::{k}_kernel" in n or f"gdn::{k}" in n]
        wk = [v for n, v in write.items() if f"gdn::{k}_kernel" in n or f"gdn::{k}" in n]
        if not fk or not wk:
            continue
        rd, wr = fk[0] * 1024.0 * f_scale, wk[0] * 1024.0 * w_scale
        rec = {"kernel": k, "workload": WORKLOAD, "source_hash": src,
               "fetch_kib_per_dispatch": round(fk[0], 1), "write_kib_per_dispatch": round(wk[0], 1),
               "copy_fetch_scale": round(f_scale, 4), "copy_write_scale": round(w_scale, 4),
               "read_bytes": round(rd), "write_bytes": round(wr), "traffic_bytes": round(rd + wr)}
        with open(os.path.join(ROOT, "profiles", f"{k}_{WORKLOAD}_traffic.json"), "w") as fh:
            json.dump(rec, fh, indent=1)
        out[k] = rec
    cfg_bytes = kernel_bytes_per_token_head(56)
    launches = {"fwd_prep": 4, "fwd_chain": 4}
    lines = [
        f"# HBM traffic per launch, workload {WORKLOAD} (B=8, H=16, T=4096, d=56, bf16), one MI355X",
        "#",
        "# commands (from /tmp on the GPU host, TMPDIR=/tmp), one counter per run:",
        "#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d <fetch> -o p -- python3 <repo>/bench.py --profile-run 2",
        "#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d <write> -o p -- python3 <repo>/bench.py --profile-run 2",
        "#   python3 <repo>/bench.py --traffic-summary <fetch> <write>   (writes this file and the *_traffic.json)",
        "#",
        "# Calibration: --profile-run ends with one plain 256 MiB device-to-device copy;",
        f"# its counters give scale factors {f_scale:.2f} (FETCH_SIZE) and {w_scale:.2f} (WRITE_SIZE),",
        "# applied to every kernel below. The forward launches prep and its serial pass once per",
        "# chunk range (4 per step); the backward kernels once per step.",
        "",
        f"{'kernel':12s} {'launches':>8s} {'fetch KiB':>10s} {'write KiB':>10s} {'read MB':>8s} {'write MB':>9s}"
        f" {'total MB':>9s} {'algorithmic MB':>15s} {'ratio':>6s}  source_hash",
    ]
    for k, rec in out.items():
        nl = launches.get(k, 1)
        alg = cfg_bytes[k] * 8 * 4096 * 16 / nl / 1e6
        tot = rec["traffic_bytes"] / 1e6
        ratio = f"{tot / alg:6.2f}" if alg > 0 else "   nan"
        lines.append(f"{k:12s} {nl:8d} {rec['fetch_kib_per_dispatch']:10.1f} {rec['write_kib_per_dispatch']:10.1f}"
                     f" {rec['read_bytes'] / 1e6:8.1f} {rec['write_bytes'] / 1e6:9.1f} {tot:9.1f} {alg:15.1f}"
                     f" {ratio}  {rec['source_hash']}")
    lines += ["", "# algorithmic = the operation's own inputs and outputs only (kernel_bytes_per_token_head);",
              "# the rest is the library's own context and workspace traffic (U, -Kw, Tm, chunk states,",
              "# dh per chunk, the decay) plus partially used cache lines."]
    with open(os.path.join(ROOT, "profiles", f"traffic_{WORKLOAD}.txt"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(json.dumps(out, indent=1))


def forward_bench(gi, to_dev, dev, steps, warmup):
    """The inference forward at the layer shape (workload fwd_model: B=8,
    H=16, T=4096, d 56, bf16, zero initial state, final state returned, no
    context saved for a backward)."""
    import torch

    import gated_delta_rule_74_amd as gdn

    c = gi.CONFIGS["fwd_model"]
    x = gi.gen_config("fwd_model")
    q, k, v, g, beta, A_log = (to_dev(x[n]) for n in ("q", "k", "v", "g", "beta", "A_log"))
    o = torch.empty_like(v)
    hT = torch.empty(c.B, c.H, c.dk, c.dv, dtype=torch.float32, device=dev)
    ws = torch.empty(gdn.fwd_workspace_size(q, v), dtype=torch.uint8, device=dev)

    def fwd():
        gdn.fwd(q, k, v, g, beta, A_log, None, o=o, hT=hT, workspace=ws, save_context=False)

    def prefill():  # state-only pass: the final state without the outputs
        gdn.fwd(q, k, v, g, beta, A_log, None, hT=hT, workspace=ws, save_context=False, want_o=False)

    def timed(f):
        for _ in range(warmup):
            f()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            f()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    ms = timed(fwd)
    ms_state = timed(prefill)
    nch = c.B * c.H * ((c.T + C - 1) // C)
    d = c.dk
    flops = nch * (10 * C * C * d + 6 * C * d * d + C ** 3 / 3)
    nbytes = c.B * c.T * c.H * (4 * 2 * d + 8) + c.B * c.H * d * d * 4  # q,k,v in, o out, g,beta; hT
    return {"workload": "fwd_model", "B": c.B, "H": c.H, "T": c.T, "d_k": c.dk, "d_v": c.dv,
            "ms": round(ms, 4), "tokens_per_s": c.B * c.T / (ms * 1e-3),
            "hbm_bytes": nbytes, "hbm_frac": round(nbytes / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
            "flops": flops, "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
            "mfma_frac": round(flops / (ms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12), 4),
            "state_only_ms": round(ms_state, 4),
            "state_only_tokens_per_s": c.B * c.T / (ms_state * 1e-3)}


def decode_bytes_per_step(N, H, dk, dv, S=1):
    """Algorithmic HBM bytes of one decode call of S tokens: the fp32 state
    read and written once, bf16 q, k, v read and o written and fp32 g and
    beta read for every token."""
    return N * H * (2 * dk * dv * 4 + S * ((2 * dk + dv) * 2 + dv * 2 + 8))


def decode_bench(dev, n_sets_cold=6):
    """The decode workload: 1024 consecutive single-token steps of 256
    sequences x 16 heads from a carried state, and the same tokens as 341
    steps of 3 tokens (a multi-token prediction's draft verified per step).
    Hot: one state set updated in place (51 MB, which the 256 MB Infinity
    Cache can hold between steps). Cold: n_sets_cold independent state sets
    served round-robin (> 256 MB), so each step's state comes from HBM."""
    import numpy as np
    import torch

    import gated_delta_rule_74_amd as gdn
    import gdn_inputs as gi

    cfg = gi.CONFIGS["decode_step"]
    N, H, dk, dv, T = cfg.B, cfg.H, cfg.dk, cfg.dv, cfg.steps
    x = gi.gen_decode(N, H, dk, dv, T, cfg.dtype, seed=cfg.seed)

    def to_dev(a):
        if isinstance(a, gi.Tensor):
            return torch.from_numpy(a.data.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    q, k, v, g, beta, A_log, h0 = (to_dev(x[n]) for n in ("q", "k", "v", "g", "beta", "A_log", "h0"))
    del x

    def tokens_of(S):
        """[steps, N, S, H, *] copies of the first steps * S tokens."""
        n = T // S
        grp = lambda t: t[: n * S].reshape(n, S, *t.shape[1:]).transpose(1, 2).contiguous()
        return n, [grp(t) for t in (q, k, v, g, beta)]

    def run(n_sets, S):
        n_steps, (qs, ks, vs, gs, bs) = tokens_of(S) if S > 1 else (T, (q, k, v, g, beta))
        o = torch.empty((N, S, H, dv) if S > 1 else (N, H, dv), dtype=q.dtype, device=dev)

        def chain(hs):
            for t in range(n_steps):
                h = hs[t % len(hs)]
                if S > 1:
                    gdn.step_tokens(qs[t], ks[t], vs[t], gs[t], bs[t], A_log, h, h, o=o)
                else:
                    gdn.step(qs[t], ks[t], vs[t], gs[t], bs[t], A_log, h, h, o=o)

        hs = [h0.clone() for _ in range(n_sets)]
        # eager reference of one pass, then the same pass as one graph replay
        chain(hs)
        torch.cuda.synchronize()
        ref = [h.clone() for h in hs]
        graph = None
        try:
            for h in hs:
                h.copy_(h0)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                chain(hs)
            for h in hs:
                h.copy_(h0)
            graph.replay()
            torch.cuda.synchronize()
            if not all(torch.equal(a, b) for a, b in zip(hs, ref)):
                graph = None
        except RuntimeError:
            graph = None
        for _ in range(2):  # warm
            graph.replay() if graph else chain(hs)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        graph.replay() if graph else chain(hs)
        e1.record()
        torch.cuda.synchronize()
        total_ms = e0.elapsed_time(e1)
        # the kernel's duration is taken as the whole chain's time per call
        # (gaps between the graph's launches included, so an upper bound):
        # events around each ~20 us launch would add their own overhead
        kern_ms = total_ms / n_steps
        nbytes = decode_bytes_per_step(N, H, dk, dv, S)
        achieved = nbytes / (kern_ms * 1e-3) / 1e9
        return {"state_sets": n_sets, "tokens_per_call": S, "graph": graph is not None,
                "us_per_step": round(total_ms * 1e3 / n_steps, 3),
                "tokens_per_s": N * n_steps * S / (total_ms * 1e-3),
                "roofline": {"bound": "hbm", "kernel": "gdn_step", "achieved": round(achieved, 1),
                             "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                             "bytes_per_launch": nbytes, "avg_launch_ms": round(kern_ms, 5),
                             "timing": f"graph of {n_steps} launches, per launch"}}

    out = {"workload": "decode_step", "sequences": N, "heads": H, "d_k": dk, "d_v": dv, "steps": T,
           "dtype": "bf16 tokens, fp32 state", "hot": run(1, 1), "cold": run(n_sets_cold, 1)}
    out["mtp3_hot"] = run(1, 3)
    out["mtp3_cold"] = run(n_sets_cold, 3)
    return out


MFMA_COUNTERS = "SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F32 GRBM_GUI_ACTIVE"
SIMD_NUM = 256 * 4  # MI355X: 256 compute units x 4 SIMDs
XCD_NUM = 8         # GRBM_GUI_ACTIVE comes summed over the 8 XCDs


def _last_json(path):
    with open(path) as f:
        return json.loads([ln for ln in f if ln.startswith("{")][-1])


def trace_summary(kt_dir, kt_log, bench_log):
    """Write profiles/kernel_trace_{fwdbwd_model,decode_step}.txt from the
    kernel statistics of a rocprofv3 --kernel-trace --stats run of bench.py
    (KT_DIR, with the run's own JSON line in KT_LOG) and the JSON line of a
    bench.py run without the profiler (BENCH_LOG)."""
    import csv
    import glob

    b, k = _last_json(bench_log), _last_json(kt_log)
    stats = glob.glob(os.path.join(kt_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not stats:
        raise SystemExit(f"no kernel_stats.csv under {kt_dir}")
    with open(stats[0]) as f:
        rows = list(csv.DictReader(f))
    cmd = ["#   cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats --output-format csv \\",
           "#     -d <out> -o bench -- python3 <repo>/bench.py --steps 10 --warmup 2 --no-cpu-baseline > <kt.log>",
           "#   python3 <repo>/bench.py > <bench.log>   (no profiler)",
           "#   python3 <repo>/bench.py --trace-summary <out> <kt.log> <bench.log>   (writes this file)"]

    def table(keep):
        out = [f"{'kernel':72s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s}"]
        for r in rows:
            if keep(r["Name"]):
                out.append(f"{r['Name'][:72]:72s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.1f}"
                           f" {float(r['MinNs']) / 1e3:9.1f} {float(r['MaxNs']) / 1e3:9.1f}")
        return out

    f, rl = b["forward"], b["roofline"]
    lines = ["# Kernel trace: gated delta rule fwd+bwd step, workload fwdbwd_model",
             "# (B=8, H=16, T=4096, d_k=d_v=56, bf16, chunk 64), one MI355X", "#",
             "# commands (from the repository root, on the GPU host):"] + cmd + [
        "#",
        "# 22 steps = 2 warmup + 10 timed + 10 per-kernel-timed, then the forward-only and decode",
        "# workloads. The forward runs in 4 chunk ranges (prep and serial pass launched 4 times per",
        "# step, prep of the next range overlapping the serial pass of the current one); each backward",
        "# kernel runs once per step. The rows below count every launch of the run (fwd+bwd steps",
        "# and the forward-only timing).",
        f"# the profiled run's own line: {k['ms_per_step']} ms per step; per-kernel HIP-event sums per step:"
        f" {k['kernels_ms']}",
        f"# bench.py without the profiler (separate run, 20 steps): {b['ms_per_step']} ms per step,"
        f" {b['value']:.4g} tokens/s;",
        f"#   per-kernel sums per step {b['kernels_ms']}",
        f"#   dominant kernel bwd_local: {rl['avg_launch_ms']} ms per launch, {rl['achieved']} GB/s algorithmic"
        f" = {rl['frac'] * 100:.1f} % of 8 TB/s",
        f"#   forward alone (fwd_model, no context): {f['ms']} ms = {f['tokens_per_s']:.4g} tokens/s,"
        f" {f['hbm_frac'] * 100:.1f} % of HBM, {f['tflops']} TFLOP/s",
        ""] + table(lambda n: "gdn::" in n and "step_" not in n)
    with open(os.path.join(ROOT, "profiles", "kernel_trace_fwdbwd_model.txt"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    d = b["decode_step"]
    lines = ["# Kernel trace: decode step, workload decode_step",
             "# (256 sequences x 16 heads, d_k=d_v=56, bf16 tokens, fp32 state in place, 1024 consecutive"
             " tokens), one MI355X", "#",
             "# commands (the same runs as kernel_trace_fwdbwd_model.txt; bench.py times the decode workload"
             " after the fwd+bwd step):"] + cmd + [
        "#",
        "# bench.py runs the 1024 single-token steps for one state set (hot: 51 MB, held by the 256 MB"
        " Infinity Cache)",
        "# and for 6 state sets served round-robin (cold: 308 MB), then the same tokens as 341 calls of 3"
        " tokens",
        "# (gdn_step_tokens); per variant an eager pass, a captured graph checked bitwise against it, 2 warm",
        "# replays and 1 timed replay. step_kernel<..., true> is the one-token instance, step_pre_kernel the"
        " 3-token calls.",
        f"# bench.py without the profiler: hot {d['hot']['us_per_step']} us per step ="
        f" {d['hot']['roofline']['achieved']} GB/s ({d['hot']['roofline']['frac'] * 100:.1f} % of 8 TB/s),",
        f"#   cold {d['cold']['us_per_step']} us per step = {d['cold']['roofline']['achieved']} GB/s"
        f" ({d['cold']['roofline']['frac'] * 100:.1f} %), {d['hot']['roofline']['bytes_per_launch']}"
        " algorithmic bytes per step;",
        f"#   3 tokens per call: hot {d['mtp3_hot']['us_per_step']} us = {d['mtp3_hot']['tokens_per_s']:.4g}"
        f" tokens/s, cold {d['mtp3_cold']['us_per_step']} us = {d['mtp3_cold']['tokens_per_s']:.4g} tokens/s",
        ""] + table(lambda n: "gdn::step_" in n)
    with open(os.path.join(ROOT, "profiles", "kernel_trace_decode_step.txt"), "w") as fh:
        fh.write("\n".join(lines) + "\n")


def mfma_summary(counter_dir):
    """MFMA use per kernel from one rocprofv3 --pmc run of the counters in
    MFMA_COUNTERS over `bench.py --profile-run N`: busy % = MFMA busy cycles
    summed over SIMDs / (active cycles of one XCD x SIMDs); MFMA flops =
    MFMA ops x 512 (the counters count ops in units of 512); TFLOP/s over the
    dispatch's own start and end timestamps; all averaged over launches."""
    import collections
    import csv
    import glob

    per = collections.defaultdict(dict)
    name = {}
    for f in glob.glob(os.path.join(counter_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                d = r["Dispatch_Id"]
                per[d][r["Counter_Name"]] = per[d].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
                per[d]["ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
                name[d] = r["Kernel_Name"]
    nch = 8 * 16 * 64
    d = 56
    alg = {"fwd_prep": nch * (4 * C * C * d + C ** 3 / 3) / 4,  # K K^T, U, Kw, inverse; 4 launches
           "fwd_chain": nch * (6 * C * C * d + 6 * C * d * d) / 4,
           "bwd_chain": nch * (2 * C * C * d + 6 * C * d * d),
           "bwd_local": nch * (18 * C * C * d + 6 * C * d * d + 4 * C ** 3)}
    lines = [
        f"# MFMA use per launch, workload {WORKLOAD} (B=8, H=16, T=4096, d=56, bf16), one MI355X",
        "#",
        "# command (from /tmp on the GPU host, TMPDIR=/tmp):",
        f"#   rocprofv3 --pmc {MFMA_COUNTERS} --output-format csv -d <dir> -o p -- python3 <repo>/bench.py --profile-run 2",
        "#   python3 <repo>/bench.py --mfma-summary <dir>   (writes this file)",
        "#",
        f"# busy % = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {XCD_NUM} XCDs x {SIMD_NUM} SIMDs);",
        "# MFMA flops = (MOPS_BF16 + MOPS_F32) x 512, which counts the padding of d = 56 to 64 and the",
        "# masked halves of the 64 x 64 products; TFLOP/s over each dispatch's own duration (profiled);",
        "# algorithmic flops = the chunk-form count of the kernel's products per launch.",
        f"# source_hash {source_hash()}",
        "",
        f"{'kernel':12s} {'launches':>8s} {'busy %':>7s} {'bf16 GFLOP':>11s} {'fp32 GFLOP':>11s} {'alg. GFLOP':>11s}"
        f" {'us':>8s} {'MFMA TFLOP/s':>13s}",
    ]
    for k in KERNELS:
        ds = [x for x in per if f"gdn::{k}" in name[x]]
        if not ds:
            continue
        mean = lambda key: sum(per[x].get(key, 0.0) for x in ds) / len(ds)
        act = mean("GRBM_GUI_ACTIVE") / XCD_NUM
        util = 100.0 * mean("SQ_VALU_MFMA_BUSY_CYCLES") / (act * SIMD_NUM) if act > 0 else float("nan")
        fb, ff = mean("SQ_INSTS_VALU_MFMA_MOPS_BF16") * 512, mean("SQ_INSTS_VALU_MFMA_MOPS_F32") * 512
        ns = mean("ns")
        lines.append(f"{k:12s} {len(ds):8d} {util:7.2f} {fb / 1e9:11.3f} {ff / 1e9:11.3f} {alg.get(k, 0) / 1e9:11.3f}"
                     f" {ns / 1e3:8.1f} {(fb + ff) / (ns * 1e-9) / 1e12:13.1f}")
    with open(os.path.join(ROOT, "profiles", f"mfma_{WORKLOAD}.txt"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cpu_threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def cpu_baseline(x, B, T, H, budget_s):
    """The fp64 oracle (forward + reverse pass) on a bounded sample of the
    workload's (b, h) units, threaded over units."""
    import numpy as np

    import oracle

    oracle.build()
    f = {k: (v.f64() if hasattr(v, "f64") else (None if v is None else np.asarray(v, np.float64)))
         for k, v in x.items()}
    cores = cpu_threads()
    # size the sample from a one-unit probe so the timed run lasts about budget_s
    t0 = time.perf_counter()
    oracle.fwd(f["q"], f["k"], f["v"], f["g"], f["beta"], f["A_log"], f["h0"], units=[0], nthreads=1)
    oracle.bwd(f["q"], f["k"], f["v"], f["g"], f["beta"], f["A_log"], f["h0"], f["do"], units=[0],
               nthreads=1)
    per_unit = time.perf_counter() - t0
    n_units = int(min(B * H, max(cores, round(budget_s * cores / max(per_unit, 1e-6)))))
    n_units = max(1, (n_units // cores) * cores) if n_units >= cores else n_units
    units = list(range(n_units))
    reps = 0
    t0 = time.perf_counter()
    while True:  # repeat a small sample until the time budget is used
        oracle.fwd(f["q"], f["k"], f["v"], f["g"], f["beta"], f["A_log"], f["h0"], units=units,
                   nthreads=cores)
        oracle.bwd(f["q"], f["k"], f["v"], f["g"], f["beta"], f["A_log"], f["h0"], f["do"],
                   units=units, nthreads=cores)
        reps += 1
        wall = time.perf_counter() - t0
        if wall >= budget_s or reps >= 100:
            break
    tokens = reps * n_units * T / H  # one token carries H heads
    return {"value": tokens / wall, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{n_units} of {B * H} (batch, head) units at full T={T}, fwd+bwd in fp64, "
                      f"{reps} pass(es), {wall:.1f} s wall"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--profile-run", type=int, default=0, metavar="N")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--mfma-summary", metavar="COUNTER_DIR")
    ap.add_argument("--trace-summary", nargs=3, metavar=("KT_DIR", "KT_LOG", "BENCH_LOG"))
    args = ap.parse_args()
    if args.trace_summary:
        trace_summary(*args.trace_summary)
        return
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary)
        return
    if args.mfma_summary:
        mfma_summary(args.mfma_summary)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the gated delta rule path here is built and timed "
              "on a single MI355X ((batch, head) units would be split across GPUs with no "
              "communication but one all-reduce of dA_log); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gated_delta_rule_74_amd as gdn
    import gdn_inputs as gi

    cfg = gi.CONFIGS[WORKLOAD]
    B, T, H, dk, dv = cfg.B, cfg.T, cfg.H, cfg.dk, cfg.dv
    x = gi.gen_config(WORKLOAD)
    dev = torch.device("cuda:0")

    def to_dev(a):
        if a is None:
            return None
        if isinstance(a, gi.Tensor):
            return torch.from_numpy(a.data.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    t = {k: to_dev(v) for k, v in x.items()}
    q, k, v, g, beta, A_log, h0, do = (t[n] for n in ("q", "k", "v", "g", "beta", "A_log", "h0", "do"))
    o = torch.empty_like(v)
    hT = torch.empty(B, H, dk, dv, dtype=torch.float32, device=dev)
    ctx = torch.empty(gdn.context_size(q, v), dtype=torch.uint8, device=dev)
    fws = torch.empty(gdn.fwd_workspace_size(q, v), dtype=torch.uint8, device=dev)
    bws = torch.empty(gdn.bwd_workspace_size(q, v), dtype=torch.uint8, device=dev)
    grads = {"dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v),
             "dg": torch.empty_like(g), "dbeta": torch.empty_like(beta),
             "dA_log": torch.empty_like(A_log),
             "dh0": torch.empty(B, H, dk, dv, dtype=torch.float32, device=dev)}

    def step():
        gdn.fwd(q, k, v, g, beta, A_log, h0, o=o, hT=hT, context=ctx, workspace=fws)
        gdn.bwd(q, k, v, g, beta, A_log, do, h0, None, context=ctx, workspace=bws, out=grads)

    if args.profile_run:
        for i in range(args.profile_run):
            step()
            torch.cuda.synchronize()
            print(f"profile step {i + 1}/{args.profile_run}", flush=True)
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"calibration copy of {COPY_BYTES} bytes done", flush=True)
        return

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K whole steps
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - w0
    ms = e0.elapsed_time(e1) / args.steps

    # per-kernel durations: the same steps again with every launch bracketed
    # (a forward may launch its kernels once per chunk range; they are summed
    # per step, and the roofline uses the average single launch)
    timer = gdn.LaunchTimer(64 * args.steps)
    with timer:
        for _ in range(args.steps):
            step()
    d = timer.durations_ms()
    kinds = timer.kinds()
    if not d or len(d) != len(kinds):
        raise RuntimeError("launch bracketing failed")
    per_kernel = {k: 0.0 for k in KERNELS}
    launches = {k: [] for k in KERNELS}
    for name, ms_i in zip(kinds, d):
        per_kernel[name] += ms_i / args.steps
        launches[name].append(ms_i)

    tokens = B * T
    flops, step_bytes = step_model(B, T, H, dk)
    dom = max(per_kernel, key=per_kernel.get)
    n_launch = len(launches[dom]) / args.steps
    kb = kernel_bytes_per_token_head(dk)[dom] * B * T * H / n_launch
    avg_ms = float(np.mean(launches[dom]))
    achieved = kb / (avg_ms * 1e-3) / 1e9
    roof = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": load_traffic(dom), "bytes_per_launch": round(kb),
            "avg_launch_ms": round(avg_ms, 4), "launches_per_step": n_launch}

    out = {
        "metric": "GDN fwd+bwd tokens/s at B8·H16·T4096·d56; % of MFMA/HBM roofline",
        "value": tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded gdn_inputs workload fwdbwd_model)",
        "config": {"workload": WORKLOAD, "B": B, "H": H, "T": T, "d_k": dk, "d_v": dv, "chunk": C,
                   "global_batch": B, "seq_len": T, "parallelism": "none (one GPU)"},
        "roofline": roof,
        "step_roofline": {
            "hbm_bytes": step_bytes, "flops": flops,
            "hbm_frac": round(step_bytes / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
            "mfma_frac": round(flops / (ms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12), 4),
            "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
        },
        "kernels_ms": {k2: round(v2, 4) for k2, v2 in per_kernel.items()},  # summed per step
        "wall_s_timed": round(wall_s, 3),
        "cpu_baseline": None,
    }
    out["forward"] = forward_bench(gi, to_dev, dev, args.steps, args.warmup)
    if not args.no_decode:
        out["decode_step"] = decode_bench(dev)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(x, B, T, H, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
