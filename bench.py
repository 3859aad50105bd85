#!/usr/bin/env python3
"""Benchmark of the gated delta rule hot path on one MI355X.

One step = one forward (saving its context) + one backward over one batch of
the layer shape B=8, H=16, T=4096, d_k=d_v=56, bf16 q/k/v/do, fp32 gates and
state, chunk 64, seeded synthetic inputs (gdn_inputs, workload
"fwdbwd_model"), all resident in HBM before timing starts.

Timing protocol: W untimed warmup steps; then K steps, each preceded (outside
its own pair of HIP events) by a 512 MiB device fill that evicts the L2 and
the 256 MB Infinity Cache, so every step reads its inputs from HBM; the
reported time per step is the median of the K event pairs. The line also
gives the mean and the back-to-back time without the flush.

Prints one JSON line with whole-step throughput (tokens/s), the roofline of
the dominant kernel (per-kernel durations measured here with HIP events
around every library launch) and the fp64 CPU oracle timed on a bounded
sample of the same workload on this host's cores.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--no-decode]
                    [--no-long-ctx] [--workload fwdbwd_model|long_ctx]

Objects on the line besides the headline:
  "forward"      the inference forward alone at the layer shape (no context
                 saved; "state_only_*" times the same pass without outputs)
  "long_ctx"     forward + backward of B=1, H=16, T=32768, d 128 (bf16, h0 =
                 0.1 N(0,1)), same protocol, its own dominant-kernel roofline
  "decode_step"  the single-token state update on its own workload (256
                 sequences x 16 heads x d 56, 1024 consecutive steps, fp32
                 state in place, fresh bf16 tokens per step), timed as one
                 captured HIP graph of the 1024 launches: "cold" (6 state
                 sets served round-robin, > 256 MB, so the state comes from
                 HBM: the HBM roofline) and "hot" (one 51 MB state set that
                 the Infinity Cache holds: cache-resident rate, no HBM
                 fraction); "mtp3_*" three tokens per call
  "stream_copy"  a plain 1 GiB device-to-device copy: the HBM rate the box
                 reaches on a streaming kernel (context, not a denominator)
  "cpu_baseline" the fp64 oracle, fwd+bwd of the headline workload, and
  "oracle_times" its per-configuration timings (fwd, fwd+bwd, the 1024-step
                 decode chain, a one-thread forward)

--workload long_ctx prints only the long-context object (for profiler runs).

Profiling aids (the counter runs behind the committed summaries):
    python bench.py --profile-run N [--workload W]
                                         N untimed steps of workload W, then
                                         one plain 256 MiB device copy (the
                                         calibration kernel for the HBM byte
                                         counters)
    python bench.py --traffic-summary FETCH_DIR WRITE_DIR [--workload W]
                                         turn two rocprofv3 --pmc runs
                                         (FETCH_SIZE, then WRITE_SIZE) of the
                                         above into per-kernel HBM traffic,
                                         written to profiles/
    python bench.py --mfma-summary DIR [--workload W]
                                         per-kernel MFMA busy % and flops from
                                         one --pmc run of MFMA_COUNTERS
    python bench.py --counter-summary DIR1 DIR2 [--workload W]
                                         per-kernel LDS busy and bank-conflict
                                         share, waits and instruction mix from
                                         one --pmc run per COUNTER_PASSES entry
    python bench.py --trace-summary KT_DIR KT_LOG BENCH_LOG [--workload W]
                                         kernel-trace table from one rocprofv3
                                         --kernel-trace --stats run of bench.py
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
HEADLINE = "fwdbwd_model"
C = 64
FLUSH_BYTES = 512 << 20    # larger than the Infinity Cache (256 MB) and the L2s

# Kernels in launch order within one step (forward with context, backward).
KERNELS = ["fwd_prep", "fwd_chain", "fwd_scan", "bwd_chain", "bwd_scan", "bwd_local", "dA_reduce"]


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
        "fwd_scan": 0,
        "bwd_scan": 0,
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


def kernel_flops(B, T, H, d):
    """Algorithmic flops of each kernel per step (the chunk-form counts of
    its products)."""
    nch = B * H * ((T + C - 1) // C)
    return {"fwd_prep": nch * (4 * C * C * d + C ** 3 / 3),  # K K^T, U, Kw, inverse
            "fwd_chain": nch * (6 * C * C * d + 6 * C * d * d),
            "bwd_chain": nch * (2 * C * C * d + 6 * C * d * d),
            "bwd_local": nch * (18 * C * C * d + 6 * C * d * d + 4 * C ** 3)}


# translation unit of each timed kernel; every kernel also depends on the
# shared headers and on the launch code of the C ABI
KERNEL_SOURCE = {"fwd_prep": "gdn_fwd.hip", "fwd_chain": "gdn_fwd.hip", "fwd_scan": "gdn_fwd.hip",
                 "bwd_chain": "gdn_bwd.hip", "bwd_scan": "gdn_fwd.hip", "bwd_local": "gdn_bwd.hip",
                 "dA_reduce": "gdn_bwd.hip"}
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


def load_traffic(kernel, workload):
    """HBM traffic of a kernel from the committed counter summary, if it was
    taken on the current kernel sources; else None."""
    p = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("source_hash") != source_hash(kernel):
        return None
    return t.get("traffic_bytes")


def kernel_of(name):
    """Which timed kernel a device kernel's symbol belongs to (None: not ours)."""
    if "gdn::" not in name:
        return None
    if "gdn::range_scan" in name:  # one kernel serves the scans of both directions
        return "fwd_scan"
    for k in KERNELS:
        if f"gdn::{k}" in name:  # fwd_chain_ws_kernel and bwd_local_wide_kernel included
            return k
    return None


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


def _by_timed_kernel(tab):
    """Group per-dispatch values of device kernels by timed kernel."""
    import collections
    out = collections.defaultdict(list)
    for name, vals in tab.items():
        k = kernel_of(name)
        if k:
            out[k].extend(vals)
    return out


def _workload_text(workload):
    import gdn_inputs as gi
    c = gi.CONFIGS[workload]
    return f"B={c.B}, H={c.H}, T={c.T}, d={c.dk}, {c.dtype}"


def traffic_summary(fetch_dir, write_dir, workload):
    """HBM bytes per launch of every gdn kernel from FETCH_SIZE / WRITE_SIZE
    (KiB per dispatch), each scaled by the reading of the same counter for the
    plain 256 MiB copy (expected bytes / counted bytes)."""
    import gdn_inputs as gi
    fetch_all = _per_kernel(_counter_rows(fetch_dir), "FETCH_SIZE")
    write_all = _per_kernel(_counter_rows(write_dir), "WRITE_SIZE")

    def copy_of(tab):
        # the largest dispatch of the runtime's copy kernel is the 256 MiB copy
        cands = [max(v) for k, v in tab.items() if "copy" in k.lower() and "gdn" not in k]
        if not cands:
            raise SystemExit("calibration copy kernel not found in the counter output")
        return max(cands)

    f_scale = COPY_BYTES / (copy_of(fetch_all) * 1024.0)
    w_scale = COPY_BYTES / (copy_of(write_all) * 1024.0)
    fetch, write = _by_timed_kernel(fetch_all), _by_timed_kernel(write_all)
    steps = len(fetch.get("dA_reduce", [])) or 1  # one dA_log reduction per step
    c = gi.CONFIGS[workload]
    out = {}
    for k in KERNELS:
        if not fetch.get(k) or not write.get(k):
            continue
        fk = sum(fetch[k]) / len(fetch[k])
        wk = sum(write[k]) / len(write[k])
        rd, wr = fk * 1024.0 * f_scale, wk * 1024.0 * w_scale
        rec = {"kernel": k, "workload": workload, "source_hash": source_hash(k),
               "launches_per_step": len(fetch[k]) / steps,
               "fetch_kib_per_dispatch": round(fk, 1), "write_kib_per_dispatch": round(wk, 1),
               "copy_fetch_scale": round(f_scale, 4), "copy_write_scale": round(w_scale, 4),
               "read_bytes": round(rd), "write_bytes": round(wr), "traffic_bytes": round(rd + wr)}
        with open(os.path.join(ROOT, "profiles", f"{k}_{workload}_traffic.json"), "w") as fh:
            json.dump(rec, fh, indent=1)
        out[k] = rec
    cfg_bytes = kernel_bytes_per_token_head(c.dk)
    wl = f" --workload {workload}" if workload != HEADLINE else ""
    lines = [
        f"# HBM traffic per launch, workload {workload} ({_workload_text(workload)}), one MI355X",
        "#",
        "# commands (from /tmp on the GPU host, TMPDIR=/tmp), one counter per run:",
        f"#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d <fetch> -o p -- python3 <repo>/bench.py --profile-run 2{wl}",
        f"#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d <write> -o p -- python3 <repo>/bench.py --profile-run 2{wl}",
        f"#   python3 <repo>/bench.py --traffic-summary <fetch> <write>{wl}   (writes this file and the *_traffic.json)",
        "#",
        "# Calibration: --profile-run ends with one plain 256 MiB device-to-device copy;",
        f"# its counters give scale factors {f_scale:.2f} (FETCH_SIZE) and {w_scale:.2f} (WRITE_SIZE),",
        "# applied to every kernel below (values are averages over the kernel's dispatches).",
        "",
        f"{'kernel':12s} {'launches':>8s} {'fetch KiB':>10s} {'write KiB':>10s} {'read MB':>8s} {'write MB':>9s}"
        f" {'total MB':>9s} {'algorithmic MB':>15s} {'ratio':>6s}  source_hash",
    ]
    for k, rec in out.items():
        nl = rec["launches_per_step"]
        alg = cfg_bytes[k] * c.B * c.T * c.H / nl / 1e6
        tot = rec["traffic_bytes"] / 1e6
        ratio = f"{tot / alg:6.2f}" if alg > 0 else "   nan"
        lines.append(f"{k:12s} {nl:8.0f} {rec['fetch_kib_per_dispatch']:10.1f} {rec['write_kib_per_dispatch']:10.1f}"
                     f" {rec['read_bytes'] / 1e6:8.1f} {rec['write_bytes'] / 1e6:9.1f} {tot:9.1f} {alg:15.1f}"
                     f" {ratio}  {rec['source_hash']}")
    lines += ["", "# algorithmic = the operation's own inputs and outputs only (kernel_bytes_per_token_head);",
              "# the rest is the library's own context and workspace traffic (U, -Kw, Tm, chunk states,",
              "# dh per chunk, the decay) plus partially used cache lines."]
    with open(os.path.join(ROOT, "profiles", f"traffic_{workload}.txt"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(json.dumps(out, indent=1))


# ------------------------------------------------------------------ timing

def _flusher(dev):
    import torch
    buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    return lambda: buf.zero_()


def time_steps(step, steps, warmup, flush):
    """Median / mean of `steps` event-timed calls of step(), each preceded by
    flush() outside its events; also the back-to-back mean without flushes."""
    import numpy as np
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    e1 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for i in range(steps):
        flush()
        e0[i].record()
        step()
        e1[i].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    per = [a.elapsed_time(b) for a, b in zip(e0, e1)]
    b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    b0.record()
    for _ in range(steps):
        step()
    b1.record()
    torch.cuda.synchronize()
    return {"median": float(np.median(per)), "mean": float(np.mean(per)), "min": float(np.min(per)),
            "warm": b0.elapsed_time(b1) / steps, "wall": wall}


def per_kernel_times(step, steps, flush):
    """Per-step sums and per-launch lists of every library kernel's duration,
    from HIP events the library records around each launch (flush between
    the steps, outside the bracketed launches)."""
    import torch

    import gated_delta_rule_74_amd as gdn
    timer = gdn.LaunchTimer(64 * steps)
    with timer:
        for _ in range(steps):
            torch.cuda.synchronize()
            flush()
            step()
    d = timer.durations_ms()
    kinds = timer.kinds()
    if not d or len(d) != len(kinds):
        raise RuntimeError("launch bracketing failed")
    per_kernel = {k: 0.0 for k in KERNELS}
    launches = {k: [] for k in KERNELS}
    for name, ms_i in zip(kinds, d):
        per_kernel[name] += ms_i / steps
        launches[name].append(ms_i)
    return per_kernel, launches


def dominant_roofline(per_kernel, launches, steps, cfg, workload):
    """HBM roofline of the kernel with the largest time per step: algorithmic
    bytes per launch / average launch duration, against 8 TB/s."""
    import numpy as np
    dom = max(per_kernel, key=per_kernel.get)
    n_launch = len(launches[dom]) / steps
    kb = kernel_bytes_per_token_head(cfg.dk)[dom] * cfg.B * cfg.T * cfg.H / n_launch
    avg_ms = float(np.mean(launches[dom]))
    achieved = kb / (avg_ms * 1e-3) / 1e9
    return {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": load_traffic(dom, workload), "bytes_per_launch": round(kb),
            "avg_launch_ms": round(avg_ms, 4), "launches_per_step": n_launch}


def _to_dev(gi, dev):
    import numpy as np
    import torch

    def f(a):
        if a is None:
            return None
        if isinstance(a, gi.Tensor):
            if a.dtype == "bf16":
                return torch.from_numpy(a.data.view(np.int16)).to(dev).view(torch.bfloat16)
            return torch.from_numpy(a.data).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    return f


def seq_workload(workload, dev):
    """Inputs and output buffers of one fwd+bwd workload, all on the device;
    returns (cfg, host inputs, step function)."""
    import torch

    import gated_delta_rule_74_amd as gdn
    import gdn_inputs as gi
    cfg = gi.CONFIGS[workload]
    x = gi.gen_config(workload)
    to_dev = _to_dev(gi, dev)
    t = {k: to_dev(v) for k, v in x.items()}
    q, k, v, g, beta, A_log, h0, do = (t[n] for n in ("q", "k", "v", "g", "beta", "A_log", "h0", "do"))
    B, H, dk, dv = cfg.B, cfg.H, cfg.dk, cfg.dv
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

    return cfg, x, step


def fwdbwd_measure(workload, dev, steps, warmup, flush):
    """Whole-step timing, per-kernel sums and the dominant kernel's roofline
    of one fwd+bwd workload."""
    cfg, x, step = seq_workload(workload, dev)
    t = time_steps(step, steps, warmup, flush)
    per_kernel, launches = per_kernel_times(step, steps, flush)
    ms = t["median"]
    flops, nbytes = step_model(cfg.B, cfg.T, cfg.H, cfg.dk)
    res = {"workload": workload, "B": cfg.B, "H": cfg.H, "T": cfg.T, "d_k": cfg.dk, "d_v": cfg.dv,
           "ms_per_step": round(ms, 4), "ms_mean": round(t["mean"], 4), "ms_min": round(t["min"], 4),
           "ms_warm": round(t["warm"], 4), "tokens_per_s": cfg.B * cfg.T / (ms * 1e-3),
           "step_roofline": {
               "hbm_bytes": nbytes, "flops": flops,
               "hbm_frac": round(nbytes / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
               "mfma_frac": round(flops / (ms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12), 4),
               "tflops": round(flops / (ms * 1e-3) / 1e12, 2)},
           "kernels_ms": {k: round(v, 4) for k, v in per_kernel.items()},
           "roofline": dominant_roofline(per_kernel, launches, steps, cfg, workload)}
    return res, t, x


def forward_bench(dev, steps, warmup, flush):
    """The inference forward at the layer shape (workload fwd_model: B=8,
    H=16, T=4096, d 56, bf16, zero initial state, final state returned, no
    context saved for a backward)."""
    import torch

    import gated_delta_rule_74_amd as gdn
    import gdn_inputs as gi

    c = gi.CONFIGS["fwd_model"]
    x = gi.gen_config("fwd_model")
    to_dev = _to_dev(gi, dev)
    q, k, v, g, beta, A_log = (to_dev(x[n]) for n in ("q", "k", "v", "g", "beta", "A_log"))
    o = torch.empty_like(v)
    hT = torch.empty(c.B, c.H, c.dk, c.dv, dtype=torch.float32, device=dev)
    ws = torch.empty(gdn.fwd_workspace_size(q, v), dtype=torch.uint8, device=dev)

    def fwd():
        gdn.fwd(q, k, v, g, beta, A_log, None, o=o, hT=hT, workspace=ws, save_context=False)

    def prefill():  # state-only pass: the final state without the outputs
        gdn.fwd(q, k, v, g, beta, A_log, None, hT=hT, workspace=ws, save_context=False, want_o=False)

    t = time_steps(fwd, steps, warmup, flush)
    ts = time_steps(prefill, steps, warmup, flush)
    ms, ms_state = t["median"], ts["median"]
    nch = c.B * c.H * ((c.T + C - 1) // C)
    d = c.dk
    flops = nch * (10 * C * C * d + 6 * C * d * d + C ** 3 / 3)
    nbytes = c.B * c.T * c.H * (4 * 2 * d + 8) + c.B * c.H * d * d * 4  # q,k,v in, o out, g,beta; hT
    return {"workload": "fwd_model", "B": c.B, "H": c.H, "T": c.T, "d_k": c.dk, "d_v": c.dv,
            "ms": round(ms, 4), "ms_warm": round(t["warm"], 4), "tokens_per_s": c.B * c.T / (ms * 1e-3),
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
    Cold: n_sets_cold independent state sets served round-robin (> 256 MB),
    so each step's state comes from HBM (the HBM roofline). Hot: one state
    set updated in place (51 MB, which the 256 MB Infinity Cache holds
    between steps): a cache-resident rate, not an HBM fraction. Returns the
    result and the host inputs."""
    import torch

    import gated_delta_rule_74_amd as gdn
    import gdn_inputs as gi

    cfg = gi.CONFIGS["decode_step"]
    N, H, dk, dv, T = cfg.B, cfg.H, cfg.dk, cfg.dv, cfg.steps
    x = gi.gen_decode(N, H, dk, dv, T, cfg.dtype, seed=cfg.seed)
    to_dev = _to_dev(gi, dev)
    q, k, v, g, beta, A_log, h0 = (to_dev(x[n]) for n in ("q", "k", "v", "g", "beta", "A_log", "h0"))

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
        r = {"state_sets": n_sets, "tokens_per_call": S, "graph": graph is not None,
             "us_per_step": round(total_ms * 1e3 / n_steps, 3),
             "tokens_per_s": N * n_steps * S / (total_ms * 1e-3),
             "bytes_per_launch": nbytes, "avg_launch_ms": round(kern_ms, 5),
             "timing": f"graph of {n_steps} launches, per launch"}
        if n_sets > 1:
            r["roofline"] = {"bound": "hbm", "kernel": "gdn_step", "achieved": round(achieved, 1),
                             "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
        else:
            r["cache_resident"] = {"achieved": round(achieved, 1), "unit": "GB/s",
                                   "note": "state held in the Infinity Cache between steps: "
                                           "an effective rate, not an HBM fraction"}
        return r

    out = {"workload": "decode_step", "sequences": N, "heads": H, "d_k": dk, "d_v": dv, "steps": T,
           "dtype": "bf16 tokens, fp32 state", "cold": run(n_sets_cold, 1), "hot": run(1, 1)}
    out["roofline"] = out["cold"]["roofline"]
    out["mtp3_cold"] = run(n_sets_cold, 3)
    out["mtp3_hot"] = run(1, 3)
    return out, x


# ------------------------------------------------------------ summaries

MFMA_COUNTERS = "SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F32 GRBM_GUI_ACTIVE"
SIMD_NUM = 256 * 4  # MI355X: 256 compute units x 4 SIMDs
XCD_NUM = 8         # GRBM_GUI_ACTIVE comes summed over the 8 XCDs


def _last_json(path):
    with open(path) as f:
        return json.loads([ln for ln in f if ln.startswith("{")][-1])


def trace_summary(kt_dir, kt_log, bench_log, workload):
    """Write profiles/kernel_trace_<workload>.txt (and, for the headline
    run, kernel_trace_decode_step.txt) from the kernel statistics of a
    rocprofv3 --kernel-trace --stats run of bench.py (KT_DIR, with the run's
    own JSON line in KT_LOG) and the JSON line of a bench.py run without the
    profiler (BENCH_LOG)."""
    import csv
    import glob

    b, k = _last_json(bench_log), _last_json(kt_log)
    stats = glob.glob(os.path.join(kt_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not stats:
        raise SystemExit(f"no kernel_stats.csv under {kt_dir}")
    with open(stats[0]) as f:
        rows = list(csv.DictReader(f))
    wl = "" if workload == HEADLINE else f" --workload {workload}"
    cmd = ["#   cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats --output-format csv \\",
           f"#     -d <out> -o bench -- python3 <repo>/bench.py --steps 10 --warmup 2 --no-cpu-baseline{wl} > <kt.log>",
           f"#   python3 <repo>/bench.py{wl} > <bench.log>   (no profiler)",
           f"#   python3 <repo>/bench.py --trace-summary <out> <kt.log> <bench.log>{wl}   (writes this file)"]

    def table(keep):
        out = [f"{'kernel':72s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s}"]
        for r in rows:
            if keep(r["Name"]):
                out.append(f"{r['Name'][:72]:72s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.1f}"
                           f" {float(r['MinNs']) / 1e3:9.1f} {float(r['MaxNs']) / 1e3:9.1f}")
        return out

    rl = b["roofline"]
    head = [f"# Kernel trace: gated delta rule fwd+bwd step, workload {workload}",
            f"# ({_workload_text(workload)}, chunk 64), one MI355X", "#",
            "# commands (from the repository root, on the GPU host):"] + cmd + [
        "#",
        "# Every step is preceded by a 512 MiB device fill (cache flush). The rows below count every",
        "# launch of the run (warmup, median-timed, back-to-back and per-kernel-timed steps"
        + (", then the forward-only workload)." if workload == HEADLINE else ")."),
        f"# the profiled run's own line: {k['ms_per_step']} ms per step (median); per-kernel HIP-event sums"
        f" per step: {k['kernels_ms']}",
        f"# bench.py without the profiler (separate run): {b['ms_per_step']} ms per step (median),"
        f" {b['value']:.4g} tokens/s;",
        f"#   per-kernel sums per step {b['kernels_ms']}",
        f"#   dominant kernel {rl['kernel']}: {rl['avg_launch_ms']} ms per launch, {rl['achieved']} GB/s algorithmic"
        f" = {rl['frac'] * 100:.1f} % of 8 TB/s"]
    if workload == HEADLINE:
        f = b["forward"]
        head.append(f"#   forward alone (fwd_model, no context): {f['ms']} ms = {f['tokens_per_s']:.4g} tokens/s,"
                    f" {f['hbm_frac'] * 100:.1f} % of HBM, {f['tflops']} TFLOP/s")
    lines = head + [""] + table(lambda n: kernel_of(n) is not None)
    with open(os.path.join(ROOT, "profiles", f"kernel_trace_{workload}.txt"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    if workload != HEADLINE or "decode_step" not in b:
        return
    d = b["decode_step"]
    lines = ["# Kernel trace: decode step, workload decode_step",
             "# (256 sequences x 16 heads, d_k=d_v=56, bf16 tokens, fp32 state in place, 1024 consecutive"
             " tokens), one MI355X", "#",
             "# commands (the same runs as kernel_trace_fwdbwd_model.txt; bench.py times the decode workload"
             " after the fwd+bwd step):"] + cmd + [
        "#",
        "# bench.py runs the 1024 single-token steps for 6 state sets served round-robin (cold: 308 MB,",
        "# from HBM) and for one state set (hot: 51 MB, held by the 256 MB Infinity Cache), then the same",
        "# tokens as 341 calls of 3 tokens (gdn_step_tokens); per variant an eager pass, a captured graph",
        "# checked bitwise against it, 2 warm replays and 1 timed replay. step_kernel<..., true> is the",
        "# one-token instance, step_pre_kernel the 3-token calls.",
        f"# bench.py without the profiler: cold {d['cold']['us_per_step']} us per step ="
        f" {d['cold']['roofline']['achieved']} GB/s ({d['cold']['roofline']['frac'] * 100:.1f} % of 8 TB/s),",
        f"#   hot {d['hot']['us_per_step']} us per step = {d['hot']['cache_resident']['achieved']} GB/s"
        f" (cache-resident), {d['cold']['bytes_per_launch']} algorithmic bytes per step;",
        f"#   3 tokens per call: cold {d['mtp3_cold']['us_per_step']} us = {d['mtp3_cold']['tokens_per_s']:.4g}"
        f" tokens/s, hot {d['mtp3_hot']['us_per_step']} us = {d['mtp3_hot']['tokens_per_s']:.4g} tokens/s",
        ""] + table(lambda n: "gdn::step_" in n)
    with open(os.path.join(ROOT, "profiles", "kernel_trace_decode_step.txt"), "w") as fh:
        fh.write("\n".join(lines) + "\n")


def mfma_summary(counter_dir, workload):
    """MFMA use per kernel from one rocprofv3 --pmc run of the counters in
    MFMA_COUNTERS over `bench.py --profile-run N`: busy % = MFMA busy cycles
    summed over SIMDs / (active cycles of one XCD x SIMDs); MFMA flops =
    MFMA ops x 512 (the counters count ops in units of 512); TFLOP/s over the
    dispatch's own start and end timestamps; all averaged over launches."""
    import collections
    import csv
    import glob

    import gdn_inputs as gi

    per = collections.defaultdict(dict)
    name = {}
    for f in glob.glob(os.path.join(counter_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                d = r["Dispatch_Id"]
                per[d][r["Counter_Name"]] = per[d].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
                per[d]["ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
                name[d] = r["Kernel_Name"]
    c = gi.CONFIGS[workload]
    alg = kernel_flops(c.B, c.T, c.H, c.dk)
    steps = max(1, sum(1 for x in per if kernel_of(name[x]) == "dA_reduce"))
    wl = "" if workload == HEADLINE else f" --workload {workload}"
    lines = [
        f"# MFMA use per launch, workload {workload} ({_workload_text(workload)}), one MI355X",
        "#",
        "# command (from /tmp on the GPU host, TMPDIR=/tmp):",
        f"#   rocprofv3 --pmc {MFMA_COUNTERS} --output-format csv -d <dir> -o p -- python3 <repo>/bench.py --profile-run 2{wl}",
        f"#   python3 <repo>/bench.py --mfma-summary <dir>{wl}   (writes this file)",
        "#",
        f"# busy % = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {XCD_NUM} XCDs x {SIMD_NUM} SIMDs);",
        "# MFMA flops = (MOPS_BF16 + MOPS_F32) x 512, which counts the padding of the head dim to the",
        "# tile size and the masked halves of the 64 x 64 products; TFLOP/s over each dispatch's own",
        "# duration (profiled); algorithmic flops = the chunk-form count of the kernel's products per launch.",
        f"# source_hash {source_hash()}",
        "",
        f"{'kernel':12s} {'launches':>8s} {'busy %':>7s} {'bf16 GFLOP':>11s} {'fp32 GFLOP':>11s} {'alg. GFLOP':>11s}"
        f" {'us':>8s} {'MFMA TFLOP/s':>13s}",
    ]
    for k in KERNELS:
        ds = [x for x in per if kernel_of(name[x]) == k]
        if not ds:
            continue
        nl = len(ds) / steps
        mean = lambda key: sum(per[x].get(key, 0.0) for x in ds) / len(ds)
        act = mean("GRBM_GUI_ACTIVE") / XCD_NUM
        util = 100.0 * mean("SQ_VALU_MFMA_BUSY_CYCLES") / (act * SIMD_NUM) if act > 0 else float("nan")
        fb, ff = mean("SQ_INSTS_VALU_MFMA_MOPS_BF16") * 512, mean("SQ_INSTS_VALU_MFMA_MOPS_F32") * 512
        ns = mean("ns")
        lines.append(f"{k:12s} {nl:8.0f} {util:7.2f} {fb / 1e9:11.3f} {ff / 1e9:11.3f} "
                     f"{alg.get(k, 0) / nl / 1e9:11.3f} {ns / 1e3:8.1f} {(fb + ff) / (ns * 1e-9) / 1e12:13.1f}")
    with open(os.path.join(ROOT, "profiles", f"mfma_{workload}.txt"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


# Counter passes behind profiles/counters_<workload>.txt (each within one
# rocprofv3 run's limits: at most 8 SQ counters and the GRBM clock).
COUNTER_PASSES = [
    "SQ_LDS_IDX_ACTIVE SQ_LDS_BANK_CONFLICT SQ_BUSY_CU_CYCLES SQ_WAIT_INST_LDS SQ_WAVE_CYCLES SQ_WAIT_ANY "
    "SQ_ACTIVE_INST_LDS GRBM_GUI_ACTIVE",
    "SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_INSTS_SALU SQ_INSTS_VMEM_RD SQ_INSTS_VMEM_WR SQ_WAVES "
    "GRBM_GUI_ACTIVE",
]
CU_NUM = 256


def counter_summary(dirs, workload):
    """Per-kernel LDS use, waits and instruction mix from the rocprofv3 --pmc
    runs of COUNTER_PASSES (one directory each) over `bench.py --profile-run
    N`, averaged over launches: LDS busy % = SQ_LDS_IDX_ACTIVE / (active
    cycles of one XCD x CUs), bank-conflict share of that time, wave-cycles
    spent waiting, and instructions per wave by kind."""
    import collections
    import csv
    import glob

    per = collections.defaultdict(lambda: collections.defaultdict(float))
    name = {}
    for i, d in enumerate(dirs):
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    key = (i, r["Dispatch_Id"])
                    per[key][r["Counter_Name"]] += float(r["Counter_Value"])
                    name[key] = r["Kernel_Name"]
    wl = "" if workload == HEADLINE else f" --workload {workload}"
    lines = [f"# LDS, waits and instruction mix per launch, workload {workload} ({_workload_text(workload)}),"
             " one MI355X", "#", "# commands (from /tmp on the GPU host, TMPDIR=/tmp), one run per pass:"]
    for i, cs in enumerate(COUNTER_PASSES):
        lines.append(f"#   rocprofv3 --pmc {cs} --output-format csv -d <dir{i + 1}> -o p -- "
                     f"python3 <repo>/bench.py --profile-run 2{wl}")
    lines += [f"#   python3 <repo>/bench.py --counter-summary <dir1> <dir2>{wl}   (writes this file)", "#",
              f"# cycles = GRBM_GUI_ACTIVE / {XCD_NUM} (one XCD's active cycles); LDS busy % ="
              f" SQ_LDS_IDX_ACTIVE / (cycles x {CU_NUM} CUs);",
              "# conflict % = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE; wait % = SQ_WAIT_ANY / SQ_WAVE_CYCLES"
              " (wave-cycles",
              "# waiting on any dependency or barrier); instructions per wave = SQ_INSTS_* / SQ_WAVES.",
              f"# source_hash {source_hash()}", "",
              f"{'kernel':12s} {'us@clk':>8s} {'LDS busy%':>9s} {'conflict%':>9s} {'wait%':>6s} "
              f"{'VALU/wave':>9s} {'MFMA/wave':>9s} {'LDS/wave':>8s} {'SALU/wave':>9s} {'VMEM/wave':>9s}"]
    for k in KERNELS:
        res = {}
        for i in range(len(dirs)):
            ds = [x for x in per if x[0] == i and kernel_of(name[x]) == k]
            for c in set().union(*[per[x].keys() for x in ds]) if ds else ():
                res[(i, c)] = sum(per[x][c] for x in ds) / len(ds)
        if not res:
            continue
        g = lambda c: next((v for (i, cc), v in res.items() if cc == c), float("nan"))
        cyc = res.get((0, "GRBM_GUI_ACTIVE"), g("GRBM_GUI_ACTIVE")) / XCD_NUM
        lds = g("SQ_LDS_IDX_ACTIVE")
        waves = g("SQ_WAVES")
        per_wave = lambda c: g(c) / waves if waves and waves == waves else float("nan")
        lines.append(f"{k:12s} {cyc / 2.4e3:8.1f} {100 * lds / (cyc * CU_NUM):9.1f} "
                     f"{100 * g('SQ_LDS_BANK_CONFLICT') / lds if lds else float('nan'):9.1f} "
                     f"{100 * g('SQ_WAIT_ANY') / g('SQ_WAVE_CYCLES'):6.1f} {per_wave('SQ_INSTS_VALU'):9.0f} "
                     f"{per_wave('SQ_INSTS_MFMA'):9.0f} {per_wave('SQ_INSTS_LDS'):8.0f} {per_wave('SQ_INSTS_SALU'):9.0f} "
                     f"{per_wave('SQ_INSTS_VMEM_RD') + per_wave('SQ_INSTS_VMEM_WR'):9.0f}")
    lines += ["", "# us@clk: one XCD's active cycles at 2.4 GHz (the counters' own view of the launch length)."]
    with open(os.path.join(ROOT, "profiles", f"counters_{workload}.txt"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


# ------------------------------------------------------------ CPU oracle

def _f64_inputs(x):
    import numpy as np
    return {k: (v.f64() if hasattr(v, "f64") else (None if v is None else np.asarray(v, np.float64)))
            for k, v in x.items()}


def _sample_units(probe_s, total, cores, budget_s):
    """Units to time so that the run lasts about budget_s (a multiple of the
    thread count when possible, at least one, at most all)."""
    n = int(min(total, max(1, round(budget_s * cores / max(probe_s, 1e-6)))))
    if n >= cores:
        n = (n // cores) * cores
    return max(1, n)


def cpu_baseline(x, B, T, H, budget_s):
    """The fp64 oracle (forward + reverse pass) on a bounded sample of the
    workload's (b, h) units, threaded over units."""
    import oracle

    oracle.build()
    f = _f64_inputs(x)
    cores = oracle.default_threads()
    # size the sample from a one-unit probe so the timed run lasts about budget_s
    t0 = time.perf_counter()
    oracle.fwd(f["q"], f["k"], f["v"], f["g"], f["beta"], f["A_log"], f["h0"], units=[0], nthreads=1)
    oracle.bwd(f["q"], f["k"], f["v"], f["g"], f["beta"], f["A_log"], f["h0"], f["do"], units=[0],
               nthreads=1)
    per_unit = time.perf_counter() - t0
    n_units = _sample_units(per_unit, B * H, cores, budget_s)
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
                      f"{reps} pass(es), {wall:.1f} s wall; threads = the affinity mask capped by "
                      f"OMP_NUM_THREADS (the host's CPU share of one GPU)"}


def oracle_times(x_decode, budget_s=3.0):
    """Per-configuration wall times of the fp64 oracle on this host: the
    forward at the layer shape (threaded and on one thread), the long-context
    fwd+bwd and the 1024-step decode chain, each on a bounded sample of its
    independent units (extrapolated to the whole workload in est_full_s)."""
    import numpy as np

    import gdn_inputs as gi
    import oracle

    cores = oracle.default_threads()
    out = {"threads": cores}

    def seq(name, with_bwd, threads, budget):
        c = gi.CONFIGS[name]
        f = _f64_inputs(gi.gen_config(name))
        args = (f["q"], f["k"], f["v"], f["g"], f["beta"], f["A_log"], f["h0"])

        def run(units, nt):
            oracle.fwd(*args, units=units, nthreads=nt)
            if with_bwd:
                oracle.bwd(*args, f["do"], units=units, nthreads=nt)

        t0 = time.perf_counter()
        run([0], 1)
        probe = time.perf_counter() - t0
        n = _sample_units(probe, c.B * c.H, threads, budget)
        t0 = time.perf_counter()
        run(list(range(n)), threads)
        wall = time.perf_counter() - t0
        total = c.B * c.H
        return {"op": "fwd+bwd" if with_bwd else "fwd", "units": n, "of_units": total, "threads": threads,
                "wall_s": round(wall, 3), "est_full_s": round(wall * total / n, 3),
                "tokens_per_s": n * c.T / c.H / wall}

    out["fwd_model_fwd"] = seq("fwd_model", False, cores, budget_s)
    out["fwd_model_fwd_1thread"] = seq("fwd_model", False, 1, budget_s)
    out["fwdbwd_model_fwdbwd"] = seq("fwdbwd_model", True, cores, budget_s)
    out["long_ctx_fwdbwd"] = seq("long_ctx", True, cores, budget_s)

    # decode chain: a sample of sequences (all heads), 1024 oracle steps each
    c = gi.CONFIGS["decode_step"]
    nseq = max(1, min(c.B, 16))
    sl = lambda a, t: (a.data[t, :nseq] if isinstance(a, gi.Tensor) else a[t, :nseq])
    conv = lambda a, t: (gi.Tensor(sl(a, t), a.dtype).f64() if isinstance(a, gi.Tensor)
                         else np.asarray(sl(a, t), np.float64))
    h = np.asarray(x_decode["h0"][:nseq], np.float64)
    A = np.asarray(x_decode["A_log"], np.float64)
    steps = [[conv(x_decode[n], t) for n in ("q", "k", "v", "g", "beta")] for t in range(c.steps)]
    t0 = time.perf_counter()
    for t in range(c.steps):
        q, k, v, g, b = steps[t]
        _, h = oracle.step(q, k, v, g, b, A, h, nthreads=cores)
    wall = time.perf_counter() - t0
    out["decode_chain"] = {"op": f"{c.steps} steps", "units": nseq * c.H, "of_units": c.B * c.H,
                           "threads": cores, "wall_s": round(wall, 3),
                           "est_full_s": round(wall * c.B / nseq, 3),
                           "tokens_per_s": nseq * c.steps / wall}
    return out


# ------------------------------------------------------------------ main

def copy_bench(dev, nbytes=1 << 30, reps=10):
    """A plain device-to-device copy (torch's copy kernel) of 1 GiB, read and
    write bytes both counted: the HBM rate this machine reaches on the simplest
    streaming kernel. Context for the roofline fractions, never their
    denominator (that is the 8 TB/s peak)."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(2):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    gbs = 2 * nbytes / (ms * 1e-3) / 1e9
    del src, dst
    return {"bytes_per_copy": 2 * nbytes, "ms": round(ms, 4), "GB_s": round(gbs, 1),
            "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
            "note": "torch device-to-device copy of 1 GiB (read + write counted), mean of 10 back to back; "
                    "context, not a roofline denominator"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-long-ctx", action="store_true")
    ap.add_argument("--workload", default=HEADLINE, choices=[HEADLINE, "long_ctx"])
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--profile-run", type=int, default=0, metavar="N")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--mfma-summary", metavar="COUNTER_DIR")
    ap.add_argument("--counter-summary", nargs="+", metavar="PASS_DIR")
    ap.add_argument("--trace-summary", nargs=3, metavar=("KT_DIR", "KT_LOG", "BENCH_LOG"))
    args = ap.parse_args()
    if args.trace_summary:
        trace_summary(*args.trace_summary, args.workload)
        return
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary, args.workload)
        return
    if args.mfma_summary:
        mfma_summary(args.mfma_summary, args.workload)
        return
    if args.counter_summary:
        counter_summary(args.counter_summary, args.workload)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the gated delta rule path here is built and timed "
              "on a single MI355X ((batch, head) units would be split across GPUs with no "
              "communication but one all-reduce of dA_log); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    dev = torch.device("cuda:0")
    flush = _flusher(dev)

    if args.profile_run:
        _, _, step = seq_workload(args.workload, dev)
        for i in range(args.profile_run):
            flush()
            step()
            torch.cuda.synchronize()
            print(f"profile step {i + 1}/{args.profile_run}", flush=True)
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"calibration copy of {COPY_BYTES} bytes done", flush=True)
        return

    if args.workload != HEADLINE:
        res, t, _ = fwdbwd_measure(args.workload, dev, args.steps, args.warmup, flush)
        res["value"] = res["tokens_per_s"]
        print(json.dumps(res), flush=True)
        return

    res, t, x = fwdbwd_measure(HEADLINE, dev, args.steps, args.warmup, flush)
    cfg_B, cfg_T, cfg_H = res["B"], res["T"], res["H"]
    ms = res["ms_per_step"]
    print(f"fwd+bwd {HEADLINE}: {ms} ms per step (median)", file=sys.stderr, flush=True)
    out = {
        "metric": "GDN fwd+bwd tokens/s at B8·H16·T4096·d56; % of MFMA/HBM roofline",
        "value": res["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded gdn_inputs workload fwdbwd_model)",
        "config": {"workload": HEADLINE, "B": cfg_B, "H": cfg_H, "T": cfg_T, "d_k": res["d_k"],
                   "d_v": res["d_v"], "chunk": C, "global_batch": cfg_B, "seq_len": cfg_T,
                   "parallelism": "none (one GPU)"},
        "timing": {"protocol": "512 MiB cache flush before each step (outside its events); median of K",
                   "ms_mean": res["ms_mean"], "ms_min": res["ms_min"], "ms_warm_back_to_back": res["ms_warm"],
                   "wall_s_timed": round(t["wall"], 3)},
        "roofline": res["roofline"],
        "step_roofline": res["step_roofline"],
        "kernels_ms": res["kernels_ms"],  # summed per step
        "cpu_baseline": None,
    }
    out["forward"] = forward_bench(dev, args.steps, args.warmup, flush)
    print(f"forward: {out['forward']['ms']} ms", file=sys.stderr, flush=True)
    out["stream_copy"] = copy_bench(dev)
    print(f"stream copy: {out['stream_copy']['GB_s']} GB/s", file=sys.stderr, flush=True)
    if not args.no_long_ctx:
        lc, _, _ = fwdbwd_measure("long_ctx", dev, max(3, args.steps // 2), 2, flush)
        out["long_ctx"] = lc
        print(f"long_ctx: {lc['ms_per_step']} ms per step", file=sys.stderr, flush=True)
    x_decode = None
    if not args.no_decode:
        out["decode_step"], x_decode = decode_bench(dev)
        print(f"decode: cold {out['decode_step']['cold']['us_per_step']} us per step", file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(x, cfg_B, cfg_T, cfg_H, args.cpu_seconds)
        if x_decode is not None:
            out["oracle_times"] = oracle_times(x_decode)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
