#!/usr/bin/env python3
"""Benchmark of the attention hot path on one MI355X.

One step = one forward (fa_fwd) plus one backward (fa_bwd: row-term
kernel, dK/dV kernel, dQ kernel) over the workload's inputs, which are
resident in HBM before timing starts. The metric is attention TFLOP/s for
fwd+bwd with the FLOP convention 4 * n_q * n_k * d per (batch, head) for the
forward, halved under the causal mask, and 2.5x that for the backward.

Prints one JSON line (the last line of stdout). For the headline workload
(2 x 32 heads, 4096 tokens, d = 128, causal):
  * value: K bare steps, wall clock between two device synchronisations;
    step_ms: median / min / mean of those steps from one event per step;
  * kernels / roofline: per-kernel durations from HIP events recorded
    between the kernels in a separate loop of K steps (each event costs a
    few microseconds, so that loop's steps are longer than bare ones); the
    roofline entry is the dominant kernel's credited FLOPs (the method's
    products only) per launch over its mean duration;
  * configs: the other workloads, forward-only and fwd+bwd, median / min of
    30 event-timed steps after 5 warm-up steps;
  * device: rocminfo's CU count and maximum engine clock;
  * power: socket power and GFX clock sampled with amd-smi while the
    headline step runs back to back for a few seconds (on N(0,1) bf16 data
    the matrix cores run at about 1.8-1.9 GHz, below the 2.4 GHz clock the
    peak assumes);
  * cpu_baseline: the fp64 oracle on whole heads of each workload, on a
    thread pool over (head, row chunk) with one BLAS thread per worker, on
    the host cores this job may use; with the GPU/oracle time ratios.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-configs] [--no-power]
  python bench.py --shape BxHxNQxNKxD [--mask none|top_left|bottom_right]   # any bf16 shape
  python bench.py --rows [--rows-shape RxC]   # standalone row softmax kernel (HBM roofline)
  python bench.py --io [--io-n N]             # fused vs materialising forward, one head (page 1, section 4)
  python bench.py --summarize-io DIR --summary-out F   # HBM bytes per call of both forwards
  python bench.py --summarize-pmc FETCH_DIR WRITE_DIR --summary-out F   # HBM bytes per kernel
  python bench.py --summarize-stats DIR --summary-out F                  # kernel durations
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 256 * 4096 * 2.4e9 / 1e12   # 256 CUs x 4096 FLOP/clk x 2.4 GHz = 2516.6
METRIC = "attention TFLOP/s fwd+bwd (bf16, causal, n=4096, d=128); % MFMA peak"
CSRC = os.path.join(ROOT, "exact_tiled_attention_29_amd", "csrc")
PMC_SUMMARY = os.path.join(ROOT, "profiles", "hbm_traffic_self_b2h32_n4096_d128_causal.txt")
SQ_SUMMARY = os.path.join(ROOT, "profiles", "sq_counters_self_b2h32_n4096_d128_causal.txt")
IO_SUMMARY = os.path.join(ROOT, "profiles", "io_forward_h1_d128_bf16.txt")
IO_SIZES = (1024, 4096, 16384, 65536)
IO_D = 128
IO_SRAM_ELEMS = 100 * 1024 // 2   # the pages' M: about 100 KB of on-chip memory, in bf16 elements
FUSED_KEYS = ("fwd_pp_kernel", "fwd_bf16_kernel")
# Substrings of the bench kernels' mangled names in the rocprofv3 summaries.
KERNEL_KEYS = {"fwd": "fwd_pp_kernel", "bwd_pre": "bwd_pre_kernel", "bwd_dkdv": "bwd_dkdv",
               "bwd_dq": "bwd_dq_kernel"}


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(CSRC, "*"))):
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# --------------------------------------------------------------------------
# HBM traffic from rocprofv3 counter runs
# --------------------------------------------------------------------------

def _read_counter_csv(d):
    import csv
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    return rows


def summarize_pmc(fetch_dir, write_dir, copy_bytes, out_path, command=""):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of each kernel, scaled by
    what the counters read for a plain copy kernel of copy_bytes bytes."""
    def per_kernel(d, counter):
        acc = {}
        for r in _read_counter_csv(d):
            if r.get("Counter_Name") != counter:
                continue
            name = r.get("Kernel_Name", "")
            acc.setdefault(name, []).append(float(r["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in acc.items()}
    fetch = per_kernel(fetch_dir, "FETCH_SIZE")
    write = per_kernel(write_dir, "WRITE_SIZE")
    copy_f = [v for k, v in fetch.items() if "copy" in k.lower() or "elementwise" in k.lower()]
    copy_w = [v for k, v in write.items() if "copy" in k.lower() or "elementwise" in k.lower()]
    fs = copy_bytes / (max(copy_f) * 1024) if copy_f else 1.0
    ws = copy_bytes / (max(copy_w) * 1024) if copy_w else 1.0
    lines = [f"command: {command}", f"source_hash {kernel_source_hash()}",
             f"copy_bytes {copy_bytes} fetch_scale {fs:.4f} write_scale {ws:.4f}"]
    for k in sorted(set(fetch) | set(write)):
        f_ = fetch.get(k, float("nan")) * 1024 * fs
        w_ = write.get(k, float("nan")) * 1024 * ws
        lines.append(f"kernel {k[:120]!r} fetch_bytes {f_:.0f} write_bytes {w_:.0f}")
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_stats(stats_dir, out_path, command):
    """Per-kernel call count and average duration from rocprofv3 --stats."""
    import csv
    rows = []
    for f in glob.glob(os.path.join(stats_dir, "**", "*kernel_stats.csv"), recursive=True):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    lines = [f"command: {command}", f"source_hash {kernel_source_hash()}",
             f"{'kernel':60s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'pct':>6s}"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        lines.append(f"{r['Name'][:60]:60s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} "
                     f"{float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f} "
                     f"{float(r['Percentage']):6.2f}")
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_counters(dirs, out_path, command):
    """Average per dispatch of every counter (raw or derived) found in the
    rocprofv3 --pmc output directories, one row per kernel."""
    acc = {}
    for d in dirs:
        for r in _read_counter_csv(d):
            key = (r.get("Kernel_Name", ""), r.get("Counter_Name", ""))
            acc.setdefault(key, []).append(float(r["Counter_Value"]))
    kernels = sorted({k for k, _ in acc})
    counters = sorted({c for _, c in acc})
    lines = [f"command: {command}", f"source_hash {kernel_source_hash()}",
             "values: average per kernel dispatch (derived counters as rocprofv3 defines them)"]
    for k in kernels:
        if not any((k, c) in acc for c in counters):
            continue
        lines.append(f"kernel {k[:100]!r}")
        for c in counters:
            if (k, c) in acc:
                v = acc[(k, c)]
                lines.append(f"  {c:32s} {sum(v) / len(v):.6g}")
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def traffic_from_summary(kernel_key):
    """HBM bytes per launch of the kernel, or None when no summary exists or
    the kernels changed since the counters were taken."""
    if not os.path.exists(PMC_SUMMARY):
        return None
    lines = open(PMC_SUMMARY).read().splitlines()
    src = next((l.split()[1] for l in lines if l.startswith("source_hash")), None)
    if src != kernel_source_hash():
        return None
    for l in lines:
        if l.startswith("kernel") and kernel_key in l:
            parts = l.split()
            return float(parts[parts.index("fetch_bytes") + 1]) + float(parts[parts.index("write_bytes") + 1])
    return None


def counter_from_summary(kernel_key, counter):
    """Average per dispatch of `counter` for the kernel from the SQ counter
    summary, or None when it is missing or the kernels changed since."""
    if not os.path.exists(SQ_SUMMARY):
        return None
    lines = open(SQ_SUMMARY).read().splitlines()
    src = next((l.split()[1] for l in lines if l.startswith("source_hash")), None)
    if src != kernel_source_hash():
        return None
    inside = False
    for l in lines:
        if l.startswith("kernel"):
            inside = kernel_key in l
        elif inside and l.split() and l.split()[0] == counter:
            return float(l.split()[1])
    return None


# --------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on bounded samples, on the host's cores
# --------------------------------------------------------------------------

ORACLE_ROW_CHUNK = 512     # query rows per oracle task
ORACLE_SAMPLE_FLOP = 2e12  # the oracle's own FLOP per timed sample (whole heads)
CPU_SHARE = 16             # host cores a one-GPU job may use (the box's share)


def oracle_flop_per_head(w) -> float:
    """The oracle's own fp64 FLOP count per (batch, head) for fwd+bwd: the
    materialised S, P V, dO V^T, dS K, dS^T Q and P^T dO products, 12 n_q n_k d
    with no causal skip (the oracle computes full score rows)."""
    return 12.0 * w.n_q * w.n_k * w.d


def cpu_oracle_times(w, q, k, v, do, heads):
    """Wall seconds of the fp64 oracle (oracle.attention_head) for the given
    (b, h) heads, forward only and fwd+bwd, on a thread pool over (head,
    chunk of ORACLE_ROW_CHUNK query rows) with one BLAS thread per worker
    (numpy releases the GIL inside its kernels). A chunk's task returns its
    rows' O, L (and dQ) and its rows' share of dK, dV; shares of one head
    add up to the head's gradients."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    visible = len(os.sched_getaffinity(0))
    workers = max(1, min(visible, CPU_SHARE))
    f = lambda t: t.float().numpy().astype(np.float64)  # noqa: E731
    data = {(b, h): (f(q[b, h]), f(k[b, h]), f(v[b, h]), f(do[b, h])) for b, h in heads}
    chunks = [np.arange(r0, min(r0 + ORACLE_ROW_CHUNK, w.n_q)) for r0 in range(0, w.n_q, ORACLE_ROW_CHUNK)]
    tasks = [(hd, c) for hd in heads for c in chunks]

    def run(with_grads):
        def one(t):
            (b, h), rows = t
            Q, K, V, dO = data[(b, h)]
            return oracle.attention_head(Q, K, V, dO if with_grads else None, w.causal, rows=rows,
                                         visit=rows)
        t0 = time.perf_counter()
        with ThreadPoolExecutor(max_workers=workers) as ex:
            res = list(ex.map(one, tasks))
        dt = time.perf_counter() - t0
        assert all(np.isfinite(r["O"]).all() for r in res)
        return dt

    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            t_fwd, t_all = run(False), run(True)
    else:  # pragma: no cover
        t_fwd, t_all = run(False), run(True)
    return {"fwd_s": t_fwd, "fwd_bwd_s": t_all, "workers": workers, "host_cores_visible": visible}


def cpu_baseline_entry(w, q, k, v, do, heads, gpu_fwd_ms, gpu_step_ms):
    """Oracle times on a sample of whole heads of workload w, next to the GPU
    times of the full workload scaled to the same heads."""
    t = cpu_oracle_times(w, q, k, v, do, heads)
    nbh = w.batch * w.heads
    frac = len(heads) / nbh
    e = {
        "sample": f"{len(heads)} of {nbh} heads (whole heads, every query row)",
        "oracle_fwd_s": round(t["fwd_s"], 3), "oracle_fwd_bwd_s": round(t["fwd_bwd_s"], 3),
        "oracle_flop_fwd_bwd": oracle_flop_per_head(w) * len(heads),
        "cores": t["workers"], "host_cores_visible": t["host_cores_visible"],
        "metric_tflops_fwd_bwd": round(w.fwd_bwd_flop() * frac / t["fwd_bwd_s"] / 1e12, 5),
    }
    if gpu_step_ms:
        e["gpu_over_oracle_fwd_bwd"] = round(t["fwd_bwd_s"] / (gpu_step_ms * 1e-3 * frac), 1)
    if gpu_fwd_ms:
        e["gpu_over_oracle_fwd"] = round(t["fwd_s"] / (gpu_fwd_ms * 1e-3 * frac), 1)
    return e


def oracle_sample(w):
    """Whole heads the oracle times for workload w: at most 2e12 of its fp64
    FLOP (several seconds on 16 cores: every head of the 4096-token and
    smaller workloads) or a single head."""
    nbh = w.batch * w.heads
    per_head = oracle_flop_per_head(w)
    n = max(1, min(nbh, int(ORACLE_SAMPLE_FLOP // per_head)))
    idx = [(i * 7) % nbh for i in range(n)] if n < nbh else list(range(nbh))
    return [(i // w.heads, i % w.heads) for i in sorted(set(idx))]


# --------------------------------------------------------------------------
# Standalone row softmax / logsumexp kernel
# --------------------------------------------------------------------------

# --------------------------------------------------------------------------
# Page 1 ("05_flash_attention.py"), section 4, measured: one head, bf16,
# d = 128, the fused forward beside the materialising one
# --------------------------------------------------------------------------

def io_inputs(n, dev):
    """Seeded Q, K, V of one head (n x 128, bf16) on the device, and the
    materialising path's operands prepared on the host: scale * Q (bf16)
    and K^T (contiguous), so that path's calls run only its three kernels."""
    import math
    import torch
    import workloads
    w = workloads.custom(1, 1, n, n, IO_D, "bf16", False, name=f"io_n{n}")
    q, k, v, _ = workloads.make_inputs(w, seed=0)
    scale = 1.0 / math.sqrt(IO_D)
    qs = (q[0, 0].float() * scale).to(torch.bfloat16)
    kt = k[0, 0].t().contiguous()
    up = lambda t: t.contiguous().to(dev)  # noqa: E731
    return up(q), up(k), up(v), up(qs), up(kt), up(v[0, 0])


def materialising_forward(qs, kt, v):
    """Standard attention as page 1, section 2 writes it (standard_attention):
    S = Q K^T / sqrt(d) and P = softmax(S) are n x n bf16 matrices in HBM
    (page 1, section 4 counts exactly these two), O = P V. Plain torch ops
    (hipBLASLt GEMMs, torch's softmax): the comparison baseline of the IO
    table, not part of the library."""
    import torch
    s = torch.mm(qs, kt)
    p = torch.softmax(s, dim=-1)
    return torch.mm(p, v)


def fa_forward_workspace(n):
    """Bytes of the key-split workspace the fused forward takes for one head
    of n x n, d = 128 (0 when it does not split)."""
    import exact_tiled_attention_29_amd as fa
    return fa.fa_fwd_workspace_bytes(1, 1, n, n, IO_D, fa.FA_BF16, 0)


IO_PATHS = ("materialising", "fused", "fused_split")


def io_compare(n, calls=10, warmup=2, paths=IO_PATHS):
    """Times `calls` calls of each forward (after `warmup`), measures the
    device memory each allocates beyond its inputs (peak), and the largest
    difference between the outputs. Paths: the materialising forward, the
    fused forward without the key split (fa_fwd) and with it (fa_fwd_ws,
    only where the library splits this size)."""
    import torch
    import exact_tiled_attention_29_amd as fa
    dev = torch.device("cuda:0")
    q, k, v, qs, kt, v2 = io_inputs(n, dev)
    fns = {"materialising": lambda: materialising_forward(qs, kt, v2),
           "fused": lambda: fa.forward(q, k, v, False, split=False)[0],
           "fused_split": lambda: fa.forward(q, k, v, False)[0]}
    ws = fa_forward_workspace(n)
    out = {"n": n, "d": IO_D, "fused_split_workspace_bytes": int(ws)}
    res = {}
    for name in paths:
        if name == "fused_split" and ws == 0:
            continue
        fn = fns[name]
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats()
        base = torch.cuda.memory_allocated()
        o = fn()
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated() - base
        res[name] = o.reshape(n, IO_D)
        del o
        for _ in range(max(0, warmup - 1)):
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(calls)]
        torch.cuda.synchronize()
        for a, b in ev:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        out[name] = {"ms": _stats([a.elapsed_time(b) for a, b in ev]), "peak_extra_bytes": int(peak)}
    if "materialising" in res:
        ref = res["materialising"].float()
        for name in res:
            if name != "materialising":
                out[name]["max_abs_diff_vs_materialising"] = float((res[name].float() - ref).abs().max())
    # the pages' estimates (page 1, section 4): S and P held as bf16 n x n
    # matrices against one fp32 vector; 4 n^2 accesses against n^2 d^2 / M
    out["page_memory_bytes"] = {"materialising": 2 * n * n * 2, "fused": 4 * n}
    out["page_io_elements"] = {"materialising": 4 * n * n,
                               "fused": round(n * n * IO_D * IO_D / IO_SRAM_ELEMS)}
    return out


def io_traffic_from_summary(n):
    """HBM bytes per call of each forward at size n from the committed IO
    summary ({} when absent or older than the kernel sources)."""
    if not os.path.exists(IO_SUMMARY):
        return {}
    lines = open(IO_SUMMARY).read().splitlines()
    if f"source_hash {kernel_source_hash()}" not in lines:
        return {}
    out = {}
    for line in lines:
        t = line.split()
        if len(t) == 5 and t[0] == "n" and int(t[1]) == n and t[3] == "bytes_per_call":
            out[t[2]] = float(t[4])
    return out


def _io_anchor(path, kernel):
    """Whether `kernel` runs exactly once per call of `path` (it counts the calls)."""
    if path == "materialising":
        return "softmax" in kernel.lower()
    if path == "fused_split":
        return "fwd_merge_kernel" in kernel
    return any(f in kernel for f in FUSED_KEYS)


def _io_member(path, kernel):
    """Whether `kernel` belongs to `path` (set-up and copy kernels do not)."""
    if path == "materialising":
        return "Cijk" in kernel or "gemm" in kernel.lower() or "softmax" in kernel.lower()
    return any(f in kernel for f in FUSED_KEYS) or "fwd_merge_kernel" in kernel


def summarize_io(base_dir, out_path, command, copy_bytes=512 << 20):
    """HBM bytes per call of each forward from rocprofv3 --pmc runs of
    `bench.py --io --io-n N --io-path PATH --copy-mib 512`, one path per
    process: FETCH_SIZE in base_dir/fN_PATH, WRITE_SIZE in base_dir/wN_PATH.
    The copy kernel of copy_bytes gives the counters' scale factors; the
    path's kernels (GEMMs and softmax; the attention and merge kernels) are
    summed, and one kernel that runs once per call counts the calls."""
    lines = [f"command: {command}", f"source_hash {kernel_source_hash()}",
             "bytes per call; FETCH_SIZE and WRITE_SIZE scaled by the copy kernel of "
             f"{copy_bytes} bytes read and written in the same process"]
    runs = []
    for d in glob.glob(os.path.join(base_dir, "f*_*")):
        if os.path.isdir(d):
            n, path = os.path.basename(d)[1:].split("_", 1)
            if n.isdigit() and path in IO_PATHS:
                runs.append((int(n), path))
    for n, path in sorted(runs, key=lambda r: (r[0], IO_PATHS.index(r[1]))):
        total = 0.0
        for counter, sub in (("FETCH_SIZE", "f"), ("WRITE_SIZE", "w")):
            acc = {}
            for r in _read_counter_csv(os.path.join(base_dir, f"{sub}{n}_{path}")):
                if r.get("Counter_Name") == counter:
                    acc.setdefault(r.get("Kernel_Name", ""), []).append(float(r["Counter_Value"]) * 1024)
            copy = [max(v) for k, v in acc.items() if "copy" in k.lower()]
            scale = copy_bytes / max(copy) if copy else 1.0
            calls = sum(len(v) for k, v in acc.items() if _io_anchor(path, k)) or 1
            for k, v in acc.items():
                member = _io_member(path, k)
                if member:
                    total += sum(v) * scale / calls
                lines.append(f"  n {n} {path} {counter} {'counted' if member else 'other'} kernel "
                             f"{k[:90]!r} dispatches {len(v)} bytes {sum(v) * scale:.0f}")
        lines.append(f"n {n} {path} bytes_per_call {total:.0f}")
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def bench_io(args):
    """Page 1, section 4's table (one head, bf16, d = 128), measured: time
    per call, peak device memory beyond the inputs and, from the committed
    rocprofv3 summary, HBM bytes per call of the materialising forward and
    of the fused forward without and with the key split."""
    import torch
    import exact_tiled_attention_29_amd as fa
    fa.load_library()
    torch.cuda.set_device(0)
    if args.copy_mib:
        a = torch.empty(args.copy_mib << 20, dtype=torch.uint8, device="cuda").fill_(1)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    sizes = [args.io_n] if args.io_n else list(IO_SIZES)
    paths = IO_PATHS if args.io_path == "all" else (args.io_path,)
    entries = []
    for n in sizes:
        e = io_compare(n, calls=args.io_calls, warmup=min(2, args.io_calls), paths=paths)
        e["hbm_bytes_per_call"] = io_traffic_from_summary(n)
        entries.append(e)
        parts = [f"{p} {e[p]['ms']['median']:.4f} ms, {e[p]['peak_extra_bytes'] / 1e6:.2f} MB"
                 for p in IO_PATHS if p in e]
        log(f"[io] n={n}: " + "; ".join(parts) + f"; HBM bytes {e['hbm_bytes_per_call']}")
    last = entries[-1]
    result = {
        "metric": "forward time, materialising / fused (one head, bf16, d=128)",
        "value": (round(last["materialising"]["ms"]["median"] / last["fused"]["ms"]["median"], 3)
                  if "materialising" in last and "fused" in last else None),
        "unit": "x", "n_gpus": 1, "steps": args.io_calls, "warmup": 2,
        "higher_is_better": True, "scaling": "strong", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1), bf16)",
        "config": {"workload": f"io_h1_d{IO_D}_n{last['n']}", "sizes": sizes},
        "io": entries,
    }
    print(json.dumps(result), flush=True)
    return 0


def bench_rows(args):
    """Times fa_row_softmax (softmax + logsumexp of every row) on a bf16
    matrix resident in HBM; the roofline is HBM: one read of x, one write of
    y and of L per call."""
    import numpy as np
    import torch
    import exact_tiled_attention_29_amd as fa

    rows, cols = (int(t) for t in args.rows_shape.lower().split("x"))
    dev = torch.device("cuda:0")
    fa.load_library()
    g = torch.Generator(device=dev).manual_seed(0)
    x = (torch.randn(rows, cols, generator=g, device=dev) * 3.0).to(torch.bfloat16)
    y = torch.empty_like(x)
    lse = torch.empty(rows, dtype=torch.float32, device=dev)
    scale = 1.0 / np.sqrt(128.0)
    run = lambda: fa.row_softmax(x, scale, True, torch.bfloat16, lse=lse, out=y)  # noqa: E731
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    K = args.steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(K):
        run()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / K
    nbytes = rows * cols * 2 * 2 + rows * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"[bench] row softmax {rows}x{cols} bf16: {ms:.4f} ms/call -> {gbs:.0f} GB/s "
        f"({100 * gbs / 8000:.1f}% of 8000)")
    result = {
        "metric": "row softmax + logsumexp GB/s (bf16)", "value": round(gbs, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / K, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,9) bf16 rows)",
        "config": {"workload": f"rows_{rows}x{cols}_bf16", "rows": rows, "cols": cols},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": 8000.0, "unit": "GB/s",
                     "frac": round(gbs / 8000.0, 4), "traffic": None, "kernel": "row_softmax",
                     "avg_ms": round(ms, 4)},
        "cpu_baseline": None,
    }
    print(json.dumps(result), flush=True)
    return 0


# --------------------------------------------------------------------------
# Device facts: rocminfo's CU count and clock, and power / clock under load
# --------------------------------------------------------------------------

def device_info():
    """CU count and max engine clock of the gfx950 agent from rocminfo."""
    import re
    import subprocess
    info = {"rocminfo_compute_units": None, "rocminfo_max_clock_mhz": None, "name": None}
    try:
        out = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
    except Exception:  # pragma: no cover
        return info
    for agent in out.split("Agent ")[1:]:
        if "gfx950" not in agent:
            continue
        m = re.search(r"Compute Unit:[ \t]+(\d+)", agent)
        c = re.search(r"Max Clock Freq\. \(MHz\):[ \t]+(\d+)", agent)
        n = re.search(r"Marketing Name:[ \t]*(\S.*)", agent)
        info["rocminfo_compute_units"] = int(m.group(1)) if m else None
        info["rocminfo_max_clock_mhz"] = int(c.group(1)) if c else None
        info["name"] = n.group(1).strip() if n else None
        break
    return info


def parse_amd_smi(text):
    """Socket power (W) and the first GFX clock (MHz) from `amd-smi metric -p
    -c` output; None where absent."""
    import re
    p = re.search(r"SOCKET_POWER:\s*([\d.]+)\s*W", text)
    c = re.search(r"GFX_0:\s*\n\s*CLK:\s*([\d.]+)\s*MHz", text)
    return (float(p.group(1)) if p else None, float(c.group(1)) if c else None)


def sustained_power(step, seconds):
    """Run step() back to back for about `seconds` while sampling amd-smi
    twice from a side thread; returns the mean socket power and GFX clock."""
    import shutil
    import subprocess
    import threading
    import torch
    if not shutil.which("amd-smi"):
        return None
    samples = []
    stop = threading.Event()

    def sampler():
        time.sleep(min(1.5, seconds / 3))
        while not stop.is_set() and len(samples) < 2:
            try:
                out = subprocess.run(["amd-smi", "metric", "-p", "-c"], capture_output=True,
                                     text=True, timeout=20).stdout
                samples.append(parse_amd_smi(out))
            except Exception:  # pragma: no cover
                break
            time.sleep(0.5)

    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds and (th.is_alive() or time.perf_counter() - t0 < 1.0):
        for _ in range(20):
            step()
        torch.cuda.synchronize()
    stop.set()
    th.join(timeout=30)
    pw = [p for p, _ in samples if p is not None]
    ck = [c for _, c in samples if c is not None]
    if not pw and not ck:
        return None
    clk = sum(ck) / len(ck) if ck else None
    return {"socket_power_w": round(sum(pw) / len(pw), 1) if pw else None,
            "gfx_clock_mhz": round(clk, 1) if clk else None,
            "samples": len(samples)}


# --------------------------------------------------------------------------
# GPU benchmark
# --------------------------------------------------------------------------

def _stats(xs):
    ys = sorted(xs)
    n = len(ys)
    med = ys[n // 2] if n % 2 else 0.5 * (ys[n // 2 - 1] + ys[n // 2])
    return {"median": round(med, 5), "min": round(ys[0], 5), "mean": round(sum(ys) / n, 5)}


def time_per_step(fn, steps, warmup):
    """Per-step GPU times (ms) from events recorded between steps on the
    current stream, after warmup untimed steps."""
    import torch
    for _ in range(warmup):
        fn()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(steps):
        fn()
        ev[i + 1].record()
    torch.cuda.synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]


class Problem:
    """Device buffers of one workload and its fwd / fwd+bwd step functions."""

    def __init__(self, w, cpu_inputs=None, split=True):
        import torch
        import exact_tiled_attention_29_amd as fa
        import workloads
        self.w = w
        self.cpu = cpu_inputs if cpu_inputs is not None else workloads.make_inputs(w)
        dev = torch.device("cuda:0")
        self.q, self.k, self.v, self.do = (t.to(dev) for t in self.cpu)
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty(w.batch, w.heads, w.n_q, dtype=torch.float32, device=dev)
        self.grads = (torch.empty_like(self.q), torch.empty_like(self.k), torch.empty_like(self.v))
        dt = fa.FA_BF16 if w.dtype == "bf16" else fa.FA_F32
        need = fa.fa_bwd_workspace_bytes(w.batch, w.heads, w.n_q, w.n_k, w.d, dt, fa._mask_code(w.causal))
        self.ws = torch.empty(max(1, need), dtype=torch.uint8, device=dev)
        # the forward's key-split workspace (grids with few query tiles)
        need_f = fa.fa_fwd_workspace_bytes(w.batch, w.heads, w.n_q, w.n_k, w.d, dt,
                                           fa._mask_code(w.causal)) if split else 0
        self.split = split
        self.fws = torch.empty(need_f, dtype=torch.uint8, device=dev) if need_f else None
        self.fa = fa

    def fwd(self, ev=None):
        if ev is not None:
            ev[0].record()
        self.fa.forward(self.q, self.k, self.v, self.w.causal, out=self.o, lse=self.lse,
                        split=self.split, workspace=self.fws)
        if ev is not None:
            ev[1].record()

    def step(self, evf=None, evb=None):
        self.fwd(evf)
        self.fa.backward(self.q, self.k, self.v, self.o, self.lse, self.do, self.w.causal,
                         workspace=self.ws, grads=self.grads, events=evb)


def config_entry(name, steps=30, warmup=5, split=True):
    """Forward-only and fwd+bwd times of a named workload (median and min of
    `steps` event-timed steps) with the metric's FLOP convention."""
    import workloads
    w = workloads.WORKLOADS[name]
    pr = Problem(w, split=split)
    f = _stats(time_per_step(pr.fwd, steps, warmup))
    a = _stats(time_per_step(pr.step, steps, warmup))
    fl_f, fl_a = w.fwd_flop(), w.fwd_bwd_flop()
    e = {"workload": name, "dtype": w.dtype, "causal": w.causal,
         "shape": [w.batch, w.heads, w.n_q, w.n_k, w.d],
         "fwd_ms": f, "fwd_bwd_ms": a,
         "fwd_tflops": round(fl_f / (f["median"] * 1e-3) / 1e12, 2),
         "fwd_bwd_tflops": round(fl_a / (a["median"] * 1e-3) / 1e12, 2)}
    if w.dtype == "bf16":
        e["fwd_pct_of_peak"] = round(100 * e["fwd_tflops"] / PEAK_BF16_TFLOPS, 2)
        e["fwd_bwd_pct_of_peak"] = round(100 * e["fwd_bwd_tflops"] / PEAK_BF16_TFLOPS, 2)
    log(f"[bench] {name}: fwd {f['median']:.4f} ms ({e['fwd_tflops']} TFLOP/s), fwd+bwd "
        f"{a['median']:.4f} ms ({e['fwd_bwd_tflops']} TFLOP/s) [median of {steps}]")
    return e, pr


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--shape", default=None, metavar="BxHxNQxNKxD",
                    help="time a bf16 shape of your own instead of a named workload (not the "
                         "headline metric)")
    ap.add_argument("--mask", default="top_left", choices=["none", "top_left", "bottom_right"],
                    help="mask of --shape")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads' fwd and fwd+bwd times (the 'configs' entry)")
    ap.add_argument("--no-power", action="store_true",
                    help="skip the sustained run that samples socket power and clock")
    ap.add_argument("--power-seconds", type=float, default=4.0)
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarize-stats", metavar="DIR")
    ap.add_argument("--summarize-counters", nargs="+", metavar="DIR",
                    help="average every counter of rocprofv3 --pmc runs per kernel dispatch")
    ap.add_argument("--summary-out", default=PMC_SUMMARY)
    ap.add_argument("--summary-copy-mib", type=int, default=512)
    ap.add_argument("--summary-command", default="", help="command line recorded in a summary")
    ap.add_argument("--no-split", action="store_true",
                    help="never split the forward's keys over workgroups (fa_fwd instead of fa_fwd_ws)")
    ap.add_argument("--io", action="store_true",
                    help="fused vs materialising forward, one head, d = 128 (page 1, section 4)")
    ap.add_argument("--io-n", type=int, default=0, help="one size for --io (default: all)")
    ap.add_argument("--io-calls", type=int, default=10, help="timed calls per path for --io")
    ap.add_argument("--io-path", default="all", choices=("all",) + IO_PATHS,
                    help="one forward only (for a profiler run of that path)")
    ap.add_argument("--summarize-io", metavar="DIR",
                    help="write the IO summary from DIR/fN (FETCH_SIZE) and DIR/wN (WRITE_SIZE)")
    ap.add_argument("--rows", action="store_true",
                    help="benchmark the standalone row softmax / logsumexp kernel instead")
    ap.add_argument("--rows-shape", default="262144x4096",
                    help="rows x cols of the row kernel's bf16 input (default: the score rows of "
                         "the 2x32x4096 workload)")
    args = ap.parse_args()

    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.summary_copy_mib << 20,
                      args.summary_out, args.summary_command)
        return 0
    if args.summarize_stats:
        summarize_stats(args.summarize_stats, args.summary_out, args.summary_command)
        return 0
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.summary_out, args.summary_command)
        return 0
    if args.summarize_io:
        summarize_io(args.summarize_io, args.summary_out, args.summary_command,
                     copy_bytes=args.summary_copy_mib << 20)
        return 0

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: the attention path is benchmarked on a single "
              "MI355X (heads shard across GPUs with no communication); use --gpus 1.",
              file=sys.stderr)
        return 2

    import torch
    import exact_tiled_attention_29_amd as fa
    import workloads

    if args.rows:
        return bench_rows(args)
    if args.io:
        return bench_io(args)

    if args.shape:
        B, H, NQ, NK, D = (int(x) for x in args.shape.lower().split("x"))
        causal = {"none": False, "top_left": True, "bottom_right": "bottom_right"}[args.mask]
        w = workloads.custom(B, H, NQ, NK, D, "bf16", causal,
                             name=f"b{B}h{H}_q{NQ}_k{NK}_d{D}_{args.mask}")
    else:
        w = workloads.WORKLOADS[args.workload or workloads.HEADLINE]
    headline = w.name == workloads.HEADLINE
    metric = METRIC if headline else \
        f"attention TFLOP/s fwd+bwd ({w.dtype}, mask {w.causal}, n_q={w.n_q}, n_k={w.n_k}, d={w.d})"
    fa.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    dinfo = device_info()
    dinfo["torch_multi_processor_count"] = props.multi_processor_count
    dinfo["torch_name"] = props.name
    dinfo["gcn_arch"] = getattr(props, "gcnArchName", None)
    log(f"[bench] device {dinfo.get('name') or props.name}: {dinfo['rocminfo_compute_units']} CUs, "
        f"max clock {dinfo['rocminfo_max_clock_mhz']} MHz (rocminfo)")

    log(f"[bench] workload {w.name}: B={w.batch} H={w.heads} n_q={w.n_q} n_k={w.n_k} d={w.d} "
        f"{w.dtype} causal={w.causal}")
    pr = Problem(w, split=not args.no_split)

    if args.copy_mib:
        a = torch.empty(args.copy_mib << 20, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    for _ in range(args.warmup):
        pr.step()
    torch.cuda.synchronize()

    K = args.steps
    # Timed region 1, the per-kernel durations: K steps with HIP events
    # recorded between the kernels on the library's stream (torch's current
    # stream). Each timing event costs a few microseconds of GPU time, so
    # the kernel times add up to more than a bare step; this loop is not the
    # metric. It also brings the GPU to its sustained clock.
    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    evf = [[E(), E()] for _ in range(K)]
    evb = [[E(), E(), E(), E()] for _ in range(K)]
    for e in evf + evb:                # create the events before the timed region
        for x in e:
            x.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(K):
        pr.step(evf[i], evb[i])
    torch.cuda.synchronize()
    wall_ev = time.perf_counter() - t1

    # Timed region 2, the metric: K steps, wall clock between two device
    # synchronisations; one event per step boundary gives the per-step
    # median and min.
    sev = [E() for _ in range(K + 1)]
    for x in sev:
        x.record()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    sev[0].record()
    for i in range(K):
        pr.step()
        sev[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = [sev[i].elapsed_time(sev[i + 1]) for i in range(K)]

    kern = {
        "fwd": [a.elapsed_time(b) for a, b in evf],
        "bwd_pre": [e[0].elapsed_time(e[1]) for e in evb],
        "bwd_dkdv": [e[1].elapsed_time(e[2]) for e in evb],
        "bwd_dq": [e[2].elapsed_time(e[3]) for e in evb],
    }
    kstats = {k_: _stats(v_) for k_, v_ in kern.items()}
    ms_step = wall * 1e3 / K
    f_fwd = w.fwd_flop()
    f_all = w.fwd_bwd_flop()
    value = f_all / (ms_step * 1e-3) / 1e12
    mean_ms = {k_: st["mean"] for k_, st in kstats.items()}
    dom = max(mean_ms, key=mean_ms.get)
    # Credited FLOPs per kernel: the method's own products, one product =
    # half the forward count. Forward: S and PV. dK/dV kernel: the S
    # recompute, dV, dP and dK (4). dQ kernel: dQ only; the S and dP it
    # forms again are work the split costs, not the method's, and are not
    # credited (they are in "executed_tflops").
    credit = {"fwd": 1.0, "bwd_dkdv": 2.0, "bwd_dq": 0.5}
    executed = {"fwd": 1.0, "bwd_dkdv": 2.0, "bwd_dq": 1.5}
    if w.dtype == "bf16" and dom in credit:
        ach = credit[dom] * f_fwd / (mean_ms[dom] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": round(PEAK_BF16_TFLOPS, 1),
                "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic_from_summary(KERNEL_KEYS[dom]) if headline else None,
                "kernel": dom, "avg_ms": round(mean_ms[dom], 4),
                "algorithmic_flop": credit[dom] * f_fwd}
    else:
        roof = {"bound": "mfma", "achieved": None, "peak": round(PEAK_BF16_TFLOPS, 1),
                "unit": "TFLOP/s", "frac": None, "traffic": None, "kernel": dom,
                "avg_ms": round(mean_ms[dom], 4)}

    per_kernel = {}
    for kname, st in kstats.items():
        e = {"ms": st}
        if kname in credit:
            e["tflops"] = round(credit[kname] * f_fwd / (st["mean"] * 1e-3) / 1e12, 1)
            e["executed_tflops"] = round(executed[kname] * f_fwd / (st["mean"] * 1e-3) / 1e12, 1)
        if headline:
            tr = traffic_from_summary(KERNEL_KEYS[kname])
            e["hbm_gb_s"] = round(tr / (st["mean"] * 1e-3) / 1e9, 1) if tr is not None else None
            e["mfma_util_pct"] = counter_from_summary(KERNEL_KEYS[kname], "MfmaUtil")
        per_kernel[kname] = e
    log(f"[bench] {K} steps with per-kernel events: {wall_ev * 1e3 / K:.4f} ms/step")
    log(f"[bench] {K} steps: {ms_step:.4f} ms/step -> {value:.1f} TFLOP/s "
        f"({100 * value / PEAK_BF16_TFLOPS:.1f}% of {PEAK_BF16_TFLOPS:.1f}); per step median "
        f"{_stats(step_ms)['median']:.4f} min {_stats(step_ms)['min']:.4f} ms")
    for kname, st in kstats.items():
        log(f"[bench]   {kname:15s} {st['mean']:.4f} ms (median {st['median']:.4f}, min {st['min']:.4f})")

    result = {
        "metric": metric, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic (seeded N(0,1) inputs, workloads.py)",
        "config": {"workload": w.name, "batch": w.batch, "heads": w.heads, "n_q": w.n_q,
                   "n_k": w.n_k, "d": w.d, "causal": w.causal, "parallelism": "single GPU"},
        "pct_of_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "step_ms": _stats(step_ms),
        "fwd_tflops": round(f_fwd / (kstats["fwd"]["mean"] * 1e-3) / 1e12, 2),
        "bwd_tflops": round(2.5 * f_fwd / (sum(kstats[k_]["mean"] for k_ in ("bwd_pre", "bwd_dkdv", "bwd_dq"))
                                           * 1e-3) / 1e12, 2),
        "kernel_ms": {k_: st["mean"] for k_, st in kstats.items()},
        "kernels": per_kernel,
        "ms_per_step_with_kernel_events": round(wall_ev * 1e3 / K, 4),
        "device": dinfo,
        "roofline": roof,
    }

    # The other workloads: fwd and fwd+bwd, median and min of 30 steps each.
    cfg_probs = {}
    if headline and not args.no_configs:
        configs = {}
        for name in ("tiny_f32", "tiny_f32_causal", "self_b4h16_n1024_d64",
                     "long_b1h8_n32768_d128_causal", "cross_b8h12_q1000_k3000_d64"):
            configs[name], cfg_probs[name] = config_entry(name, split=not args.no_split)
        result["configs"] = configs

    # Socket power and clock while the headline step runs back to back: the
    # matrix cores run below the 2.4 GHz clock the peak assumes on N(0,1) data.
    if not args.no_power:
        pw = sustained_power(pr.step, args.power_seconds)
        if pw and pw.get("gfx_clock_mhz"):
            cus = dinfo["rocminfo_compute_units"] or props.multi_processor_count
            pw["mfma_peak_at_clock_tflops"] = round(cus * 4096 * pw["gfx_clock_mhz"] * 1e6 / 1e12, 1)
            pw["pct_of_peak_at_clock"] = round(100 * value / pw["mfma_peak_at_clock_tflops"], 2)
        result["power"] = pw
        if pw:
            log(f"[bench] sustained: {pw.get('socket_power_w')} W, GFX clock {pw.get('gfx_clock_mhz')} MHz")

    if not args.no_cpu_baseline:
        log(f"[bench] timing the fp64 oracle on {len(os.sched_getaffinity(0))} visible cores "
            f"(pool of at most {CPU_SHARE}) ...")
        heads = oracle_sample(w)
        cb = cpu_baseline_entry(w, *pr.cpu, heads, kstats["fwd"]["median"], _stats(step_ms)["median"])
        result["cpu_baseline"] = {
            "value": cb["metric_tflops_fwd_bwd"], "unit": "TFLOP/s", "cores": cb["cores"],
            "kind": "oracle",
            "sample": f"{cb['sample']} of {w.name}, fwd+bwd in fp64 on a pool of {cb['cores']} threads "
                      f"({cb['oracle_fwd_bwd_s']} s; metric FLOP convention)",
            "detail": cb,
        }
        log(f"[bench] oracle {w.name}: {cb['oracle_fwd_bwd_s']} s fwd+bwd, {cb['oracle_fwd_s']} s fwd "
            f"on {len(heads)} heads; GPU is {cb.get('gpu_over_oracle_fwd_bwd')}x faster")
        if cfg_probs:
            per_cfg = {}
            for name, p_ in cfg_probs.items():
                c = result["configs"][name]
                per_cfg[name] = cpu_baseline_entry(p_.w, *p_.cpu, oracle_sample(p_.w),
                                                   c["fwd_ms"]["median"], c["fwd_bwd_ms"]["median"])
                log(f"[bench] oracle {name}: {per_cfg[name]['oracle_fwd_bwd_s']} s fwd+bwd "
                    f"({per_cfg[name]['sample']})")
            result["cpu_baseline"]["configs"] = per_cfg
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
