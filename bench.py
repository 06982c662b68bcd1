#!/usr/bin/env python3
"""Benchmark of the Gated MLA attention path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--all] [--no-cpu]

Prints ONE JSON line.  ``value`` is the causal prefill throughput in TFLOP/s on the
workload B=2 T=4096 H=96 D=128 bf16 (algorithmic flops 4*D*B*H*T(T+1)/2 per call,
inputs resident in HBM); the decode half of the metric (HBM GB/s of one query
against 1001 keys, B=8 H=96 D=128 bf16, algorithmic bytes K + V + Q + O) is the
``decode`` object.  Each is timed with HIP events recorded on the stream the
kernels run on, over exactly K timed calls after W warm-up calls.  ``roofline``
compares the dominant kernel with MI355X's published peaks; ``cpu_baseline`` times
the plain CPU oracle on a bounded sample of the same workload.

Profiling helpers (no compute of their own):
    python bench.py --only prefill|decode|layer|decode_long|decode_latent|copy --steps K
        run just that part, for rocprofv3 --kernel-trace or --pmc passes;
    python bench.py --only prefill --loop SECONDS
        call the prefill back to back (to sample clocks with rocm-smi meanwhile);
    python bench.py --summarize-stats DIR --name NAME --cmd "..."
    python bench.py --summarize-mfma DIR --name NAME --cmd "..."
        turn rocprofv3 kernel statistics in DIR into profiles/NAME.md;
    python bench.py --summarize-traffic DIR_FETCH DIR_WRITE COPY_FETCH COPY_WRITE --kernel K --cmd "..."
        turn FETCH_SIZE / WRITE_SIZE passes (kernel and a 1 GiB copy for scale)
        into the entry for kernel K in profiles/traffic.json.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import sys
import time

METRIC = "causal attn TFLOP/s prefill T=4096; decode HBM GB/s at 1001 keys"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0     # MI355X HBM3E
HERE = os.path.dirname(os.path.abspath(__file__))
PROFILES = os.path.join(HERE, "profiles")
TRAFFIC_FILE = os.path.join(PROFILES, "traffic.json")
COPY_BYTES = 1 << 30

# sources of each timed kernel: its traffic record is valid only for these bytes
KERNEL_SOURCES = {
    "prefill_bf16_kernel": ["causal_softmax_attention_gmla_amd/csrc/prefill_bf16.hip",
                            "causal_softmax_attention_gmla_amd/csrc/gmla_internal.h"],
    "decode_split_kernel": ["causal_softmax_attention_gmla_amd/csrc/decode.hip",
                            "causal_softmax_attention_gmla_amd/csrc/gmla_internal.h"],
    "latent_split_kernel_512": ["causal_softmax_attention_gmla_amd/csrc/decode_latent.hip",
                                "causal_softmax_attention_gmla_amd/csrc/gmla_internal.h"],
}


def prefill_flops(B, T, H, D):
    # QK^T and PV over the T(T+1)/2 visible (query, key) pairs: 2 * 2 * D flop each
    return 4 * D * B * H * T * (T + 1) // 2


def decode_bytes(B, H, N, D, elem=2):
    # every K and V row once, plus Q in and O out
    return (2 * B * H * N * D + 2 * B * H * D) * elem


def source_digest(kernel: str) -> str:
    """Digest of the code of a kernel's sources: `//` comments and blank lines are left
    out, so a comment edit keeps the recorded counters valid and any code edit voids them."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(HERE, f)) as fh:
            for line in fh:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def measured_traffic(kernel: str):
    """HBM bytes per launch from committed rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE
    passes, only if the kernel source is unchanged since they were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_digest") != source_digest(kernel):
        return None
    return rec.get("bytes_per_launch")


def time_calls(torch, fn, steps, warmup, rotate=1):
    """Run fn(i) warmup + steps times back to back; return the average milliseconds per
    call over the timed region (HIP events on the current stream before the first and
    after the last timed call only, so launch gaps count against the kernel but no event
    sits between two calls), the best per-call average of five further untimed runs of
    ten calls each (timed the same way), and the wall time of the timed region."""
    for i in range(warmup):
        fn(i % rotate)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        fn(i % rotate)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    region = e0.elapsed_time(e1)
    fastest = float("inf")
    for _ in range(5):
        e0.record(stream)
        for i in range(10):
            fn(i % rotate)
        e1.record(stream)
        torch.cuda.synchronize()
        fastest = min(fastest, e0.elapsed_time(e1) / 10)
    return region / steps, fastest, wall


LATENT_SWEEP = (1, 2, 4, 7, 8, 16)
SWEEP_UNTIMED, SWEEP_TIMED, SWEEP_AFTER = 20, 40, 50  # time_calls adds five 10-call runs


def lib_ranges(N, requested):
    """Key ranges the latent decode uses when `requested` are asked for (rounded to whole
    32-row tiles, none empty)."""
    rows = -(-N // requested)
    rows = -(-rows // 32) * 32
    return -(-N // rows)


def summarize_sweep(d, name, cmd):
    """Per-kernel kernel-trace durations of the latent decode range sweep: calls are three
    launches each; per range count (in LATENT_SWEEP order, after the benchmark's own calls)
    SWEEP_UNTIMED warm-up calls, SWEEP_TIMED timed ones and SWEEP_AFTER more; the averages
    cover the timed calls."""
    seq = sorted((int(r["Start_Timestamp"]), r["Kernel_Name"],
                  int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
                 for r in _read_csvs(d, "kernel_trace.csv") if "latent_" in r["Kernel_Name"])
    per = (SWEEP_UNTIMED + SWEEP_TIMED + SWEEP_AFTER) * 3
    block = seq[len(seq) - per * len(LATENT_SWEEP):]
    lines = [f"# {name}", "", "Command:", "", "```", cmd, "```", "",
             "Latent-cache decode B8 H96 N1001 d_c 512 at several key-range counts; "
             f"kernel-trace averages (us) over {SWEEP_TIMED} timed calls each.", "",
             "| ranges | absorb | split | merge | sum |", "|---|---|---|---|---|"]
    for j, sp in enumerate(LATENT_SWEEP):
        calls = block[j * per:(j + 1) * per][SWEEP_UNTIMED * 3:(SWEEP_UNTIMED + SWEEP_TIMED) * 3]
        avg = {}
        for part in ("absorb", "split", "merge"):
            v = [x[2] for x in calls if f"latent_{part}" in x[1]]
            avg[part] = sum(v) / len(v) / 1e3
        used = lib_ranges(1001, sp)
        lines.append(f"| {used} | {avg['absorb']:.1f} | {avg['split']:.1f} | {avg['merge']:.1f} | "
                     f"{sum(avg.values()):.1f} |")
    os.makedirs(PROFILES, exist_ok=True)
    out = os.path.join(PROFILES, f"{name}.md")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(out)


def settle(torch, fn, seconds):
    """Call fn back to back for about `seconds`, untimed.  From idle, a GPU's first few
    dozen calls of sustained matrix-core work run up to 30% slower than the rest while its
    power management brings the clock from the idle boost down to the sustained level and
    back up (traced per dispatch: 804, 919, 1055, ... 790 us for the prefill workload);
    this puts the timed calls after that transient.  Returns the number of calls."""
    if seconds <= 0:
        return 0
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            fn(0)
        n += 20
        torch.cuda.synchronize()
    return n


def loop_calls(torch, fn, seconds, work, unit):
    """Call fn back to back for about `seconds`, printing the rate of each 20-call batch
    every half second (for sampling clocks or power from another process meanwhile)."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = last = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        e0.record()
        for i in range(20):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        if time.perf_counter() - last > 0.5:
            last = time.perf_counter()
            rate = work * 20 / (e0.elapsed_time(e1) * 1e-3) / (1e12 if unit == "TFLOP/s" else 1e9)
            print(json.dumps({"t": round(last - t0, 2), "value": round(rate, 1), "unit": unit}),
                  flush=True)


def measure_achievable(torch, dev):
    """What the device reaches on this run: a register-only MFMA loop (bf16, two waves
    per SIMD) and a plain non-temporal streaming read of 2 GiB (libgmla_probe.so)."""
    import ctypes

    path = os.path.join(HERE, "causal_softmax_attention_gmla_amd", "libgmla_probe.so")
    lib = ctypes.CDLL(path)
    lib.gmla_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.gmla_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                    ctypes.c_void_p, ctypes.c_void_p]
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    blocks, iters = 512, 2000
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    flops = blocks * 4 * iters * 16 * 32 * 32 * 16 * 2

    def mfma(i):
        assert lib.gmla_probe_mfma(blocks, iters, ctypes.c_void_p(out.data_ptr()), sp) == 0

    # ~60 ms of warm-up: the clock the matrix cores hold settles only under sustained load
    mavg, _, _ = time_calls(torch, mfma, 20, 60)
    lib.gmla_probe_mfma_random.argtypes = lib.gmla_probe_mfma.argtypes

    def mfma_random(i):
        assert lib.gmla_probe_mfma_random(blocks, iters, ctypes.c_void_p(out.data_ptr()), sp) == 0

    ravg_m, _, _ = time_calls(torch, mfma_random, 20, 60)
    nbytes = 2 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    rblocks = 2048
    rout = torch.empty(rblocks, dtype=torch.int32, device=dev)

    def read(i):
        assert lib.gmla_probe_read(ctypes.c_void_p(buf.data_ptr()), nbytes, rblocks,
                                   ctypes.c_void_p(rout.data_ptr()), sp) == 0

    ravg, _, _ = time_calls(torch, read, 10, 10)
    del buf
    return {"mfma_bf16_tflops": round(flops / (mavg * 1e-3) / 1e12, 1),
            "mfma_bf16_random_tflops": round(flops / (ravg_m * 1e-3) / 1e12, 1),
            "hbm_read_gbps": round(nbytes / (ravg * 1e-3) / 1e9, 1),
            "how": "libgmla_probe.so: register-only v_mfma_f32_32x32x16_bf16 loop (512 x 256 "
                   "threads, 4 chains per wave) on constant operands and on eight rotating sets "
                   "of random bf16 operands; 2 GiB non-temporal 16-byte read stream"}


def host_cpu():
    """The host's CPU model, its logical CPU count, and the CPUs this process may use."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    return {"cpu_model": model, "nproc": os.cpu_count(), "usable_cpus": usable}


def cpu_prefill_baseline(q, k, v, budget_s=12.0):
    """The oracle on whole, distinct heads of the prefill workload (a seeded order over all
    (batch, head) pairs, none repeated) until ~budget_s of CPU time or every head is done."""
    import numpy as np

    import oracle
    B, T, H, D = q.shape
    threads = oracle.default_threads()
    oracle.load()
    order = np.random.default_rng(0).permutation(B * H)
    done_flops, heads, t0 = 0, 0, time.perf_counter()
    for idx in order:
        b, h = divmod(int(idx), H)
        qh = q[b, :, h].float().cpu().numpy()
        kh = k[b, :, h].float().cpu().numpy()
        vh = v[b, :, h].float().cpu().numpy()
        oracle.attend_head(qh, kh, vh, 1.0 / math.sqrt(D), True, nthreads=threads)
        done_flops += prefill_flops(1, T, 1, D)
        heads += 1
        if time.perf_counter() - t0 > budget_s:
            break
    el = time.perf_counter() - t0
    return {"value": round(done_flops / el / 1e12, 5), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", **host_cpu(),
            "sample": f"{heads} distinct of {B * H} (batch, head) pairs, all {T} query rows each, of "
                      f"the prefill workload, {el:.1f} s including host copies, float64, "
                      f"{threads} threads over query rows"}


def cpu_decode_baseline(q, k, v, budget_s=6.0):
    """The oracle on distinct (batch, head) decode rows of the 1001-key workload, the rows
    spread over a thread pool (the oracle runs one query row per call; its C code releases
    the interpreter lock), until ~budget_s or every row is done."""
    import concurrent.futures as cf

    import numpy as np

    import oracle
    B, H, N, D = k.shape
    threads = oracle.default_threads()
    oracle.load()
    kh_all = k.float().cpu().numpy()
    vh_all = v.float().cpu().numpy()
    qh_all = q.float().cpu().numpy()
    order = [divmod(int(i), H) for i in np.random.default_rng(0).permutation(B * H)]
    t0 = time.perf_counter()
    heads = 0
    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        for c0 in range(0, len(order), 4 * threads):
            chunk = order[c0:c0 + 4 * threads]
            list(ex.map(lambda bh: oracle.attend_head(qh_all[bh[0], bh[1]][None], kh_all[bh[0], bh[1]],
                                                      vh_all[bh[0], bh[1]], 1.0 / math.sqrt(D), True,
                                                      nthreads=1), chunk))
            heads += len(chunk)
            if time.perf_counter() - t0 > budget_s:
                break
    el = time.perf_counter() - t0
    nbytes = decode_bytes(1, 1, N, D) * heads
    return {"value": round(nbytes / el / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            **host_cpu(),
            "sample": f"{heads} distinct of {B * H} (batch, head) decode rows of {N} keys, {el:.1f} s, "
                      f"float64, {threads} threads (one row per call)"}


# ----------------------------------------------------------------------------- profiles


def _read_csvs(d, suffix):
    rows = []
    for f in sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)):
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def _short(name: str) -> str:
    name = name.replace("(anonymous namespace)", "{anon}").split("(")[0]
    return name if len(name) < 90 else name[:87] + "..."


def _bench_line(log):
    """The benchmark's JSON line from the log of the profiled run."""
    with open(log) as f:
        lines = [l for l in f if l.startswith("{")]
    if not lines:
        sys.exit(f"no JSON line in {log}")
    return lines[-1].strip()


def summarize_stats(d, name, cmd, window=None, log=None):
    rows = _read_csvs(d, "kernel_stats.csv")
    if not rows:
        sys.exit(f"no *kernel_stats.csv under {d}")
    lines = [f"# {name}", "", "Command:", "", "```", cmd, "```", "",
             "| kernel | calls | average (us) | min (us) | max (us) | share (%) |",
             "|---|---|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: -float(r.get("Percentage", 0))):
        ns = lambda k: float(r.get(k, "nan")) / 1e3  # noqa: E731
        lines.append(f"| {_short(r['Name'])} | {r['Calls']} | {ns('AverageNs'):.1f} | "
                     f"{ns('MinNs'):.1f} | {ns('MaxNs'):.1f} | {float(r['Percentage']):.2f} |")
    if window:
        # The statistics above average every dispatch, the warm-up calls included (a fresh
        # GPU runs its first calls slower while the clocks settle); the timed region of
        # bench.py is dispatches W .. W+K-1 of each kernel, in launch order.
        w, k = window
        per = {}
        for r in _read_csvs(d, "kernel_trace.csv"):
            per.setdefault(r["Kernel_Name"], []).append(
                (int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
        lines += ["", f"Dispatches {w} .. {w + k - 1} of each library kernel launched at least "
                      f"{w + k} times (the timed calls after {w} warm-up calls), from the kernel "
                      f"trace:", "",
                  "| kernel | warm-up average (us) | timed average (us) |", "|---|---|---|"]
        for kname, v in sorted(per.items(), key=lambda kv: -sum(x[1] for x in kv[1])):
            if len(v) < w + k or "gmla" not in kname:
                continue
            v.sort()
            warm = sum(x[1] for x in v[:w]) / max(w, 1) / 1e3
            timed = sum(x[1] for x in v[w:w + k]) / k / 1e3
            lines.append(f"| {_short(kname)} | {warm:.1f} | {timed:.1f} |")
    # a library kernel that serves several shapes (one launch grid each), per grid
    grids = {}
    for r in _read_csvs(d, "kernel_trace.csv"):
        if "gmla" not in r["Kernel_Name"]:
            continue
        wg = int(r["Grid_Size_X"]) // max(int(r["Workgroup_Size_X"]), 1)
        grids.setdefault(r["Kernel_Name"], {}).setdefault(wg, []).append(
            int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    multi = {k: v for k, v in grids.items() if len(v) > 1}
    if multi:
        lines += ["", "Library kernels launched with more than one grid, per grid size (from the "
                      "kernel trace):", "", "| kernel | workgroups | calls | average (us) |",
                  "|---|---|---|---|"]
        for kname, per in sorted(multi.items()):
            for wg, v in sorted(per.items()):
                lines.append(f"| {_short(kname)} | {wg} | {len(v)} | {sum(v) / len(v) / 1e3:.1f} |")
    if log:
        lines += ["", "The benchmark's own line from the same run (event timing; under the "
                      "profiler):", "", "```", _bench_line(log), "```"]
    os.makedirs(PROFILES, exist_ok=True)
    out = os.path.join(PROFILES, f"{name}.md")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(out)


def _counter_per_dispatch(d, counter, match):
    vals = {}
    for r in _read_csvs(d, "counter_collection.csv"):
        if r["Counter_Name"] != counter or match not in r["Kernel_Name"]:
            continue
        key = r["Dispatch_Id"]
        vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
    if not vals:
        sys.exit(f"no {counter} for {match} under {d}")
    ordered = [vals[k] for k in sorted(vals, key=int)]
    return ordered[-1], len(ordered)  # last dispatch: warm caches, steady state


def summarize_traffic(d_fetch, d_write, c_fetch, c_write, kernel, cmd, key=None):
    kf, _ = _counter_per_dispatch(d_fetch, "FETCH_SIZE", kernel)
    kw, _ = _counter_per_dispatch(d_write, "WRITE_SIZE", kernel)
    cf, _ = _counter_per_dispatch(c_fetch, "FETCH_SIZE", "copyBuffer")
    cw, _ = _counter_per_dispatch(c_write, "WRITE_SIZE", "copyBuffer")
    # each counter reads in KiB; a plain copy of COPY_BYTES fixes its scale
    fetch_scale = COPY_BYTES / (cf * 1024.0)
    write_scale = COPY_BYTES / (cw * 1024.0)
    fetch = kf * 1024.0 * fetch_scale
    write = kw * 1024.0 * write_scale
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        data = {}
    key = key or kernel
    data[key] = {"source_digest": source_digest(kernel), "bytes_per_launch": round(fetch + write),
                    "fetch_bytes": round(fetch), "write_bytes": round(write),
                    "fetch_scale": round(fetch_scale, 4), "write_scale": round(write_scale, 4),
                    "raw_fetch_kib": kf, "raw_write_kib": kw, "copy_fetch_kib": cf,
                    "copy_write_kib": cw, "command": cmd}
    os.makedirs(PROFILES, exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
    print(json.dumps(data[key]))


def summarize_counters(d, kernel, name, cmd):
    """Every counter of the last dispatch of `kernel` in a --pmc pass, as a table."""
    vals, last = {}, None
    for r in _read_csvs(d, "counter_collection.csv"):
        if kernel not in r["Kernel_Name"]:
            continue
        did = int(r["Dispatch_Id"])
        if last is None or did > last:
            last, vals = did, {}
        if did == last:
            vals[r["Counter_Name"]] = vals.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    if not vals:
        sys.exit(f"no counters for {kernel} under {d}")
    lines = [f"# {name}", "", f"Counters of the last dispatch of `{kernel}` (dispatch {last}).", "",
             "Command:", "", "```", cmd, "```", "", "| counter | value |", "|---|---|"]
    lines += [f"| {k} | {v:.6g} |" for k, v in sorted(vals.items())]
    os.makedirs(PROFILES, exist_ok=True)
    out = os.path.join(PROFILES, f"{name}.md")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(out)


def summarize_ramp(dirs, labels, name, cmd, n=60):
    """Per-dispatch durations of the first n prefill launches of each run (a GPU starting
    from idle), side by side, from kernel traces."""
    cols = []
    for d in dirs:
        v = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
                   for r in _read_csvs(d, "kernel_trace.csv") if "prefill_bf16_kernel" in r["Kernel_Name"])
        if len(v) < n:
            sys.exit(f"fewer than {n} prefill dispatches under {d}")
        cols.append([x[1] / 1e3 for x in v[:n]])
    lines = [f"# {name}", "", "Command:", "", "```", cmd, "```", "",
             "Duration (us) of the first prefill launches after an idle GPU, in launch order.", "",
             "| launch | " + " | ".join(labels) + " |", "|---" * (len(labels) + 1) + "|"]
    for i in range(n):
        lines.append(f"| {i} | " + " | ".join(f"{c[i]:.1f}" for c in cols) + " |")
    lines += ["", "| mean of launches | " + " | ".join(labels) + " |", "|---" * (len(labels) + 1) + "|"]
    for a, b in ((0, 10), (10, 40), (40, n)):
        lines.append(f"| {a} .. {b - 1} | " + " | ".join(f"{sum(c[a:b]) / (b - a):.1f}" for c in cols) + " |")
    os.makedirs(PROFILES, exist_ok=True)
    out = os.path.join(PROFILES, f"{name}.md")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(out)


def summarize_mfma(d, name, cmd):
    """MFMA utilisation of every GPU kernel in a --pmc pass with SQ_VALU_MFMA_BUSY_CYCLES
    and GRBM_GUI_ACTIVE: busy cycles summed over the 1024 SIMDs, against the dispatch's
    active cycles (GRBM_GUI_ACTIVE sums the 8 XCDs), for the last dispatch of each."""
    per = {}
    for r in _read_csvs(d, "counter_collection.csv"):
        k, did = _short(r["Kernel_Name"]), int(r["Dispatch_Id"])
        slot = per.setdefault(k, {})
        if slot.get("id", -1) < did:
            per[k] = slot = {"id": did}
        if slot["id"] == did:
            slot[r["Counter_Name"]] = slot.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    lines = [f"# {name}", "", "Command:", "", "```", cmd, "```", "",
             "MFMA utilisation = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE / 8 XCDs), "
             "last dispatch of each kernel.", "",
             "| kernel | MFMA instructions | MFMA busy | GRBM active | MFMA utilisation |",
             "|---|---|---|---|---|"]
    for k, v in sorted(per.items(), key=lambda kv: -kv[1].get("SQ_VALU_MFMA_BUSY_CYCLES", 0)):
        busy, act = v.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0), v.get("GRBM_GUI_ACTIVE", 0.0)
        if busy <= 0 or act <= 0:
            continue
        util = busy / (1024.0 * act / 8.0)
        lines.append(f"| {k} | {v.get('SQ_INSTS_MFMA', 0):.4g} | {busy:.4g} | {act:.4g} | {util:.1%} |")
    os.makedirs(PROFILES, exist_ok=True)
    out = os.path.join(PROFILES, f"{name}.md")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(out)


# ----------------------------------------------------------------------------- main


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # A fresh GPU runs the first few dozen prefill calls up to 30% slower while its clocks
    # settle under sustained matrix-core load; 60 untimed calls reach the steady state.
    ap.add_argument("--warmup", type=int, default=60)
    ap.add_argument("--settle", type=float, default=0.5,
                    help="seconds of untimed prefill calls before the warm-up (0: none)")
    ap.add_argument("--all", action="store_true", help="also time the layer, the 131072-key decode and the latent-cache decode")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--decode-splits", type=int, default=0)
    ap.add_argument("--only", choices=["prefill", "decode", "layer", "decode_long", "decode_latent",
                                       "gate_out", "copy"])
    ap.add_argument("--summarize-stats", metavar="DIR")
    ap.add_argument("--timed-window", nargs=2, type=int, metavar=("W", "K"),
                    help="with --summarize-stats: also average dispatches W .. W+K-1 per kernel")
    ap.add_argument("--summarize-traffic", nargs=4, metavar="DIR")
    ap.add_argument("--summarize-counters", metavar="DIR")
    ap.add_argument("--summarize-mfma", metavar="DIR")
    ap.add_argument("--summarize-ramp", nargs="+", metavar="DIR=LABEL",
                    help="first prefill dispatches of each kernel-trace directory, side by side")
    ap.add_argument("--latent-sweep", action="store_true",
                    help="with --only decode_latent: also time key-range counts " + str(LATENT_SWEEP))
    ap.add_argument("--summarize-sweep", metavar="DIR")
    ap.add_argument("--zero-inputs", action="store_true",
                    help="with --only prefill: all-zero Q, K and V (a diagnostic: the same work on "
                         "data that draws little power)")
    ap.add_argument("--loop", type=float, metavar="SECONDS",
                    help="with --only prefill: call it back to back for SECONDS, printing rates")
    ap.add_argument("--name")
    ap.add_argument("--kernel")
    ap.add_argument("--key", help="record name in traffic.json (default: the kernel)")
    ap.add_argument("--cmd", default="")
    ap.add_argument("--log", help="with --summarize-stats: the profiled run's output, whose JSON "
                                  "line is appended")
    args = ap.parse_args()
    if args.summarize_stats:
        return summarize_stats(args.summarize_stats, args.name, args.cmd, args.timed_window, args.log)
    if args.summarize_traffic:
        return summarize_traffic(*args.summarize_traffic, args.kernel, args.cmd, args.key)
    if args.summarize_counters:
        return summarize_counters(args.summarize_counters, args.kernel, args.name, args.cmd)
    if args.summarize_mfma:
        return summarize_mfma(args.summarize_mfma, args.name, args.cmd)
    if args.summarize_sweep:
        return summarize_sweep(args.summarize_sweep, args.name, args.cmd)
    if args.summarize_ramp:
        pairs = [a.split("=", 1) for a in args.summarize_ramp]
        return summarize_ramp([p[0] for p in pairs], [p[1] for p in pairs], args.name, args.cmd)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU "
              f"sharding is described, not built.", file=sys.stderr)
        sys.exit(2)

    import torch

    import causal_softmax_attention_gmla_amd as gm
    from causal_softmax_attention_gmla_amd import inputs as I

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    gm.library()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    K, W = args.steps, args.warmup
    only = args.only

    if only == "copy":  # scale reference for the FETCH_SIZE / WRITE_SIZE counters
        a = torch.ones(COPY_BYTES, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(max(K, 1)):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": COPY_BYTES, "copies": max(K, 1)}))
        return

    result = {"metric": METRIC, "unit": "TFLOP/s", "n_gpus": 1, "steps": K, "warmup": W,
              "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
              "data": "synthetic"}

    # ---------------- prefill: B=2 T=4096 H=96 D=128 bf16, causal
    q = k = v = None
    if only in (None, "prefill"):
        pw = I.WORKLOADS["prefill_b2_t4096"]
        d = pw.dims
        q, k, v, _ = I.workload_inputs(pw.name, dev)
        if args.zero_inputs:
            if only != "prefill":
                sys.exit("--zero-inputs is a diagnostic for --only prefill")
            q.zero_(), k.zero_(), v.zero_()
        out = torch.empty((d["B"], d["T"], d["H"] * d["D"]), dtype=q.dtype, device=dev)
        flops = prefill_flops(d["B"], d["T"], d["H"], d["D"])
        if args.loop:
            return loop_calls(torch, lambda i: gm.attend_prefill(q, k, v, out=out), args.loop,
                              flops, "TFLOP/s")
        settle_calls = settle(torch, lambda i: gm.attend_prefill(q, k, v, out=out), args.settle)
        avg, fastest, wall = time_calls(torch, lambda i: gm.attend_prefill(q, k, v, out=out), K, W)
        tflops = flops / (avg * 1e-3) / 1e12
        result.update({
            "value": round(tflops, 2), "ms_per_step": round(wall * 1e3 / K, 4),
            "config": {"workload": pw.name, "B": d["B"], "T": d["T"], "H": d["H"], "D": d["D"],
                       "causal": True, "inputs": "all zero (diagnostic)" if args.zero_inputs else "N(0,1) rounded to bf16, seeded"},
            "clock_settle": {"seconds": args.settle, "calls": settle_calls,
                             "note": "untimed back-to-back calls before the warm-up, so that the "
                                     "timed calls run at the sustained clock"},
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                         "traffic": measured_traffic("prefill_bf16_kernel"),
                         "kernel": "prefill_bf16_kernel", "algorithmic_flop_per_launch": flops,
                         "avg_launch_ms": round(avg, 4), "best_10_launch_ms": round(fastest, 4)},
        })

    # ---------------- decode: B=8 H=96 N=1001 D=128 bf16, rotated over 4 input sets
    sets = None
    if only in (None, "decode"):
        dw = I.WORKLOADS["decode_b8_n1001"]
        dd = dw.dims
        sets = []
        for r in range(4):
            qd, kd, vd, _ = I.decode_inputs(dd["B"], dd["H"], dd["N"], dd["D"], dw.dtype, dev,
                                            seed=I.seed_of(dw.name) + 10 * r)
            sets.append((qd, kd, vd, torch.empty((dd["B"], dd["H"] * dd["D"]), dtype=dw.dtype,
                                                 device=dev)))
        splits = args.decode_splits or gm.decode_num_splits(dd["B"], dd["H"], dd["N"], dd["D"])
        wsb = gm.decode_workspace_bytes(dd["B"], dd["H"], dd["N"], dd["D"], splits)
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
        nbytes = decode_bytes(dd["B"], dd["H"], dd["N"], dd["D"])

        def dec(i):
            qd, kd, vd, od = sets[i]
            gm.attend_decode(qd, kd, vd, num_splits=splits, workspace=ws, out=od)

        dcalls = max(K, 20)
        davg, dfast, dwall = time_calls(torch, dec, dcalls, W, rotate=4)
        gbps = nbytes / (davg * 1e-3) / 1e9
        result["decode"] = {
            "workload": dw.name, "value": round(gbps, 1), "unit": "GB/s", "splits": splits,
            "calls": dcalls, "avg_call_ms": round(davg, 5), "best_10_call_ms": round(dfast, 5),
            "rotation": "4 input sets (1.58 GB) cycled so the 256 MB last-level cache cannot hold them",
            "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS,
                         "unit": "GB/s", "frac": round(gbps / PEAK_HBM_GBPS, 4),
                         "traffic": measured_traffic("decode_split_kernel"),
                         "kernel": "decode_split_kernel" + (" + decode_merge_kernel" if splits > 1 else ""),
                         "algorithmic_bytes_per_call": nbytes},
        }
        if only == "decode":
            result.update({"value": round(gbps, 1), "unit": "GB/s",
                           "ms_per_step": round(dwall * 1e3 / dcalls, 4)})

    if args.all or only in ("layer", "decode_long", "decode_latent", "gate_out"):
        extra = {}
        if only == "gate_out":
            # the output projection with the gate applied in the GEMM prologue (one launch
            # of the register-staged kernel) against the gate applied by its own kernel and
            # the LDS-pipelined GEMM (two launches), at the layer's shape
            M_, dm_ = 2048, 12288
            o_ = I.normal((M_, dm_), torch.bfloat16, dev, seed=7201)
            g_ = I.normal((M_, dm_), torch.bfloat16, dev, seed=7202)
            w_ = I.normal((dm_, dm_), torch.bfloat16, dev, seed=7203, std=dm_ ** -0.5)
            gflop = 2 * M_ * dm_ * dm_
            a1, _, _ = time_calls(torch, lambda i: gm.gate_out(o_, w_, g_, fused_gate=True),
                                  max(5, K // 5), max(2, W // 3))
            a2, _, _ = time_calls(torch, lambda i: gm.gate_out(o_, w_, g_), max(5, K // 5), max(2, W // 3))
            extra["gate_out_t2048"] = {
                "prologue_gate_ms": round(a1, 4), "prologue_gate_tflops": round(gflop / (a1 * 1e-3) / 1e12, 1),
                "separate_gate_ms": round(a2, 4), "separate_gate_tflops": round(gflop / (a2 * 1e-3) / 1e12, 1),
                "algorithmic_flop": gflop}
            del o_, g_, w_
        if only in (None, "layer"):
            lw = I.WORKLOADS["layer_t2048"]
            ld = lw.dims
            x, wts = I.workload_inputs(lw.name, dev)
            largs = (x, wts["Wq"], wts["Wc"], wts["Wk"], wts["Wv"], wts["Wg"], wts["Wo"], ld["H"], True)
            # both forms timed at the sustained clock (otherwise the first one timed also
            # pays for the clock's settling)
            settle(torch, lambda i: gm.gated_mla(*largs), args.settle)
            lavg, _, _ = time_calls(torch, lambda i: gm.gated_mla(*largs), max(5, K // 5),
                                    max(2, W // 3))
            favg, _, _ = time_calls(torch, lambda i: gm.gated_mla(*largs, fused_latent=True),
                                    max(5, K // 5), max(2, W // 3))
            T_, dm, dc = ld["T"], ld["d_model"], ld["d_c"]
            lflops = 2 * T_ * (3 * dm * dm + 3 * dm * dc) + prefill_flops(1, T_, ld["H"], dm // ld["H"])
            extra[lw.name] = {"value": round(lflops / (lavg * 1e-3) / 1e12, 1), "unit": "TFLOP/s",
                              "frac": round(lflops / (lavg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                              "avg_call_ms": round(lavg, 4), "algorithmic_flop": lflops,
                              "fused_latent": {"value": round(lflops / (favg * 1e-3) / 1e12, 1),
                                               "avg_call_ms": round(favg, 4),
                                               "note": "keys and values rebuilt from the latent "
                                                       "inside the attention launch"}}
            del x, wts
        if only in (None, "decode_long"):
            cw = I.WORKLOADS["decode_b4_n131072"]
            cd = cw.dims
            qc, kc, vc, _ = I.workload_inputs(cw.name, dev)
            cavg, _, _ = time_calls(torch, lambda i: gm.attend_decode(qc, kc, vc), max(5, K // 5),
                                    max(2, W // 10))
            cb = decode_bytes(cd["B"], cd["H"], cd["N"], cd["D"])
            extra[cw.name] = {"value": round(cb / (cavg * 1e-3) / 1e9, 1), "unit": "GB/s",
                              "frac": round(cb / (cavg * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                              "avg_call_ms": round(cavg, 4), "algorithmic_bytes": cb,
                              "splits": gm.decode_num_splits(cd["B"], cd["H"], cd["N"], cd["D"])}
            del qc, kc, vc
        if only in (None, "decode_latent"):
            # decode over the latent cache at the 1001-key shape: C [8, 1001, 512] is the whole
            # cache; keys and values are never formed.  Eight input sets (cache and both
            # up-projections, 34 MB each) rotate so the 256 MB last-level cache cannot hold
            # them, as W_k and W_v would come from HBM in a model's decode step.
            B_, N_, H_, D_, dc = 8, 1001, 96, 128, 512
            lsets = []
            for r in range(8):
                lsets.append((I.normal((B_, H_, D_), torch.bfloat16, dev, seed=7001 + 10 * r),
                              I.normal((B_, N_, dc), torch.bfloat16, dev, seed=7002 + 10 * r),
                              I.normal((H_ * D_, dc), torch.bfloat16, dev, seed=7003 + 10 * r,
                                       std=dc ** -0.5),
                              I.normal((H_ * D_, dc), torch.bfloat16, dev, seed=7004 + 10 * r,
                                       std=dc ** -0.5),
                              torch.empty((B_, H_ * D_), dtype=torch.bfloat16, device=dev)))
            lws = torch.empty(gm.decode_latent_workspace_bytes(B_, H_, N_, dc), dtype=torch.uint8,
                              device=dev)

            def dec_lat(i):
                ql, cl, wkl, wvl, ol = lsets[i]
                gm.attend_decode_latent(ql, cl, wkl, wvl, workspace=lws, out=ol)

            lcalls = max(K, 20)
            lavg2, lfast2, _ = time_calls(torch, dec_lat, lcalls, max(W, 5), rotate=8)
            lbytes = (B_ * N_ * dc + 2 * H_ * D_ * dc + 2 * B_ * H_ * D_) * 2
            lflop = 2 * B_ * H_ * N_ * dc * 2 + 2 * B_ * H_ * D_ * dc * 2
            # A decode loop replays captured launches: the eight rotated calls also go into
            # one HIP graph, replayed back to back.  Equal eager and replayed rates show that
            # the host issuing the three launches per call is not what limits the eager rate.
            graph = torch.cuda.CUDAGraph()
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                for i in range(8):
                    dec_lat(i)  # the calls run once eagerly before capture
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            with torch.cuda.graph(graph):
                for i in range(8):
                    dec_lat(i)
            reps = max(lcalls // 8, 4)
            gavg, gfast, _ = time_calls(torch, lambda i: graph.replay(), reps, 3)
            gavg, gfast = gavg / 8, gfast / 8
            extra["decode_latent_b8_n1001"] = {
                "value": round(lbytes / (lavg2 * 1e-3) / 1e9, 1), "unit": "GB/s",
                "avg_call_ms": round(lavg2, 5), "best_10_call_ms": round(lfast2, 5),
                "algorithmic_bytes_per_call": lbytes, "algorithmic_flop_per_call": lflop,
                "splits": gm.decode_latent_num_splits(B_, H_, N_, dc),
                "roofline": {"bound": "hbm", "achieved": round(lbytes / (lavg2 * 1e-3) / 1e9, 1),
                             "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                             "frac": round(lbytes / (lavg2 * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)},
                "graph_replay": {"value": round(lbytes / (gavg * 1e-3) / 1e9, 1), "unit": "GB/s",
                                 "avg_call_ms": round(gavg, 5), "best_10_call_ms": round(gfast, 5),
                                 "frac": round(lbytes / (gavg * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                                 "how": "the 8 rotated calls captured in one HIP graph, replayed "
                                        f"{reps} times; per-call time = replay time / 8"},
                "cache_bytes_per_token": dc * 2, "direct_decode_cache_bytes_per_token": 2 * H_ * D_ * 2,
                "rotation": "8 input sets (270 MB) cycled",
                "note": "latent cache + W_k + W_v read per call (keys and values never formed): "
                        "absorb, split attention over the latent rows, merge + W_v"}
            if args.latent_sweep:
                # the same call at several key-range counts: 20 untimed and 40 timed calls
                # each, in this order (the kernel trace of such a run is grouped by
                # --summarize-sweep)
                sweep = []
                for sp in LATENT_SWEEP:
                    sws = torch.empty(gm.decode_latent_workspace_bytes(B_, H_, N_, dc, sp),
                                      dtype=torch.uint8, device=dev)

                    def dec_sp(i, sp=sp, sws=sws):
                        ql, cl, wkl, wvl, ol = lsets[i]
                        gm.attend_decode_latent(ql, cl, wkl, wvl, workspace=sws, out=ol,
                                                num_splits=sp)

                    savg, _, _ = time_calls(torch, dec_sp, SWEEP_TIMED, SWEEP_UNTIMED, rotate=8)
                    used = lib_ranges(N_, sp)
                    sweep.append({"ranges_requested": sp, "ranges": used,
                                  "avg_call_ms": round(savg, 5)})
                extra["decode_latent_range_sweep"] = sweep
            del lsets, lws, graph
        result["extra"] = extra

    if not args.no_cpu and only is None:
        result["cpu_baseline"] = cpu_prefill_baseline(q, k, v)
        qd, kd, vd, _ = sets[0]
        result["decode"]["cpu_baseline"] = cpu_decode_baseline(qd, kd, vd)

    if only in (None, "prefill", "decode"):
        ach = measure_achievable(torch, dev)
        if "roofline" in result:
            result["roofline"]["achievable"] = ach["mfma_bf16_tflops"]
            result["roofline"]["frac_of_achievable"] = round(
                result["roofline"]["achieved"] / ach["mfma_bf16_tflops"], 4)
            result["roofline"]["achievable_random_operands"] = ach["mfma_bf16_random_tflops"]
            result["roofline"]["frac_of_achievable_random_operands"] = round(
                result["roofline"]["achieved"] / ach["mfma_bf16_random_tflops"], 4)
        if "decode" in result:
            rl = result["decode"]["roofline"]
            rl["achievable"] = ach["hbm_read_gbps"]
            rl["frac_of_achievable"] = round(rl["achieved"] / ach["hbm_read_gbps"], 4)
        result["achievable"] = ach

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
