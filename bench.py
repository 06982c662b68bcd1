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
"""
from __future__ import annotations

import argparse
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
TRAFFIC_FILE = os.path.join(HERE, "profiles", "traffic.json")


def prefill_flops(B, T, H, D):
    # QK^T and PV over the T(T+1)/2 visible (query, key) pairs: 2 * 2 * D flop each
    return 4 * D * B * H * T * (T + 1) // 2


def decode_bytes(B, H, N, D, elem=2):
    # every K and V row once, plus Q in and O out
    return (2 * B * H * N * D + 2 * B * H * D) * elem


def source_digest(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(HERE, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, files):
    """HBM bytes per launch from committed rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs,
    only if the kernel source is unchanged since they were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_digest") != source_digest(files):
        return None
    return rec.get("bytes_per_launch")


def time_calls(torch, fn, steps, warmup, rotate=1):
    """Run fn(i) warmup + steps times; return per-call milliseconds of the timed calls
    (HIP events on the current stream) and the wall time of the timed region."""
    for i in range(warmup):
        fn(i % rotate)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        evs[i][0].record(stream)
        fn(i % rotate)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return [a.elapsed_time(b) for a, b in evs], wall


def cpu_prefill_baseline(q, k, v, budget_s=12.0):
    """The oracle on whole heads of the prefill workload until ~budget_s of CPU time."""
    import numpy as np

    import oracle
    B, T, H, D = q.shape
    threads = oracle.default_threads()
    oracle.load()
    done_flops, heads, t0 = 0, 0, time.perf_counter()
    rng = np.random.default_rng(0)
    while True:
        b, h = int(rng.integers(B)), int(rng.integers(H))
        qh = q[b, :, h].float().cpu().numpy()
        kh = k[b, :, h].float().cpu().numpy()
        vh = v[b, :, h].float().cpu().numpy()
        ts = time.perf_counter()
        oracle.attend_head(qh, kh, vh, 1.0 / math.sqrt(D), True, nthreads=threads)
        done_flops += prefill_flops(1, T, 1, D)
        heads += 1
        if time.perf_counter() - t0 > budget_s or heads >= B * H:
            break
        _ = ts
    el = time.perf_counter() - t0
    return {"value": done_flops / el / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{heads} of {B * H} heads (all {T} query rows each) of the prefill workload, "
                      f"{el:.1f} s, float64, {threads} threads"}


def cpu_decode_baseline(q, k, v, budget_s=6.0):
    import numpy as np

    import oracle
    B, H, N, D = k.shape
    threads = oracle.default_threads()
    oracle.load()
    kh_all = k.float().cpu().numpy()
    vh_all = v.float().cpu().numpy()
    qh_all = q.float().cpu().numpy()
    nbytes, heads, t0 = 0, 0, time.perf_counter()
    rng = np.random.default_rng(0)
    while True:
        b, h = int(rng.integers(B)), int(rng.integers(H))
        oracle.attend_head(qh_all[b, h][None], kh_all[b, h], vh_all[b, h], 1.0 / math.sqrt(D), True,
                           nthreads=1)
        nbytes += decode_bytes(1, 1, N, D)
        heads += 1
        if time.perf_counter() - t0 > budget_s or heads >= 4 * B * H:
            break
    el = time.perf_counter() - t0
    return {"value": nbytes / el / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{heads} (batch, head) decode rows of 1001 keys, {el:.1f} s, float64, 1 thread "
                      f"(one query row cannot be split across threads by the oracle)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--all", action="store_true", help="also time the layer and the 131072-key decode")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--decode-splits", type=int, default=0)
    args = ap.parse_args()
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

    # ---------------- prefill: B=2 T=4096 H=96 D=128 bf16, causal
    pw = I.WORKLOADS["prefill_b2_t4096"]
    d = pw.dims
    q, k, v, _ = I.workload_inputs(pw.name, dev)
    out = torch.empty((d["B"], d["T"], d["H"] * d["D"]), dtype=q.dtype, device=dev)
    flops = prefill_flops(d["B"], d["T"], d["H"], d["D"])
    ms, wall = time_calls(torch, lambda i: gm.attend_prefill(q, k, v, out=out), K, W)
    avg = sum(ms) / len(ms)
    tflops = flops / (avg * 1e-3) / 1e12
    pre_files = ["causal_softmax_attention_gmla_amd/csrc/prefill_bf16.hip",
                 "causal_softmax_attention_gmla_amd/csrc/gmla_internal.h"]
    result = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": round(wall * 1e3 / K, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": pw.name, "B": d["B"], "T": d["T"], "H": d["H"], "D": d["D"],
                   "causal": True, "inputs": "N(0,1) rounded to bf16, seeded"},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic("prefill_bf16_kernel", pre_files),
                     "kernel": "prefill_bf16_kernel", "algorithmic_flop_per_launch": flops,
                     "avg_launch_ms": round(avg, 4), "min_launch_ms": round(min(ms), 4)},
    }

    # ---------------- decode: B=8 H=96 N=1001 D=128 bf16, rotated over 4 input sets
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

    dms, dwall = time_calls(torch, dec, max(K, 20), W, rotate=4)
    davg = sum(dms) / len(dms)
    gbps = nbytes / (davg * 1e-3) / 1e9
    dec_files = ["causal_softmax_attention_gmla_amd/csrc/decode.hip",
                 "causal_softmax_attention_gmla_amd/csrc/gmla_internal.h"]
    result["decode"] = {
        "workload": dw.name, "value": round(gbps, 1), "unit": "GB/s", "splits": splits,
        "calls": len(dms), "avg_call_ms": round(davg, 5), "min_call_ms": round(min(dms), 5),
        "rotation": "4 input sets (1.58 GB) cycled so the 256 MB last-level cache cannot hold them",
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(gbps / PEAK_HBM_GBPS, 4),
                     "traffic": measured_traffic("decode_split_kernel", dec_files),
                     "kernel": "decode_split_kernel (+ decode_merge_kernel when splits > 1)",
                     "algorithmic_bytes_per_call": nbytes},
    }

    if args.all:
        extra = {}
        # full layer B=1 T=2048 d_model=12288 d_c=512
        lw = I.WORKLOADS["layer_t2048"]
        ld = lw.dims
        x, wts = I.workload_inputs(lw.name, dev)
        lms, _ = time_calls(torch, lambda i: gm.gated_mla(x, wts["Wq"], wts["Wc"], wts["Wk"], wts["Wv"],
                                                          wts["Wg"], wts["Wo"], ld["H"], True),
                            max(5, K // 5), 2)
        T_, dm, dc = ld["T"], ld["d_model"], ld["d_c"]
        lflops = 2 * T_ * (3 * dm * dm + 3 * dm * dc) + prefill_flops(1, T_, ld["H"], dm // ld["H"])
        lavg = sum(lms) / len(lms)
        extra[lw.name] = {"value": round(lflops / (lavg * 1e-3) / 1e12, 1), "unit": "TFLOP/s",
                          "avg_call_ms": round(lavg, 4), "algorithmic_flop": lflops}
        del x, wts
        # long decode B=4 H=96 N=131072
        cw = I.WORKLOADS["decode_b4_n131072"]
        cd = cw.dims
        qc, kc, vc, _ = I.workload_inputs(cw.name, dev)
        cms, _ = time_calls(torch, lambda i: gm.attend_decode(qc, kc, vc), max(5, K // 5), 2)
        cavg = sum(cms) / len(cms)
        cb = decode_bytes(cd["B"], cd["H"], cd["N"], cd["D"])
        extra[cw.name] = {"value": round(cb / (cavg * 1e-3) / 1e9, 1), "unit": "GB/s",
                          "avg_call_ms": round(cavg, 4), "algorithmic_bytes": cb,
                          "splits": gm.decode_num_splits(cd["B"], cd["H"], cd["N"], cd["D"])}
        del qc, kc, vc
        result["extra"] = extra

    if not args.no_cpu:
        result["cpu_baseline"] = cpu_prefill_baseline(q, k, v)
        qd, kd, vd, _ = sets[0]
        result["decode"]["cpu_baseline"] = cpu_decode_baseline(qd, kd, vd)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
