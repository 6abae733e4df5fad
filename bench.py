#!/usr/bin/env python3
"""Benchmark of the fused RMSNorm -> QKV(+LoRA) -> RoPE operator on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama3|llama2|decode|train|tiny]

A step is one call of the whole operator on one batch of synthetic, seeded input that is
already resident in HBM: the forward for the layer and decode workloads, forward then
backward for the training workload.  W untimed warm-up steps, then K timed steps between
two device synchronisations; one JSON line is printed.  The K steps are launched as one
replay of a HIP graph that holds them (``--graph off``: eager calls), so the host's launch
cost neither bounds a decode step nor leaves gaps between the kernels of a layer step.

* ``value``: tokens per second of the whole job (one GPU).
* ``roofline``: the dominant kernel's algorithmic FLOPs (or bytes, for the bandwidth-bound
  decode workload) per launch over its average launch duration, against MI355X's published
  peak (bf16 dense MFMA 2500 TFLOP/s, HBM 8000 GB/s).  The duration comes from the
  library's measurement hook (HIP events recorded on the launch stream around that one
  kernel in every timed call); ``call_ms`` is the whole library call, timed the same way
  from here.  ``traffic`` comes from rocprofv3 FETCH_SIZE/WRITE_SIZE counters recorded
  under profiles/ for the same kernel source (null if the source changed).
* ``cpu_baseline``: the CPU oracle (float64 numpy, untuned) timed on this host on a bounded
  sample of the same workload's rows.

``--copy-probe`` instead runs a plain device copy of known size (the calibration kernel for
the FETCH_SIZE / WRITE_SIZE counters).  ``--record-traffic`` turns the counter files of
such runs into profiles/traffic.json (no GPU needed):

    python bench.py --record-traffic WORKLOAD --family FAMILY --kernel NAME \
        --fetch DIR --write DIR --calib-fetch DIR --calib-write DIR --calib-bytes N
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused RMSNorm+LoRA-QKV+RoPE tokens/s, TFLOP/s (% MFMA peak) on 1×MI355X"
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def algorithmic_work(w, T=None):
    """Matmul FLOPs (forward, backward) and forward bytes of one call; RMSNorm, bias and RoPE
    are O(T (d + N)) and not counted, nor is any recomputation."""
    T = w.n_tokens if T is None else T
    d, N, r = w.d_model, w.n_out, w.lora_rank
    cols = w.target_columns()
    f_fwd = 2.0 * T * d * N
    f_bwd = 2.0 * T * N * d
    lora_bytes = 0
    for t, (lo, hi) in cols.items():
        if w.lora_targets & t:
            nt = hi - lo
            f_fwd += 2.0 * T * d * r + 2.0 * T * r * nt
            # V = G B, dh += s V A, U recompute, dB = G^T U, dA = V^T h
            f_bwd += 2.0 * T * nt * r + 2.0 * T * r * d + 2.0 * T * d * r + 2.0 * T * nt * r + 2.0 * T * r * d
            lora_bytes += (r * d + nt * r)
    eb = 4 if w.dtype == "f32" else 2
    bytes_fwd = eb * (T * d + d + N * d + (N if w.has_bias else 0) + lora_bytes + T * N) + 4 * T
    return f_fwd, f_bwd, bytes_fwd


def dominant_kernel_work(w, family: str, backward: bool):
    """Algorithmic work of one launch of a call's dominant kernel: (amount, unit kind).

    Forward, tiled or generic: every matmul FLOP of the forward.  Forward, decode: the bytes
    the streaming kernel must move (x, gamma, W, bias, the targets' A, positions, and the
    outputs of columns without an adapter; the LoRA-up pass writes the rest).  Backward,
    tiled: dh = G W + sum_t V'_t A_t, 2 T d (N + sum of ranks) FLOPs.  Backward, generic:
    every matmul FLOP of the backward."""
    f_fwd, f_bwd, _ = algorithmic_work(w)
    T, d, N, r = w.n_tokens, w.d_model, w.n_out, w.lora_rank
    cols = w.target_columns()
    ranks = sum(r for t in cols if w.lora_targets & t)
    if backward:
        return (2.0 * T * d * (N + ranks), "flop") if family == "tiled" else (f_bwd, "flop")
    if family == "decode":
        eb = 2
        unadapted = sum(hi - lo for t, (lo, hi) in cols.items() if not (w.lora_targets & t))
        nbytes = eb * (T * d + d + N * d + (N if w.has_bias else 0) + ranks * d + T * unadapted) + 4 * T
        return nbytes, "bytes"
    return f_fwd, "flop"


def kernel_source_digest(variant_name: str) -> str:
    """sha256 of the sources that define a kernel family (for matching stored counters)."""
    files = {"tiled": ["fwd_tiled.hip", "tile_common.h"], "decode": ["fwd_decode.hip", "tile_common.h"],
             "generic": ["fwd_generic.hip"], "bwd_tiled": ["bwd_tiled.hip", "tile_common.h"],
             "bwd_generic": ["bwd_generic.hip"]}[variant_name]
    h = hashlib.sha256()
    for f in files + ["lrq_internal.h"]:
        p = os.path.join(ROOT, "layer_rmsnorm_qkv_amd", "csrc", f)
        if os.path.exists(p):
            h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def stored_traffic(workload: str, kernel: str):
    try:
        data = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    rec = data.get(f"{workload}:{kernel}")
    if not rec or rec.get("source_sha") != kernel_source_digest(kernel):
        return None
    return rec.get("bytes_per_launch")


def _counter_means(directory: str, kernel_prefix: str):
    """Mean counter value (KiB per dispatch) over the dispatches of one kernel in a
    rocprofv3 --pmc csv directory, and the number of dispatches."""
    import csv
    import glob
    vals = []
    for f in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            name = r["Kernel_Name"].replace("lrq::(anonymous namespace)::", "").replace("void ", "")
            if name.startswith(kernel_prefix):
                vals.append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no dispatch of {kernel_prefix} in {directory}")
    return sum(vals) / len(vals), len(vals)


def record_traffic(args):
    """HBM bytes per launch of one kernel from FETCH_SIZE / WRITE_SIZE passes, each scaled by
    what the same counter reads for a device copy of known size; stored with the digest of
    the kernel's source so that bench.py drops it once the kernel changes."""
    fetch, nf = _counter_means(args.fetch, args.kernel)
    write, nw = _counter_means(args.write, args.kernel)
    cf, _ = _counter_means(args.calib_fetch, "__amd_rocclr_copyBuffer")
    cw, _ = _counter_means(args.calib_write, "__amd_rocclr_copyBuffer")
    # the copy probe's largest dispatch is the copy itself; smaller ones are fills
    import csv
    import glob

    def largest(directory):
        best = 0.0
        for f in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if "copyBuffer" in r["Kernel_Name"]:
                    best = max(best, float(r["Counter_Value"]))
        return best
    cf, cw = largest(args.calib_fetch), largest(args.calib_write)
    ff = args.calib_bytes / (cf * 1024.0)
    fw = args.calib_bytes / (cw * 1024.0)
    rec = {"kernel": args.kernel, "source_sha": kernel_source_digest(args.family),
           "fetch_size_kib": fetch, "write_size_kib": write, "fetch_factor": ff, "write_factor": fw,
           "fetch_bytes": fetch * 1024.0 * ff, "write_bytes": write * 1024.0 * fw,
           "bytes_per_launch": fetch * 1024.0 * ff + write * 1024.0 * fw, "dispatches": [nf, nw],
           "calibration": f"{args.calib_bytes} B device copy (bench.py --copy-probe {args.calib_bytes}): "
                          f"FETCH_SIZE {cf:.0f} KiB, WRITE_SIZE {cw:.0f} KiB per dispatch"}
    try:
        data = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        data = {}
    data[f"{args.record_traffic}:{args.family}"] = rec
    json.dump(data, open(TRAFFIC_FILE, "w"), indent=1, sort_keys=True)
    print(json.dumps(rec))


def cpu_baseline(w, inp, budget_s: float, rows_cap: int, gpu_rows_fn=None):
    """Time the float64 oracle on a bounded, seeded sample of rows of the same workload."""
    import numpy as np
    import oracle.lrq_oracle as o
    try:
        import threadpoolctl
        threads = max((i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()), default=1)
    except Exception:  # noqa: BLE001
        threads = 1
    spec = o.Spec(d_model=w.d_model, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads, head_dim=w.head_dim,
                  lora_rank=w.lora_rank if w.lora_targets else 0, lora_alpha=w.lora_alpha,
                  lora_targets=w.lora_targets, eps=w.eps, rope_theta=w.rope_theta)
    T = w.n_tokens
    rng = np.random.default_rng(12345)
    order = rng.permutation(T)

    def run(rows):
        t0 = time.perf_counter()
        out = o.forward_rows(spec, rows, inp["x"], inp["gamma"], inp["w"], inp["bias"], inp["a"], inp["b"],
                             inp["positions"])
        if w.backward:
            o.backward(spec, inp["x"][rows], inp["gamma"], inp["w"], inp["bias"], inp["a"], inp["b"],
                       inp["positions"][rows], inp["dy"][rows])
        return time.perf_counter() - t0, out

    probe = min(T, 32)
    dt, _ = run(np.sort(order[:probe]))
    n = int(min(T, rows_cap, max(probe, probe * budget_s / max(dt, 1e-6))))
    rows = np.sort(order[:n])
    dt, out = run(rows)
    # when the whole sample takes much less than the budget, repeat it (a steadier rate)
    reps, total = 1, dt
    while total < 0.8 * budget_s and reps < 256:
        total += run(rows)[0]
        reps += 1
    res = {"value": n * reps / total, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": f"{n} of {T} rows (seeded) x {reps} passes, "
                     f"{'forward+backward' if w.backward else 'forward'}, float64 numpy, {total:.2f} s"}
    if gpu_rows_fn is not None:  # the same rows from the GPU forward, for a parity figure
        res["gpu_parity_rel_fro"] = o.rel_frobenius(gpu_rows_fn(rows), out)
    return res


def copy_probe(nbytes: int, reps: int):
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "reps": reps}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30, help="untimed steps first (the clocks settle within about 20 steps of sustained MFMA load)")
    ap.add_argument("--workload", default="llama3", choices=["tiny", "llama3", "llama2", "decode", "train"])
    ap.add_argument("--variant", default="auto", choices=["auto", "generic", "tiled", "decode"])
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--w-copies", type=int, default=0,
                    help="rotate among this many W_qkv copies (defeats the 256 MB MALL; default 4 for decode)")
    ap.add_argument("--graph", choices=["on", "off"], default="on",
                    help="launch the K timed steps as one replay of a HIP graph that holds them (on), or as "
                         "eager library calls (off)")
    ap.add_argument("--kv-cache", action="store_true",
                    help="forward through lrq_forward_kv: every token also writes its k and v rows to a "
                         "cache of T rows (slot t for token t)")
    ap.add_argument("--copy-probe", type=int, default=0, help="run a device copy of this many bytes and exit")
    ap.add_argument("--record-traffic", default="", help="workload name: store counter traffic and exit")
    ap.add_argument("--family", default="", help="kernel family key (tiled, decode, bwd_tiled, ...)")
    ap.add_argument("--kernel", default="", help="kernel name prefix in the counter files")
    ap.add_argument("--fetch", default="")
    ap.add_argument("--write", default="")
    ap.add_argument("--calib-fetch", default="")
    ap.add_argument("--calib-write", default="")
    ap.add_argument("--calib-bytes", type=int, default=1 << 30)
    args = ap.parse_args()
    if args.record_traffic:
        record_traffic(args)
        return

    if args.gpus != 1:
        print(f"bench.py: this operator is measured on one GPU only; --gpus {args.gpus} is not supported "
              f"(the path shards by tokens with no communication in the forward).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_probe:
        copy_probe(args.copy_probe, 5)
        return

    from layer_rmsnorm_qkv_amd import binding as B
    from layer_rmsnorm_qkv_amd import workloads as wl
    from layer_rmsnorm_qkv_amd.device import DeviceProblem, desc_for

    B.load()
    w = wl.get(args.workload)
    variant = {"auto": B.LRQ_VARIANT_AUTO, "generic": B.LRQ_VARIANT_GENERIC, "tiled": B.LRQ_VARIANT_TILED,
               "decode": B.LRQ_VARIANT_DECODE}[args.variant]
    inp = wl.make_inputs(w, with_dy=w.backward)
    prob = DeviceProblem(w, inp, variant=variant, backward=w.backward)
    vname = B.VARIANT_NAMES[prob.variant]
    stream = torch.cuda.current_stream()

    n_copies = args.w_copies or (4 if w.name == "decode" else 1)
    w_list = [prob.w_qkv] + [prob.w_qkv.clone() for _ in range(n_copies - 1)]
    kvw = w.n_kv_heads * w.head_dim
    if args.kv_cache:
        k_cache = torch.zeros((w.n_tokens, kvw), dtype=prob.out.dtype, device=prob.out.device)
        v_cache = torch.zeros_like(k_cache)
        slots = torch.arange(w.n_tokens, dtype=torch.int32, device=prob.out.device)

    def forward(s=None):
        s = stream if s is None else s
        if args.kv_cache:
            B.lrq_forward_kv(prob.desc, prob.x, prob.gamma, prob.w_qkv, prob.bias, prob.a, prob.b, prob.positions,
                             prob.out, k_cache, v_cache, slots, w.n_tokens, prob.workspace, stream=s)
        else:
            prob.forward(stream=s)
        return prob.out

    def step(i, s=None):
        prob.w_qkv = w_list[i % n_copies]
        forward(s)
        if w.backward:
            prob.backward(stream=stream if s is None else s)

    for i in range(args.warmup):
        step(i)

    use_graph = args.graph == "on"
    if use_graph:
        # One graph holds the K steps, each with the library's timing events around its dominant
        # kernel (the events are created by an eager pass first: nothing is created during
        # capture).  One untimed replay, then the timed one.
        B.lrq_kernel_timing(True)
        for i in range(args.steps):
            step(i)
        torch.cuda.synchronize()
        B.lrq_kernel_timing(True)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            cap = torch.cuda.current_stream()
            for i in range(args.steps):
                step(i, cap)
        graph.replay()
        torch.cuda.synchronize()

    # timed region: exactly K steps, nothing else on the stream but the library's own timing
    # events around each call's dominant kernel (the roofline's per-launch duration)
    torch.cuda.synchronize()
    if not use_graph:
        B.lrq_kernel_timing(True)
    t0 = time.perf_counter()
    if use_graph:
        graph.replay()
    else:
        for i in range(args.steps):
            step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kfwd_ms, n_fwd = B.lrq_kernel_time_ms(False)
    kbwd_ms, n_bwd = B.lrq_kernel_time_ms(True)
    B.lrq_kernel_timing(False)
    assert n_fwd == args.steps and n_bwd == (args.steps if w.backward else 0), (n_fwd, n_bwd)

    # whole library calls, timed with events on the stream in a separate (untimed) pass
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        e0, e1, e2 = ev[i]
        prob.w_qkv = w_list[i % n_copies]
        e0.record(stream)
        forward()
        e1.record(stream)
        if w.backward:
            prob.backward(stream=stream)
        e2.record(stream)
    torch.cuda.synchronize()
    fwd_ms = float(np.mean([a.elapsed_time(b) for a, b, _ in ev]))
    bwd_ms = float(np.mean([b.elapsed_time(c) for _, b, c in ev])) if w.backward else 0.0

    ms_per_step = wall * 1e3 / args.steps
    tokens = w.n_tokens
    f_fwd, f_bwd, bytes_fwd = algorithmic_work(w)
    if args.kv_cache:
        bytes_fwd += 2 * w.n_tokens * kvw * (4 if w.dtype == "f32" else 2)  # the cache rows written
    result = {
        "metric": METRIC, "value": tokens / (ms_per_step * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32" if w.dtype == "f32" else "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "description": w.description, "tokens": tokens, "d_model": w.d_model,
                   "n_out": w.n_out, "lora_rank": w.lora_rank, "lora_targets": w.lora_targets,
                   "kernel_family": vname, "parallelism": "none (1 GPU)",
                   "pass": "forward+backward" if w.backward else "forward",
                   "kv_cache": bool(args.kv_cache),
                   "launch": "one HIP graph replay of the K steps" if use_graph else "eager calls"},
    }
    # call-level rates (whole library calls)
    tflops_fwd = f_fwd / (fwd_ms * 1e-3) / 1e12
    result["tflops_forward"] = tflops_fwd
    result["call_ms"] = {"forward": fwd_ms}
    if w.backward:
        result["tflops_backward"] = f_bwd / (bwd_ms * 1e-3) / 1e12
        result["tflops_step"] = (f_fwd + f_bwd) / (ms_per_step * 1e-3) / 1e12
        result["call_ms"]["backward"] = bwd_ms
    if w.name == "decode":
        result["gbs_forward_call"] = bytes_fwd / (fwd_ms * 1e-3) / 1e9
    # dominant kernel: the longer of the forward and backward calls' dominant kernels
    backward_dominant = w.backward and kbwd_ms > kfwd_ms
    family = B.VARIANT_NAMES[prob.bwd_variant] if backward_dominant else vname
    dom_ms = kbwd_ms if backward_dominant else kfwd_ms
    work, kind = dominant_kernel_work(w, family, backward_dominant)
    kname = {("tiled", False): "fwd_tiled_kernel", ("decode", False): "decode_main_kernel",
             ("generic", False): "fwd_generic_kernel", ("tiled", True): "bwd_main_kernel",
             ("generic", True): "bwd_generic_kernel"}[(family, backward_dominant)]
    traffic = stored_traffic(w.name, ("bwd_" if backward_dominant else "") + family)
    if kind == "bytes":
        ach = work / (dom_ms * 1e-3) / 1e9
        result["roofline"] = {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                              "frac": ach / PEAK_HBM_GBS, "traffic": traffic, "kernel": kname,
                              "launch_ms": dom_ms, "algorithmic_bytes": work}
    else:
        peak = PEAK_FP32_TFLOPS if w.dtype == "f32" else PEAK_BF16_TFLOPS
        ach = work / (dom_ms * 1e-3) / 1e12
        result["roofline"] = {"bound": "mfma", "achieved": ach, "peak": peak, "unit": "TFLOP/s",
                              "frac": ach / peak, "traffic": traffic, "kernel": kname,
                              "launch_ms": dom_ms, "algorithmic_flop": work}
    if not args.no_cpu_baseline:
        prob.w_qkv = w_list[0]
        got = forward()
        torch.cuda.synchronize()
        got = got.float().cpu().numpy().astype(np.float64)
        result["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_budget, rows_cap=w.n_tokens,
                                              gpu_rows_fn=lambda rows: got[rows])
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
