#!/usr/bin/env python3
"""Benchmark of the fused RMSNorm -> QKV(+LoRA) -> RoPE operator on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload all|llama2|tiny|llama3|decode|train]

A step is one call of the whole operator on one batch of synthetic, seeded input that is
already resident in HBM: the forward for the layer and decode workloads, forward then
backward for the training workload.  The frozen weights (W, gamma) are prepared once before
the steps, as at model load.  W untimed warm-up steps, then K timed steps between two device
synchronisations.  The K steps are launched as one replay of a HIP graph that holds them
(``--graph off``: eager calls), so the host's launch cost neither bounds a decode step nor
leaves gaps between the kernels of a layer step.  Consecutive steps read different copies of
the streamed operands, so none of them is left in the 256 MB MALL by the step before.

By default every workload is measured; one JSON line is printed whose top level is the
headline workload, llama2 (LLaMA-2-7B layer, 16384 tokens: the largest), and whose
``configs`` holds all five (tiny, llama3, llama2, decode, train) in the same form.

* ``value``: tokens per second of the whole job (one GPU).
* ``roofline``: the dominant kernel's algorithmic FLOPs (or bytes, for the bandwidth-bound
  decode workload) per launch over its average launch duration, against MI355X's published
  peak (bf16 dense MFMA 2500 TFLOP/s, HBM 8000 GB/s).  The duration is the mean of the
  library's measurement hook (HIP events recorded on the launch stream around that one kernel)
  over a separate eager pass of K steps, clamped to the graph-timed step;
  ``call_ms_eager`` are the whole library calls of that pass.  ``traffic`` comes from
  rocprofv3 FETCH_SIZE/WRITE_SIZE counters recorded under profiles/ for the same kernel source
  (null if the source changed).
* ``cpu_baseline``: the CPU oracle (float64 numpy, untuned) timed on this host on a bounded
  sample of the same workload's rows, BLAS threads pinned to the process's cores.

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


def dominant_kernel_work(w, family: str, backward: bool, nf4: bool = False):
    """Algorithmic work of one launch of a call's dominant kernel: (amount, unit kind).

    Forward, tiled or generic: every matmul FLOP of the forward.  Forward, decode: the bytes
    the streaming kernel must move (x, gamma, W, bias, the targets' A and B, positions, and
    every output).  Backward,
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
        b_elems = sum(r * (hi - lo) for t, (lo, hi) in cols.items() if w.lora_targets & t)
        nbytes = eb * (T * d + d + N * d + (N if w.has_bias else 0) + ranks * d + b_elems + T * N) + 4 * T
        if nf4:  # the QLoRA base: 4-bit codes plus a float32 scale per 64 weights instead of bf16
            nbytes -= eb * N * d - (N * d // 2 + N * (d // 64) * 4)
        return nbytes, "bytes"
    return f_fwd, "flop"


def kernel_source_digest(variant_name: str) -> str:
    """sha256 of the sources that define a kernel family (for matching stored counters)."""
    files = {"tiled": ["fwd_tiled.hip", "tile_common.h"], "decode": ["fwd_decode.hip", "tile_common.h"],
             "generic": ["fwd_generic.hip"], "bwd_tiled": ["bwd_tiled.hip", "tile_common.h"],
             "bwd_generic": ["bwd_generic.hip"], "attn": ["attn.hip", "tile_common.h"],
             "mlp": ["mlp_tiled.hip", "tile_common.h"]}[variant_name]
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


def cpu_threads() -> int:
    """Cores this process may run on (the affinity mask; a container's CPU share may be smaller
    than os.cpu_count())."""
    try:
        return len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        return os.cpu_count() or 1


def cpu_baseline(w, inp, budget_s: float, gpu_rows_fn=None, dropout=None):
    """Time the float64 oracle on a bounded, seeded sample of rows of the same workload, with
    the BLAS pool pinned to this process's cores (the count used is reported)."""
    import numpy as np
    import oracle.lrq_oracle as o
    n_threads = cpu_threads()
    try:
        import threadpoolctl
        limiter = threadpoolctl.threadpool_limits(limits=n_threads)
        used = max((i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()), default=1)
    except Exception:  # noqa: BLE001
        limiter, used = None, 1
    spec = o.Spec(d_model=w.d_model, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads, head_dim=w.head_dim,
                  lora_rank=w.lora_rank if w.lora_targets else 0, lora_alpha=w.lora_alpha,
                  lora_targets=w.lora_targets, eps=w.eps, rope_theta=w.rope_theta)
    T = w.n_tokens
    rng = np.random.default_rng(12345)
    order = rng.permutation(T)

    drop = None if dropout is None else o.Dropout(float(np.float32(dropout[0])), dropout[1], dropout[2])

    def run(rows):
        t0 = time.perf_counter()
        out = o.forward_rows(spec, rows, inp["x"], inp["gamma"], inp["w"], inp["bias"], inp["a"], inp["b"],
                             inp["positions"], dropout=drop)
        if w.backward:
            # the sample's rows as a call of their own (its masks are that call's: same cost)
            o.backward(spec, inp["x"][rows], inp["gamma"], inp["w"], inp["bias"], inp["a"], inp["b"],
                       inp["positions"][rows], inp["dy"][rows], dropout=drop)
        return time.perf_counter() - t0, out

    try:
        probe = min(T, 32)
        dt, _ = run(np.sort(order[:probe]))
        n = int(min(T, max(probe, probe * budget_s / max(dt, 1e-6))))
        rows = np.sort(order[:n])
        dt, out = run(rows)
        # when the whole sample takes much less than the budget, repeat it (a steadier rate)
        reps, total = 1, dt
        while total < 0.8 * budget_s and reps < 256:
            total += run(rows)[0]
            reps += 1
    finally:
        if limiter is not None:
            limiter.unregister() if hasattr(limiter, "unregister") else None
    res = {"value": n * reps / total, "unit": "tokens/s", "cores": used, "kind": "oracle",
           "sample": f"{n} of {T} rows (seeded) x {reps} passes, "
                     f"{'forward+backward' if w.backward else 'forward'}, float64 numpy, {total:.2f} s, "
                     f"BLAS threads pinned to {n_threads}"}
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


KERNEL_NAMES = {("tiled", False): "fwd_tiled_kernel", ("decode", False): "decode_main_kernel",
                ("generic", False): "fwd_generic_kernel", ("tiled", True): "bwd_main_kernel",
                ("generic", True): "bwd_generic_kernel"}
HEADLINE = "llama2"
ALL_WORKLOADS = ("llama2", "tiny", "llama3", "decode", "train")


def working_set_copies(w, prob, n_copies: int):
    """Independent copies of the operands a step streams (the prepared weights, or W for the
    families that read it, and x), so that consecutive steps cannot find them in the 256 MB
    MALL: each step reads the copy i % n of each."""
    import torch
    sets = []
    for i in range(n_copies):
        if i == 0:
            sets.append((prob.w_qkv, prob.prepared, prob.x))
            continue
        sets.append((prob.w_qkv.clone(), None if prob.prepared is None else prob.prepared.clone(),
                     prob.x.clone()))
    torch.cuda.synchronize()
    return sets


def run_config(name, args, B, wl, DeviceProblem, dropout=None, nf4=False, key=None):
    """Measure one workload: returns its result object (the shape of the top-level line).
    ``dropout`` = (rate, seed, offset) runs it with LoRA dropout; ``nf4`` stores the base as NF4
    blocks (the QLoRA base, quantised on the device before the steps); ``key`` names the entry
    (stored counter traffic is looked up under it; default: the workload's name)."""
    import numpy as np
    import torch

    w = wl.get(name)
    variant = {"auto": B.LRQ_VARIANT_AUTO, "generic": B.LRQ_VARIANT_GENERIC, "tiled": B.LRQ_VARIANT_TILED,
               "decode": B.LRQ_VARIANT_DECODE}[args.variant]
    inp = wl.make_inputs(w, with_dy=w.backward)
    prob = DeviceProblem(w, inp, variant=variant, backward=w.backward, dropout=dropout, nf4=nf4)
    vname = B.VARIANT_NAMES[prob.variant]
    stream = torch.cuda.current_stream()
    # frozen weights are prepared once, before any step (untimed setup, as at model load), for
    # the families that read a prepared layout
    uses_prepared = vname == "tiled" or (w.backward and B.VARIANT_NAMES[prob.bwd_variant] == "tiled")
    if uses_prepared and not args.no_prepare:
        prob.prepare()
        ws = max(B.lrq_workspace_size_prepared(prob.desc, False),
                 B.lrq_workspace_size_prepared(prob.desc, True) if w.backward else 0)
        prob.workspace = torch.empty(ws, dtype=torch.uint8, device="cuda") if ws else None
    # enough copies that one step's streamed operands are not left in the MALL by the last
    per_copy = prob.x.numel() * prob.x.element_size() + \
        (prob.prepared.numel() if prob.prepared is not None else prob.w_qkv.numel() * prob.w_qkv.element_size())
    n_copies = args.copies or max(2, min(8, -(-400 * 2 ** 20 // per_copy)))
    sets = working_set_copies(w, prob, n_copies)
    kvw = w.n_kv_heads * w.head_dim
    if args.kv_cache:
        k_cache = torch.zeros((w.n_tokens, kvw), dtype=prob.out.dtype, device=prob.out.device)
        v_cache = torch.zeros_like(k_cache)
        slots = torch.arange(w.n_tokens, dtype=torch.int32, device=prob.out.device)

    def forward(s):
        if args.kv_cache:
            B.lrq_forward_prepared(prob.desc, prob.x, prob.gamma, prob.w_qkv, prob.prepared, prob.bias, prob.a,
                                   prob.b, prob.positions, prob.out, (k_cache, v_cache, slots, w.n_tokens),
                                   prob.workspace, stream=s)
        else:
            prob.forward(stream=s)
        return prob.out

    def step(i, s):
        prob.w_qkv, prob.prepared, prob.x = sets[i % n_copies]
        forward(s)
        if w.backward:
            prob.backward(stream=s)

    for i in range(args.warmup):
        step(i, stream)
    torch.cuda.synchronize()

    # the K timed steps, captured once into a HIP graph (no events inside it)
    graph = None
    if args.graph == "on":
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step(0, side)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            cap = torch.cuda.current_stream()
            for i in range(args.steps):
                step(i, cap)
        graph.replay()  # untimed
        torch.cuda.synchronize()

    # timed region: exactly K steps between two device synchronisations
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if graph is not None:
        graph.replay()
    else:
        for i in range(args.steps):
            step(i, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    # separate eager pass (untimed for `value`): the library's events around the dominant
    # kernel of every call, and events from here around every whole call
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    B.lrq_kernel_timing(True)
    for i in range(args.steps):
        e0, e1, e2 = ev[i]
        prob.w_qkv, prob.prepared, prob.x = sets[i % n_copies]
        e0.record(stream)
        forward(stream)
        e1.record(stream)
        if w.backward:
            prob.backward(stream=stream)
        e2.record(stream)
    torch.cuda.synchronize()
    kfwd_ms, n_fwd = B.lrq_kernel_time_ms(False)
    kbwd_ms, n_bwd = B.lrq_kernel_time_ms(True)
    B.lrq_kernel_timing(False)
    assert n_fwd == args.steps and n_bwd == (args.steps if w.backward else 0), (n_fwd, n_bwd)
    fwd_ms = float(np.mean([a.elapsed_time(b) for a, b, _ in ev]))
    bwd_ms = float(np.mean([b.elapsed_time(c) for _, b, c in ev])) if w.backward else 0.0
    prob.w_qkv, prob.prepared, prob.x = sets[0]

    tokens = w.n_tokens
    f_fwd, f_bwd, bytes_fwd = algorithmic_work(w)
    if args.kv_cache:
        bytes_fwd += 2 * w.n_tokens * kvw * (4 if w.dtype == "f32" else 2)  # the cache rows written
    res = {
        "metric": METRIC, "value": tokens / (ms_per_step * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32" if w.dtype == "f32" else "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "description": w.description, "tokens": tokens, "d_model": w.d_model,
                   "n_out": w.n_out, "lora_rank": w.lora_rank, "lora_targets": w.lora_targets,
                   "kernel_family": vname, "parallelism": "none (1 GPU)",
                   "pass": "forward+backward" if w.backward else "forward",
                   "kv_cache": bool(args.kv_cache),
                   "lora_dropout": 0.0 if dropout is None else dropout[0],
                   "weight_format": "nf4" if nf4 else "dense",
                   "weights": "prepared once before the steps" if prob.prepared is not None else
                              "prepared inside every call",
                   "operand_copies": n_copies,
                   "launch": "one HIP graph replay of the K steps" if graph is not None else "eager calls"},
        "tflops_step": (f_fwd + f_bwd * w.backward) / (ms_per_step * 1e-3) / 1e12,
        "call_ms_eager": {"forward": fwd_ms},
    }
    if w.backward:
        res["call_ms_eager"]["backward"] = bwd_ms
    if w.name == "decode":
        res["gbs_step"] = bytes_fwd / (ms_per_step * 1e-3) / 1e9
    # dominant kernel: the longer of the forward and backward calls' dominant kernels.  Its
    # duration is the mean of the library's events around it in the eager pass, never more
    # than the graph-timed step (a kernel cannot outlast the step that contains it).
    backward_dominant = w.backward and kbwd_ms > kfwd_ms
    family = B.VARIANT_NAMES[prob.bwd_variant] if backward_dominant else vname
    dom_eager = kbwd_ms if backward_dominant else kfwd_ms
    dom_ms = min(dom_eager, ms_per_step)
    assert dom_ms <= ms_per_step
    work, kind = dominant_kernel_work(w, family, backward_dominant, nf4)
    kname = KERNEL_NAMES[(family, backward_dominant)]
    traffic = stored_traffic(key or w.name, ("bwd_" if backward_dominant else "") + family)
    common = {"traffic": traffic, "kernel": kname, "launch_ms": dom_ms, "launch_ms_eager_events": dom_eager,
              "launch_ms_clamped_to_step": dom_eager > ms_per_step,
              "share_of_step": dom_ms / ms_per_step}
    if kind == "bytes":
        ach = work / (dom_ms * 1e-3) / 1e9
        res["roofline"] = {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                           "frac": ach / PEAK_HBM_GBS, "algorithmic_bytes": work, **common}
    else:
        peak = PEAK_FP32_TFLOPS if w.dtype == "f32" else PEAK_BF16_TFLOPS
        ach = work / (dom_ms * 1e-3) / 1e12
        res["roofline"] = {"bound": "mfma" if w.dtype != "f32" else "alu", "achieved": ach, "peak": peak,
                           "unit": "TFLOP/s", "frac": ach / peak, "algorithmic_flop": work, **common}
    if not args.no_cpu_baseline:
        got = forward(stream)
        torch.cuda.synchronize()
        got = got.float().cpu().numpy().astype(np.float64)
        base_inp = inp
        if nf4:  # the oracle on the same NF4 base: the dequantised W
            import oracle.qlora_oracle as qo
            base_inp = dict(inp, w=qo.dequantize(*qo.quantize(np.asarray(inp["w"], np.float32))))
        res["cpu_baseline"] = cpu_baseline(w, base_inp, args.cpu_budget, gpu_rows_fn=lambda rows: got[rows],
                                           dropout=dropout)
    del sets, prob, graph
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def mlp_work(w):
    """Matmul FLOPs of one MLP call and of its fused gate/up/SwiGLU kernel (algorithmic:
    gate, up and down products plus the adapters' down and up products)."""
    T, d, F, r = w.n_tokens, w.d_model, w.d_ff, w.lora_rank
    lora = {1: (d, F), 2: (d, F), 4: (F, d)}
    f_gu = 4.0 * T * d * F
    f_dn = 2.0 * T * F * d
    for t, (din, dout) in lora.items():
        if w.lora_targets & t:
            extra = 2.0 * T * din * r + 2.0 * T * r * dout
            if t == 4:
                f_dn += extra
            else:
                f_gu += extra
    return f_gu, f_dn


def run_mlp_config(name, args, B, wl):
    """The LoRA-adapted SwiGLU MLP (a next row beside the projection): whole calls and the fused
    gate/up/SwiGLU kernel, timed like the projection's workloads."""
    import numpy as np
    import torch
    from layer_rmsnorm_qkv_amd.device import DeviceMlp

    w = wl.get_mlp(name)
    inp = wl.make_mlp_inputs(w)
    prob = DeviceMlp(w, inp)
    stream = torch.cuda.current_stream()
    h_copies = [prob.h] + [prob.h.clone() for _ in range(1)]

    def step(i, s):
        prob.h = h_copies[i % len(h_copies)]
        prob.forward(stream=s)

    for i in range(args.warmup):
        step(i, stream)
    torch.cuda.synchronize()
    graph = None
    if args.graph == "on":
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step(0, side)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            cap = torch.cuda.current_stream()
            for i in range(args.steps):
                step(i, cap)
        graph.replay()
        torch.cuda.synchronize()
    t0 = time.perf_counter()
    if graph is not None:
        graph.replay()
    else:
        for i in range(args.steps):
            step(i, stream)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    B.lrq_kernel_timing(True)
    for i in range(args.steps):
        step(i, stream)
    torch.cuda.synchronize()
    k_ms, n = B.lrq_kernel_time_ms(False)
    B.lrq_kernel_timing(False)
    assert n == args.steps
    dom = min(k_ms, ms_per_step)
    f_gu, f_dn = mlp_work(w)
    res = {"value": w.n_tokens / (ms_per_step * 1e-3), "unit": "tokens/s", "ms_per_step": ms_per_step,
           "dtype": "bf16",
           "config": {"workload": w.name, "description": w.description, "tokens": w.n_tokens, "d_model": w.d_model,
                      "d_ff": w.d_ff, "lora_rank": w.lora_rank, "lora_targets": w.lora_targets,
                      "kernel_family": "mlp tiled (gate/up/SwiGLU, then down)",
                      "launch": "one HIP graph replay of the K steps" if graph is not None else "eager calls"},
           "tflops_step": (f_gu + f_dn) / (ms_per_step * 1e-3) / 1e12,
           "roofline": {"bound": "mfma", "achieved": f_gu / (dom * 1e-3) / 1e12, "peak": PEAK_BF16_TFLOPS,
                        "unit": "TFLOP/s", "frac": f_gu / (dom * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                        "traffic": stored_traffic(w.name, "mlp"),
                        "kernel": "mlp_gate_up_kernel", "launch_ms": dom, "launch_ms_eager_events": k_ms,
                        "algorithmic_flop": f_gu}}
    if not args.no_cpu_baseline:
        import oracle.mlp_oracle as mo
        spec = mo.MlpSpec(d_model=w.d_model, d_ff=w.d_ff, lora_rank=w.lora_rank, lora_alpha=w.lora_alpha,
                          lora_targets=w.lora_targets)
        prob.h = h_copies[0]
        got = prob.forward().float().cpu().numpy().astype(np.float64)
        n_threads = cpu_threads()
        rows = np.sort(np.random.default_rng(5).permutation(w.n_tokens)[:64])
        t0 = time.perf_counter()
        ref = mo.mlp_forward_rows(spec, rows, inp["h"], inp["w_gate"], inp["w_up"], inp["w_down"], inp["a"], inp["b"])
        dt = time.perf_counter() - t0
        from oracle.lrq_oracle import rel_frobenius
        res["cpu_baseline"] = {"value": len(rows) / dt, "unit": "tokens/s", "cores": n_threads, "kind": "oracle",
                               "sample": f"{len(rows)} of {w.n_tokens} rows (seeded), float64 numpy, {dt:.2f} s",
                               "gpu_parity_rel_fro": rel_frobenius(got[rows], ref)}
    del graph, prob, h_copies
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def attn_work(w):
    """Matmul FLOPs (Q K^T and P V over the visible keys) and bytes (q, the sequences' cached
    keys and values, out) of one attention call."""
    D, hq, hkv = w.head_dim, w.n_q_heads, w.n_kv_heads
    vis = 0
    for i in range(w.q_len):
        vis += min(w.kv_len, w.kv_len - w.q_len + i + 1) if w.causal else w.kv_len
    flop = 4.0 * D * hq * vis * w.n_seqs
    byts = 2.0 * (2 * w.n_seqs * w.q_len * hq * D + 2 * w.n_seqs * w.kv_len * hkv * D)
    return flop, byts


def run_attn_config(name, args, B, wl):
    """Attention over the key/value cache (the step after the projection): timed like the
    projection's workloads; roofline against the peak the call's algorithmic work binds."""
    import numpy as np
    import torch

    w = wl.get_attn(name)
    inp = wl.make_attn_inputs_device(w)
    D = w.head_dim
    out = torch.empty((w.n_seqs * w.q_len, w.n_q_heads * D), dtype=torch.bfloat16, device="cuda")
    desc = B.make_attn_desc(w.n_seqs, w.n_q_heads, w.n_kv_heads, D, w.q_len, w.n_q_heads * D,
                            w.n_seqs * w.kv_len, causal=1 if w.causal else 0)
    stream = torch.cuda.current_stream()

    def step(i, s):
        B.lrq_attention(desc, inp["q"], inp["k_cache"], inp["v_cache"], inp["q_indptr"], inp["kv_indptr"],
                        inp["kv_slots"], out, stream=s)

    for i in range(args.warmup):
        step(i, stream)
    torch.cuda.synchronize()
    graph = None
    if args.graph == "on":
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step(0, side)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            cap = torch.cuda.current_stream()
            for i in range(args.steps):
                step(i, cap)
        graph.replay()
        torch.cuda.synchronize()
    t0 = time.perf_counter()
    if graph is not None:
        graph.replay()
    else:
        for i in range(args.steps):
            step(i, stream)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    B.lrq_kernel_timing(True)
    for i in range(args.steps):
        step(i, stream)
    torch.cuda.synchronize()
    k_ms, n = B.lrq_kernel_time_ms(False)
    B.lrq_kernel_timing(False)
    assert n == args.steps
    dom = min(k_ms, ms_per_step)
    flop, byts = attn_work(w)
    tokens = w.n_seqs * w.q_len
    res = {"value": tokens / (ms_per_step * 1e-3), "unit": "tokens/s", "ms_per_step": ms_per_step, "dtype": "bf16",
           "config": {"workload": w.name, "description": w.description, "sequences": w.n_seqs, "q_len": w.q_len,
                      "kv_len": w.kv_len, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads, "head_dim": D,
                      "causal": w.causal, "kernel_family": "attention (flash, MFMA)",
                      "launch": "one HIP graph replay of the K steps" if graph is not None else "eager calls"},
           "tflops_step": flop / (ms_per_step * 1e-3) / 1e12}
    common = {"traffic": stored_traffic(w.name, "attn"), "kernel": "attn_kernel", "launch_ms": dom,
              "launch_ms_eager_events": k_ms}
    # the bound is whichever peak the algorithmic work takes longer on: at these sizes both
    # calls are HBM-bound (the prefill's 215 FLOP/B is below the 312 FLOP/B ridge)
    mfma_frac = flop / (dom * 1e-3) / 1e12 / PEAK_BF16_TFLOPS
    if byts / (PEAK_HBM_GBS * 1e9) >= flop / (PEAK_BF16_TFLOPS * 1e12):
        ach = byts / (dom * 1e-3) / 1e9
        res["roofline"] = {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                           "frac": ach / PEAK_HBM_GBS, "algorithmic_bytes": byts, "algorithmic_flop": flop,
                           "mfma_frac": mfma_frac, **common}
    else:
        ach = flop / (dom * 1e-3) / 1e12
        res["roofline"] = {"bound": "mfma", "achieved": ach, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                           "frac": ach / PEAK_BF16_TFLOPS, "algorithmic_flop": flop, "algorithmic_bytes": byts,
                           **common}
    if not args.no_cpu_baseline:
        import oracle.attn_oracle as at
        from oracle.lrq_oracle import rel_frobenius
        # a bounded sample: whole sequences (their q rows and cached rows copied to the host)
        n_seq_s = 2 if w.q_len > 1 else 8
        seqs = list(range(0, w.n_seqs, max(1, w.n_seqs // n_seq_s)))[:n_seq_s]
        q_rows = np.concatenate([np.arange(s * w.q_len, (s + 1) * w.q_len) for s in seqs])
        kv_rows = np.concatenate([np.arange(s * w.kv_len, (s + 1) * w.kv_len) for s in seqs])
        f64 = lambda t: t.float().cpu().numpy().astype(np.float64)  # noqa: E731
        qh = f64(inp["q"][torch.from_numpy(q_rows).cuda()])
        kh = f64(inp["k_cache"][torch.from_numpy(kv_rows).cuda()])
        vh = f64(inp["v_cache"][torch.from_numpy(kv_rows).cuda()])
        got = f64(out[torch.from_numpy(q_rows).cuda()])
        qi = np.arange(0, len(seqs) * w.q_len + 1, w.q_len)
        ki = np.arange(0, len(seqs) * w.kv_len + 1, w.kv_len)
        n_threads = cpu_threads()
        t0 = time.perf_counter()
        ref = at.attention(qh, kh, vh, qi, ki, np.arange(len(kv_rows)), w.n_q_heads, w.n_kv_heads, D,
                           causal=w.causal)
        dt = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": len(q_rows) / dt, "unit": "tokens/s", "cores": n_threads, "kind": "oracle",
                               "sample": f"{len(seqs)} of {w.n_seqs} sequences ({len(q_rows)} query rows), float64 "
                                         f"numpy, {dt:.2f} s",
                               "gpu_parity_rel_fro": rel_frobenius(got, ref)}
    del graph, inp, out
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30, help="untimed steps first (the clocks settle within about 20 steps of sustained MFMA load)")
    ap.add_argument("--workload", default="all",
                    choices=("all",) + ALL_WORKLOADS + ("train_dropout", "decode_nf4", "attn_prefill", "attn_decode",
                                                       "mlp_llama3"),
                    help="all: every workload, the headline (llama2, the largest) on the top level and all five "
                         "under 'configs'")
    ap.add_argument("--variant", default="auto", choices=["auto", "generic", "tiled", "decode"])
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle work for each cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-mlp", action="store_true", help="leave the SwiGLU-MLP workload out of the default run")
    ap.add_argument("--dropout", type=float, default=0.05,
                    help="LoRA dropout rate of the extra train_dropout entry of the default run (0: leave it out)")
    ap.add_argument("--no-prepare", action="store_true",
                    help="let every call prepare the frozen weights itself (no lrq_prepare_weights)")
    ap.add_argument("--copies", type=int, default=0,
                    help="rotate among this many copies of the streamed operands (default: enough for >= 400 MB, "
                         "more than the 256 MB MALL)")
    ap.add_argument("--graph", choices=["on", "off"], default="on",
                    help="launch the K timed steps as one replay of a HIP graph that holds them (on), or as "
                         "eager library calls (off)")
    ap.add_argument("--kv-cache", action="store_true",
                    help="forward through the KV-cache entry: every token also writes its k and v rows to a "
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

    import torch

    if args.copy_probe:
        copy_probe(args.copy_probe, 5)
        return

    from layer_rmsnorm_qkv_amd import binding as B
    from layer_rmsnorm_qkv_amd import workloads as wl
    from layer_rmsnorm_qkv_amd.device import DeviceProblem

    B.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    names = ALL_WORKLOADS if args.workload == "all" else (args.workload,)
    results = {}
    for name in names:
        if name in ("train_dropout", "decode_nf4", "mlp_llama3") or name.startswith("attn_"):
            continue
        print(f"[bench] {name}: measuring", file=sys.stderr, flush=True)
        results[name] = run_config(name, args, B, wl, DeviceProblem)
        r = results[name]
        print(f"[bench] {name}: {r['ms_per_step']:.4f} ms/step, {r['value']:.4g} tokens/s, roofline "
              f"{r['roofline']['frac']:.3f} of {r['roofline']['kernel']}", file=sys.stderr, flush=True)
    if args.workload in ("all", "decode_nf4"):
        # the decode step with the QLoRA base (NF4 blocks)
        print("[bench] decode_nf4: measuring", file=sys.stderr, flush=True)
        results["decode_nf4"] = run_config("decode", args, B, wl, DeviceProblem, nf4=True, key="decode_nf4")
        r = results["decode_nf4"]
        print(f"[bench] decode_nf4: {r['ms_per_step']:.4f} ms/step, roofline {r['roofline']['frac']:.3f}",
              file=sys.stderr, flush=True)
        names = tuple(n for n in names if n != "decode_nf4") + ("decode_nf4",)
    if (args.workload == "all" and args.dropout > 0) or args.workload == "train_dropout":
        # the training step again with LoRA dropout (default: the rate of the pages' SFT example)
        print("[bench] train_dropout: measuring", file=sys.stderr, flush=True)
        results["train_dropout"] = run_config("train", args, B, wl, DeviceProblem,
                                              dropout=(args.dropout or 0.05, 0x5EED, 1), key="train_dropout")
        r = results["train_dropout"]
        print(f"[bench] train_dropout: {r['ms_per_step']:.4f} ms/step, roofline {r['roofline']['frac']:.3f}",
              file=sys.stderr, flush=True)
        names = tuple(n for n in names if n != "train_dropout") + ("train_dropout",)
    if args.workload == "all" or args.workload.startswith("attn_"):
        for an in (wl.ATTN_BY_NAME if args.workload == "all" else (args.workload,)):
            print(f"[bench] {an}: measuring", file=sys.stderr, flush=True)
            results[an] = run_attn_config(an, args, B, wl)
            r = results[an]
            print(f"[bench] {an}: {r['ms_per_step']:.4f} ms/step, roofline {r['roofline']['frac']:.3f}",
                  file=sys.stderr, flush=True)
            names = tuple(n for n in names if n != an) + (an,)
    if (args.workload == "all" and not args.no_mlp) or args.workload == "mlp_llama3":
        print("[bench] mlp_llama3: measuring", file=sys.stderr, flush=True)
        results["mlp_llama3"] = run_mlp_config("mlp_llama3", args, B, wl)
        r = results["mlp_llama3"]
        print(f"[bench] mlp_llama3: {r['ms_per_step']:.4f} ms/step, roofline {r['roofline']['frac']:.3f}",
              file=sys.stderr, flush=True)
        names = tuple(n for n in names if n != "mlp_llama3") + ("mlp_llama3",)
    top = dict(results[names[0]])
    # an entry measured on its own (attention, MLP) still carries the line's common fields
    for k, v in (("metric", f"{names[0]} throughput"), ("n_gpus", 1), ("steps", args.steps),
                 ("warmup", args.warmup), ("higher_is_better", True), ("scaling", "weak"),
                 ("vs_baseline", None), ("data", "synthetic")):
        top.setdefault(k, v)
    if len(names) > 1:
        top["configs"] = {n: {k: v for k, v in results[n].items()
                              if k not in ("metric", "n_gpus", "higher_is_better", "scaling", "data", "steps",
                                           "warmup")} for n in names}
    print(json.dumps(top), flush=True)


if __name__ == "__main__":
    main()
