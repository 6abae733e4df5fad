"""Shared plumbing of the GPU parity tests: run the HIP path through the C ABI and the
oracle on the same seeded inputs, and measure the relative Frobenius error."""
from __future__ import annotations

import sys

import numpy as np

import oracle.lrq_oracle as o
from layer_rmsnorm_qkv_amd import binding as B
from layer_rmsnorm_qkv_amd import workloads as wl

TOL = {"f32": 1e-5, "bf16": 5e-3}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def spec_of(w: wl.Workload) -> o.Spec:
    return o.Spec(d_model=w.d_model, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads, head_dim=w.head_dim,
                  lora_rank=w.lora_rank if w.lora_targets else 0, lora_alpha=w.lora_alpha,
                  lora_targets=w.lora_targets, eps=w.eps, rope_theta=w.rope_theta)


def to_np(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def oracle_forward(w, inp, rows=None):
    spec = spec_of(w)
    if rows is None:
        return o.forward_chunked(spec, inp["x"], inp["gamma"], inp["w"], inp["bias"], inp["a"], inp["b"],
                                 inp["positions"])
    return o.forward_rows(spec, rows, inp["x"], inp["gamma"], inp["w"], inp["bias"], inp["a"], inp["b"],
                          inp["positions"])


def forward_errors(w, got: np.ndarray, ref: np.ndarray):
    """Relative Frobenius error of the whole output and of each of the q, k, v blocks."""
    errs = {"out": o.rel_frobenius(got, ref)}
    for name, t in (("q", wl.TARGET_Q), ("k", wl.TARGET_K), ("v", wl.TARGET_V)):
        lo, hi = w.target_columns()[t]
        errs[name] = o.rel_frobenius(got[:, lo:hi], ref[:, lo:hi])
    return errs


def sample_rows(T: int, n: int, seed: int = 0) -> np.ndarray:
    """First and last rows plus a seeded sample (covers both ends of the tile grid)."""
    if T <= n:
        return np.arange(T)
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(1, T - 1), size=n - 2, replace=False)
    return np.sort(np.concatenate([[0, T - 1], mid]))
