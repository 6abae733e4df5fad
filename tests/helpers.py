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


# Per-element bound |g - o| <= C_REL |o| + C_ABS rms(reference row) [+ C_LORA e_lora], per
# dtype.  For bf16 (8 significant bits) the unit roundoff is u = 2^-8: the output's own rounding
# contributes at most u |o| (C_REL = u), and one rounding of each operand of a length-d dot
# product (the weights with gamma folded in, h or x) adds a random error of about 0.8 u times
# the RMS of the row's values when W ~ N(0, 1/d), so C_ABS = 6u is about 7 standard deviations
# of that part (a CPU emulation of the kernels' rounding points reaches 0.45 of the bound on
# 3 million elements), still ~40x below the O(rms) error of one wrong element.  Float32
# (u = 2^-24) takes the same form with room for the library's sin / cos and accumulation
# order: C_ABS = 2e-5 (twice the Frobenius bar).
#
# The rank-r LoRA intermediate (U = A h in the forward, V = s G B in the backward) is also
# rounded once to bf16 before its r-term product, and with few ranks that error does not
# average out: it is at most u |U_k| per rank, so an element gains at most
# u * s * sum_k |B_nk| |U_k| (forward; summed over a rotation pair, since RoPE mixes the pair)
# or u * inv * |gamma_j| * sum_k |V_k| |A_kj| (dx).  Tests whose adapters dominate the output
# pass that term as e_lora (lora_bound_forward / lora_bound_dx), with C_LORA = 1.25 u (room for
# U itself carrying fp32 accumulation error before its rounding).
C_REL = {"bf16": 2.0 ** -8, "f32": 2.0 ** -23}
C_ABS = {"bf16": 12 * 2.0 ** -9, "f32": 2e-5}
ROW_FACTOR = 2.0  # per-row relative Frobenius error bar = ROW_FACTOR x the tensor bar


def row_rel_errors(got: np.ndarray, ref: np.ndarray) -> float:
    """Largest relative Frobenius error of one row (a row whose reference is all zero must be
    reproduced exactly)."""
    if got.size == 0:
        return 0.0
    num = np.linalg.norm(got - ref, axis=1)
    den = np.linalg.norm(ref, axis=1)
    zero = den == 0.0
    rel = np.where(zero, np.where(num == 0.0, 0.0, np.inf), num / np.where(zero, 1.0, den))
    return float(np.max(rel))


C_LORA = {"bf16": 1.25 * 2.0 ** -8, "f32": 1.25 * 2.0 ** -24}


def elem_ratio(got: np.ndarray, ref: np.ndarray, dtype: str, scale: str = "row", lora=None) -> float:
    """max over elements of |g - o| / (C_REL |o| + C_ABS s [+ C_LORA e_lora]), s = the RMS of the
    element's reference row (scale="row") or of the whole tensor ("tensor"), e_lora = ``lora``
    (an array of the same shape, see lora_bound_*); <= 1 passes."""
    if got.size == 0:
        return 0.0
    err = np.abs(got - ref)
    if scale == "row":
        s = np.sqrt(np.mean(ref * ref, axis=1, keepdims=True))
    else:
        s = np.sqrt(np.mean(ref * ref))
    bound = C_REL[dtype] * np.abs(ref) + C_ABS[dtype] * s
    if lora is not None:
        bound = bound + C_LORA[dtype] * lora
    ratio = np.where(bound > 0.0, err / np.where(bound > 0.0, bound, 1.0), np.where(err == 0.0, 0.0, np.inf))
    return float(np.max(ratio))


def _keep(w, t_index, dropout, n_rows, rows):
    if dropout is None or dropout.p == 0.0:
        return 1.0
    return o.dropout_keep(n_rows, w.d_model, t_index, dropout.p, dropout.seed, dropout.offset, rows=rows)


def lora_bound_forward(w, inp, dropout=None, rows=None) -> np.ndarray:
    """e_lora of the forward output [rows, N]: s * |U_t| |B_t|^T in target t's columns, with U_t
    the exact rank-r intermediate (of the dropped-out input), summed over each rotation pair on
    q and k."""
    x = np.asarray(inp["x"], np.float64)
    rows = np.arange(x.shape[0]) if rows is None else np.asarray(rows)
    h = o.rms_normalise(x[rows], inp["gamma"], w.eps)
    p = 0.0 if dropout is None else dropout.p
    e = np.zeros((len(rows), w.n_out))
    s = w.lora_alpha / w.lora_rank
    cols = w.target_columns()
    for i, t in enumerate((wl.TARGET_Q, wl.TARGET_K, wl.TARGET_V)):
        if not (w.lora_targets & t):
            continue
        hin = h * _keep(w, i, dropout, x.shape[0], rows) / (1.0 - p)
        u = hin @ np.asarray(inp["a"][t], np.float64).T
        lo, hi = cols[t]
        e[:, lo:hi] = s * (np.abs(u) @ np.abs(np.asarray(inp["b"][t], np.float64)).T)
    cv, half = cols[wl.TARGET_V][0], w.head_dim // 2
    rot = e[:, :cv].reshape(len(rows), -1, 2, half)
    pair = rot[:, :, 0, :] + rot[:, :, 1, :]
    e[:, :cv] = np.stack([pair, pair], axis=2).reshape(len(rows), cv)
    return e


def lora_bound_dx(w, inp, dropout=None, rows=None) -> np.ndarray:
    """e_lora of dx [rows, d]: inv * |gamma_j| * sum_t keep_t * (|V_t| |A_t|)_j / (1 - p), with
    V_t = s G_t B_t the exact rank-r intermediate of the backward."""
    spec = spec_of(w)
    x = np.asarray(inp["x"], np.float64)
    rows = np.arange(x.shape[0]) if rows is None else np.asarray(rows)
    inv = o.rms_inverse(x, w.eps)[rows]
    g = o.unrotate_grad(spec, inp["dy"], inp["positions"])[rows]
    s = w.lora_alpha / w.lora_rank
    p = 0.0 if dropout is None else dropout.p
    e = np.zeros((len(rows), w.d_model))
    cols = w.target_columns()
    for i, t in enumerate((wl.TARGET_Q, wl.TARGET_K, wl.TARGET_V)):
        if not (w.lora_targets & t):
            continue
        lo, hi = cols[t]
        v = s / (1.0 - p) * (g[:, lo:hi] @ np.asarray(inp["b"][t], np.float64))
        e += (np.abs(v) @ np.abs(np.asarray(inp["a"][t], np.float64))) * _keep(w, i, dropout, x.shape[0], rows)
    return e * inv[:, None] * np.abs(np.asarray(inp["gamma"], np.float64))[None, :]


def forward_errors(w, got: np.ndarray, ref: np.ndarray):
    """Relative Frobenius error of the whole output and of each of the q, k, v blocks, plus the
    worst row ("row": relative Frobenius error of one row) and the worst element ("elem": the
    ratio to the per-element bound)."""
    errs = {"out": o.rel_frobenius(got, ref)}
    for name, t in (("q", wl.TARGET_Q), ("k", wl.TARGET_K), ("v", wl.TARGET_V)):
        lo, hi = w.target_columns()[t]
        errs[name] = o.rel_frobenius(got[:, lo:hi], ref[:, lo:hi])
    errs["row"] = row_rel_errors(got, ref)
    errs["elem"] = elem_ratio(got, ref, w.dtype)
    return errs


def assert_parity(errs, dtype: str, what=""):
    """Frobenius errors against the dtype's bar, per-row errors ("...row") against ROW_FACTOR
    times it, per-element ratios ("...elem") against 1."""
    for k, v in errs.items():
        bar = 1.0 if k.endswith("elem") else (ROW_FACTOR * TOL[dtype] if k.endswith("row") else TOL[dtype])
        assert v <= bar, (what, k, v, bar, errs)


def sample_rows(T: int, n: int, seed: int = 0) -> np.ndarray:
    """First and last rows plus a seeded sample (covers both ends of the tile grid)."""
    if T <= n:
        return np.arange(T)
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(1, T - 1), size=n - 2, replace=False)
    return np.sort(np.concatenate([[0, T - 1], mid]))
