"""CPU oracle for the fused RMSNorm -> QKV projection (+ LoRA) -> RoPE operator.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The
product path (the HIP library and its Python binding) never touches it, and it
shares no code with that path: plain float64 numpy, written from the
definitions, with no tiling, fusion or reordering beyond what the definitions
state.  ``numpy @`` (BLAS dgemm) is the only library primitive used.

What it computes, per token t with row x_t (length d):

    inv_t   = 1 / sqrt( mean_j x_tj^2 + eps )                  RMSNorm statistics
    h_t     = x_t * inv_t * gamma                              normalised activations
    y_t     = W h_t + b                                        fused q|k|v projection
    y_t[c]  += (alpha / r) * B_c (A_c h_t)                     LoRA on target c in {q,k,v}
    out_t   = RoPE(y_t; pos_t)                                 rotate-half on q and k heads

Sources (the web pages on Liger-Kernel, cited by title and section):

* RMSNorm with eps inside the square root of the mean of squares, then times
  the norm weight: page "Liger-Kernel底层优化：新一代内核级推理加速引擎深度解析",
  fused-kernel pseudocode, "Step 1: RMSNorm"; projection with bias before the
  rotary step: same pseudocode, "Step 2: QKV Projection".
* The unfused chain that the fused operator replaces (normalise, project to
  q, k, v, rotate q and k but not v): page "Swift-All一文详解：如何用Liger-Kernel
  提升训练效率", section 2.2 (1) "RMSNorm + Rotary Embedding + Attention QKV 融合";
  and the decoder-layer op sequence on the inference-engine page above.
* LoRA as a frozen projection plus the product of a down matrix A [r, d_in] and
  an up matrix B [d_out, r] (down applied to x first, up to its result): page
  "Liger-Kernel内核级优化：GPU利用率飙升至90%以上", section "为什么传统微调会卡脖子"
  (the y = Wx + B(Ax) formula and its unfused decomposition).  The scale alpha/r
  and LoRA acting on the normalised input are readings (see below).
* Rotary embedding: the pages' pseudocode indexes frequencies by
  ``feature mod (head_dim/2)``, which is the half-split (GPT-NeoX,
  "rotate-half") pairing; the rest of that pseudocode does not rotate pairs of
  one head, so the standard rotate-half rotation with base theta is used:
  omega_i = theta^(-2i/D), phi = pos * omega_i, and the pair
  (y[i], y[i + D/2]) -> (a cos phi - b sin phi, b cos phi + a sin phi).

Readings where the pages are silent or garbled: LoRA scale s = alpha / r; LoRA
applied to the normalised activations h (the input of q_proj/k_proj/v_proj);
LoRA dropout (when a ``Dropout`` is given) on each adapter's input only, with its own
Philox4x32-10 mask (section "LoRA dropout" below), the identity otherwise; the output
columns are q heads | k heads | v heads, head-major; v is never rotated; bias (if any) is
added before RoPE.

Backward (frozen W, gamma and b; upstream gradient dy w.r.t. the rotated
output): G = RoPE^-1(dy) on q and k blocks (dy on v); V_c = G_c B_c;
dh = W^T G + sum_c s A_c^T V_c; dx = inv * gamma * dh - inv^3 * x * <gamma x, dh> / d;
dA_c = s sum_t V_c^T h;  dB_c = s sum_t G_c^T U_c with U_c = A_c h.  This is
the chain rule of the forward above, nothing more.

Every function here is pinned by tests against things other than itself:
closed forms, special cases, an independent complex-number formulation of the
rotation, the merged-weight formulation of LoRA, scalar brute force on tiny
inputs, and central finite differences for the backward.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Mapping, Optional, Sequence, Tuple

import numpy as np

TARGET_Q = 1
TARGET_K = 2
TARGET_V = 4
TARGETS = (TARGET_Q, TARGET_K, TARGET_V)


@dataclass(frozen=True)
class Spec:
    """Shape and hyper-parameters of one call (the oracle's own copy; no import from the product)."""
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    lora_rank: int = 0
    lora_alpha: float = 0.0
    lora_targets: int = 0
    eps: float = 1e-6
    rope_theta: float = 10000.0

    @property
    def n_out(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def lora_scale(self) -> float:
        # reading: the LoRA update is scaled by alpha / r
        return self.lora_alpha / self.lora_rank if self.lora_rank > 0 else 0.0

    def columns(self, target: int) -> Tuple[int, int]:
        """Output columns of one of q, k, v: q heads, then k heads, then v heads."""
        D = self.head_dim
        nq, nkv = self.n_q_heads * D, self.n_kv_heads * D
        return {TARGET_Q: (0, nq), TARGET_K: (nq, nq + nkv), TARGET_V: (nq + nkv, nq + 2 * nkv)}[target]

    def rotated_columns(self) -> Tuple[int, int]:
        """q and k heads are rotated; they are the first (Hq + Hkv) * D columns."""
        return 0, (self.n_q_heads + self.n_kv_heads) * self.head_dim


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------- RMSNorm

def rms_inverse(x: np.ndarray, eps: float) -> np.ndarray:
    """inv_t = 1/sqrt(mean_j x_tj^2 + eps) (eps inside the root, mean over the hidden size).

    Inference-engine page, fused-kernel pseudocode, "Step 1: RMSNorm".
    """
    x = _f64(x)
    return 1.0 / np.sqrt(np.mean(x * x, axis=-1) + eps)


def rms_normalise(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """h = x * inv * gamma: normalise each row, then multiply by the norm weight.

    Inference-engine page, pseudocode "Step 1" / "Step 2" (the projection input is
    x * inv_rms * weight[i]).
    """
    x = _f64(x)
    return x * rms_inverse(x, eps)[:, None] * _f64(gamma)[None, :]


# --------------------------------------------------------------------------- RoPE

def rope_frequencies(head_dim: int, theta: float) -> np.ndarray:
    """omega_i = theta^(-2i/D) for i in [0, D/2): one frequency per half-split pair."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * i / head_dim)


def rope_angles(positions: np.ndarray, head_dim: int, theta: float) -> np.ndarray:
    """phi[t, i] = pos_t * omega_i."""
    return _f64(positions)[:, None] * rope_frequencies(head_dim, theta)[None, :]


def rope_rotate(y: np.ndarray, positions: np.ndarray, head_dim: int, theta: float,
                inverse: bool = False) -> np.ndarray:
    """Rotate-half RoPE applied to every head of ``y`` ([T, n_heads * D]).

    Within each head the pair (a, b) = (y[i], y[i + D/2]) becomes
    (a cos phi - b sin phi, b cos phi + a sin phi); ``inverse`` rotates by -phi.
    Swift-All page section 2.2 (1) (q and k are rotated); inference-engine
    pseudocode "Step 3" (frequency index = feature mod D/2).
    """
    y = _f64(y)
    T, n = y.shape
    D = head_dim
    half = D // 2
    phi = rope_angles(positions, D, theta)
    if inverse:
        phi = -phi
    c, s = np.cos(phi)[:, None, :], np.sin(phi)[:, None, :]
    heads = y.reshape(T, n // D, D)
    a, b = heads[:, :, :half], heads[:, :, half:]
    out = np.empty_like(heads)
    out[:, :, :half] = a * c - b * s
    out[:, :, half:] = b * c + a * s
    return out.reshape(T, n)


# --------------------------------------------------------------------------- LoRA dropout
#
# The LoRA configuration on the pages carries a dropout rate (lora_dropout 0.05 in the
# Swift-All page's SftArguments, section 3.2; 0.1 in the LoRAConfig of the inference-engine
# page's usage section).  Reading: as in the standard LoRA training recipe, dropout acts on the
# adapter's input only -- the frozen projection sees h itself -- with an independent mask per
# adapted projection (q, k, v each have their own), kept values scaled by 1 / (1 - p).
# The masks come from the counter-based generator Philox4x32-10 (Salmon, Moraes, Dror and
# Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011), so that a backward pass can
# regenerate them: counter (j // 4, row, target, offset), key (seed low, seed high); word
# j % 4 of the output keeps feature j of that row iff it is >= floor(p * 2^32).

_PHILOX_M0, _PHILOX_M1 = 0xD2511F53, 0xCD9E8D57
_PHILOX_W0, _PHILOX_W1 = 0x9E3779B9, 0xBB67AE85
_U32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(ctr: np.ndarray, key: Tuple[int, int]) -> np.ndarray:
    """Philox4x32 with 10 rounds on counters ``ctr`` ([..., 4] of uint32 values), one key
    (k0, k1): each round multiplies words 0 and 2 by the two multipliers (64-bit products),
    and the new words are (hi(M1 x2) ^ x1 ^ k0, lo(M1 x2), hi(M0 x0) ^ x3 ^ k1, lo(M0 x0));
    the key is bumped by the two Weyl constants between rounds.  Returns uint32 words."""
    x = np.asarray(ctr, dtype=np.uint64) & _U32
    x0, x1, x2, x3 = x[..., 0], x[..., 1], x[..., 2], x[..., 3]
    k0, k1 = np.uint64(key[0] & 0xFFFFFFFF), np.uint64(key[1] & 0xFFFFFFFF)
    for rnd in range(10):
        if rnd > 0:
            k0 = (k0 + np.uint64(_PHILOX_W0)) & _U32
            k1 = (k1 + np.uint64(_PHILOX_W1)) & _U32
        p0 = np.uint64(_PHILOX_M0) * x0
        p1 = np.uint64(_PHILOX_M1) * x2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _U32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _U32
        x0, x1, x2, x3 = hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0
    return np.stack([x0, x1, x2, x3], axis=-1).astype(np.uint32)


def dropout_threshold(p: float) -> int:
    """floor(p * 2^32): a generator word below it drops its feature."""
    return int(np.floor(float(p) * 4294967296.0))


def dropout_keep(n_rows: int, d: int, target_index: int, p: float, seed: int, offset: int,
                 rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Boolean keep mask [rows, d] of adapter ``target_index`` (0 q, 1 k, 2 v) for the call's
    token rows (all n_rows rows, or the given subset)."""
    rows = np.arange(n_rows) if rows is None else np.asarray(rows, dtype=np.int64)
    nq = (d + 3) // 4
    ctr = np.zeros((len(rows), nq, 4), dtype=np.uint64)
    ctr[..., 0] = np.arange(nq, dtype=np.uint64)[None, :]
    ctr[..., 1] = rows.astype(np.uint64)[:, None]
    ctr[..., 2] = np.uint64(target_index)
    ctr[..., 3] = np.uint64(offset & 0xFFFFFFFF)
    words = philox4x32_10(ctr, (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)).reshape(len(rows), nq * 4)[:, :d]
    return words >= np.uint32(dropout_threshold(p)) if p > 0 else np.ones((len(rows), d), dtype=bool)


@dataclass(frozen=True)
class Dropout:
    """LoRA dropout of one call: rate p in [0, 1), generator seed and per-call offset."""
    p: float
    seed: int = 0
    offset: int = 0


def _adapter_inputs(spec: Spec, h: np.ndarray, dropout: Optional[Dropout], rows=None) -> Dict[int, np.ndarray]:
    """The input each adapter sees: h, or h * mask / (1 - p) under dropout."""
    out = {}
    for i, c in enumerate(TARGETS):
        if not (spec.lora_targets & c):
            continue
        if dropout is None or dropout.p == 0.0:
            out[c] = h
        else:
            r_idx = np.arange(h.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
            keep = dropout_keep(h.shape[0], spec.d_model, i, dropout.p, dropout.seed, dropout.offset, rows=r_idx)
            out[c] = h * keep / (1.0 - dropout.p)
    return out


# --------------------------------------------------------------------------- forward

def lora_update(spec: Spec, h: np.ndarray, a: Mapping[int, np.ndarray],
                b: Mapping[int, np.ndarray], dropout: Optional[Dropout] = None,
                rows=None) -> Dict[int, np.ndarray]:
    """For each target c: s * B_c (A_c h_c) ([T, N_c]), h_c the adapter's input (h, or h
    with dropout applied; ``rows`` are the call's row indices of h's rows).

    LoRA page "Liger-Kernel内核级优化", y = Wx + B(Ax) and its unfused two-step
    decomposition (down, then up); scale s = alpha / r (reading).
    """
    out = {}
    ins = _adapter_inputs(spec, h, dropout, rows)
    for c in TARGETS:
        if spec.lora_targets & c:
            u = ins[c] @ _f64(a[c]).T       # [T, r]   down projection
            out[c] = spec.lora_scale * (u @ _f64(b[c]).T)   # [T, N_c] up projection
    return out


def pre_rope(spec: Spec, x, gamma, w, bias, a, b, dropout: Optional[Dropout] = None, rows=None) -> np.ndarray:
    """y = W h + b + LoRA updates, before the rotation ([T, N])."""
    h = rms_normalise(x, gamma, spec.eps)
    y = h @ _f64(w).T
    if bias is not None:
        y = y + _f64(bias)[None, :]
    for c, upd in lora_update(spec, h, a, b, dropout, rows).items():
        lo, hi = spec.columns(c)
        y[:, lo:hi] += upd
    return y


def forward(spec: Spec, x, gamma, w, bias, a, b, positions, dropout: Optional[Dropout] = None,
            rows=None) -> np.ndarray:
    """out = RoPE(W h + b + s B(A h)) with h = RMSNorm(x) * gamma; [T, N] float64.

    The unfused chain of the Swift-All page, section 2.2 (1), plus the LoRA
    branch of the LoRA page; v columns are not rotated.  With ``dropout``, each adapter
    sees its own dropped-out copy of h (``rows``: the call's row indices of x's rows, for
    the mask; default 0..T-1).
    """
    y = pre_rope(spec, x, gamma, w, bias, a, b, dropout, rows)
    lo, hi = spec.rotated_columns()
    y[:, lo:hi] = rope_rotate(y[:, lo:hi], positions, spec.head_dim, spec.rope_theta)
    return y


def forward_rows(spec: Spec, rows: Sequence[int], x, gamma, w, bias, a, b, positions,
                 dropout: Optional[Dropout] = None) -> np.ndarray:
    """``forward`` on a subset of token rows (rows are independent given their positions)."""
    rows = np.asarray(rows, dtype=np.int64)
    return forward(spec, np.asarray(x)[rows], gamma, w, bias, a, b, np.asarray(positions)[rows], dropout,
                   rows=rows)


def forward_chunked(spec: Spec, x, gamma, w, bias, a, b, positions, chunk: int = 2048,
                    dropout: Optional[Dropout] = None) -> np.ndarray:
    """``forward`` over all rows, ``chunk`` rows at a time to bound float64 memory."""
    T = np.asarray(x).shape[0]
    out = np.empty((T, spec.n_out), dtype=np.float64)
    for s0 in range(0, T, chunk):
        s1 = min(T, s0 + chunk)
        out[s0:s1] = forward(spec, np.asarray(x)[s0:s1], gamma, w, bias, a, b,
                             np.asarray(positions)[s0:s1], dropout, rows=np.arange(s0, s1))
    return out


# --------------------------------------------------------------------------- key/value cache

def kv_cache_write(spec: Spec, out, slots, k_cache, v_cache) -> Tuple[np.ndarray, np.ndarray]:
    """The caches after a forward call writes its keys and values: a copy of each cache with
    row slots[t] replaced by token t's k block (columns of the k heads) and v block of
    ``out``, for every token whose slot lies in [0, num_slots); other rows are kept.  The
    attention step that follows the projection reads the rotated k and the v (decoder-layer
    op sequence on the inference-engine page; the same page lists a fused attention kernel
    with KV-cache handling).  The row-per-token layout is a reading: the pages define none.
    Slots must be distinct among the written tokens (several correct results otherwise)."""
    out = _f64(out)
    kc, vc = _f64(k_cache).copy(), _f64(v_cache).copy()
    k_lo, k_hi = spec.columns(TARGET_K)
    v_lo, v_hi = spec.columns(TARGET_V)
    n = kc.shape[0]
    for t, slot in enumerate(np.asarray(slots).tolist()):
        if 0 <= slot < n:
            kc[slot] = out[t, k_lo:k_hi]
            vc[slot] = out[t, v_lo:v_hi]
    return kc, vc


# --------------------------------------------------------------------------- backward

def unrotate_grad(spec: Spec, dy, positions) -> np.ndarray:
    """G = gradient w.r.t. the pre-rotation y: the transpose (= inverse) rotation on q, k."""
    g = _f64(dy).copy()
    lo, hi = spec.rotated_columns()
    g[:, lo:hi] = rope_rotate(g[:, lo:hi], positions, spec.head_dim, spec.rope_theta, inverse=True)
    return g


def backward(spec: Spec, x, gamma, w, bias, a, b, positions, dy,
             dx_rows: Optional[Sequence[int]] = None, dropout: Optional[Dropout] = None):
    """Gradients of <dy, forward(x)> w.r.t. x and the LoRA factors (W, gamma, b frozen).

    Returns (dx, dA, dB): dx [T, d] (or [len(dx_rows), d]); dA[c] [r, d] and dB[c]
    [N_c, r] for every target c, summed over all tokens.  The LoRA page notes
    that the fused backward recomputes rather than stores; here everything is
    simply recomputed from x.  ``bias`` does not enter the gradients.  With ``dropout``
    the same masks as the forward's are regenerated; an adapter's gradient then reaches
    h only through the kept features (its input is h * mask / (1 - p)).
    """
    del bias
    x = _f64(x)
    s = spec.lora_scale
    inv = rms_inverse(x, spec.eps)
    h = rms_normalise(x, gamma, spec.eps)
    G = unrotate_grad(spec, dy, positions)
    ins = _adapter_inputs(spec, h, dropout)
    dA, dB, V = {}, {}, {}
    for c in TARGETS:
        if spec.lora_targets & c:
            lo, hi = spec.columns(c)
            Ac, Bc = _f64(a[c]), _f64(b[c])
            V[c] = G[:, lo:hi] @ Bc                 # [T, r]
            U = ins[c] @ Ac.T                       # [T, r]
            dA[c] = s * (V[c].T @ ins[c])           # [r, d]
            dB[c] = s * (G[:, lo:hi].T @ U)         # [N_c, r]
    rows = np.arange(x.shape[0]) if dx_rows is None else np.asarray(dx_rows, dtype=np.int64)
    dh = G[rows] @ _f64(w)
    for i, c in enumerate(TARGETS):
        if c not in V:
            continue
        term = s * (V[c][rows] @ _f64(a[c]))
        if dropout is not None and dropout.p > 0.0:
            # d(input)/dh = mask / (1 - p): the adapter's gradient flows through kept features
            keep = dropout_keep(x.shape[0], spec.d_model, i, dropout.p, dropout.seed, dropout.offset, rows=rows)
            term = term * keep / (1.0 - dropout.p)
        dh += term
    gam = _f64(gamma)
    xr, invr = x[rows], inv[rows]
    c_row = np.sum(gam[None, :] * xr * dh, axis=1)      # <gamma x, dh> per row
    d = x.shape[1]
    dx = invr[:, None] * gam[None, :] * dh - (invr ** 3)[:, None] * xr * (c_row / d)[:, None]
    return dx, dA, dB


# --------------------------------------------------------------------------- error metric

def rel_frobenius(got, ref) -> float:
    """||got - ref||_F / ||ref||_F in float64 (0 when both are empty or ref is all zero and equal)."""
    got, ref = _f64(got), _f64(ref)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((got - ref).ravel())
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)
