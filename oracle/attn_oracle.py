"""Oracle of the attention step that reads the key/value cache (the part of the KV-cache row
that follows the projection).  Test infrastructure: only tests/, the smoke check and the
benchmark's CPU baseline import it.

Page "Liger-Kernel底层优化：新一代内核级推理加速引擎深度解析" lists a fused attention kernel
with KV-cache handling next to the fused norm/QKV/RoPE kernel, and its decoder-layer op
sequence computes the attention output from the rotated q, k and v
(scaled_dot_product_attention(q, k, v)).  The pages define nothing further.  Readings:
  (R-A1) scaled dot-product attention: softmax over keys of q.k * scale, scale = 1/sqrt(D)
         unless given, weights applied to v, per query head;
  (R-A2) grouped-query heads: query head h reads kv head h // (Hq / Hkv) (q heads of one kv
         head are consecutive, the layout of the projection's q and k blocks);
  (R-A3) causal, as in decoder-only models: the queries of a sequence are its last q_len
         tokens, and query i (0-based within the call's queries of the sequence) sees keys
         0 .. kv_len - q_len + i; with causal off every query sees all kv_len keys;
  (R-A4) the keys and values of a sequence are cache rows named by a slot list (one row of
         Hkv * D values per token, the layout the projection's cache write uses), in token
         order; q rows come from the projection's output (q heads first in each row);
  (R-A5) degenerate cases: a sequence without queries contributes nothing, and a query that
         sees no key (kv_len < q_len puts early queries before the first key) gets a zero row.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np


def attention(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, q_indptr: Sequence[int],
              kv_indptr: Sequence[int], kv_slots: Sequence[int], n_q_heads: int, n_kv_heads: int,
              head_dim: int, scale: Optional[float] = None, causal: bool = True) -> np.ndarray:
    """q [T_q, >= Hq*D] (q heads in the first Hq*D columns), caches [num_slots, Hkv*D];
    sequence b has query rows q_indptr[b] .. q_indptr[b+1] and keys kv_slots[kv_indptr[b] ..
    kv_indptr[b+1]].  Returns out [T_q, Hq*D] in float64."""
    q = np.asarray(q, np.float64)
    kc = np.asarray(k_cache, np.float64)
    vc = np.asarray(v_cache, np.float64)
    D, Hq, Hkv = head_dim, n_q_heads, n_kv_heads
    group = Hq // Hkv
    s = 1.0 / np.sqrt(D) if scale is None else float(scale)
    out = np.zeros((q.shape[0], Hq * D))
    for b in range(len(q_indptr) - 1):
        q0, q1 = int(q_indptr[b]), int(q_indptr[b + 1])
        slots = np.asarray(kv_slots[int(kv_indptr[b]):int(kv_indptr[b + 1])], dtype=np.int64)
        q_len, kv_len = q1 - q0, len(slots)
        if q_len == 0:
            continue
        n_vis = np.minimum(kv_len, kv_len - q_len + np.arange(q_len) + 1) if causal else np.full(q_len, kv_len)
        seen = n_vis > 0                                             # rows with at least one key (R-A5)
        for h in range(Hq):
            g = h // group
            keys = kc[slots, g * D:(g + 1) * D]                     # [kv_len, D]
            vals = vc[slots, g * D:(g + 1) * D]
            scores = q[q0:q1, h * D:(h + 1) * D] @ keys.T * s        # [q_len, kv_len]
            if causal:
                visible = np.arange(kv_len)[None, :] <= (kv_len - q_len + np.arange(q_len))[:, None]
                scores = np.where(visible, scores, -np.inf)
            if not np.any(seen):
                continue
            sc = scores[seen]
            m = np.max(sc, axis=1, keepdims=True)
            w = np.exp(sc - m)
            out[q0 + np.flatnonzero(seen), h * D:(h + 1) * D] = (w @ vals) / np.sum(w, axis=1, keepdims=True)
    return out


def attention_rows(rows: Sequence[int], q, k_cache, v_cache, q_indptr, kv_indptr, kv_slots, n_q_heads,
                   n_kv_heads, head_dim, scale=None, causal=True) -> np.ndarray:
    """The output rows ``rows`` only: each row as a one-query sequence over the keys it sees."""
    q_indptr = np.asarray(q_indptr, np.int64)
    kv_indptr = np.asarray(kv_indptr, np.int64)
    slots = np.asarray(kv_slots, np.int64)
    res = np.zeros((len(rows), n_q_heads * head_dim))
    for n, r in enumerate(rows):
        b = int(np.searchsorted(q_indptr, r, side="right") - 1)
        kv_len = int(kv_indptr[b + 1] - kv_indptr[b])
        last = kv_len - int(q_indptr[b + 1] - q_indptr[b]) + (r - int(q_indptr[b])) if causal else kv_len - 1
        if last < 0:
            continue  # no visible key: a zero row (R-A5)
        mine = slots[int(kv_indptr[b]):int(kv_indptr[b]) + last + 1]
        res[n] = attention(np.asarray(q)[r:r + 1], k_cache, v_cache, [0, 1], [0, len(mine)], mine, n_q_heads,
                           n_kv_heads, head_dim, scale, causal=False)[0]
    return res
