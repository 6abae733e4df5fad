"""Checks that pin the attention oracle to things other than itself: closed forms (one key, equal
scores), torch's scaled_dot_product_attention in float64 (grouped heads repeated, an explicit
bottom-right causal mask), scalar loops over a paged multi-sequence case, causality, the slot
indirection and the row-subset helper.  Used by ``test_attn_oracle.py`` on the real oracle and on
planted mistakes."""
from __future__ import annotations

import math

import numpy as np


def paged_case(seed=0, lens=((3, 5), (1, 6), (4, 4)), hq=4, hkv=2, D=8, extra_slots=5):
    """Sequences with (q_len, kv_len), cache rows in shuffled order (a paged cache)."""
    rng = np.random.default_rng(seed)
    q_ind, kv_ind = [0], [0]
    for ql, kl in lens:
        q_ind.append(q_ind[-1] + ql)
        kv_ind.append(kv_ind[-1] + kl)
    n_slots = kv_ind[-1] + extra_slots
    slots = rng.permutation(n_slots)[:kv_ind[-1]]
    q = rng.standard_normal((q_ind[-1], hq * D + 3 * D))      # wider rows: k and v blocks follow
    kc = rng.standard_normal((n_slots, hkv * D))
    vc = rng.standard_normal((n_slots, hkv * D))
    return dict(q=q, k_cache=kc, v_cache=vc, q_indptr=q_ind, kv_indptr=kv_ind, kv_slots=slots,
                n_q_heads=hq, n_kv_heads=hkv, head_dim=D)


def _close(got, want, tol, what):
    err = float(np.max(np.abs(np.asarray(got) - np.asarray(want))))
    assert err <= tol, f"{what}: {err:.3e} > {tol:.1e}"


def check_closed_forms(a):
    """One visible key gives its value; q = 0 makes every score equal, so the output is the mean
    of the visible values (query i of a causal sequence sees kv_len - q_len + i + 1 keys)."""
    c = paged_case(seed=1, lens=((1, 1), (2, 2)))
    out = a.attention(**c)
    g = c["n_q_heads"] // c["n_kv_heads"]
    D = c["head_dim"]
    for h in range(c["n_q_heads"]):
        kvh = h // g
        _close(out[0, h * D:(h + 1) * D], c["v_cache"][c["kv_slots"][0], kvh * D:(kvh + 1) * D], 1e-14, "one key")
        _close(out[1, h * D:(h + 1) * D], c["v_cache"][c["kv_slots"][1], kvh * D:(kvh + 1) * D], 1e-14,
               "first query of a causal sequence")
    c = paged_case(seed=2, lens=((3, 5),))
    c["q"] = np.zeros_like(c["q"])
    out = a.attention(**c)
    for i in range(3):
        vis = c["kv_slots"][:5 - 3 + i + 1]
        for h in range(c["n_q_heads"]):
            kvh = h // g
            _close(out[i, h * D:(h + 1) * D], np.mean(c["v_cache"][vis, kvh * D:(kvh + 1) * D], axis=0), 1e-14,
                   "equal scores")


def check_torch_sdpa(a):
    """Against torch.nn.functional.scaled_dot_product_attention in float64, with the kv heads
    repeated for their query groups and an explicit mask: a prefill sequence (q_len = kv_len)
    and a chunk (q_len < kv_len, the last queries of the sequence); also causal off."""
    import torch
    for lens, causal in ((((7, 7),), True), (((3, 9),), True), (((4, 6),), False)):
        c = paged_case(seed=3, lens=lens, hq=6, hkv=2, D=16)
        ql, kl = lens[0]
        D, hq, hkv = 16, 6, 2
        slots = np.asarray(c["kv_slots"])
        qt = torch.from_numpy(c["q"][:, :hq * D].reshape(ql, hq, D).transpose(1, 0, 2).copy())
        kt = torch.from_numpy(c["k_cache"][slots].reshape(kl, hkv, D).transpose(1, 0, 2).copy())
        vt = torch.from_numpy(c["v_cache"][slots].reshape(kl, hkv, D).transpose(1, 0, 2).copy())
        kt = kt.repeat_interleave(hq // hkv, dim=0)
        vt = vt.repeat_interleave(hq // hkv, dim=0)
        mask = None
        if causal:
            mask = torch.from_numpy(np.arange(kl)[None, :] <= (kl - ql + np.arange(ql))[:, None])
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
        ref = ref.permute(1, 0, 2).reshape(ql, hq * D).numpy()
        _close(a.attention(**dict(c, n_q_heads=hq, n_kv_heads=hkv, head_dim=D), causal=causal), ref, 1e-12,
               f"torch sdpa {lens} causal={causal}")


def brute(c, scale=None, causal=True):
    q, kc, vc = c["q"], c["k_cache"], c["v_cache"]
    hq, hkv, D = c["n_q_heads"], c["n_kv_heads"], c["head_dim"]
    s = 1.0 / math.sqrt(D) if scale is None else scale
    out = np.zeros((q.shape[0], hq * D))
    for b in range(len(c["q_indptr"]) - 1):
        q0, q1 = c["q_indptr"][b], c["q_indptr"][b + 1]
        slots = list(c["kv_slots"][c["kv_indptr"][b]:c["kv_indptr"][b + 1]])
        for i in range(q0, q1):
            last = len(slots) - (q1 - q0) + (i - q0) if causal else len(slots) - 1
            for h in range(hq):
                g = h // (hq // hkv)
                sc = [s * sum(q[i][h * D + e] * kc[slots[j]][g * D + e] for e in range(D)) for j in range(last + 1)]
                mx = max(sc)
                w = [math.exp(v - mx) for v in sc]
                tot = sum(w)
                for e in range(D):
                    out[i][h * D + e] = sum(w[j] * vc[slots[j]][g * D + e] for j in range(last + 1)) / tot
    return out


def check_brute_force(a):
    """Scalar loops over a paged cache with three sequences (decode, chunk and prefill shapes),
    default and explicit scale, causal on and off."""
    c = paged_case(seed=4)
    _close(a.attention(**c), brute(c), 1e-12, "brute force causal")
    _close(a.attention(**c, scale=0.3), brute(c, scale=0.3), 1e-12, "brute force scale 0.3")
    _close(a.attention(**c, causal=False), brute(c, causal=False), 1e-12, "brute force non-causal")


def check_causality_and_slots(a):
    """Keys a query cannot see do not change it, a visible one does; permuting the cache rows
    together with the slot list changes nothing; rows of other sequences are untouched."""
    c = paged_case(seed=5, lens=((2, 6), (1, 3)))
    base = a.attention(**c)
    c2 = dict(c, v_cache=c["v_cache"].copy(), k_cache=c["k_cache"].copy())
    c2["v_cache"][c["kv_slots"][5]] += 10.0      # the last key of sequence 0: only its last query sees it
    got = a.attention(**c2)
    _close(got[0], base[0], 0.0, "first query must not see the last key")
    assert np.max(np.abs(got[1] - base[1])) > 1e-3
    _close(got[2], base[2], 0.0, "other sequence")
    perm = np.random.default_rng(6).permutation(c["k_cache"].shape[0])
    inv = np.argsort(perm)
    c3 = dict(c, k_cache=c["k_cache"][perm], v_cache=c["v_cache"][perm], kv_slots=inv[np.asarray(c["kv_slots"])])
    _close(a.attention(**c3), base, 1e-13, "slot indirection")


def check_rows_helper(a):
    """attention_rows equals the full output's rows (unsorted, repeated), causal on and off."""
    c = paged_case(seed=7)
    rows = [7, 0, 3, 3, 5]
    for causal in (True, False):
        full = a.attention(**c, causal=causal)
        _close(a.attention_rows(rows, **c, causal=causal), full[rows], 1e-13, f"rows causal={causal}")


def check_degenerate_sequences(a):
    """A sequence without queries (with or without keys) writes nothing and leaves the other
    sequences' rows as they are alone; with kv_len < q_len the queries before the first key get
    zero rows and the others see their windows (checked by scalar loops)."""
    c = paged_case(seed=8, lens=((0, 0), (2, 3), (0, 4)))
    alone = paged_case(seed=8, lens=((0, 0), (2, 3), (0, 4)))
    alone.update(q_indptr=[0, 2], kv_indptr=[0, 3], kv_slots=c["kv_slots"][0:3])
    _close(a.attention(**c), a.attention(**alone), 1e-15, "sequences without queries")
    c = paged_case(seed=9, lens=((4, 2),))
    out = a.attention(**c)
    assert not np.any(out[:2])
    _close(out[2:], brute(dict(c, q=c["q"][2:], q_indptr=[0, 2]))[:, :out.shape[1]], 1e-12, "late queries")


ALL_CHECKS = [check_closed_forms, check_torch_sdpa, check_brute_force, check_causality_and_slots, check_rows_helper,
              check_degenerate_sequences]
