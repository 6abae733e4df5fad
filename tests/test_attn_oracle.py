"""The attention oracle against its pins, and plausible planted mistakes that the pins must
reject (CPU only)."""
import numpy as np
import pytest

import attn_pins
import oracle.attn_oracle as a


@pytest.mark.parametrize("check", attn_pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check(a)


_real = a.attention


def _no_scale(*args, scale=None, causal=True, **kw):
    return _real(*args, scale=1.0 if scale is None else scale, causal=causal, **kw)


def _window_short(q, k_cache, v_cache, q_indptr, kv_indptr, kv_slots, n_q_heads, n_kv_heads, head_dim,
                  scale=None, causal=True):
    # each query loses its own key (strict instead of inclusive window), first query sees key 0
    out = np.zeros((np.asarray(q).shape[0], n_q_heads * head_dim))
    for b in range(len(q_indptr) - 1):
        q0, q1 = q_indptr[b], q_indptr[b + 1]
        slots = np.asarray(kv_slots)[kv_indptr[b]:kv_indptr[b + 1]]
        for i in range(q0, q1):
            last = max(len(slots) - (q1 - q0) + (i - q0) - 1, 0) if causal else len(slots) - 1
            out[i] = _real(np.asarray(q)[i:i + 1], k_cache, v_cache, [0, 1], [0, last + 1], slots[:last + 1],
                           n_q_heads, n_kv_heads, head_dim, scale, causal=False)[0]
    return out


def _gqa_modulo(q, k_cache, v_cache, q_indptr, kv_indptr, kv_slots, n_q_heads, n_kv_heads, head_dim,
                scale=None, causal=True):
    # query head h reads kv head h % Hkv instead of h // (Hq / Hkv)
    D, g = head_dim, n_q_heads // n_kv_heads
    kc = np.asarray(k_cache, np.float64)
    vc = np.asarray(v_cache, np.float64)
    kc2, vc2 = np.zeros((kc.shape[0], n_q_heads * D)), np.zeros((vc.shape[0], n_q_heads * D))
    for h in range(n_q_heads):
        kc2[:, h * D:(h + 1) * D] = kc[:, (h % n_kv_heads) * D:(h % n_kv_heads + 1) * D]
        vc2[:, h * D:(h + 1) * D] = vc[:, (h % n_kv_heads) * D:(h % n_kv_heads + 1) * D]
    del g
    return _real(q, kc2, vc2, q_indptr, kv_indptr, kv_slots, n_q_heads, n_q_heads, head_dim, scale, causal)


def _values_are_keys(q, k_cache, v_cache, *args, **kw):
    return _real(q, k_cache, k_cache, *args, **kw)


def _bottom_left_top_right(q, k_cache, v_cache, q_indptr, kv_indptr, kv_slots, n_q_heads, n_kv_heads, head_dim,
                           scale=None, causal=True):
    # causal window anchored at the first key (query i sees keys 0..i), as if q_len == kv_len
    out = np.zeros((np.asarray(q).shape[0], n_q_heads * head_dim))
    for b in range(len(q_indptr) - 1):
        q0, q1 = q_indptr[b], q_indptr[b + 1]
        slots = np.asarray(kv_slots)[kv_indptr[b]:kv_indptr[b + 1]]
        for i in range(q0, q1):
            last = (i - q0) if causal else len(slots) - 1
            out[i] = _real(np.asarray(q)[i:i + 1], k_cache, v_cache, [0, 1], [0, last + 1], slots[:last + 1],
                           n_q_heads, n_kv_heads, head_dim, scale, causal=False)[0]
    return out


MUTANTS = {
    "no 1/sqrt(D) scale": _no_scale,
    "causal window excludes the query's own key": _window_short,
    "grouped heads mapped by modulo": _gqa_modulo,
    "values read from the key cache": _values_are_keys,
    "causal window anchored at the first key": _bottom_left_top_right,
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    monkeypatch.setattr(a, "attention", MUTANTS[name])
    failed = []
    for chk in attn_pins.ALL_CHECKS:
        if chk is attn_pins.check_rows_helper:
            continue  # compares the oracle with itself
        try:
            chk(a)
        except Exception:  # noqa: BLE001
            failed.append(chk.__name__)
    assert failed, f"no pin caught the planted mistake '{name}'"
