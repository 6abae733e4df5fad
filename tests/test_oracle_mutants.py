"""Plant plausible mistakes in the CPU oracle and check that the pins reject each one.

Each mutant replaces one piece of ``oracle.lrq_oracle`` (on the CPU, for the
duration of one test) with a wrong variant; the pin suite must then fail at
least one check.  This shows the pins are strong enough to catch a dropped
term, a wrong sign or index, or a transposed operand anywhere in the oracle.
"""
import numpy as np
import pytest

import oracle.lrq_oracle as o
import pins


def _eps_outside(x, eps):
    x = np.asarray(x, np.float64)
    return 1.0 / np.sqrt(np.mean(x * x, axis=-1)) + eps


def _sum_not_mean(x, eps):
    x = np.asarray(x, np.float64)
    return 1.0 / np.sqrt(np.sum(x * x, axis=-1) + eps)


def _no_sqrt(x, eps):
    x = np.asarray(x, np.float64)
    return 1.0 / (np.mean(x * x, axis=-1) + eps)


def _no_gamma(x, gamma, eps):
    x = np.asarray(x, np.float64)
    return x * o.rms_inverse(x, eps)[:, None]


def _freq_half_exponent(head_dim, theta):
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(theta), -1.0 * i / head_dim)


def _freq_off_by_one(head_dim, theta):
    i = np.arange(1, head_dim // 2 + 1, dtype=np.float64)
    return np.power(float(theta), -2.0 * i / head_dim)


_real_rotate = o.rope_rotate


def _rotate_wrong_sign(y, positions, head_dim, theta, inverse=False):
    return _real_rotate(y, positions, head_dim, theta, inverse=not inverse)


def _rotate_interleaved(y, positions, head_dim, theta, inverse=False):
    # pairs (2i, 2i+1) instead of (i, i + D/2)
    y = np.asarray(y, np.float64)
    T, n = y.shape
    phi = o.rope_angles(positions, head_dim, theta) * (-1 if inverse else 1)
    c, s = np.cos(phi)[:, None, :], np.sin(phi)[:, None, :]
    hh = y.reshape(T, n // head_dim, head_dim // 2, 2)
    a, b = hh[..., 0], hh[..., 1]
    out = np.stack([a * c - b * s, b * c + a * s], axis=-1)
    return out.reshape(T, n)


def _rotated_all(self):
    return 0, self.n_out


def _rotated_q_only(self):
    return 0, self.n_q_heads * self.head_dim


def _scale_alpha(self):
    return self.lora_alpha


def _lora_on_x(spec, h, a, b):
    # LoRA applied to a rescaled input instead of h (drops gamma)
    out = {}
    for c in o.TARGETS:
        if spec.lora_targets & c:
            hh = h / np.sqrt(np.mean(h * h, axis=1, keepdims=True))
            out[c] = spec.lora_scale * ((hh @ np.asarray(a[c]).T) @ np.asarray(b[c]).T)
    return out


def _lora_wrong_block(self, target):
    D = self.head_dim
    nq, nkv = self.n_q_heads * D, self.n_kv_heads * D
    # v adapter lands on the k block
    return {o.TARGET_Q: (0, nq), o.TARGET_K: (nq, nq + nkv), o.TARGET_V: (nq, nq + nkv)}[target]


_real_backward = o.backward


def _bwd_drop_inv3(spec, x, gamma, w, bias, a, b, positions, dy, dx_rows=None):
    # dx = inv * gamma * dh only: the RMSNorm term through the row statistic is dropped
    _, dA, dB = _real_backward(spec, x, gamma, w, bias, a, b, positions, dy, dx_rows)
    x = np.asarray(x, np.float64)
    rows = np.arange(x.shape[0]) if dx_rows is None else np.asarray(dx_rows)
    G = o.unrotate_grad(spec, dy, positions)
    dh = G @ np.asarray(w, np.float64)
    for c in dA:
        lo, hi = spec.columns(c)
        dh += spec.lora_scale * ((G[:, lo:hi] @ np.asarray(b[c])) @ np.asarray(a[c]))
    inv = o.rms_inverse(x, spec.eps)
    return (inv[:, None] * np.asarray(gamma)[None, :] * dh)[rows], dA, dB


def _bwd_db_with_h(spec, x, gamma, w, bias, a, b, positions, dy, dx_rows=None):
    dx, dA, dB = _real_backward(spec, x, gamma, w, bias, a, b, positions, dy, dx_rows)
    G = o.unrotate_grad(spec, dy, positions)
    h = o.rms_normalise(x, gamma, spec.eps)
    for c in dB:
        lo, hi = spec.columns(c)
        dB[c] = spec.lora_scale * (G[:, lo:hi].T @ h[:, :dB[c].shape[1]])
    return dx, dA, dB


def _bwd_no_unrotate(spec, dy, positions):
    return np.asarray(dy, np.float64).copy()


def _kv_swapped(spec, out, slots, k_cache, v_cache):
    kc, vc = _real_kv(spec, out, slots, k_cache, v_cache)
    return vc, kc


def _kv_clamped(spec, out, slots, k_cache, v_cache):
    n = np.asarray(k_cache).shape[0]
    return _real_kv(spec, out, np.clip(np.asarray(slots), 0, n - 1), k_cache, v_cache)


_real_kv = o.kv_cache_write


def _rows_positions_unsliced(spec, rows, x, gamma, w, bias, a, b, positions):
    # the rows' activations are taken, but the positions of the first len(rows) tokens
    rows = np.asarray(rows, dtype=np.int64)
    return o.forward(spec, np.asarray(x)[rows], gamma, w, bias, a, b, np.asarray(positions)[:len(rows)])


def _chunks_restart_positions(spec, x, gamma, w, bias, a, b, positions, chunk=2048):
    # every chunk is rotated with the positions of the first chunk (a chunk-boundary slip)
    T = np.asarray(x).shape[0]
    out = np.empty((T, spec.n_out))
    for s0 in range(0, T, chunk):
        s1 = min(T, s0 + chunk)
        out[s0:s1] = o.forward(spec, np.asarray(x)[s0:s1], gamma, w, bias, a, b, np.asarray(positions)[0:s1 - s0])
    return out


def _chunks_overlapping_short(spec, x, gamma, w, bias, a, b, positions, chunk=2048):
    # chunk bounds that step by chunk - 1: chunks overlap and the last row is never written
    T = np.asarray(x).shape[0]
    out = np.zeros((T, spec.n_out))
    for s0 in range(0, max(T - 1, 1), max(chunk - 1, 1)):
        s1 = min(T - 1, s0 + chunk)
        out[s0:s1] = o.forward(spec, np.asarray(x)[s0:s1], gamma, w, bias, a, b, np.asarray(positions)[s0:s1])
    return out


_real_keep = o.dropout_keep
_real_inputs = o._adapter_inputs


def _keep_inverted(n_rows, d, target_index, p, seed, offset, rows=None):
    m = _real_keep(n_rows, d, target_index, p, seed, offset, rows)
    return ~m if p > 0 else m


def _keep_shared_across_targets(n_rows, d, target_index, p, seed, offset, rows=None):
    return _real_keep(n_rows, d, 0, p, seed, offset, rows)


def _keep_offset_ignored(n_rows, d, target_index, p, seed, offset, rows=None):
    return _real_keep(n_rows, d, target_index, p, seed, 0, rows)


def _dropout_unscaled(spec, h, dropout, rows=None):
    out = _real_inputs(spec, h, dropout, rows)
    if dropout is not None and dropout.p > 0:
        out = {c: v * (1.0 - dropout.p) for c, v in out.items()}
    return out


def _philox_nine_rounds(ctr, key):
    x = np.asarray(ctr, dtype=np.uint64) & np.uint64(0xFFFFFFFF)
    x0, x1, x2, x3 = x[..., 0], x[..., 1], x[..., 2], x[..., 3]
    k0, k1 = np.uint64(key[0]), np.uint64(key[1])
    m = np.uint64(0xFFFFFFFF)
    for rnd in range(9):
        if rnd > 0:
            k0, k1 = (k0 + np.uint64(0x9E3779B9)) & m, (k1 + np.uint64(0xBB67AE85)) & m
        p0, p1 = np.uint64(0xD2511F53) * x0, np.uint64(0xCD9E8D57) * x2
        x0, x1, x2, x3 = (p1 >> np.uint64(32)) ^ x1 ^ k0, p1 & m, (p0 >> np.uint64(32)) ^ x3 ^ k1, p0 & m
    return np.stack([x0, x1, x2, x3], axis=-1).astype(np.uint32)


MUTANTS = {
    "eps outside sqrt": ("rms_inverse", _eps_outside),
    "sum instead of mean": ("rms_inverse", _sum_not_mean),
    "missing sqrt": ("rms_inverse", _no_sqrt),
    "gamma dropped": ("rms_normalise", _no_gamma),
    "frequency exponent -i/D": ("rope_frequencies", _freq_half_exponent),
    "frequency index off by one": ("rope_frequencies", _freq_off_by_one),
    "rotation sign flipped": ("rope_rotate", _rotate_wrong_sign),
    "interleaved pairs": ("rope_rotate", _rotate_interleaved),
    "v rotated too": ("Spec.rotated_columns", _rotated_all),
    "k not rotated": ("Spec.rotated_columns", _rotated_q_only),
    "scale alpha not alpha/r": ("Spec.lora_scale", property(_scale_alpha)),
    "LoRA input without gamma": ("lora_update", _lora_on_x),
    "adapter on wrong block": ("Spec.columns", _lora_wrong_block),
    "dx missing inv^3 term": ("backward", _bwd_drop_inv3),
    "dB uses h instead of U": ("backward", _bwd_db_with_h),
    "gradient not un-rotated": ("unrotate_grad", _bwd_no_unrotate),
    "k and v cache rows swapped": ("kv_cache_write", _kv_swapped),
    "out-of-range slots clamped into the cache": ("kv_cache_write", _kv_clamped),
    "row subset keeps the first rows' positions": ("forward_rows", _rows_positions_unsliced),
    "chunks restart the positions": ("forward_chunked", _chunks_restart_positions),
    "overlapping chunks, last row unwritten": ("forward_chunked", _chunks_overlapping_short),
    "dropout keeps the words below the threshold": ("dropout_keep", _keep_inverted),
    "one dropout mask for all adapters": ("dropout_keep", _keep_shared_across_targets),
    "dropout offset ignored": ("dropout_keep", _keep_offset_ignored),
    "dropout without the 1/(1-p) scale": ("_adapter_inputs", _dropout_unscaled),
    "Philox with nine rounds": ("philox4x32_10", _philox_nine_rounds),
}


def _failures(checks):
    failed = []
    for chk in checks:
        try:
            chk(o)
        except Exception:  # noqa: BLE001 - any failure counts as "caught"
            failed.append(chk.__name__)
    return failed


# a mutant may divide by zero on the pins' all-zero rows; that is part of how it fails
@pytest.mark.filterwarnings("ignore::RuntimeWarning")
@pytest.mark.parametrize("name", list(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    where, repl = MUTANTS[name]
    if where.startswith("Spec."):
        monkeypatch.setattr(o.Spec, where[5:], repl)
    else:
        monkeypatch.setattr(o, where, repl)
    failed = _failures(pins.ALL_CHECKS)
    assert failed, f"no pin caught the planted mistake '{name}'"
