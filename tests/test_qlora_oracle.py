"""The NF4 (QLoRA base) oracle against its pins, and plausible planted mistakes that the pins
must reject (CPU only)."""
import numpy as np
import pytest

import oracle.qlora_oracle as q
import qlora_pins


@pytest.mark.parametrize("check", qlora_pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check(q)


_real_quantize = q.quantize
_real_pack = q.pack


def _levels_wrong_delta():
    return q.nf4_construction(delta=1.0 / 32.0).astype(np.float32)


def _levels_symmetric():
    from scipy.stats import norm
    v = norm.ppf(np.linspace(0.02, 0.98, 16))
    return (v / v.max()).astype(np.float32)


def _quantize_ties_up(w, levels=None):
    w = np.asarray(w, dtype=np.float32)
    n, d = w.shape
    blocks = w.reshape(n, d // 64, 64)
    absmax = np.max(np.abs(blocks), axis=2).astype(np.float32)
    safe = np.where(absmax > 0, absmax, np.float32(1.0)).astype(np.float32)
    y = (blocks / safe[:, :, None]).astype(np.float32)
    codes = np.sum(y[..., None] >= q.midpoints(levels)[None, None, None, :], axis=-1).astype(np.uint8)
    codes = np.where(absmax[:, :, None] > 0, codes, np.uint8(7)).astype(np.uint8)
    return codes.reshape(n, d), absmax


def _quantize_row_scale(w, levels=None):
    w = np.asarray(w, dtype=np.float32)
    n, d = w.shape
    absmax = np.max(np.abs(w), axis=1, keepdims=True).astype(np.float32)
    y = (w / np.where(absmax > 0, absmax, 1.0)).astype(np.float32)
    codes = np.sum(y[..., None] > q.midpoints(levels)[None, None, :], axis=-1).astype(np.uint8)
    return codes, np.repeat(absmax, d // 64, axis=1)


def _pack_high_first(codes, scales):
    codes = np.asarray(codes, dtype=np.uint8)
    swapped = codes.copy()
    swapped[:, 0::2], swapped[:, 1::2] = codes[:, 1::2], codes[:, 0::2]
    return _real_pack(swapped, scales)


def _dequantize_no_scale(codes, scales, levels=None):
    return q.NF4_LEVELS.astype(np.float64)[np.asarray(codes, np.int64)]


MUTANTS = {
    "code book with delta = 1/32": ("NF4_LEVELS", _levels_wrong_delta()),
    "symmetric code book without an exact zero": ("NF4_LEVELS", _levels_symmetric()),
    "ties to the upper level": ("quantize", _quantize_ties_up),
    "one scale per row instead of per block": ("quantize", _quantize_row_scale),
    "high nibble first": ("pack", _pack_high_first),
    "dequantise without the block scale": ("dequantize", _dequantize_no_scale),
}


@pytest.mark.filterwarnings("ignore::RuntimeWarning")
@pytest.mark.parametrize("name", list(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    where, repl = MUTANTS[name]
    monkeypatch.setattr(q, where, repl)
    failed = []
    for chk in qlora_pins.ALL_CHECKS:
        try:
            chk(q)
        except Exception:  # noqa: BLE001
            failed.append(chk.__name__)
    assert failed, f"no pin caught the planted mistake '{name}'"
