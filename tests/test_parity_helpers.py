"""The GPU parity checks themselves, on the CPU: a defect confined to one element, or to one
row, passes the relative Frobenius bar of a whole tensor but not the per-row or per-element
bounds; a result with only rounding-sized errors passes all three."""
import numpy as np
import pytest

from helpers import TOL, assert_parity, forward_errors
from layer_rmsnorm_qkv_amd import workloads as wl


def _case():
    w = wl.get("llama3").replace(n_tokens=64, d_model=256, n_q_heads=4, n_kv_heads=2)
    rng = np.random.default_rng(5)
    ref = rng.standard_normal((w.n_tokens, w.n_out))
    # rounding-sized noise: one bf16 rounding of the output plus a small random term
    got = wl.round_to_bf16(ref + 2.0 ** -10 * rng.standard_normal(ref.shape)).astype(np.float64)
    return w, got, ref


def test_rounding_sized_errors_pass():
    w, got, ref = _case()
    assert_parity(forward_errors(w, got, ref), "bf16")


def test_one_wrong_element_is_caught():
    w, got, ref = _case()
    bad = got.copy()
    bad[17, 300] += 1.0  # one element off by about one RMS
    errs = forward_errors(w, bad, ref)
    assert errs["out"] <= TOL["bf16"]  # the tensor-wide bar alone would not see it
    with pytest.raises(AssertionError):
        assert_parity(errs, "bf16")


def test_one_wrong_row_is_caught():
    w, got, ref = _case()
    bad = got.copy()
    bad[9, :32] *= 1.25  # one 32-column group of one row scaled
    errs = forward_errors(w, bad, ref)
    assert errs["out"] <= TOL["bf16"]
    with pytest.raises(AssertionError):
        assert_parity(errs, "bf16")
