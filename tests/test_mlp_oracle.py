"""The SwiGLU-MLP oracle against its pins, and plausible planted mistakes that the pins must
reject (CPU only)."""
import numpy as np
import pytest

import mlp_pins
import oracle.mlp_oracle as o


@pytest.mark.parametrize("check", mlp_pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check(o)


_real_silu = o.silu
_real_lora = o.lora_linear
_real_fwd = o.mlp_forward


def _sigmoid_not_silu(z):
    z = np.asarray(z, np.float64)
    return 1.0 / (1.0 + np.exp(-z))


def _relu_not_silu(z):
    return np.maximum(np.asarray(z, np.float64), 0.0)


def _silu_sign_flipped(z):
    z = np.asarray(z, np.float64)
    return z / (1.0 + np.exp(z))


def _lora_without_scale(spec, x, w, a, b):
    y = np.asarray(x, np.float64) @ np.asarray(w, np.float64).T
    if a is not None:
        y = y + (np.asarray(x) @ np.asarray(a).T) @ np.asarray(b).T
    return y


def _gate_up_swapped(spec, h, w_gate, w_up, w_down, a, b):
    return _real_fwd(spec, h, w_up, w_gate, w_down, {1: a.get(2), 2: a.get(1), 4: a.get(4)},
                     {1: b.get(2), 2: b.get(1), 4: b.get(4)})


def _down_lora_on_h(spec, h, w_gate, w_up, w_down, a, b):
    no_down = o.MlpSpec(spec.d_model, spec.d_ff, spec.lora_rank, spec.lora_alpha, spec.lora_targets & 3)
    y = _real_fwd(no_down, h, w_gate, w_up, w_down, a, b)
    if spec.lora_targets & 4 and a[4].shape[1] == np.asarray(h).shape[1]:
        y = y + spec.lora_scale * ((np.asarray(h) @ a[4].T) @ b[4].T)
    elif spec.lora_targets & 4:
        y = y + 1e-3  # wrong input shape for the down adapter: any change is a mistake
    return y


MUTANTS = {
    "sigmoid instead of SiLU": ("silu", _sigmoid_not_silu),
    "ReLU instead of SiLU": ("silu", _relu_not_silu),
    "SiLU with the sign flipped": ("silu", _silu_sign_flipped),
    "LoRA scale dropped": ("lora_linear", _lora_without_scale),
    "gate and up swapped": ("mlp_forward", _gate_up_swapped),
    "down adapter applied to h": ("mlp_forward", _down_lora_on_h),
}


@pytest.mark.filterwarnings("ignore::RuntimeWarning")
@pytest.mark.parametrize("name", list(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    where, repl = MUTANTS[name]
    monkeypatch.setattr(o, where, repl)
    failed = []
    for chk in mlp_pins.ALL_CHECKS:
        try:
            chk(o)
        except Exception:  # noqa: BLE001
            failed.append(chk.__name__)
    assert failed, f"no pin caught the planted mistake '{name}'"
