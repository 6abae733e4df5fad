"""CPU oracle for the LoRA-adapted SwiGLU MLP (the fused MLP the pages describe next to the
fused attention-input projection).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The product path never
touches it and shares no code with it: plain float64 numpy, written from the definitions,
with no tiling, fusion or reordering beyond what they state.  ``numpy @`` (BLAS dgemm) is the
only library primitive used.

What it computes, per token row h (length d, the MLP's input):

    g = W_g h + (alpha / r) B_g (A_g h)        gate projection  [F]   (LoRA when targeted)
    u = W_u h + (alpha / r) B_u (A_u h)        up projection    [F]
    a = SiLU(g) * u,   SiLU(z) = z / (1 + exp(-z))              SwiGLU
    y = W_d a + (alpha / r) B_d (A_d a)        down projection  [d]

Sources (web pages on Liger-Kernel, cited by title and section):

* SwiGLU MLP fused end to end (Linear -> SwiGLU -> Linear) for LLaMA-family FFNs, so the
  intermediate activations need not be stored: "Swift-All一文详解：如何用Liger-Kernel提升训练效率",
  section 2.2 (2) "SwiGLU 激活函数融合".
* A LoRA linear (frozen W plus up(down(x))) with the SiLU activation fused into its last
  step, instead of separate matmul, add and SiLU launches: "Liger-Kernel内核级优化：GPU利用率
  飙升至90%以上", section "内核融合".
* The MLP's three projections (gate_proj, up_proj, down_proj) and the gated SwiGLU
  activation as fused components: "Liger-Kernel底层优化：新一代内核级推理加速引擎深度解析",
  the fused-kernel list and the list of covered components.

Readings (the pages do not spell them out): SwiGLU is SiLU(gate) times up (the LLaMA MLP);
LoRA scale alpha / r and the A [r, d_in] / B [d_out, r] roles as in the attention projection;
the MLP takes its input h as given (its RMSNorm is a separate operator on the pages' layer
listing); no biases; dropout is the identity.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Mapping, Optional, Sequence

import numpy as np

TARGET_GATE = 1
TARGET_UP = 2
TARGET_DOWN = 4
TARGETS = (TARGET_GATE, TARGET_UP, TARGET_DOWN)


@dataclass(frozen=True)
class MlpSpec:
    d_model: int
    d_ff: int
    lora_rank: int = 0
    lora_alpha: float = 0.0
    lora_targets: int = 0

    @property
    def lora_scale(self) -> float:
        return self.lora_alpha / self.lora_rank if self.lora_rank > 0 else 0.0


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def silu(z) -> np.ndarray:
    """SiLU(z) = z * sigmoid(z) = z / (1 + exp(-z)); exp overflows to inf for very negative z,
    which gives the correct limit -0."""
    z = _f64(z)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def lora_linear(spec: MlpSpec, x, w, a: Optional[np.ndarray], b: Optional[np.ndarray]) -> np.ndarray:
    """x W^T, plus (alpha / r) (x A^T) B^T when an adapter is given: the frozen projection plus
    up(down(x)) of the LoRA page's formula."""
    y = _f64(x) @ _f64(w).T
    if a is not None:
        y = y + spec.lora_scale * ((_f64(x) @ _f64(a).T) @ _f64(b).T)
    return y


def mlp_forward(spec: MlpSpec, h, w_gate, w_up, w_down, a: Mapping[int, np.ndarray],
                b: Mapping[int, np.ndarray]) -> np.ndarray:
    """y = down(SiLU(gate(h)) * up(h)) for every row of h ([T, d] -> [T, d], float64)."""
    def ad(t):
        on = spec.lora_targets & t
        return (a[t], b[t]) if on else (None, None)
    g = lora_linear(spec, h, w_gate, *ad(TARGET_GATE))
    u = lora_linear(spec, h, w_up, *ad(TARGET_UP))
    act = silu(g) * u
    return lora_linear(spec, act, w_down, *ad(TARGET_DOWN))


def mlp_forward_rows(spec: MlpSpec, rows: Sequence[int], h, w_gate, w_up, w_down, a, b) -> np.ndarray:
    """``mlp_forward`` on a subset of token rows (rows are independent)."""
    rows = np.asarray(rows, dtype=np.int64)
    return mlp_forward(spec, np.asarray(h)[rows], w_gate, w_up, w_down, a, b)


def mlp_activation(spec: MlpSpec, h, w_gate, w_up, a, b) -> np.ndarray:
    """a = SiLU(gate(h)) * up(h), the intermediate the fused gate/up kernel produces."""
    def ad(t):
        on = spec.lora_targets & t
        return (a[t], b[t]) if on else (None, None)
    return silu(lora_linear(spec, h, w_gate, *ad(TARGET_GATE))) * lora_linear(spec, h, w_up, *ad(TARGET_UP))
