"""Device buffers for one call of the operator (torch for memory and streams only).

``DeviceProblem`` uploads the host arrays of a workload (see ``workloads``) to torch
device tensors of the workload dtype -- the values are exactly representable, so the
cast is exact -- builds the ``lrq_desc`` and calls the binding.  No arithmetic of the
operator happens here.
"""
from __future__ import annotations

from typing import Dict, Optional, Tuple

import numpy as np

from . import binding as B
from .workloads import TARGET_K, TARGET_Q, TARGET_V, Workload


def torch_dtype(w: Workload):
    import torch
    return torch.float32 if w.dtype == "f32" else torch.bfloat16


def desc_for(w: Workload, n_tokens: Optional[int] = None, variant: int = B.LRQ_VARIANT_AUTO,
             dropout: Optional[Tuple[float, int, int]] = None, nf4: bool = False) -> B.LrqDesc:
    """Descriptor of workload ``w``; ``dropout`` = (rate, seed, offset) turns on LoRA dropout,
    ``nf4`` stores W_qkv as NF4 blocks (the QLoRA base)."""
    p, seed, offset = dropout if dropout is not None else (0.0, 0, 0)
    return B.make_desc(w.n_tokens if n_tokens is None else n_tokens, w.d_model, w.n_q_heads, w.n_kv_heads,
                       w.head_dim, B.LRQ_F32 if w.dtype == "f32" else B.LRQ_BF16, w.eps, w.rope_theta,
                       w.lora_rank if w.lora_targets else 0, w.lora_alpha, w.lora_targets,
                       1 if w.has_bias else 0, variant, lora_dropout=p, dropout_offset=offset,
                       dropout_seed=seed, weight_format=B.LRQ_WEIGHT_NF4 if nf4 else B.LRQ_WEIGHT_DENSE)


class DeviceProblem:
    """All device tensors of one forward (+ backward) call."""

    def __init__(self, w: Workload, inputs: Dict[str, object], device: str = "cuda",
                 variant: int = B.LRQ_VARIANT_AUTO, backward: bool = False,
                 dropout: Optional[Tuple[float, int, int]] = None, nf4: bool = False):
        import torch
        self.w = w
        dt = torch_dtype(w)
        T = inputs["x"].shape[0]
        self.T = T
        self.desc = desc_for(w, T, variant, dropout, nf4)

        def up(a):
            return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(device=device, dtype=dt)

        self.x = up(inputs["x"])
        self.gamma = up(inputs["gamma"])
        self.w_qkv = up(inputs["w"])
        self.w_dense = self.w_qkv
        if nf4:
            # the QLoRA base: W quantised to NF4 blocks on the device; every call takes the buffer
            self.w_qkv = torch.empty(B.lrq_nf4_weight_size(self.desc), dtype=torch.uint8, device=device)
            B.lrq_quantize_nf4(self.desc, self.w_dense, self.w_qkv)
        self.bias = up(inputs["bias"])
        self.a = [up(inputs["a"].get(t)) for t in (TARGET_Q, TARGET_K, TARGET_V)]
        self.b = [up(inputs["b"].get(t)) for t in (TARGET_Q, TARGET_K, TARGET_V)]
        self.positions = torch.from_numpy(np.ascontiguousarray(inputs["positions"], dtype=np.int32)).to(device)
        self.out = torch.empty((T, w.n_out), dtype=dt, device=device)
        self.variant = B.lrq_select_variant(self.desc, False)
        ws = B.lrq_workspace_size(self.desc, False)
        self.dy = self.dx = None
        self.da = self.db = None
        if backward:
            self.dy = up(inputs["dy"])
            self.dx = torch.empty((T, w.d_model), dtype=dt, device=device)
            self.da = [torch.empty_like(a, dtype=torch.float32) if a is not None else None for a in self.a]
            self.db = [torch.empty_like(b, dtype=torch.float32) if b is not None else None for b in self.b]
            self.bwd_variant = B.lrq_select_variant(self.desc, True)
            ws = max(ws, B.lrq_workspace_size(self.desc, True))
        self.workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=device) if ws > 0 else None
        self.backward_enabled = backward
        self.prepared = None  # set by prepare(): forward/backward then pass the prepared weights

    def prepare(self, stream=None):
        """Build the prepared frozen-weight layouts of (gamma, w_qkv) once; later forward and
        backward calls pass them (the library then skips its per-call weight preparation)."""
        import torch
        n = B.lrq_prepared_size(self.desc, self.backward_enabled)
        self.prepared = torch.empty(max(n, 1), dtype=torch.uint8, device=self.x.device) if n > 0 else None
        if self.prepared is not None:
            B.lrq_prepare_weights(self.desc, self.backward_enabled, self.gamma, self.w_qkv, self.prepared,
                                  stream=stream)
        return self.prepared

    def forward(self, stream=None, out=None):
        o = self.out if out is None else out
        if self.prepared is None:
            B.lrq_forward(self.desc, self.x, self.gamma, self.w_qkv, self.bias, self.a, self.b, self.positions,
                          o, self.workspace, stream=stream)
        else:
            B.lrq_forward_prepared(self.desc, self.x, self.gamma, self.w_qkv, self.prepared, self.bias, self.a,
                                   self.b, self.positions, o, None, self.workspace, stream=stream)
        return o

    def backward(self, y=None, stream=None):
        yy = self.out if y is None else y
        if self.prepared is None:
            B.lrq_backward(self.desc, self.x, self.gamma, self.w_qkv, self.bias, self.a, self.b, self.positions,
                           yy, self.dy, self.dx, self.da, self.db, self.workspace, stream=stream)
        else:
            B.lrq_backward_prepared(self.desc, self.x, self.gamma, self.w_qkv, self.prepared, self.bias, self.a,
                                    self.b, self.positions, yy, self.dy, self.dx, self.da, self.db,
                                    self.workspace, stream=stream)
        return self.dx, self.da, self.db


class DeviceMlp:
    """Device tensors of one call of the LoRA-adapted SwiGLU MLP (lrq_mlp_forward)."""

    def __init__(self, w, inputs: Dict[str, object], device: str = "cuda"):
        import torch
        from .workloads import MLP_TARGET_DOWN, MLP_TARGET_GATE, MLP_TARGET_UP
        self.w = w
        T = inputs["h"].shape[0]
        self.desc = B.make_mlp_desc(T, w.d_model, w.d_ff, B.LRQ_BF16, w.lora_rank if w.lora_targets else 0,
                                    w.lora_alpha, w.lora_targets)

        def up(a):
            return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(device=device,
                                                                                         dtype=torch.bfloat16)

        self.h = up(inputs["h"])
        self.w_gate, self.w_up, self.w_down = up(inputs["w_gate"]), up(inputs["w_up"]), up(inputs["w_down"])
        self.a = [up(inputs["a"].get(t)) for t in (MLP_TARGET_GATE, MLP_TARGET_UP, MLP_TARGET_DOWN)]
        self.b = [up(inputs["b"].get(t)) for t in (MLP_TARGET_GATE, MLP_TARGET_UP, MLP_TARGET_DOWN)]
        self.out = torch.empty((T, w.d_model), dtype=torch.bfloat16, device=device)
        ws = B.lrq_mlp_workspace_size(self.desc)
        self.workspace = torch.empty(ws, dtype=torch.uint8, device=device) if ws else None

    def forward(self, stream=None):
        B.lrq_mlp_forward(self.desc, self.h, self.w_gate, self.w_up, self.w_down, self.a, self.b, self.out,
                          self.workspace, stream=stream)
        return self.out
