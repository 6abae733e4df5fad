"""Seeded synthetic workloads for the fused RMSNorm -> QKV(+LoRA) -> RoPE projection.

This module only *draws inputs*. It holds none of the operator's arithmetic, so
both the CPU oracle (tests, bench baseline) and the HIP path can be fed from it
without sharing any of the computation.

The five workloads are layer shapes of the models the source pages fine-tune
("Liger-Kernel内核级优化" — Llama-3-8B + LoRA table; "Swift-All一文详解" —
LLaMA-2-7B LoRA throughput table), with synthetic values, since no weights or
datasets are used:

  tiny    fp32  T=8,      d=64,   4q/2kv x 16,  N=128,   r=4 on q,v,   alpha 8
  llama3  bf16  T=8192,   d=4096, 32q/8kv x 128, N=6144,  r=8 on q,v,   alpha 16, theta 5e5
  llama2  bf16  T=16384,  d=4096, 32 MHA x 128,  N=12288, r=64 on q,k,v, alpha 16, theta 1e4
  decode  bf16  T=64 rows at random positions in [0, 8192), llama2 shape + bias
  train   bf16  T=16384 (4 x 4096), llama3 shape, forward + backward

Conventions
-----------
* ``N(0, v)`` means mean 0 and *variance* v; ``U(+-a)`` is uniform on [-a, a].
* Every tensor comes from its own PCG64 stream ``default_rng([seed, tensor_id])``
  with ``seed = 20261202 + workload index``; values are drawn in float64 and
  rounded once to the workload dtype (round-to-nearest-even, via float32 for
  bf16).  Arrays are returned as float32 holding exactly those values, so the
  same bits reach the oracle (upcast to float64) and the GPU (cast to bf16,
  which is exact here).
* Positions are int32.  Batched sequences are contiguous, so token t of a batch
  of sequences of length S sits at position ``t mod S``.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional, Tuple

import numpy as np

TARGET_Q = 1
TARGET_K = 2
TARGET_V = 4

BASE_SEED = 20261202

# tensor ids: fixed so that adding a tensor never perturbs the others
_TID = {"x": 1, "gamma": 2, "w": 3, "bias": 4, "a_q": 5, "a_k": 6, "a_v": 7,
        "b_q": 8, "b_k": 9, "b_v": 10, "pos": 11, "dy": 12}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int
    dtype: str                  # "f32" or "bf16"
    n_tokens: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    lora_rank: int
    lora_alpha: float
    lora_targets: int           # bitmask of TARGET_*
    has_bias: bool
    rope_theta: float
    eps: float
    seq_len: int                # positions = t mod seq_len; 0 = uniform random positions
    max_position: int           # exclusive upper bound for random positions
    # value distributions
    w_var: float
    a_kind: str                 # "normal" (variance a_scale) or "uniform" (+-a_scale)
    a_scale: float
    b_var: float
    gamma_std: float
    bias_var: float
    backward: bool = False
    description: str = ""

    @property
    def n_out(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def seed(self) -> int:
        return BASE_SEED + self.index

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    def target_columns(self) -> Dict[int, Tuple[int, int]]:
        """Column range of each of q, k, v inside the [T, N] output (pure layout)."""
        D = self.head_dim
        q = self.n_q_heads * D
        kv = self.n_kv_heads * D
        return {TARGET_Q: (0, q), TARGET_K: (q, q + kv), TARGET_V: (q + kv, q + 2 * kv)}


WORKLOADS = [
    Workload("tiny", 0, "f32", 8, 64, 4, 2, 16, 4, 8.0, TARGET_Q | TARGET_V, False,
             10000.0, 1e-6, 8, 8, 1.0 / 64, "normal", 1.0 / 64, 0.1, 0.1, 0.0,
             description="tiny fp32: T=8, d=64, 4q+2kv heads x 16, r=4 on q,v, alpha 8"),
    Workload("llama3", 1, "bf16", 16 * 512, 4096, 32, 8, 128, 8, 16.0, TARGET_Q | TARGET_V, False,
             500000.0, 1e-6, 512, 512, 1.0 / 4096, "uniform", 1.0 / 64, 0.02, 0.05, 0.0,
             description="Llama-3-8B layer: 16x512 tokens, d=4096, 32q/8kv x 128, r=8 on q,v"),
    Workload("llama2", 2, "bf16", 8 * 2048, 4096, 32, 32, 128, 64, 16.0,
             TARGET_Q | TARGET_K | TARGET_V, False,
             10000.0, 1e-6, 2048, 2048, 1.0 / 4096, "uniform", 1.0 / 64, 0.02, 0.05, 0.0,
             description="LLaMA-2-7B layer: 8x2048 tokens, d=4096, 32 MHA x 128, r=64 on q,k,v"),
    Workload("decode", 3, "bf16", 64, 4096, 32, 32, 128, 64, 16.0,
             TARGET_Q | TARGET_K | TARGET_V, True,
             10000.0, 1e-6, 0, 8192, 1.0 / 4096, "uniform", 1.0 / 64, 0.02, 0.05, 0.02,
             description="decode: 64 single-token rows at random positions, LLaMA-2-7B shape + bias"),
    Workload("train", 4, "bf16", 4 * 4096, 4096, 32, 8, 128, 8, 16.0, TARGET_Q | TARGET_V, False,
             500000.0, 1e-6, 4096, 4096, 1.0 / 4096, "uniform", 1.0 / 64, 0.02, 0.05, 0.0,
             backward=True,
             description="LoRA training step: 4x4096 tokens, Llama-3-8B shape, forward + backward"),
]
BY_NAME = {w.name: w for w in WORKLOADS}


def get(name_or_index) -> Workload:
    if isinstance(name_or_index, int):
        return WORKLOADS[name_or_index]
    return BY_NAME[name_or_index]


# --------------------------------------------------------------------------- rounding of inputs

def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round to the nearest bfloat16 (ties to even), returned as float32.

    float64 -> float32 (RNE, numpy) -> bfloat16 (RNE on the bit pattern).  NaN is
    not produced by the generators and is not handled specially.
    """
    f = np.ascontiguousarray(a, dtype=np.float32)
    bits = f.view(np.uint32).astype(np.uint64)
    lsb = (bits >> np.uint64(16)) & np.uint64(1)
    bits = (bits + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)
    return bits.astype(np.uint32).view(np.float32)


def to_dtype(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "bf16":
        return round_to_bf16(a)
    raise ValueError(dtype)


# --------------------------------------------------------------------------- generators

def _rng(w: Workload, name: str, seed: Optional[int]) -> np.random.Generator:
    return np.random.default_rng([w.seed if seed is None else seed, _TID[name]])


def _normal(rng, shape, var):
    return rng.standard_normal(shape) * np.sqrt(var)


def positions(w: Workload, n_tokens: Optional[int] = None, seed: Optional[int] = None) -> np.ndarray:
    T = w.n_tokens if n_tokens is None else n_tokens
    if w.seq_len > 0:
        return (np.arange(T, dtype=np.int64) % w.seq_len).astype(np.int32)
    return _rng(w, "pos", seed).integers(0, w.max_position, size=T).astype(np.int32)


def make_inputs(w: Workload, n_tokens: Optional[int] = None, seed: Optional[int] = None,
                with_dy: Optional[bool] = None) -> Dict[str, object]:
    """Draw every input of one call of the operator for workload ``w``.

    Returns a dict with float32 arrays (values exactly representable in the
    workload dtype): ``x [T,d]``, ``gamma [d]``, ``w [N,d]``, ``bias [N]`` or
    None, ``a`` / ``b``: dicts target -> ``A_t [r,d]`` / ``B_t [N_t,r]``,
    ``positions`` int32 ``[T]`` and, for backward workloads, ``dy [T,N]``.
    """
    T = w.n_tokens if n_tokens is None else n_tokens
    d, N, r = w.d_model, w.n_out, w.lora_rank
    dt = w.dtype
    out: Dict[str, object] = {}
    out["x"] = to_dtype(_normal(_rng(w, "x", seed), (T, d), 1.0), dt)
    out["gamma"] = to_dtype(1.0 + w.gamma_std * _rng(w, "gamma", seed).standard_normal(d), dt)
    out["w"] = to_dtype(_normal(_rng(w, "w", seed), (N, d), w.w_var), dt)
    out["bias"] = (to_dtype(_normal(_rng(w, "bias", seed), (N,), w.bias_var), dt)
                   if w.has_bias else None)
    cols = w.target_columns()
    a, b = {}, {}
    for t, an, bn in ((TARGET_Q, "a_q", "b_q"), (TARGET_K, "a_k", "b_k"), (TARGET_V, "a_v", "b_v")):
        if not (w.lora_targets & t):
            continue
        rng_a = _rng(w, an, seed)
        if w.a_kind == "uniform":
            av = rng_a.uniform(-w.a_scale, w.a_scale, size=(r, d))
        else:
            av = _normal(rng_a, (r, d), w.a_scale)
        a[t] = to_dtype(av, dt)
        n_t = cols[t][1] - cols[t][0]
        b[t] = to_dtype(_normal(_rng(w, bn, seed), (n_t, r), w.b_var), dt)
    out["a"], out["b"] = a, b
    out["positions"] = positions(w, T, seed)
    if w.backward if with_dy is None else with_dy:
        out["dy"] = to_dtype(_normal(_rng(w, "dy", seed), (T, N), 1.0), dt)
    return out


# --------------------------------------------------------------------------- SwiGLU MLP workloads
#
# The LoRA-adapted SwiGLU MLP of a Llama-3-8B layer (d = 4096, intermediate 14336), fed by
# 16 x 512 tokens as the attention projection's llama3 workload; LoRA on gate, up and down
# with r = 16, alpha 32.  The MLP input is the output of the layer's second RMSNorm, so
# h ~ N(0, 1) (unit RMS); W_g, W_u ~ N(0, 1/d), W_d ~ N(0, 1/F); A ~ U(+-1/64); B ~ N(0, 0.02).

MLP_TARGET_GATE = 1
MLP_TARGET_UP = 2
MLP_TARGET_DOWN = 4

_MLP_TID = {"h": 21, "wg": 22, "wu": 23, "wd": 24, "a_g": 25, "a_u": 26, "a_d": 27, "b_g": 28, "b_u": 29,
            "b_d": 30}


@dataclasses.dataclass(frozen=True)
class MlpWorkload:
    name: str
    index: int
    n_tokens: int
    d_model: int
    d_ff: int
    lora_rank: int
    lora_alpha: float
    lora_targets: int
    a_scale: float = 1.0 / 64
    b_var: float = 0.02
    dtype: str = "bf16"
    description: str = ""

    @property
    def seed(self) -> int:
        return BASE_SEED + self.index

    def replace(self, **kw) -> "MlpWorkload":
        return dataclasses.replace(self, **kw)


MLP_WORKLOADS = [
    MlpWorkload("mlp_llama3", 10, 16 * 512, 4096, 14336, 16, 32.0,
                MLP_TARGET_GATE | MLP_TARGET_UP | MLP_TARGET_DOWN,
                description="Llama-3-8B SwiGLU MLP: 16x512 tokens, d=4096, F=14336, r=16 on gate, up, down"),
]
MLP_BY_NAME = {w.name: w for w in MLP_WORKLOADS}


def get_mlp(name: str) -> MlpWorkload:
    return MLP_BY_NAME[name]


def make_mlp_inputs(w: MlpWorkload, n_tokens: Optional[int] = None, seed: Optional[int] = None) -> Dict[str, object]:
    """Every input of one MLP call: h [T, d], w_gate / w_up [F, d], w_down [d, F], and dicts
    target -> A_t [r, d_in] / B_t [d_out, r] for the adapted projections (float32 holding
    values exactly representable in the workload dtype)."""
    T = w.n_tokens if n_tokens is None else n_tokens
    d, F, r, dt = w.d_model, w.d_ff, w.lora_rank, w.dtype

    def rng(name):
        return np.random.default_rng([w.seed if seed is None else seed, _MLP_TID[name]])

    out: Dict[str, object] = {
        "h": to_dtype(_normal(rng("h"), (T, d), 1.0), dt),
        "w_gate": to_dtype(_normal(rng("wg"), (F, d), 1.0 / d), dt),
        "w_up": to_dtype(_normal(rng("wu"), (F, d), 1.0 / d), dt),
        "w_down": to_dtype(_normal(rng("wd"), (d, F), 1.0 / F), dt),
    }
    a, b = {}, {}
    for t, an, bn, din, dout in ((MLP_TARGET_GATE, "a_g", "b_g", d, F), (MLP_TARGET_UP, "a_u", "b_u", d, F),
                                 (MLP_TARGET_DOWN, "a_d", "b_d", F, d)):
        if w.lora_targets & t:
            a[t] = to_dtype(rng(an).uniform(-w.a_scale, w.a_scale, size=(r, din)), dt)
            b[t] = to_dtype(_normal(rng(bn), (dout, r), w.b_var), dt)
    out["a"], out["b"] = a, b
    return out


# --------------------------------------------------------------------------- attention workloads
#
# The attention step over the key/value cache, with the Llama-3-8B heads (32 q, 8 kv, D 128) of
# the llama3 projection workload: a prefill batch of 16 sequences of 512 tokens (the projection
# workload's 8192 tokens) and a decode batch of 64 sequences with 4096 cached tokens each.  The
# cache is one row per token (a contiguous cache per sequence: slot = sequence * kv_len + t);
# q, k and v are N(0, 1) bf16 (values of a rotated projection output have that scale when the
# layer's weights are N(0, 1/d)).

@dataclasses.dataclass(frozen=True)
class AttnWorkload:
    name: str
    index: int
    n_seqs: int
    q_len: int            # queries per sequence
    kv_len: int           # cached keys per sequence (>= q_len)
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    causal: bool
    description: str = ""

    @property
    def seed(self) -> int:
        return BASE_SEED + self.index


ATTN_WORKLOADS = [
    AttnWorkload("attn_prefill", 20, 16, 512, 512, 32, 8, 128, True,
                 description="causal attention, 16 sequences x 512 tokens, Llama-3-8B heads (32 q / 8 kv, D 128)"),
    AttnWorkload("attn_decode", 21, 64, 1, 4096, 32, 8, 128, True,
                 description="decode attention, 64 sequences x 1 query over 4096 cached tokens, Llama-3-8B heads"),
]
ATTN_BY_NAME = {w.name: w for w in ATTN_WORKLOADS}


def get_attn(name: str) -> AttnWorkload:
    return ATTN_BY_NAME[name]


def make_attn_inputs_device(w: AttnWorkload, device: str = "cuda") -> Dict[str, object]:
    """Seeded device tensors of one attention call: q [S*q_len, Hq*D], k_cache / v_cache
    [S*kv_len, Hkv*D] bf16 N(0, 1) (drawn on the device with torch's seeded generator: the cache
    of the decode workload is 0.5 GB per tensor), q_indptr, kv_indptr and the slot list (int32)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(w.seed)
    D = w.head_dim
    nq, nk = w.n_seqs * w.q_len, w.n_seqs * w.kv_len
    q = torch.randn((nq, w.n_q_heads * D), generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
    k = torch.randn((nk, w.n_kv_heads * D), generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
    v = torch.randn((nk, w.n_kv_heads * D), generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
    q_ind = torch.arange(0, nq + 1, w.q_len, dtype=torch.int32, device=device)
    kv_ind = torch.arange(0, nk + 1, w.kv_len, dtype=torch.int32, device=device)
    slots = torch.arange(nk, dtype=torch.int32, device=device)
    return dict(q=q, k_cache=k, v_cache=v, q_indptr=q_ind, kv_indptr=kv_ind, kv_slots=slots)
