"""GPU parity of the LoRA-adapted SwiGLU MLP (lrq_mlp_forward), through the C ABI, against the
float64 oracle: small shapes in full (ragged token counts, every adapter subset, a rank that
is not a multiple of 8), the Llama-3-8B MLP at full size on sampled rows, B = 0 equal bit for
bit to no adapters, repeated calls identical, and replay in a HIP graph.  Bars as for the
projection: relative Frobenius error <= 5e-3 (bf16 inputs, fp32 accumulation) plus the
per-row and per-element bounds."""
import numpy as np
import pytest
import torch

import oracle.mlp_oracle as mo
from oracle.lrq_oracle import rel_frobenius
from helpers import assert_parity, elem_ratio, log, row_rel_errors, sample_rows, to_np
from layer_rmsnorm_qkv_amd import binding as B
from layer_rmsnorm_qkv_amd import workloads as wl
from layer_rmsnorm_qkv_amd.device import DeviceMlp

pytestmark = pytest.mark.gpu

G, U, D = wl.MLP_TARGET_GATE, wl.MLP_TARGET_UP, wl.MLP_TARGET_DOWN
BASE = wl.get_mlp("mlp_llama3")
SMALL = {
    "t70_all_r8": BASE.replace(n_tokens=70, d_model=256, d_ff=256, lora_rank=8, lora_alpha=16.0),
    "t300_gate_down_r16": BASE.replace(n_tokens=300, d_model=512, d_ff=384, lora_targets=G | D),
    "t257_noadapt": BASE.replace(n_tokens=257, d_model=256, d_ff=512, lora_targets=0),
    "t33_up_r5": BASE.replace(n_tokens=33, d_model=256, d_ff=256, lora_rank=5, lora_alpha=10.0, lora_targets=U),
    "t1_all_r32": BASE.replace(n_tokens=1, d_model=512, d_ff=640, lora_rank=32, lora_alpha=16.0),
}


def spec_of(w):
    return mo.MlpSpec(d_model=w.d_model, d_ff=w.d_ff, lora_rank=w.lora_rank if w.lora_targets else 0,
                      lora_alpha=w.lora_alpha, lora_targets=w.lora_targets)


def errors(w, got, ref):
    return {"out": rel_frobenius(got, ref), "row": row_rel_errors(got, ref), "elem": elem_ratio(got, ref, "bf16")}


def run(w, rows=None):
    inp = wl.make_mlp_inputs(w)
    log(f"[gpu] mlp {w.name} T={w.n_tokens} d={w.d_model} F={w.d_ff} r={w.lora_rank} targets={w.lora_targets}")
    prob = DeviceMlp(w, inp)
    got = to_np(prob.forward())
    torch.cuda.synchronize()
    spec = spec_of(w)
    if rows is None:
        ref = mo.mlp_forward(spec, inp["h"], inp["w_gate"], inp["w_up"], inp["w_down"], inp["a"], inp["b"])
    else:
        got = got[rows]
        ref = mo.mlp_forward_rows(spec, rows, inp["h"], inp["w_gate"], inp["w_up"], inp["w_down"], inp["a"],
                                  inp["b"])
    return got, ref, prob, inp


@pytest.mark.parametrize("name", list(SMALL))
def test_mlp_small(name):
    w = SMALL[name]
    got, ref, _, _ = run(w)
    errs = errors(w, got, ref)
    log(f"  errors {errs}")
    assert_parity(errs, "bf16", name)


def test_mlp_llama3_full_size_sampled():
    """The Llama-3-8B MLP (8192 tokens, d 4096, F 14336, r 16 on gate, up, down), in the launch
    configuration the benchmark times, on 96 sampled rows including the first and last."""
    w = BASE
    got, ref, _, _ = run(w, rows=sample_rows(w.n_tokens, 96, seed=10))
    errs = errors(w, got, ref)
    log(f"  errors {errs}")
    assert_parity(errs, "bf16")


def test_mlp_zero_b_equals_no_adapters_bitwise():
    w = SMALL["t300_gate_down_r16"].replace(lora_targets=G | U | D)
    inp = wl.make_mlp_inputs(w)
    log("[gpu] mlp zero-B bitwise")
    zero = dict(inp, b={t: np.zeros_like(v) for t, v in inp["b"].items()})
    o1 = DeviceMlp(w, zero).forward()
    o2 = DeviceMlp(w.replace(lora_targets=0), inp).forward()
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_mlp_repeated_and_graph_replay():
    w = SMALL["t70_all_r8"]
    prob = DeviceMlp(w, wl.make_mlp_inputs(w))
    log("[gpu] mlp determinism and graph replay")
    first = prob.forward().clone()
    for _ in range(2):
        assert torch.equal(prob.forward(), first)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        prob.forward()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        prob.forward()
    for _ in range(3):
        prob.out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(prob.out, first)
        prob.forward()
        torch.cuda.synchronize()


@pytest.mark.parametrize("seed", range(8))
def test_mlp_random_shape(seed):
    """Seeded random MLPs in the kernel's range: 1-400 tokens, d a multiple of 256 up to 768,
    d_ff a multiple of 128 up to 1024, rank 1-32, any subset of gate / up / down adapted."""
    rng = np.random.default_rng(700 + seed)
    w = BASE.replace(name=f"mlp_rand{seed}", n_tokens=int(rng.integers(1, 401)),
                     d_model=256 * int(rng.integers(1, 4)), d_ff=128 * int(rng.integers(1, 9)),
                     lora_rank=int(rng.choice([1, 5, 8, 16, 24, 32])), lora_targets=int(rng.integers(0, 8)),
                     lora_alpha=float(rng.choice([8.0, 16.0, 32.0])))
    got, ref, _, _ = run(w)
    errs = errors(w, got, ref)
    log(f"  errors {errs}")
    assert_parity(errs, "bf16", w.name)
