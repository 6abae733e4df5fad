"""Seeded random shapes through the C ABI against the oracle: token counts with ragged tails,
model widths, head counts and group sizes, head sizes, ranks, target subsets, bias, rotary
bases and positions (negative ones included), for every forward family that covers the shape
and for the tiled and generic backward.  Each case is small enough for the oracle to finish in
about a second; the bars are the ones of the other parity tests."""
import numpy as np
import pytest

import oracle.lrq_oracle as o
from helpers import (assert_parity, elem_ratio, forward_errors, log, oracle_forward, row_rel_errors, spec_of,
                     to_np)
from layer_rmsnorm_qkv_amd import binding as B
from layer_rmsnorm_qkv_amd import workloads as wl
from layer_rmsnorm_qkv_amd.device import DeviceProblem, desc_for

pytestmark = pytest.mark.gpu

L3 = wl.get("llama3")
FWD_VARIANTS = {"auto": B.LRQ_VARIANT_AUTO, "generic": B.LRQ_VARIANT_GENERIC, "tiled": B.LRQ_VARIANT_TILED,
                "decode": B.LRQ_VARIANT_DECODE}
BWD_VARIANTS = {"generic": B.LRQ_VARIANT_GENERIC, "tiled": B.LRQ_VARIANT_TILED}


def random_case(seed: int, backward: bool = False):
    """A bf16 workload and its seeded inputs; a quarter of the cases get negative positions."""
    rng = np.random.default_rng(1000 + seed)
    # mostly shapes the MFMA families cover (head size 128, even head counts), some that only
    # the generic family does; half the cases in the decode family's row range
    D = int(rng.choice([64, 128, 128, 128]))
    hkv = int(rng.choice([1, 2, 2, 4]))
    hq = hkv * int(rng.choice([1, 2, 4]))
    d = int(rng.choice([256, 512, 768]))
    T = int(rng.integers(1, 257)) if rng.random() < 0.5 else int(rng.integers(257, 520))
    targets = int(rng.integers(0, 8))
    r = int(rng.choice([1, 5, 8, 16, 24, 32, 64]))
    bias = bool(rng.integers(0, 2))
    seq_len = int(rng.choice([0, 64, 512]))
    w = L3.replace(name=f"rand{seed}", n_tokens=T, d_model=d, n_q_heads=hq, n_kv_heads=hkv, head_dim=D,
                   lora_rank=r, lora_targets=targets, lora_alpha=float(rng.choice([8.0, 16.0, 32.0])),
                   has_bias=bias, bias_var=0.02, rope_theta=float(rng.choice([1e4, 5e5])), seq_len=seq_len,
                   max_position=int(rng.choice([4096, 1 << 20])), w_var=1.0 / d, backward=backward)
    inp = wl.make_inputs(w, seed=seed, with_dy=backward)
    if rng.random() < 0.25:
        pos = np.asarray(inp["positions"], dtype=np.int64)
        neg = rng.random(T) < 0.5
        inp["positions"] = np.where(neg, -rng.integers(1, 100000, size=T), pos).astype(np.int32)
    return w, inp


@pytest.mark.parametrize("variant", list(FWD_VARIANTS))
@pytest.mark.parametrize("seed", range(16))
def test_forward_random_shape(seed, variant):
    import torch
    w, inp = random_case(seed)
    desc = desc_for(w, variant=FWD_VARIANTS[variant])
    if B.lrq_select_variant(desc) < 0:
        pytest.skip(f"variant {variant} does not cover this shape ({B.lrq_last_error()})")
    log(f"[gpu] random forward seed={seed} T={w.n_tokens} d={w.d_model} heads={w.n_q_heads}/{w.n_kv_heads}x"
        f"{w.head_dim} r={w.lora_rank} targets={w.lora_targets} bias={w.has_bias} variant={variant}")
    prob = DeviceProblem(w, inp, variant=FWD_VARIANTS[variant])
    got = to_np(prob.forward())
    torch.cuda.synchronize()
    errs = forward_errors(w, got, oracle_forward(w, inp))
    log(f"  errors {errs}")
    assert_parity(errs, "bf16")


@pytest.mark.parametrize("variant", list(BWD_VARIANTS))
@pytest.mark.parametrize("seed", range(8))
def test_backward_random_shape(seed, variant):
    import torch
    w, inp = random_case(100 + seed, backward=True)
    desc = desc_for(w, variant=BWD_VARIANTS[variant])
    if B.lrq_select_variant(desc, True) < 0:
        pytest.skip(f"backward variant {variant} does not cover this shape ({B.lrq_last_error()})")
    log(f"[gpu] random backward seed={seed} T={w.n_tokens} d={w.d_model} heads={w.n_q_heads}/{w.n_kv_heads}x"
        f"{w.head_dim} r={w.lora_rank} targets={w.lora_targets} bias={w.has_bias} variant={variant}")
    prob = DeviceProblem(w, inp, variant=BWD_VARIANTS[variant], backward=True)
    # the forward's output from the family that covers the shape (the tiled backward also
    # takes head sizes its forward does not)
    y = DeviceProblem(w, inp).forward()
    dx, da, db = prob.backward(y=y)
    torch.cuda.synchronize()
    rdx, rda, rdb = o.backward(spec_of(w), inp["x"], inp["gamma"], inp["w"], inp["bias"], inp["a"], inp["b"],
                               inp["positions"], inp["dy"])
    got_dx = to_np(dx)
    errs = {"dx": o.rel_frobenius(got_dx, rdx), "dx_row": row_rel_errors(got_dx, rdx),
            "dx_elem": elem_ratio(got_dx, rdx, w.dtype)}
    for i, t in enumerate((wl.TARGET_Q, wl.TARGET_K, wl.TARGET_V)):
        if w.lora_targets & t:
            ga, gb = to_np(da[i]), to_np(db[i])
            errs[f"dA{i}"] = o.rel_frobenius(ga, rda[t])
            errs[f"dB{i}"] = o.rel_frobenius(gb, rdb[t])
            errs[f"dA{i}_elem"] = elem_ratio(ga, rda[t], w.dtype, scale="tensor")
            errs[f"dB{i}_elem"] = elem_ratio(gb, rdb[t], w.dtype, scale="tensor")
    log(f"  errors {errs}")
    assert_parity(errs, "bf16")
