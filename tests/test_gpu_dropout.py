"""GPU parity of LoRA dropout (forward and backward, both families), through the C ABI,
against the oracle's Philox4x32-10 masks.

Two kinds of check:
  * parity on LoRA-heavy inputs (B with unit variance, so that the adapters' term is as large
    as the frozen projection's and one wrong keep bit moves the result far past the bar);
  * exact mask checks: with W = 0 and selection matrices as the adapters, the zero / non-zero
    pattern of the output (forward), of dA_t and of dx (backward) is the keep mask itself, which
    must equal the oracle's bit for bit (an integer decision taken in the same precision: the
    rate is the float32 value that the descriptor carries)."""
import numpy as np
import pytest

import oracle.lrq_oracle as o
from helpers import (assert_parity, elem_ratio, log, lora_bound_dx, lora_bound_forward, row_rel_errors,
                     sample_rows, spec_of, to_np)
from layer_rmsnorm_qkv_amd import binding as B
from layer_rmsnorm_qkv_amd import workloads as wl
from layer_rmsnorm_qkv_amd.device import DeviceProblem, desc_for

pytestmark = pytest.mark.gpu

TQ, TK, TV = wl.TARGET_Q, wl.TARGET_K, wl.TARGET_V
TINY, TRAIN = wl.get("tiny"), wl.get("train")
VARIANTS = {"generic": B.LRQ_VARIANT_GENERIC, "tiled": B.LRQ_VARIANT_TILED}

CASES = {
    "f32_t37_allt": TINY.replace(n_tokens=37, d_model=96, lora_targets=TQ | TK | TV, b_var=1.0, backward=True),
    "bf16_t300_qv_r16": TRAIN.replace(n_tokens=300, d_model=512, n_q_heads=4, n_kv_heads=2, lora_rank=16,
                                      b_var=1.0),
    "bf16_t513_allt_r64_bias": wl.get("decode").replace(n_tokens=513, d_model=768, n_q_heads=4, n_kv_heads=4,
                                                        lora_rank=64, b_var=0.25, backward=True),
    "bf16_t200_r5_k": TRAIN.replace(n_tokens=200, d_model=512, n_q_heads=4, n_kv_heads=2, lora_rank=5,
                                    lora_targets=TK, b_var=1.0),
}
RATES = [0.05, 0.5]


def p32(p):
    return float(np.float32(p))


def dropout_of(p, seed, offset):
    return o.Dropout(p32(p), seed, offset)


def problem(w, inp, variant, p, seed, offset, backward=False, skip=True):
    drop = (p, seed, offset)
    desc = desc_for(w, variant=variant, dropout=drop)
    if B.lrq_select_variant(desc, False) < 0 or (backward and B.lrq_select_variant(desc, True) < 0):
        if skip:
            pytest.skip(f"variant {variant} does not cover this shape")
        raise AssertionError("variant must cover this shape")
    return DeviceProblem(w, inp, variant=variant, backward=backward, dropout=drop)


@pytest.mark.parametrize("p", RATES)
@pytest.mark.parametrize("variant", list(VARIANTS))
@pytest.mark.parametrize("name", list(CASES))
def test_dropout_forward(name, variant, p):
    import torch
    w = CASES[name]
    inp = wl.make_inputs(w)
    seed, offset = 0x1234_5678_9ABC + w.index, 17
    prob = problem(w, inp, VARIANTS[variant], p, seed, offset)
    log(f"[gpu] dropout forward {name} variant={variant} p={p}")
    got = to_np(prob.forward())
    torch.cuda.synchronize()
    drop = dropout_of(p, seed, offset)
    ref = o.forward(spec_of(w), inp["x"], inp["gamma"], inp["w"], inp["bias"], inp["a"], inp["b"],
                    inp["positions"], dropout=drop)
    errs = {"out": o.rel_frobenius(got, ref), "out_row": row_rel_errors(got, ref),
            "out_elem": elem_ratio(got, ref, w.dtype, lora=lora_bound_forward(w, inp, drop))}
    log(f"  errors {errs}")
    assert_parity(errs, w.dtype)


@pytest.mark.parametrize("p", RATES)
@pytest.mark.parametrize("variant", list(VARIANTS))
@pytest.mark.parametrize("name", list(CASES))
def test_dropout_backward(name, variant, p):
    import torch
    w = CASES[name]
    inp = wl.make_inputs(w, with_dy=True)
    seed, offset = 99 + w.index, 3
    prob = problem(w, inp, VARIANTS[variant], p, seed, offset, backward=True)
    log(f"[gpu] dropout backward {name} variant={variant} p={p}")
    prob.forward()
    dx, da, db = prob.backward()
    torch.cuda.synchronize()
    drop = dropout_of(p, seed, offset)
    rdx, rda, rdb = o.backward(spec_of(w), inp["x"], inp["gamma"], inp["w"], inp["bias"], inp["a"], inp["b"],
                               inp["positions"], inp["dy"], dropout=drop)
    got_dx = to_np(dx)
    errs = {"dx": o.rel_frobenius(got_dx, rdx), "dx_row": row_rel_errors(got_dx, rdx),
            "dx_elem": elem_ratio(got_dx, rdx, w.dtype, lora=lora_bound_dx(w, inp, drop))}
    for i, t in enumerate((TQ, TK, TV)):
        if w.lora_targets & t:
            ga, gb = to_np(da[i]), to_np(db[i])
            errs[f"dA{i}"] = o.rel_frobenius(ga, rda[t])
            errs[f"dB{i}"] = o.rel_frobenius(gb, rdb[t])
            errs[f"dA{i}_elem"] = elem_ratio(ga, rda[t], w.dtype, scale="tensor")
            errs[f"dB{i}_elem"] = elem_ratio(gb, rdb[t], w.dtype, scale="tensor")
    log(f"  errors {errs}")
    assert_parity(errs, w.dtype)


@pytest.mark.parametrize("variant", list(VARIANTS))
@pytest.mark.parametrize("seed", range(6))
def test_dropout_random_shape(seed, variant):
    """Seeded random layers (the generator of the random-shape sweep) at a random rate, seed and
    offset: forward output, then dx, dA and dB, against the oracle with the same masks."""
    import torch
    from test_gpu_random_shapes import random_case
    w, inp = random_case(400 + seed, backward=True)
    rng = np.random.default_rng(900 + seed)
    p = float(rng.choice([0.05, 0.3, 0.7]))
    dseed, offset = int(rng.integers(0, 1 << 62)), int(rng.integers(0, 1 << 20))
    prob = problem(w, inp, VARIANTS[variant], p, dseed, offset, backward=True)
    log(f"[gpu] dropout random seed={seed} T={w.n_tokens} d={w.d_model} heads={w.n_q_heads}/{w.n_kv_heads}x"
        f"{w.head_dim} r={w.lora_rank} targets={w.lora_targets} p={p} variant={variant}")
    got = to_np(prob.forward())
    dx, da, db = prob.backward()
    torch.cuda.synchronize()
    drop = dropout_of(p, dseed, offset)
    args = (spec_of(w), inp["x"], inp["gamma"], inp["w"], inp["bias"], inp["a"], inp["b"], inp["positions"])
    ref = o.forward(*args, dropout=drop)
    rdx, rda, rdb = o.backward(*args, inp["dy"], dropout=drop)
    gdx = to_np(dx)
    errs = {"out": o.rel_frobenius(got, ref), "out_row": row_rel_errors(got, ref),
            "out_elem": elem_ratio(got, ref, w.dtype, lora=lora_bound_forward(w, inp, drop)),
            "dx": o.rel_frobenius(gdx, rdx), "dx_row": row_rel_errors(gdx, rdx),
            "dx_elem": elem_ratio(gdx, rdx, w.dtype, lora=lora_bound_dx(w, inp, drop))}
    for i, t in enumerate((TQ, TK, TV)):
        if w.lora_targets & t:
            ga, gb = to_np(da[i]), to_np(db[i])
            errs[f"dA{i}"] = o.rel_frobenius(ga, rda[t])
            errs[f"dB{i}"] = o.rel_frobenius(gb, rdb[t])
            errs[f"dA{i}_elem"] = elem_ratio(ga, rda[t], w.dtype, scale="tensor")
            errs[f"dB{i}_elem"] = elem_ratio(gb, rdb[t], w.dtype, scale="tensor")
    log(f"  errors {errs}")
    assert_parity(errs, w.dtype)


# ---------------------------------------------------------------- exact masks
MASK_W = TRAIN.replace(n_tokens=300, d_model=512, n_q_heads=2, n_kv_heads=2, lora_rank=64,
                       lora_targets=TQ | TK | TV, has_bias=False, gamma_std=0.0)


def selection_inputs(w, j0, dtype_np=np.float32):
    """W = 0, gamma = 1; A_t selects features j0 .. j0 + 63 (rank k -> feature j0 + k) and B_t
    copies rank k to the target's column k (head 0, first half)."""
    inp = wl.make_inputs(w, with_dy=True)
    inp["w"] = np.zeros_like(inp["w"])
    inp["gamma"] = np.ones_like(inp["gamma"])
    cols = w.target_columns()
    for t in (TQ, TK, TV):
        a = np.zeros((w.lora_rank, w.d_model), dtype_np)
        a[np.arange(64), j0 + np.arange(64)] = 1.0
        n_t = cols[t][1] - cols[t][0]
        b = np.zeros((n_t, w.lora_rank), dtype_np)
        b[np.arange(64), np.arange(64)] = 1.0
        inp["a"][t], inp["b"][t] = a, b
    return inp


@pytest.mark.parametrize("dtype,variant", [("f32", "generic"), ("bf16", "generic"), ("bf16", "tiled")])
def test_dropout_forward_masks_exact(dtype, variant):
    """Kept features give a non-zero output column, dropped ones exactly 0 (rotated q and k:
    the pair (i, i + 64) is non-zero iff feature i is kept)."""
    import torch
    w = MASK_W.replace(dtype=dtype)
    p, seed, offset = 0.3, 0xDEADBEEF_0BADF00D, 5
    keep_ref = {i: o.dropout_keep(w.n_tokens, w.d_model, i, p32(p), seed, offset) for i in range(3)}
    cols = w.target_columns()
    for j0 in range(0, w.d_model, 64):
        inp = selection_inputs(w, j0)
        prob = problem(w, inp, VARIANTS[variant], p, seed, offset, skip=False)
        log(f"[gpu] dropout mask forward {dtype} {variant} j0={j0}")
        out = to_np(prob.forward())
        torch.cuda.synchronize()
        for i, t in enumerate((TQ, TK, TV)):
            c = cols[t][0]
            nz = (out[:, c:c + 64] != 0) | (out[:, c + 64:c + 128] != 0) if t != TV else out[:, c:c + 64] != 0
            want = keep_ref[i][:, j0:j0 + 64]
            bad = int(np.count_nonzero(nz != want))
            assert bad == 0, f"target {i}, features {j0}..{j0 + 63}: {bad} keep bits differ"


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_dropout_backward_masks_exact(variant):
    """dy on one row only and W = 0: for each single target, the non-zero pattern of dA (the
    adapter's input) is the row's keep mask.  The tiled family takes the RMSNorm backward's row
    term from y, so with y = 0 that row's dx is inv * gamma * dh, whose non-zero pattern (the
    masked dh term of the main kernel's epilogue) is the keep mask too; the generic family
    forms the row term from dh itself, so there only the rows without dy are checked (zero)."""
    import torch
    p, seed, offset = 0.3, 77, 0xFFFFFFFF
    for t_i, t in enumerate((TQ, TK, TV)):
        w = MASK_W.replace(lora_targets=t, lora_rank=16, b_var=1.0)
        keep = o.dropout_keep(w.n_tokens, w.d_model, t_i, p32(p), seed, offset)
        inp = wl.make_inputs(w, with_dy=True)
        inp["w"] = np.zeros_like(inp["w"])
        for rho in (0, 255, 256, w.n_tokens - 1):
            dy = np.zeros_like(inp["dy"])
            dy[rho] = inp["dy"][rho]
            inp2 = dict(inp, dy=dy)
            prob = problem(w, inp2, VARIANTS[variant], p, seed, offset, backward=True, skip=False)
            log(f"[gpu] dropout mask backward {variant} target={t_i} row={rho}")
            y0 = torch.zeros_like(prob.out)
            dx, da, db = prob.backward(y=y0)
            torch.cuda.synchronize()
            ga, gdx = to_np(da[t_i]), to_np(dx)
            assert not np.any(np.delete(gdx, rho, axis=0)), "dx of rows without dy must be 0"
            if variant == "tiled":
                assert np.array_equal(gdx[rho] != 0, keep[rho]), f"dx row {rho}: keep bits differ"
            assert np.array_equal(np.any(ga != 0, axis=0), keep[rho]), f"dA row {rho}: keep bits differ"


def test_dropout_zero_rate_and_seeds():
    """Rate 0 is bit-identical to no dropout whatever the seed; a call is deterministic; another
    seed or offset changes the output."""
    import torch
    w = CASES["bf16_t300_qv_r16"]
    inp = wl.make_inputs(w)

    def run(drop, variant=B.LRQ_VARIANT_AUTO):
        prob = DeviceProblem(w, inp, variant=variant, dropout=drop)
        out = prob.forward().clone()
        torch.cuda.synchronize()
        return out

    for variant in VARIANTS.values():
        base = run(None, variant)
        assert torch.equal(run((0.0, 12345, 9), variant), base)
        a1, a2 = run((0.1, 7, 1), variant), run((0.1, 7, 1), variant)
        assert torch.equal(a1, a2)
        assert not torch.equal(a1, run((0.1, 8, 1), variant))
        assert not torch.equal(a1, run((0.1, 7, 2), variant))
        assert not torch.equal(a1, base)


def test_dropout_train_full_size():
    """The training workload at full size (16384 tokens, tiled family) with the pages' rate
    0.05: forward and dx on sampled rows, dA / dB in full."""
    import torch
    w = TRAIN
    inp = wl.make_inputs(w, with_dy=True)
    p, seed, offset = 0.05, 2024, 11
    prob = problem(w, inp, B.LRQ_VARIANT_TILED, p, seed, offset, backward=True, skip=False)
    log(f"[gpu] dropout full-size train T={w.n_tokens}")
    prob.prepare()
    out = prob.forward()
    dx, da, db = prob.backward()
    torch.cuda.synchronize()
    rows = sample_rows(w.n_tokens, 192, seed=5)
    drop = dropout_of(p, seed, offset)
    spec = spec_of(w)
    ref_out = o.forward_rows(spec, rows, inp["x"], inp["gamma"], inp["w"], inp["bias"], inp["a"], inp["b"],
                             inp["positions"], dropout=drop)
    got_out = to_np(out)[rows]
    rdx, rda, rdb = o.backward(spec, inp["x"], inp["gamma"], inp["w"], inp["bias"], inp["a"], inp["b"],
                               inp["positions"], inp["dy"], dx_rows=rows, dropout=drop)
    got_dx = to_np(dx)[rows]
    errs = {"out": o.rel_frobenius(got_out, ref_out), "out_row": row_rel_errors(got_out, ref_out),
            "out_elem": elem_ratio(got_out, ref_out, "bf16", lora=lora_bound_forward(w, inp, drop, rows)),
            "dx": o.rel_frobenius(got_dx, rdx), "dx_row": row_rel_errors(got_dx, rdx),
            "dx_elem": elem_ratio(got_dx, rdx, "bf16", lora=lora_bound_dx(w, inp, drop, rows))}
    for i, t in enumerate((TQ, TK, TV)):
        if w.lora_targets & t:
            errs[f"dA{i}"] = o.rel_frobenius(to_np(da[i]), rda[t])
            errs[f"dB{i}"] = o.rel_frobenius(to_np(db[i]), rdb[t])
    log(f"  errors {errs}")
    assert_parity(errs, "bf16")
