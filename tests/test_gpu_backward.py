"""GPU parity of the backward (dx, dA_t, dB_t), through the C ABI, against the oracle.

dx is compared in full on small cases and on sampled rows at full size; dA and dB are
sums over every token and are always compared in full."""
import numpy as np
import pytest

import oracle.lrq_oracle as o
from helpers import TOL, assert_parity, elem_ratio, log, row_rel_errors, sample_rows, spec_of, to_np
from layer_rmsnorm_qkv_amd import binding as B
from layer_rmsnorm_qkv_amd import workloads as wl
from layer_rmsnorm_qkv_amd.device import DeviceProblem, desc_for

pytestmark = pytest.mark.gpu

TQ, TK, TV = wl.TARGET_Q, wl.TARGET_K, wl.TARGET_V
TINY = wl.get("tiny")
TRAIN = wl.get("train")
VARIANTS = {"generic": B.LRQ_VARIANT_GENERIC, "tiled": B.LRQ_VARIANT_TILED}

CASES = {
    "tiny_f32": TINY,
    "f32_t37_bias_allt": TINY.replace(n_tokens=37, d_model=96, has_bias=True, bias_var=0.02,
                                      lora_targets=TQ | TK | TV, seq_len=0, max_position=5000),
    "f32_t5_kv4": TINY.replace(n_tokens=5, n_q_heads=4, n_kv_heads=4, head_dim=8, lora_targets=TK),
    "bf16_train_small": TRAIN.replace(n_tokens=300, d_model=512, n_q_heads=8, n_kv_heads=2),
    "bf16_allt_bias": wl.get("decode").replace(n_tokens=129, d_model=384, n_q_heads=3, n_kv_heads=3,
                                               lora_rank=16),
    # shapes the MFMA family covers: ragged token counts, rank above one 32-block, bias
    "bf16_allt_bias_t300_r64": wl.get("decode").replace(n_tokens=300, d_model=512, n_q_heads=4, n_kv_heads=4,
                                                        lora_rank=64),
    "bf16_gqa_t513_r24": TRAIN.replace(n_tokens=513, d_model=768, n_q_heads=4, n_kv_heads=2, lora_rank=24,
                                       lora_targets=TQ | TK, seq_len=0, max_position=9000),
    "bf16_noadapt_t77": TRAIN.replace(n_tokens=77, d_model=256, n_q_heads=2, n_kv_heads=2, lora_targets=0),
    # a rank that is not a multiple of 8 (ragged rank columns in every LoRA pass)
    "bf16_t200_r5_v": TRAIN.replace(n_tokens=200, d_model=512, n_q_heads=4, n_kv_heads=2, lora_rank=5,
                                    lora_targets=TV),
}


def run_backward(w, variant, dx_rows=None, negative_positions=False, fwd_variant=None):
    import torch
    inp = wl.make_inputs(w, with_dy=True)
    if negative_positions:
        # half of the rows at negative positions, down to -9000 (positions are not range-checked)
        pos = np.asarray(inp["positions"], dtype=np.int64)
        rng = np.random.default_rng(7)
        neg = rng.random(pos.shape[0]) < 0.5
        inp["positions"] = np.where(neg, -rng.integers(1, 9001, size=pos.shape[0]), pos).astype(np.int32)
    desc = desc_for(w, variant=variant)
    if B.lrq_select_variant(desc, True) < 0:
        pytest.skip(f"backward variant {variant} does not cover this shape")
    log(f"[gpu] backward {w.name} T={w.n_tokens} d={w.d_model} N={w.n_out} variant={variant}")
    prob = DeviceProblem(w, inp, variant=variant, backward=True)
    if fwd_variant is None:
        prob.forward()
        dx, da, db = prob.backward()
    else:
        # the forward output from another family (one that covers the shape)
        y = DeviceProblem(w, inp, variant=fwd_variant).forward()
        dx, da, db = prob.backward(y=y)
    torch.cuda.synchronize()
    spec = spec_of(w)
    rdx, rda, rdb = o.backward(spec, inp["x"], inp["gamma"], inp["w"], inp["bias"], inp["a"], inp["b"],
                               inp["positions"], inp["dy"], dx_rows=dx_rows)
    got_dx = to_np(dx) if dx_rows is None else to_np(dx)[dx_rows]
    errs = {"dx": o.rel_frobenius(got_dx, rdx), "dx_row": row_rel_errors(got_dx, rdx),
            "dx_elem": elem_ratio(got_dx, rdx, w.dtype)}
    for i, t in enumerate((TQ, TK, TV)):
        if w.lora_targets & t:
            ga, gb = to_np(da[i]), to_np(db[i])
            errs[f"dA{i}"] = o.rel_frobenius(ga, rda[t])
            errs[f"dB{i}"] = o.rel_frobenius(gb, rdb[t])
            # sums over every token: element bound against the RMS of the whole gradient
            errs[f"dA{i}_elem"] = elem_ratio(ga, rda[t], w.dtype, scale="tensor")
            errs[f"dB{i}_elem"] = elem_ratio(gb, rdb[t], w.dtype, scale="tensor")
    log(f"  errors {errs}")
    return errs


@pytest.mark.parametrize("variant", list(VARIANTS))
@pytest.mark.parametrize("name", list(CASES))
def test_backward_small(name, variant):
    w = CASES[name]
    errs = run_backward(w, VARIANTS[variant])
    assert_parity(errs, w.dtype)


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_backward_train_full_size(variant):
    """The training workload at full size (16384 tokens); dx on sampled rows."""
    if variant == "generic":
        pytest.skip("the generic family is too slow for 16384 tokens; covered on smaller cases")
    w = TRAIN
    errs = run_backward(w, VARIANTS[variant], dx_rows=sample_rows(w.n_tokens, 192, seed=4))
    assert_parity(errs, "bf16")


def test_backward_zero_tokens_zeroes_lora_grads():
    import torch
    w = CASES["bf16_train_small"]
    prob = DeviceProblem(w, wl.make_inputs(w, with_dy=True), backward=True)
    for t in prob.da + prob.db:
        if t is not None:
            t.fill_(7.0)
    d0 = desc_for(w, n_tokens=0)
    B.lrq_backward(d0, prob.x, prob.gamma, prob.w_qkv, prob.bias, prob.a, prob.b, prob.positions, prob.out,
                   prob.dy, prob.dx, prob.da, prob.db, prob.workspace)
    torch.cuda.synchronize()
    for t in prob.da + prob.db:
        if t is not None:
            assert torch.count_nonzero(t).item() == 0


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_backward_zero_tokens_null_inputs(variant):
    """With T == 0 the header lets x, gamma, w_qkv, positions, y, dy and dx be NULL; the LoRA
    gradients are still set to zero, and nothing reads the NULL arrays (the tiled family's
    gradient reduction used to read gamma even with no token chunks)."""
    import torch
    w = CASES["bf16_train_small"]
    prob = DeviceProblem(w, wl.make_inputs(w, with_dy=True), backward=True)
    d0 = desc_for(w, n_tokens=0, variant=VARIANTS[variant])
    if B.lrq_select_variant(d0, True) < 0:
        pytest.skip(f"backward variant {variant} does not cover this shape")
    log(f"[gpu] backward T=0 with NULL inputs variant={variant}")
    for t in prob.da + prob.db:
        if t is not None:
            t.fill_(7.0)
    ws = B.lrq_workspace_size(d0, True)
    work = torch.empty(max(ws, 1), dtype=torch.uint8, device="cuda") if ws else None
    B.lrq_backward(d0, None, None, None, None, prob.a, prob.b, None, None, None, None, prob.da, prob.db, work)
    torch.cuda.synchronize()
    for t in prob.da + prob.db:
        if t is not None:
            assert torch.count_nonzero(t).item() == 0


HEADS = {
    # the tiled family's rows pass at other head sizes: its 16-byte path (64, 256; 8 frequencies
    # per lane) and its one-pair-per-lane path (96), with bias and rotation of q and k
    "bf16_head64": TRAIN.replace(n_tokens=70, d_model=256, head_dim=64, n_q_heads=4, n_kv_heads=2, has_bias=True,
                                 bias_var=0.02, lora_targets=TQ | TV, seq_len=0, max_position=9000),
    "bf16_head96": TRAIN.replace(n_tokens=70, d_model=256, head_dim=96, n_q_heads=2, n_kv_heads=2, has_bias=True,
                                 bias_var=0.02, lora_targets=TQ | TV, seq_len=0, max_position=9000),
    "bf16_head256": TRAIN.replace(n_tokens=70, d_model=256, head_dim=256, n_q_heads=2, n_kv_heads=1, has_bias=True,
                                  bias_var=0.02, lora_targets=TQ | TK, seq_len=0, max_position=9000),
}


@pytest.mark.parametrize("name", list(HEADS))
def test_backward_tiled_head_sizes(name):
    """The tiled backward at head sizes other than 128 (the forward's output comes from the
    generic family, the one that covers them)."""
    w = HEADS[name]
    errs = run_backward(w, B.LRQ_VARIANT_TILED, fwd_variant=B.LRQ_VARIANT_GENERIC)
    assert_parity(errs, w.dtype)


LIMITS = {
    # the largest rank on every target with d = 8192 (a 130-step main product) and a ragged tile
    "bf16_d8192_r64_allt": TRAIN.replace(n_tokens=300, d_model=8192, n_q_heads=4, n_kv_heads=2, lora_rank=64,
                                         lora_targets=TQ | TK | TV),
    # the generic family's largest head (256), float32
    "f32_head256_r64": TINY.replace(n_tokens=12, d_model=64, head_dim=256, n_q_heads=2, n_kv_heads=1,
                                    lora_rank=64, lora_targets=TQ | TK | TV),
}


@pytest.mark.parametrize("variant", list(VARIANTS))
@pytest.mark.parametrize("name", list(LIMITS))
def test_backward_at_size_limits(name, variant):
    w = LIMITS[name]
    errs = run_backward(w, VARIANTS[variant])
    assert_parity(errs, w.dtype)


def test_forward_and_backward_replay_in_a_hip_graph():
    """A forward and a backward call captured in one HIP graph (the calls allocate nothing,
    clear nothing with memset and never synchronise) replay to the eager results, with eager
    calls and synchronisations between the replays."""
    import torch
    w = CASES["bf16_gqa_t513_r24"]
    inp = wl.make_inputs(w, with_dy=True)
    if B.lrq_select_variant(desc_for(w, variant=B.LRQ_VARIANT_TILED), True) < 0:
        pytest.skip("tiled family does not cover this shape")
    log("[gpu] graph capture and replay (tiled forward + backward)")
    prob = DeviceProblem(w, inp, variant=B.LRQ_VARIANT_TILED, backward=True)
    y = prob.forward().clone()
    dx, da, db = prob.backward(y=y)
    ref = [dx.clone()] + [t.clone() for t in da + db if t is not None]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        prob.forward()
        prob.backward(y=y)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        prob.forward()
        prob.backward(y=y)
    for _ in range(3):
        prob.out.zero_()
        prob.dx.zero_()
        graph.replay()
        torch.cuda.synchronize()
        got = [prob.dx] + [t for t in prob.da + prob.db if t is not None]
        assert torch.equal(prob.out, y)
        assert all(torch.equal(g, r) for g, r in zip(got, ref))
        prob.forward()
        torch.cuda.synchronize()


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_backward_negative_positions(variant):
    """The inverse rotation of the backward at negative positions, as in the oracle."""
    errs = run_backward(CASES["bf16_train_small"], VARIANTS[variant], negative_positions=True)
    assert_parity(errs, "bf16")
