"""GPU parity of the QLoRA base (W_qkv as NF4 blocks), through the C ABI, against the NF4
oracle: the device quantiser byte for byte (an integer decision taken in float32 on both sides),
then forward and backward of every family that takes NF4 weights, per call and prepared."""
import numpy as np
import pytest

import oracle.lrq_oracle as o
import oracle.qlora_oracle as q
from helpers import assert_parity, elem_ratio, log, row_rel_errors, sample_rows, spec_of, to_np
from layer_rmsnorm_qkv_amd import binding as B
from layer_rmsnorm_qkv_amd import workloads as wl
from layer_rmsnorm_qkv_amd.device import DeviceProblem, desc_for

pytestmark = pytest.mark.gpu

TQ, TK, TV = wl.TARGET_Q, wl.TARGET_K, wl.TARGET_V
TRAIN = wl.get("train")
VARIANTS = {"generic": B.LRQ_VARIANT_GENERIC, "tiled": B.LRQ_VARIANT_TILED, "decode": B.LRQ_VARIANT_DECODE}

CASES = {
    "f32_t37_allt_bias": wl.get("tiny").replace(n_tokens=37, d_model=128, lora_targets=TQ | TK | TV,
                                                has_bias=True, bias_var=0.02, backward=True),
    "bf16_t300_qv_r16": TRAIN.replace(n_tokens=300, d_model=512, n_q_heads=4, n_kv_heads=2, lora_rank=16),
    "bf16_t513_allt_r64_bias": wl.get("decode").replace(n_tokens=513, d_model=768, n_q_heads=4, n_kv_heads=4,
                                                        lora_rank=64, backward=True),
    "bf16_t64_decode_shape": wl.get("decode").replace(n_tokens=64, d_model=1024, n_q_heads=8, n_kv_heads=8,
                                                      backward=True),
}


def oracle_nf4(inp):
    return q.quantize(np.asarray(inp["w"], np.float32))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quantize_matches_oracle_bytes(dtype):
    """The device quantiser's buffer equals the oracle's, byte for byte: random weights, a block
    much larger than its neighbours, an all-zero block and (float32) the exact midpoints."""
    import torch
    w = CASES["bf16_t300_qv_r16"].replace(dtype=dtype)
    inp = wl.make_inputs(w)
    wq = np.array(inp["w"], np.float32)
    wq[3, 64:128] *= 50.0
    wq[5, :64] = 0.0
    if dtype == "f32":
        lv = q.NF4_LEVELS.astype(np.float32)
        wq[7, :15] = (lv[:-1] + lv[1:]) * np.float32(0.5)
        wq[7, 15] = 1.0
        wq[7, 16:64] = 0.25
    inp["w"] = wl.to_dtype(wq, dtype)  # values exact in the call's dtype (the scaled block)
    prob = DeviceProblem(w, inp, nf4=True)
    torch.cuda.synchronize()
    log(f"[gpu] nf4 quantiser {dtype} N={w.n_out} d={w.d_model}")
    got = prob.w_qkv.cpu().numpy()
    codes, scales = oracle_nf4(inp)
    want = q.pack(codes, scales)
    assert got.size == want.size == B.lrq_nf4_weight_size(prob.desc)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{bad.size} bytes differ, first at {bad[:8]}"


def run_case(w, inp, variant, backward, prepared=False, dropout=None):
    import torch
    desc = desc_for(w, variant=variant, nf4=True, dropout=dropout)
    if B.lrq_select_variant(desc, False) < 0 or (backward and B.lrq_select_variant(desc, True) < 0):
        pytest.skip(f"variant {variant} does not cover this shape")
    prob = DeviceProblem(w, inp, variant=variant, backward=backward, nf4=True, dropout=dropout)
    if prepared:
        prob.prepare()
    out = prob.forward()
    res = {"out": out}
    if backward:
        res["dx"], res["da"], res["db"] = prob.backward()
    torch.cuda.synchronize()
    return prob, res


@pytest.mark.parametrize("variant", list(VARIANTS))
@pytest.mark.parametrize("name", list(CASES))
def test_qlora_forward_backward(name, variant):
    w = CASES[name]
    inp = wl.make_inputs(w, with_dy=True)
    log(f"[gpu] qlora {name} variant={variant}")
    check_qlora(w, inp, variant)


@pytest.mark.parametrize("variant", list(VARIANTS))
@pytest.mark.parametrize("seed", range(6))
def test_qlora_random_shape(seed, variant):
    """Seeded random layers (the generator of the random-shape sweep; for the decode family at
    most 256 rows and d = 512) with the base stored as NF4, forward and (tiled, generic) backward."""
    from test_gpu_random_shapes import random_case
    w, _ = random_case(300 + seed, backward=True)
    if variant == "decode":
        w = w.replace(n_tokens=1 + (w.n_tokens - 1) % 256, d_model=512, w_var=1.0 / 512)
    inp = wl.make_inputs(w, seed=seed, with_dy=True)
    log(f"[gpu] qlora random seed={seed} T={w.n_tokens} d={w.d_model} heads={w.n_q_heads}/{w.n_kv_heads}x"
        f"{w.head_dim} r={w.lora_rank} targets={w.lora_targets} variant={variant}")
    check_qlora(w, inp, variant)


def check_qlora(w, inp, variant):
    prob, res = run_case(w, inp, VARIANTS[variant], backward=variant != "decode")
    codes, scales = oracle_nf4(inp)
    spec = spec_of(w)
    ref = q.forward(spec, inp["x"], inp["gamma"], codes, scales, inp["bias"], inp["a"], inp["b"], inp["positions"])
    got = to_np(res["out"])
    errs = {"out": o.rel_frobenius(got, ref), "out_row": row_rel_errors(got, ref),
            "out_elem": elem_ratio(got, ref, w.dtype)}
    if variant == "decode":  # a forward family
        log(f"  errors {errs}")
        assert_parity(errs, w.dtype)
        return
    rdx, rda, rdb = q.backward(spec, inp["x"], inp["gamma"], codes, scales, inp["bias"], inp["a"], inp["b"],
                               inp["positions"], inp["dy"])
    gdx = to_np(res["dx"])
    errs.update({"dx": o.rel_frobenius(gdx, rdx), "dx_row": row_rel_errors(gdx, rdx),
                 "dx_elem": elem_ratio(gdx, rdx, w.dtype)})
    for i, t in enumerate((TQ, TK, TV)):
        if w.lora_targets & t:
            errs[f"dA{i}"] = o.rel_frobenius(to_np(res["da"][i]), rda[t])
            errs[f"dB{i}"] = o.rel_frobenius(to_np(res["db"][i]), rdb[t])
    log(f"  errors {errs}")
    assert_parity(errs, w.dtype)


def test_qlora_prepared_equals_per_call():
    """Prepared NF4 weights (dequantised and folded once) give the same bits as the per-call
    preparation, forward and backward."""
    import torch
    w = CASES["bf16_t513_allt_r64_bias"]
    inp = wl.make_inputs(w, with_dy=True)
    _, a = run_case(w, inp, B.LRQ_VARIANT_TILED, backward=True)
    _, b = run_case(w, inp, B.LRQ_VARIANT_TILED, backward=True, prepared=True)
    assert torch.equal(a["out"], b["out"]) and torch.equal(a["dx"], b["dx"])
    for x, y in zip(a["da"] + a["db"], b["da"] + b["db"]):
        if x is not None:
            assert torch.equal(x, y)


def test_qlora_with_dropout():
    """The NF4 base together with LoRA dropout (tiled family)."""
    w = CASES["bf16_t300_qv_r16"]
    inp = wl.make_inputs(w, with_dy=True)
    p, seed, offset = 0.1, 31, 2
    _, res = run_case(w, inp, B.LRQ_VARIANT_TILED, backward=True, dropout=(p, seed, offset))
    codes, scales = oracle_nf4(inp)
    drop = o.Dropout(float(np.float32(p)), seed, offset)
    spec = spec_of(w)
    ref = q.forward(spec, inp["x"], inp["gamma"], codes, scales, inp["bias"], inp["a"], inp["b"], inp["positions"],
                    dropout=drop)
    rdx, _, _ = q.backward(spec, inp["x"], inp["gamma"], codes, scales, inp["bias"], inp["a"], inp["b"],
                           inp["positions"], inp["dy"], dropout=drop)
    got, gdx = to_np(res["out"]), to_np(res["dx"])
    errs = {"out": o.rel_frobenius(got, ref), "out_elem": elem_ratio(got, ref, "bf16"),
            "dx": o.rel_frobenius(gdx, rdx), "dx_elem": elem_ratio(gdx, rdx, "bf16")}
    log(f"  errors {errs}")
    assert_parity(errs, "bf16")


def test_qlora_decode_full_size_with_cache():
    """The decode workload (64 rows, Llama-2-7B layer, rank 64 on q, k, v, bias) with its base
    in NF4, through the decode family with a key/value cache: every output row, and the cache
    rows equal to the output's k and v blocks bit for bit."""
    import torch
    w = wl.get("decode")
    inp = wl.make_inputs(w)
    desc = desc_for(w, nf4=True)
    assert B.lrq_select_variant(desc) == B.LRQ_VARIANT_DECODE
    prob = DeviceProblem(w, inp, nf4=True)
    kvw = w.n_kv_heads * w.head_dim
    n_slots = 100
    slots = np.random.default_rng(3).permutation(n_slots)[:w.n_tokens].astype(np.int32)
    kc = torch.zeros((n_slots, kvw), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    B.lrq_forward_kv(prob.desc, prob.x, prob.gamma, prob.w_qkv, prob.bias, prob.a, prob.b, prob.positions,
                     prob.out, kc, vc, torch.from_numpy(slots).cuda(), n_slots, prob.workspace)
    torch.cuda.synchronize()
    codes, scales = oracle_nf4(inp)
    ref = q.forward(spec_of(w), inp["x"], inp["gamma"], codes, scales, inp["bias"], inp["a"], inp["b"],
                    inp["positions"])
    got = to_np(prob.out)
    errs = {"out": o.rel_frobenius(got, ref), "out_row": row_rel_errors(got, ref),
            "out_elem": elem_ratio(got, ref, "bf16")}
    log(f"  errors {errs}")
    assert_parity(errs, "bf16")
    k0 = w.target_columns()[wl.TARGET_K][0]
    assert torch.equal(kc[torch.from_numpy(slots).long().cuda()], prob.out[:, k0:k0 + kvw])
    assert torch.equal(vc[torch.from_numpy(slots).long().cuda()], prob.out[:, k0 + kvw:k0 + 2 * kvw])


def test_qlora_llama3_full_size():
    """The Llama-3-8B projection (8192 tokens) with its base in NF4: forward on sampled rows."""
    import torch
    w = wl.get("llama3")
    inp = wl.make_inputs(w)
    desc = desc_for(w, nf4=True)
    assert B.lrq_select_variant(desc) == B.LRQ_VARIANT_TILED
    prob = DeviceProblem(w, inp, nf4=True)
    prob.prepare()
    log(f"[gpu] qlora llama3 T={w.n_tokens} NF4 bytes={B.lrq_nf4_weight_size(desc)}")
    out = prob.forward()
    torch.cuda.synchronize()
    rows = sample_rows(w.n_tokens, 192, seed=8)
    codes, scales = oracle_nf4(inp)
    ref = o.forward_rows(spec_of(w), rows, inp["x"], inp["gamma"], q.dequantize(codes, scales), inp["bias"],
                         inp["a"], inp["b"], inp["positions"])
    got = to_np(out)[rows]
    errs = {"out": o.rel_frobenius(got, ref), "out_row": row_rel_errors(got, ref),
            "out_elem": elem_ratio(got, ref, "bf16")}
    log(f"  errors {errs}")
    assert_parity(errs, "bf16")
