"""GPU parity of the key/value cache write (lrq_forward_kv), through the C ABI.

Bars: the cache rows are byte work, so they must equal the oracle's cache update of the GPU
output bit for bit (written rows hold exactly the k and v blocks of out; every other row keeps
its old value); the output itself meets the forward's bar against the oracle and is the same,
bit for bit, as lrq_forward's.  Every family is covered: the decode family stores the rows from
the streaming kernel's epilogue (after the LoRA term for columns with an adapter), the tiled
family from the epilogue that stores out, and the generic family copies them from out.  A
seeded sweep of random shapes runs each through every family that covers it."""
import numpy as np
import pytest

import oracle.lrq_oracle as o
from helpers import TOL, assert_parity, forward_errors, log, oracle_forward, spec_of, to_np
from layer_rmsnorm_qkv_amd import binding as B
from layer_rmsnorm_qkv_amd import workloads as wl
from layer_rmsnorm_qkv_amd.device import DeviceProblem, desc_for, torch_dtype

pytestmark = pytest.mark.gpu

TQ, TK, TV = wl.TARGET_Q, wl.TARGET_K, wl.TARGET_V
L3, DEC, TINY = wl.get("llama3"), wl.get("decode"), wl.get("tiny")

CASES = {
    # name: (workload, family)
    "tiny_f32": (TINY, B.LRQ_VARIANT_GENERIC),
    "f32_d6_allt": (TINY.replace(n_tokens=65, head_dim=6, n_q_heads=4, n_kv_heads=4,
                                 lora_targets=TQ | TK | TV, lora_rank=3, lora_alpha=5.0), B.LRQ_VARIANT_GENERIC),
    "l3_t70_tiled": (L3.replace(n_tokens=70, d_model=512, n_q_heads=8, n_kv_heads=2), B.LRQ_VARIANT_TILED),
    "l3_t70_generic": (L3.replace(n_tokens=70, d_model=512, n_q_heads=8, n_kv_heads=2), B.LRQ_VARIANT_GENERIC),
    # the tiled epilogue's cache stores: several token tiles with a ragged last one, k and v
    # adapted (rank 64, the second adapter layout) with bias; and four kv heads without adapters
    "l3_t300_tiled_r64_allt": (L3.replace(n_tokens=300, d_model=512, n_q_heads=8, n_kv_heads=2, lora_rank=64,
                                          lora_targets=TQ | TK | TV, has_bias=True, bias_var=0.02),
                               B.LRQ_VARIANT_TILED),
    "l3_t520_tiled_kv4_noadapt": (L3.replace(n_tokens=520, d_model=512, n_q_heads=4, n_kv_heads=4, lora_targets=0),
                                  B.LRQ_VARIANT_TILED),
    # k and v adapted: the rows are stored after the LoRA term handed over from the A blocks
    "dec_t200_allt": (L3.replace(n_tokens=200, d_model=1024, n_q_heads=8, n_kv_heads=2, lora_rank=24,
                                 lora_targets=TQ | TK | TV, has_bias=True, bias_var=0.02), B.LRQ_VARIANT_DECODE),
    # k and v without adapters: no wait for a LoRA term before the store
    "dec_t33_q_only": (DEC.replace(n_tokens=33, d_model=512, n_q_heads=4, n_kv_heads=4, lora_targets=TQ),
                       B.LRQ_VARIANT_DECODE),
    "dec_t1_noadapt": (DEC.replace(n_tokens=1, d_model=512, n_q_heads=4, n_kv_heads=4, lora_targets=0),
                       B.LRQ_VARIANT_DECODE),
}


def make_slots(T: int, num_slots: int, seed: int) -> np.ndarray:
    """Distinct rows for most tokens, a few padding tokens (-1) and one slot past the cache."""
    rng = np.random.default_rng(seed)
    slots = rng.permutation(num_slots)[:T].astype(np.int32)
    if T >= 4:
        slots[rng.choice(T, size=max(1, T // 8), replace=False)] = -1
        slots[T // 2] = num_slots + 3
    return slots


def run(w, variant, num_slots, slots, seed=0, rows=None):
    import torch
    inp = wl.make_inputs(w, seed=seed)
    desc = desc_for(w, variant=variant)
    if B.lrq_select_variant(desc) < 0:
        pytest.skip(f"family {variant} does not cover this shape ({B.lrq_last_error()})")
    prob = DeviceProblem(w, inp, variant=variant)
    kvw = w.n_kv_heads * w.head_dim
    rng = np.random.default_rng(seed + 7)
    init = rng.standard_normal((2, num_slots if rows is None else rows, kvw))
    # values exactly representable in the cache dtype, so the float64 expectation is exact
    init = wl.round_to_bf16(init) if w.dtype != "f32" else init.astype(np.float32).astype(np.float64)
    dt = torch_dtype(w)
    kc = torch.from_numpy(init[0]).to(device="cuda", dtype=dt)
    vc = torch.from_numpy(init[1]).to(device="cuda", dtype=dt)
    sl = torch.from_numpy(slots).to("cuda")
    log(f"[gpu] forward_kv {w.name} T={w.n_tokens} N={w.n_out} family={B.VARIANT_NAMES[prob.variant]} "
        f"slots={num_slots}")
    B.lrq_forward_kv(prob.desc, prob.x, prob.gamma, prob.w_qkv, prob.bias, prob.a, prob.b, prob.positions,
                     prob.out, kc, vc, sl, num_slots, prob.workspace)
    out_kv = prob.out.clone()
    prob.forward()
    torch.cuda.synchronize()
    return inp, prob, out_kv, kc, vc, init


@pytest.mark.parametrize("name", list(CASES))
def test_forward_kv_cache(name):
    w, variant = CASES[name]
    num_slots = w.n_tokens + 7
    slots = make_slots(w.n_tokens, num_slots, seed=11)
    inp, prob, out_kv, kc, vc, init = run(w, variant, num_slots, slots)
    import torch
    assert torch.equal(out_kv, prob.out), "lrq_forward_kv and lrq_forward disagree on out"
    got = to_np(out_kv)
    errs = forward_errors(w, got, oracle_forward(w, inp))
    log(f"  errors {errs}")
    assert_parity(errs, w.dtype)
    ek, ev = o.kv_cache_write(spec_of(w), got, slots, init[0], init[1])
    assert np.array_equal(to_np(kc), ek)
    assert np.array_equal(to_np(vc), ev)


def test_decode_workload_cache_at_positions():
    """The decode workload (64 rows at positions in [0, 8192)) writing a contiguous cache of 8192
    rows at its positions, in the launch configuration the benchmark times."""
    w = DEC
    inp = wl.make_inputs(w)
    slots = np.asarray(inp["positions"], dtype=np.int32).copy()
    seen = set()
    for t, s in enumerate(slots.tolist()):  # a repeated position is written once (unique result)
        if s in seen:
            slots[t] = -1
        seen.add(s)
    _, prob, out_kv, kc, vc, init = run(w, B.LRQ_VARIANT_AUTO, 8192, slots)
    assert prob.variant == B.LRQ_VARIANT_DECODE
    got = to_np(out_kv)
    ek, ev = o.kv_cache_write(spec_of(w), got, slots, init[0], init[1])
    assert np.array_equal(to_np(kc), ek)
    assert np.array_equal(to_np(vc), ev)


@pytest.mark.parametrize("name", ["dec_t33_q_only", "l3_t70_tiled"])
def test_zero_slots_writes_nothing(name):
    """num_slots = 0: every slot is outside the cache, so the caches keep their contents."""
    w, variant = CASES[name]
    slots = make_slots(w.n_tokens, w.n_tokens + 7, seed=3)
    _, prob, out_kv, kc, vc, init = run(w, variant, 0, slots, rows=16)
    assert np.array_equal(to_np(kc), init[0]) and np.array_equal(to_np(vc), init[1])


@pytest.mark.parametrize("variant", ["generic", "tiled", "decode"])
@pytest.mark.parametrize("seed", range(6))
def test_forward_kv_cache_random_shape(seed, variant):
    """Seeded random layers (the generator of the random-shape forward sweep; for the decode
    family at most 256 rows and d = 512) through lrq_forward_kv with padding tokens and a slot past the
    cache, in every family that covers the shape: out to the forward's bar, the cache rows bit
    for bit."""
    from test_gpu_random_shapes import random_case
    w, _ = random_case(200 + seed)
    if variant == "decode":  # the decode family's range: at most 256 rows, d a multiple of 512
        w = w.replace(n_tokens=1 + (w.n_tokens - 1) % 256, d_model=512, w_var=1.0 / 512)
    v = {"generic": B.LRQ_VARIANT_GENERIC, "tiled": B.LRQ_VARIANT_TILED, "decode": B.LRQ_VARIANT_DECODE}[variant]
    num_slots = w.n_tokens + 5
    slots = make_slots(w.n_tokens, num_slots, seed=seed)
    inp, prob, out_kv, kc, vc, init = run(w, v, num_slots, slots, seed=seed)
    import torch
    assert torch.equal(out_kv, prob.out), "lrq_forward_kv and lrq_forward disagree on out"
    got = to_np(out_kv)
    errs = forward_errors(w, got, oracle_forward(w, inp))
    log(f"  errors {errs}")
    assert_parity(errs, w.dtype)
    ek, ev = o.kv_cache_write(spec_of(w), got, slots, init[0], init[1])
    assert np.array_equal(to_np(kc), ek)
    assert np.array_equal(to_np(vc), ev)
