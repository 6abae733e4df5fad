"""GPU parity of the forward, through the C ABI, against the CPU oracle.

Bars: max relative Frobenius error (whole output, and each of the q, k, v blocks)
<= 1e-5 for float32 and <= 5e-3 for bf16 inputs with fp32 accumulation.  Small cases
are compared in full; the full-size layer workloads are compared on sampled rows (rows
are independent given their positions), in the launch configuration the benchmark
times."""
import numpy as np
import pytest

from helpers import TOL, assert_parity, forward_errors, log, oracle_forward, sample_rows, to_np
from layer_rmsnorm_qkv_amd import binding as B
from layer_rmsnorm_qkv_amd import workloads as wl
from layer_rmsnorm_qkv_amd.device import DeviceProblem, desc_for

pytestmark = pytest.mark.gpu

VARIANTS = {"generic": B.LRQ_VARIANT_GENERIC, "tiled": B.LRQ_VARIANT_TILED, "decode": B.LRQ_VARIANT_DECODE}

TQ, TK, TV = wl.TARGET_Q, wl.TARGET_K, wl.TARGET_V
TINY = wl.get("tiny")
L3 = wl.get("llama3")
L2 = wl.get("llama2")
DEC = wl.get("decode")

# small shapes: ragged token counts, odd widths, every target subset, bias on/off
SMALL_F32 = {
    "tiny": TINY,
    "t1": TINY.replace(n_tokens=1),
    "t33_d100_bias": TINY.replace(n_tokens=33, d_model=100, has_bias=True, bias_var=0.02, seq_len=0,
                                  max_position=9000),
    "t65_d6_allt": TINY.replace(n_tokens=65, head_dim=6, n_q_heads=4, n_kv_heads=4,
                                lora_targets=TQ | TK | TV, lora_rank=3, lora_alpha=5.0),
    "t40_k_only_gqa8": TINY.replace(n_tokens=40, n_q_heads=8, n_kv_heads=1, lora_targets=TK),
    "t9_noadapt": TINY.replace(n_tokens=9, lora_targets=0),
}
SMALL_BF16 = {
    "l3_t70": L3.replace(n_tokens=70, d_model=512, n_q_heads=8, n_kv_heads=2),
    "l2_t257_allt": L2.replace(n_tokens=257, d_model=768, n_q_heads=6, n_kv_heads=6),
    "dec_t64": DEC.replace(d_model=1024, n_q_heads=8, n_kv_heads=8),
    "l3_t1": L3.replace(n_tokens=1, d_model=256, n_q_heads=4, n_kv_heads=1),
    "l3_d64head": L3.replace(n_tokens=45, d_model=256, n_q_heads=4, n_kv_heads=2, head_dim=64),
    # decode-family shapes: one row, several 64-row groups with a ragged tail, GQA with a rank
    # that is not a multiple of 16 on all targets plus bias, 64-wide heads with one target
    "dec_t1": DEC.replace(n_tokens=1, d_model=512, n_q_heads=4, n_kv_heads=4),
    "dec_t200_gqa_r24": L3.replace(n_tokens=200, d_model=1024, n_q_heads=8, n_kv_heads=2, lora_rank=24,
                                   lora_targets=TQ | TK | TV, has_bias=True, bias_var=0.02),
    "dec_d64head_konly": DEC.replace(n_tokens=33, d_model=512, n_q_heads=4, n_kv_heads=2, head_dim=64,
                                     lora_targets=TK, lora_rank=5),
    # the decode family's LoRA hand-over: a second row group holding one row, a rank that is
    # not a multiple of 8 (element loads of B) on every target, bias, GQA
    "dec_t65_r5_allt": L3.replace(n_tokens=65, d_model=512, n_q_heads=8, n_kv_heads=2, lora_rank=5,
                                  lora_targets=TQ | TK | TV, has_bias=True, bias_var=0.02),
    # a rank that is not a multiple of 8 in the MFMA families (element loads of B in the
    # tiled epilogue, a ragged rank block)
    "l3_t130_r5_konly": L3.replace(n_tokens=130, d_model=512, n_q_heads=4, n_kv_heads=2, lora_rank=5,
                                   lora_targets=TK),
}


def run_case(w, variant, rows=None, seed=None):
    inp = wl.make_inputs(w, seed=seed)
    desc = desc_for(w, variant=variant)
    if B.lrq_select_variant(desc) < 0:
        pytest.skip(f"variant {variant} does not cover this shape ({B.lrq_last_error()})")
    log(f"[gpu] forward {w.name} T={w.n_tokens} d={w.d_model} N={w.n_out} variant={variant}")
    prob = DeviceProblem(w, inp, variant=variant)
    got = to_np(prob.forward())
    import torch
    torch.cuda.synchronize()
    if rows is not None:
        got = got[rows]
    ref = oracle_forward(w, inp, rows)
    return got, ref, prob


@pytest.mark.parametrize("name", list(SMALL_F32))
def test_forward_f32_small(name):
    w = SMALL_F32[name]
    got, ref, _ = run_case(w, B.LRQ_VARIANT_GENERIC)
    errs = forward_errors(w, got, ref)
    log(f"  errors {errs}")
    assert_parity(errs, "f32")


@pytest.mark.parametrize("variant", list(VARIANTS))
@pytest.mark.parametrize("name", list(SMALL_BF16))
def test_forward_bf16_small(name, variant):
    w = SMALL_BF16[name]
    got, ref, _ = run_case(w, VARIANTS[variant])
    errs = forward_errors(w, got, ref)
    log(f"  errors {errs}")
    assert_parity(errs, "bf16")


@pytest.mark.parametrize("variant", list(VARIANTS))
@pytest.mark.parametrize("name", ["llama3", "llama2", "decode", "train"])
def test_forward_full_size_sampled(name, variant):
    """The layer workloads at their full sizes, checked on sampled rows."""
    w = wl.get(name)
    if variant == "generic" and w.n_tokens > 4096:
        pytest.skip("generic family is checked at full size on the decode workload only")
    rows = sample_rows(w.n_tokens, 256, seed=w.index)
    got, ref, _ = run_case(w, VARIANTS[variant], rows=rows)
    errs = forward_errors(w, got, ref)
    log(f"  errors {errs}")
    assert_parity(errs, "bf16")


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_zero_b_equals_no_adapters_bitwise(variant):
    """B = 0 gives bit-for-bit the output of the same call without adapters."""
    import torch
    w = SMALL_BF16["dec_t200_gqa_r24" if variant == "decode" else "l2_t257_allt"]
    inp = wl.make_inputs(w)
    if B.lrq_select_variant(desc_for(w, variant=VARIANTS[variant])) < 0:
        pytest.skip("variant does not cover this shape")
    log(f"[gpu] zero-B bitwise variant={variant}")
    zero_b = dict(inp, b={t: np.zeros_like(v) for t, v in inp["b"].items()})
    p1 = DeviceProblem(w, zero_b, variant=VARIANTS[variant])
    p2 = DeviceProblem(w.replace(lora_targets=0), inp, variant=VARIANTS[variant])
    o1, o2 = p1.forward(), p2.forward()
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_repeated_runs_bitwise_identical(variant):
    import torch
    w = SMALL_BF16["l3_t70"]
    if B.lrq_select_variant(desc_for(w, variant=VARIANTS[variant])) < 0:
        pytest.skip("variant does not cover this shape")
    log(f"[gpu] determinism variant={variant}")
    prob = DeviceProblem(w, wl.make_inputs(w), variant=VARIANTS[variant])
    first = prob.forward().clone()
    for _ in range(3):
        assert torch.equal(prob.forward(), first)


def test_zero_rows_and_extreme_positions():
    """All-zero rows (h = 0, output = rotated bias) and positions near 2^31 / 8191."""
    import torch
    w = DEC.replace(d_model=512, n_q_heads=4, n_kv_heads=4, n_tokens=16)
    inp = wl.make_inputs(w)
    inp["x"][3] = 0.0
    inp["positions"][:] = np.array([0, 1, 8191, 2 ** 31 - 1] * 4, dtype=np.int32)
    for variant in VARIANTS.values():
        if B.lrq_select_variant(desc_for(w, variant=variant)) < 0:
            continue
        log(f"[gpu] zero rows / extreme positions variant={variant}")
        got = to_np(DeviceProblem(w, inp, variant=variant).forward())
        torch.cuda.synchronize()
        ref = oracle_forward(w, inp)
        errs = forward_errors(w, got, ref)
        assert_parity(errs, "bf16", variant)
        assert np.all(np.isfinite(got))


def test_zero_tokens_launches_nothing():
    import torch
    w = SMALL_BF16["l3_t70"]
    prob = DeviceProblem(w, wl.make_inputs(w))
    empty = torch.empty((0, w.n_out), dtype=torch.bfloat16, device="cuda")
    d0 = desc_for(w, n_tokens=0)
    B.lrq_forward(d0, prob.x, prob.gamma, prob.w_qkv, prob.bias, prob.a, prob.b, prob.positions, empty,
                  prob.workspace)
    torch.cuda.synchronize()


def test_timing_hook_counts_calls():
    """The measurement hook records one interval per call while enabled (forward and
    backward separately), none while disabled, and its mean lies within the whole call's."""
    import torch
    w = SMALL_BF16["l3_t70"]
    inp = wl.make_inputs(w, with_dy=True)
    prob = DeviceProblem(w, inp, variant=B.LRQ_VARIANT_TILED, backward=True)
    log("[gpu] timing hook")
    prob.forward()
    torch.cuda.synchronize()
    B.lrq_kernel_timing(True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(3):
        prob.forward()
    e1.record()
    prob.backward()
    torch.cuda.synchronize()
    ms_f, n_f = B.lrq_kernel_time_ms(False)
    ms_b, n_b = B.lrq_kernel_time_ms(True)
    assert (n_f, n_b) == (3, 1)
    assert 0.0 < ms_f <= e0.elapsed_time(e1) / 3 * 1.5 and ms_b > 0.0
    B.lrq_kernel_timing(False)
    prob.forward()
    torch.cuda.synchronize()
    assert B.lrq_kernel_time_ms(False) == (0.0, 0)


LIMITS = {
    # the decode family's largest shape (d = 8192, 256 rows) at the largest rank on every target
    "dec_max_d_rows_rank": DEC.replace(n_tokens=256, d_model=8192, n_q_heads=8, n_kv_heads=8, lora_rank=64,
                                       lora_targets=TQ | TK | TV),
    # a long K loop (128 steps of 64) with a ragged token tile in the tiled family
    "l3_d8192_t300": L3.replace(n_tokens=300, d_model=8192, n_q_heads=4, n_kv_heads=2, lora_rank=32),
}


@pytest.mark.parametrize("variant", list(VARIANTS))
@pytest.mark.parametrize("name", list(LIMITS))
def test_forward_at_size_limits(name, variant):
    w = LIMITS[name]
    got, ref, _ = run_case(w, VARIANTS[variant])
    errs = forward_errors(w, got, ref)
    log(f"  errors {errs}")
    assert_parity(errs, "bf16")


def test_forward_f32_largest_head():
    """The generic family's largest head (256) at the largest rank, float32."""
    w = TINY.replace(n_tokens=20, d_model=64, head_dim=256, n_q_heads=2, n_kv_heads=1, lora_rank=64,
                     lora_targets=TQ | TK | TV)
    got, ref, _ = run_case(w, B.LRQ_VARIANT_GENERIC)
    errs = forward_errors(w, got, ref)
    log(f"  errors {errs}")
    assert_parity(errs, "f32")


@pytest.mark.parametrize("variant", ["tiled", "decode"])
def test_forward_replays_in_a_hip_graph(variant):
    """Forward calls captured in a HIP graph replay to the eager result, with eager calls and
    synchronisations between the replays (a decode step is the launch-bound case)."""
    import torch
    w = SMALL_BF16["dec_t200_gqa_r24"]
    if B.lrq_select_variant(desc_for(w, variant=VARIANTS[variant])) < 0:
        pytest.skip("variant does not cover this shape")
    log(f"[gpu] graph capture and replay variant={variant}")
    prob = DeviceProblem(w, wl.make_inputs(w), variant=VARIANTS[variant])
    eager = prob.forward().clone()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        prob.forward()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        prob.forward()
    for _ in range(3):
        prob.out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(prob.out, eager)
        prob.forward()
        torch.cuda.synchronize()


@pytest.mark.parametrize("variant", ["tiled", "decode"])
def test_graph_replays_follow_new_inputs(variant):
    """A captured forward replayed over new x in the same buffer gives each new input's eager
    result, bit for bit (in the decode family the W blocks wait for this launch's U_t, never
    for the one a previous replay stored)."""
    import torch
    w = SMALL_BF16["dec_t200_gqa_r24"]
    if B.lrq_select_variant(desc_for(w, variant=VARIANTS[variant])) < 0:
        pytest.skip("variant does not cover this shape")
    log(f"[gpu] graph replays over new inputs variant={variant}")
    prob = DeviceProblem(w, wl.make_inputs(w), variant=VARIANTS[variant])
    xs = [prob.x.clone()] + [DeviceProblem(w, wl.make_inputs(w, seed=11 + k), variant=VARIANTS[variant]).x
                             for k in range(3)]
    expect = []
    for x in xs:
        prob.x.copy_(x)
        expect.append(prob.forward().clone())
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        prob.forward()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        prob.forward()
    for rnd in range(2):
        for k in range(len(xs)):
            prob.x.copy_(xs[k])
            prob.out.zero_()
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(prob.out, expect[k]), (rnd, k)


def test_decode_calls_on_two_streams_at_once():
    """Two decode calls in flight together on two streams, each with its own workspace (the
    blocks of each launch hand U_t over through their own count words): both results equal
    the same calls made one at a time, bit for bit, over several rounds."""
    import torch
    w = SMALL_BF16["dec_t200_gqa_r24"]
    log("[gpu] decode on two streams at once")
    pa = DeviceProblem(w, wl.make_inputs(w), variant=B.LRQ_VARIANT_DECODE)
    pb = DeviceProblem(w, wl.make_inputs(w, seed=9), variant=B.LRQ_VARIANT_DECODE)
    ea, eb = pa.forward().clone(), pb.forward().clone()
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(4):
        pa.out.zero_()
        pb.out.zero_()
        torch.cuda.synchronize()
        for _ in range(3):
            pa.forward(stream=sa.cuda_stream)
            pb.forward(stream=sb.cuda_stream)
        torch.cuda.synchronize()
        assert torch.equal(pa.out, ea) and torch.equal(pb.out, eb)


@pytest.mark.parametrize("fill", ["zeros", "ones", "random"])
def test_decode_ignores_what_the_workspace_held(fill):
    """The decode family's LoRA-down blocks hand U_t to the W blocks through count words in the
    workspace.  Whatever the workspace held before (zeros, all bits set, random bytes), and with
    a call on other inputs through the same workspace in between, the result is the same, bit
    for bit, as the first call's."""
    import torch
    w = SMALL_BF16["dec_t200_gqa_r24"]
    log(f"[gpu] decode over a used workspace fill={fill}")
    prob = DeviceProblem(w, wl.make_inputs(w), variant=B.LRQ_VARIANT_DECODE)
    other = DeviceProblem(w, wl.make_inputs(w, seed=7), variant=B.LRQ_VARIANT_DECODE)
    other.workspace = prob.workspace
    eager = prob.forward().clone()
    other_ref = other.forward().clone()
    torch.cuda.synchronize()
    gen = torch.Generator(device="cpu").manual_seed(5)
    for _ in range(3):
        if fill == "zeros":
            prob.workspace.zero_()
        elif fill == "ones":
            prob.workspace.fill_(255)
        else:
            prob.workspace.copy_(torch.randint(0, 256, prob.workspace.shape, generator=gen, dtype=torch.uint8))
        prob.out.zero_()
        prob.forward()
        other.forward()
        torch.cuda.synchronize()
        assert torch.equal(prob.out, eager)
        assert torch.equal(other.out, other_ref)


def test_forward_output_past_2_31_elements():
    """T x N above 2^31 output elements (360448 tokens x 6144 columns, d = 512): every row and
    column offset must be formed in 64 bits.  Checked on sampled rows, including the last."""
    import torch
    w = L3.replace(n_tokens=360448, d_model=512, lora_rank=16)
    assert w.n_tokens * w.n_out > 2 ** 31
    log(f"[gpu] forward T={w.n_tokens} N={w.n_out} (T*N = {w.n_tokens * w.n_out}); generating inputs")
    inp = wl.make_inputs(w)
    prob = DeviceProblem(w, inp, variant=B.LRQ_VARIANT_TILED)
    rows = sample_rows(w.n_tokens, 128, seed=11)
    out = prob.forward()
    got = to_np(out[torch.as_tensor(rows, device=out.device)])
    torch.cuda.synchronize()
    errs = forward_errors(w, got, oracle_forward(w, inp, rows))
    log(f"  errors {errs}")
    assert_parity(errs, "bf16")


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_forward_negative_positions(variant):
    """Positions are not range-checked: a negative position rotates by a negative angle, in
    every family as in the oracle (half of the rows negative, down to -9000)."""
    w = SMALL_BF16["l3_t70"]
    inp = wl.make_inputs(w)
    pos = np.asarray(inp["positions"], dtype=np.int64)
    rng = np.random.default_rng(7)
    neg = rng.random(pos.shape[0]) < 0.5
    pos = np.where(neg, -rng.integers(1, 9001, size=pos.shape[0]), pos)
    inp["positions"] = pos.astype(np.int32)
    desc = desc_for(w, variant=VARIANTS[variant])
    if B.lrq_select_variant(desc) < 0:
        pytest.skip(f"variant {variant} does not cover this shape")
    log(f"[gpu] forward negative positions {w.name} variant={variant}")
    prob = DeviceProblem(w, inp, variant=VARIANTS[variant])
    got = to_np(prob.forward())
    errs = forward_errors(w, got, oracle_forward(w, inp))
    log(f"  errors {errs}")
    assert_parity(errs, "bf16")
