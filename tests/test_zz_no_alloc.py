"""The no-allocation forward (lrq_forward_noalloc) on the GPU, through the C ABI: two calls in
a row -- the second with fewer tokens -- each equal, bit for bit, to lrq_forward_prepared with
a caller workspace on the same inputs (so within the forward's parity bar), for the tiled
family with prepared weights and for the decode family; plus one parity check against the
oracle, and a refused oversized call that launches nothing."""
import pytest
import torch

from helpers import assert_parity, forward_errors, log, oracle_forward, to_np
from layer_rmsnorm_qkv_amd import binding as B
from layer_rmsnorm_qkv_amd import workloads as wl
from layer_rmsnorm_qkv_amd.device import DeviceProblem

pytestmark = pytest.mark.gpu

CASES = {
    # tiled family (more than 256 rows), prepared weights; then a smaller call
    "tiled": (wl.get("llama2").replace(n_tokens=700, d_model=1024, n_q_heads=8, n_kv_heads=8, has_bias=True,
                                       bias_var=0.02), 300),
    # decode family; then a single row
    "decode": (wl.get("decode").replace(d_model=1024, n_q_heads=8, n_kv_heads=8), 1),
}


def _problem(w, n_tokens, seed):
    w2 = w.replace(n_tokens=n_tokens)
    prob = DeviceProblem(w2, wl.make_inputs(w2, seed=seed))
    prob.prepare()
    return w2, prob


def _pair(prob):
    """(reference via lrq_forward_prepared with a workspace, result of lrq_forward_noalloc)."""
    ref = torch.empty_like(prob.out)
    got = torch.empty_like(prob.out)
    ws = B.lrq_workspace_size_prepared(prob.desc)
    work = torch.empty(ws, dtype=torch.uint8, device="cuda") if ws else None
    B.lrq_forward_prepared(prob.desc, prob.x, prob.gamma, prob.w_qkv, prob.prepared, prob.bias, prob.a, prob.b,
                           prob.positions, ref, None, work)
    B.lrq_forward_noalloc(prob.desc, prob.x, prob.gamma, prob.w_qkv, prob.prepared, prob.bias, prob.a, prob.b,
                          prob.positions, got)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("name", list(CASES))
def test_noalloc_matches_the_workspace_call_twice(name):
    w, small = CASES[name]
    for i, T in enumerate((w.n_tokens, small)):
        w2, prob = _problem(w, T, seed=100 + i)
        log(f"[gpu] no-alloc forward {name} call {i + 1}: T={T} d={w2.d_model} N={w2.n_out} "
            f"family={B.VARIANT_NAMES[prob.variant]}")
        assert B.lrq_workspace_size_prepared(prob.desc) <= B.NOALLOC_SCRATCH_BYTES
        ref, got = _pair(prob)
        assert torch.equal(ref, got), (name, T)
        if i == 0:
            inp = wl.make_inputs(w2, seed=100)
            errs = forward_errors(w2, to_np(got), oracle_forward(w2, inp))
            log(f"  errors {errs}")
            assert_parity(errs, "bf16")


def test_noalloc_refuses_an_oversized_call():
    w = wl.get("llama3").replace(n_tokens=512, d_model=8192, n_q_heads=4, n_kv_heads=4)
    prob = DeviceProblem(w, wl.make_inputs(w))
    log("[gpu] no-alloc forward refused without prepared weights")
    assert B.lrq_workspace_size(prob.desc) > B.NOALLOC_SCRATCH_BYTES
    with pytest.raises(B.LrqError) as ei:
        B.lrq_forward_noalloc(prob.desc, prob.x, prob.gamma, prob.w_qkv, None, prob.bias, prob.a, prob.b,
                              prob.positions, prob.out)
    assert ei.value.status == B.LRQ_ERR_UNSUPPORTED
