"""Prepared frozen weights on the GPU: forward and backward calls that pass the buffer written
by lrq_prepare_weights give the same results, bit for bit, as the calls that prepare the weights
themselves, with the smaller workspace; a call whose family takes no prepared layout (decode,
generic) ignores it; and the prepared calls replay in a HIP graph."""
import pytest
import torch

from helpers import log
from layer_rmsnorm_qkv_amd import binding as B
from layer_rmsnorm_qkv_amd import workloads as wl
from layer_rmsnorm_qkv_amd.device import DeviceProblem, desc_for

pytestmark = pytest.mark.gpu

TQ, TK, TV = wl.TARGET_Q, wl.TARGET_K, wl.TARGET_V
CASES = {
    "l2_t257_allt_r64": wl.get("llama2").replace(n_tokens=257, d_model=768, n_q_heads=6, n_kv_heads=6),
    "l3_t300_gqa_bias": wl.get("train").replace(n_tokens=300, d_model=512, n_q_heads=8, n_kv_heads=2,
                                                has_bias=True, bias_var=0.02),
    "l3_noadapt": wl.get("train").replace(n_tokens=260, d_model=512, n_q_heads=4, n_kv_heads=2, lora_targets=0),
}


def _pair(w, variant=B.LRQ_VARIANT_AUTO):
    inp = wl.make_inputs(w, with_dy=True)
    plain = DeviceProblem(w, inp, variant=variant, backward=True)
    prep = DeviceProblem(w, inp, variant=variant, backward=True)
    prep.prepare()
    # the prepared calls get only the smaller workspace they need
    ws = max(B.lrq_workspace_size_prepared(prep.desc, False), B.lrq_workspace_size_prepared(prep.desc, True))
    prep.workspace = torch.empty(ws, dtype=torch.uint8, device="cuda") if ws else None
    return plain, prep


@pytest.mark.parametrize("name", list(CASES))
def test_prepared_equals_unprepared_bitwise(name):
    w = CASES[name]
    log(f"[gpu] prepared weights {name}")
    plain, prep = _pair(w)
    assert prep.prepared is not None
    y0 = plain.forward().clone()
    y1 = prep.forward().clone()
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
    g0 = [t.clone() for t in plain.backward(y=y0)[0:1]] + [t.clone() for t in plain.da + plain.db if t is not None]
    g1 = [t.clone() for t in prep.backward(y=y0)[0:1]] + [t.clone() for t in prep.da + prep.db if t is not None]
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(g0, g1))


def test_prepared_ignored_by_the_decode_family():
    w = wl.get("decode").replace(n_tokens=33, d_model=512, n_q_heads=4, n_kv_heads=4)
    log("[gpu] prepared weights with a decode-family call")
    plain, prep = _pair(w)
    assert plain.variant == B.LRQ_VARIANT_DECODE
    prep.workspace = plain.workspace
    assert torch.equal(plain.forward().clone(), prep.forward().clone())


def test_prepared_calls_replay_in_a_hip_graph():
    w = CASES["l3_t300_gqa_bias"]
    log("[gpu] prepared forward + backward in a HIP graph")
    plain, prep = _pair(w)
    y = plain.forward().clone()
    ref = [t.clone() for t in plain.backward(y=y)[0:1]] + [t.clone() for t in plain.da + plain.db if t is not None]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        prep.forward()
        prep.backward(y=y)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        prep.forward()
        prep.backward(y=y)
    for _ in range(3):
        prep.out.zero_()
        prep.dx.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(prep.out, y)
        got = [prep.dx] + [t for t in prep.da + prep.db if t is not None]
        assert all(torch.equal(a, b) for a, b in zip(got, ref))
        prep.forward()
        torch.cuda.synchronize()
