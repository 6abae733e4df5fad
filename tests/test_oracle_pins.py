"""The CPU oracle against its pins (closed forms, special cases, independent formulations,
brute force, finite differences).  CPU only."""
import numpy as np
import pytest

import oracle.lrq_oracle as o
import pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check(o)


def test_rel_frobenius():
    a = np.array([[3.0, 4.0]])
    assert o.rel_frobenius(a, a) == 0.0
    assert abs(o.rel_frobenius(a + np.array([[0.0, 0.5]]), a) - 0.1) < 1e-15
    assert o.rel_frobenius(np.zeros((0, 3)), np.zeros((0, 3))) == 0.0


def test_workload_shapes_match_descriptions():
    """Workload recipe: shapes, head layout, LoRA scale, positions, distributions."""
    from layer_rmsnorm_qkv_amd import workloads as wl
    assert [w.n_out for w in wl.WORKLOADS] == [128, 6144, 12288, 12288, 6144]
    assert [w.n_tokens for w in wl.WORKLOADS] == [8, 8192, 16384, 64, 16384]
    assert [w.lora_alpha / w.lora_rank for w in wl.WORKLOADS] == [2.0, 2.0, 0.25, 0.25, 2.0]
    tiny = wl.get("tiny")
    inp = wl.make_inputs(tiny)
    assert inp["x"].shape == (8, 64) and inp["w"].shape == (128, 64)
    assert sorted(inp["a"]) == [wl.TARGET_Q, wl.TARGET_V]
    assert inp["b"][wl.TARGET_V].shape == (32, 4)
    assert list(inp["positions"]) == list(range(8))
    dec = wl.make_inputs(wl.get("decode"), n_tokens=64)
    assert dec["positions"].min() >= 0 and dec["positions"].max() < 8192
    assert dec["bias"].shape == (12288,)


def test_bf16_rounding_of_inputs():
    """Inputs are rounded to bf16 with ties to even; the generators are deterministic."""
    from layer_rmsnorm_qkv_amd import workloads as wl
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 3.0e38], dtype=np.float64)
    got = wl.round_to_bf16(vals)
    assert list(got[:5]) == [1.0, 1.0, 1.0 + 4 * 2 ** -8, 1.0, -2.5]
    import torch
    ref = torch.from_numpy(vals.astype(np.float32)).to(torch.bfloat16).float().numpy()
    assert np.array_equal(got, ref)
    w = wl.get("llama3").replace(n_tokens=4, d_model=64, n_q_heads=2, n_kv_heads=1, head_dim=16)
    i1, i2 = wl.make_inputs(w), wl.make_inputs(w)
    assert np.array_equal(i1["x"], i2["x"]) and np.array_equal(i1["w"], i2["w"])
    assert np.array_equal(wl.round_to_bf16(i1["x"]), i1["x"])



def test_rope_negative_positions_rotate_backwards():
    """Rotating by a negative position -p is the inverse rotation by p (R(-phi) = R(phi)^T), and
    the norm of every rotate-half pair is kept: the oracle's reading of negative positions,
    which the GPU tests use as their reference."""
    rng = np.random.default_rng(3)
    D, heads, T = 16, 3, 9
    y = rng.standard_normal((T, heads * D))
    p = rng.integers(1, 9001, size=T).astype(np.int32)
    neg = o.rope_rotate(y, -p, D, 1e4)
    inv = o.rope_rotate(y, p, D, 1e4, inverse=True)
    np.testing.assert_allclose(neg, inv, rtol=0, atol=1e-12)
    back = o.rope_rotate(neg, p, D, 1e4)
    np.testing.assert_allclose(back, y, rtol=0, atol=1e-12)
    a = y.reshape(T, heads, 2, D // 2)
    b = neg.reshape(T, heads, 2, D // 2)
    np.testing.assert_allclose((b ** 2).sum(axis=2), (a ** 2).sum(axis=2), rtol=1e-12)
