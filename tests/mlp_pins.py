"""Checks that pin the SwiGLU-MLP oracle to things other than itself: SiLU's closed forms and
its reflection identity, torch's own silu in float64, the LoRA merged-weight identity, the
special cases of zero weights and zero adapters, and a scalar pure-Python brute force of the
whole MLP.  Used by ``test_mlp_oracle.py`` on the real oracle and on planted mistakes."""
from __future__ import annotations

import math

import numpy as np

TG, TU, TD = 1, 2, 4


def tiny_mlp(o, seed=0, T=5, d=6, F=8, r=2, alpha=3.0, targets=TG | TU | TD):
    rng = np.random.default_rng(seed)
    spec = o.MlpSpec(d_model=d, d_ff=F, lora_rank=r, lora_alpha=alpha, lora_targets=targets)
    c = dict(h=rng.standard_normal((T, d)), wg=rng.standard_normal((F, d)) / math.sqrt(d),
             wu=rng.standard_normal((F, d)) / math.sqrt(d), wd=rng.standard_normal((d, F)) / math.sqrt(F))
    a, b = {}, {}
    for t, (din, dout) in ((TG, (d, F)), (TU, (d, F)), (TD, (F, d))):
        a[t] = rng.standard_normal((r, din)) / math.sqrt(din)
        b[t] = 0.5 * rng.standard_normal((dout, r))
    c["a"], c["b"] = a, b
    return spec, c


def _fwd(o, spec, c):
    return o.mlp_forward(spec, c["h"], c["wg"], c["wu"], c["wd"], c["a"], c["b"])


def _close(got, want, tol, what):
    got, want = np.asarray(got, np.float64), np.asarray(want, np.float64)
    assert got.shape == want.shape, f"{what}: shape {got.shape} != {want.shape}"
    err = float(np.max(np.abs(got - want))) if got.size else 0.0
    scale = max(1.0, float(np.max(np.abs(want)))) if want.size else 1.0
    assert err <= tol * scale, f"{what}: max abs err {err:.3e} > {tol:.1e} x {scale:.3g}"


def check_silu_closed_forms(o):
    """SiLU(0) = 0; SiLU(1) = sigmoid(1) = e / (1 + e); SiLU(z) - SiLU(-z) = z exactly (since
    sigmoid(z) + sigmoid(-z) = 1); SiLU(z) -> z for large z and -> 0 for very negative z;
    SiLU(ln 3) = (3/4) ln 3."""
    assert o.silu(np.array([0.0]))[0] == 0.0
    _close(o.silu(np.array([1.0])), [math.e / (1.0 + math.e)], 1e-15, "SiLU(1)")
    _close(o.silu(np.array([math.log(3.0)])), [0.75 * math.log(3.0)], 1e-15, "SiLU(ln 3)")
    z = np.linspace(-30.0, 30.0, 241)
    _close(o.silu(z) - o.silu(-z), z, 1e-13, "reflection")
    _close(o.silu(np.array([40.0, 80.0])), [40.0, 80.0], 1e-15, "large z")
    assert abs(o.silu(np.array([-800.0]))[0]) == 0.0


def check_silu_torch(o):
    """Against torch.nn.functional.silu in float64 (an independent implementation)."""
    import torch
    z = np.random.default_rng(3).standard_normal(500) * 6
    ref = torch.nn.functional.silu(torch.from_numpy(z)).numpy()
    _close(o.silu(z), ref, 1e-14, "torch silu")


def brute_mlp(spec, c):
    """The whole MLP as scalar loops (tiny shapes only)."""
    h, wg, wu, wd, A, B = c["h"], c["wg"], c["wu"], c["wd"], c["a"], c["b"]
    T, d = h.shape
    F = wg.shape[0]
    s = spec.lora_alpha / spec.lora_rank if spec.lora_rank else 0.0
    r = spec.lora_rank

    def lin(x, w, t, nout, nin):
        out = []
        for n in range(nout):
            acc = sum(w[n][k] * x[k] for k in range(nin))
            if spec.lora_targets & t:
                uu = [sum(A[t][q][k] * x[k] for k in range(nin)) for q in range(r)]
                acc += s * sum(B[t][n][q] * uu[q] for q in range(r))
            out.append(acc)
        return out

    res = []
    for i in range(T):
        g = lin(h[i], wg, TG, F, d)
        u = lin(h[i], wu, TU, F, d)
        act = [g[f] / (1.0 + math.exp(-g[f])) * u[f] for f in range(F)]
        res.append(lin(act, wd, TD, d, F))
    return np.array(res)


def check_mlp_brute_force(o):
    """Equal to scalar loops, for every subset of adapted projections."""
    for seed, targets in ((1, TG | TU | TD), (2, 0), (3, TG), (4, TU | TD), (5, TD)):
        spec, c = tiny_mlp(o, seed=seed, targets=targets)
        _close(_fwd(o, spec, c), brute_mlp(spec, c), 1e-12, f"brute force targets={targets}")


def check_mlp_merged_weights(o):
    """An adapter equals its merged weight W + (alpha / r) B A (how LoRA folds into a layer)."""
    spec, c = tiny_mlp(o, seed=6)
    s = spec.lora_alpha / spec.lora_rank
    merged = dict(c, wg=c["wg"] + s * c["b"][TG] @ c["a"][TG], wu=c["wu"] + s * c["b"][TU] @ c["a"][TU],
                  wd=c["wd"] + s * c["b"][TD] @ c["a"][TD])
    plain = o.MlpSpec(d_model=spec.d_model, d_ff=spec.d_ff)
    _close(_fwd(o, spec, c), _fwd(o, plain, merged), 1e-12, "merged weights")


def check_mlp_special_cases(o):
    """B = 0 gives the adapter-free MLP bit for bit; W_g = 0 without a gate adapter makes every
    SiLU(g) = 0, so the output is exactly 0; without a down adapter the output is linear in W_d;
    rows are independent (the row-subset helper equals the full result's rows)."""
    spec, c = tiny_mlp(o, seed=7)
    zero_b = dict(c, b={t: np.zeros_like(v) for t, v in c["b"].items()})
    plain = o.MlpSpec(d_model=spec.d_model, d_ff=spec.d_ff)
    assert np.array_equal(_fwd(o, spec, zero_b), _fwd(o, plain, c))
    spec2 = o.MlpSpec(d_model=spec.d_model, d_ff=spec.d_ff, lora_rank=2, lora_alpha=3.0, lora_targets=TU | TD)
    assert not np.any(_fwd(o, spec2, dict(c, wg=np.zeros_like(c["wg"]))))
    spec3 = o.MlpSpec(d_model=spec.d_model, d_ff=spec.d_ff, lora_rank=2, lora_alpha=3.0, lora_targets=TG | TU)
    _close(_fwd(o, spec3, dict(c, wd=2.5 * c["wd"])), 2.5 * _fwd(o, spec3, c), 1e-13, "linear in W_d")
    rows = [4, 0, 0, 2]
    _close(o.mlp_forward_rows(spec, rows, c["h"], c["wg"], c["wu"], c["wd"], c["a"], c["b"]),
           _fwd(o, spec, c)[rows], 1e-14, "row subset")
    act = o.mlp_activation(spec, c["h"], c["wg"], c["wu"], c["a"], c["b"])
    _close(o.lora_linear(spec, act, c["wd"], c["a"][TD], c["b"][TD]), _fwd(o, spec, c), 1e-14,
           "activation then down projection")


ALL_CHECKS = [check_silu_closed_forms, check_silu_torch, check_mlp_brute_force, check_mlp_merged_weights,
              check_mlp_special_cases]
