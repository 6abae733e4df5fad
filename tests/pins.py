"""Checks that pin the CPU oracle to things other than itself.

Each ``check_*`` takes the oracle module and raises AssertionError (or any
exception) when the oracle disagrees with:

* closed forms of RMSNorm (RMS of the output, constant rows) and torch's own
  ``rms_norm`` in float64;
* special cases of LoRA (B = 0, W = 0) and the merged-weight formulation
  W + s B A, which is how a LoRA adapter is folded into its base layer;
* the rotation's closed forms, position 0, pair norms, the relative-position
  property and the complex-number (RoFormer) formulation of rotate-half RoPE;
* a scalar pure-Python brute force of the whole forward on tiny shapes;
* central finite differences of <dy, forward> for the backward.

They are used twice: by ``test_oracle_pins.py`` on the real oracle and by
``test_oracle_mutants.py`` on oracles with planted mistakes, each of which at
least one check must reject.
"""
from __future__ import annotations

import math

import numpy as np

TQ, TK, TV = 1, 2, 4


def tiny_case(o, seed=0, T=5, d=8, hq=2, hkv=1, D=4, r=2, alpha=3.0, targets=TQ | TK | TV,
              bias=True, theta=50.0, eps=1e-6, max_pos=9):
    """A small random problem (float64) with every feature switched on."""
    rng = np.random.default_rng(seed)
    spec = o.Spec(d_model=d, n_q_heads=hq, n_kv_heads=hkv, head_dim=D, lora_rank=r,
                  lora_alpha=alpha, lora_targets=targets, eps=eps, rope_theta=theta)
    N = spec.n_out
    x = rng.standard_normal((T, d))
    gamma = 1.0 + 0.3 * rng.standard_normal(d)
    w = rng.standard_normal((N, d)) / math.sqrt(d)
    b = 0.1 * rng.standard_normal(N) if bias else None
    a, bb = {}, {}
    for c in (TQ, TK, TV):
        if targets & c:
            lo, hi = spec.columns(c)
            a[c] = rng.standard_normal((r, d)) / math.sqrt(d)
            bb[c] = 0.5 * rng.standard_normal((hi - lo, r))
    pos = rng.integers(0, max_pos, size=T).astype(np.int32)
    return spec, dict(x=x, gamma=gamma, w=w, bias=b, a=a, b=bb, positions=pos)


def _fwd(o, spec, c):
    return o.forward(spec, c["x"], c["gamma"], c["w"], c["bias"], c["a"], c["b"], c["positions"])


def _close(got, want, tol, what):
    got, want = np.asarray(got, np.float64), np.asarray(want, np.float64)
    assert got.shape == want.shape, f"{what}: shape {got.shape} != {want.shape}"
    err = np.max(np.abs(got - want)) if got.size else 0.0
    scale = max(1.0, float(np.max(np.abs(want)))) if want.size else 1.0
    assert err <= tol * scale, f"{what}: max abs err {err:.3e} > {tol:.1e} x {scale:.3g}"


# --------------------------------------------------------------------------- RMSNorm

def check_rms_closed_form(o):
    """gamma = 1: the RMS of each output row is sqrt(ms / (ms + eps)); eps = 0 gives exactly 1."""
    rng = np.random.default_rng(1)
    x = rng.standard_normal((6, 32)) * np.array([1e-3, 0.1, 1, 3, 10, 100])[:, None]
    d = x.shape[1]
    for eps in (0.0, 1e-6, 1e-2):
        h = o.rms_normalise(x, np.ones(d), eps)
        ms = np.array([sum(v * v for v in row) / d for row in x])
        _close(np.sqrt(np.mean(h * h, axis=1)), np.sqrt(ms / (ms + eps)), 1e-12, f"RMS(h) eps={eps}")


def check_rms_constant_row(o):
    """x = c * ones gives h = c / sqrt(c^2 + eps) * gamma; a zero row gives h = 0 (no NaN)."""
    d, eps = 16, 1e-4
    gamma = np.linspace(0.5, 1.5, d)
    for cval in (0.0, 1e-3, -0.7, 2.0, 50.0):
        h = o.rms_normalise(np.full((1, d), cval), gamma, eps)
        _close(h[0], cval / math.sqrt(cval * cval + eps) * gamma, 1e-13, f"constant row {cval}")


def check_rms_torch(o):
    """Agrees with torch.nn.functional.rms_norm (float64, CPU)."""
    import torch
    rng = np.random.default_rng(2)
    x = rng.standard_normal((7, 24))
    g = 1 + 0.2 * rng.standard_normal(24)
    for eps in (1e-6, 0.5):
        ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (24,), weight=torch.from_numpy(g),
                                           eps=eps).numpy()
        _close(o.rms_normalise(x, g, eps), ref, 1e-13, "torch rms_norm")


def check_scale_invariance(o):
    """gamma -> lam*gamma with b = 0 scales the output by lam; x -> lam*x leaves it unchanged (eps=0)."""
    spec, c = tiny_case(o, seed=3, bias=False, eps=0.0)
    base = _fwd(o, spec, c)
    c2 = dict(c, gamma=2.5 * c["gamma"])
    _close(_fwd(o, spec, c2), 2.5 * base, 1e-12, "gamma scaling")
    c3 = dict(c, x=7.0 * c["x"])
    _close(_fwd(o, spec, c3), base, 1e-12, "x scaling")


# --------------------------------------------------------------------------- LoRA

def _no_lora(o, spec):
    return o.Spec(d_model=spec.d_model, n_q_heads=spec.n_q_heads, n_kv_heads=spec.n_kv_heads,
                  head_dim=spec.head_dim, eps=spec.eps, rope_theta=spec.rope_theta)


def check_lora_zero_b(o):
    """B = 0 (any A) gives exactly the base projection without adapters."""
    spec, c = tiny_case(o, seed=4)
    zb = {k: np.zeros_like(v) for k, v in c["b"].items()}
    with_zero = o.forward(spec, c["x"], c["gamma"], c["w"], c["bias"], c["a"], zb, c["positions"])
    base = o.forward(_no_lora(o, spec), c["x"], c["gamma"], c["w"], c["bias"], {}, {}, c["positions"])
    assert np.array_equal(with_zero, base), "B=0 must equal the base projection exactly"


def check_lora_merged_weight(o):
    """Adapters equal the merged weight W' = W + (alpha/r) B_c A_c on the target rows."""
    hq, hkv, D = 4, 2, 4
    rows = {TQ: slice(0, hq * D), TK: slice(hq * D, (hq + hkv) * D), TV: slice((hq + hkv) * D, (hq + 2 * hkv) * D)}
    for targets in (TQ, TK, TV, TQ | TV, TQ | TK | TV):
        spec, c = tiny_case(o, seed=5 + targets, targets=targets, hq=hq, hkv=hkv, D=D, r=3, alpha=6.0)
        wm = c["w"].copy()
        for t, A in c["a"].items():
            wm[rows[t]] += (6.0 / 3) * (c["b"][t] @ A)
        merged = o.forward(_no_lora(o, spec), c["x"], c["gamma"], wm, c["bias"], {}, {}, c["positions"])
        _close(_fwd(o, spec, c), merged, 1e-12, f"merged weight targets={targets}")


def check_lora_only(o):
    """W = 0, b = 0, positions 0: the output is (alpha/r) B (A h) on the target columns, 0 elsewhere."""
    spec, c = tiny_case(o, seed=6, targets=TQ | TV, bias=False)
    c = dict(c, w=np.zeros_like(c["w"]), positions=np.zeros_like(c["positions"]))
    out = _fwd(o, spec, c)
    x, g, eps = c["x"], c["gamma"], spec.eps
    want = np.zeros_like(out)
    for i in range(x.shape[0]):
        ms = sum(v * v for v in x[i]) / x.shape[1]
        hrow = [x[i, j] / math.sqrt(ms + eps) * g[j] for j in range(x.shape[1])]
        for t in (TQ, TV):
            lo, _ = spec.columns(t)
            A, B = c["a"][t], c["b"][t]
            u = [sum(A[k, j] * hrow[j] for j in range(len(hrow))) for k in range(A.shape[0])]
            for n in range(B.shape[0]):
                want[i, lo + n] = spec.lora_alpha / spec.lora_rank * sum(B[n, k] * u[k] for k in range(len(u)))
    _close(out, want, 1e-12, "LoRA-only output")


# --------------------------------------------------------------------------- RoPE

def check_rope_closed_form(o):
    """Head of size 2: omega = 1, so (1, 0) at position p becomes (cos p, sin p).
    Head of size 4, theta = 100: omega_1 = 0.1, so (0, 1, 0, 0) at position 10 becomes
    (0, cos 1, 0, sin 1) and (0, 0, 0, 1) becomes (0, -sin 1, 0, cos 1)."""
    for p in (0, 1, 2, 5, 100):
        y = o.rope_rotate(np.array([[1.0, 0.0]]), np.array([p]), 2, 10000.0)
        _close(y[0], [math.cos(p), math.sin(p)], 1e-13, f"D=2 pos={p}")
    y = o.rope_rotate(np.array([[0.0, 1.0, 0.0, 0.0], [0.0, 0.0, 0.0, 1.0]]), np.array([10, 10]), 4, 100.0)
    _close(y[0], [0.0, math.cos(1.0), 0.0, math.sin(1.0)], 1e-13, "D=4 e1")
    _close(y[1], [0.0, -math.sin(1.0), 0.0, math.cos(1.0)], 1e-13, "D=4 e3")


def check_rope_complex_form(o):
    """Equals multiplying z_i = y_i + i*y_{i+D/2} by exp(i * pos * theta^(-2i/D)) (RoFormer form)."""
    rng = np.random.default_rng(7)
    D, theta, nh = 8, 777.0, 3
    y = rng.standard_normal((5, nh * D))
    pos = np.array([0, 1, 3, 250, 8191])
    got = o.rope_rotate(y, pos, D, theta)
    want = np.empty_like(y)
    for t in range(5):
        for h in range(nh):
            seg = y[t, h * D:(h + 1) * D]
            z = seg[:D // 2] + 1j * seg[D // 2:]
            freq = np.exp(-np.log(theta) * np.arange(0, D, 2) / D)
            z = z * np.exp(1j * pos[t] * freq)
            want[t, h * D:(h + 1) * D] = np.concatenate([z.real, z.imag])
    _close(got, want, 1e-12, "complex form")
    back = o.rope_rotate(got, pos, D, theta, inverse=True)
    _close(back, y, 1e-12, "inverse rotation")


def check_rope_position_zero(o):
    """At position 0 the whole operator equals the unrotated projection (v included)."""
    spec, c = tiny_case(o, seed=8)
    c0 = dict(c, positions=np.zeros_like(c["positions"]))
    pre = o.pre_rope(spec, c["x"], c["gamma"], c["w"], c["bias"], c["a"], c["b"])
    assert np.array_equal(_fwd(o, spec, c0), pre), "position 0 must be the identity"


def check_rope_pair_norms_and_v(o):
    """Rotation keeps each (i, i+D/2) pair's norm on q and k heads and leaves v columns untouched."""
    spec, c = tiny_case(o, seed=9, hq=4, hkv=2, D=8, max_pos=5000)
    pre = o.pre_rope(spec, c["x"], c["gamma"], c["w"], c["bias"], c["a"], c["b"])
    out = _fwd(o, spec, c)
    D, half = spec.head_dim, spec.head_dim // 2
    nrot = (spec.n_q_heads + spec.n_kv_heads) * D
    for hs in range(0, nrot, D):
        for i in range(half):
            n_pre = np.hypot(pre[:, hs + i], pre[:, hs + i + half])
            n_out = np.hypot(out[:, hs + i], out[:, hs + i + half])
            _close(n_out, n_pre, 1e-12, "pair norm")
    assert np.array_equal(out[:, nrot:], pre[:, nrot:]), "v must not be rotated"
    assert not np.allclose(out[:, :nrot], pre[:, :nrot]), "q/k must be rotated"


def check_rope_relative(o):
    """q_m . k_n depends on m - n only: shifting every position leaves the q.k Gram matrix unchanged."""
    spec, c = tiny_case(o, seed=10, hq=2, hkv=1, D=8, T=6, max_pos=100, theta=1000.0)
    D = spec.head_dim
    grams = []
    for shift in (0, 17, 3000):
        out = _fwd(o, spec, dict(c, positions=c["positions"] + shift))
        q = out[:, 0:D]
        k = out[:, spec.n_q_heads * D: spec.n_q_heads * D + D]
        grams.append(q @ k.T)
    _close(grams[1], grams[0], 1e-11, "relative position (shift 17)")
    _close(grams[2], grams[0], 1e-10, "relative position (shift 3000)")


# --------------------------------------------------------------------------- brute force

def brute_forward(spec, c):
    """The whole forward as scalar loops (tiny shapes only)."""
    x, g, w, bias, A, B, pos = (c["x"], c["gamma"], c["w"], c["bias"], c["a"], c["b"], c["positions"])
    T, d = x.shape
    D, N = spec.head_dim, spec.n_out
    s = spec.lora_alpha / spec.lora_rank if spec.lora_rank else 0.0
    nq, nkv = spec.n_q_heads * D, spec.n_kv_heads * D
    blocks = {TQ: (0, nq), TK: (nq, nq + nkv), TV: (nq + nkv, nq + 2 * nkv)}
    out = [[0.0] * N for _ in range(T)]
    for t in range(T):
        ss = 0.0
        for j in range(d):
            ss += x[t][j] * x[t][j]
        inv = 1.0 / math.sqrt(ss / d + spec.eps)
        h = [x[t][j] * inv * g[j] for j in range(d)]
        y = [0.0] * N
        for n in range(N):
            acc = 0.0
            for j in range(d):
                acc += w[n][j] * h[j]
            y[n] = acc + (bias[n] if bias is not None else 0.0)
        for tg, (lo, hi) in blocks.items():
            if not (spec.lora_targets & tg):
                continue
            u = [sum(A[tg][k][j] * h[j] for j in range(d)) for k in range(spec.lora_rank)]
            for n in range(lo, hi):
                y[n] += s * sum(B[tg][n - lo][k] * u[k] for k in range(spec.lora_rank))
        for hs in range(0, nq + nkv, D):
            for i in range(D // 2):
                ang = pos[t] * spec.rope_theta ** (-(2.0 * i) / D)
                a_, b_ = y[hs + i], y[hs + i + D // 2]
                y[hs + i] = a_ * math.cos(ang) - b_ * math.sin(ang)
                y[hs + i + D // 2] = b_ * math.cos(ang) + a_ * math.sin(ang)
        out[t] = y
    return np.array(out)


def check_brute_force(o):
    """The vectorised oracle equals scalar loops on tiny shapes (GQA, MHA, each target subset)."""
    cases = [dict(seed=11), dict(seed=12, hq=4, hkv=2, targets=TQ | TV, bias=False),
             dict(seed=13, hq=2, hkv=2, D=6, targets=TK, r=1), dict(seed=14, targets=0, r=0, alpha=0.0),
             dict(seed=15, T=1, d=4, hq=1, hkv=1, D=2, r=4, targets=TV, max_pos=3)]
    for kw in cases:
        spec, c = tiny_case(o, **kw)
        _close(_fwd(o, spec, c), brute_forward(spec, c), 1e-12, f"brute force {kw}")


# --------------------------------------------------------------------------- row subsets, chunks

def check_forward_rows(o):
    """forward_rows (the reference of every sampled-row GPU check) equals the scalar brute force
    on exactly the rows asked for, in the order asked for -- unsorted and repeated rows included
    -- so each row keeps its own position; and it equals forward()[rows] to within rounding (BLAS
    picks a different kernel for a different row count, so the last bits may differ)."""
    spec, c = tiny_case(o, seed=21, T=9, max_pos=300)
    full = brute_forward(spec, c)
    for rows in ([0], [8, 3, 3, 0, 5], list(range(9))[::-1], [4, 4, 4]):
        got = o.forward_rows(spec, rows, c["x"], c["gamma"], c["w"], c["bias"], c["a"], c["b"], c["positions"])
        _close(got, full[rows], 1e-12, f"forward_rows {rows} vs brute force")
        _close(got, _fwd(o, spec, c)[rows], 1e-14, f"forward_rows {rows} vs forward()[rows]")


def check_forward_chunked(o):
    """forward_chunked (the reference of every full-output GPU check) equals the scalar brute
    force on every row, for chunk lengths that leave a ragged last chunk (10 rows in chunks of
    3), one chunk per row, and a single chunk longer than T."""
    spec, c = tiny_case(o, seed=22, T=10, max_pos=500)
    full = brute_forward(spec, c)
    for chunk in (3, 1, 4, 64):
        got = o.forward_chunked(spec, c["x"], c["gamma"], c["w"], c["bias"], c["a"], c["b"], c["positions"],
                                chunk=chunk)
        _close(got, full, 1e-12, f"forward_chunked chunk={chunk} vs brute force")


# --------------------------------------------------------------------------- backward

def check_backward_finite_differences(o):
    """dx, dA, dB equal central finite differences of L = <dy, forward> (float64)."""
    spec, c = tiny_case(o, seed=16, T=3, d=6, hq=2, hkv=1, D=4, r=2, targets=TQ | TV, max_pos=40)
    rng = np.random.default_rng(17)
    dy = rng.standard_normal((3, spec.n_out))

    def loss(cc):
        return float(np.sum(dy * _fwd(o, spec, cc)))

    dx, dA, dB = o.backward(spec, c["x"], c["gamma"], c["w"], c["bias"], c["a"], c["b"], c["positions"], dy)
    step = 1e-6

    def fd(get, put):
        base = get()
        g = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            plus, minus = base.copy(), base.copy()
            plus[idx] += step
            minus[idx] -= step
            g[idx] = (loss(put(plus)) - loss(put(minus))) / (2 * step)
        return g

    _close(dx, fd(lambda: c["x"], lambda v: dict(c, x=v)), 1e-7, "dx")
    for t in c["a"]:
        _close(dA[t], fd(lambda: c["a"][t], lambda v: dict(c, a={**c["a"], t: v})), 1e-7, f"dA[{t}]")
        _close(dB[t], fd(lambda: c["b"][t], lambda v: dict(c, b={**c["b"], t: v})), 1e-7, f"dB[{t}]")
    # row subset gives the same rows
    dx_sub, _, _ = o.backward(spec, c["x"], c["gamma"], c["w"], c["bias"], c["a"], c["b"], c["positions"],
                              dy, dx_rows=[2, 0])
    _close(dx_sub, dx[[2, 0]], 1e-13, "dx row subset")


def check_kv_cache_by_hand(o):
    """Cache rows after a forward call writes its keys and values, written out by hand: 2 q heads,
    1 kv head, head size 2 (columns q 0..3 | k 4, 5 | v 6, 7), four tokens, a cache of four rows
    filled with -1.  Token 1 has a negative slot and token 3 a slot past the cache: neither is
    written; rows 1 and 3 keep their old values; the caches passed in are not modified."""
    spec = o.Spec(d_model=4, n_q_heads=2, n_kv_heads=1, head_dim=2)
    out = np.arange(32, dtype=np.float64).reshape(4, 8)
    k0, v0 = -np.ones((4, 2)), -np.ones((4, 2))
    kc, vc = o.kv_cache_write(spec, out, [2, -1, 0, 5], k0, v0)
    assert np.asarray(kc).tolist() == [[20.0, 21.0], [-1.0, -1.0], [4.0, 5.0], [-1.0, -1.0]]
    assert np.asarray(vc).tolist() == [[22.0, 23.0], [-1.0, -1.0], [6.0, 7.0], [-1.0, -1.0]]
    assert (k0 == -1.0).all() and (v0 == -1.0).all()


# --------------------------------------------------------------------------- LoRA dropout

def check_philox_known_answers(o):
    """Philox4x32-10 against the known-answer vectors published with the generator's reference
    implementation (Random123): zero counter and key; all-ones counter and key; the digits of
    pi as counter and key."""
    cases = [((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
             ((0xFFFFFFFF,) * 4, (0xFFFFFFFF, 0xFFFFFFFF), (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
             ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
              (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1))]
    for ctr, key, want in cases:
        got = [int(v) for v in o.philox4x32_10(np.array(ctr, dtype=np.uint64), key)]
        assert got == list(want), (ctr, [hex(g) for g in got])


def check_dropout_mask_by_hand(o):
    """Seed 0, offset 0, target q, row 0: features 0..3 use counter (0, 0, 0, 0) and key (0, 0),
    whose words are the first known answer above; with p = 1/2 (threshold 2^31) word
    0x6627e8d5 drops feature 0 and the other three keep theirs; with p = 0.1 all four are kept;
    p = 0 keeps everything."""
    assert o.dropout_threshold(0.5) == 2 ** 31 and o.dropout_threshold(0.0) == 0
    assert o.dropout_keep(1, 4, 0, 0.5, 0, 0).tolist() == [[False, True, True, True]]
    assert o.dropout_keep(1, 4, 0, 0.1, 0, 0).tolist() == [[True, True, True, True]]
    assert o.dropout_keep(3, 10, 2, 0.0, 5, 9).all()


def check_dropout_statistics(o):
    """Keep rate within 5 standard deviations of 1 - p over 2^19 features; the masks of the
    three adapters, and of two offsets, are different (and equal for equal arguments); a row
    subset gets exactly the rows of the full mask."""
    n = 512 * 1024
    for p in (0.05, 0.1, 0.5):
        keep = o.dropout_keep(512, 1024, 1, p, 1234567890123, 77)
        sd = math.sqrt(p * (1 - p) / n)
        assert abs(keep.mean() - (1 - p)) < 5 * sd, (p, keep.mean())
    m = [o.dropout_keep(64, 256, t, 0.3, 42, 5) for t in range(3)]
    assert not np.array_equal(m[0], m[1]) and not np.array_equal(m[1], m[2])
    assert not np.array_equal(m[0], o.dropout_keep(64, 256, 0, 0.3, 42, 6))
    assert np.array_equal(m[0], o.dropout_keep(64, 256, 0, 0.3, 42, 5))
    assert np.array_equal(o.dropout_keep(64, 256, 0, 0.3, 42, 5, rows=[63, 7, 7]), m[0][[63, 7, 7]])


def brute_forward_masked(spec, c, inputs):
    """brute_forward with each adapter's input given explicitly (a dict target -> [T, d])."""
    x, g, w, bias, A, B, pos = (c["x"], c["gamma"], c["w"], c["bias"], c["a"], c["b"], c["positions"])
    T, d = x.shape
    D, N = spec.head_dim, spec.n_out
    s = spec.lora_alpha / spec.lora_rank if spec.lora_rank else 0.0
    nq, nkv = spec.n_q_heads * D, spec.n_kv_heads * D
    blocks = {TQ: (0, nq), TK: (nq, nq + nkv), TV: (nq + nkv, nq + 2 * nkv)}
    out = []
    for t in range(T):
        inv = 1.0 / math.sqrt(sum(x[t][j] * x[t][j] for j in range(d)) / d + spec.eps)
        h = [x[t][j] * inv * g[j] for j in range(d)]
        y = [sum(w[n][j] * h[j] for j in range(d)) + (bias[n] if bias is not None else 0.0) for n in range(N)]
        for tg, (lo, hi) in blocks.items():
            if spec.lora_targets & tg:
                hin = inputs[tg][t]
                u = [sum(A[tg][k][j] * hin[j] for j in range(d)) for k in range(spec.lora_rank)]
                for n in range(lo, hi):
                    y[n] += s * sum(B[tg][n - lo][k] * u[k] for k in range(spec.lora_rank))
        for hs in range(0, nq + nkv, D):
            for i in range(D // 2):
                ang = pos[t] * spec.rope_theta ** (-(2.0 * i) / D)
                a_, b_ = y[hs + i], y[hs + i + D // 2]
                y[hs + i] = a_ * math.cos(ang) - b_ * math.sin(ang)
                y[hs + i + D // 2] = b_ * math.cos(ang) + a_ * math.sin(ang)
        out.append(y)
    return np.array(out)


def check_dropout_forward(o):
    """With dropout the forward equals scalar loops fed each adapter's masked, rescaled copy of h
    (the frozen projection sees h itself); p = 0 equals the no-dropout forward bit for bit; a
    row subset and chunks use the rows' own masks."""
    spec, c = tiny_case(o, seed=31, T=6, d=12)
    drop = o.Dropout(p=0.4, seed=987654321, offset=3)
    h = o.rms_normalise(c["x"], c["gamma"], spec.eps)
    inputs = {}
    for i, tg in enumerate((TQ, TK, TV)):
        keep = [[None] * 12 for _ in range(6)]
        km = o.dropout_keep(6, 12, i, 0.4, 987654321, 3)
        inputs[tg] = [[h[t][j] * (1.0 if km[t][j] else 0.0) / 0.6 for j in range(12)] for t in range(6)]
        del keep
    got = o.forward(spec, c["x"], c["gamma"], c["w"], c["bias"], c["a"], c["b"], c["positions"], drop)
    _close(got, brute_forward_masked(spec, c, inputs), 1e-12, "dropout brute force")
    assert np.array_equal(o.forward(spec, c["x"], c["gamma"], c["w"], c["bias"], c["a"], c["b"], c["positions"],
                                    o.Dropout(0.0, 99, 1)), _fwd(o, spec, c))
    rows = [5, 1, 1]
    _close(o.forward_rows(spec, rows, c["x"], c["gamma"], c["w"], c["bias"], c["a"], c["b"], c["positions"], drop),
           got[rows], 1e-14, "dropout row subset")
    _close(o.forward_chunked(spec, c["x"], c["gamma"], c["w"], c["bias"], c["a"], c["b"], c["positions"], chunk=4,
                             dropout=drop), got, 1e-14, "dropout chunks")


def check_dropout_backward_finite_differences(o):
    """dx, dA, dB with dropout equal central finite differences of <dy, forward> at the same
    (fixed) masks; p = 0 gives the no-dropout gradients bit for bit."""
    spec, c = tiny_case(o, seed=32, T=3, d=8, hq=2, hkv=1, D=4, r=2, targets=TQ | TK | TV, max_pos=40)
    drop = o.Dropout(p=0.3, seed=2024, offset=11)
    dy = np.random.default_rng(33).standard_normal((3, spec.n_out))

    def loss(cc):
        return float(np.sum(dy * o.forward(spec, cc["x"], cc["gamma"], cc["w"], cc["bias"], cc["a"], cc["b"],
                                           cc["positions"], drop)))

    dx, dA, dB = o.backward(spec, c["x"], c["gamma"], c["w"], c["bias"], c["a"], c["b"], c["positions"], dy,
                            dropout=drop)
    step = 1e-6

    def fd(get, put):
        base = get()
        g = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            plus, minus = base.copy(), base.copy()
            plus[idx] += step
            minus[idx] -= step
            g[idx] = (loss(put(plus)) - loss(put(minus))) / (2 * step)
        return g

    _close(dx, fd(lambda: c["x"], lambda v: dict(c, x=v)), 1e-7, "dropout dx")
    for t in c["a"]:
        _close(dA[t], fd(lambda: c["a"][t], lambda v: dict(c, a={**c["a"], t: v})), 1e-7, f"dropout dA[{t}]")
        _close(dB[t], fd(lambda: c["b"][t], lambda v: dict(c, b={**c["b"], t: v})), 1e-7, f"dropout dB[{t}]")
    dx_sub, _, _ = o.backward(spec, c["x"], c["gamma"], c["w"], c["bias"], c["a"], c["b"], c["positions"], dy,
                              dx_rows=[2, 0], dropout=drop)
    _close(dx_sub, dx[[2, 0]], 1e-13, "dropout dx row subset")
    plain = o.backward(spec, c["x"], c["gamma"], c["w"], c["bias"], c["a"], c["b"], c["positions"], dy)
    zero = o.backward(spec, c["x"], c["gamma"], c["w"], c["bias"], c["a"], c["b"], c["positions"], dy,
                      dropout=o.Dropout(0.0, 5, 5))
    assert np.array_equal(plain[0], zero[0])


ALL_CHECKS = [check_rms_closed_form, check_rms_constant_row, check_rms_torch, check_scale_invariance,
              check_lora_zero_b, check_lora_merged_weight, check_lora_only,
              check_rope_closed_form, check_rope_complex_form, check_rope_position_zero,
              check_rope_pair_norms_and_v, check_rope_relative, check_brute_force,
              check_forward_rows, check_forward_chunked,
              check_backward_finite_differences, check_kv_cache_by_hand,
              check_philox_known_answers, check_dropout_mask_by_hand, check_dropout_statistics,
              check_dropout_forward, check_dropout_backward_finite_differences]
