"""Checks that pin the NF4 (QLoRA base) oracle to things other than itself: the code book
against its construction from quantiles of the normal distribution (scipy), the quantiser
against a scalar nearest-level search, the fixed tie rule on exact midpoints, the block
structure, the stored byte layout written out by hand, and the dequantised forward against
scalar loops.  Used by ``test_qlora_oracle.py`` on the real oracle and on planted mistakes."""
from __future__ import annotations

import math

import numpy as np

import pins


def _bf16(a):
    """Round float64 values to bfloat16 (round to nearest even), returned as float32."""
    import torch
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).float().numpy()


def check_levels_against_construction(q):
    """The code book: 16 increasing values with -1, an exact 0 at code 7 and +1; 8 positive and
    7 negative levels; each within two float32 ulps of the construction from N(0, 1) quantiles
    (delta = (1/32 + 1/30) / 2)."""
    lv = q.NF4_LEVELS.astype(np.float64)
    assert lv.shape == (16,) and np.all(np.diff(lv) > 0)
    assert lv[0] == -1.0 and lv[q.ZERO_CODE] == 0.0 and lv[15] == 1.0
    assert np.sum(lv > 0) == 8 and np.sum(lv < 0) == 7
    from scipy.stats import norm
    delta = 0.5 * (1.0 / 32.0 + 1.0 / 30.0)
    pos = norm.ppf(0.5 + (0.5 - delta) * np.arange(8, 0, -1) / 8.0)
    neg = -norm.ppf(0.5 + (0.5 - delta) * np.arange(7, 0, -1) / 7.0)
    ref = np.sort(np.concatenate([pos, [0.0], neg])) / norm.ppf(1.0 - delta)
    assert np.max(np.abs(lv - ref)) <= 2.4e-7, np.max(np.abs(lv - ref))


def _nearest_ok(y, code, lv):
    """code is a nearest level to y (up to the float32 rounding of the midpoints)."""
    dist = abs(y - lv[code])
    return all(dist <= abs(y - lv[j]) + 1e-7 for j in range(16))


def check_quantize_nearest_level(q):
    """Every code is a nearest code-book value to w / absmax of its block (scalar search), the
    scale is the block's largest magnitude, and blocks are independent of one another."""
    rng = np.random.default_rng(11)
    w = _bf16(rng.standard_normal((3, 192)) * 0.02)
    w[1, 64:128] *= 40.0          # one block much larger than its neighbours
    codes, scales = q.quantize(w)
    lv = q.NF4_LEVELS.astype(np.float64)
    for r in range(w.shape[0]):
        for blk in range(w.shape[1] // 64):
            seg = w[r, 64 * blk:64 * (blk + 1)]
            a = max(abs(float(v)) for v in seg)
            assert scales[r, blk] == np.float32(a)
            for k, v in enumerate(seg):
                y = float(np.float32(v) / np.float32(a))
                assert _nearest_ok(y, int(codes[r, 64 * blk + k]), lv), (r, blk, k)
    # changing one block leaves the others' codes and scales alone
    w2 = w.copy()
    w2[0, :64] = 0.5
    c2, s2 = q.quantize(w2)
    assert np.array_equal(c2[:, 64:], codes[:, 64:]) and np.array_equal(s2[:, 1:], scales[:, 1:])
    assert np.array_equal(c2[1:], codes[1:])


def check_quantize_ties_and_special_blocks(q):
    """Exact float32 midpoints (absmax 1) take the lower level; the largest magnitude of a block
    maps to -1 or +1 and dequantises exactly; an all-zero block gives code 7 and scale 0; zero
    weights give code 7 whatever the block."""
    lv = q.NF4_LEVELS.astype(np.float32)
    mids = ((lv[:-1] + lv[1:]) * np.float32(0.5)).astype(np.float32)
    row = np.zeros(64, np.float32)
    row[:15] = mids
    row[15] = 1.0
    row[16] = -0.75
    w = np.stack([row, np.zeros(64, np.float32)])
    codes, scales = q.quantize(w)
    assert list(codes[0, :15]) == list(range(15)), codes[0, :15]
    assert codes[0, 15] == 15 and scales[0, 0] == 1.0
    assert codes[0, 17] == q.ZERO_CODE
    assert np.all(codes[1] == q.ZERO_CODE) and scales[1, 0] == 0.0
    deq = q.dequantize(codes, scales)
    assert deq[0, 15] == 1.0 and np.all(deq[1] == 0.0)
    neg = np.zeros((1, 64), np.float32)
    neg[0, 3] = -2.5
    c3, s3 = q.quantize(neg)
    assert c3[0, 3] == 0 and q.dequantize(c3, s3)[0, 3] == -2.5


def check_quantize_error_bound(q):
    """|w - dequant(quant(w))| <= absmax * (largest gap between levels) / 2 elementwise."""
    rng = np.random.default_rng(5)
    w = _bf16(rng.standard_normal((8, 256)))
    codes, scales = q.quantize(w)
    deq = q.dequantize(codes, scales)
    gap = float(np.max(np.diff(q.NF4_LEVELS.astype(np.float64))))
    bound = np.repeat(scales.astype(np.float64), 64, axis=1) * gap / 2 * (1 + 1e-6)
    assert np.all(np.abs(w - deq) <= bound)


def check_pack_layout(q):
    """Byte layout written out by hand: weight 2i in the low nibble of byte i, 2i + 1 in the
    high nibble; the scales start at the codes' size rounded up to 256 bytes."""
    codes = np.zeros((2, 64), np.uint8)
    codes[0, 0], codes[0, 1], codes[0, 2], codes[0, 3] = 1, 2, 15, 0
    codes[1, 62], codes[1, 63] = 9, 6
    scales = np.array([[0.5], [3.0]], np.float32)
    buf = q.pack(codes, scales)
    assert buf.size == 256 + 8 == q.stored_size(2, 64)
    assert buf[0] == 0x21 and buf[1] == 0x0F and buf[63] == 0x69
    assert np.array_equal(buf[256:264].view(np.float32), scales.reshape(-1))
    c2, s2 = q.unpack(buf, 2, 64)
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales)


def check_forward_on_dequantised_base(q):
    """The NF4-base forward equals the operator on W built by scalar loops from codes and
    scales (tiny case, every adapter, bias)."""
    from oracle import lrq_oracle as o
    spec, c = pins.tiny_case(o, T=3, d=64, hq=2, hkv=1, D=8, r=2, targets=7, bias=True)
    c["dy"] = np.random.default_rng(9).standard_normal((3, spec.n_out))
    codes, scales = q.quantize(_bf16(c["w"]))
    lv = [float(v) for v in q.NF4_LEVELS]
    n, d = codes.shape
    wq = np.array([[lv[int(codes[i, k])] * float(scales[i, k // 64]) for k in range(d)] for i in range(n)])
    got = q.forward(spec, c["x"], c["gamma"], codes, scales, c["bias"], c["a"], c["b"], c["positions"])
    want = o.forward(spec, c["x"], c["gamma"], wq, c["bias"], c["a"], c["b"], c["positions"])
    assert np.max(np.abs(got - want)) <= 1e-13 * max(1.0, float(np.max(np.abs(want))))
    dx, da, db = q.backward(spec, c["x"], c["gamma"], codes, scales, c["bias"], c["a"], c["b"], c["positions"], c["dy"])
    dx2, da2, db2 = o.backward(spec, c["x"], c["gamma"], wq, c["bias"], c["a"], c["b"], c["positions"], c["dy"])
    assert np.max(np.abs(dx - dx2)) <= 1e-13 * max(1.0, float(np.max(np.abs(dx2))))
    assert math.isfinite(float(np.sum(dx)))


ALL_CHECKS = [check_levels_against_construction, check_quantize_nearest_level, check_quantize_ties_and_special_blocks,
              check_quantize_error_bound, check_pack_layout, check_forward_on_dequantised_base]
