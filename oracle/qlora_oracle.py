"""Oracle of the QLoRA base: the frozen W_qkv stored as 4-bit NormalFloat (NF4) blocks, with
the LoRA adapters and everything else of the operator unchanged.  Test infrastructure: only
tests/, the smoke check and the benchmark's CPU baseline import it.

The pages name QLoRA as one of the fine-tuning settings the fused kernels serve (page
"Liger-Kernel内核级优化：GPU利用率飙升至90%以上", opening section; page "Swift-All一文详解：
如何用Liger-Kernel提升训练效率", section 2.3, the Qwen-VL-Chat QLoRA row of the table; page
"Liger-Kernel底层优化：新一代内核级推理加速引擎深度解析", system-integration section) but never
define the stored format.  Reading (R-Q1): the format of the QLoRA paper (Dettmers, Pagnoni,
Holtzman and Zettlemoyer, "QLoRA: Efficient Finetuning of Quantized LLMs", NeurIPS 2023):
  * NF4 code book: the 16 values of the 4-bit NormalFloat data type, as the paper publishes
    them (its appendix); they come from quantiles of N(0, 1): 8 positive levels at evenly
    spaced probabilities from 1 - delta down to 1/2 (exclusive), 7 negative ones the same way
    with one point fewer, an exact zero, all divided by the largest, delta = (1/32 + 1/30) / 2.
    The pins check the table against that construction (scipy's normal quantile function).
  * blocks of 64 consecutive weights along d (each row of W [N, d] separately), one float32
    scale per block: its largest magnitude (absmax); no second-level quantisation of the
    scales (the paper's "double quantisation" is a memory option, left out).
  * dequantised weight = code book value * block scale; the frozen projection uses it in
    place of W (LoRA factors, RMSNorm, bias and RoPE are untouched).
Reading (R-Q2) of the quantiser, fixed so that every implementation takes the same integer
decision: in float32, y = w / absmax (correctly rounded); the code is the number of midpoints
m_i = (L_i + L_{i+1}) / 2 (float32 sum, halved) that y exceeds, so an exact tie goes to the
lower level; a block whose absmax is 0 gets code 7 (the zero) and scale 0.
Storage (R-Q3, the library's): codes [N, d / 2] bytes, weight k of a row in the low nibble of
byte k / 2 when k is even and in the high nibble when k is odd; then the scales [N, d / 64]
float32, starting at the codes' size rounded up to 256 bytes.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

BLOCK = 64
ZERO_CODE = 7

# The NF4 code book as published with the QLoRA paper (float32 values).
NF4_LEVELS = np.array([
    -1.0, -0.6961928009986877, -0.5250730514526367, -0.39491748809814453,
    -0.28444138169288635, -0.18477343022823334, -0.09105003625154495, 0.0,
    0.07958029955625534, 0.16093020141124725, 0.24611230194568634, 0.33791524171829224,
    0.44070982933044434, 0.5626170039176941, 0.7229568362236023, 1.0], dtype=np.float32)


def nf4_construction(delta: float = 0.5 * (1.0 / 32.0 + 1.0 / 30.0)) -> np.ndarray:
    """The code book from its definition: quantiles of N(0, 1), normalised to [-1, 1]."""
    from scipy.stats import norm
    top = 1.0 - delta
    pos = norm.ppf(np.linspace(top, 0.5, 9)[:-1])      # 8 positive levels
    neg = -norm.ppf(np.linspace(top, 0.5, 8)[:-1])     # 7 negative levels
    v = np.sort(np.concatenate([pos, [0.0], neg]))
    return v / v.max()


def midpoints(levels=None) -> np.ndarray:
    """float32 decision thresholds between consecutive levels (R-Q2)."""
    lv = (NF4_LEVELS if levels is None else levels).astype(np.float32)
    return ((lv[:-1] + lv[1:]) * np.float32(0.5)).astype(np.float32)


def quantize(w: np.ndarray, levels=None) -> Tuple[np.ndarray, np.ndarray]:
    """W [N, d] (values exact in float32) -> (codes [N, d] uint8 in 0..15, scales [N, d / 64]
    float32), by R-Q2."""
    w = np.asarray(w, dtype=np.float32)
    n, d = w.shape
    assert d % BLOCK == 0, "d must be a multiple of 64"
    blocks = w.reshape(n, d // BLOCK, BLOCK)
    absmax = np.max(np.abs(blocks), axis=2).astype(np.float32)
    safe = np.where(absmax > 0, absmax, np.float32(1.0)).astype(np.float32)
    y = (blocks / safe[:, :, None]).astype(np.float32)
    codes = np.sum(y[..., None] > midpoints(levels)[None, None, None, :], axis=-1).astype(np.uint8)
    codes = np.where(absmax[:, :, None] > 0, codes, np.uint8(ZERO_CODE)).astype(np.uint8)
    return codes.reshape(n, d), absmax


def dequantize(codes: np.ndarray, scales: np.ndarray, levels=None) -> np.ndarray:
    """float64 weights: level of each code times its block's scale."""
    codes = np.asarray(codes)
    n, d = codes.shape
    table = (NF4_LEVELS if levels is None else levels).astype(np.float64)
    lv = table[codes.astype(np.int64)].reshape(n, d // BLOCK, BLOCK)
    return (lv * np.asarray(scales, np.float64)[:, :, None]).reshape(n, d)


def pack(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """The stored buffer of R-Q3 as bytes."""
    codes = np.asarray(codes, dtype=np.uint8)
    n, d = codes.shape
    body = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8).reshape(-1)
    off = (body.size + 255) // 256 * 256
    out = np.zeros(off + scales.size * 4, dtype=np.uint8)
    out[:body.size] = body
    out[off:] = np.ascontiguousarray(scales, dtype=np.float32).reshape(-1).view(np.uint8)
    return out


def unpack(buf: np.ndarray, n: int, d: int) -> Tuple[np.ndarray, np.ndarray]:
    """Inverse of pack: (codes [N, d], scales [N, d / 64])."""
    buf = np.asarray(buf, dtype=np.uint8)
    nbody = n * d // 2
    body = buf[:nbody].reshape(n, d // 2)
    codes = np.empty((n, d), dtype=np.uint8)
    codes[:, 0::2] = body & 0x0F
    codes[:, 1::2] = body >> 4
    off = (nbody + 255) // 256 * 256
    scales = buf[off:off + n * (d // BLOCK) * 4].view(np.float32).reshape(n, d // BLOCK)
    return codes, scales


def stored_size(n: int, d: int) -> int:
    """Bytes of the stored buffer of an [n, d] weight."""
    return (n * d // 2 + 255) // 256 * 256 + n * (d // BLOCK) * 4


def forward(spec, x, gamma, codes, scales, bias, a, b, positions, dropout=None, rows=None):
    """The operator with the NF4 base: the dense oracle on the dequantised W."""
    from oracle import lrq_oracle as o
    return o.forward(spec, x, gamma, dequantize(codes, scales), bias, a, b, positions, dropout=dropout, rows=rows)


def backward(spec, x, gamma, codes, scales, bias, a, b, positions, dy, dx_rows=None, dropout=None):
    """Gradients with the NF4 base (frozen, as in QLoRA): the dense oracle on the dequantised W."""
    from oracle import lrq_oracle as o
    return o.backward(spec, x, gamma, dequantize(codes, scales), bias, a, b, positions, dy, dx_rows=dx_rows,
                      dropout=dropout)
