"""NumPy oracle of the W4A16 weight variant. TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this module. It shares no code, tables or constants with the
HIP library under ``moe_token_amax_amd/``.

Page: [LOWBIT] "超大 MoE 的低比特推理：INT4、FP4 与量化感知训练". What the page
fixes: the INT4 weight format with one BF16 scale per 32 weights (0.5 + 2/32
bytes per parameter, "4 比特对万亿 MoE 意味着什么"); the quantizer of its QAT
section ("为什么要量化感知训练"): symmetric, one group per G = 32 input
channels, scale = group amax / 7, codes = round(w / scale) clamped to
[-8, 7]; and the W4A16 kernel row of "不同硬件上的 kernel": the weights are
dequantized to BF16 in registers and multiplied by BF16 matrix units, which
pays off for decode, where reading the weights is the bound.

Readings (the page gives the recipe, not the rounding of a stored format):
  * the scale is stored as BF16: s = BF16(fl32(amax / 7)), round half to even;
    the codes are taken against the stored scale: q = clamp(rint(fl32(w / s)),
    -8, 7) (IEEE fp32 division, ties to even as the page's round); a group
    with amax 0 gets s = 0 and q = 0;
  * dequantization: w_deq = BF16(q * s) (q * s is exact in fp32), round half
    to even;
  * the linear: y[m, n] = BF16 of the exact sum over k of x[m, k] w_deq[n, k]
    (float64 here; the GPU accumulates the exact BF16 products in fp32 and is
    compared within a derived tolerance); no bias.

Parity status (tests/test_oracle_w4a16_pins.py): the quantizer pinned by hand
groups (exact scales, ties to even, the clamp, a BF16-rounded scale, the zero
group), by exact-rational recomputation and by the half-step error bound; the
dequantization by exact recomputation; the linear by brute force.
"""

from __future__ import annotations

import numpy as np

from .w8a8_ref import bf16_to_f32, f32_to_bf16

__all__ = ["W4_GROUP", "w4_quant", "w4_dequant", "w4a16_linear_ref64"]

W4_GROUP = 32


def w4_quant(w_bits):
    """BF16 weight [N, K] (K % 32 == 0) -> (codes int8 [N, K] in [-8, 7],
    scales as BF16 bits [N, K / 32])."""
    w = bf16_to_f32(w_bits)
    N, K = w.shape
    if K % W4_GROUP:
        raise ValueError("K must be a multiple of 32")
    g = w.reshape(N, K // W4_GROUP, W4_GROUP)
    amax = np.max(np.abs(g), axis=2).astype(np.float32)
    s_bits = f32_to_bf16((amax / np.float32(7.0)).astype(np.float32))
    s = bf16_to_f32(s_bits)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (g / s[:, :, None]).astype(np.float32)             # one fp32 division each
    q = np.clip(np.rint(t), -8, 7)
    q = np.where(s[:, :, None] > 0, q, 0).astype(np.int8)
    return q.reshape(N, K), s_bits


def w4_dequant(q, s_bits):
    """BF16 bits of q * s, per group of 32 along K."""
    q = np.asarray(q, np.int8)
    N, K = q.shape
    s = bf16_to_f32(s_bits)
    prod = (q.reshape(N, K // W4_GROUP, W4_GROUP).astype(np.float32) * s[:, :, None]).astype(np.float32)
    return f32_to_bf16(prod.reshape(N, K))


def w4a16_linear_ref64(x_bits, q, s_bits):
    """float64 sum over k of x[m, k] * BF16(q * s)[n, k]."""
    x = bf16_to_f32(x_bits).astype(np.float64)
    w = bf16_to_f32(w4_dequant(q, s_bits)).astype(np.float64)
    return x @ w.T
