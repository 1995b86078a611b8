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

FP4 weights (the same W4A16 row lists "INT4 / FP4"; MXFP4 = one E8M0 scale
per 32 values, 0.5 + 1/32 bytes per parameter): E2M1 values (1 sign, 2
exponent bits with bias 1, 1 mantissa bit: magnitudes 0, 0.5, 1, 1.5, 2, 3,
4, 6). Readings, as for the MXFP8 variant's rule 0: the shared exponent of a
group of 32 along K is E = floor(log2 amax) - 2 (2 is E2M1's largest
exponent), clamped to [-127, 127], byte E + 127; amax 0 gives byte 0 and zero
codes; each value w / 2^E (exact) is encoded to the nearest E2M1 value, ties
to the even code, saturating at 6, the sign kept (-0 is code 8). The
dequantized weight 2^E * value is exact in BF16.

MoE form (the same kernel row: the grouped expert matmul takes the low-bit
expert weights). Readings: rows grouped by expert as on the INT8 path
(group_list = rows per expert, [DSV4] §三); activations stay BF16 (A16): the
W13 output h is rounded once to BF16 (through fp32), the SwiGLU output a =
BF16(silu(gate) * up) by the fixed fp32 sequence of ``w8a8_ref.swiglu``, and
the W2 output is compared as the dense linear's; no requant between them.

Parity status (tests/test_oracle_w4a16_pins.py): the INT4 quantizer pinned by
hand groups (exact scales, ties to even, the clamp, a BF16-rounded scale, the
zero group), by exact-rational recomputation and by the half-step error bound;
the dequantization by exact recomputation; the linear by brute force. The FP4
quantizer by hand groups (every tie), an exhaustive nearest-value search and
the half-step bound; its dequantization and linear by brute force. The grouped
form by brute force per expert on the page's row counts 12/7/0/19 (an empty
expert included), the SwiGLU by hand values (signed zero, overflowing exp), and
the chain stage by stage against brute force.
"""

from __future__ import annotations

import numpy as np

from .w8a8_ref import bf16_to_f32, f32_to_bf16, group_offsets, swiglu

__all__ = ["W4_GROUP", "w4_quant", "w4_dequant", "w4a16_linear_ref64", "E2M1_VALUES", "fp4_quant",
           "fp4_dequant", "fp4_linear_ref64", "lowbit_dequant", "lowbit_grouped_ref64",
           "lowbit_swiglu", "lowbit_moe"]

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


# E2M1 magnitudes by code (bits e1 e0 m): exponent field 0 is subnormal (m * 0.5)
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _e2m1_encode(t):
    """float64 values -> E2M1 codes (uint8 0..15): nearest magnitude, ties to the
    even code, saturating at 6, sign bit 8."""
    t = np.asarray(t, np.float64)
    a = np.minimum(np.abs(t), 6.0)
    d = np.abs(a[..., None] - E2M1_VALUES)            # distance to every magnitude
    best = d.min(axis=-1, keepdims=True)
    tie = d == best
    # among the nearest, the even code (mantissa bit 0) when there are two
    idx = np.arange(8)
    even_pick = np.where(tie & (idx % 2 == 0), idx, 99).min(axis=-1)
    any_pick = np.where(tie, idx, 99).min(axis=-1)
    code = np.where(tie.sum(axis=-1) > 1, even_pick, any_pick)
    return (code + 8 * np.signbit(t)).astype(np.uint8)


def fp4_quant(w_bits):
    """BF16 weight [N, K] (K % 32 == 0) -> (E2M1 codes uint8 [N, K], E8M0 scale
    bytes uint8 [N, K / 32])."""
    w = bf16_to_f32(w_bits).astype(np.float64)
    N, K = w.shape
    if K % W4_GROUP:
        raise ValueError("K must be a multiple of 32")
    g = w.reshape(N, K // W4_GROUP, W4_GROUP)
    amax = np.max(np.abs(g), axis=2)
    _, ex = np.frexp(amax)                            # amax = f * 2**ex, f in [0.5, 1)
    e = np.clip(ex.astype(np.int64) - 1 - 2, -127, 127)
    codes = _e2m1_encode(np.ldexp(g, -e[:, :, None]))
    codes = np.where((amax > 0)[:, :, None], codes, codes & 8)   # zero groups: signed zeros
    scales = np.where(amax > 0, e + 127, 0).astype(np.uint8)
    return codes.reshape(N, K), scales


def fp4_dequant(codes, scales):
    """BF16 bits of the exact values 2^(scale - 127) * E2M1(code)."""
    c = np.asarray(codes, np.uint8)
    N, K = c.shape
    mag = E2M1_VALUES[c & 7] * np.where(c & 8, -1.0, 1.0)
    v = mag.reshape(N, K // W4_GROUP, W4_GROUP) * np.ldexp(1.0, scales.astype(np.int64) - 127)[:, :, None]
    return f32_to_bf16(v.reshape(N, K).astype(np.float32))


def fp4_linear_ref64(x_bits, codes, scales):
    """float64 sum over k of x[m, k] * dequantized FP4 weight[n, k]."""
    x = bf16_to_f32(x_bits).astype(np.float64)
    w = bf16_to_f32(fp4_dequant(codes, scales)).astype(np.float64)
    return x @ w.T


# ---------------------------------------------------------------------------
# MoE form: grouped matmul over low-bit expert weights, and the expert chain
# ---------------------------------------------------------------------------

def lowbit_dequant(fmt, codes, scales):
    """BF16 bits of one expert's dequantized weight: fmt "int4" (codes int8,
    BF16 scale bits) or "fp4" (E2M1 codes, E8M0 bytes)."""
    return w4_dequant(codes, scales) if fmt == "int4" else fp4_dequant(codes, scales)


def lowbit_grouped_ref64(fmt, x_bits, group_list, codes, scales):
    """Rows of expert e (rows grouped by expert, group_list = rows per expert)
    times expert e's dequantized weight [N, K]: float64 sums [R, N]."""
    off = group_offsets(group_list)
    x = bf16_to_f32(x_bits).astype(np.float64)
    N = np.asarray(codes).shape[1]
    y = np.zeros((x.shape[0], N))
    for e in range(len(off) - 1):
        a, b = int(off[e]), int(off[e + 1])
        if b > a:
            w = bf16_to_f32(lowbit_dequant(fmt, codes[e], scales[e])).astype(np.float64)
            y[a:b] = x[a:b] @ w.T
    return y


def lowbit_swiglu(h_bits, inter):
    """a = BF16(silu(gate) * up) of h = [gate | up] [R, 2I] (BF16 out)."""
    return f32_to_bf16(swiglu(h_bits, inter))


def lowbit_moe(fmt, group_list, x_bits, w13_codes, w13_scales, w2_codes, w2_scales, keep=False):
    """Low-bit expert chain on expert-grouped BF16 rows x [R, H]: h = BF16 of the
    W13 sums, a = BF16 SwiGLU of h, y64 = the float64 W2 sums of a (unrounded).
    Returns y64, or a dict of every stage when ``keep``."""
    inter = np.asarray(w13_codes).shape[1] // 2
    h64 = lowbit_grouped_ref64(fmt, x_bits, group_list, w13_codes, w13_scales)
    h = f32_to_bf16(h64.astype(np.float32))
    a = lowbit_swiglu(h, inter)
    y64 = lowbit_grouped_ref64(fmt, a, group_list, w2_codes, w2_scales)
    if keep:
        return dict(h64=h64, h=h, a=a, y64=y64)
    return y64
