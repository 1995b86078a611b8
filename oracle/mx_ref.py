"""NumPy oracle of the MXFP8 variant. TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this module. It shares no code or tables with the HIP library.

Source: "Qwen3.8-FP8 on Ascend 950: Why Weights Become MXFP8 at Load Time"
  * Deep Dive 1: the checkpoint holds E4M3 weights plus one fp32
    ``weight_scale_inv`` per (B_N x B_K) source tile.
  * Deep Dive 2 (the resolve equation): W[i, j] = float32(W_fp8[i, j]) times
    S[floor(i / B_N), floor(j / B_K)], multiplied in fp32 and written in the
    model dtype (BF16 here); edge tiles are cropped.
  * Deep Dive 3: the resolved matrix is re-quantized to an E4M3 payload plus one
    E8M0 scale per 32 values along K; K must be a multiple of 32.
  * Deep Dive 5: at run time the activation is MX-quantized the same way and the
    block-scaled matmul returns the model dtype.

Readings (the pages name the formats, not their rounding rules):
  * E4M3 is OCP E4M3FN: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits, no
    infinities, 0x7F / 0xFF are NaN, largest finite 448. Encoding rounds to the
    nearest representable value, ties to the even code, keeps subnormals,
    saturates magnitudes above 448 to 448 and keeps the sign of zero.
  * E8M0 byte b stands for 2**(b - 127) (255 is NaN, never produced).
  * Shared exponent, scale_alg 0 (the default the page says normal models
    use): E = floor(log2(amax)) - 8 (8 is the largest E4M3 exponent), clamped
    to [-127, 127]; a group with amax 0 gets byte 0 (and zero payloads that
    keep their sign, like every other zero).
    scale_alg 1 (reserved on the page for another model, algorithm not given):
    the smallest E with amax / 2**E <= 448, so no element saturates.
  * The block-scaled product accumulates in fp32 on the GPU; the oracle's value
    is the float64 sum of the exactly dequantized products, and the BF16 output
    is compared with the 2**-8 relative / 1e-5 absolute tolerance.

Parity status: e4m3_encode pinned against torch.float8_e4m3fn (in range) and
hand values; mx_quant pinned by hand groups and the page's K = 128 example;
mx_resolve pinned by loops and the page's 4 x 8 tile example; mx_gemm_ref64 by
brute force. scale_alg 1 is a reading with no pin beyond its definition
(parity unpinned as a choice between the two rules).
"""

from __future__ import annotations

import numpy as np

from .w8a8_ref import f32_to_bf16

__all__ = [
    "E4M3_MAX",
    "e4m3_values",
    "e4m3_decode",
    "e4m3_encode",
    "e8m0_decode",
    "mx_shared_exponent",
    "mx_quant",
    "mx_dequant",
    "mx_resolve",
    "mx_gemm_ref64",
]

E4M3_MAX = 448.0


def e4m3_values() -> np.ndarray:
    """Value of every E4M3FN code 0..255 as float64 (NaN for 0x7F and 0xFF)."""
    codes = np.arange(256)
    s = np.where(codes & 0x80, -1.0, 1.0)
    e = (codes >> 3) & 0xF
    m = codes & 0x7
    v = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    v = s * v
    v[(e == 15) & (m == 7)] = np.nan
    return v


_VALUES = e4m3_values()
_POS = _VALUES[:0x7F]  # codes 0x00..0x7E: 0, subnormals, normals up to 448 (sorted)


def e4m3_decode(b) -> np.ndarray:
    return _VALUES[np.asarray(b, np.uint8)]


def e4m3_encode(v) -> np.ndarray:
    """Nearest E4M3FN code, ties to the even code, saturating at 448."""
    v = np.asarray(v, np.float64)
    a = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.searchsorted(_POS, a, side="left")       # first value >= a
    hi = np.minimum(hi, len(_POS) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS[lo]
    d_hi = _POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return (code | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


def e8m0_decode(b) -> np.ndarray:
    return np.ldexp(1.0, np.asarray(b, np.int64) - 127)


def mx_shared_exponent(amax: np.ndarray, scale_alg: int = 0) -> np.ndarray:
    """E per group (int64), before the +127 bias; amax 0 -> -127."""
    amax = np.asarray(amax, np.float64)
    _, ex = np.frexp(amax)                 # amax = f * 2**ex, f in [0.5, 1)
    e = ex.astype(np.int64) - 1 - 8        # floor(log2(amax)) - emax(E4M3)
    if scale_alg == 1:
        e = e + (np.ldexp(amax, -e) > E4M3_MAX)
    elif scale_alg != 0:
        raise ValueError("scale_alg must be 0 or 1")
    e = np.clip(e, -127, 127)
    return np.where(amax > 0, e, -127)


def mx_quant(x, scale_alg: int = 0):
    """Per row, per 32 values along K: E8M0 scale byte and E4M3 payload.

    x: float values [M, K] (exact in float64). Returns (payload uint8 [M, K],
    scale bytes uint8 [M, K / 32]).
    """
    x = np.asarray(x, np.float64)
    M, K = x.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    g = x.reshape(M, K // 32, 32)
    amax = np.max(np.abs(g), axis=2)
    e = mx_shared_exponent(amax, scale_alg)
    payload = e4m3_encode(np.ldexp(g, -e[:, :, None]))   # exact power-of-two scaling
    return payload.reshape(M, K), (e + 127).astype(np.uint8)


def mx_dequant(payload, scales) -> np.ndarray:
    """float64 values: payload * 2**(scale - 127), exact."""
    p = e4m3_decode(payload)
    M, K = p.shape
    s = e8m0_decode(scales)
    return (p.reshape(M, K // 32, 32) * s[:, :, None]).reshape(M, K)


def mx_resolve(w_e4m3, scale_inv, bn: int, bk: int) -> np.ndarray:
    """Block-FP8 resolve to BF16 bits: BF16(fl32(fp32(e4m3) * S[i // bn, j // bk]))."""
    w = e4m3_decode(w_e4m3).astype(np.float32)        # exact
    N, K = w.shape
    S = np.asarray(scale_inv, np.float32)
    if S.shape != (-(-N // bn), -(-K // bk)):
        raise ValueError("scale shape does not match the tile grid")
    s_full = np.repeat(np.repeat(S, bn, axis=0), bk, axis=1)[:N, :K]   # cropped edges
    return f32_to_bf16((w * s_full).astype(np.float32))


def mx_gemm_ref64(a_payload, a_scales, w_payload, w_scales) -> np.ndarray:
    """sum_k A[m, k] * W[n, k] over the dequantized MX operands, in float64."""
    return mx_dequant(a_payload, a_scales) @ mx_dequant(w_payload, w_scales).T
