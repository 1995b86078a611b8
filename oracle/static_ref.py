"""NumPy oracle of the static W8A8 scheme. TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg
may import this module. It shares no code, tables or constants with the HIP
library under ``moe_token_amax_amd/``.

Page: [DSV4] "DeepSeek-V4 W8A8 执行链从量化权重到 Ascend INT8 算子", the static
W8A8 comparison at the end of the page (deq_scale and quant_bias derivation,
and the static flow diagram). What the page fixes:
  * deq_scale = input_scale * weight_scale;
  * correction = (sum over k of the INT8 weight row, as float) * input_offset;
  * quant_bias = round(fp_bias / deq_scale - correction), as int32;
  * flow: BF16 X, with a fixed input_scale / input_offset, goes through
    npu_quantize to INT8 X; npu_quant_matmul(x, W, deq_scale, bias=quant_bias)
    returns BF16 Y.

Readings (the page prints the two formulas and the flow, not the arithmetic of
npu_quantize or of the matmul epilogue):
  * static quant: q = clamp(RNE(fl32(fl32(x / input_scale) + input_offset)),
    -128, 127): the offset is the zero point that the correction term removes
    again (x ~ (q - input_offset) * input_scale), so it is added after the
    division; one IEEE fp32 operation per step; the clamp is the INT8 range
    (an asymmetric code uses both ends).
  * epilogue: y = BF16(fl32(fp32(acc + quant_bias) * deq_scale)): the bias is an
    integer added to the exact INT32 accumulator, then one conversion, one
    multiply and the BF16 rounding (RNE). This is what makes
    deq_scale * (acc + quant_bias) ~ x @ W^T + fp_bias.
  * deq_scale = fl32(input_scale * w_scale[n]); correction = fl32(fp32(S_n) *
    input_offset) with S_n the exact integer row sum (equal to a float32
    running sum while |S_n| < 2**24, i.e. for K <= 132,104);
    quant_bias = clamp(RNE(fl32(fl32(fp_bias / deq_scale) - correction)),
    -2**31, 2**31 - 1) (a saturating conversion).
  * input_scale > 0 and every w_scale > 0; acc + quant_bias must fit in int32.

Parity status (tests/test_oracle_static_pins.py): static_quant pinned by hand
rows and an exact-rational brute force; static_prepare by a hand example and an
exact-rational recomputation; static_linear by hand values and the float64
dequantized product within the bound the readings imply.
"""

from __future__ import annotations

import numpy as np

from .w8a8_ref import bf16_to_f32, f32_to_bf16, int8_matmul_acc

F32 = np.float32

__all__ = [
    "static_quant_f32",
    "static_quant",
    "static_prepare",
    "static_epilogue_bf16",
    "static_linear",
    "static_linear_ref64",
]


def static_quant_f32(x, input_scale: float, input_offset: float) -> np.ndarray:
    """npu_quantize with a fixed per-tensor scale and offset on a float32 matrix
    ([DSV4] static flow): q = clamp(RNE(fl32(fl32(x / s) + o)), -128, 127)."""
    x = np.asarray(x, dtype=np.float32)
    s = F32(input_scale)
    o = F32(input_offset)
    assert s > 0
    t = (x / s).astype(np.float32)          # fl32(x / s)
    t = (t + o).astype(np.float32)          # fl32(t + o)
    return np.clip(np.rint(t), -128, 127).astype(np.int8)


def static_quant(x_bits, input_scale: float, input_offset: float) -> np.ndarray:
    """static_quant_f32 on a BF16 matrix given as uint16 bits."""
    return static_quant_f32(bf16_to_f32(x_bits), input_scale, input_offset)


def static_prepare(w, w_scale, bias_bits, input_scale: float, input_offset: float):
    """Load-time constants of the static scheme ([DSV4] static comparison).

    w int8 [N, K] (the INT8 weight Qw), w_scale float32 [N], bias BF16 [N] bits or
    None (fp_bias = 0). Returns (deq_scale float32 [N], quant_bias int32 [N]).
    """
    w = np.asarray(w, dtype=np.int8)
    ws = np.asarray(w_scale, dtype=np.float32)
    assert np.all(ws > 0) and input_scale > 0
    deq = (F32(input_scale) * ws).astype(np.float32)                 # fl32(s * ws)
    rowsum = w.astype(np.int64).sum(axis=1)                           # exact
    corr = (rowsum.astype(np.float32) * F32(input_offset)).astype(np.float32)
    fb = (bf16_to_f32(bias_bits) if bias_bits is not None
          else np.zeros(w.shape[0], np.float32)).astype(np.float32)
    t = (fb / deq).astype(np.float32)                                 # fl32(fp_bias / deq)
    t = (t - corr).astype(np.float32)                                 # fl32(t - correction)
    r = np.rint(t.astype(np.float64))
    r = np.clip(r, -2.0 ** 31, 2.0 ** 31 - 1)
    return deq, r.astype(np.int32)


def static_epilogue_bf16(acc, deq_scale, quant_bias) -> np.ndarray:
    """y = BF16(fl32(fp32(acc + quant_bias[n]) * deq_scale[n])) (reading above)."""
    s = np.asarray(acc, np.int64) + np.asarray(quant_bias, np.int64)[None, :]
    assert np.all(np.abs(s) < 2 ** 31), "acc + quant_bias must fit in int32"
    t = s.astype(np.float32)                                          # RNE int -> fp32
    t = (t * np.asarray(deq_scale, np.float32)[None, :]).astype(np.float32)
    return f32_to_bf16(t)


def static_linear(q, w, deq_scale, quant_bias):
    """npu_quant_matmul(x, W, deq_scale, bias=quant_bias) with BF16 output.
    Returns (y_bf16_bits [M, N], acc int64 [M, N])."""
    acc = int8_matmul_acc(q, w)
    return static_epilogue_bf16(acc, deq_scale, quant_bias), acc


def static_linear_ref64(q, w, w_scale, bias_bits, input_scale: float,
                        input_offset: float) -> np.ndarray:
    """The float64 product the scheme stands for: ((q - o) * s) @ (Qw * ws)^T +
    fp_bias, with the stored fp32 constants. static_linear differs from it by the
    rounding of quant_bias (at most half a unit, times deq_scale), the fp32
    rounding of deq_scale and correction, and the final fp32 / BF16 roundings."""
    xq = (np.asarray(q, np.float64) - float(F32(input_offset))) * float(F32(input_scale))
    wq = np.asarray(w, np.float64) * np.asarray(w_scale, np.float32).astype(np.float64)[:, None]
    y = xq @ wq.T
    if bias_bits is not None:
        y = y + bf16_to_f32(bias_bits).astype(np.float64)[None, :]
    return y

