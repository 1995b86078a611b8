"""NumPy oracle of the W8A8_DYNAMIC hot path. TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg
may import this module. It shares no code, tables or constants with the HIP
library under ``moe_token_amax_amd/``.

Page tags used below:
  [DSV4]  "DeepSeek-V4 W8A8 执行链从量化权重到 Ascend INT8 算子"
  [MXFP8] "Qwen3.8-FP8 on Ascend 950: Why Weights Become MXFP8 at Load Time"
  [LOWBIT] "超大 MoE 的低比特推理：INT4、FP4 与量化感知训练"

Numeric conventions (the pages do not fix them; each is a stated reading):
  * BF16 -> fp32 is exact; fp32 -> BF16 rounds to nearest, ties to even.
  * Every fp32 step is one IEEE binary32 operation on NumPy float32 arrays
    (NumPy never fuses a multiply into an add).
  * Integer accumulation is exact: float64 BLAS on integer-valued operands is
    exact while every partial sum stays below 2**53.

Parity status (what pins each function, see tests/test_oracle_pins.py):
  dynamic_quant        pinned: hand rows, exact-rational brute force, invariants
  int8_matmul_acc      pinned: brute-force integer loops
  epilogue_bf16        pinned: hand case, torch bf16 rounding, float64 bound
  grouped_gemm_*       pinned: worked group counts [DSV4 §三], per-row brute force
  exp_spec / silu      pinned: float64 exp / silu within 2 ulp, special values
  swiglu_quant         pinned: exact-rational brute force on small rows
  moe_grouped          pinned: composition of the pinned stages + float64 bound
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "bf16_to_f32",
    "f32_to_bf16",
    "dynamic_quant",
    "dynamic_quant_f32",
    "int8_matmul_acc",
    "epilogue_bf16",
    "linear",
    "linear_ref64",
    "group_offsets",
    "expert_of_rows",
    "grouped_gemm_acc",
    "grouped_gemm_bf16",
    "exp_spec",
    "silu_spec",
    "swiglu",
    "swiglu_quant",
    "moe_grouped",
    "bf16_within_tolerance",
    "REL_TOL",
    "ABS_FLOOR",
]

F32 = np.float32

# BF16 output tolerance: max relative error 2**-8 with an absolute floor of 1e-5,
# measured against the unrounded float64 value of the same expression.
REL_TOL = 2.0 ** -8
ABS_FLOOR = 1e-5


# ---------------------------------------------------------------------------
# BF16 <-> fp32
# ---------------------------------------------------------------------------

def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """BF16 bit patterns (uint16) -> float32, exactly (the top half of an fp32)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> BF16 bits with round-to-nearest, ties-to-even.

    The 16 dropped bits are rounded: add 0x7FFF plus the lowest kept bit, then
    shift. Inputs are finite (NaN is out of scope for this path).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


# ---------------------------------------------------------------------------
# a1: per-token symmetric INT8 quantization
# ---------------------------------------------------------------------------

def dynamic_quant_f32(x: np.ndarray):
    """Per-row symmetric INT8 quantization of a float32 matrix.

    [DSV4 §一]: the activation recipe is per_token, int8, symmetric.
    [DSV4 §二]: npu_dynamic_quant returns the INT8 activation plus one scale per
    row, which the matmul later takes as ``pertoken_scale``.
    The recipe is the usual symmetric one (scale = row max |x| / 127, value =
    round(x / scale)); the same pattern (amax / qmax, round, clamp) is written out
    for INT4 in [LOWBIT, 为什么要量化感知训练].

    Readings: the division is one IEEE fp32 division (not a reciprocal
    multiply); rounding is half-to-even; the clamp is [-127, 127]; a row whose
    max |x| is 0 gets scale 0 and all-zero codes.

    Returns (q int8 [M,K], scale float32 [M]).
    """
    x = np.asarray(x, dtype=np.float32)
    assert x.ndim == 2
    M, K = x.shape
    if M == 0:
        return np.zeros((0, K), np.int8), np.zeros((0,), np.float32)
    amax = np.max(np.abs(x), axis=1)                         # exact
    scale = (amax / F32(127.0)).astype(np.float32)           # fl32(amax / 127)
    q = np.zeros((M, K), dtype=np.int8)
    nz = scale > 0
    if np.any(nz):
        v = x[nz] / scale[nz][:, None]                       # fl32(x / scale)
        q[nz] = np.clip(np.rint(v), -127, 127).astype(np.int8)
    return q, scale


def dynamic_quant(x_bits: np.ndarray):
    """npu_dynamic_quant on a BF16 matrix given as uint16 bits [DSV4 §二]."""
    return dynamic_quant_f32(bf16_to_f32(x_bits))


# ---------------------------------------------------------------------------
# a3: INT8 x INT8 -> INT32 accumulation, a5: dequant epilogue
# ---------------------------------------------------------------------------

def int8_matmul_acc(q: np.ndarray, w: np.ndarray) -> np.ndarray:
    """acc[m, n] = sum_k q[m, k] * w[n, k], exactly (int64 result).

    [DSV4 §二]: W is the offline INT8 [N, K] weight, X the INT8 activation; the
    quant matmul multiplies them with integer accumulation. Computed as one
    float64 matrix product of integer-valued operands, exact because
    |partial sum| <= K * 127**2 < 2**53 for every K this path accepts.
    """
    q = np.asarray(q, dtype=np.int8)
    w = np.asarray(w, dtype=np.int8)
    assert q.shape[1] == w.shape[1]
    assert q.shape[1] * 127 * 127 < 2 ** 53
    acc = q.astype(np.float64) @ w.astype(np.float64).T
    return acc.astype(np.int64)


def epilogue_bf16(acc, x_scale, w_scale, bias_bits=None) -> np.ndarray:
    """y = BF16(((fp32(acc) * x_scale[m]) * w_scale[n]) + bias[n]).

    [DSV4 §二]: npu_quant_matmul takes the per-channel weight scale, the
    per-token scale and an optional bias, and returns output_dtype (BF16).
    The operands are the pages'; the order of the fp32 operations is a reading
    (left to right, one rounding per operation, no fused multiply-add).
    """
    acc = np.asarray(acc)
    t = acc.astype(np.float32)                                # RNE int -> fp32
    t = t * np.asarray(x_scale, np.float32)[:, None]
    t = t * np.asarray(w_scale, np.float32)[None, :]
    if bias_bits is not None:
        t = t + bf16_to_f32(bias_bits)[None, :]
    return f32_to_bf16(t)


def linear(q, x_scale, w, w_scale, bias_bits=None):
    """Dense W8A8_DYNAMIC linear after the activation quant [DSV4 §二].

    Returns (y_bf16_bits [M,N], acc int64 [M,N]).
    """
    acc = int8_matmul_acc(q, w)
    return epilogue_bf16(acc, x_scale, w_scale, bias_bits), acc


def linear_ref64(acc, x_scale, w_scale, bias_bits=None) -> np.ndarray:
    """Unrounded float64 value of acc * x_scale * w_scale + bias (tolerance ref)."""
    y = np.asarray(acc, np.float64) * np.asarray(x_scale, np.float64)[:, None]
    y = y * np.asarray(w_scale, np.float64)[None, :]
    if bias_bits is not None:
        y = y + bf16_to_f32(bias_bits).astype(np.float64)[None, :]
    return y


def bf16_within_tolerance(y_bits, ref64) -> np.ndarray:
    """Element mask: |y - ref| <= max(2**-8 * |ref|, 1e-5)."""
    y = bf16_to_f32(y_bits).astype(np.float64)
    ref64 = np.asarray(ref64, np.float64)
    return np.abs(y - ref64) <= np.maximum(REL_TOL * np.abs(ref64), ABS_FLOOR)


# ---------------------------------------------------------------------------
# a6 / a8: grouped GEMM driven by per-expert row counts
# ---------------------------------------------------------------------------

def group_offsets(group_list) -> np.ndarray:
    """Start row of every expert: exclusive prefix sum of the per-expert counts.

    [DSV4 §三]: expert_tokens / group_list tells the kernel how many rows each
    expert owns (e.g. 12, 7, 0, 19, ...); rows are grouped by expert.
    """
    g = np.asarray(group_list, dtype=np.int64)
    assert np.all(g >= 0)
    off = np.zeros(len(g) + 1, dtype=np.int64)
    off[1:] = np.cumsum(g)
    return off


def expert_of_rows(group_list) -> np.ndarray:
    """Per-row expert id implied by the counts (rows grouped by expert)."""
    g = np.asarray(group_list, dtype=np.int64)
    return np.repeat(np.arange(len(g), dtype=np.int64), g)


def grouped_gemm_acc(q, group_list, w) -> np.ndarray:
    """acc[r, n] = sum_k q[r, k] * w[e(r), n, k] for the expert e(r) owning row r.

    [DSV4 §三]: one grouped matmul over all experts; an expert with 0 rows
    contributes nothing. Weights are [E, N, K] (W13: [E, 2I, H]; W2: [E, H, I]).
    """
    q = np.asarray(q, np.int8)
    off = group_offsets(group_list)
    R = q.shape[0]
    assert off[-1] == R, "sum(group_list) must equal the number of rows"
    N = w.shape[1]
    acc = np.zeros((R, N), dtype=np.int64)
    for e in range(len(off) - 1):
        a, b = int(off[e]), int(off[e + 1])
        if b > a:
            acc[a:b] = int8_matmul_acc(q[a:b], w[e])
    return acc


def grouped_gemm_bf16(q, x_scale, group_list, w, w_scale):
    """Grouped GEMM with the per-expert epilogue (no bias) -> BF16 bits [R, N].

    [DSV4 §三]: npu_grouped_matmul with scale=[weight_scale] (per expert and
    channel) and per_token_scale. Returns (y_bits, acc).
    """
    acc = grouped_gemm_acc(q, group_list, w)
    ex = expert_of_rows(group_list)
    t = acc.astype(np.float32)
    t = t * np.asarray(x_scale, np.float32)[:, None]
    t = t * np.asarray(w_scale, np.float32)[ex]
    return f32_to_bf16(t), acc


# ---------------------------------------------------------------------------
# a7: SwiGLU + per-token requant
# ---------------------------------------------------------------------------

# exp is evaluated by one fixed fp32 sequence on both sides so that the INT8
# codes after the requant can be compared bit for bit. Method: Cody-Waite range
# reduction (t = k*ln2 + r, ln2 split in a 16-bit head and a tail) and the
# degree-7 Taylor polynomial of e**r, evaluated by Horner's rule.
_LOG2E = F32(1.0 / math.log(2.0))
_LN2_HI = F32(math.floor(math.log(2.0) * 2.0 ** 16) / 2.0 ** 16)  # ln2 to 16 bits
_LN2_LO = F32(math.log(2.0) - float(_LN2_HI))
_TAYLOR = [F32(1.0 / math.factorial(n)) for n in range(8)]       # c0 .. c7
_EXP_CLAMP = F32(127.0)


def exp_spec(t: np.ndarray) -> np.ndarray:
    """e**t in float32 by the fixed sequence above (about 1 ulp accurate).

    1. t <- clamp(t, -127, 127)            (keeps |k| < 2**8, so k*LN2_HI is exact)
    2. k = rint(fl32(t * LOG2E))
    3. r = fl32(fl32(t - fl32(k * LN2_HI)) - fl32(k * LN2_LO))
    4. p = c7; p = fl32(fl32(p * r) + c_n) for n = 6 .. 0
    5. result = p * 2**k (one correctly rounded scaling; overflows to +inf,
       underflows through the subnormals to +0).
    """
    t = np.asarray(t, np.float32)
    t = np.minimum(np.maximum(t, -_EXP_CLAMP), _EXP_CLAMP)
    k = np.rint(t * _LOG2E).astype(np.float32)
    r = (t - k * _LN2_HI) - k * _LN2_LO
    p = np.full_like(r, _TAYLOR[7])
    for n in range(6, -1, -1):
        p = p * r + _TAYLOR[n]          # two separate float32 roundings
    with np.errstate(over="ignore", under="ignore"):
        return np.ldexp(p, k.astype(np.int32)).astype(np.float32)


def silu_spec(g: np.ndarray) -> np.ndarray:
    """silu(g) = g / (1 + e**-g), each step one fp32 rounding."""
    g = np.asarray(g, np.float32)
    d = F32(1.0) + exp_spec(-g)
    with np.errstate(over="ignore", divide="ignore", invalid="ignore"):
        return (g / d).astype(np.float32)


def swiglu(h_bits: np.ndarray, inter: int) -> np.ndarray:
    """a[:, j] = silu(gate[:, j]) * up[:, j] in fp32, from BF16 h [R, 2I].

    [DSV4 §一]: W13 is gate_proj + up_proj, so columns [0, I) of the W13 output
    are the gate and [I, 2I) the up projection (concatenation order).
    [DSV4 §三]: the runner applies SwiGLU to the W13 output, then requantizes.
    """
    h = bf16_to_f32(h_bits)
    assert h.shape[1] == 2 * inter
    g = h[:, :inter]
    u = h[:, inter:]
    return (silu_spec(g) * u).astype(np.float32)


def swiglu_quant(h_bits: np.ndarray, inter: int):
    """SwiGLU followed by the per-token requant of the fp32 result.

    [DSV4 §三, §五]: "SwiGLU + Requant" is one fused box that produces a new INT8
    payload and a new per-token scale. Reading: the fp32 SwiGLU output is
    quantized directly (no BF16 rounding in between).
    Returns (q2 int8 [R, I], s2 float32 [R]).
    """
    return dynamic_quant_f32(swiglu(h_bits, inter))


# ---------------------------------------------------------------------------
# MoE expert chain
# ---------------------------------------------------------------------------

def moe_grouped(group_list, w13, w13_scale, w2, w2_scale, *, x_bits=None,
                q=None, x_scale=None, keep=False):
    """Routed hidden -> W13 grouped matmul -> SwiGLU -> requant -> W2 -> BF16.

    [DSV4 §三]: the W8A8 MoE method quantizes the routed hidden states only
    when no per-token scale came with them (``if pertoken_scale is None``);
    otherwise the INT8 rows and their scale go straight into W13.
    Input: either ``x_bits`` (BF16 [R, H]) or ``q`` + ``x_scale``.
    Output rows stay in the expert-grouped order (no top-k combine).
    Returns y_bits [R, H], or a dict of every stage when ``keep``.
    """
    if x_scale is None:
        q, x_scale = dynamic_quant(x_bits)
    inter = w13.shape[1] // 2
    h, acc13 = grouped_gemm_bf16(q, x_scale, group_list, w13, w13_scale)
    q2, s2 = swiglu_quant(h, inter)
    y, acc2 = grouped_gemm_bf16(q2, s2, group_list, w2, w2_scale)
    if keep:
        return dict(q=q, x_scale=x_scale, acc13=acc13, h=h, q2=q2, s2=s2,
                    acc2=acc2, y=y)
    return y
