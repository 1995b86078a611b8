"""Pins of the static W8A8 oracle (oracle/static_ref.py) against facts other than
itself (CPU only): hand-computed codes and constants, exact-rational recomputation
of every fp32 step, the quantization error bound, and the float64 dequantized
product. A slip such as a reciprocal instead of the division, the offset added
after the rounding, a dropped or sign-flipped correction, or a missing bias
fails one of them.
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np

import oracle as O
from tests.exact_fp import f32_round, frac

S = O.static


def f32(xs):
    return np.asarray(xs, dtype=np.float32)


def test_static_quant_hand_rows():
    # s = 0.5, o = 3: x / s exact, + 3 exact; ties to even; both INT8 ends
    x = f32([1.0, -2.5, 0.25, -0.25, 0.75, 100.0, -100.0, 0.0])
    assert S.static_quant_f32(x[None, :], 0.5, 3.0).tolist() == [[5, -2, 4, 2, 4, 127, -128, 3]]
    # the offset is added before the rounding: 0.25 / 0.5 + 1 = 1.5 -> 2 (rint(0.5) + 1 would be 1)
    assert S.static_quant_f32(f32([[0.25]]), 0.5, 1.0).tolist() == [[2]]
    # a non-integer offset: 0 + 0.5 -> 0, 1 + 0.5 -> 2, -2 + 0.5 -> -2
    assert S.static_quant_f32(f32([[0.0, 0.5, -1.0]]), 0.5, 0.5).tolist() == [[0, 2, -2]]


def _code_exact(x, s, o) -> int:
    t = f32_round(frac(x) / frac(s))
    t = f32_round(t + frac(o))
    return max(-128, min(127, int(round(t))))


def test_static_quant_exact_rational():
    rng = np.random.default_rng(5)
    for s, o in ((0.0371, 0.0), (0.013, 7.0), (0.5, -3.0), (1.7e-3, 2.5), (0.0999, -128.0)):
        s32, o32 = np.float32(s), np.float32(o)
        # random values plus values placed on and next to the ties of the code
        xs = list(rng.standard_normal(600).astype(np.float32) * np.float32(40 * s32))
        for k in range(-140, 140, 3):
            c = np.float32((k + 0.5 - float(o32)) * float(s32))
            xs += [c, np.nextafter(c, np.float32(np.inf)), np.nextafter(c, np.float32(-np.inf))]
        x = f32(xs)
        got = S.static_quant_f32(x[None, :], s, o)[0]
        want = [_code_exact(v, s32, o32) for v in x]
        assert got.tolist() == want


def test_static_quant_error_bound():
    # unclamped codes dequantize to within half a step (plus fp32 rounding)
    rng = np.random.default_rng(6)
    s, o = 0.02, 4.0
    x = (rng.standard_normal((8, 512)) * 0.8).astype(np.float32)
    q = S.static_quant_f32(x, s, o).astype(np.float64)
    inside = (q > -128) & (q < 127)
    err = np.abs((q - o) * np.float64(np.float32(s)) - x.astype(np.float64))
    assert np.all(err[inside] <= 0.5 * s * (1 + 2 ** -20) + 2 ** -24 * np.abs(x[inside]) * 4)
    assert inside.mean() > 0.99


W_HAND = np.array([[1, -2, 3, 4], [-5, 0, 2, 1]], np.int8)   # row sums 6, -2


def test_static_prepare_hand():
    ws = f32([0.25, 0.125])
    bias = O.f32_to_bf16(f32([1.0, -0.5]))
    deq, qb = S.static_prepare(W_HAND, ws, bias, 0.5, 3.0)
    # deq = 0.5 * ws; correction = 3 * (6, -2) = (18, -6); bias / deq = (8, -8)
    assert deq.tolist() == [0.125, 0.0625]
    assert qb.tolist() == [8 - 18, -8 + 6]
    deq, qb = S.static_prepare(W_HAND, ws, None, 0.5, 3.0)      # no bias
    assert qb.tolist() == [-18, 6]


def test_static_prepare_exact_rational():
    rng = np.random.default_rng(7)
    N, K = 64, 300
    w = rng.integers(-128, 128, (N, K)).astype(np.int8)
    ws = (rng.uniform(1e-3, 1e-2, N)).astype(np.float32)
    bias = O.f32_to_bf16((rng.standard_normal(N) * 0.1).astype(np.float32))
    for s, o in ((0.031, 0.0), (0.0123, 3.0), (0.07, -5.5)):
        deq, qb = S.static_prepare(w, ws, bias, s, o)
        s32, o32 = np.float32(s), np.float32(o)
        fb = O.bf16_to_f32(bias)
        for n in range(N):
            d = f32_round(frac(s32) * frac(ws[n]))
            corr = f32_round(Fraction(int(w[n].astype(np.int64).sum())) * frac(o32))
            t = f32_round(frac(fb[n]) / d)
            t = f32_round(t - corr)
            assert float(deq[n]) == float(d)
            assert int(qb[n]) == int(round(t)), (n, s, o)


def test_static_linear_hand():
    ws = f32([0.25, 0.125])
    bias = O.f32_to_bf16(f32([1.0, -0.5]))
    deq, qb = S.static_prepare(W_HAND, ws, bias, 0.5, 3.0)
    q = np.array([[1, 0, 0, 0], [0, 0, 0, 2]], np.int8)
    y, acc = S.static_linear(q, W_HAND, deq, qb)
    # acc = (1, -5), (8, 2); + quant_bias (-10, -2) -> (-9, -7), (-2, 0); times (0.125, 0.0625)
    assert acc.tolist() == [[1, -5], [8, 2]]
    assert O.bf16_to_f32(y).tolist() == [[-1.125, -0.4375], [-0.25, 0.0]]


def test_static_linear_float64_bound():
    rng = np.random.default_rng(8)
    M, N, K = 12, 40, 512
    s, o = 0.03, 5.0
    x = (rng.standard_normal((M, K)) * 0.9).astype(np.float32)
    w = rng.integers(-127, 128, (N, K)).astype(np.int8)
    ws = rng.uniform(1e-3, 1e-2, N).astype(np.float32)
    bias = O.f32_to_bf16((rng.standard_normal(N) * 0.1).astype(np.float32))
    q = S.static_quant_f32(x, s, o)
    deq, qb = S.static_prepare(w, ws, bias, s, o)
    y, acc = S.static_linear(q, w, deq, qb)
    ref = S.static_linear_ref64(q, w, ws, bias, s, o)
    yf = O.bf16_to_f32(y).astype(np.float64)
    d = deq.astype(np.float64)[None, :]
    so = np.abs(w.astype(np.int64).sum(axis=1) * o)[None, :]
    bound = (0.5 * d * (1 + 2 ** -10) + 2 ** -20 * d * (np.abs(acc) + np.abs(qb)[None, :] + so)
             + 2 ** -8 * np.abs(ref) + 1e-12)
    assert np.all(np.abs(yf - ref) <= bound)
    # the bound is tight enough to see the correction: a quant_bias without it
    # (round(fp_bias / deq_scale) alone) breaks the bound in most columns
    qb_bad = np.rint(O.bf16_to_f32(bias).astype(np.float64) / deq.astype(np.float64))
    y_bad = (acc + qb_bad[None, :]) * d
    assert np.mean(np.abs(y_bad - ref) > bound) > 0.9
