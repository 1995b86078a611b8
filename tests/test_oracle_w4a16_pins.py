"""Pins of the W4A16 oracle (oracle/w4a16_ref.py), CPU only: hand groups
(exact and BF16-rounded scales, ties to even, the zero group), exact-rational
recomputation of the quantizer and the dequantization, the half-step error
bound, the page's recipe itself where the scale is exactly representable, and
a brute-force product. A slip such as amax / 8, a truncating round, the fp32
scale instead of the stored BF16 one, groups along N, or a dropped scale
fails one of them.
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np
import torch

import oracle as O
from tests.exact_fp import f32_round, frac

W4 = O.w4a16


def _group(vals, K=32):
    g = np.zeros((1, K), np.float32)
    g[0, :len(vals)] = vals
    return O.f32_to_bf16(g)


def test_hand_group_exact_scale():
    # amax 7 -> s = 1 exactly; 3.5 and 6.5 tie to the even codes 4 and 6, 2.5 to 2
    w = _group([7.0, -7.0, 3.5, 2.5, -2.5, 0.49, -0.51, 6.5, 0.0, 1.0])
    q, s = W4.w4_quant(w)
    assert O.bf16_to_f32(s).tolist() == [[1.0]]
    assert q[0, :10].tolist() == [7, -7, 4, 2, -2, 0, -1, 6, 0, 1]
    assert not q[0, 10:].any()


def test_hand_group_bf16_scale():
    # amax 1: 1/7 = 1.0010010010..b x 2^-3 rounds to the BF16 1.0010010b x 2^-3 =
    # 0.142578125 (bits 0x3E12); codes are taken against that stored scale:
    # 1 / 0.142578125 = 7.0137 -> 7, 0.5 -> 3.5068 -> 4, -0.25 -> -1.7534 -> -2
    w = _group([1.0, 0.5, -0.25, 0.0625])
    q, s = W4.w4_quant(w)
    assert s.tolist() == [[0x3E12]]
    assert q[0, :4].tolist() == [7, 4, -2, 0]


def test_zero_group_and_groups_along_k():
    w = np.zeros((2, 64), np.float32)
    w[0, 40] = 3.5                    # second group of row 0 only
    w[1, 0] = -14.0                   # first group of row 1 only
    q, s = W4.w4_quant(O.f32_to_bf16(w))
    assert O.bf16_to_f32(s).tolist() == [[0.0, 0.5], [2.0, 0.0]]
    assert q[0, 40] == 7 and q[1, 0] == -7 and np.count_nonzero(q) == 2


def _bf16_round(v: Fraction) -> Fraction:
    """RNE of an fp32 value to BF16 (v already a binary32 number)."""
    b = O.f32_to_bf16(np.array([float(v)], np.float32))
    return frac(O.bf16_to_f32(b)[0])


def _rne(t: Fraction) -> int:
    fl = t.numerator // t.denominator
    r = t - fl
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return fl


def test_quant_and_dequant_exact_rational():
    rng = np.random.default_rng(2)
    N, K = 6, 96
    w = (rng.standard_normal((N, K)) * rng.uniform(0.01, 3.0, (N, 1))).astype(np.float32)
    wb = O.f32_to_bf16(w)
    q, s = W4.w4_quant(wb)
    d = W4.w4_dequant(q, s)
    wf = O.bf16_to_f32(wb)
    for n in range(N):
        for g in range(K // 32):
            vals = [frac(v) for v in wf[n, 32 * g:32 * g + 32]]
            amax = max(abs(v) for v in vals)
            sc = _bf16_round(f32_round(amax / 7))
            assert frac(O.bf16_to_f32(s[n:n + 1, g:g + 1])[0, 0]) == sc
            for j, v in enumerate(vals):
                code = max(-8, min(7, _rne(f32_round(v / sc)))) if sc else 0
                k = 32 * g + j
                assert q[n, k] == code, (n, k)
                want = _bf16_round(f32_round(Fraction(code) * sc))
                assert frac(O.bf16_to_f32(d[n:n + 1, k:k + 1])[0, 0]) == want


def test_half_step_error_bound():
    rng = np.random.default_rng(3)
    w = O.f32_to_bf16((rng.standard_normal((16, 256)) * 0.05).astype(np.float32))
    q, s = W4.w4_quant(w)
    wf = O.bf16_to_f32(w).astype(np.float64)
    sf = np.repeat(O.bf16_to_f32(s).astype(np.float64), 32, axis=1)
    err = np.abs(wf - q.astype(np.float64) * sf)
    assert np.all(err <= sf * (0.5 + 2.0 ** -20))
    assert np.all(np.abs(q) <= 7)          # the symmetric scale never reaches -8


def test_page_recipe_where_the_scale_is_exact():
    # groups whose amax / 7 is a power of two: the stored BF16 scale equals the
    # page's fp32 one, so the codes equal the page's recipe written in torch
    # (amax / 7, round half to even, clamp to [-8, 7])
    rng = np.random.default_rng(4)
    N, K = 8, 128
    w = rng.uniform(-1.0, 1.0, (N, K)).astype(np.float32)
    g = w.reshape(N, K // 32, 32)
    target = 7.0 * 2.0 ** rng.integers(-6, 2, (N, K // 32))
    g /= np.abs(g).max(axis=2, keepdims=True)
    g *= target[:, :, None]
    wb = O.f32_to_bf16(w)
    q, _ = W4.w4_quant(wb)
    t = torch.from_numpy(O.bf16_to_f32(wb)).view(N, -1, 32)
    sc = t.abs().amax(-1, keepdim=True) / 7
    page = (t / sc).round().clamp(-8, 7).to(torch.int8).view(N, K).numpy()
    assert np.array_equal(q, page)


def test_linear_brute_force():
    rng = np.random.default_rng(5)
    M, N, K = 3, 4, 64
    x = O.f32_to_bf16(rng.standard_normal((M, K)).astype(np.float32))
    q, s = W4.w4_quant(O.f32_to_bf16((rng.standard_normal((N, K)) * 0.02).astype(np.float32)))
    ref = W4.w4a16_linear_ref64(x, q, s)
    xf = O.bf16_to_f32(x)
    sf = O.bf16_to_f32(s)
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                wq = float(O.bf16_to_f32(O.f32_to_bf16(np.array([np.float32(q[n, k]) * sf[n, k // 32]],
                                                                np.float32)))[0])
                acc += float(xf[m, k]) * wq
            assert ref[m, n] == acc or abs(ref[m, n] - acc) <= 1e-12 * abs(acc)
