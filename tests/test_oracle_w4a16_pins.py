"""Pins of the W4A16 oracle (oracle/w4a16_ref.py), CPU only: hand groups
(exact and BF16-rounded scales, ties to even, the zero group), exact-rational
recomputation of the quantizer and the dequantization, the half-step error
bound, the page's recipe itself where the scale is exactly representable, and
a brute-force product; for the FP4 (E2M1 + E8M0) weights, hand groups with
every tie and the saturation, an independent nearest-value search, the error
bound and a brute-force product. A slip such as amax / 8, a truncating
round, the fp32 scale instead of the stored BF16 one, groups along N, a
dropped scale, emax 3 instead of 2 or ties away from zero fails one of them.
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


# ---------------------------------------------------------------------------
# FP4 (E2M1 + E8M0 per 32) weights
# ---------------------------------------------------------------------------

def test_fp4_hand_group():
    # amax 6 -> E = floor(log2 6) - 2 = 0 (byte 127): the values themselves are
    # encoded; 0.25 / 0.75 / 1.25 / 1.75 / 2.5 / 3.5 / 5 are ties and go to the
    # even codes 0 (0), 2 (1.0), 2 (1.0), 4 (2.0), 4 (2.0), 6 (4.0), 6 (4.0);
    # -0.0 keeps its sign (code 8); 0.3 -> 0.5 (code 1); -6 -> code 15
    w = _group([6.0, -6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.0, 0.3])
    c, s = W4.fp4_quant(w)
    assert s.tolist() == [[127]]
    assert c[0, :11].tolist() == [7, 15, 0, 2, 2, 4, 4, 6, 6, 8, 1]
    # amax 1 -> E = -2 (byte 125): 1.0 / 2^-2 = 4 -> code 6; 0.375 -> 1.5 ->
    # code 3; -0.125 -> -0.5 -> code 1 + 8
    c, s = W4.fp4_quant(_group([1.0, 0.375, -0.125]))
    assert s.tolist() == [[125]] and c[0, :3].tolist() == [6, 3, 9]
    # amax 7 -> E = 0: 7 saturates to 6 (code 7); a zero group gets byte 0
    c, s = W4.fp4_quant(np.concatenate([_group([7.0]), _group([0.0])], axis=1))
    assert s.tolist() == [[127, 0]] and c[0, 0] == 7 and not c[0, 32:].any()


def test_fp4_exhaustive_nearest_and_bound():
    rng = np.random.default_rng(6)
    N, K = 5, 128
    w = (rng.standard_normal((N, K)) * np.exp(rng.uniform(-6, 3, (N, 1)))).astype(np.float32)
    wb = O.f32_to_bf16(w)
    c, s = W4.fp4_quant(wb)
    wf = O.bf16_to_f32(wb).astype(np.float64)
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for n in range(N):
        for g in range(K // 32):
            grp = wf[n, 32 * g:32 * g + 32]
            amax = float(np.max(np.abs(grp)))
            e = int(np.floor(np.log2(amax))) - 2
            assert s[n, g] == e + 127
            for j, v in enumerate(grp):
                t = min(abs(v) / 2.0 ** e, 6.0)
                dist = [abs(t - m) for m in mags]
                best = min(dist)
                cands = [i for i in range(8) if dist[i] == best]
                code = cands[0] if len(cands) == 1 else [i for i in cands if i % 2 == 0][0]
                code += 8 if np.signbit(v) else 0
                assert c[n, 32 * g + j] == code, (n, g, j, v)
    d = O.bf16_to_f32(W4.fp4_dequant(c, s)).astype(np.float64)
    step = np.repeat(2.0 ** (s.astype(np.float64) - 127), 32, axis=1)
    assert np.all(np.abs(d - wf) <= 0.25 * np.abs(wf) + 0.25 * step)


def test_fp4_linear_brute_force():
    rng = np.random.default_rng(7)
    M, N, K = 2, 3, 64
    x = O.f32_to_bf16(rng.standard_normal((M, K)).astype(np.float32))
    c, s = W4.fp4_quant(O.f32_to_bf16((rng.standard_normal((N, K)) * 0.02).astype(np.float32)))
    ref = W4.fp4_linear_ref64(x, c, s)
    xf = O.bf16_to_f32(x)
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                v = mags[c[n, k] & 7] * (-1.0 if c[n, k] & 8 else 1.0) * 2.0 ** (int(s[n, k // 32]) - 127)
                acc += float(xf[m, k]) * v
            assert abs(ref[m, n] - acc) <= 1e-12 * abs(acc) + 1e-300


# ---------------------------------------------------------------------------
# MoE form: grouped matmul over low-bit expert weights, and the expert chain
# ---------------------------------------------------------------------------

def _golden_counts():
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "moe_group_counts.txt")
    line = [l for l in open(path, encoding="utf-8") if not l.startswith("#") and l.strip()][0]
    return [int(v) for v in line.split()]


def _experts(fmt, E, N, K, seed):
    rng = np.random.default_rng(seed)
    codes, scales = [], []
    for e in range(E):
        # experts of very different magnitude, so that a row multiplied by the
        # wrong expert's weight cannot pass
        w = O.f32_to_bf16((rng.standard_normal((N, K)) * 0.02 * 4.0 ** e).astype(np.float32))
        c, s = W4.w4_quant(w) if fmt == "int4" else W4.fp4_quant(w)
        codes.append(c)
        scales.append(s)
    return np.stack(codes), np.stack(scales)


def _value(fmt, codes, scales, n, k):
    """Dequantized weight element by its definition (one element, plain Python)."""
    if fmt == "int4":
        s = float(O.bf16_to_f32(np.array([scales[n, k // 32]], np.uint16))[0])
        v = np.float32(codes[n, k]) * np.float32(s)
        return float(O.bf16_to_f32(O.f32_to_bf16(np.array([v], np.float32)))[0])
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    return mags[codes[n, k] & 7] * (-1.0 if codes[n, k] & 8 else 1.0) * 2.0 ** (int(scales[n, k // 32]) - 127)


def _brute_grouped(fmt, x_bits, counts, codes, scales):
    xf = O.bf16_to_f32(x_bits)
    N, K = codes.shape[1], codes.shape[2]
    out, r = [], 0
    for e, n_e in enumerate(counts):          # rows grouped by expert, in order
        for _ in range(n_e):
            out.append([sum(float(xf[r, k]) * _value(fmt, codes[e], scales[e], n, k) for k in range(K))
                        for n in range(N)])
            r += 1
    return np.array(out)


def test_lowbit_grouped_brute_force_on_the_page_counts():
    counts = _golden_counts()            # 12, 7, 0, 19: the third expert is empty
    rng = np.random.default_rng(8)
    R, N, K = sum(counts), 3, 64
    x = O.f32_to_bf16(rng.standard_normal((R, K)).astype(np.float32))
    for fmt in ("int4", "fp4"):
        c, s = _experts(fmt, len(counts), N, K, seed=9)
        ref = W4.lowbit_grouped_ref64(fmt, x, np.array(counts), c, s)
        want = _brute_grouped(fmt, x, counts, c, s)
        assert np.allclose(ref, want, rtol=1e-12, atol=1e-300), fmt


def test_lowbit_swiglu_hand_values():
    # silu(2) * 3 = 2 / (1 + e^-2) * 3 = 5.28478...; BF16 neighbours 5.28125 and
    # 5.3125 -> 5.28125. silu(0) * 7 = 0; silu(-100) * 1 = -0 (the exponential
    # overflows to +inf); gate 20: silu(20) = 19.99999996 -> 20 after BF16.
    g = np.array([[2.0, 0.0, -100.0, 20.0]], np.float32)
    u = np.array([[3.0, 7.0, 1.0, 1.0]], np.float32)
    a = O.bf16_to_f32(W4.lowbit_swiglu(O.f32_to_bf16(np.concatenate([g, u], axis=1)), 4))[0]
    assert a.tolist() == [5.28125, 0.0, 0.0, 20.0]
    assert np.signbit(a[2])


def test_lowbit_moe_chain_brute_force():
    import math
    counts = [3, 0, 2]
    rng = np.random.default_rng(10)
    R, H, I = sum(counts), 64, 32
    x = O.f32_to_bf16(rng.standard_normal((R, H)).astype(np.float32))
    for fmt in ("int4", "fp4"):
        c13, s13 = _experts(fmt, len(counts), 2 * I, H, seed=11)
        c2, s2 = _experts(fmt, len(counts), H, I, seed=12)
        st = W4.lowbit_moe(fmt, np.array(counts), x, c13, s13, c2, s2, keep=True)
        h64 = _brute_grouped(fmt, x, counts, c13, s13)
        assert np.allclose(st["h64"], h64, rtol=1e-12, atol=1e-300)
        h = O.f32_to_bf16(h64.astype(np.float32))
        assert np.array_equal(st["h"], h)
        hf = O.bf16_to_f32(h).astype(np.float64)
        a_exact = hf[:, :I] / (1.0 + np.exp(-hf[:, :I])) * hf[:, I:]
        af = O.bf16_to_f32(st["a"]).astype(np.float64)
        # BF16 of the exact value, except where it sits within fp32 noise of a
        # rounding boundary (the fixed exp is ~1 ulp accurate)
        want = O.bf16_to_f32(O.f32_to_bf16(a_exact.astype(np.float32))).astype(np.float64)
        near = np.abs(a_exact - want) > 0.49 * np.abs(want) * 2.0 ** -8
        assert np.all((af == want) | near)
        y64 = _brute_grouped(fmt, st["a"], counts, c2, s2)
        assert np.allclose(st["y64"], y64, rtol=1e-12, atol=1e-300)
        assert math.isfinite(float(np.abs(y64).max()))
