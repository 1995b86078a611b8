"""Pins of the MXFP8 MoE oracle (oracle/mx_moe_ref.py), CPU only: hand-computed
codes and scales (ties to the even E4M3 code, signed zero groups), the page's
worked resolve tile placed inside one expert of a stack, expert independence,
the MX error bound against the resolved weight, hand and brute-force grouped
products, and the whole chain against an unquantized float64 chain. A slip
such as a wrong expert's weight, a transposed operand, gate and up swapped, a
missing BF16 rounding of the SwiGLU output or a per-stack instead of
per-expert scale fails one of them.
"""

from __future__ import annotations

import os

import numpy as np

import oracle as O
import synth

MX = O.mx
MM = O.mx_moe
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mx_examples.txt")


def _resolve_tile():
    for line in open(GOLDEN):
        if line.startswith("resolve_tile"):
            return [int(v) for v in line.split()[1:]]
    raise AssertionError("resolve_tile missing")


def _within_mx_error(d, v, payload, scales):
    """d = dequantized MX values of v: within half an E4M3 step (2**-4 relative)
    or the subnormal spacing of the group, except saturated codes (+-448 times
    the group scale), which need |v| at or above the midpoint 432 below them."""
    step = 2.0 ** (scales.astype(np.float64).repeat(32, 1) - 127.0)
    sat = (payload & 0x7F) == 0x7E
    ok = np.abs(d - v) <= np.abs(v) * 2.0 ** -4 + step * 2.0 ** -10
    ok_sat = (np.abs(d) == 448.0 * step) & (np.abs(v) >= 432.0 * step) & (np.sign(d) == np.sign(v))
    return np.all(np.where(sat, ok_sat | ok, ok))


def _random_stack(E, N, K, bn, bk, seed):
    r = np.random.default_rng(seed)
    w = synth.e4m3_bits(r.standard_normal((E, N, K), dtype=np.float32))
    s = r.uniform(1e-3, 1e-2, size=(E, -(-N // bn), -(-K // bk))).astype(np.float32)
    return w, s


def test_prepare_worked_tile_in_one_expert():
    # [MXFP8] Deep Dive 1: one source scale covers a 4 x 8 tile. Expert 1 holds
    # 1.0 everywhere with power-of-two tile scales, so its resolved values are
    # the scales and its MX codes follow by hand.
    bn, bk = _resolve_tile()
    E, N, K = 3, 8, 32
    w, s = _random_stack(E, N, K, bn, bk, seed=1)
    w[1] = 0x38                                            # E4M3 1.0
    s[1] = [[1.0, 0.5, 0.25, 2.0], [2.0 ** -3, 2.0 ** -3, 2.0 ** -3, 2.0 ** -3]]
    p, sc = MM.mx_moe_prepare(w, s, bn, bk)
    # rows 0..3: amax 2 -> E = 1 - 8 = -7 (byte 120); 1, 0.5, 0.25, 2 scaled by
    # 2**7 are 128, 64, 32, 256: E4M3 codes 0x70, 0x68, 0x60, 0x78
    row = np.repeat(np.array([0x70, 0x68, 0x60, 0x78], np.uint8), 8)
    assert np.array_equal(p[1, :4], np.tile(row, (4, 1)))
    assert sc[1, :4].tolist() == [[120]] * 4
    # rows 4..7: 2**-3 everywhere -> E = -3 - 8 = -11 (byte 116), payload 256
    assert np.all(p[1, 4:] == 0x78) and sc[1, 4:].tolist() == [[116]] * 4
    # the other experts are prepared on their own: swapping them swaps the results
    w2, s2 = w[[2, 1, 0]], s[[2, 1, 0]]
    p2, sc2 = MM.mx_moe_prepare(w2, s2, bn, bk)
    assert np.array_equal(p2, p[[2, 1, 0]]) and np.array_equal(sc2, sc[[2, 1, 0]])


def test_prepare_within_mx_error_of_resolved_weight():
    E, N, K, bn, bk = 2, 16, 96, 8, 32
    w, s = _random_stack(E, N, K, bn, bk, seed=2)
    p, sc = MM.mx_moe_prepare(w, s, bn, bk)
    vals = MX.e4m3_values()
    for e in range(E):
        # resolved weight from its definition: E4M3 value times its tile's scale
        res = np.array([[np.float32(vals[w[e, i, j]]) * s[e, i // bn, j // bk]
                         for j in range(K)] for i in range(N)], np.float32)
        res = O.bf16_to_f32(O.f32_to_bf16(res)).astype(np.float64)
        assert _within_mx_error(MX.mx_dequant(p[e], sc[e]), res, p[e], sc[e])


def test_swiglu_mx_quant_hand_rows():
    I = 32
    g = np.zeros((2, I), np.float32)
    u = np.zeros((2, I), np.float32)
    # row 0: silu(100) == 100 in fp32, a = 100 u: 200, 100, 50 -> amax 200,
    # E = 7 - 8 = -1; 400, 200, 100 are ties between E4M3 neighbours and go to
    # the even codes 384 (0x7C), 192 (0x74), 96 (0x6C)
    g[0] = 100.0
    u[0, 0::3], u[0, 1::3], u[0, 2::3] = 2.0, 1.0, 0.5
    # row 1: gate 0 gives a = 0 * u; negative up values give -0.0 (sign kept)
    u[1] = -1.0
    h = O.f32_to_bf16(np.concatenate([g, u], axis=1))
    p, sc, a = MM.swiglu_mx_quant(h, I)
    want = np.array([0x7C, 0x74, 0x6C] * 11, np.uint8)[:I]
    assert p[0].tolist() == want.tolist() and sc[0].tolist() == [126]
    assert np.all(p[1] == 0x80) and sc[1].tolist() == [0]
    assert np.all(a[1] == 0x8000)


def test_swiglu_mx_quant_rounds_through_bf16():
    # the MX input is the BF16-rounded SwiGLU output: values whose fp32 SwiGLU is
    # not a BF16 number quantize like their BF16 rounding
    rng = np.random.default_rng(5)
    R, I = 6, 64
    h = O.f32_to_bf16((rng.standard_normal((R, 2 * I)) * 3).astype(np.float32))
    p, sc, a = MM.swiglu_mx_quant(h, I)
    hf = O.bf16_to_f32(h).astype(np.float64)
    a64 = hf[:, :I] / (1.0 + np.exp(-hf[:, :I])) * hf[:, I:]
    af = O.bf16_to_f32(a).astype(np.float64)
    assert np.all(np.abs(af - a64) <= 2.0 ** -8 * np.abs(a64) + 1e-30 + 2.0 ** -20 * np.abs(a64))
    assert _within_mx_error(MX.mx_dequant(p, sc), af, p, sc)


def test_mx_grouped_gemm_hand():
    # rows of ones; expert e's row n is (n + 1) * 2**e; expert 1 empty
    K, N = 32, 2
    gl = np.array([2, 0, 1], np.int64)
    a_p, a_s = MX.mx_quant(np.ones((3, K)))
    w = np.stack([np.repeat(((np.arange(N) + 1) * 2.0 ** e)[:, None], K, 1) for e in range(3)])
    w_p = np.stack([MX.mx_quant(w[e])[0] for e in range(3)])
    w_s = np.stack([MX.mx_quant(w[e])[1] for e in range(3)])
    y = O.bf16_to_f32(MM.mx_grouped_gemm(gl, a_p, a_s, w_p, w_s))
    assert y.tolist() == [[32.0, 64.0], [32.0, 64.0], [128.0, 256.0]]


def test_mx_grouped_gemm_brute_force():
    rng = np.random.default_rng(6)
    E, N, K = 4, 5, 64
    gl = np.array([3, 0, 4, 2], np.int64)
    R = int(gl.sum())
    a_p, a_s = MX.mx_quant(rng.standard_normal((R, K)))
    w_p, w_s = zip(*(MX.mx_quant(rng.standard_normal((N, K)) * 0.01) for _ in range(E)))
    w_p, w_s = np.stack(w_p), np.stack(w_s)
    y = O.bf16_to_f32(MM.mx_grouped_gemm(gl, a_p, a_s, w_p, w_s))
    expert = np.repeat(np.arange(E), gl)          # row r belongs to expert expert[r]
    av = MX.e4m3_values()
    for r in range(R):
        e = int(expert[r])
        for n in range(N):
            acc = 0.0
            for k in range(K):
                acc += (av[a_p[r, k]] * 2.0 ** (int(a_s[r, k // 32]) - 127)
                        * av[w_p[e, n, k]] * 2.0 ** (int(w_s[e, n, k // 32]) - 127))
            assert abs(y[r, n] - acc) <= 2.0 ** -8 * abs(acc) + 1e-30


def _nearest_code(t):
    """E4M3 code of t by brute force over the code table: nearest value, ties to
    the even code, saturating at 448."""
    vals = MX.e4m3_values()[:0x7F]
    a = min(abs(float(t)), 448.0)
    d = np.abs(vals - a)
    cand = np.flatnonzero(d == d.min())
    c = int(cand[0]) if len(cand) == 1 else int(cand[cand % 2 == 0][0])
    return c | (0x80 if t < 0 else 0)


def test_swiglu_mx_quant_quantizes_the_bf16_value():
    # a SwiGLU output whose BF16 rounding moves it onto an E4M3 tie while its
    # fp32 value is off the tie: the code is the BF16 value's (ties to even),
    # not the fp32 value's
    I = 32
    from oracle.w8a8_ref import silu_spec
    grid = O.bf16_to_f32(O.f32_to_bf16(np.linspace(0.5, 6.0, 400).astype(np.float32)))
    found = None
    for gv in np.unique(grid):
        sg = silu_spec(np.array([gv], np.float32))[0]
        for uv in np.unique(grid):
            a32 = np.float32(sg * np.float32(uv))
            ab = O.bf16_to_f32(O.f32_to_bf16(np.array([a32], np.float32)))[0]
            # group amax 448 * 2**-5 = 14 fixes E = 3 - 8 = -5 (byte 122)
            if abs(a32) < 14 and _nearest_code(a32 * 32) != _nearest_code(ab * 32):
                found = (gv, uv, a32, ab)
                break
        if found:
            break
    assert found is not None
    gv, uv, a32, ab = found
    g = np.full((1, I), 0.0, np.float32)
    u = np.full((1, I), 0.0, np.float32)
    g[0, 0], u[0, 0] = gv, uv
    g[0, 1], u[0, 1] = 100.0, 0.140625          # silu(100) * 0.140625 = 14.0625 -> BF16 14.0625
    h = O.f32_to_bf16(np.concatenate([g, u], axis=1))
    p, sc, _ = MM.swiglu_mx_quant(h, I)
    amax = O.bf16_to_f32(O.f32_to_bf16(np.array([100.0 * 0.140625], np.float32)))[0]
    E = int(np.floor(np.log2(amax))) - 8
    assert sc[0, 0] == E + 127
    assert p[0, 0] == _nearest_code(ab * 2.0 ** -E)
    assert p[0, 0] != _nearest_code(float(a32) * 2.0 ** -E)


def test_mx_moe_chain_stages_and_float64_chain():
    E, H, I, bn, bk = 3, 64, 32, 32, 32
    gl = np.array([5, 0, 7], np.int64)
    R = int(gl.sum())
    # activations scaled so that the W13 outputs (rms about 3) reach the range
    # where SwiGLU is not symmetric in gate and up
    x = O.f32_to_bf16(O.bf16_to_f32(synth.activations(R, H, 0.0, seed=7)) * np.float32(64))
    w13, s13 = _random_stack(E, 2 * I, H, bn, bk, seed=8)
    w2, s2 = _random_stack(E, H, I, bn, bk, seed=9)
    p13, sc13 = MM.mx_moe_prepare(w13, s13, bn, bk)
    p2, sc2 = MM.mx_moe_prepare(w2, s2, bn, bk)
    st = MM.mx_moe_grouped(gl, x, p13, sc13, p2, sc2, keep=True)
    # stages
    q1, s1 = MX.mx_quant(O.bf16_to_f32(x))
    assert np.array_equal(st["q1"], q1) and np.array_equal(st["s1"], s1)
    assert np.array_equal(st["h"], MM.mx_grouped_gemm(gl, q1, s1, p13, sc13))
    q2, sq2, a = MM.swiglu_mx_quant(st["h"], I)
    assert np.array_equal(st["q2"], q2) and np.array_equal(st["a"], a)
    assert np.array_equal(st["y"], MM.mx_grouped_gemm(gl, q2, sq2, p2, sc2))
    # unquantized float64 chain on the resolved weights. Four MX roundings
    # (x, W13, a, W2) change an element by at most 1/16 of it, or 1/8 when a
    # group maximum saturates under the default scale rule, and by about 1/40
    # RMS: the rows land 5 to 12 % (normwise) from the float64 chain. A wrong
    # expert, a transposed W2 or gate and up swapped land 30 % to 180 % away.
    off = np.concatenate([[0], np.cumsum(gl)])
    xf = O.bf16_to_f32(x).astype(np.float64)
    y = O.bf16_to_f32(st["y"]).astype(np.float64)
    for e in range(E):
        a0, a1 = off[e], off[e + 1]
        if a1 == a0:
            continue
        W13 = O.bf16_to_f32(MX.mx_resolve(w13[e], s13[e], bn, bk)).astype(np.float64)
        W2 = O.bf16_to_f32(MX.mx_resolve(w2[e], s2[e], bn, bk)).astype(np.float64)
        hh = xf[a0:a1] @ W13.T
        aa = hh[:, :I] / (1.0 + np.exp(-hh[:, :I])) * hh[:, I:]
        ref = aa @ W2.T
        err = np.linalg.norm(y[a0:a1] - ref, axis=1) / np.linalg.norm(ref, axis=1)
        assert np.all(err < 0.25), (e, err)
