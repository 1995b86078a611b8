"""Pins of the CPU oracle against facts other than itself (CPU only).

Each check ties one oracle function to a closed form, a hand-computed case, an
exact-rational brute force, a library routine or a worked example printed on
the pages, chosen so that a plausible slip (reciprocal instead of division,
dropped bias, swapped gate/up, transposed weight, wrong group offsets) fails.
"""

from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests.exact_fp import f32_round, frac, quant_row_exact, to_f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32(xs):
    return np.asarray(xs, dtype=np.float32)


def f32_hex(v) -> int:
    return int(np.float32(v).view(np.uint32))


# ---------------------------------------------------------------------------
# BF16 conversions
# ---------------------------------------------------------------------------

def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(200_000).astype(np.float32) * np.float32(50)
    # exact ties and near-ties around 1.0 and 256.0
    extra = f32([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20, -(1 + 2 ** -8),
                 256 + 1, 257.0, 3.0e38, -3.0e38, 1e-40, -1e-40, 0.0, -0.0])
    x = np.concatenate([x, extra])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.f32_to_bf16(x), ref)


def test_bf16_hand_values():
    # 1.0 = 0x3F80; 1 + 2^-8 is a tie between 0x3F80 and 0x3F81 -> even (0x3F80);
    # 1 + 3*2^-8 is a tie between 0x3F81 and 0x3F82 -> even (0x3F82).
    assert list(O.f32_to_bf16(f32([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -2.0]))) == \
        [0x3F80, 0x3F80, 0x3F82, 0xC000]
    assert list(O.bf16_to_f32(np.array([0x3F80, 0xC040, 0x0001], np.uint16))) == \
        [1.0, -3.0, np.float32(2.0 ** -133)]


# ---------------------------------------------------------------------------
# a1 dynamic quant
# ---------------------------------------------------------------------------

def test_quant_hand_rows():
    # amax 127 -> scale exactly 1.0; ties go to even: 2.5->2, -0.5->0, 1.5->2, -3.5->-4
    q, s = O.dynamic_quant_f32(f32([[127, 2.5, -0.5, 1.5, -3.5]]))
    assert f32_hex(s[0]) == 0x3F800000
    assert list(q[0]) == [127, 2, 0, 2, -4]
    # amax 254 -> scale exactly 2.0: 5/2=2.5->2, 7/2=3.5->4, -1/2=-0.5->0
    q, s = O.dynamic_quant_f32(f32([[254, 5, 7, -1]]))
    assert s[0] == 2.0 and list(q[0]) == [127, 2, 4, 0]


def test_quant_division_sensitive_rows():
    # These rows land within one fp32 rounding of a .5 tie, so the result
    # depends on evaluating fl32(x / fl32(amax/127)) and not x * (127/amax).
    # Expected codes computed exactly with rational arithmetic below.
    rows = [[22.0, -11.0], [15.25, 7.625], [12.75, 6.375]]
    for row in rows:
        s_exact, q_exact = quant_row_exact(row)
        q, s = O.dynamic_quant_f32(f32([row]))
        assert frac(s[0]) == s_exact
        assert list(q[0]) == q_exact
    # the hand values of those three rows
    assert list(O.dynamic_quant_f32(f32([[22.0, -11.0]]))[0][0]) == [127, -63]
    assert list(O.dynamic_quant_f32(f32([[15.25, 7.625]]))[0][0]) == [127, 64]
    assert list(O.dynamic_quant_f32(f32([[12.75, 6.375]]))[0][0]) == [127, 64]


def _recip_quant(x):
    """A planted mistake: multiply by 127/amax instead of dividing by the scale."""
    x = f32(x)
    amax = np.max(np.abs(x), axis=1)
    inv = (np.float32(127) / amax).astype(np.float32)
    return np.clip(np.rint(x * inv[:, None]), -127, 127).astype(np.int8)


def test_planted_reciprocal_is_caught():
    rows = f32([[22.0, -11.0], [15.25, 7.625], [12.75, 6.375]])
    good = O.dynamic_quant_f32(rows)[0]
    assert not np.array_equal(good, _recip_quant(rows))


def test_quant_exact_brute_force_random_rows():
    d = synth.tiny(seed=0)
    x = O.bf16_to_f32(d.x)
    q, s = O.dynamic_quant_f32(x)
    for m in range(x.shape[0]):
        s_exact, q_exact = quant_row_exact(x[m])
        assert frac(s[m]) == s_exact
        assert list(q[m]) == q_exact


def test_quant_near_tie_brute_force():
    # rows built so that many x/s land close to k + 0.5
    rng = np.random.default_rng(7)
    rows = []
    for _ in range(40):
        amax = np.float32(rng.uniform(0.5, 40))
        s = np.float32(amax / np.float32(127))
        ks = rng.integers(-126, 126, size=15)
        row = (ks + 0.5).astype(np.float64) * float(s)
        rows.append(np.concatenate([[amax], row]).astype(np.float32))
    x = np.stack(rows)
    q, s = O.dynamic_quant_f32(x)
    for m in range(x.shape[0]):
        s_exact, q_exact = quant_row_exact(x[m])
        assert frac(s[m]) == s_exact
        assert list(q[m]) == q_exact


def test_quant_invariants_and_zero_row():
    d = synth.prefill(seed=3, M=64)
    x = O.bf16_to_f32(d.x)
    x[5] = 0.0
    q, s = O.dynamic_quant_f32(x)
    assert np.all(np.abs(q.astype(np.int32)) <= 127)
    # row 5 is all zero -> scale 0, codes 0
    assert s[5] == 0.0 and not np.any(q[5])
    for m in range(x.shape[0]):
        if m == 5:
            continue
        j = int(np.argmax(np.abs(x[m])))
        assert abs(int(q[m, j])) == 127
        assert np.sign(q[m, j]) == np.sign(x[m, j])
        # sign(q) in {sign(x), 0}
        sq, sx = np.sign(q[m].astype(np.int32)), np.sign(x[m])
        assert np.all((sq == 0) | (sq == sx))
    # rows are independent: quantizing a gathered subset gives gathered results
    idx = np.array([7, 2, 2, 63, 0])
    q2, s2 = O.dynamic_quant_f32(x[idx])
    assert np.array_equal(q2, q[idx]) and np.array_equal(s2, s[idx])


def test_quant_empty():
    q, s = O.dynamic_quant_f32(np.zeros((0, 32), np.float32))
    assert q.shape == (0, 32) and s.shape == (0,)


# ---------------------------------------------------------------------------
# a3 INT32 accumulation
# ---------------------------------------------------------------------------

def _acc_loops(q, w):
    M, K = q.shape
    N = w.shape[0]
    out = np.zeros((M, N), np.int64)
    for m in range(M):
        for n in range(N):
            t = 0
            for k in range(K):
                t += int(q[m, k]) * int(w[n, k])
            out[m, n] = t
    return out


def test_acc_brute_force():
    rng = np.random.default_rng(11)
    q = rng.integers(-127, 128, size=(5, 37), dtype=np.int8)
    w = rng.integers(-127, 128, size=(7, 37), dtype=np.int8)
    assert np.array_equal(O.int8_matmul_acc(q, w), _acc_loops(q, w))
    # a transposed weight is caught
    w_sq = rng.integers(-127, 128, size=(37, 37), dtype=np.int8)
    q_sq = rng.integers(-127, 128, size=(37, 37), dtype=np.int8)
    assert not np.array_equal(O.int8_matmul_acc(q_sq, w_sq), _acc_loops(q_sq, w_sq.T.copy()))
    assert np.array_equal(O.int8_matmul_acc(q_sq, w_sq), _acc_loops(q_sq, w_sq))


def test_acc_hand_and_extremes():
    assert O.int8_matmul_acc(np.array([[1, 2]], np.int8), np.array([[3, 4]], np.int8))[0, 0] == 11
    K = 7168
    q = np.full((2, K), 127, np.int8)
    q[1] = -127
    w = np.full((1, K), 127, np.int8)
    acc = O.int8_matmul_acc(q, w)
    assert acc[0, 0] == K * 127 * 127 and acc[1, 0] == -K * 127 * 127


# ---------------------------------------------------------------------------
# a5 epilogue
# ---------------------------------------------------------------------------

def test_epilogue_hand_case():
    # 11 * 0.5 = 5.5; * 0.25 = 1.375; + 0.125 = 1.5 -> BF16 0x3FC0
    y = O.epilogue_bf16(np.array([[11]]), f32([0.5]), f32([0.25]),
                        O.f32_to_bf16(f32([0.125])))
    assert y[0, 0] == 0x3FC0
    # without the bias the value is 1.375 = 0x3FB0 (a dropped bias is caught)
    y = O.epilogue_bf16(np.array([[11]]), f32([0.5]), f32([0.25]), None)
    assert y[0, 0] == 0x3FB0


def _epilogue_exact(acc, xs, ws, b):
    t = f32_round(Fraction(int(acc)))
    t = f32_round(t * frac(xs))
    t = f32_round(t * frac(ws))
    if b is not None:
        t = f32_round(t + frac(b))
    return t


def test_epilogue_exact_rational_sequence():
    d = synth.tiny(seed=0)
    q, s = O.dynamic_quant(d.x)
    y, acc = O.linear(q, s, d.w, d.w_scale, d.bias)
    bias = O.bf16_to_f32(d.bias)
    rng = np.random.default_rng(5)
    for _ in range(300):
        m, n = int(rng.integers(16)), int(rng.integers(128))
        t = _epilogue_exact(acc[m, n], s[m], d.w_scale[n], bias[n])
        assert O.f32_to_bf16(f32([to_f32(t)]))[0] == y[m, n]


def test_epilogue_within_float64_bound():
    for d in (synth.tiny(seed=0), synth.prefill(seed=1, M=32)):
        q, s = O.dynamic_quant(d.x)
        y, acc = O.linear(q, s, d.w, d.w_scale, d.bias)
        ref = O.linear_ref64(acc, s, d.w_scale, d.bias)
        assert O.bf16_within_tolerance(y, ref).all()


# ---------------------------------------------------------------------------
# a6 / a8 grouped GEMM
# ---------------------------------------------------------------------------

def _golden_counts():
    with open(os.path.join(GOLDEN, "moe_group_counts.txt")) as f:
        lines = [l for l in f if not l.startswith("#") and l.strip()]
    return np.array([int(v) for v in lines[0].split()], np.int64)


def test_group_offsets_worked_counts():
    g = _golden_counts()
    assert list(g) == [12, 7, 0, 19]
    assert list(O.group_offsets(g)) == [0, 12, 19, 19, 38]
    assert list(np.bincount(O.expert_of_rows(g), minlength=4)) == [12, 7, 0, 19]


def test_grouped_gemm_brute_force_worked_counts():
    g = _golden_counts()
    R = int(g.sum())
    rng = np.random.default_rng(2)
    K, N = 24, 10
    q = rng.integers(-127, 128, size=(R, K), dtype=np.int8)
    w = rng.integers(-127, 128, size=(4, N, K), dtype=np.int8)
    acc = O.grouped_gemm_acc(q, g, w)
    for r in range(R):
        # find the owning expert by walking the counts
        e, left = 0, r
        while left >= g[e]:
            left -= g[e]
            e += 1
        for n in range(N):
            assert acc[r, n] == sum(int(q[r, k]) * int(w[e, n, k]) for k in range(K))
    xs = rng.uniform(0.1, 1, R).astype(np.float32)
    ws = rng.uniform(1e-3, 1e-2, (4, N)).astype(np.float32)
    y, _ = O.grouped_gemm_bf16(q, xs, g, w, ws)
    ex = O.expert_of_rows(g)
    ref = acc * xs[:, None].astype(np.float64) * ws[ex].astype(np.float64)
    assert O.bf16_within_tolerance(y, ref).all()


def test_grouped_gemm_single_hot_expert():
    g = np.array([0, 0, 9, 0, 0], np.int64)
    rng = np.random.default_rng(3)
    q = rng.integers(-127, 128, size=(9, 16), dtype=np.int8)
    w = rng.integers(-127, 128, size=(5, 6, 16), dtype=np.int8)
    assert np.array_equal(O.grouped_gemm_acc(q, g, w), O.int8_matmul_acc(q, w[2]))


# ---------------------------------------------------------------------------
# a7 SwiGLU + requant
# ---------------------------------------------------------------------------

def _ulp_err(approx, exact64):
    approx = approx.astype(np.float64)
    ulp = np.spacing(np.abs(exact64).astype(np.float32)).astype(np.float64)
    return np.abs(approx - exact64) / ulp


def test_exp_spec_accuracy():
    t = np.linspace(-87.0, 88.0, 2_000_001, dtype=np.float64).astype(np.float32)
    err = _ulp_err(O.exp_spec(t), np.exp(t.astype(np.float64)))
    assert err.max() < 2.0
    assert O.exp_spec(f32([0.0]))[0] == 1.0
    assert O.exp_spec(f32([1.0]))[0] == np.float32(math.e)
    assert O.exp_spec(f32([200.0]))[0] == np.inf
    assert O.exp_spec(f32([-200.0]))[0] == 0.0


def test_exp_spec_subnormal_range():
    t = np.linspace(-103.0, -87.5, 100_001).astype(np.float32)
    e = O.exp_spec(t)
    ex = np.exp(t.astype(np.float64))
    # absolute error of at most about one subnormal step (2^-149) plus 2 ulp of normals
    assert np.all(np.abs(e.astype(np.float64) - ex) <= 2.0 ** -148)


def test_silu_spec_values():
    g = f32([0.0, 20.0, -100.0, 1.0, -1.0, 100.0])
    s = O.silu_spec(g)
    assert s[0] == 0.0
    assert s[1] == np.float32(20.0 / (1.0 + math.exp(-20.0)))
    assert s[2] == 0.0 and np.signbit(s[2])
    assert s[5] == 100.0
    gg = np.linspace(-80, 80, 400_001).astype(np.float32)
    ref = gg.astype(np.float64) / (1.0 + np.exp(-gg.astype(np.float64)))
    nz = np.abs(ref) > 1e-30
    assert _ulp_err(O.silu_spec(gg)[nz], ref[nz]).max() < 4.0


def test_swiglu_gate_up_order():
    # one row, I = 1: gate = 2, up = 3 -> silu(2) * 3 (swapping gives silu(3) * 2)
    h = O.f32_to_bf16(f32([[2.0, 3.0]]))
    a = O.swiglu(h, 1)[0, 0]
    want = 2.0 / (1.0 + math.exp(-2.0)) * 3.0
    swapped = 3.0 / (1.0 + math.exp(-3.0)) * 2.0
    assert abs(a - want) <= 4 * np.spacing(np.float32(want))
    assert abs(a - swapped) > 0.1


def _swiglu_quant_exact(hrow_f32, inter):
    """Requant of a row from the oracle's fp32 SwiGLU values, exactly."""
    a = O.swiglu(O.f32_to_bf16(hrow_f32[None, :]), inter)[0]
    return quant_row_exact(a)


def test_swiglu_quant_brute_force():
    rng = np.random.default_rng(9)
    inter = 24
    h = rng.standard_normal((12, 2 * inter)).astype(np.float32) * np.float32(3)
    h[3] = 0.0                                       # all-zero row -> scale 0
    hb = O.f32_to_bf16(h)
    q, s = O.swiglu_quant(hb, inter)
    for r in range(h.shape[0]):
        s_exact, q_exact = _swiglu_quant_exact(O.bf16_to_f32(hb[r]), inter)
        assert frac(s[r]) == s_exact
        assert list(q[r]) == q_exact
    assert s[3] == 0 and not q[3].any()
    # and the fp32 SwiGLU values themselves against float64
    a = O.swiglu(hb, inter)
    hf = O.bf16_to_f32(hb).astype(np.float64)
    ref = hf[:, :inter] / (1 + np.exp(-hf[:, :inter])) * hf[:, inter:]
    assert np.all(np.abs(a - ref) <= 4 * np.spacing(np.abs(ref).astype(np.float32)) + 1e-38)


# ---------------------------------------------------------------------------
# MoE chain
# ---------------------------------------------------------------------------

def _tiny_moe(seed=0):
    g = _golden_counts()
    E, H, I = 4, 64, 32
    R = int(g.sum())
    x = synth.activations(R, H, 0.01, seed)
    w13 = synth.int8_weight((E, 2 * I, H), seed, 6)
    w2 = synth.int8_weight((E, H, I), seed, 7)
    w13s = synth.scales((E, 2 * I), seed, 8)
    w2s = synth.scales((E, H), seed, 9)
    return g, x, w13, w13s, w2, w2s


def test_moe_chain_composition_and_bound():
    g, x, w13, w13s, w2, w2s = _tiny_moe()
    st = O.moe_grouped(g, w13, w13s, w2, w2s, x_bits=x, keep=True)
    # stage-by-stage recomposition by hand
    q, s = O.dynamic_quant(x)
    assert np.array_equal(q, st["q"]) and np.array_equal(s, st["x_scale"])
    ex = O.expert_of_rows(g)
    for r in range(len(ex)):
        e = ex[r]
        acc = O.int8_matmul_acc(q[r:r + 1], w13[e])
        assert np.array_equal(acc, st["acc13"][r:r + 1])
        h = O.epilogue_bf16(acc, s[r:r + 1], w13s[e])
        assert np.array_equal(h, st["h"][r:r + 1])
    # final outputs within tolerance of float64 from the oracle's own requant
    ref = st["acc2"] * st["s2"][:, None].astype(np.float64) * w2s[ex].astype(np.float64)
    assert O.bf16_within_tolerance(st["y"], ref).all()
    # skip-requant branch: INT8 rows + scale in gives identical results
    y2 = O.moe_grouped(g, w13, w13s, w2, w2s, q=q, x_scale=s)
    assert np.array_equal(y2, st["y"])


def test_routing_generator_shapes():
    m = synth.moe(T=64, H=32, I=16, E=16, top_k=4, seed=0)
    assert m.R == 256 and m.group_list.sum() == 256
    assert (np.diff(m.row_token.reshape(-1)) != 0).any()
    ex = O.expert_of_rows(m.group_list)
    # each token appears top_k times, at most once per expert
    pairs = set(zip(m.row_token.tolist(), ex.tolist()))
    assert len(pairs) == 256
