"""Pins of the MoE dispatch / combine oracle (oracle/moe_io_ref.py), CPU only:
hand-computed routes and combines, a brute-force check of the expert-major
order, the page's claim that quantizing the tokens before the gather equals
quantizing the gathered rows, one-hot combine weights, and a float64 bound.
A slip such as an unstable or token-major order, a dropped slot, a weight
applied to the wrong row or a missing invalid-id guard fails one of them.
"""

from __future__ import annotations

import numpy as np

import oracle as O
import synth

IO = O.moe_io


def f32(xs):
    return np.asarray(xs, dtype=np.float32)


def test_route_hand():
    gl, rt, pr = IO.route(np.array([[2, 0], [0, 1], [2, 2]]), 3)
    # expert 0: pairs (0,1), (1,0); expert 1: (1,1); expert 2: (0,0), (2,0), (2,1)
    assert gl.tolist() == [2, 1, 3]
    assert rt.tolist() == [0, 1, 1, 0, 2, 2]
    assert pr.tolist() == [[3, 0], [1, 2], [4, 5]]
    # ids outside [0, E) are dropped
    gl, rt, pr = IO.route(np.array([[2, 5], [0, 1], [-1, 2]]), 3)
    assert gl.tolist() == [1, 1, 2]
    assert rt.tolist() == [1, 1, 0, 2]
    assert pr.tolist() == [[2, -1], [0, 1], [-1, 3]]


def test_route_brute_force():
    rng = np.random.default_rng(3)
    T, k, E = 97, 8, 33
    ids = rng.integers(-2, E + 2, (T, k))
    gl, rt, pr = IO.route(ids, E)
    off = 0
    seen = set()
    for e in range(E):
        want = [(t, j) for t in range(T) for j in range(k) if ids[t, j] == e]   # pair order
        assert gl[e] == len(want)
        for p, (t, j) in enumerate(want):
            assert rt[off + p] == t and pr[t, j] == off + p
            seen.add((t, j))
        off += len(want)
    assert off == rt.size
    for t in range(T):
        for j in range(k):
            if (t, j) not in seen:
                assert pr[t, j] == -1 and not (0 <= ids[t, j] < E)


def test_dispatch_quantizes_once():
    # per-token quant before the gather == per-row quant after it ([DSV4] §三:
    # the INT8 dispatch path and the quant-in-the-runner path agree)
    x = synth.activations(40, 96, 0.02, seed=4)
    ids = np.random.default_rng(4).integers(0, 6, (40, 3))
    _, rt, _ = IO.route(ids, 6)
    q_rows, s_rows = IO.dispatch_int8(x, rt)
    q_after, s_after = O.dynamic_quant(x[rt])
    assert np.array_equal(q_rows, q_after)
    assert np.array_equal(s_rows.view(np.uint32), s_after.view(np.uint32))


def test_combine_hand():
    y = O.f32_to_bf16(f32([[1.0, 2.0], [0.5, -4.0], [3.0, 0.25]]))
    pr = np.array([[0, 2], [1, -1]])
    w = f32([[0.5, 0.25], [2.0, 9.0]])
    out = O.bf16_to_f32(IO.combine(y, pr, w))
    # token 0: 0.5 * (1, 2) + 0.25 * (3, 0.25); token 1: 2 * (0.5, -4), its second slot dropped
    assert out.tolist() == [[1.25, 1.0625], [1.0, -8.0]]


def test_combine_one_hot_and_bound():
    rng = np.random.default_rng(9)
    T, k, H, E = 30, 4, 64, 5
    ids = rng.integers(0, E, (T, k))
    _, rt, pr = IO.route(ids, E)
    y = O.f32_to_bf16(rng.standard_normal((rt.size, H)).astype(np.float32))
    for j in range(k):
        w = np.zeros((T, k), np.float32)
        w[:, j] = 1.0
        assert np.array_equal(IO.combine(y, pr, w), y[pr[:, j]])
    w = rng.uniform(0.0, 1.0, (T, k)).astype(np.float32)
    out = O.bf16_to_f32(IO.combine(y, pr, w)).astype(np.float64)
    yf = O.bf16_to_f32(y).astype(np.float64)
    ref = sum(w[:, j].astype(np.float64)[:, None] * yf[pr[:, j]] for j in range(k))
    mag = sum(np.abs(w[:, j].astype(np.float64)[:, None] * yf[pr[:, j]]) for j in range(k))
    assert np.all(np.abs(out - ref) <= 2.0 ** -8 * np.abs(ref) + 2.0 * k * 2.0 ** -24 * mag + 1e-30)


def test_moe_forward_matches_bf16_dispatch():
    # the whole layer with the INT8 dispatch equals the layer whose runner
    # quantizes the gathered BF16 rows itself
    rng = np.random.default_rng(11)
    T, k, E, H, I = 24, 3, 5, 64, 32
    x = synth.activations(T, H, 0.02, seed=12)
    ids = rng.integers(0, E, (T, k))
    wts = rng.uniform(0.0, 1.0, (T, k)).astype(np.float32)
    w13 = synth.int8_weight((E, 2 * I, H), 12, 1)
    w2 = synth.int8_weight((E, H, I), 12, 2)
    s13 = synth.scales((E, 2 * I), 12, 3)
    s2 = synth.scales((E, H), 12, 4)
    got = IO.moe_forward(x, ids, wts, w13, s13, w2, s2, keep=True)
    gl, rt, pr = IO.route(ids, E)
    y_rows = O.moe_grouped(gl, w13, s13, w2, s2, x_bits=x[rt])
    assert np.array_equal(got["y_rows"], y_rows)
    assert np.array_equal(got["out"], IO.combine(y_rows, pr, wts))
