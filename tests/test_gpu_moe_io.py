"""Parity of the steps around the MoE chain (route, INT8 gather, weighted
combine, whole layer), through the C ABI, with the CPU oracle.

Counts, row orders, INT8 rows, scales and BF16 outputs are compared exactly.
Inputs are seeded (``synth`` or a seeded generator here); expected values come
only from ``oracle``.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests.conftest import gpu_available
from tests.gpu_util import bf16_dev, bf16_host, dev, host, show, sync

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

IO = O.moe_io


@pytest.fixture(scope="module")
def w():
    import moe_token_amax_amd as w
    return w


def _assert_eq(got, want, what):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{what}: {len(bad)} mismatches, first at {bad[:5].tolist()}: " \
                          f"got {got[tuple(bad[0])]} want {want[tuple(bad[0])]}"


def _ids(T, k, E, kind, seed):
    rng = np.random.default_rng(seed)
    if kind == "synth":                 # skewed top-k routing, distinct experts per token
        return synth.topk_routing(T, E, k, seed)[0]
    if kind == "uniform":               # experts may repeat within a token
        return rng.integers(0, E, (T, k)).astype(np.int32)
    if kind == "invalid":               # some ids outside [0, E) are dropped
        return rng.integers(-3, E + 3, (T, k)).astype(np.int32)
    if kind == "one":                   # every pair on one expert
        return np.full((T, k), E // 2, np.int32)
    if kind == "none":                  # every id dropped
        return np.where(rng.random((T, k)) < 0.5, -1, E).astype(np.int32)
    raise ValueError(kind)


def _route_full(ids, E):
    """Oracle route with row_token padded to T * top_k (the tail holds token 0)."""
    gl, rt, pr = IO.route(ids, E)
    full = np.zeros(ids.size, np.int32)
    full[:rt.size] = rt
    return gl, full, pr


# (T, top_k, E, ids): empty, single pair, the MoE workload's routing, many
# chunks of 1024 pairs with the largest expert count, one expert for every
# pair (4 chunks of 64 equal ids per wavefront), dropped ids. Up to 32 chunks
# of 1024 pairs take the one-launch kernel; past that the count / scan /
# place launches: 33 chunks with an 8-pair last chunk, 64 full chunks, the
# 40-chunk case with E = 1024, 512 chunks (T = 65536), one expert for 40000
# pairs, a single expert.
ROUTE_CASES = [(0, 8, 4, "uniform"), (1, 1, 1, "uniform"), (97, 8, 33, "invalid"),
               (2048, 8, 256, "synth"), (5000, 8, 1024, "uniform"), (3000, 1, 4, "one"),
               (1500, 6, 7, "invalid"), (333, 3, 1000, "synth"), (4096, 8, 64, "uniform"),
               (4097, 8, 7, "invalid"), (8192, 8, 256, "synth"), (65536, 8, 256, "synth"),
               (40000, 1, 9, "one"), (33 * 1024 + 5, 1, 1, "uniform"), (6000, 7, 1000, "invalid"),
               (33 * 1024 + 1, 1, 1024, "none"), (3000, 1, 4, "none")]


@pytest.mark.parametrize("T,k,E,kind", ROUTE_CASES)
def test_route_bit_exact(w, T, k, E, kind):
    show(f"moe_route T={T} k={k} E={E} {kind}")
    ids = _ids(T, k, E, kind, seed=T + k + E)
    gl, rt, pr = w.moe_route(dev(ids), E)
    sync()
    gl_o, rt_o, pr_o = _route_full(ids, E)
    _assert_eq(host(gl), gl_o, "group_list")
    _assert_eq(host(rt), rt_o, "row_token")
    _assert_eq(host(pr), pr_o, "pair_row")


def test_route_matches_grouped_rows_of_the_workload(w):
    # the MoE workload's expert-grouped rows are the route of its top-k ids
    m = synth.moe(T=2048, H=64, I=32, E=256, top_k=8, seed=0)
    gl, rt, _ = w.moe_route(dev(m.topk_ids), m.E)
    sync()
    _assert_eq(host(gl), m.group_list, "group_list")
    _assert_eq(host(rt), m.row_token.astype(np.int32), "row_token")


@pytest.mark.parametrize("T,H,R", [(64, 4096, 512), (50, 100, 130), (7, 16, 1), (300, 7168, 2400),
                                   (5, 33, 0)])
def test_gather_bit_exact(w, T, H, R):
    show(f"moe_gather T={T} H={H} R={R}")
    rng = np.random.default_rng(T * H + R)
    q = rng.integers(-127, 128, (T, H)).astype(np.int8)
    s = rng.uniform(1e-4, 1e-1, T).astype(np.float32)
    rt = rng.integers(0, T, R).astype(np.int32)
    if R >= 4:   # tokens outside [0, T) give zero rows with scale 0
        rt[[1, R // 2, R - 1]] = [-1, T, 2 ** 31 - 1]
    qr, sr = w.moe_gather(dev(q), dev(s), dev(rt))
    sync()
    ok = (rt >= 0) & (rt < T)
    want_q = np.zeros((R, H), np.int8)
    want_s = np.zeros(R, np.float32)
    if R:
        want_q[ok] = q[rt[ok]]            # a gather is its definition: row p = token rt[p]
        want_s[ok] = s[rt[ok]]
    _assert_eq(host(qr), want_q, "q_rows")
    _assert_eq(host(sr).view(np.uint32), want_s.view(np.uint32), "s_rows")


def test_gather_of_quantized_tokens_is_the_dispatch(w):
    # quantize on the GPU, gather on the GPU == the oracle's dispatch
    T, k, E, H = 96, 4, 12, 512
    x = synth.activations(T, H, 0.01, seed=21)
    ids = _ids(T, k, E, "synth", seed=21)
    _, rt, _ = IO.route(ids, E)
    q, s = w.dynamic_quant(bf16_dev(x))
    qr, sr = w.moe_gather(q, s, dev(rt.astype(np.int32)))
    sync()
    qo, so = IO.dispatch_int8(x, rt)
    _assert_eq(host(qr), qo, "q_rows")
    _assert_eq(host(sr).view(np.uint32), so.view(np.uint32), "s_rows")


@pytest.mark.parametrize("T,k,E,H,kind", [(64, 8, 16, 4096, "synth"), (40, 3, 5, 100, "invalid"),
                                          (33, 1, 4, 8, "uniform"), (256, 8, 256, 7168, "synth"),
                                          (10, 4, 3, 36, "uniform")])
def test_combine_bit_exact(w, T, k, E, H, kind):
    show(f"moe_combine T={T} k={k} H={H} {kind}")
    rng = np.random.default_rng(T * k + H)
    ids = _ids(T, k, E, kind, seed=T + H)
    _, rt, pr = IO.route(ids, E)
    R = rt.size
    y = O.f32_to_bf16((rng.standard_normal((R, H)) * 3).astype(np.float32))
    wts = rng.uniform(0.0, 1.0, (T, k)).astype(np.float32)
    wts[0, 0] = -0.5                          # a negative weight
    pr_dev = pr.copy()
    pr_want = pr.copy()
    if T > 3 and R > 0:                       # rows past R contribute nothing
        pr_dev[3, 0] = R + 5
        pr_want[3, 0] = -1
    out = w.moe_combine(bf16_dev(y), dev(pr_dev), dev(wts))
    sync()
    _assert_eq(bf16_host(out), IO.combine(y, pr_want, wts), "out")


def _moe_layer_inputs(T, k, E, H, I, kind, seed):
    x = synth.activations(T, H, 0.01, seed)
    if kind == "synth":
        ids, wts = synth.topk_routing(T, E, k, seed)
    else:
        ids = _ids(T, k, E, kind, seed)
        wts = np.random.default_rng(seed).uniform(0.0, 1.0, (T, k)).astype(np.float32)
    w13 = synth.int8_weight((E, 2 * I, H), seed, 6)
    w2 = synth.int8_weight((E, H, I), seed, 7)
    w13s = synth.scales((E, 2 * I), seed, 8)
    w2s = synth.scales((E, H), seed, 9)
    return x, ids, wts, w13, w13s, w2, w2s


# (T, top_k, E, H, I, ids): small experts, large experts (tile path), dropped
# ids, K not a multiple of 16 (VGPR-staged tiles, element gather / combine),
# a single token, the MoE workload's routing at a reduced width
LAYER_CASES = [(64, 4, 16, 256, 128, "synth"), (600, 2, 3, 512, 256, "uniform"),
               (50, 3, 5, 64, 32, "invalid"), (30, 2, 3, 100, 40, "uniform"),
               (1, 1, 1, 64, 32, "uniform"), (512, 8, 64, 256, 128, "synth")]


@pytest.mark.parametrize("T,k,E,H,I,kind", LAYER_CASES)
def test_moe_layer_bit_exact(w, T, k, E, H, I, kind):
    show(f"moe_layer T={T} k={k} E={E} H={H} I={I} {kind}")
    x, ids, wts, w13, w13s, w2, w2s = _moe_layer_inputs(T, k, E, H, I, kind, seed=T + E + H)
    w13p, w2p = w.prepack_weight(dev(w13)), w.prepack_weight(dev(w2))
    out = w.moe_layer(bf16_dev(x), dev(ids), dev(wts), w13p, dev(w13s), w2p, dev(w2s))
    # the same layer through the separate entry points
    gl, rt, pr = w.moe_route(dev(ids), E)
    q, s = w.dynamic_quant(bf16_dev(x))
    qr, sr = w.moe_gather(q, s, rt)
    y_rows = w.moe_grouped(qr, gl, w13p, dev(w13s), w2p, dev(w2s), x_scale=sr)
    out2 = w.moe_combine(y_rows, pr, dev(wts))
    sync()
    st = IO.moe_forward(x, ids, wts, w13, w13s, w2, w2s, keep=True)
    n = st["row_token"].size
    _assert_eq(bf16_host(y_rows)[:n], st["y_rows"], "y_rows")
    _assert_eq(bf16_host(out), st["out"], "out")
    _assert_eq(bf16_host(out2), st["out"], "out (separate entry points)")


@pytest.mark.timeout(600)
def test_moe_layer_config_sampled_tokens(w):
    """The MoE workload as a whole layer; the oracle recomputes sampled tokens,
    each from its own top-k experts (rows of the chain are independent)."""
    show("moe_layer full size, sampled tokens")
    m = synth.moe(seed=0)
    E, H, I, k = m.E, m.H, m.I, m.top_k
    per13 = w.packed_weight_bytes(1, 2 * I, H)
    per2 = w.packed_weight_bytes(1, H, I)
    w13p = torch.empty(E * per13, dtype=torch.uint8, device="cuda")
    w2p = torch.empty(E * per2, dtype=torch.uint8, device="cuda")
    for e in range(E):  # prepack expert by expert (bounded staging memory)
        w.prepack_weight(dev(m.w13(e)), out=w13p[e * per13:(e + 1) * per13])
        w.prepack_weight(dev(m.w2(e)), out=w2p[e * per2:(e + 1) * per2])
        m.drop_cache()
    out = w.moe_layer(bf16_dev(m.x_tokens), dev(m.topk_ids), dev(m.topk_weights), w13p,
                      dev(m.w13_scale), w2p, dev(m.w2_scale))
    oh = bf16_host(out)
    rng = np.random.default_rng(2)
    toks = sorted(set(rng.integers(0, m.T, 4).tolist()) | {0, m.T - 1})
    for t in toks:
        ex = m.topk_ids[t].astype(np.int64)
        w13 = np.stack([m.w13(int(e)) for e in ex])
        w2 = np.stack([m.w2(int(e)) for e in ex])
        local = np.arange(k, dtype=np.int32)[None, :]      # slot j -> local expert j
        want = IO.moe_forward(m.x_tokens[t:t + 1], local, m.topk_weights[t:t + 1], w13,
                              m.w13_scale[ex], w2, m.w2_scale[ex])
        _assert_eq(oh[t:t + 1], want, f"token {t}")
        m.drop_cache()
