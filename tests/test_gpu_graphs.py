"""Entry points captured in HIP graphs and replayed (GPU).

Every call only enqueues work on its stream, so a caller may capture it. Each
case captures a path once, then replays the graph three times; before every
replay the outputs are overwritten on the host's stream (eager work between
the replays) and after it they are compared: with the oracle where the path is
bit-exact to it, else bit for bit with the same call run eagerly (whose own
parity tests are elsewhere). This covers workspace state a call must rewrite
itself (schedules, work-queue counters, the allocation-free scratch)."""

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
REPLAYS = 3


@pytest.fixture(scope="module")
def w():
    import moe_token_amax_amd as w
    return w


def _assert_eq(got, want, what):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{what}: {len(bad)} mismatches, first at {bad[:5].tolist()}"


def _spoil(outs):
    for o in outs:
        if o.dtype in (torch.bfloat16, torch.float16):
            o.view(torch.int16).fill_(-1)
        else:
            o.fill_(-7)


def _replayed(fn, outs, check):
    """Capture fn once (after an eager warm-up run), then replay it REPLAYS
    times, spoiling the outputs eagerly before each replay and checking them
    after it."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    sync()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for r in range(REPLAYS):
        _spoil(outs)
        sync()
        g.replay()
        sync()
        check(r)


def test_decode_step_graph(w):
    """The decode step's three dispatches (fused quant at M = 1, row-major
    codes at M = 4, packed codes at M = 16) in one graph."""
    show("graph: decode step")
    K, N = 2048, 512
    d = synth.dense(16, K, N, outlier_frac=0.01, bias=True, seed=21)
    x = bf16_dev(d.x)
    wp = w.prepack_weight(dev(d.w))
    ws_, b = dev(d.w_scale), bf16_dev(d.bias)
    y1 = torch.empty((1, N), dtype=torch.bfloat16, device="cuda")
    y4 = torch.empty((4, N), dtype=torch.bfloat16, device="cuda")
    y16 = torch.empty((16, N), dtype=torch.bfloat16, device="cuda")
    q4 = torch.empty((4, K), dtype=torch.int8, device="cuda")
    s4 = torch.empty((4,), dtype=torch.float32, device="cuda")
    q16 = torch.empty((w.packed_weight_bytes(1, 16, K),), dtype=torch.uint8, device="cuda")
    s16 = torch.empty((16,), dtype=torch.float32, device="cuda")
    wss = {M: torch.empty((max(1, w.linear_workspace_bytes(M, N, K)),), dtype=torch.uint8, device="cuda")
           for M in (1, 4, 16)}

    def step():
        w.linear_bf16(x[:1], wp, ws_, N, bias=b, y=y1, workspace=wss[1])
        w.dynamic_quant(x[:4], q4, s4)
        w.linear(q4, s4, wp, ws_, N, bias=b, y=y4, workspace=wss[4])
        w.dynamic_quant_packed(x[:16], q16, s16)
        w.linear_packed(q16, s16, K, wp, ws_, N, bias=b, y=y16, workspace=wss[16])

    want = {}
    for M in (1, 4, 16):
        qo, so = O.dynamic_quant(d.x[:M])
        want[M] = O.linear(qo, so, d.w, d.w_scale, d.bias)[0]

    def check(r):
        _assert_eq(bf16_host(y1), want[1], f"replay {r} M=1")
        _assert_eq(bf16_host(y4), want[4], f"replay {r} M=4")
        _assert_eq(bf16_host(y16), want[16], f"replay {r} M=16")

    _replayed(step, [y1, y4, y16, q4, s4, q16, s16], check)


def test_prefill_linear_graph(w):
    """Packed quant + the LDS-DMA tile kernel (several tiles, ragged edges)."""
    show("graph: prefill-sized linear")
    M, K, N = 300, 1088, 600
    d = synth.dense(M, K, N, outlier_frac=0.01, bias=True, seed=22)
    x = bf16_dev(d.x)
    wp = w.prepack_weight(dev(d.w))
    ws_, b = dev(d.w_scale), bf16_dev(d.bias)
    q = torch.empty((w.packed_weight_bytes(1, M, K),), dtype=torch.uint8, device="cuda")
    s = torch.empty((M,), dtype=torch.float32, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty((max(1, w.linear_workspace_bytes(M, N, K)),), dtype=torch.uint8, device="cuda")

    def step():
        w.dynamic_quant_packed(x, q, s)
        w.linear_packed(q, s, K, wp, ws_, N, bias=b, y=y, workspace=ws)

    qo, so = O.dynamic_quant(d.x)
    want = O.linear(qo, so, d.w, d.w_scale, d.bias)[0]
    _replayed(step, [y, q, s], lambda r: _assert_eq(bf16_host(y), want, f"replay {r}"))


def test_moe_chain_graph(w):
    show("graph: INT8 MoE chain")
    counts, H, I = [0, 200, 3, 0, 70], 256, 128
    g = np.asarray(counts, np.int64)
    E, R = len(g), int(g.sum())
    x = synth.activations(R, H, 0.01, 23)
    w13 = synth.int8_weight((E, 2 * I, H), 23, 6)
    w2 = synth.int8_weight((E, H, I), 23, 7)
    w13s = synth.scales((E, 2 * I), 23, 8)
    w2s = synth.scales((E, H), 23, 9)
    want = O.moe_grouped(g, w13, w13s, w2, w2s, x_bits=x)
    want = want["y"] if isinstance(want, dict) else want
    w13p, w2p = w.prepack_weight(dev(w13)), w.prepack_weight(dev(w2))
    xd, gd, w13sd, w2sd = bf16_dev(x), dev(g), dev(w13s), dev(w2s)
    y = torch.empty((R, H), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty((w.moe_workspace_bytes(R, E, H, I),), dtype=torch.uint8, device="cuda")
    _replayed(lambda: w.moe_grouped(xd, gd, w13p, w13sd, w2p, w2sd, y=y, workspace=ws), [y],
              lambda r: _assert_eq(bf16_host(y), want, f"replay {r}"))


def test_moe_layer_graph(w):
    """Quantize, route, gather, chain, combine: the whole layer in one graph."""
    show("graph: INT8 MoE layer")
    T, k, E, H, I = 64, 4, 16, 256, 128
    x = synth.activations(T, H, 0.01, 24)
    ids = synth.topk_routing(T, E, k, 24)[0]
    wts = np.random.default_rng(24).uniform(0.0, 1.0, (T, k)).astype(np.float32)
    w13 = synth.int8_weight((E, 2 * I, H), 24, 6)
    w2 = synth.int8_weight((E, H, I), 24, 7)
    w13s = synth.scales((E, 2 * I), 24, 8)
    w2s = synth.scales((E, H), 24, 9)
    want = IO.moe_forward(x, ids, wts, w13, w13s, w2, w2s)
    want = want["out"] if isinstance(want, dict) else want
    w13p, w2p = w.prepack_weight(dev(w13)), w.prepack_weight(dev(w2))
    xd, idd, wtd, w13sd, w2sd = bf16_dev(x), dev(ids), dev(wts), dev(w13s), dev(w2s)
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty((w.moe_layer_workspace_bytes(T, k, E, H, I),), dtype=torch.uint8, device="cuda")
    _replayed(lambda: w.moe_layer(xd, idd, wtd, w13p, w13sd, w2p, w2sd, out=out, workspace=ws), [out],
              lambda r: _assert_eq(bf16_host(out), want, f"replay {r}"))


def test_route_three_launch_graph(w):
    """The count / scan / place route (past 32768 pairs), whose count table
    lives in pair_row between its launches."""
    show("graph: route, 40000 pairs")
    T, k, E = 5000, 8, 256
    ids = synth.topk_routing(T, E, k, 25)[0]
    gl_o, rt_o, pr_o = IO.route(ids, E)
    rt_full = np.zeros(T * k, np.int32)
    rt_full[:rt_o.size] = rt_o
    idd = dev(ids)
    gl = torch.empty((E,), dtype=torch.int64, device="cuda")
    rt = torch.empty((T * k,), dtype=torch.int32, device="cuda")
    pr = torch.empty((T, k), dtype=torch.int32, device="cuda")

    def check(r):
        _assert_eq(host(gl), gl_o, f"replay {r} group_list")
        _assert_eq(host(rt), rt_full, f"replay {r} row_token")
        _assert_eq(host(pr), pr_o, f"replay {r} pair_row")

    _replayed(lambda: w.moe_route(idd, E, gl, rt, pr), [gl, rt, pr], check)


def test_noalloc_grouped_graph(w):
    """The allocation-free grouped GEMM keeps its schedule in the library's own
    device array: every replay must rebuild it."""
    show("graph: allocation-free grouped GEMM")
    counts, N, K = [12, 7, 0, 19, 130], 192, 320
    g = np.asarray(counts, np.int64)
    E, R = len(g), int(g.sum())
    rng = np.random.default_rng(26)
    a = rng.integers(-127, 128, (R, K), dtype=np.int8)
    s = (rng.random(R, dtype=np.float32) * 0.01 + 1e-3).astype(np.float32)
    wt = synth.int8_weight((E, N, K), 26)
    wsc = synth.scales((E, N), 26)
    want = np.concatenate([O.int8_matmul_acc(a[o:o + n], wt[e]) for e, (o, n) in
                           enumerate(zip(np.concatenate([[0], np.cumsum(g)[:-1]]), g))]).astype(np.int32)
    ad, sd, gd, wp, wsd = dev(a), dev(s), dev(g), w.prepack_weight(dev(wt)), dev(wsc)
    y = torch.empty((R, N), dtype=torch.int32, device="cuda")
    _replayed(lambda: w.grouped_gemm_noalloc(ad, sd, gd, wp, wsd, N, y, out=w.OUT_I32), [y],
              lambda r: _assert_eq(host(y), want, f"replay {r}"))


def _mx_stack(E, N, K, seed):
    r = np.random.default_rng([seed, 31])
    wq = synth.e4m3_bits(r.standard_normal((E, N, K), dtype=np.float32))
    sc = r.uniform(1e-3, 1e-2, size=(E, -(-N // 128), -(-K // 128))).astype(np.float32)
    return wq, sc


def test_mx_moe_chain_graph(w):
    show("graph: MXFP8 MoE chain")
    counts, H, I = [12, 7, 0, 19], 256, 128
    gl = np.asarray(counts, np.int64)
    E, R = len(gl), int(gl.sum())
    x = O.f32_to_bf16((np.random.default_rng(27).standard_normal((R, H)) * 8).astype(np.float32))
    w13q, s13 = _mx_stack(E, 2 * I, H, 27)
    w2q, s2 = _mx_stack(E, H, I, 28)
    _, p13 = w.mx_moe_prepare(dev(w13q), dev(s13), 128, 128)
    _, p2 = w.mx_moe_prepare(dev(w2q), dev(s2), 128, 128)
    xd, gd = bf16_dev(x), dev(gl)
    ws = torch.empty((w.mx_moe_workspace_bytes(R, E, H, I),), dtype=torch.uint8, device="cuda")
    want = bf16_host(w.mx_moe_grouped(xd, gd, p13, p2, I, workspace=ws))
    y = torch.empty((R, H), dtype=torch.bfloat16, device="cuda")
    _replayed(lambda: w.mx_moe_grouped(xd, gd, p13, p2, I, y=y, workspace=ws), [y],
              lambda r: _assert_eq(bf16_host(y), want, f"replay {r} (against the eager call)"))


@pytest.mark.parametrize("fmt", ["int4", "fp4"])
def test_lowbit_moe_chain_graph(w, fmt):
    show(f"graph: {fmt} MoE chain")
    counts, H, I = [1, 2, 0, 64, 65], 128, 96
    gl = np.asarray(counts, np.int64)
    E, R = len(gl), int(gl.sum())
    x = O.f32_to_bf16((np.random.default_rng(29).standard_normal((R, H)) * 4).astype(np.float32))
    r = np.random.default_rng(30)
    w13 = torch.from_numpy(O.f32_to_bf16((r.standard_normal((E * 2 * I, H)) * 0.02).astype(np.float32))
                           .view(np.int16)).cuda().view(torch.bfloat16)
    w2 = torch.from_numpy(O.f32_to_bf16((r.standard_normal((E * H, I)) * 0.02).astype(np.float32))
                          .view(np.int16)).cuda().view(torch.bfloat16)
    quant = w.w4a16_quant_weight if fmt == "int4" else w.fp4_quant_weight
    code = w.LOWBIT_INT4 if fmt == "int4" else w.LOWBIT_FP4
    p13 = torch.cat([quant(w13[e * 2 * I:(e + 1) * 2 * I])[2] for e in range(E)])
    p2 = torch.cat([quant(w2[e * H:(e + 1) * H])[2] for e in range(E)])
    xd, gd = bf16_dev(x), dev(gl)
    ws = torch.empty((w.w4a16_moe_workspace_bytes(R, H, I),), dtype=torch.uint8, device="cuda")
    want = bf16_host(w.w4a16_moe_grouped(xd, gd, p13, p2, I, fmt=code, workspace=ws))
    y = torch.empty((R, H), dtype=torch.bfloat16, device="cuda")
    _replayed(lambda: w.w4a16_moe_grouped(xd, gd, p13, p2, I, fmt=code, y=y, workspace=ws), [y],
              lambda r: _assert_eq(bf16_host(y), want, f"replay {r} (against the eager call)"))
