"""Parity of the HIP path (through the C ABI) with the CPU oracle.

INT8 codes, scales, INT32 accumulators and the BF16 outputs of the canonical
epilogue are compared bit for bit; BF16 outputs are also checked against the
unrounded float64 value with max(2**-8 * |ref|, 1e-5). Inputs come from the
seeded generators in ``synth``; expected values only from ``oracle``.
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


# ---------------------------------------------------------------------------
# dynamic quant
# ---------------------------------------------------------------------------

QUANT_SHAPES = [(16, 256), (1, 7168), (64, 7168), (5, 8), (3, 37), (7, 100), (4, 8200),
                (9, 16384), (130, 4096), (2, 1)]


@pytest.mark.parametrize("M,K", QUANT_SHAPES)
def test_dynamic_quant_bit_exact(w, M, K):
    show(f"dynamic_quant M={M} K={K}")
    xb = synth.activations(M, K, 0.01, seed=M * 1000 + K)
    if M > 2:
        xb[1] = 0  # all-zero row
    q, s = w.dynamic_quant(bf16_dev(xb))
    sync()
    qo, so = O.dynamic_quant(xb)
    _assert_eq(host(s).view(np.uint32), so.view(np.uint32), "scale")
    _assert_eq(host(q), qo, "q")


def test_dynamic_quant_ties(w):
    # rows whose elements sit exactly on .5 after division
    rows = np.array([[127, 2.5, -0.5, 1.5, -3.5, 0, 0, 0],
                     [254, 5, 7, -1, 0, 0, 0, 0],
                     [22, -11, 0, 0, 0, 0, 0, 0],
                     [15.25, 7.625, 0, 0, 0, 0, 0, 0]], np.float32)
    xb = O.f32_to_bf16(rows)
    q, s = w.dynamic_quant(bf16_dev(xb))
    sync()
    qo, so = O.dynamic_quant(xb)
    _assert_eq(host(q), qo, "q")
    _assert_eq(host(s), so, "scale")


@pytest.mark.parametrize("M,K", [(256, 8192), (1024, 4096)])
def test_dynamic_quant_near_ties(w, M, K):
    """The kernels take the code from x * rcp(s) unless that lands within 2^-14 of
    a half-integer, where the IEEE division decides. Random values put hundreds
    of elements in that band and in the band from 2^-14 to 2^-12 next to it
    (decided by the reciprocal alone); every code must match the oracle's.
    M <= 512 and M > 512 take different kernels."""
    xb = synth.activations(M, K, 0.01, seed=99 + M)
    x = O.bf16_to_f32(xb).astype(np.float64)
    s = O.dynamic_quant_f32(O.bf16_to_f32(xb))[1].astype(np.float64)
    t = np.abs(x / np.where(s > 0, s, 1.0)[:, None])
    d = np.abs(t - np.floor(t) - 0.5)
    inner = int((d < 2.0 ** -14).sum())
    outer = int(((d >= 2.0 ** -14) & (d < 2.0 ** -12)).sum())
    assert inner >= 20 and outer >= 50, (inner, outer)
    show(f"near-tie elements: {inner} within 2^-14, {outer} from 2^-14 to 2^-12")
    q, sc = w.dynamic_quant(bf16_dev(xb))
    qp, scp = w.dynamic_quant_packed(bf16_dev(xb))
    sync()
    qo, so = O.dynamic_quant(xb)
    _assert_eq(host(q), qo, "q")
    _assert_eq(_unpack_codes(host(qp), M, K), qo, "q (blocks)")


def test_dynamic_quant_empty(w):
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    q, s = w.dynamic_quant(x)
    assert q.shape == (0, 64) and s.shape == (0,)


# ---------------------------------------------------------------------------
# prepack + dense linear
# ---------------------------------------------------------------------------

def _run_linear(w, d: synth.Dense, out):
    xb = bf16_dev(d.x)
    q, s = w.dynamic_quant(xb)
    wp = w.prepack_weight(dev(d.w))
    y = w.linear(q, s, wp, dev(d.w_scale), d.N,
                 bias=None if d.bias is None else bf16_dev(d.bias), out=out)
    sync()
    return q, s, y


LINEAR_SHAPES = [  # M, K, N, bias
    (16, 256, 128, True), (1, 64, 16, False), (17, 100, 50, True), (3, 37, 5, False),
    (33, 448, 96, True), (64, 1024, 192, False), (129, 320, 144, True), (300, 512, 260, False),
    (4, 7168, 512, False), (16, 7168, 256, True),
    # decode kernel, 16-byte rows with a ragged last k-block (K % 64 == 16)
    (4, 2064, 160, True), (40, 1040, 96, False),
    # prefill-sized M (LDS-DMA tiles): ragged K (K % 64 != 0), tiny K, N tails,
    # a single partial 256-row tile, several tiles in both directions
    (100, 80, 300, True), (65, 16, 40, False), (257, 4096, 512, True), (520, 1088, 600, False),
    (96, 48, 16, True),
    # prefill-sized M with K % 16 != 0 (VGPR-staged fallback)
    (65, 100, 50, True), (200, 37, 33, False),
    # 33..64 rows with K % 16 != 0: the element-wise decode kernel on two
    # 32-row groups of 2 x 2 blocks, a partial second group and N tail
    (48, 100, 72, True), (33, 200, 40, False),
]


@pytest.mark.parametrize("M,K,N,bias", LINEAR_SHAPES)
def test_linear_acc_and_bf16_bit_exact(w, M, K, N, bias):
    show(f"linear M={M} K={K} N={N} bias={bias}")
    d = synth.dense(M, K, N, outlier_frac=0.01, bias=bias, seed=M + K + N)
    q, s, acc = _run_linear(w, d, w.OUT_I32)
    qo, so = O.dynamic_quant(d.x)
    _assert_eq(host(q), qo, "q")
    acc_o = O.int8_matmul_acc(qo, d.w)
    _assert_eq(host(acc), acc_o.astype(np.int32), "acc")
    _, _, y = _run_linear(w, d, w.OUT_BF16)
    yo, _ = O.linear(qo, so, d.w, d.w_scale, d.bias)
    yh = bf16_host(y)
    _assert_eq(yh, yo, "y")
    assert O.bf16_within_tolerance(yh, O.linear_ref64(acc_o, so, d.w_scale, d.bias)).all()


def test_tiny_config(w):
    """The tiny config through quant + linear and through the BF16-input linear
    the benchmark step uses (quant inside the product kernel: 16 x 256 values)."""
    d = synth.tiny(seed=0)
    _, _, y = _run_linear(w, d, w.OUT_BF16)
    y_in = w.linear_bf16(bf16_dev(d.x), w.prepack_weight(dev(d.w)), dev(d.w_scale), d.N,
                         bias=bf16_dev(d.bias))
    sync()
    qo, so = O.dynamic_quant(d.x)
    yo, _ = O.linear(qo, so, d.w, d.w_scale, d.bias)
    _assert_eq(bf16_host(y), yo, "tiny y")
    _assert_eq(bf16_host(y_in), yo, "tiny y (BF16 input)")


def _decode_dispatch(w, M, x, wp, ws_, N, K, bias=None):
    """The entry points a decode step uses for M rows: BF16 straight into the
    linear (quant fused into the product) for 1 or 2 rows and up to 16 rows of
    M * K <= 16384 values;
    else row-major codes below 16 rows and codes in the packed 1 KB blocks from
    16 rows up."""
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    wsp = torch.empty((max(1, w.linear_workspace_bytes(M, N, K)),), dtype=torch.uint8,
                      device="cuda")
    if (M <= 2 or (M <= 16 and M * K <= 16384)) and K <= 16384 and K % 8 == 0:
        w.linear_bf16(x, wp, ws_, N, bias=bias, y=y, workspace=wsp)
        return "bf16 in (fused quant)", None, y
    if M >= 16 and K % 8 == 0:
        qp, sp = w.dynamic_quant_packed(x)
        w.linear_packed(qp, sp, K, wp, ws_, N, bias=bias, y=y, workspace=wsp)
        return "packed codes", _unpack_codes(host(qp), M, K), y
    q, s = w.dynamic_quant(x)
    w.linear(q, s, wp, ws_, N, bias=bias, y=y, workspace=wsp)
    return "row-major codes", host(q), y


@pytest.mark.parametrize("M", [1, 2, 4, 16, 64])
def test_decode_config_full(w, M):
    """The decode workload in full (M x 4096 x 7168), through the same entry
    points and workspace the benchmark step uses; codes and BF16 outputs equal
    the oracle's bit for bit."""
    d = synth.decode(seed=0, M=M)
    wp = w.prepack_weight(dev(d.w))
    path, q, y = _decode_dispatch(w, M, bf16_dev(d.x), wp, dev(d.w_scale), d.N, d.K)
    sync()
    show(f"decode M={M}: {path}")
    qo, so = O.dynamic_quant(d.x)
    if q is not None:
        _assert_eq(q, qo, "q")
    yo, acc = O.linear(qo, so, d.w, d.w_scale, None)
    yh = bf16_host(y)
    _assert_eq(yh, yo, f"y ({path})")
    assert O.bf16_within_tolerance(yh, O.linear_ref64(acc, so, d.w_scale, None)).all()


@pytest.mark.timeout(600)
def test_prefill_config_full(w):
    """The prefill workload in full (8192 x 4096 x 7168 with bias), every row:
    the packed path the benchmark step takes (codes in 1 KB blocks, LDS-DMA
    tiles) and the row-major path, INT32 and BF16 against the oracle."""
    show("prefill full size, all rows")
    d = synth.prefill(seed=0)
    x = bf16_dev(d.x)
    wp = w.prepack_weight(dev(d.w))
    ws_, bias = dev(d.w_scale), bf16_dev(d.bias)
    qp, sp = w.dynamic_quant_packed(x)
    acc_pk = host(w.linear_packed(qp, sp, d.K, wp, ws_, d.N, out=w.OUT_I32))
    y_pk = bf16_host(w.linear_packed(qp, sp, d.K, wp, ws_, d.N, bias=bias))
    q, s = w.dynamic_quant(x)
    y_rm = bf16_host(w.linear(q, s, wp, ws_, d.N, bias=bias))
    sync()
    qo, so = O.dynamic_quant(d.x)
    _assert_eq(host(q), qo, "q")
    _assert_eq(host(s).view(np.uint32), so.view(np.uint32), "scale")
    _assert_eq(_unpack_codes(host(qp), d.M, d.K), qo, "q (blocks)")
    _assert_eq(host(sp).view(np.uint32), so.view(np.uint32), "scale (packed path)")
    del q, s, qp, sp
    yo, acc = O.linear(qo, so, d.w, d.w_scale, d.bias)
    _assert_eq(acc_pk, acc.astype(np.int32), "acc (packed)")
    _assert_eq(y_pk, yo, "y (packed)")
    _assert_eq(y_rm, yo, "y (row-major)")
    assert O.bf16_within_tolerance(y_pk, O.linear_ref64(acc, so, d.w_scale, d.bias)).all()


# ---------------------------------------------------------------------------
# grouped GEMM
# ---------------------------------------------------------------------------

def _grouped_case(counts, N, K, seed):
    g = np.asarray(counts, np.int64)
    R, E = int(g.sum()), len(g)
    a = synth.int8_weight((R, K), seed, 11)
    xs = synth.scales(R, seed, 12)
    wt = synth.int8_weight((E, N, K), seed, 13)
    ws = synth.scales((E, N), seed, 14)
    return g, a, xs, wt, ws


GROUPED_CASES = [
    ([12, 7, 0, 19], 48, 64),
    ([12, 7, 0, 19], 20, 100),
    ([0, 0, 9, 0, 0], 130, 256),
    ([0, 300, 1, 0, 129, 2, 0], 256, 320),
    ([5] * 33, 64, 128),
    ([0, 0, 0], 16, 64),
    # small/large boundary (64 rows streamed, 65 rows tiled), a multi-tile
    # expert, ragged K (K % 64 != 0) and an N tail on the tiled path
    ([64, 65, 0, 600], 200, 208),
    ([1, 700, 2, 64, 0, 257], 272, 1024),
]


@pytest.mark.parametrize("counts,N,K", GROUPED_CASES)
def test_grouped_gemm_bit_exact(w, counts, N, K):
    show(f"grouped counts={counts} N={N} K={K}")
    g, a, xs, wt, ws = _grouped_case(counts, N, K, seed=len(counts) + N)
    R, E = int(g.sum()), len(g)
    wp = w.prepack_weight(dev(wt))
    if R == 0:
        a_d = torch.empty((0, K), dtype=torch.int8, device="cuda")
        y = w.grouped_gemm(a_d, torch.empty(0, device="cuda"), dev(g), wp, dev(ws), N)
        assert y.shape == (0, N)
        return
    acc = w.grouped_gemm(dev(a), dev(xs), dev(g), wp, dev(ws), N, out=w.OUT_I32)
    y = w.grouped_gemm(dev(a), dev(xs), dev(g), wp, dev(ws), N, out=w.OUT_BF16)
    sync()
    yo, acc_o = O.grouped_gemm_bf16(a, xs, g, wt, ws)
    _assert_eq(host(acc), acc_o.astype(np.int32), "acc")
    _assert_eq(bf16_host(y), yo, "y")


# ---------------------------------------------------------------------------
# SwiGLU + requant
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("R,I", [(16, 2048), (5, 24), (3, 37), (9, 4096), (2, 8200), (64, 512)])
def test_swiglu_quant_bit_exact(w, R, I):
    show(f"swiglu_quant R={R} I={I}")
    rng = np.random.default_rng(R * 7 + I)
    h = (rng.standard_normal((R, 2 * I)) * 4).astype(np.float32)
    h[0, :4] = [100.0, -100.0, 0.0, -90.0]       # saturating exp on both sides
    if R > 2:
        h[2] = 0.0                               # all-zero row
    hb = O.f32_to_bf16(h)
    q, s = w.swiglu_quant(bf16_dev(hb))
    sync()
    qo, so = O.swiglu_quant(hb, I)
    _assert_eq(host(s).view(np.uint32), so.view(np.uint32), "scale")
    _assert_eq(host(q), qo, "q")


# ---------------------------------------------------------------------------
# MoE chain
# ---------------------------------------------------------------------------

def _moe_small(counts, H, I, seed):
    g = np.asarray(counts, np.int64)
    E, R = len(g), int(g.sum())
    x = synth.activations(R, H, 0.01, seed)
    w13 = synth.int8_weight((E, 2 * I, H), seed, 6)
    w2 = synth.int8_weight((E, H, I), seed, 7)
    w13s = synth.scales((E, 2 * I), seed, 8)
    w2s = synth.scales((E, H), seed, 9)
    return g, x, w13, w13s, w2, w2s


@pytest.mark.parametrize("counts,H,I", [([12, 7, 0, 19], 64, 32), ([0, 200, 3, 0, 70], 256, 128)])
def test_moe_chain_bit_exact(w, counts, H, I):
    show(f"moe chain counts={counts} H={H} I={I}")
    g, x, w13, w13s, w2, w2s = _moe_small(counts, H, I, seed=H)
    st = O.moe_grouped(g, w13, w13s, w2, w2s, x_bits=x, keep=True)
    w13p, w2p = w.prepack_weight(dev(w13)), w.prepack_weight(dev(w2))
    y = w.moe_grouped(bf16_dev(x), dev(g), w13p, dev(w13s), w2p, dev(w2s))
    # stage by stage through the sub-stage entry points
    q, s = w.dynamic_quant(bf16_dev(x))
    h = w.grouped_gemm(q, s, dev(g), w13p, dev(w13s), 2 * I)
    q2, s2 = w.swiglu_quant(h)
    # the pre-quantized entry: INT8 rows + scale skip the first quant
    y2 = w.moe_grouped(q, dev(g), w13p, dev(w13s), w2p, dev(w2s), x_scale=s)
    sync()
    _assert_eq(bf16_host(h), st["h"], "h")
    _assert_eq(host(q2), st["q2"], "q2")
    _assert_eq(host(s2), st["s2"], "s2")
    _assert_eq(bf16_host(y), st["y"], "y")
    _assert_eq(bf16_host(y2), st["y"], "y (int8 input)")


@pytest.mark.timeout(900)
def test_moe_config_all_rows(w):
    """Full MoE workload (2048 tokens top-8 over 256 experts, H 4096, I 2048):
    every one of the 16384 output rows against the oracle, one expert at a
    time (the oracle's chain on that expert's rows alone; experts are
    independent, so this is the oracle's whole chain)."""
    show("moe full size, all rows")
    m = synth.moe(seed=0)
    E, H, I = m.E, m.H, m.I
    w13p = torch.empty(w.packed_weight_bytes(E, 2 * I, H), dtype=torch.uint8, device="cuda")
    w2p = torch.empty(w.packed_weight_bytes(E, H, I), dtype=torch.uint8, device="cuda")
    per13 = w.packed_weight_bytes(1, 2 * I, H)
    per2 = w.packed_weight_bytes(1, H, I)
    for e in range(E):  # prepack expert by expert (bounded staging memory)
        w.prepack_weight(dev(m.w13(e)), out=w13p[e * per13:(e + 1) * per13])
        w.prepack_weight(dev(m.w2(e)), out=w2p[e * per2:(e + 1) * per2])
        m.drop_cache()
    xr = m.x_rows()
    y = w.moe_grouped(bf16_dev(xr), dev(m.group_list), w13p, dev(m.w13_scale), w2p,
                      dev(m.w2_scale))
    yh = bf16_host(y)
    del w13p, w2p
    off = O.group_offsets(m.group_list)
    done = 0
    for e in range(E):
        a, b = int(off[e]), int(off[e + 1])
        if b == a:
            continue
        st = O.moe_grouped(np.array([b - a], np.int64), m.w13(e)[None], m.w13_scale[e][None],
                           m.w2(e)[None], m.w2_scale[e][None], x_bits=xr[a:b])
        _assert_eq(yh[a:b], st, f"rows {a}..{b - 1} (expert {e})")
        m.drop_cache()
        done += b - a
        if e % 32 == 31:
            show(f"  experts 0..{e}: {done} rows equal")
    assert done == m.R


# ---------------------------------------------------------------------------
# packed activation codes (dynamic_quant_packed + linear on blocks)
# ---------------------------------------------------------------------------

def _unpack_codes(buf, M, K):
    """1 KB blocks [ceil(M/16)][ceil(K/64)] -> int8 [M, K]: byte (r + 16 c) * 16 + j of
    block (b, kb) is element (16 b + r, 64 kb + 16 c + j)."""
    MB, KB = -(-M // 16), -(-K // 64)
    b = np.asarray(buf)[:MB * KB * 1024].reshape(MB, KB, 4, 16, 16)
    return b.transpose(0, 3, 1, 2, 4).reshape(MB * 16, KB * 64)[:M, :K].view(np.int8)


PACKED_QUANT_SHAPES = [(1, 7168), (16, 256), (17, 7168), (64, 7168), (300, 1024), (5, 96), (33, 520),
                       (600, 520), (1030, 7168), (513, 64),
                       # many-row kernels: K % 16 == 8 (one pass), K > 8192 (two passes)
                       (520, 1032), (530, 8200)]


@pytest.mark.parametrize("M,K", PACKED_QUANT_SHAPES)
def test_dynamic_quant_packed_bit_exact(w, M, K):
    show(f"dynamic_quant_packed M={M} K={K}")
    xb = synth.activations(M, K, 0.01, seed=M * 31 + K)
    q, s = w.dynamic_quant_packed(bf16_dev(xb))
    sync()
    qo, so = O.dynamic_quant(xb)
    _assert_eq(host(s).view(np.uint32), so.view(np.uint32), "scale")
    _assert_eq(_unpack_codes(host(q), M, K), qo, "q (blocks)")


PACKED_LINEAR_SHAPES = [(1, 4096, 7168), (4, 256, 512), (16, 4096, 7168), (33, 300, 1024),
                        (64, 512, 7168), (64, 4096, 7168), (65, 300, 520), (300, 1088, 600), (520, 512, 1024),
                        # M <= 64 with two k-iterations per wavefront (next weights loaded
                        # ahead), a ragged last k-block and a clamped fourth m-block
                        (40, 264, 7000)]


@pytest.mark.parametrize("M,N,K", PACKED_LINEAR_SHAPES)
def test_linear_packed_matches_row_major(w, M, N, K):
    show(f"linear packed M={M} N={N} K={K}")
    d = synth.dense(M, K, N, outlier_frac=0.005, bias=True, seed=M + N + K)
    wp = w.prepack_weight(dev(d.w))
    ws_ = dev(d.w_scale)
    bias = bf16_dev(d.bias)
    x = bf16_dev(d.x)
    q, s = w.dynamic_quant(x)
    qp, sp = w.dynamic_quant_packed(x)
    y_rm = w.linear(q, s, wp, ws_, N, bias=bias)
    y_pk = w.linear_packed(qp, sp, K, wp, ws_, N, bias=bias)
    acc_pk = w.linear_packed(qp, sp, K, wp, ws_, N, out=w.OUT_I32)
    sync()
    qo, so = O.dynamic_quant(d.x)
    yo, acc_o = O.linear(qo, so, d.w, d.w_scale, d.bias)
    _assert_eq(host(acc_pk), acc_o, "packed INT32")
    _assert_eq(bf16_host(y_pk), yo, "packed BF16 vs oracle")
    _assert_eq(bf16_host(y_rm), yo, "row-major BF16 vs oracle")


# ---------------------------------------------------------------------------
# BF16-input linear (quant inside; fused with the product for M <= 4)
# ---------------------------------------------------------------------------

BF16_LINEAR_SHAPES = [(1, 4096, 7168), (2, 256, 512), (3, 100, 256), (4, 4096, 7168), (5, 300, 520),
                      (16, 4096, 7168), (64, 512, 7168), (65, 300, 520), (3, 64, 100), (300, 1088, 600),
                      (4, 64, 16392),
                      # quant inside the product for up to 16 rows of M * K <= 16384
                      # values (chunks numbered flat): the tiny shape, exactly
                      # 16384 values, K % 64 != 0 (zero code chunks), M * Kp / 8
                      # near the 3 chunks per thread, K = 8; then just past the
                      # limit (quant launch + product)
                      (16, 128, 256), (16, 200, 1024), (9, 96, 1000), (7, 48, 2336), (15, 40, 8),
                      (16, 64, 1032),
                      # two rows of K = 16384 (fused; past the 16384-value limit)
                      (2, 80, 16384)]


@pytest.mark.parametrize("M,N,K", BF16_LINEAR_SHAPES)
def test_linear_bf16_input_matches_quant_then_linear(w, M, N, K):
    show(f"linear bf16 M={M} N={N} K={K}")
    d = synth.dense(M, K, N, outlier_frac=0.01, bias=True, seed=M * 7 + N + K)
    if M > 2:
        d.x[1] = 0  # all-zero row
    wp = w.prepack_weight(dev(d.w))
    ws_ = dev(d.w_scale)
    bias = bf16_dev(d.bias)
    x = bf16_dev(d.x)
    q, s = w.dynamic_quant(x)
    y_ref = w.linear(q, s, wp, ws_, N, bias=bias)
    y = w.linear_bf16(x, wp, ws_, N, bias=bias)
    acc = w.linear_bf16(x, wp, ws_, N, out=w.OUT_I32)
    sync()
    qo, so = O.dynamic_quant(d.x)
    yo, acc_o = O.linear(qo, so, d.w, d.w_scale, d.bias)
    _assert_eq(host(acc), acc_o, "BF16 input INT32")
    _assert_eq(bf16_host(y), yo, "BF16 input vs oracle")
    _assert_eq(bf16_host(y_ref), yo, "quant + linear vs oracle")
