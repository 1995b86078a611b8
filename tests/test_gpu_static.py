"""Parity of the static W8A8 path (through the C ABI) with the CPU oracle.

Codes, dequant scales (bits), integer biases and INT32 accumulators are
compared exactly, and so are the BF16 outputs of the static epilogue. Inputs
come from the seeded generators in ``synth``; expected values only from
``oracle``.
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

S = O.static

# fixed per-tensor calibration of N(0, 1) activations with x20 outliers: the
# bulk inside the code range, the outliers clamped at both ends
SCALE, OFFSET = 6.0 / 127.0, 3.0


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


# (M, K, scale, offset): vector path (M K % 8 == 0), element path, clamps at both
# ends, a non-integer offset, a tiny scale (most codes clamp)
QUANT_CASES = [(16, 256, SCALE, OFFSET), (1, 7168, SCALE, OFFSET), (5, 100, 0.02, -2.5),
               (3, 37, SCALE, 0.0), (300, 1000, 0.01, 7.0), (1024, 4096, SCALE, -1.0),
               (7, 64, 1e-4, 0.5)]


@pytest.mark.parametrize("M,K,s,o", QUANT_CASES)
def test_static_quant_bit_exact(w, M, K, s, o):
    show(f"static_quant M={M} K={K} s={s} o={o}")
    xb = synth.activations(M, K, 0.01, seed=M * 13 + K)
    q = w.static_quant(bf16_dev(xb), s, o)
    sync()
    _assert_eq(host(q), S.static_quant(xb, s, o), "q")


@pytest.mark.parametrize("N,K,bias", [(128, 256, True), (50, 100, False), (4096, 7168, True),
                                      (33, 520, True)])
def test_static_prepare_bit_exact(w, N, K, bias):
    show(f"static_prepare N={N} K={K} bias={bias}")
    d = synth.dense(1, K, N, outlier_frac=0.0, bias=bias, seed=N + K)
    for s, o in ((SCALE, OFFSET), (0.013, -5.5), (0.5, 0.0)):
        deq, qb = w.static_prepare(dev(d.w), dev(d.w_scale), None if d.bias is None else bf16_dev(d.bias),
                                   s, o)
        sync()
        deq_o, qb_o = S.static_prepare(d.w, d.w_scale, d.bias, s, o)
        _assert_eq(host(deq).view(np.uint32), deq_o.view(np.uint32), "deq_scale bits")
        _assert_eq(host(qb), qb_o, "quant_bias")


LINEAR_CASES = [  # M, K, N, bias
    (1, 7168, 512, True), (4, 7168, 512, False), (16, 1024, 96, True), (64, 2048, 256, True),
    (33, 520, 50, True),                                   # decode kernel, ragged N and K
    (300, 1024, 260, True), (520, 1088, 600, False),        # LDS-DMA tiles, partial tiles
    (100, 100, 50, True),                                   # K % 16 != 0: VGPR-staged tiles
    (3, 37, 5, False),                                      # decode kernel, rows not 16-byte
]


@pytest.mark.parametrize("M,K,N,bias", LINEAR_CASES)
def test_static_linear_bit_exact(w, M, K, N, bias):
    show(f"static_linear M={M} K={K} N={N} bias={bias}")
    d = synth.dense(M, K, N, outlier_frac=0.005, bias=bias, seed=M + 3 * K + N)
    bias_dev = None if d.bias is None else bf16_dev(d.bias)
    q = w.static_quant(bf16_dev(d.x), SCALE, OFFSET)
    deq, qb = w.static_prepare(dev(d.w), dev(d.w_scale), bias_dev, SCALE, OFFSET)
    wp = w.prepack_weight(dev(d.w))
    y = w.static_linear(q, wp, deq, qb, N)
    acc = w.static_linear(q, wp, deq, qb, N, out=w.OUT_I32)
    sync()
    qo = S.static_quant(d.x, SCALE, OFFSET)
    _assert_eq(host(q), qo, "q")
    deq_o, qb_o = S.static_prepare(d.w, d.w_scale, d.bias, SCALE, OFFSET)
    yo, acc_o = S.static_linear(qo, d.w, deq_o, qb_o)
    _assert_eq(host(acc), acc_o.astype(np.int32), "acc")
    _assert_eq(bf16_host(y), yo, "y")


@pytest.mark.timeout(300)
def test_static_prefill_shape_sampled_rows(w):
    show("static linear, prefill shape, sampled rows")
    d = synth.prefill(seed=1)
    M, N = d.x.shape[0], d.w.shape[0]
    q = w.static_quant(bf16_dev(d.x), SCALE, OFFSET)
    deq, qb = w.static_prepare(dev(d.w), dev(d.w_scale), bf16_dev(d.bias), SCALE, OFFSET)
    y = w.static_linear(q, w.prepack_weight(dev(d.w)), deq, qb, N)
    sync()
    qo = S.static_quant(d.x, SCALE, OFFSET)
    _assert_eq(host(q), qo, "q")
    deq_o, qb_o = S.static_prepare(d.w, d.w_scale, d.bias, SCALE, OFFSET)
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(1).integers(0, M, 24)]))
    yo, _ = S.static_linear(qo[rows], d.w, deq_o, qb_o)
    _assert_eq(bf16_host(y)[rows], yo, "y rows")


def _unpack(buf, M, K):
    """Packed 1 KB blocks -> int8 [M, K] (test-side inverse of the layout)."""
    KB = -(-K // 64)
    b = np.asarray(buf, np.uint8).view(np.int8)[: -(-M // 16) * KB * 1024]
    b = b.reshape(-(-M // 16), KB, 4, 16, 16)          # [mb][kb][chunk][row][byte]
    full = b.transpose(0, 3, 1, 2, 4).reshape(-(-M // 16) * 16, KB * 64)
    return full[:M, :K]


@pytest.mark.parametrize("M,K,s,o", [(16, 256, SCALE, OFFSET), (5, 100, 0.02, -2.5),
                                     (33, 520, 0.01, 7.0), (300, 1032, SCALE, -1.0),
                                     (1, 7168, SCALE, OFFSET), (17, 37, 0.05, 2.0)])
def test_static_quant_packed_bit_exact(w, M, K, s, o):
    show(f"static_quant_packed M={M} K={K}")
    xb = synth.activations(M, K, 0.01, seed=M * 7 + K)
    qp = w.static_quant_packed(bf16_dev(xb), s, o)
    sync()
    buf = host(qp)
    _assert_eq(_unpack(buf, M, K), S.static_quant(xb, s, o), "q (blocks)")
    # rows past M and columns past K carry zero codes
    KB = -(-K // 64)
    full = np.asarray(buf, np.uint8).view(np.int8)[: -(-M // 16) * KB * 1024]
    full = full.reshape(-(-M // 16), KB, 4, 16, 16).transpose(0, 3, 1, 2, 4).reshape(-(-M // 16) * 16, KB * 64)
    assert not full[M:].any() and not full[:, K:].any()


@pytest.mark.parametrize("M,K,N", [(1, 7168, 512), (16, 1024, 96), (64, 2048, 256), (300, 1024, 260),
                                   (520, 1088, 600), (33, 520, 50)])
def test_static_linear_packed_matches_row_major(w, M, K, N):
    show(f"static_linear packed M={M} K={K} N={N}")
    d = synth.dense(M, K, N, outlier_frac=0.005, bias=True, seed=M + 5 * K + N)
    x = bf16_dev(d.x)
    deq, qb = w.static_prepare(dev(d.w), dev(d.w_scale), bf16_dev(d.bias), SCALE, OFFSET)
    wp = w.prepack_weight(dev(d.w))
    y_rm = w.static_linear(w.static_quant(x, SCALE, OFFSET), wp, deq, qb, N)
    qp = w.static_quant_packed(x, SCALE, OFFSET)
    y_pk = w.static_linear(qp, wp, deq, qb, N, M=M, K=K)
    acc_pk = w.static_linear(qp, wp, deq, qb, N, out=w.OUT_I32, M=M, K=K)
    sync()
    _assert_eq(bf16_host(y_pk), bf16_host(y_rm), "packed vs row-major BF16")
    qo = S.static_quant(d.x, SCALE, OFFSET)
    deq_o, qb_o = S.static_prepare(d.w, d.w_scale, d.bias, SCALE, OFFSET)
    yo, acc_o = S.static_linear(qo, d.w, deq_o, qb_o)
    _assert_eq(host(acc_pk), acc_o.astype(np.int32), "packed INT32")
    _assert_eq(bf16_host(y_pk), yo, "packed BF16 vs oracle")
