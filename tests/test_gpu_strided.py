"""Row-strided operands of the dynamic quant and the dense linear (GPU).

A caller's activation is often a column slice of a wider matrix (a fused QKV
or gate/up output) and its result goes into a slice of a wider buffer. The
strided entry points read and write such slices in place; every case here
compares them bit for bit with the oracle on the slice's contents and checks
that nothing outside the slice was written. Offsets and strides cover the
16-byte vector paths (strides and offsets multiples of 8 or 16) and the
element-wise fallbacks (odd strides and offsets), for decode-sized M (one
weight pass) and prefill-sized M (256x256 tiles)."""

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


def _outside(full: np.ndarray, off: int, width: int) -> np.ndarray:
    """The columns of a wide buffer outside [off, off + width)."""
    return np.concatenate([full[:, :off], full[:, off + width:]], axis=1)


# M, K, extra columns of the wide x, column offset of x, extra columns of the
# wide q, column offset of q
QUANT_CASES = [
    (5, 256, 64, 8, 32, 16),      # vector path, offsets and strides multiples of 8
    (3, 7168, 128, 64, 64, 0),    # one workgroup per row, two pieces per thread
    (130, 4096, 8, 0, 16, 8),     # many rows
    (7, 100, 5, 3, 3, 1),         # odd strides and offsets: element-wise path
    (600, 512, 24, 8, 8, 8),      # M > 512
    (4, 37, 0, 0, 11, 2),         # only q strided
]


@pytest.mark.parametrize("M,K,xe,xo,qe,qo", QUANT_CASES)
def test_dynamic_quant_strided(w, M, K, xe, xo, qe, qo):
    show(f"dynamic_quant strided M={M} K={K} ldx={K + xe} x_off={xo} ldq={K + qe} q_off={qo}")
    wide = synth.activations(M, K + xe, 0.01, seed=M * 31 + K)
    if M > 2:
        wide[1, xo:xo + K] = 0  # all-zero row of the slice
    xb = np.ascontiguousarray(wide[:, xo:xo + K])
    x = bf16_dev(wide)[:, xo:xo + K]
    qfull = torch.full((M, K + qe), 77, dtype=torch.int8, device="cuda")
    q = qfull[:, qo:qo + K]
    scale = torch.empty((M,), dtype=torch.float32, device="cuda")
    w.dynamic_quant(x, q, scale)
    sync()
    q_ref, s_ref = O.dynamic_quant(xb)
    qh = host(qfull)
    _assert_eq(qh[:, qo:qo + K], q_ref, "q")
    _assert_eq(host(scale).view(np.uint32), s_ref.view(np.uint32), "scale")
    assert (_outside(qh, qo, K) == 77).all(), "codes written outside the slice"


# M, K, N, bias, extra columns of the wide codes, offset of q, extra columns
# of the wide y, offset of y (even: y must stay 4-byte aligned)
LINEAR_CASES = [
    (1, 7168, 512, True, 64, 0, 16, 8),      # decode, 16-byte code rows
    (4, 2064, 160, False, 48, 16, 8, 0),     # decode, ragged last k-block
    (16, 1024, 256, True, 7, 5, 3, 2),       # decode, unaligned code rows
    (40, 1040, 96, False, 16, 0, 0, 0),      # decode, only q strided
    (40, 1040, 96, True, 3, 1, 0, 0),        # decode, 33..64 rows on unaligned code rows
    (64, 4096, 512, True, 128, 64, 64, 0),   # decode M = 64
    (300, 1088, 600, True, 64, 0, 40, 8),    # prefill tiles through the LDS ring
    (257, 4096, 512, False, 16, 16, 7, 2),   # prefill, odd ldy: element-wise stores
    (200, 512, 300, True, 5, 3, 0, 0),       # prefill, unaligned rows: VGPR-staged tiles
    (520, 256, 64, False, 0, 0, 32, 16),     # only y strided
]


@pytest.mark.parametrize("M,K,N,bias,qe,qo,ye,yo", LINEAR_CASES)
def test_linear_strided(w, M, K, N, bias, qe, qo, ye, yo):
    show(f"linear strided M={M} K={K} N={N} ldq={K + qe} q_off={qo} ldy={N + ye} y_off={yo}")
    d = synth.dense(M, K, N, outlier_frac=0.01, bias=bias, seed=M * 3 + K + N)
    q_ref, s_ref = O.dynamic_quant(d.x)
    y_ref, acc_ref = O.linear(q_ref, s_ref, d.w, d.w_scale, d.bias)
    rng = np.random.default_rng(M + N)
    qwide = rng.integers(-128, 128, size=(M, K + qe), dtype=np.int8)
    qwide[:, qo:qo + K] = q_ref
    q = dev(qwide)[:, qo:qo + K]
    s = dev(s_ref)
    wp = w.prepack_weight(dev(d.w))
    ws_ = dev(d.w_scale)
    b = None if d.bias is None else bf16_dev(d.bias)
    ybf = torch.full((M, N + ye), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    yi = torch.full((M, N + ye), -7, dtype=torch.int32, device="cuda")
    w.linear(q, s, wp, ws_, N, bias=b, y=ybf[:, yo:yo + N])
    w.linear(q, s, wp, ws_, N, out=w.OUT_I32, y=yi[:, yo:yo + N])
    sync()
    yh = bf16_host(ybf)
    ih = host(yi)
    _assert_eq(ih[:, yo:yo + N], acc_ref, "INT32")
    _assert_eq(yh[:, yo:yo + N], y_ref, "BF16")
    assert (_outside(yh, yo, N) == 0xFFFF).all(), "BF16 written outside the slice"
    assert (_outside(ih, yo, N) == -7).all(), "INT32 written outside the slice"


def test_quant_then_linear_on_slices(w):
    """A decode step whose activation is the middle third of a fused output and
    whose result lands in the left half of a wider buffer: quant and linear
    both on slices, no copies."""
    M, K, N = 8, 2048, 1024
    d = synth.dense(M, K, N, outlier_frac=0.01, bias=True, seed=5)
    wide = np.zeros((M, 3 * K), np.uint16)
    wide[:, K:2 * K] = d.x
    x = bf16_dev(wide)[:, K:2 * K]
    q, s = w.dynamic_quant(x)
    wp = w.prepack_weight(dev(d.w))
    yfull = torch.zeros((M, 2 * N), dtype=torch.bfloat16, device="cuda")
    w.linear(q, s, wp, dev(d.w_scale), N, bias=bf16_dev(d.bias), y=yfull[:, :N])
    sync()
    q_ref, s_ref = O.dynamic_quant(d.x)
    y_ref, _ = O.linear(q_ref, s_ref, d.w, d.w_scale, d.bias)
    yh = bf16_host(yfull)
    _assert_eq(yh[:, :N], y_ref, "BF16")
    assert (yh[:, N:] == 0).all()


def test_strided_rejects_bad_strides(w):
    x = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        w.dynamic_quant(x.t())  # columns not contiguous
    q = torch.zeros((4, 64), dtype=torch.int8, device="cuda")
    with pytest.raises(ValueError):
        w.dynamic_quant(x, q[:, ::2].contiguous()[:, :32])  # wrong shape
