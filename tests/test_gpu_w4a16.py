"""Parity of the W4A16 weight variant, INT4 and FP4 weights (through the C ABI),
with the CPU oracle.

Codes, BF16 scales and the packed layout are compared exactly. The linear
multiplies exactly dequantized BF16 weights (BF16 x BF16 products are exact in
fp32) and accumulates in fp32, so its BF16 output is compared with the float64
sum under the BF16 bound max(2**-8 |ref|, 1e-5) plus an allowance for the fp32
additions: LAMBDA * sqrt(K) * 2**-24 * sum_k |x w| (the probabilistic bound of
Higham & Mary, 2019, for sums whose rounding errors are independent and of
random sign, as with these inputs). Inputs are seeded; expected values come
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

W4 = O.w4a16
LAMBDA = 6.0


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


def _weight(N, K, seed):
    r = np.random.default_rng([seed, 44])
    w = r.standard_normal((N, K)).astype(np.float32) * r.uniform(0.005, 0.05, (N, 1)).astype(np.float32)
    w[0, :32] = 0.0                          # an all-zero group
    return O.f32_to_bf16(w)


def _unpack(buf, N, K):
    """Test-side inverse of the packed layout: codes [N, K] and BF16 scale bits
    [N, K/32] from the 1152-byte (16 columns x 128 k) chunks."""
    NB, KC = -(-N // 16), -(-K // 128)
    b = np.asarray(buf, np.uint8)[:NB * KC * 1152].reshape(NB, KC, 1152)
    codes = b[:, :, :1024].reshape(NB, KC, 4, 16, 4, 4)      # [nb][kc][l/16][col][step][byte]
    lo = (codes & 0xF).astype(np.int16) - 8
    hi = (codes >> 4).astype(np.int16) - 8
    nib = np.stack([lo, hi], axis=-1).reshape(NB, KC, 4, 16, 4, 8)   # ...[step][i]
    # k = 128 kc + 32 step + 8 (l / 16) + i
    q = nib.transpose(0, 3, 1, 4, 2, 5).reshape(NB * 16, KC * 128)[:N, :K].astype(np.int8)
    sc = b[:, :, 1024:].view(np.uint16).reshape(NB, KC, 16, 4)        # [nb][kc][col][step]
    s = sc.transpose(0, 2, 1, 3).reshape(NB * 16, KC * 4)[:N, :K // 32]
    return q, s


@pytest.mark.parametrize("N,K", [(64, 128), (50, 96), (33, 32), (4096, 7168), (160, 2080)])
def test_w4_quant_and_pack_bit_exact(w, N, K):
    show(f"w4a16_quant_weight N={N} K={K}")
    wb = _weight(N, K, seed=N + K)
    q, s, p = w.w4a16_quant_weight(bf16_dev(wb), codes=True, scales=True, pack=True)
    p2 = w.w4a16_pack(q, s)
    sync()
    q_o, s_o = W4.w4_quant(wb)
    _assert_eq(host(q), q_o, "codes")
    _assert_eq(host(s.view(torch.int16)).view(np.uint16), s_o, "scales")
    qu, su = _unpack(host(p), N, K)
    _assert_eq(qu, q_o, "packed codes")
    _assert_eq(su, s_o, "packed scales")
    _assert_eq(host(p2), host(p), "pack of the codes == quant's packing")


def _check_linear(y_bits, x_bits, q, s):
    ref = W4.w4a16_linear_ref64(x_bits, q, s)
    xf = O.bf16_to_f32(x_bits).astype(np.float64)
    wf = O.bf16_to_f32(W4.w4_dequant(q, s)).astype(np.float64)
    mag = np.abs(xf) @ np.abs(wf).T
    allow = LAMBDA * np.sqrt(xf.shape[1]) * 2.0 ** -24 * mag
    y = O.bf16_to_f32(y_bits).astype(np.float64)
    err = np.abs(y - ref)
    base = np.maximum(O.REL_TOL * np.abs(ref), O.ABS_FLOOR)
    ok = err <= base + allow
    show(f"  max|err| {err.max():.3e}, past the BF16 bound alone {int((err > base).sum())} "
         f"of {err.size}")
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        raise AssertionError(f"{int((~ok).sum())} of {ok.size} outside tolerance, first {i}: "
                             f"got {y[i]} want {ref[i]} allowance {allow[i]}")


# (M, K, N): decode rows 1 / 4 / 16 / 64, rows past a 16- and a 64-row block,
# K not a multiple of 128, N not a multiple of 16
LINEAR_CASES = [(1, 256, 64), (4, 1024, 96), (16, 512, 50), (17, 320, 64), (64, 2048, 512),
                (100, 2048, 256), (3, 96, 40), (1, 7168, 4096),
                # M > 16 with several chunks per wavefront (the next chunk's codes
                # loaded ahead), a ragged last chunk (K % 128 = 64), ragged N
                (80, 4160, 72),
                # row groups of 32 (INT4) / 16 (FP4) with a partial last one,
                # a last chunk a quarter inside K, a partial last column group;
                # one partial chunk for 16 wavefronts; a larger decode-like case
                (33, 1056, 200), (5, 32, 16), (48, 7168, 1024)]


@pytest.mark.parametrize("M,K,N", LINEAR_CASES)
def test_w4a16_linear_within_tolerance(w, M, K, N):
    show(f"w4a16_linear M={M} K={K} N={N}")
    x = synth.activations(M, K, 0.005, seed=M + K + N)
    wb = _weight(N, K, seed=K + N)
    _, _, p = w.w4a16_quant_weight(bf16_dev(wb))
    y = w.w4a16_linear(bf16_dev(x), p, N)
    sync()
    q_o, s_o = W4.w4_quant(wb)
    _check_linear(bf16_host(y), x, q_o, s_o)


@pytest.mark.timeout(300)
def test_w4a16_decode_config(w):
    """The decode-shaped linear in full: X BF16 [M in 1, 4, 16, 64, K = 7168]
    (0.5 % x20 outliers), the weight [4096, 7168] quantized to INT4 per 32."""
    d = synth.decode(seed=0)
    K, N = d.x.shape[1], 4096
    wb = _weight(N, K, seed=0)
    _, _, p = w.w4a16_quant_weight(bf16_dev(wb))
    q_o, s_o = W4.w4_quant(wb)
    for M in (1, 4, 16, 64):
        show(f"w4a16 decode config M={M}")
        y = w.w4a16_linear(bf16_dev(d.x[:M]), p, N)
        sync()
        _check_linear(bf16_host(y), d.x[:M], q_o, s_o)


def test_w4a16_zero_rows(w):
    _, _, p = w.w4a16_quant_weight(bf16_dev(_weight(32, 64, 1)))
    y = w.w4a16_linear(torch.empty((0, 64), dtype=torch.bfloat16, device="cuda"), p, 32)
    sync()
    assert y.shape == (0, 32)


# ---------------------------------------------------------------------------
# FP4 (E2M1 + E8M0 per 32) weights in the same packed layout
# ---------------------------------------------------------------------------

def _unpack_fp4(buf, N, K):
    """Test-side inverse of the FP4 layout: 1088-byte chunks (1 KB of codes in
    the INT4 layout's order, then the E8M0 bytes [16 columns][4 groups])."""
    NB, KC = -(-N // 16), -(-K // 128)
    b = np.asarray(buf, np.uint8)[:NB * KC * 1088].reshape(NB, KC, 1088)
    codes = b[:, :, :1024].reshape(NB, KC, 4, 16, 4, 4)
    nib = np.stack([codes & 0xF, codes >> 4], axis=-1).reshape(NB, KC, 4, 16, 4, 8)
    c = nib.transpose(0, 3, 1, 4, 2, 5).reshape(NB * 16, KC * 128)[:N, :K]
    sc = b[:, :, 1024:1088].reshape(NB, KC, 16, 4)                    # [nb][kc][col][step]
    s = sc.transpose(0, 2, 1, 3).reshape(NB * 16, KC * 4)[:N, :K // 32]
    return c, s


@pytest.mark.parametrize("N,K", [(64, 128), (50, 96), (33, 32), (4096, 7168), (160, 2080)])
def test_fp4_quant_and_pack_bit_exact(w, N, K):
    show(f"fp4_quant_weight N={N} K={K}")
    wb = _weight(N, K, seed=N + K + 1)
    c, s, p = w.fp4_quant_weight(bf16_dev(wb), codes=True, scales=True, pack=True)
    sync()
    c_o, s_o = W4.fp4_quant(wb)
    _assert_eq(host(c), c_o, "codes")
    _assert_eq(host(s), s_o, "scales")
    cu, su = _unpack_fp4(host(p), N, K)
    _assert_eq(cu, c_o, "packed codes")
    _assert_eq(su, s_o, "packed scales")
    assert p.numel() == w.fp4_packed_bytes(N, K) == -(-N // 16) * -(-K // 128) * 1088


def _check_fp4_linear(y_bits, x_bits, c, s):
    ref = W4.fp4_linear_ref64(x_bits, c, s)
    xf = O.bf16_to_f32(x_bits).astype(np.float64)
    wf = O.bf16_to_f32(W4.fp4_dequant(c, s)).astype(np.float64)
    mag = np.abs(xf) @ np.abs(wf).T
    allow = LAMBDA * np.sqrt(xf.shape[1]) * 2.0 ** -24 * mag
    y = O.bf16_to_f32(y_bits).astype(np.float64)
    err = np.abs(y - ref)
    base = np.maximum(O.REL_TOL * np.abs(ref), O.ABS_FLOOR)
    ok = err <= base + allow
    show(f"  max|err| {err.max():.3e}, past the BF16 bound alone {int((err > base).sum())} "
         f"of {err.size}")
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        raise AssertionError(f"{int((~ok).sum())} of {ok.size} outside tolerance, first {i}: "
                             f"got {y[i]} want {ref[i]} allowance {allow[i]}")


@pytest.mark.parametrize("M,K,N", LINEAR_CASES)
def test_fp4_linear_within_tolerance(w, M, K, N):
    show(f"fp4_linear M={M} K={K} N={N}")
    x = synth.activations(M, K, 0.005, seed=M + K + N + 1)
    wb = _weight(N, K, seed=K + N + 1)
    _, _, p = w.fp4_quant_weight(bf16_dev(wb))
    y = w.fp4_linear(bf16_dev(x), p, N)
    sync()
    c_o, s_o = W4.fp4_quant(wb)
    _check_fp4_linear(bf16_host(y), x, c_o, s_o)


@pytest.mark.timeout(300)
def test_fp4_decode_config(w):
    d = synth.decode(seed=0)
    K, N = d.x.shape[1], 4096
    wb = _weight(N, K, seed=0)
    _, _, p = w.fp4_quant_weight(bf16_dev(wb))
    c_o, s_o = W4.fp4_quant(wb)
    for M in (1, 4, 16, 64):
        show(f"fp4 decode config M={M}")
        y = w.fp4_linear(bf16_dev(d.x[:M]), p, N)
        sync()
        _check_fp4_linear(bf16_host(y), d.x[:M], c_o, s_o)


# ---------------------------------------------------------------------------
# Dequantized weights read back exactly: with one-hot activation rows
# (x[m, k_m] = 1, zeros elsewhere) every output is 1 * w_deq[n, k_m] plus
# exact zeros, so y[m, n] equals the BF16 dequantized weight itself.
# ---------------------------------------------------------------------------

def _wide_range_weight(N, K, seed, lo_exp, hi_exp):
    """BF16 [N, K] whose groups of 32 have magnitudes 2^e, e drawn from
    [lo_exp, hi_exp], plus an all-zero group and a group with negative zeros."""
    r = np.random.default_rng([seed, 45])
    w = r.standard_normal((N, K)) * np.ldexp(1.0, r.integers(lo_exp, hi_exp + 1, (N, K // 32))).repeat(32, axis=1)
    w[1, :32] = 0.0
    w[2, 32:64] = -0.0
    return O.f32_to_bf16(w.astype(np.float32))


def _one_hot(ks, K):
    x = np.zeros((len(ks), K), np.float32)
    x[np.arange(len(ks)), ks] = 1.0
    return O.f32_to_bf16(x)


def _readback_cases():
    # (M, ks): every k through the packed-activation path, and 16 scattered k
    # through the M <= 16 path
    K = 256
    return K, [np.arange(K), (np.arange(16) * 37 + 5) % K]


@pytest.mark.parametrize("fmt", ["int4", "fp4"])
@pytest.mark.parametrize("exps", [(-100, 100), (-133, -118), (110, 125)], ids=["normal", "tiny", "huge"])
def test_dequant_exact_through_one_hot_rows(w, fmt, exps):
    K, cases = _readback_cases()
    N = 48
    wb = _wide_range_weight(N, K, seed=3, lo_exp=exps[0], hi_exp=exps[1])
    if fmt == "int4":
        _, _, p = w.w4a16_quant_weight(bf16_dev(wb))
        q, s = W4.w4_quant(wb)
        deq = O.bf16_to_f32(W4.w4_dequant(q, s))
        lin = w.w4a16_linear
    else:
        _, _, p = w.fp4_quant_weight(bf16_dev(wb))
        c, s = W4.fp4_quant(wb)
        deq = O.bf16_to_f32(W4.fp4_dequant(c, s))
        lin = w.fp4_linear
    for ks in cases:
        show(f"{fmt} one-hot readback M={len(ks)} K={K} N={N}")
        y = lin(bf16_dev(_one_hot(ks, K)), p, N)
        sync()
        got = O.bf16_to_f32(bf16_host(y))
        want = deq[:, ks].T
        bad = np.argwhere(got != want)          # +0 and -0 compare equal
        assert bad.size == 0, f"{len(bad)} mismatches, first {bad[0].tolist()}: got {got[tuple(bad[0])]} " \
                              f"want {want[tuple(bad[0])]}"


def test_w4_pack_full_code_range_read_back_exact(w):
    """Codes the quantizer never produces (-8) and scales it never produces
    (arbitrary BF16, tiny to large, negative zero groups), packed by
    w4a16_pack and read back through the linear with one-hot rows: every
    dequantized weight equals the oracle's BF16(q * s)."""
    K, cases = _readback_cases()
    N = 40
    r = np.random.default_rng([11, 46])
    q = r.integers(-8, 8, (N, K)).astype(np.int8)
    q[0, :16] = np.arange(-8, 8)                       # every code once in one group
    s_f = (r.standard_normal((N, K // 32)) * np.ldexp(1.0, r.integers(-60, 60, (N, K // 32))))
    s_f[3, 2] = 0.0
    s = O.f32_to_bf16(np.abs(s_f).astype(np.float32))   # scales are non-negative
    p = w.w4a16_pack(dev(q), torch.from_numpy(s.view(np.int16)).cuda().view(torch.bfloat16))
    deq = O.bf16_to_f32(W4.w4_dequant(q, s))
    for ks in cases:
        show(f"w4a16_pack full code range, one-hot readback M={len(ks)}")
        y = w.w4a16_linear(bf16_dev(_one_hot(ks, K)), p, N)
        sync()
        got = O.bf16_to_f32(bf16_host(y))
        want = deq[:, ks].T
        bad = np.argwhere(got != want)
        assert bad.size == 0, f"{len(bad)} mismatches, first {bad[0].tolist()}: got {got[tuple(bad[0])]} " \
                              f"want {want[tuple(bad[0])]}"
