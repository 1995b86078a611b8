"""Parity of the grouped low-bit (INT4 / FP4 expert weight) path and its
expert chain (through the C ABI) with the CPU oracle.

The grouped matmul multiplies exactly dequantized BF16 weights and accumulates
in fp32, as the dense W4A16 linear does, so each BF16 output is compared with
the float64 sum of its own expert under the BF16 bound max(2**-8 |ref|, 1e-5)
plus the fp32 accumulation allowance LAMBDA * sqrt(K) * 2**-24 * sum_k |x w|.
The SwiGLU between W13 and W2 is a fixed fp32 sequence rounded once to BF16 and
is compared bit for bit on the GPU's own W13 output. The chain equals its three
stage calls bit for bit; its W2 stage is within the bound of the oracle run on
the GPU's own SwiGLU output, and the whole chain is within that bound plus the
propagation sum_k |a_gpu - a_oracle| |w2| of the oracle's own chain. Inputs are
seeded; expected values come only from ``oracle``.
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
FMTS = ["int4", "fp4"]


@pytest.fixture(scope="module")
def w():
    import moe_token_amax_amd as w
    return w


def _code(w, fmt):
    return w.LOWBIT_INT4 if fmt == "int4" else w.LOWBIT_FP4


def _expert_weights(E, N, K, seed):
    """BF16 bits [E, N, K]; expert magnitudes spread over 16x so that a row
    multiplied by another expert's weight cannot pass."""
    out = np.empty((E, N, K), np.uint16)
    for e in range(E):
        r = np.random.default_rng([seed, 45, e])
        out[e] = O.f32_to_bf16((r.standard_normal((N, K)) * 0.01 * 2.0 ** (e % 5)).astype(np.float32))
    return out


def _quant(w, fmt, wb):
    """GPU quant of the stacked [E * N, K] weight (N % 16 == 0: the per-expert
    packed layouts back to back) and the oracle's codes and scales per expert;
    the GPU codes and scales must equal the oracle's."""
    E, N, K = wb.shape
    stack = bf16_dev(wb.reshape(E * N, K))
    if fmt == "int4":
        q, s, p = w.w4a16_quant_weight(stack, codes=True, scales=True, pack=True)
        oq = [W4.w4_quant(wb[e]) for e in range(E)]
        sync()
        assert np.array_equal(host(q).reshape(E, N, K), np.stack([c for c, _ in oq]))
        assert np.array_equal(host(s.view(torch.int16)).view(np.uint16).reshape(E, N, K // 32),
                              np.stack([t for _, t in oq]))
    else:
        q, s, p = w.fp4_quant_weight(stack, codes=True, scales=True, pack=True)
        oq = [W4.fp4_quant(wb[e]) for e in range(E)]
        sync()
        assert np.array_equal(host(q).reshape(E, N, K), np.stack([c for c, _ in oq]))
        assert np.array_equal(host(s).reshape(E, N, K // 32), np.stack([t for _, t in oq]))
    codes = np.stack([c for c, _ in oq])
    scales = np.stack([t for _, t in oq])
    return p, codes, scales


def _check(fmt, y_bits, x_bits, gl, codes, scales, what):
    """Every row against the float64 sum of its own expert (BF16 bound plus the
    fp32 accumulation allowance); returns the max err / tolerance."""
    ref = W4.lowbit_grouped_ref64(fmt, x_bits, gl, codes, scales)
    off = O.group_offsets(gl)
    xf = O.bf16_to_f32(x_bits).astype(np.float64)
    mag = np.zeros_like(ref)
    for e in range(len(gl)):
        a, b = int(off[e]), int(off[e + 1])
        if b > a:
            wf = O.bf16_to_f32(W4.lowbit_dequant(fmt, codes[e], scales[e])).astype(np.float64)
            mag[a:b] = np.abs(xf[a:b]) @ np.abs(wf).T
    allow = LAMBDA * np.sqrt(xf.shape[1]) * 2.0 ** -24 * mag
    y = O.bf16_to_f32(y_bits).astype(np.float64)
    err = np.abs(y - ref)
    tol = np.maximum(O.REL_TOL * np.abs(ref), O.ABS_FLOOR) + allow
    ok = err <= tol
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        raise AssertionError(f"{what}: {int((~ok).sum())} of {ok.size} outside tolerance, first {i}: "
                             f"got {y[i]} want {ref[i]} tolerance {tol[i]}")
    worst = float((err / tol).max()) if err.size else 0.0
    show(f"  {what}: max err/tolerance {worst:.3f}")
    return ref, worst


# (counts, N, K): the page's worked counts with an empty expert; experts of 70
# and 130 rows (64-row tiles plus ragged 6- and 2-row tiles), N = 272 (a second
# 256-column group that only its first wavefront fills), K = 416 (a last chunk
# of one step); eight 1-row experts and one of 40 (1-, 2- and 4-block tiles),
# K = 4160 (33 chunks: a last chunk of two steps past the 3-chunk rotation);
# all rows in one expert of a long list; one expert of 129 rows
GROUPED_CASES = [
    ([12, 7, 0, 19], 256, 256),
    ([0, 70, 0, 5, 130], 272, 416),
    ([1] * 8 + [40], 512, 4160),
    ([300, 0, 17, 33, 64, 65], 1024, 2048),
    ([0, 0, 50, 0] + [0] * 60, 64, 128),
    ([129], 48, 96),
]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("counts,N,K", GROUPED_CASES)
def test_lowbit_grouped_gemm_within_tolerance(w, fmt, counts, N, K):
    show(f"w4a16_grouped_gemm fmt={fmt} counts={counts[:9]} N={N} K={K}")
    gl = np.asarray(counts, np.int64)
    E, R = len(gl), int(gl.sum())
    x = synth.activations(R, K, 0.005, seed=R + N + K)
    wb = _expert_weights(E, N, K, seed=N + K)
    p, codes, scales = _quant(w, fmt, wb)
    y = w.w4a16_grouped_gemm(bf16_dev(x), dev(gl), p, N, fmt=_code(w, fmt))
    sync()
    _check(fmt, bf16_host(y), x, gl, codes, scales, "grouped")


@pytest.mark.parametrize("fmt", FMTS)
def test_lowbit_grouped_gemm_rows_past_the_counts_untouched(w, fmt):
    """Rows not owned by any expert (counts summing below R) keep their old
    values; the owned rows are right."""
    gl = np.array([5, 0, 20], np.int64)
    R, N, K = 40, 64, 128
    x = synth.activations(R, K, 0.0, seed=7)
    wb = _expert_weights(3, N, K, seed=8)
    p, codes, scales = _quant(w, fmt, wb)
    y = torch.full((R, N), 3.0, dtype=torch.bfloat16, device="cuda")
    w.w4a16_grouped_gemm(bf16_dev(x), dev(gl), p, N, fmt=_code(w, fmt), y=y)
    sync()
    yh = bf16_host(y)
    assert np.all(O.bf16_to_f32(yh[25:]) == 3.0)
    _check(fmt, yh[:25], x[:25], gl, codes, scales, "owned rows")


def test_lowbit_grouped_gemm_zero_rows(w):
    gl = torch.zeros(4, dtype=torch.int64, device="cuda")
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    p = torch.zeros(4 * w.w4a16_packed_bytes(32, 64), dtype=torch.uint8, device="cuda")
    y = w.w4a16_grouped_gemm(x, gl, p, 32)
    sync()
    assert y.shape == (0, 32)


@pytest.mark.parametrize("R,I", [(37, 64), (5, 8), (3, 5)])
def test_lowbit_swiglu_bit_exact(w, R, I):
    """Vector (I % 8 == 0) and element paths against the oracle's fixed
    sequence, on values that reach both tails of the exponential."""
    show(f"w4a16_swiglu R={R} I={I}")
    r = np.random.default_rng(R * I)
    h = O.f32_to_bf16((r.standard_normal((R, 2 * I)) * 8).astype(np.float32))
    # gates 0, -100 (exp overflows: -0), 100, 20
    h[0, :4] = O.f32_to_bf16(np.array([0.0, -100.0, 100.0, 20.0], np.float32))
    a = w.w4a16_swiglu(bf16_dev(h))
    sync()
    want = W4.lowbit_swiglu(h, I)
    got = bf16_host(a)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} mismatches, first {bad[0].tolist()}: {got[tuple(bad[0])]} vs " \
                          f"{want[tuple(bad[0])]}"


CHAIN_CASES = [([12, 7, 0, 19], 256, 128), ([0, 70, 3, 130], 512, 256), ([1, 2, 0, 64, 65], 128, 96)]


def _chain(w, fmt, gl, x, H, I, seed):
    E = len(gl)
    w13 = _expert_weights(E, 2 * I, H, seed)
    w2 = _expert_weights(E, H, I, seed + 1)
    p13, c13, s13 = _quant(w, fmt, w13)
    p2, c2, s2 = _quant(w, fmt, w2)
    return p13, p2, (c13, s13), (c2, s2)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("counts,H,I", CHAIN_CASES)
def test_lowbit_moe_chain(w, fmt, counts, H, I):
    show(f"w4a16_moe_grouped fmt={fmt} counts={counts} H={H} I={I}")
    gl = np.asarray(counts, np.int64)
    R = int(gl.sum())
    # activations large enough that the W13 outputs reach SwiGLU's nonlinear range
    x = O.f32_to_bf16((np.random.default_rng(H + I).standard_normal((R, H)) * 4).astype(np.float32))
    p13, p2, o13, o2 = _chain(w, fmt, gl, x, H, I, seed=H + I)
    code = _code(w, fmt)
    xd, gd = bf16_dev(x), dev(gl)
    ws = torch.empty(w.w4a16_moe_workspace_bytes(R, H, I), dtype=torch.uint8, device="cuda")
    y = w.w4a16_moe_grouped(xd, gd, p13, p2, I, fmt=code, workspace=ws)
    h = w.w4a16_grouped_gemm(xd, gd, p13, 2 * I, fmt=code)
    a = w.w4a16_swiglu(h)
    y3 = w.w4a16_grouped_gemm(a, gd, p2, H, fmt=code)
    sync()
    yh, hh, ah = bf16_host(y), bf16_host(h), bf16_host(a)
    assert np.array_equal(yh, bf16_host(y3)), "chain == its three stage calls"
    # the workspace keeps h and a
    hb = R * 2 * I * 2
    assert np.array_equal(host(ws[:hb]).view(np.uint16).reshape(R, 2 * I), hh)
    a_off = -(-hb // 256) * 256
    assert np.array_equal(host(ws[a_off:a_off + R * I * 2]).view(np.uint16).reshape(R, I), ah)
    _check(fmt, hh, x, gl, *o13, "W13")
    assert np.array_equal(ah, W4.lowbit_swiglu(hh, I)), "SwiGLU on the GPU's own W13 output"
    _check(fmt, yh, ah, gl, *o2, "W2 on the GPU's own SwiGLU output")
    # the whole chain against the oracle's own chain
    st = W4.lowbit_moe(fmt, gl, x, *o13, *o2, keep=True)
    n_h = int((st["h"] != hh).sum())
    da = np.abs(O.bf16_to_f32(ah).astype(np.float64) - O.bf16_to_f32(st["a"]).astype(np.float64))
    off = O.group_offsets(gl)
    prop = np.zeros((R, H))
    mag = np.zeros((R, H))
    af = O.bf16_to_f32(ah).astype(np.float64)
    for e in range(len(gl)):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi > lo:
            wf = np.abs(O.bf16_to_f32(W4.lowbit_dequant(fmt, o2[0][e], o2[1][e])).astype(np.float64))
            prop[lo:hi] = da[lo:hi] @ wf.T
            mag[lo:hi] = np.abs(af[lo:hi]) @ wf.T
    ref = st["y64"]
    ref_g = W4.lowbit_grouped_ref64(fmt, ah, gl, *o2)
    tol = np.maximum(O.REL_TOL * np.abs(ref_g), O.ABS_FLOOR) + LAMBDA * np.sqrt(I) * 2.0 ** -24 * mag
    err = np.abs(O.bf16_to_f32(yh).astype(np.float64) - ref)
    ok = err <= tol + prop * (1 + 2.0 ** -40)
    assert ok.all(), f"chain output {np.argwhere(~ok)[0].tolist()} outside bound + propagation"
    show(f"  {n_h} of {hh.size} W13 outputs differ from the oracle's BF16 rounding by one unit; "
         f"{int((da > 0).sum())} SwiGLU outputs differ")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("fmt", FMTS)
def test_lowbit_moe_config_sampled_rows(w, fmt):
    """The MoE workload (2048 tokens, top-8 of 256 experts, H 4096, I 2048)
    with low-bit experts at full size. Experts of the sampled rows are
    quantized from their seeded BF16 weights; the others hold zero bytes (zero
    weights in either format, same launch shapes). The oracle recomputes the
    sampled rows one by one: W13 within the bound, SwiGLU bit-exact on the
    GPU's W13 output, W2 within the bound on the GPU's SwiGLU output."""
    show(f"w4a16_moe full size fmt={fmt}, sampled rows")
    m = synth.lowbit_moe(seed=0)
    E, H, I = m.E, m.H, m.I
    code = _code(w, fmt)
    b13 = w.w4a16_packed_bytes(2 * I, H) if fmt == "int4" else w.fp4_packed_bytes(2 * I, H)
    b2 = w.w4a16_packed_bytes(H, I) if fmt == "int4" else w.fp4_packed_bytes(H, I)
    off = O.group_offsets(m.group_list)
    ex = np.repeat(np.arange(E), m.group_list)
    rng = np.random.default_rng(5)
    big = int(np.argmax(m.group_list))
    rows = sorted(set(rng.integers(0, m.R, 10).tolist()) | {0, m.R - 1, int(off[big + 1]) - 1})
    experts = sorted({int(ex[r]) for r in rows})
    p13 = torch.zeros(E * b13, dtype=torch.uint8, device="cuda")
    p2 = torch.zeros(E * b2, dtype=torch.uint8, device="cuda")
    quant = w.w4a16_quant_weight if fmt == "int4" else w.fp4_quant_weight
    ref_w = {}
    for e in experts:
        wa, wb2 = m.w13(e), m.w2(e)
        _, _, pa = quant(bf16_dev(wa))
        _, _, pb = quant(bf16_dev(wb2))
        p13[e * b13:(e + 1) * b13] = pa
        p2[e * b2:(e + 1) * b2] = pb
        qa = W4.w4_quant(wa) if fmt == "int4" else W4.fp4_quant(wa)
        qb = W4.w4_quant(wb2) if fmt == "int4" else W4.fp4_quant(wb2)
        ref_w[e] = (qa, qb)
    xr = m.x_rows()
    xd, gd = bf16_dev(xr), dev(m.group_list)
    ws = torch.empty(w.w4a16_moe_workspace_bytes(m.R, H, I), dtype=torch.uint8, device="cuda")
    y = w.w4a16_moe_grouped(xd, gd, p13, p2, I, fmt=code, workspace=ws)
    sync()
    yh = bf16_host(y)
    hh = host(ws[:m.R * 2 * I * 2]).view(np.uint16).reshape(m.R, 2 * I)
    a_off = -(-(m.R * 2 * I * 2) // 256) * 256
    ah = host(ws[a_off:a_off + m.R * I * 2]).view(np.uint16).reshape(m.R, I)
    one = np.array([1], np.int64)
    for r in rows:
        e = int(ex[r])
        (qa, sa), (qb, sb) = ref_w[e]
        _check(fmt, hh[r:r + 1], xr[r:r + 1], one, qa[None], sa[None], f"W13 row {r} (expert {e})")
        assert np.array_equal(ah[r:r + 1], W4.lowbit_swiglu(hh[r:r + 1], I)), f"SwiGLU row {r}"
        _check(fmt, yh[r:r + 1], ah[r:r + 1], one, qb[None], sb[None], f"W2 row {r} (expert {e})")
