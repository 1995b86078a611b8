"""Parity of the MXFP8 MoE path (through the C ABI) with the CPU oracle.

The one-expert-at-a-time preparation (payload written back over the source
bytes, E8M0 scales, kernel layout) and the SwiGLU -> BF16 -> MX quant are
compared exactly. Every output of the grouped block-scaled matmul is held to
max(2**-8 |ref|, 1e-5) against the float64 sum of the exactly dequantized
products. The chain is compared with the oracle's chain element by element
(see ``_check_chain``).
Inputs are seeded (``synth``); expected values come only from ``oracle``.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests.conftest import gpu_available
from tests.gpu_util import bf16_dev, bf16_host, dev, host, show, sync
from tests.test_gpu_mx import _assert_mx

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

MX = O.mx
MM = O.mx_moe


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


def _stack(E, N, K, bn, bk, seed):
    r = np.random.default_rng([seed, 31])
    wq = synth.e4m3_bits(r.standard_normal((E, N, K), dtype=np.float32))
    s = r.uniform(1e-3, 1e-2, size=(E, -(-N // bn), -(-K // bk))).astype(np.float32)
    return wq, s


def _unpack_mx(buf, N, K):
    """Test-side inverse of the packed MX weight: payload [N, K] from the P16x64
    blocks, scales [N, K/32] from the k-block-major [KB][Np][2] view."""
    NB, KB = -(-N // 16), -(-K // 64)
    buf = np.asarray(buf, np.uint8)
    pay = buf[:NB * KB * 1024].reshape(NB, KB, 4, 16, 16)
    pay = pay.transpose(0, 3, 1, 2, 4).reshape(NB * 16, KB * 64)[:N, :K]
    off = -(-(NB * KB * 1024) // 256) * 256
    sc = buf[off:off + KB * NB * 16 * 2].reshape(KB, NB * 16, 2).transpose(1, 0, 2)
    sc = sc.reshape(NB * 16, KB * 2)[:N, :K // 32]
    return pay, sc


# (E, N, K, bn, bk): the page's 128 x 128 source tiles, cropped edge tiles, an
# odd group count (K % 64 == 32)
PREP_CASES = [(3, 64, 96, 32, 32), (2, 40, 160, 128, 128), (4, 256, 512, 128, 128),
              (1, 48, 32, 16, 8)]


@pytest.mark.parametrize("E,N,K,bn,bk", PREP_CASES)
@pytest.mark.parametrize("alg", [0, 1])
def test_mx_moe_prepare_bit_exact(w, E, N, K, bn, bk, alg):
    show(f"mx_moe_prepare E={E} N={N} K={K} tile={bn}x{bk} alg={alg}")
    wq, s = _stack(E, N, K, bn, bk, seed=E + N + K)
    wd = dev(wq)
    e8, packed = w.mx_moe_prepare(wd, dev(s), bn, bk, scale_alg=alg)
    sync()
    p_o, s_o = MM.mx_moe_prepare(wq, s, bn, bk, scale_alg=alg)
    _assert_eq(host(wd), p_o, "payload written over the source")
    _assert_eq(host(e8), s_o, "e8m0")
    stride = w.mx_moe_packed_bytes(1, N, K)
    buf = host(packed)
    for e in range(E):
        pay, sc = _unpack_mx(buf[e * stride:(e + 1) * stride], N, K)
        _assert_eq(pay, p_o[e], f"packed payload of expert {e}")
        _assert_eq(sc, s_o[e], f"packed scales of expert {e}")


@pytest.mark.parametrize("R,I", [(1, 32), (37, 64), (300, 2048), (64, 96)])
@pytest.mark.parametrize("alg", [0, 1])
def test_mx_swiglu_quant_bit_exact(w, R, I, alg):
    show(f"mx_swiglu_quant R={R} I={I} alg={alg}")
    rng = np.random.default_rng(R + I)
    h = (rng.standard_normal((R, 2 * I)) * 4).astype(np.float32)
    h[0, :4] = [100.0, -100.0, 0.0, -90.0]       # saturating exp on both sides
    if R > 2:
        h[2] = 0.0                               # all-zero row: scale byte 0
    hb = O.f32_to_bf16(h)
    p, sc = w.mx_swiglu_quant(bf16_dev(hb), scale_alg=alg)
    sync()
    p_o, s_o, _ = MM.swiglu_mx_quant(hb, I, scale_alg=alg)
    _assert_eq(host(sc), s_o, "e8m0")
    _assert_eq(host(p), p_o, "e4m3")


def _per_expert(gl, yh, ap, as_, wp, ws, what):
    """Every output within the BF16 bound of its expert's float64 product."""
    off = O.group_offsets(gl)
    refs, rows = [], []
    for e in range(len(gl)):
        a, b = int(off[e]), int(off[e + 1])
        if b == a:
            continue
        refs.append(MX.mx_gemm_ref64(ap[a:b], as_[a:b], wp[e], ws[e]))
        rows.append(yh[a:b])
    _assert_mx(np.concatenate(rows), np.concatenate(refs), what)


def _grouped_case(counts, N, K, act, seed):
    gl = np.asarray(counts, np.int64)
    E, R = len(gl), int(gl.sum())
    Kx = 2 * K if act else K
    x = O.f32_to_bf16((np.random.default_rng(seed).standard_normal((R, Kx)) *
                       (3.0 if act else 1.0)).astype(np.float32))
    wq, s = _stack(E, N, K, 128, 128, seed)
    return gl, x, wq, s


# (counts, N, K): empty and tiny experts, experts spanning several 192-row
# tiles with ragged ends, a partial n-tile, an odd group count
GROUPED_CASES = [([5, 0, 17, 1], 256, 128), ([200, 0, 3, 450, 64], 300, 256),
                 ([0, 0, 37], 512, 96), ([193, 191, 16], 256, 2048)]


@pytest.mark.parametrize("counts,N,K", GROUPED_CASES)
@pytest.mark.parametrize("act", [0, 1])
def test_mx_grouped_gemm_within_tolerance(w, counts, N, K, act):
    show(f"mx_grouped_gemm counts={counts} N={N} K={K} act={act}")
    gl, x, wq, s = _grouped_case(counts, N, K, act, seed=N + K + act)
    _, packed = w.mx_moe_prepare(dev(wq), dev(s), 128, 128)
    y = w.mx_grouped_gemm(bf16_dev(x), dev(gl), packed, N, act=act)
    sync()
    p_o, s_o = MM.mx_moe_prepare(wq, s, 128, 128)
    if act:
        ap, as_, _ = MM.swiglu_mx_quant(x, K)
    else:
        ap, as_ = MX.mx_quant(O.bf16_to_f32(x))
    _per_expert(gl, bf16_host(y), ap, as_, p_o, s_o, "grouped")


def test_mx_grouped_gemm_zero_rows(w):
    gl = np.zeros(4, np.int64)
    wq, s = _stack(4, 64, 64, 128, 128, 1)
    _, packed = w.mx_moe_prepare(dev(wq), dev(s), 128, 128)
    y = w.mx_grouped_gemm(torch.empty((0, 64), dtype=torch.bfloat16, device="cuda"), dev(gl),
                          packed, 64)
    sync()
    assert y.shape == (0, 64)


# (counts, H, I): small experts, multi-tile experts, odd group counts
CHAIN_CASES = [([12, 7, 0, 19], 64, 32), ([0, 200, 3, 0, 70], 256, 128),
               ([300, 5, 190], 512, 256)]

# Element-wise check of the chain. The W13 stage sums exact products in fp32,
# so its BF16 output h can be either BF16 neighbour of the exact sum when that
# sum lies near a rounding boundary: several chains are correct. The oracle
# brackets what any fp32 accumulation in 64-deep k-blocks can return (each
# MFMA step adds a partial sum of at most 16 exact products to the fp32
# accumulator within one fp32 ulp of the magnitudes involved):
#   delta = 2^-23 (4 sum_b |S_(b-1)| + 20 sum_k |p_k|),
# S_b the exact partial sum after k-block b. The admissible h are the BF16
# roundings of [h64 - delta, h64 + delta]; the GPU's h must be one of them.
# Where an element has more than one, the oracle bounds how far SwiGLU ->
# BF16 -> MX quant can move each dequantized value of the row over those
# choices (_row_delta), Delta[r, k]; a chain output may then move by
# sum_k Delta[r, k] |W2[n, k]| on top of the BF16 bound. Rows without such
# an element are held to the BF16 bound alone.
U23 = 2.0 ** -23


def _accumulation_bound(A, W):
    """(delta, exact sums) of the product A @ W.T over dequantized operands."""
    S = np.zeros((A.shape[0], W.shape[0]))
    tot = np.zeros_like(S)
    for k0 in range(0, A.shape[1], 64):
        tot += 4.0 * np.abs(S)
        S += A[:, k0:k0 + 64] @ W[:, k0:k0 + 64].T
    return U23 * (tot + 20.0 * (np.abs(A) @ np.abs(W).T)) * 1.01, S


def _bf16_of64(v):
    return O.f32_to_bf16(np.asarray(v, np.float64).astype(np.float32))


def _row_delta(h_o, lo, hi, inter, base_deq):
    """Largest change of each dequantized SwiGLU-MX value of one row when every
    element of h (BF16 bits, [gate | up]) may take any value of its admissible
    range [lo, hi] instead of the oracle's h_o. Interval bound: a = BF16(silu(g)
    * u) is evaluated at the corners of its (gate, up) box (over such a short
    range both factors are monotone), the group's shared exponent can be any
    E of its amax range, and for each such E the quantizer (monotone) maps the
    ends of an element's range to the ends of its codes."""
    hs = [h_o]
    for gsel in (lo, hi):
        for usel in (lo, hi):
            hs.append(np.concatenate([gsel[:inter], usel[inter:]]))
    a = O.bf16_to_f32(O.f32_to_bf16(O.swiglu(np.stack(hs), inter))).astype(np.float64)
    a_min, a_max = a.min(axis=0), a.max(axis=0)
    abs_min = np.where((a_min <= 0) & (a_max >= 0), 0.0, np.minimum(np.abs(a_min), np.abs(a_max)))
    abs_max = np.maximum(np.abs(a_min), np.abs(a_max))
    G = inter // 32
    e_lo = MX.mx_shared_exponent(abs_min.reshape(G, 32).max(axis=1))
    e_hi = MX.mx_shared_exponent(abs_max.reshape(G, 32).max(axis=1))
    base = base_deq.reshape(G, 32)
    delta = np.zeros((G, 32))
    for de in range(int((e_hi - e_lo).max()) + 1):
        E = np.minimum(e_lo + de, e_hi)[:, None].astype(np.float64)
        for v in (a_min, a_max):
            q = MX.e4m3_decode(MX.e4m3_encode(np.ldexp(v.reshape(G, 32), -E.astype(np.int64))))
            delta = np.maximum(delta, np.abs(np.ldexp(q, E.astype(np.int64)) - base))
    return delta.reshape(inter)


def _check_chain(gl, st, o13, o2, h_gpu, y_gpu, what):
    """h_gpu within the admissible W13 outputs; every chain output within the
    BF16 bound of the oracle chain's float64 W2 sum plus the allowance of its
    row (zero for rows whose h has a single admissible value)."""
    inter = o13[0].shape[1] // 2
    off = O.group_offsets(gl)
    hv = O.bf16_to_f32(h_gpu).astype(np.float64)
    yv = O.bf16_to_f32(y_gpu).astype(np.float64)
    n_two = n_rows = n_used = 0
    worst = 0.0
    for e in range(len(gl)):
        a, b = int(off[e]), int(off[e + 1])
        if b == a:
            continue
        A1 = MX.mx_dequant(st["q1"][a:b], st["s1"][a:b])
        d, h64 = _accumulation_bound(A1, MX.mx_dequant(o13[0][e], o13[1][e]))
        lo, hi = _bf16_of64(h64 - d), _bf16_of64(h64 + d)
        lv, hv_ = O.bf16_to_f32(lo).astype(np.float64), O.bf16_to_f32(hi).astype(np.float64)
        inside = (hv[a:b] >= lv) & (hv[a:b] <= hv_)
        assert inside.all(), (f"{what}: W13 output outside the fp32-accumulation range at "
                              f"{np.argwhere(~inside)[0].tolist()} (expert {e})")
        W2 = MX.mx_dequant(o2[0][e], o2[1][e])
        A2 = MX.mx_dequant(st["q2"][a:b], st["s2"][a:b])
        y64 = A2 @ W2.T
        allow = np.zeros_like(y64)
        for r in range(b - a):
            if (lo[r] != hi[r]).any():
                n_two += int((lo[r] != hi[r]).sum())
                n_rows += 1
                allow[r] = np.abs(W2) @ _row_delta(st["h"][a + r], lo[r], hi[r], inter, A2[r])
        base = np.maximum(O.REL_TOL * np.abs(y64), O.ABS_FLOOR)
        err = np.abs(yv[a:b] - y64)
        n_used += int((err > base).sum())
        worst = max(worst, float(np.max(err / (base + 1.004 * allow))))
        ok = err <= base + 1.004 * allow
        assert ok.all(), (f"{what}: chain output {np.argwhere(~ok)[0].tolist()} of expert {e} "
                          f"outside the bound + allowance")
    show(f"  {what}: {n_two} W13 outputs with two admissible values in {n_rows} rows; "
         f"{n_used} chain outputs past the BF16 bound alone; max err/tolerance {worst:.4f}")


@pytest.mark.parametrize("counts,H,I", CHAIN_CASES)
def test_mx_moe_chain(w, counts, H, I):
    """The chain equals its two grouped calls bit for bit; stage 1 is within the
    BF16 bound of the oracle's W13; stage 2 run on the oracle's own W13 output
    is within the bound of the oracle's W2; every chain output is within the
    bound (plus its row's rounding allowance) of the oracle's chain."""
    show(f"mx_moe chain counts={counts} H={H} I={I}")
    gl = np.asarray(counts, np.int64)
    E, R = len(gl), int(gl.sum())
    # activations scaled so that the W13 outputs reach SwiGLU's nonlinear range
    x = O.f32_to_bf16((np.random.default_rng(H).standard_normal((R, H)) * 64).astype(np.float32))
    w13q, s13 = _stack(E, 2 * I, H, 128, 128, seed=H + 1)
    w2q, s2 = _stack(E, H, I, 128, 128, seed=H + 2)
    _, p13 = w.mx_moe_prepare(dev(w13q), dev(s13), 128, 128)
    _, p2 = w.mx_moe_prepare(dev(w2q), dev(s2), 128, 128)
    o13 = MM.mx_moe_prepare(w13q, s13, 128, 128)
    o2 = MM.mx_moe_prepare(w2q, s2, 128, 128)
    st = MM.mx_moe_grouped(gl, x, *o13, *o2, keep=True)
    y = w.mx_moe_grouped(bf16_dev(x), dev(gl), p13, p2, I)
    h = w.mx_grouped_gemm(bf16_dev(x), dev(gl), p13, 2 * I)
    y2 = w.mx_grouped_gemm(h, dev(gl), p2, H, act=w.ACT_SWIGLU)
    y3 = w.mx_grouped_gemm(bf16_dev(st["h"]), dev(gl), p2, H, act=w.ACT_SWIGLU)
    sync()
    _assert_eq(bf16_host(y), bf16_host(y2), "chain == two grouped calls")
    _per_expert(gl, bf16_host(h), st["q1"], st["s1"], *o13, "W13")
    _per_expert(gl, bf16_host(y3), st["q2"], st["s2"], *o2, "W2 on the oracle's h")
    _check_chain(gl, st, o13, o2, bf16_host(h), bf16_host(y), "chain")


@pytest.mark.timeout(900)
def test_mx_moe_config_sampled_rows(w):
    """The MoE workload with MXFP8 experts at full size. Experts of the sampled
    rows are prepared from their block-FP8 source; the others hold zero bytes
    (valid E4M3 / E8M0, same launch shapes). The oracle recomputes the sampled
    rows one by one: W13 within the BF16 bound, every chain output within the
    bound plus its row's rounding allowance."""
    show("mx_moe full size, sampled rows")
    m = synth.mx_moe(seed=0)
    E, H, I = m.E, m.H, m.I
    off = O.group_offsets(m.group_list)
    ex = np.repeat(np.arange(E), m.group_list)
    rng = np.random.default_rng(3)
    big = int(np.argmax(m.group_list))
    rows = sorted(set(rng.integers(0, m.R, 13).tolist()) | {0, m.R - 1, int(off[big + 1]) - 1})
    experts = sorted({int(ex[r]) for r in rows})
    s13b = w.mx_moe_packed_bytes(1, 2 * I, H)
    s2b = w.mx_moe_packed_bytes(1, H, I)
    p13 = torch.zeros(E * s13b, dtype=torch.uint8, device="cuda")
    p2 = torch.zeros(E * s2b, dtype=torch.uint8, device="cuda")
    src = {}
    for e in experts:
        (wa, sa), (wb, sb) = m.w13(e), m.w2(e)
        src[e] = (wa, sa, wb, sb)
        w.mx_moe_prepare(dev(wa[None]), dev(sa[None]), m.bn, m.bk, packed=p13[e * s13b:(e + 1) * s13b])
        w.mx_moe_prepare(dev(wb[None]), dev(sb[None]), m.bn, m.bk, packed=p2[e * s2b:(e + 1) * s2b])
    xr = m.x_rows()
    xd, gd = bf16_dev(xr), dev(m.group_list)
    y = w.mx_moe_grouped(xd, gd, p13, p2, I)
    h = w.mx_grouped_gemm(xd, gd, p13, 2 * I)
    yh = bf16_host(y)
    hh = bf16_host(h)
    one = np.array([1], np.int64)
    prepared = {}
    for r in rows:
        e = int(ex[r])
        if e not in prepared:
            wa, sa, wb, sb = src[e]
            prepared = {e: (MM.mx_moe_prepare(wa[None], sa[None], m.bn, m.bk),
                            MM.mx_moe_prepare(wb[None], sb[None], m.bn, m.bk))}
        o13, o2 = prepared[e]
        st = MM.mx_moe_grouped(one, xr[r:r + 1], *o13, *o2, keep=True)
        _per_expert(one, hh[r:r + 1], st["q1"], st["s1"], *o13, f"W13 row {r}")
        _check_chain(one, st, o13, o2, hh[r:r + 1], yh[r:r + 1], f"chain row {r} (expert {e})")
