"""Pins of the MXFP8 oracle (CPU only)."""

import os

import numpy as np
import pytest
import torch

from oracle import mx

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mx_examples.txt")


def _golden():
    out = {}
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        k, *v = line.split()
        out[k] = [int(x) for x in v]
    return out


def test_e4m3_hand_values():
    v = [1.0, 0.5, -1.75, 240.0, 256.0, 448.0, 2.0 ** -9, 2.0 ** -10, 1.5 * 2.0 ** -10, -0.0,
         464.0, 500.0, 1e6]
    want = [0x38, 0x30, 0xBE, 0x77, 0x78, 0x7E, 0x01, 0x00, 0x01, 0x80, 0x7E, 0x7E, 0x7E]
    assert list(mx.e4m3_encode(np.array(v))) == want


def test_e4m3_matches_torch_in_range():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.normal(0, 40, 200_000), rng.uniform(-448, 448, 100_000),
                        rng.normal(0, 2.0 ** -7, 100_000)]).astype(np.float32)
    # every midpoint between neighbouring codes (ties) and every code itself
    pos = mx.e4m3_values()[:0x7F]
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)
    v = np.concatenate([v, mids, -mids, pos.astype(np.float32)])
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(mx.e4m3_encode(v), ref)


def test_e4m3_round_trip_all_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    assert np.array_equal(mx.e4m3_encode(mx.e4m3_decode(codes)), codes)


def test_e4m3_saturates():
    assert mx.e4m3_encode(np.array([449.0, 480.0, -1000.0])).tolist() == [0x7E, 0x7E, 0xFE]


def test_shared_exponent_hand_groups():
    row = np.zeros((3, 32))
    row[0, 0] = 1.0          # E = -8 -> byte 0x77, 1.0 * 2^8 = 256 -> 0x78
    row[1, 5] = 1.875        # 480 saturates to 448 under rule 0
    row[2, :] = 0.0          # empty group -> byte 0
    p, s = mx.mx_quant(row, scale_alg=0)
    assert s[:, 0].tolist() == [0x77, 0x77, 0x00]
    assert p[0, 0] == 0x78 and p[1, 5] == 0x7E and not p[2].any()
    p1, s1 = mx.mx_quant(row, scale_alg=1)     # no saturation: E = -7, 240 -> 0x77
    assert s1[1, 0] == 0x78 and p1[1, 5] == 0x77


def test_mx_quant_groups_per_row_worked_example():
    K, groups = _golden()["groups_per_row"]
    x = np.random.default_rng(1).normal(size=(3, K))
    p, s = mx.mx_quant(x)
    assert p.shape == (3, K) and s.shape == (3, groups)
    with pytest.raises(ValueError):
        mx.mx_quant(np.ones((2, 48)))


def test_mx_quant_brute_force_and_bounds():
    rng = np.random.default_rng(2)
    x = (rng.normal(size=(6, 96)) * rng.uniform(1e-3, 1e3, size=(6, 1))).astype(np.float32)
    x[1, 32:64] = 0.0
    p, s = mx.mx_quant(x)
    vals = mx.e4m3_values()
    for r in range(6):
        for g in range(3):
            grp = x[r, 32 * g:32 * g + 32].astype(np.float64)
            amax = np.abs(grp).max()
            if amax == 0:
                assert s[r, g] == 0
                continue
            e = int(np.floor(np.log2(amax))) - 8
            assert s[r, g] == e + 127
            for j in range(32):
                t = grp[j] / 2.0 ** e
                # nearest code by exhaustive search, ties to even, saturating
                cands = [(abs(abs(t) - vals[c]), c % 2, c) for c in range(0x7F)]
                best = min(cands)[2]
                if abs(t) >= 448:
                    best = 0x7E
                code = best | (0x80 if np.signbit(t) else 0)
                assert p[r, 32 * g + j] == code
    # dequantized error bounded by half a step of the group's scale (or saturation)
    d = mx.mx_dequant(p, s)
    assert np.all(np.abs(d - x) <= np.abs(x) * 2.0 ** -4 + 2.0 ** (s.repeat(32, 1) - 127.0 - 10))


def test_resolve_worked_tile_and_brute_force():
    bn, bk = _golden()["resolve_tile"]
    rng = np.random.default_rng(3)
    N, K = 10, 20                      # ragged: edge tiles cropped
    w = rng.integers(0, 256, size=(N, K)).astype(np.uint8)
    w[(w & 0x7F) == 0x7F] = 0x38        # no NaN codes
    S = rng.uniform(1e-3, 1e-2, size=(-(-N // bn), -(-K // bk))).astype(np.float32)
    got = mx.mx_resolve(w, S, bn, bk)
    vals = mx.e4m3_values()
    import oracle
    for i in range(N):
        for j in range(K):
            prod = np.float32(vals[w[i, j]]) * S[i // bn, j // bk]
            assert got[i, j] == oracle.f32_to_bf16(np.array([prod], np.float32))[0]
    # one source scale covers exactly a bn x bk block
    S2 = np.ones_like(S)
    S2[0, 0] = 2.0
    w1 = np.full((N, K), 0x38, np.uint8)        # 1.0 everywhere
    r = oracle.bf16_to_f32(mx.mx_resolve(w1, S2, bn, bk))
    assert (r == 2.0).sum() == bn * bk and np.all(r[:bn, :bk] == 2.0)
    with pytest.raises(ValueError):
        mx.mx_resolve(w, S[:-1], bn, bk)


def test_mx_gemm_ref_brute_force():
    rng = np.random.default_rng(4)
    a = rng.normal(size=(3, 64))
    w = rng.normal(size=(4, 64)) * 0.01
    ap, as_ = mx.mx_quant(a)
    wp, ws = mx.mx_quant(w)
    ref = mx.mx_gemm_ref64(ap, as_, wp, ws)
    vals = mx.e4m3_values()
    for m in range(3):
        for n in range(4):
            t = 0.0
            for k in range(64):
                g = k // 32
                t += vals[ap[m, k]] * 2.0 ** (int(as_[m, g]) - 127) * \
                    vals[wp[n, k]] * 2.0 ** (int(ws[n, g]) - 127)
            assert np.isclose(ref[m, n], t, rtol=1e-12, atol=0)
