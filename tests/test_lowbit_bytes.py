"""Bytes per parameter of the two low-bit weight formats against the totals the
page "超大 MoE 的低比特推理：INT4、FP4 与量化感知训练" prints for a 1e12-parameter
model (section "4 比特对万亿 MoE 意味着什么", tests/golden/lowbit_weight_bytes.txt).

Pinned on both sides without a GPU: the oracle's own representation (codes and
scales as the oracle returns them) and the C ABI's packed sizes (host queries).
A format that dropped its scales, stored a scale per 16 values, or padded each
group would print a different total.
"""

import os

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "lowbit_weight_bytes.txt")


def _golden():
    rows = {}
    for line in open(GOLDEN, encoding="utf-8"):
        if line.startswith("#") or not line.strip():
            continue
        name, group, sbytes, tb = line.split()
        rows[name] = (int(group), int(sbytes), tb)
    return rows


def _printed(bytes_per_param):
    """The page's figure: 1e12 parameters times the bytes per parameter, in TB,
    two decimals."""
    return f"{1e12 * bytes_per_param / 1e12:.2f}"


def test_oracle_int4_and_fp4_storage_match_printed_totals():
    g = _golden()
    N, K = 64, 1024
    w = O.f32_to_bf16(np.random.default_rng(0).standard_normal((N, K)).astype(np.float32))
    q, s = O.w4a16.w4_quant(w)
    # 4-bit codes (half a byte each) + one BF16 scale per group of 32
    int4 = (q.size * 0.5 + s.size * s.itemsize) / (N * K)
    assert s.shape == (N, K // g["INT4"][0]) and s.itemsize == g["INT4"][1]
    assert _printed(int4) == g["INT4"][2]
    c, e = O.w4a16.fp4_quant(w)
    fp4 = (c.size * 0.5 + e.size * e.itemsize) / (N * K)
    assert e.shape == (N, K // g["MXFP4"][0]) and e.itemsize == g["MXFP4"][1]
    assert _printed(fp4) == g["MXFP4"][2]


@pytest.mark.parametrize("N,K", [(4096, 7168), (5120, 17408), (160, 2048)])
def test_packed_sizes_match_printed_totals(N, K):
    import moe_token_amax_amd as w
    g = _golden()
    int4 = w.w4a16_packed_bytes(N, K) / (N * K)
    fp4 = w.fp4_packed_bytes(N, K) / (N * K)
    assert int4 == 0.5 + g["INT4"][1] / g["INT4"][0]
    assert fp4 == 0.5 + g["MXFP4"][1] / g["MXFP4"][0]
    assert _printed(int4) == g["INT4"][2]
    assert _printed(fp4) == g["MXFP4"][2]
