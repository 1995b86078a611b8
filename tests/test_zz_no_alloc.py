"""The grouped GEMM entry point that allocates nothing (schedule in the
library's own device array) against w8a8_grouped_gemm, through the C ABI:
two calls in a row, the second on fewer rows and experts, bit for bit."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from tests.conftest import gpu_available
from tests.gpu_util import bf16_host, dev, host, show, sync

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def w():
    import moe_token_amax_amd as w
    return w


def _case(counts, N, K, seed):
    g = np.asarray(counts, np.int64)
    R, E = int(g.sum()), len(g)
    a = synth.int8_weight((R, K), seed, 11)
    xs = synth.scales(R, seed, 12)
    wt = synth.int8_weight((E, N, K), seed, 13)
    ws = synth.scales((E, N), seed, 14)
    return g, a, xs, wt, ws


def test_grouped_gemm_noalloc_matches_workspace_call(w):
    # first call: 300 rows over 7 experts (small and tiled experts, an empty
    # one); second: 40 rows over 3 experts, so the schedule it leaves behind is
    # shorter than the first one's
    cases = [([0, 120, 1, 64, 0, 90, 25], 272, 1024), ([17, 0, 23], 96, 320)]
    for i, (counts, N, K) in enumerate(cases):
        show(f"grouped_gemm_noalloc call {i}: counts={counts} N={N} K={K}")
        g, a, xs, wt, ws = _case(counts, N, K, seed=5 + i)
        R = int(g.sum())
        wp = w.prepack_weight(dev(wt))
        ad, xsd, gd, wsd = dev(a), dev(xs), dev(g), dev(ws)
        for out, dt in ((w.OUT_BF16, torch.bfloat16), (w.OUT_I32, torch.int32)):
            want = w.grouped_gemm(ad, xsd, gd, wp, wsd, N, out=out)
            got = torch.empty((R, N), dtype=dt, device="cuda")
            w.grouped_gemm_noalloc(ad, xsd, gd, wp, wsd, N, got, out=out)
            sync()
            gh = bf16_host(got) if out == w.OUT_BF16 else host(got)
            wh = bf16_host(want) if out == w.OUT_BF16 else host(want)
            assert np.array_equal(gh, wh), f"call {i} out {out}: {int((gh != wh).sum())} differ"


def test_grouped_gemm_noalloc_rejects_too_many_experts(w):
    R, K, N, E = 4, 64, 16, 1025
    a = torch.zeros((R, K), dtype=torch.int8, device="cuda")
    g = torch.zeros((E,), dtype=torch.int64, device="cuda")
    g[0] = R
    wp = torch.zeros((w.packed_weight_bytes(E, N, K),), dtype=torch.uint8, device="cuda")
    with pytest.raises(w.W8A8Error) as e:
        w.grouped_gemm_noalloc(a, torch.ones(R, device="cuda"), g, wp,
                               torch.ones((E, N), device="cuda"), N,
                               torch.empty((R, N), dtype=torch.bfloat16, device="cuda"))
    assert e.value.status == 4  # W8A8_ERR_UNSUPPORTED, before any launch
