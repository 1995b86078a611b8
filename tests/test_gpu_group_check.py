"""W8A8_CHECK: host validation of group_list in every grouped call (GPU).

With W8A8_CHECK=1 in the environment each call that takes a group_list copies
it to the host first and refuses a negative count or counts summing past R
with W8A8_ERR_SHAPE, launching nothing: the output buffer keeps its sentinel.
A valid list gives the same bits as without the check. Invalid lists are only
ever passed with the check on, so no kernel sees them here."""

from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import synth
from tests.conftest import gpu_available
from tests.gpu_util import dev, show, sync

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

E, N, K, H, I = 4, 64, 128, 128, 64


@pytest.fixture(scope="module")
def w():
    import moe_token_amax_amd as w
    return w


@pytest.fixture
def checked():
    old = os.environ.get("W8A8_CHECK")
    os.environ["W8A8_CHECK"] = "1"
    yield
    if old is None:
        del os.environ["W8A8_CHECK"]
    else:
        os.environ["W8A8_CHECK"] = old


def _int8_case(R, seed=0):
    rng = np.random.default_rng(seed)
    a = dev(rng.integers(-127, 128, (R, K), dtype=np.int8))
    s = dev((rng.random(R, dtype=np.float32) * 0.01 + 1e-3).astype(np.float32))
    wt = synth.int8_weight((E, N, K), seed)
    ws = dev(synth.scales(E * N, seed).reshape(E, N))
    return a, s, dev(wt), ws


BAD_LISTS = [([3, -1, 4, 2], "negative"), ([5, 5, 5, 5], "pass R")]


@pytest.mark.parametrize("counts,msg", BAD_LISTS)
def test_grouped_gemm_rejects(w, checked, counts, msg):
    R = 8
    show(f"W8A8_CHECK grouped_gemm counts={counts}")
    a, s, wt, ws = _int8_case(R)
    wp = w.prepack_weight(wt)
    y = torch.full((R, N), 7, dtype=torch.int32, device="cuda")
    with pytest.raises(w.W8A8Error) as ei:
        w.grouped_gemm(a, s, dev(np.array(counts, np.int64)), wp, ws, N, out=w.OUT_I32, y=y)
    assert ei.value.status == 2 and msg in str(ei.value)
    with pytest.raises(w.W8A8Error) as ei:
        w.grouped_gemm_noalloc(a, s, dev(np.array(counts, np.int64)), wp, ws, N, y, out=w.OUT_I32)
    assert ei.value.status == 2 and msg in str(ei.value)
    sync()
    assert (y.cpu().numpy() == 7).all(), "a refused call wrote its output"


@pytest.mark.parametrize("counts", [[3, 0, 4, 1], [2, 0, 1, 1]])
def test_grouped_gemm_valid_list_same_bits(w, counts):
    """Counts summing to R, and to less than R (rows past the sum untouched)."""
    R = 8
    show(f"W8A8_CHECK grouped_gemm valid counts={counts}")
    a, s, wt, ws = _int8_case(R, seed=3)
    wp = w.prepack_weight(wt)
    gl = dev(np.array(counts, np.int64))
    y0 = torch.full((R, N), 7, dtype=torch.int32, device="cuda")
    w.grouped_gemm(a, s, gl, wp, ws, N, out=w.OUT_I32, y=y0)
    os.environ["W8A8_CHECK"] = "1"
    try:
        y1 = torch.full((R, N), 7, dtype=torch.int32, device="cuda")
        w.grouped_gemm(a, s, gl, wp, ws, N, out=w.OUT_I32, y=y1)
        y2 = torch.full((R, N), 7, dtype=torch.int32, device="cuda")
        w.grouped_gemm_noalloc(a, s, gl, wp, ws, N, y2, out=w.OUT_I32)
    finally:
        del os.environ["W8A8_CHECK"]
    sync()
    assert torch.equal(y0, y1) and torch.equal(y0, y2)
    assert (y0[sum(counts):].cpu().numpy() == 7).all()


@pytest.mark.parametrize("counts,msg", BAD_LISTS)
def test_chains_reject(w, checked, counts, msg):
    R = 8
    show(f"W8A8_CHECK chains counts={counts}")
    gl = dev(np.array(counts, np.int64))
    x = torch.zeros((R, H), dtype=torch.bfloat16, device="cuda")
    sentinel = torch.full((R, H), -1, dtype=torch.int16, device="cuda")
    # INT8 chain: weights never read (the call is refused before any launch)
    w13 = torch.zeros((w.packed_weight_bytes(E, 2 * I, H),), dtype=torch.uint8, device="cuda")
    w2 = torch.zeros((w.packed_weight_bytes(E, H, I),), dtype=torch.uint8, device="cuda")
    y = sentinel.clone().view(torch.bfloat16)
    with pytest.raises(w.W8A8Error) as ei:
        w.moe_grouped(x, gl, w13, torch.ones((E, 2 * I), device="cuda"), w2,
                      torch.ones((E, H), device="cuda"), y=y)
    assert ei.value.status == 2 and msg in str(ei.value)
    # MXFP8 grouped matmul (N = K = H) and chain
    m13 = torch.zeros((w.mx_moe_packed_bytes(E, 2 * I, H),), dtype=torch.uint8, device="cuda")
    m2 = torch.zeros((w.mx_moe_packed_bytes(E, H, I),), dtype=torch.uint8, device="cuda")
    mhh = torch.zeros((w.mx_moe_packed_bytes(E, H, H),), dtype=torch.uint8, device="cuda")
    with pytest.raises(w.W8A8Error) as ei:
        w.mx_grouped_gemm(x, gl, mhh, H, y=y)
    assert ei.value.status == 2 and msg in str(ei.value)
    with pytest.raises(w.W8A8Error) as ei:
        w.mx_moe_grouped(x, gl, m13, m2, I, y=y)
    assert ei.value.status == 2 and msg in str(ei.value)
    # low-bit grouped matmul and chain, both formats
    for fmt in (w.LOWBIT_INT4, w.LOWBIT_FP4):
        l13 = torch.zeros((E * w._lowbit_bytes(fmt, 2 * I, H),), dtype=torch.uint8, device="cuda")
        l2 = torch.zeros((E * w._lowbit_bytes(fmt, H, I),), dtype=torch.uint8, device="cuda")
        lhh = torch.zeros((E * w._lowbit_bytes(fmt, H, H),), dtype=torch.uint8, device="cuda")
        with pytest.raises(w.W8A8Error) as ei:
            w.w4a16_grouped_gemm(x, gl, lhh, H, fmt=fmt, y=y)
        assert ei.value.status == 2 and msg in str(ei.value)
        with pytest.raises(w.W8A8Error) as ei:
            w.w4a16_moe_grouped(x, gl, l13, l2, I, fmt=fmt, y=y)
        assert ei.value.status == 2 and msg in str(ei.value)
    sync()
    assert torch.equal(y.view(torch.int16), sentinel), "a refused call wrote its output"


def test_check_off_by_zero(w):
    """W8A8_CHECK=0 is off: a valid call then needs no host copy (it is
    captured in a HIP graph, where a synchronizing copy would fail)."""
    R = 8
    a, s, wt, ws = _int8_case(R, seed=5)
    wp = w.prepack_weight(wt)
    gl = dev(np.array([3, 0, 4, 1], np.int64))
    y = torch.empty((R, N), dtype=torch.int32, device="cuda")
    ref = w.grouped_gemm(a, s, gl, wp, ws, N, out=w.OUT_I32)
    os.environ["W8A8_CHECK"] = "0"
    try:
        ws_buf = torch.empty((w.lib.w8a8_grouped_workspace_bytes(R, E, N, K),), dtype=torch.uint8,
                             device="cuda")
        g = torch.cuda.CUDAGraph()
        stream = torch.cuda.Stream()
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(g, stream=stream):
                w.grouped_gemm(a, s, gl, wp, ws, N, out=w.OUT_I32, y=y, workspace=ws_buf)
        for _ in range(3):
            y.zero_()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(y, ref)
    finally:
        del os.environ["W8A8_CHECK"]
