"""The C-ABI library loads and validates on the host (CPU only, no GPU calls).

Every call here fails argument validation before anything is launched, or is a
pure size query, so nothing touches a device.
"""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w8a8.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(w8a8_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def w():
    import moe_token_amax_amd as w
    return w


def test_exports_every_declared_symbol(w):
    names = _declared()
    assert len(names) >= 13
    raw = ctypes.CDLL(w.LIB_PATH)
    missing = [n for n in names if not hasattr(raw, n)]
    assert not missing, missing


def test_abi_and_status_strings(w):
    assert w.lib.w8a8_abi_version() == 1
    assert w.lib.w8a8_status_str(0) == b"ok"
    assert w.lib.w8a8_status_str(5) == b"workspace too small"


def test_packed_bytes_formula(w):
    # K padded to 64, N padded to 16
    assert w.packed_weight_bytes(1, 128, 256) == 128 * 256
    assert w.packed_weight_bytes(2, 17, 65) == 2 * 32 * 128
    assert w.packed_weight_bytes(256, 4096, 4096) == 256 * 4096 * 4096


def test_validation_before_launch(w):
    L = w.lib
    p = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    assert L.w8a8_dynamic_quant(p, 4, 0, p, p, None) == 2
    assert L.w8a8_dynamic_quant(None, 4, 8, None, None, None) == 1
    assert b"null" in L.w8a8_last_error()
    assert L.w8a8_dynamic_quant(None, 0, 8, None, None, None) == 0  # M == 0 is a no-op
    assert L.w8a8_linear(p, p, 4, 200000, p, p, 8, None, p, 0, None, 0, None) == 2
    assert L.w8a8_linear(p, p, 4, 64, p, p, 8, None, p, 7, None, 0, None) == 4
    assert L.w8a8_linear(p, p, 4, 64, ctypes.c_void_p(24), p, 8, None, p, 0, None, 0, None) == 3
    # the workspace serves the BF16-input branch: codes (M to 16, K to 64) + scales
    assert L.w8a8_linear_workspace_bytes(4, 4096, 7168) == 16 * 7168 + 256
    assert L.w8a8_linear_workspace_bytes(8192, 4096, 7168) == 8192 * 7168 + 32768
    # BF16 input with the packed flag is not a thing
    assert L.w8a8_linear(p, None, 4, 64, p, p, 8, None, p, 4, None, 0, None) == 4
    assert L.w8a8_grouped_gemm(p, p, p, 8, 2000, 16, 16, p, p, p, 0, None, 0, None) == 4
    assert L.w8a8_swiglu_quant(p, 4, 0, p, p, None) == 2
    assert L.w8a8_moe_grouped(p, None, p, 16, 4, 64, 32, p, p, p, p, p, None, 0, None) == 5
    # packed activation codes: K % 8 != 0 is unsupported, unknown flag bits too
    assert L.w8a8_dynamic_quant_packed(p, 4, 100, p, p, None) == 4
    assert L.w8a8_dynamic_quant_packed(ctypes.c_void_p(24), 4, 64, p, p, None) == 3
    assert L.w8a8_linear(p, p, 4, 64, p, p, 8, None, p, 8, None, 0, None) == 4
    assert L.w8a8_linear(ctypes.c_void_p(8), p, 4, 64, p, p, 8, None, p, 4, None, 0, None) == 3


def test_strided_validation_before_launch(w):
    L = w.lib
    p = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    # row strides below the row width
    assert L.w8a8_dynamic_quant_ld(p, 4, 64, 63, p, 64, p, None) == 2
    assert L.w8a8_dynamic_quant_ld(p, 4, 64, 64, p, 10, p, None) == 2
    assert L.w8a8_dynamic_quant_ld(None, 4, 64, 80, None, 72, None, None) == 1
    assert L.w8a8_dynamic_quant_ld(None, 0, 64, 80, None, 72, None, None) == 0  # M == 0
    assert L.w8a8_dynamic_quant_ld(ctypes.c_void_p(17), 4, 64, 80, p, 72, p, None) == 3
    # linear_ld: ldq < K, ldy < N, unknown output kinds (packed codes are not strided)
    assert L.w8a8_linear_ld(p, 63, p, 4, 64, p, p, 8, None, p, 8, 0, None, 0, None) == 2
    assert L.w8a8_linear_ld(p, 64, p, 4, 64, p, p, 8, None, p, 7, 0, None, 0, None) == 2
    assert L.w8a8_linear_ld(p, 64, p, 4, 64, p, p, 8, None, p, 8, 7, None, 0, None) == 4
    assert L.w8a8_linear_ld(p, 64, p, 4, 64, p, p, 8, None, p, 8, 4, None, 0, None) == 4
    assert L.w8a8_linear_ld(p, 64, None, 4, 64, p, p, 8, None, p, 8, 0, None, 0, None) == 1
    assert L.w8a8_linear_ld(p, 64, p, 4, 64, ctypes.c_void_p(24), p, 8, None, p, 8, 0, None, 0, None) == 3
    assert L.w8a8_linear_ld(None, 64, None, 0, 64, None, None, 8, None, None, 8, 0, None, 0, None) == 0


def test_mx_validation_before_launch(w):
    L = w.lib
    p = ctypes.c_void_p(256)  # never dereferenced: validation fails first
    # K must be a multiple of the MX group size 32: UNSUPPORTED, nothing launched
    assert L.w8a8_mx_quant(p, 4, 48, p, p, 0, None) == 4
    assert L.w8a8_mx_quant(p, 4, 48, p, p, 0, None) == 4 and b"32" in L.w8a8_last_error()
    assert L.w8a8_mx_prepack_weight(p, p, 16, 100, p, None) == 4
    assert L.w8a8_mx_linear(p, None, 4, 100, p, 16, p, 0, p, 1 << 20, None) == 4
    assert L.w8a8_mx_quant(p, 4, 16, p, p, 0, None) == 2          # K < 32
    assert L.w8a8_mx_quant(p, 4, 64, p, p, 2, None) == 4          # unknown scale rule
    assert L.w8a8_mx_quant(None, 0, 64, None, None, 0, None) == 0  # M == 0 is a no-op
    assert L.w8a8_mx_quant(None, 4, 64, None, None, 0, None) == 1
    assert L.w8a8_mx_linear(p, None, 4, 64, p, 16, p, 0, None, 0, None) == 5
    assert L.w8a8_mx_linear(p, None, 4, 64, ctypes.c_void_p(272), 16, p, 0, p, 1 << 20, None) == 3
    assert L.w8a8_mx_resolve_block_fp8(p, p, 0, 64, 128, 128, p, None) == 2


def test_mx_sizes(w):
    # payload: N padded to 16, K to 64; scales: ceil(K/64) k-blocks x padded N x 2
    assert w.mx_packed_bytes(5120, 17408) == 5120 * 17408 + 272 * 5120 * 2
    assert w.mx_packed_bytes(17, 96) == 32 * 128 + 256
    # activation blocks: M padded to 16, K to 64; scales: k-blocks x M padded to even x 2
    assert w.mx_linear_workspace_bytes(2048, 17408) == 2048 * 17408 + 272 * 2048 * 2
    assert w.mx_linear_workspace_bytes(3, 32) == 16 * 64 + 256
    assert w.mx_linear_workspace_bytes(257, 4096) == 272 * 4096 + 64 * 258 * 2


def test_static_validation_before_launch(w):
    L = w.lib
    p = ctypes.c_void_p(256)  # never dereferenced: validation fails first
    nan, inf = float("nan"), float("inf")
    # input_scale must be > 0 and finite, the offset finite
    assert L.w8a8_static_quant(p, 4, 64, 0.0, 0.0, p, None) == 2
    assert L.w8a8_static_quant(p, 4, 64, -1.0, 0.0, p, None) == 2
    assert L.w8a8_static_quant(p, 4, 64, inf, 0.0, p, None) == 2
    assert L.w8a8_static_quant(p, 4, 64, 0.5, nan, p, None) == 2
    assert L.w8a8_static_quant(p, 4, 0, 0.5, 0.0, p, None) == 2           # K < 1
    assert L.w8a8_static_quant(None, 0, 64, 0.5, 0.0, None, None) == 0     # M == 0 is a no-op
    assert L.w8a8_static_quant(None, 4, 64, 0.5, 0.0, None, None) == 1
    assert L.w8a8_static_quant(ctypes.c_void_p(257), 4, 64, 0.5, 0.0, p, None) == 3
    assert L.w8a8_static_prepare(p, 16, 200000, p, None, 0.5, 1.0, p, p, None) == 2
    assert L.w8a8_static_prepare(p, 16, 64, p, None, 0.0, 1.0, p, p, None) == 2
    assert L.w8a8_static_prepare(p, 16, 64, None, None, 0.5, 1.0, p, p, None) == 1
    assert L.w8a8_static_prepare(p, 16, 64, p, ctypes.c_void_p(257), 0.5, 1.0, p, p, None) == 3
    assert L.w8a8_static_linear(p, 4, 64, p, p, p, 16, p, 7, None) == 4     # unknown output kind
    assert L.w8a8_static_linear(p, 4, 64, p, p, None, 16, p, 0, None) == 1
    assert L.w8a8_static_linear(p, 4, 64, ctypes.c_void_p(264), p, p, 16, p, 0, None) == 3
    assert L.w8a8_static_linear(None, 0, 64, None, None, None, 16, None, 0, None) == 0
    assert L.w8a8_static_quant_packed(p, 4, 64, 0.5, 0.0, ctypes.c_void_p(264), None) == 3
    assert L.w8a8_static_quant_packed(None, 4, 64, 0.5, 0.0, None, None) == 1
    assert L.w8a8_static_quant_packed(p, 4, 64, 0.0, 0.0, p, None) == 2
    assert L.w8a8_static_linear(ctypes.c_void_p(8), 4, 64, p, p, p, 16, p, 4, None) == 3  # packed q
    assert L.w8a8_static_linear(p, 4, 64, p, p, p, 16, p, 8, None) == 4   # unknown flag bit


def test_moe_io_validation_before_launch(w):
    L = w.lib
    p = ctypes.c_void_p(256)  # never dereferenced: validation fails first
    # route: E in [1, 1024], top_k >= 1, T * top_k < 2^31
    assert L.w8a8_moe_route(p, 4, 2, 0, p, p, p, None) == 2
    assert L.w8a8_moe_route(p, 4, 0, 8, p, p, p, None) == 2
    assert L.w8a8_moe_route(p, 1 << 28, 8, 8, p, p, p, None) == 2
    assert L.w8a8_moe_route(p, 4, 2, 1025, p, p, p, None) == 4
    assert L.w8a8_moe_route(p, 4, 2, 8, None, p, p, None) == 1
    assert L.w8a8_moe_route(p, 4, 2, 8, p, None, p, None) == 1
    assert L.w8a8_moe_route(p, 4, 2, 8, ctypes.c_void_p(260), p, p, None) == 3  # group_list 8-byte
    assert L.w8a8_moe_route(p, 4, 2, 8, p, p, ctypes.c_void_p(258), None) == 3
    # gather
    assert L.w8a8_moe_gather(p, p, 4, 0, p, 8, p, p, None) == 2
    assert L.w8a8_moe_gather(p, p, 4, 64, p, -1, p, p, None) == 2
    assert L.w8a8_moe_gather(None, None, 4, 64, None, 0, None, None, None) == 0   # R == 0
    assert L.w8a8_moe_gather(p, p, 4, 64, p, 8, None, p, None) == 1
    assert L.w8a8_moe_gather(p, ctypes.c_void_p(258), 4, 64, p, 8, p, p, None) == 3
    # combine
    assert L.w8a8_moe_combine(p, 8, 0, p, p, 4, 2, p, None) == 2
    assert L.w8a8_moe_combine(p, 8, 64, p, p, 4, 0, p, None) == 2
    assert L.w8a8_moe_combine(None, 8, 64, None, None, 0, 2, None, None) == 0     # T == 0
    assert L.w8a8_moe_combine(p, 8, 64, p, None, 4, 2, p, None) == 1
    assert L.w8a8_moe_combine(ctypes.c_void_p(257), 8, 64, p, p, 4, 2, p, None) == 3
    # whole layer
    assert L.w8a8_moe_layer_workspace_bytes(0, 8, 256, 4096, 2048) == 0
    need = L.w8a8_moe_layer_workspace_bytes(64, 8, 16, 256, 128)
    assert need >= 64 * 256 + 64 * 8 * (256 + 2 * 256)
    assert L.w8a8_moe_layer(p, 64, 256, p, p, 8, 16, 128, p, p, p, p, p, p, need - 1, None) == 5
    assert L.w8a8_moe_layer(p, 64, 256, p, p, 8, 16, 128, p, p, p, p, p, None, need, None) == 5
    assert L.w8a8_moe_layer(p, 64, 256, p, p, 8, 2000, 128, p, p, p, p, p, p, need, None) == 4
    assert L.w8a8_moe_layer(p, 64, 256, p, None, 8, 16, 128, p, p, p, p, p, p, need, None) == 1
    assert L.w8a8_moe_layer(p, 64, 256, p, p, 8, 16, 128, ctypes.c_void_p(264), p, p, p, p, p,
                            need, None) == 3
    assert L.w8a8_moe_layer(None, 0, 256, None, None, 8, 16, 128, None, None, None, None, None,
                            None, 0, None) == 0


def test_mx_moe_validation_before_launch(w):
    L = w.lib
    p = ctypes.c_void_p(256)  # never dereferenced: validation fails first
    ws = L.w8a8_mx_grouped_workspace_bytes(100, 4, 128)
    # grouped: K % 32, E in [1, 1024], act, scale_alg, workspace, alignment
    assert L.w8a8_mx_grouped_gemm(p, p, 100, 4, 64, 100, 0, p, 0, p, p, ws, None) == 4    # K % 32
    assert L.w8a8_mx_grouped_gemm(p, p, 100, 2000, 64, 128, 0, p, 0, p, p, ws, None) == 4
    assert L.w8a8_mx_grouped_gemm(p, p, 100, 4, 64, 128, 2, p, 0, p, p, ws, None) == 4     # act
    assert L.w8a8_mx_grouped_gemm(p, p, 100, 4, 64, 128, 0, p, 3, p, p, ws, None) == 4     # scale_alg
    assert L.w8a8_mx_grouped_gemm(p, p, 100, 4, 64, 128, 0, p, 0, p, p, ws - 1, None) == 5
    assert L.w8a8_mx_grouped_gemm(p, p, 100, 4, 64, 128, 0, None, 0, p, p, ws, None) == 1
    assert L.w8a8_mx_grouped_gemm(ctypes.c_void_p(264), p, 100, 4, 64, 128, 0, p, 0, p, p, ws,
                                  None) == 3
    assert L.w8a8_mx_grouped_gemm(None, None, 0, 4, 64, 128, 0, None, 0, None, None, 0, None) == 0
    # chain
    need = L.w8a8_mx_moe_workspace_bytes(100, 4, 256, 128)
    assert need >= 100 * 2 * 128 * 2 + 100 * 256
    assert L.w8a8_mx_moe_grouped(p, p, 100, 4, 256, 128, p, p, 0, p, p, need - 1, None) == 5
    assert L.w8a8_mx_moe_grouped(p, p, 100, 4, 256, 100, p, p, 0, p, p, need, None) == 4  # I % 32
    assert L.w8a8_mx_moe_grouped(p, None, 100, 4, 256, 128, p, p, 0, p, p, need, None) == 1
    # preparation and the SwiGLU MX quant
    assert L.w8a8_mx_moe_staging_bytes(64, 96) == 64 * 96 * 2
    assert L.w8a8_mx_moe_packed_bytes(3, 64, 96) == 3 * L.w8a8_mx_packed_bytes(64, 96)
    assert L.w8a8_mx_moe_prepare(p, p, 2, 64, 96, 128, 128, 0, p, None, p, 64 * 96 * 2 - 1,
                                 None) == 5
    assert L.w8a8_mx_moe_prepare(p, p, 2, 64, 100, 128, 128, 0, p, None, p, 1 << 20, None) == 4
    assert L.w8a8_mx_moe_prepare(p, p, 2, 64, 96, 128, 128, 0, None, None, p, 1 << 20, None) == 1
    assert L.w8a8_mx_moe_prepare(p, p, 2, 64, 96, 128, 128, 0, p, ctypes.c_void_p(384), p,
                                 1 << 20, None) == 3
    assert L.w8a8_mx_swiglu_quant(p, 4, 48, 0, p, p, None) == 4                            # I % 32
    assert L.w8a8_mx_swiglu_quant(ctypes.c_void_p(264), 4, 64, 0, p, p, None) == 3
    assert L.w8a8_mx_swiglu_quant(None, 0, 64, 0, None, None, None) == 0


def test_w4a16_validation_before_launch(w):
    L = w.lib
    p = ctypes.c_void_p(256)  # never dereferenced: validation fails first
    # 1152 bytes per 16 columns and 128-deep chunk; K padded to 128, N to 16
    assert L.w8a8_w4a16_packed_bytes(4096, 7168) == 256 * 56 * 1152
    assert L.w8a8_w4a16_packed_bytes(17, 160) == 2 * 2 * 1152
    assert L.w8a8_fp4_packed_bytes(4096, 7168) == 256 * 56 * 1088
    assert L.w8a8_fp4_packed_bytes(17, 160) == 2 * 2 * 1088
    assert L.w8a8_fp4_packed_bytes(0, 160) == 0
    assert L.w8a8_w4a16_quant_weight(p, 16, 100, p, p, p, None) == 4          # K % 32
    assert L.w8a8_w4a16_quant_weight(p, 0, 64, p, p, p, None) == 2
    assert L.w8a8_w4a16_quant_weight(p, 16, 64, None, None, None, None) == 1   # no output
    assert L.w8a8_w4a16_quant_weight(p, 16, 64, None, None, ctypes.c_void_p(264), None) == 3
    assert L.w8a8_w4a16_pack(p, None, 16, 64, p, None) == 1
    assert L.w8a8_w4a16_pack(p, p, 16, 48, p, None) == 4
    assert L.w8a8_w4a16_linear(ctypes.c_void_p(264), 4, 64, p, 16, p, None, 0, None) == 3
    assert L.w8a8_w4a16_linear(p, 4, 64, None, 16, p, None, 0, None) == 1
    assert L.w8a8_w4a16_linear(None, 0, 64, None, 16, None, None, 0, None) == 0   # M == 0
    assert L.w8a8_w4a16_linear(p, -1, 64, p, 16, p, None, 0, None) == 2
    # rows past one launch's 16-row groups along the grid's y (16 * 65535)
    assert L.w8a8_w4a16_linear(p, 16 * 65535 + 1, 64, p, 16, p, p, 1 << 40, None) == 2
    assert L.w8a8_fp4_linear(p, 16 * 65535 + 1, 64, p, 16, p, p, 1 << 40, None) == 2
    # no workspace for any M (the rows are staged in LDS)
    assert L.w8a8_w4a16_linear_workspace_bytes(16, 7168) == 0
    assert L.w8a8_w4a16_linear_workspace_bytes(64, 7168) == 0


def test_fp4_validation_before_launch(w):
    L = w.lib
    p = ctypes.c_void_p(256)  # never dereferenced: validation fails first
    assert L.w8a8_fp4_quant_weight(p, 16, 100, p, p, p, None) == 4          # K % 32
    assert L.w8a8_fp4_quant_weight(p, 16, 64, None, None, None, None) == 1  # no output
    assert L.w8a8_fp4_quant_weight(p, 16, 64, None, None, ctypes.c_void_p(264), None) == 3
    assert L.w8a8_fp4_linear(p, 4, 48, p, 16, p, None, 0, None) == 4
    assert L.w8a8_fp4_linear(ctypes.c_void_p(264), 4, 64, p, 16, p, None, 0, None) == 3
    assert L.w8a8_fp4_linear(None, 0, 64, None, 16, None, None, 0, None) == 0
    assert L.w8a8_fp4_linear(p, 17, 64, p, 16, ctypes.c_void_p(257), None, 0, None) == 3  # y


def test_lowbit_grouped_validation_before_launch(w):
    L = w.lib
    p = ctypes.c_void_p(256)  # never dereferenced: validation fails first
    g = L.w8a8_w4a16_grouped_gemm
    assert g(2, p, p, 64, 4, 32, 64, p, p, None) == 4            # unknown weight format
    assert g(0, p, p, 64, 4, 24, 64, p, p, None) == 4            # N % 16
    assert g(1, p, p, 64, 4, 32, 48, p, p, None) == 4            # K % 32
    assert g(0, p, p, 64, 1025, 32, 64, p, p, None) == 4         # more than 1024 experts
    assert g(0, p, p, 64, 0, 32, 64, p, p, None) == 2            # no expert
    assert g(0, p, p, -1, 4, 32, 64, p, p, None) == 2
    assert g(0, None, None, 0, 4, 32, 64, None, None, None) == 0  # R == 0: nothing to do
    assert g(0, None, p, 64, 4, 32, 64, p, p, None) == 1
    assert g(0, ctypes.c_void_p(264), p, 64, 4, 32, 64, p, p, None) == 3   # x 16-byte aligned
    assert g(1, p, p, 64, 4, 32, 64, p, ctypes.c_void_p(260), None) == 3   # y 8-byte aligned
    s = L.w8a8_w4a16_swiglu
    assert s(p, -1, 64, p, None) == 2
    assert s(p, 4, 0, p, None) == 2
    assert s(None, 0, 64, None, None) == 0
    assert s(p, 4, 64, None, None) == 1
    # workspace: h BF16 [R, 2I], then a BF16 [R, I], each 256-byte aligned
    assert L.w8a8_w4a16_moe_workspace_bytes(16384, 4096, 2048) == 16384 * 4096 * 2 + 16384 * 2048 * 2
    assert L.w8a8_w4a16_moe_workspace_bytes(3, 64, 32) == 512 + 256
    assert L.w8a8_w4a16_moe_workspace_bytes(0, 64, 32) == 0
    m = L.w8a8_w4a16_moe_grouped
    need = L.w8a8_w4a16_moe_workspace_bytes(64, 64, 32)
    assert m(0, p, p, 64, 4, 64, 48, p, p, p, p, 1 << 30, None) == 4          # I % 32
    assert m(0, p, p, 64, 4, 48, 32, p, p, p, p, 1 << 30, None) == 4          # H % 32
    assert m(0, p, p, 64, 4, 64, 32, p, p, p, None, 0, None) == 5
    assert m(0, p, p, 64, 4, 64, 32, p, p, p, p, need - 1, None) == 5
    assert m(0, p, p, 64, 4, 64, 32, p, p, p, ctypes.c_void_p(272), need, None) == 5
    assert m(0, p, p, 64, 4, 64, 32, None, p, p, p, need, None) == 1
    assert m(1, None, None, 0, 4, 64, 32, None, None, None, None, 0, None) == 0
