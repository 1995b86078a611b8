"""Python binding of libw8a8.so, the gfx950 W8A8_DYNAMIC library.

Argument marshalling only: every function checks dtype, device and layout of the
torch tensors it is given, passes their device pointers and the current HIP
stream to the C ABI (include/w8a8.h), and raises ``RuntimeError`` with the
library's message on a non-zero status. Every step of the path runs in the HIP
kernels; there is no CPU or PyTorch fallback. Importing this package fails when
the built library is missing.
"""

from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "LIB_PATH",
    "lib",
    "W8A8Error",
    "OUT_BF16",
    "OUT_I32",
    "A_PACKED",
    "dynamic_quant",
    "dynamic_quant_packed",
    "packed_weight_bytes",
    "prepack_weight",
    "linear_workspace_bytes",
    "linear",
    "linear_packed",
    "linear_bf16",
    "grouped_gemm",
    "grouped_gemm_noalloc",
    "swiglu_quant",
    "moe_workspace_bytes",
    "moe_grouped",
    "moe_route",
    "moe_gather",
    "moe_combine",
    "moe_layer_workspace_bytes",
    "moe_layer",
    "mx_quant",
    "mx_resolve_block_fp8",
    "mx_packed_bytes",
    "mx_prepack_weight",
    "mx_linear_workspace_bytes",
    "mx_linear",
    "mx_gemm",
    "ACT_NONE",
    "ACT_SWIGLU",
    "mx_moe_staging_bytes",
    "mx_moe_packed_bytes",
    "mx_moe_prepare",
    "mx_swiglu_quant",
    "mx_grouped_workspace_bytes",
    "mx_grouped_gemm",
    "mx_moe_workspace_bytes",
    "mx_moe_grouped",
    "w4a16_packed_bytes",
    "fp4_packed_bytes",
    "w4a16_quant_weight",
    "w4a16_pack",
    "w4a16_linear_workspace_bytes",
    "w4a16_linear",
    "fp4_quant_weight",
    "fp4_linear",
    "LOWBIT_INT4",
    "LOWBIT_FP4",
    "w4a16_grouped_gemm",
    "w4a16_swiglu",
    "w4a16_moe_workspace_bytes",
    "w4a16_moe_grouped",
    "mx_workspace_operands",
    "static_quant",
    "static_quant_packed",
    "static_prepare",
    "static_linear",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libw8a8.so")

OUT_BF16 = 0
OUT_I32 = 1
A_PACKED = 4   # flag for linear's `out`: q in the packed block layout

_c_i64 = ctypes.c_int64
_c_p = ctypes.c_void_p


class W8A8Error(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"w8a8 status {status}: {msg}")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
            "or `python moe_token_amax_amd/_build.py` first")
    L = ctypes.CDLL(LIB_PATH)
    sig = {
        "w8a8_status_str": (ctypes.c_char_p, [ctypes.c_int]),
        "w8a8_last_error": (ctypes.c_char_p, []),
        "w8a8_abi_version": (ctypes.c_int, []),
        "w8a8_dynamic_quant": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_p, _c_p, _c_p]),
        "w8a8_dynamic_quant_packed": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_p, _c_p, _c_p]),
        "w8a8_dynamic_quant_ld": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_i64, _c_p, _c_p]),
        "w8a8_linear_ld": (ctypes.c_int, [_c_p, _c_i64, _c_p, _c_i64, _c_i64, _c_p, _c_p, _c_i64, _c_p, _c_p,
                                          _c_i64, ctypes.c_int, _c_p, _c_i64, _c_p]),
        "w8a8_packed_weight_bytes": (_c_i64, [_c_i64, _c_i64, _c_i64]),
        "w8a8_prepack_weight": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_p]),
        "w8a8_linear_workspace_bytes": (_c_i64, [_c_i64, _c_i64, _c_i64]),
        "w8a8_linear": (ctypes.c_int, [_c_p, _c_p, _c_i64, _c_i64, _c_p, _c_p, _c_i64, _c_p, _c_p,
                                       ctypes.c_int, _c_p, _c_i64, _c_p]),
        "w8a8_grouped_workspace_bytes": (_c_i64, [_c_i64, _c_i64, _c_i64, _c_i64]),
        "w8a8_grouped_gemm": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_i64,
                                             _c_p, _c_p, _c_p, ctypes.c_int, _c_p, _c_i64, _c_p]),
        "w8a8_grouped_gemm_noalloc": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64,
                                                     _c_i64, _c_p, _c_p, _c_p, ctypes.c_int, _c_p]),
        "w8a8_swiglu_quant": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_p, _c_p, _c_p]),
        "w8a8_moe_workspace_bytes": (_c_i64, [_c_i64, _c_i64, _c_i64, _c_i64]),
        "w8a8_moe_grouped": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_i64,
                                            _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_p]),
        "w8a8_moe_route": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p]),
        "w8a8_moe_gather": (ctypes.c_int, [_c_p, _c_p, _c_i64, _c_i64, _c_p, _c_i64, _c_p, _c_p,
                                           _c_p]),
        "w8a8_moe_combine": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_p, _c_p, _c_i64, _c_i64, _c_p,
                                            _c_p]),
        "w8a8_moe_layer_workspace_bytes": (_c_i64, [_c_i64, _c_i64, _c_i64, _c_i64, _c_i64]),
        "w8a8_moe_layer": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_p, _c_p, _c_i64, _c_i64, _c_i64,
                                          _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_p]),
        "w8a8_mx_quant": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_p, _c_p, ctypes.c_int, _c_p]),
        "w8a8_mx_resolve_block_fp8": (ctypes.c_int, [_c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_i64,
                                                     _c_p, _c_p]),
        "w8a8_mx_packed_bytes": (_c_i64, [_c_i64, _c_i64]),
        "w8a8_mx_prepack_weight": (ctypes.c_int, [_c_p, _c_p, _c_i64, _c_i64, _c_p, _c_p]),
        "w8a8_mx_linear_workspace_bytes": (_c_i64, [_c_i64, _c_i64]),
        "w8a8_mx_linear": (ctypes.c_int, [_c_p, _c_p, _c_i64, _c_i64, _c_p, _c_i64, _c_p,
                                          ctypes.c_int, _c_p, _c_i64, _c_p]),
        "w8a8_mx_gemm": (ctypes.c_int, [_c_p, _c_p, _c_i64, _c_i64, _c_p, _c_i64, _c_p, _c_p]),
        "w8a8_mx_moe_staging_bytes": (_c_i64, [_c_i64, _c_i64]),
        "w8a8_mx_moe_packed_bytes": (_c_i64, [_c_i64, _c_i64, _c_i64]),
        "w8a8_mx_moe_prepare": (ctypes.c_int, [_c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64,
                                               ctypes.c_int, _c_p, _c_p, _c_p, _c_i64, _c_p]),
        "w8a8_mx_swiglu_quant": (ctypes.c_int, [_c_p, _c_i64, _c_i64, ctypes.c_int, _c_p, _c_p,
                                                _c_p]),
        "w8a8_mx_grouped_workspace_bytes": (_c_i64, [_c_i64, _c_i64, _c_i64]),
        "w8a8_mx_grouped_gemm": (ctypes.c_int, [_c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_i64,
                                                ctypes.c_int, _c_p, ctypes.c_int, _c_p, _c_p,
                                                _c_i64, _c_p]),
        "w8a8_mx_moe_workspace_bytes": (_c_i64, [_c_i64, _c_i64, _c_i64, _c_i64]),
        "w8a8_mx_moe_grouped": (ctypes.c_int, [_c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_i64, _c_p,
                                               _c_p, ctypes.c_int, _c_p, _c_p, _c_i64, _c_p]),
        "w8a8_w4a16_packed_bytes": (_c_i64, [_c_i64, _c_i64]),
        "w8a8_fp4_packed_bytes": (_c_i64, [_c_i64, _c_i64]),
        "w8a8_w4a16_quant_weight": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p]),
        "w8a8_w4a16_pack": (ctypes.c_int, [_c_p, _c_p, _c_i64, _c_i64, _c_p, _c_p]),
        "w8a8_w4a16_linear_workspace_bytes": (_c_i64, [_c_i64, _c_i64]),
        "w8a8_w4a16_linear": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_p, _c_i64, _c_p, _c_p, _c_i64,
                                             _c_p]),
        "w8a8_fp4_quant_weight": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p]),
        "w8a8_fp4_linear": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_p, _c_i64, _c_p, _c_p, _c_i64,
                                           _c_p]),
        "w8a8_w4a16_grouped_gemm": (ctypes.c_int, [ctypes.c_int, _c_p, _c_p, _c_i64, _c_i64, _c_i64,
                                                   _c_i64, _c_p, _c_p, _c_p]),
        "w8a8_w4a16_swiglu": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_p, _c_p]),
        "w8a8_w4a16_moe_workspace_bytes": (_c_i64, [_c_i64, _c_i64, _c_i64]),
        "w8a8_w4a16_moe_grouped": (ctypes.c_int, [ctypes.c_int, _c_p, _c_p, _c_i64, _c_i64, _c_i64,
                                                  _c_i64, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_p]),
        "w8a8_static_quant": (ctypes.c_int, [_c_p, _c_i64, _c_i64, ctypes.c_float, ctypes.c_float,
                                             _c_p, _c_p]),
        "w8a8_static_quant_packed": (ctypes.c_int, [_c_p, _c_i64, _c_i64, ctypes.c_float,
                                                    ctypes.c_float, _c_p, _c_p]),
        "w8a8_static_prepare": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_p, _c_p, ctypes.c_float,
                                               ctypes.c_float, _c_p, _c_p, _c_p]),
        "w8a8_static_linear": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_i64, _c_p,
                                              ctypes.c_int, _c_p]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    return L


lib = _load()


def _check(status: int):
    if status != 0:
        raise W8A8Error(status, lib.w8a8_last_error().decode())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _rows(t: torch.Tensor, dtype, name: str) -> int:
    """A 2-D tensor whose rows are contiguous (a row stride of at least its
    width, e.g. a column slice of a wider matrix); returns the row stride."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device")
    if t.dim() != 2:
        raise ValueError(f"{name} must have 2 dims, got {t.dim()}")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name}: the elements of a row must be contiguous")
    ld = t.stride(0) if t.shape[0] > 1 else t.shape[1]
    if ld < t.shape[1]:
        raise ValueError(f"{name}: row stride below the row width")
    return int(ld)


def _need(t: torch.Tensor, dtype, name: str, ndim: int | None = None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")


def dynamic_quant(x: torch.Tensor, q: torch.Tensor | None = None,
                  scale: torch.Tensor | None = None):
    """BF16 [M, K] -> (int8 [M, K], float32 [M]). x and q may be row-strided
    (rows contiguous, e.g. column slices of wider matrices)."""
    ldx = _rows(x, torch.bfloat16, "x")
    M, K = x.shape
    if q is None:
        q = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if scale is None:
        scale = torch.empty((M,), dtype=torch.float32, device=x.device)
    ldq = _rows(q, torch.int8, "q")
    _need(scale, torch.float32, "scale", 1)
    if tuple(q.shape) != (M, K) or scale.shape[0] != M:
        raise ValueError("q / scale shape mismatch")
    if ldx == K and ldq == K:
        _check(lib.w8a8_dynamic_quant(_ptr(x), M, K, _ptr(q), _ptr(scale), _stream()))
    else:
        _check(lib.w8a8_dynamic_quant_ld(_ptr(x), M, K, ldx, _ptr(q), ldq, _ptr(scale), _stream()))
    return q, scale


def dynamic_quant_packed(x: torch.Tensor, q: torch.Tensor | None = None,
                         scale: torch.Tensor | None = None):
    """BF16 [M, K] -> (int8 codes in 1 KB blocks [ceil(M/16)][ceil(K/64)] as a uint8
    buffer, float32 [M])."""
    _need(x, torch.bfloat16, "x", 2)
    M, K = x.shape
    nbytes = packed_weight_bytes(1, M, K)
    if q is None:
        q = torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty((M,), dtype=torch.float32, device=x.device)
    _need(q, torch.uint8, "q", 1)
    _need(scale, torch.float32, "scale", 1)
    if q.numel() < nbytes or scale.shape[0] != M:
        raise ValueError("q / scale too small")
    _check(lib.w8a8_dynamic_quant_packed(_ptr(x), M, K, _ptr(q), _ptr(scale), _stream()))
    return q, scale


def packed_weight_bytes(E: int, N: int, K: int) -> int:
    return int(lib.w8a8_packed_weight_bytes(E, N, K))


def prepack_weight(w: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """int8 [N, K] or [E, N, K] -> packed uint8 buffer (stable, caller-owned)."""
    _need(w, torch.int8, "w")
    if w.dim() == 2:
        E, (N, K) = 1, w.shape
    elif w.dim() == 3:
        E, N, K = w.shape
    else:
        raise ValueError("w must be [N, K] or [E, N, K]")
    nbytes = packed_weight_bytes(E, N, K)
    if out is None:
        out = torch.empty((nbytes,), dtype=torch.uint8, device=w.device)
    _need(out, torch.uint8, "out", 1)
    if out.numel() < nbytes:
        raise ValueError(f"out needs {nbytes} bytes")
    _check(lib.w8a8_prepack_weight(_ptr(w), E, N, K, _ptr(out), _stream()))
    return out


def linear_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib.w8a8_linear_workspace_bytes(M, N, K))


def _workspace(nbytes: int, device, ws: torch.Tensor | None):
    if nbytes <= 0:
        return ws, 0
    if ws is None:
        ws = torch.empty((nbytes,), dtype=torch.uint8, device=device)
    _need(ws, torch.uint8, "workspace", 1)
    return ws, ws.numel()


def linear(q: torch.Tensor, x_scale: torch.Tensor, w_packed: torch.Tensor, w_scale: torch.Tensor,
           N: int, bias: torch.Tensor | None = None, out: int = OUT_BF16,
           y: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """INT8 [M, K] x packed W [N, K] -> BF16 [M, N] (or int32 with out=OUT_I32).
    q and y may be row-strided (rows contiguous)."""
    ldq = _rows(q, torch.int8, "q")
    _need(x_scale, torch.float32, "x_scale", 1)
    _need(w_packed, torch.uint8, "w_packed", 1)
    _need(w_scale, torch.float32, "w_scale", 1)
    M, K = q.shape
    if x_scale.shape[0] != M or w_scale.shape[0] != N:
        raise ValueError("scale shape mismatch")
    if w_packed.numel() < packed_weight_bytes(1, N, K):
        raise ValueError("w_packed too small for [N, K]")
    if bias is not None:
        _need(bias, torch.bfloat16, "bias", 1)
        if bias.shape[0] != N:
            raise ValueError("bias shape mismatch")
    ydt = torch.bfloat16 if out == OUT_BF16 else torch.int32
    if y is None:
        y = torch.empty((M, N), dtype=ydt, device=q.device)
    ldy = _rows(y, ydt, "y")
    if tuple(y.shape) != (M, N):
        raise ValueError("y shape mismatch")
    ws, ws_n = _workspace(linear_workspace_bytes(M, N, K), q.device, workspace)
    if ldq == K and ldy == N:
        _check(lib.w8a8_linear(_ptr(q), _ptr(x_scale), M, K, _ptr(w_packed), _ptr(w_scale), N,
                               _ptr(bias), _ptr(y), out, _ptr(ws), ws_n, _stream()))
    else:
        _check(lib.w8a8_linear_ld(_ptr(q), ldq, _ptr(x_scale), M, K, _ptr(w_packed), _ptr(w_scale), N,
                                  _ptr(bias), _ptr(y), ldy, out, _ptr(ws), ws_n, _stream()))
    return y


def linear_packed(q: torch.Tensor, x_scale: torch.Tensor, K: int, w_packed: torch.Tensor,
                  w_scale: torch.Tensor, N: int, bias: torch.Tensor | None = None,
                  out: int = OUT_BF16, y: torch.Tensor | None = None,
                  workspace: torch.Tensor | None = None):
    """linear() on codes in the packed block layout of dynamic_quant_packed."""
    _need(q, torch.uint8, "q", 1)
    _need(x_scale, torch.float32, "x_scale", 1)
    _need(w_packed, torch.uint8, "w_packed", 1)
    _need(w_scale, torch.float32, "w_scale", 1)
    M = x_scale.shape[0]
    if q.numel() < packed_weight_bytes(1, M, K):
        raise ValueError("q too small for [M, K] in blocks")
    if w_scale.shape[0] != N:
        raise ValueError("scale shape mismatch")
    if w_packed.numel() < packed_weight_bytes(1, N, K):
        raise ValueError("w_packed too small for [N, K]")
    if bias is not None:
        _need(bias, torch.bfloat16, "bias", 1)
        if bias.shape[0] != N:
            raise ValueError("bias shape mismatch")
    ydt = torch.bfloat16 if out == OUT_BF16 else torch.int32
    if y is None:
        y = torch.empty((M, N), dtype=ydt, device=q.device)
    _need(y, ydt, "y", 2)
    ws, ws_n = _workspace(linear_workspace_bytes(M, N, K), q.device, workspace)
    _check(lib.w8a8_linear(_ptr(q), _ptr(x_scale), M, K, _ptr(w_packed), _ptr(w_scale), N,
                           _ptr(bias), _ptr(y), out | A_PACKED, _ptr(ws), ws_n, _stream()))
    return y


def linear_bf16(x: torch.Tensor, w_packed: torch.Tensor, w_scale: torch.Tensor, N: int,
                bias: torch.Tensor | None = None, out: int = OUT_BF16,
                y: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """BF16 [M, K] -> quant (inside) -> linear; bit-identical to dynamic_quant + linear."""
    _need(x, torch.bfloat16, "x", 2)
    _need(w_packed, torch.uint8, "w_packed", 1)
    _need(w_scale, torch.float32, "w_scale", 1)
    M, K = x.shape
    if w_scale.shape[0] != N:
        raise ValueError("scale shape mismatch")
    if w_packed.numel() < packed_weight_bytes(1, N, K):
        raise ValueError("w_packed too small for [N, K]")
    if bias is not None:
        _need(bias, torch.bfloat16, "bias", 1)
        if bias.shape[0] != N:
            raise ValueError("bias shape mismatch")
    ydt = torch.bfloat16 if out == OUT_BF16 else torch.int32
    if y is None:
        y = torch.empty((M, N), dtype=ydt, device=x.device)
    _need(y, ydt, "y", 2)
    ws, ws_n = _workspace(linear_workspace_bytes(M, N, K), x.device, workspace)
    _check(lib.w8a8_linear(_ptr(x), None, M, K, _ptr(w_packed), _ptr(w_scale), N, _ptr(bias),
                           _ptr(y), out, _ptr(ws), ws_n, _stream()))
    return y


def grouped_gemm(a: torch.Tensor, a_scale: torch.Tensor, group_list: torch.Tensor,
                 w_packed: torch.Tensor, w_scale: torch.Tensor, N: int, out: int = OUT_BF16,
                 y: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """INT8 rows [R, K] grouped by expert x packed W [E, N, K] -> [R, N]."""
    _need(a, torch.int8, "a", 2)
    _need(a_scale, torch.float32, "a_scale", 1)
    _need(group_list, torch.int64, "group_list", 1)
    _need(w_packed, torch.uint8, "w_packed", 1)
    _need(w_scale, torch.float32, "w_scale", 2)
    R, K = a.shape
    E = group_list.shape[0]
    if tuple(w_scale.shape) != (E, N) or a_scale.shape[0] != R:
        raise ValueError("scale shape mismatch")
    if w_packed.numel() < packed_weight_bytes(E, N, K):
        raise ValueError("w_packed too small for [E, N, K]")
    ydt = torch.bfloat16 if out == OUT_BF16 else torch.int32
    if y is None:
        y = torch.empty((R, N), dtype=ydt, device=a.device)
    _need(y, ydt, "y", 2)
    ws, ws_n = _workspace(int(lib.w8a8_grouped_workspace_bytes(R, E, N, K)), a.device, workspace)
    _check(lib.w8a8_grouped_gemm(_ptr(a), _ptr(a_scale), _ptr(group_list), R, E, N, K,
                                 _ptr(w_packed), _ptr(w_scale), _ptr(y), out, _ptr(ws), ws_n,
                                 _stream()))
    return y


def grouped_gemm_noalloc(a: torch.Tensor, a_scale: torch.Tensor, group_list: torch.Tensor,
                         w_packed: torch.Tensor, w_scale: torch.Tensor, N: int, y: torch.Tensor,
                         out: int = OUT_BF16):
    """grouped_gemm into a caller-given y, with the schedule in the library's own
    device array (no workspace; the call allocates nothing)."""
    _need(a, torch.int8, "a", 2)
    _need(a_scale, torch.float32, "a_scale", 1)
    _need(group_list, torch.int64, "group_list", 1)
    _need(w_packed, torch.uint8, "w_packed", 1)
    _need(w_scale, torch.float32, "w_scale", 2)
    R, K = a.shape
    E = group_list.shape[0]
    if tuple(w_scale.shape) != (E, N) or a_scale.shape[0] != R:
        raise ValueError("scale shape mismatch")
    if w_packed.numel() < packed_weight_bytes(E, N, K):
        raise ValueError("w_packed too small for [E, N, K]")
    _need(y, torch.bfloat16 if out == OUT_BF16 else torch.int32, "y", 2)
    if tuple(y.shape) != (R, N):
        raise ValueError("y must be [R, N]")
    _check(lib.w8a8_grouped_gemm_noalloc(_ptr(a), _ptr(a_scale), _ptr(group_list), R, E, N, K,
                                         _ptr(w_packed), _ptr(w_scale), _ptr(y), out, _stream()))
    return y


def swiglu_quant(h: torch.Tensor, q: torch.Tensor | None = None,
                 scale: torch.Tensor | None = None):
    """BF16 h [R, 2I] (gate | up) -> (int8 [R, I], float32 [R])."""
    _need(h, torch.bfloat16, "h", 2)
    R, I2 = h.shape
    if I2 % 2:
        raise ValueError("h must have an even number of columns (gate | up)")
    I = I2 // 2
    if q is None:
        q = torch.empty((R, I), dtype=torch.int8, device=h.device)
    if scale is None:
        scale = torch.empty((R,), dtype=torch.float32, device=h.device)
    _need(q, torch.int8, "q", 2)
    _need(scale, torch.float32, "scale", 1)
    _check(lib.w8a8_swiglu_quant(_ptr(h), R, I, _ptr(q), _ptr(scale), _stream()))
    return q, scale


def moe_workspace_bytes(R: int, E: int, H: int, I: int) -> int:
    return int(lib.w8a8_moe_workspace_bytes(R, E, H, I))


def moe_grouped(x_rows: torch.Tensor, group_list: torch.Tensor, w13_packed: torch.Tensor,
                w13_scale: torch.Tensor, w2_packed: torch.Tensor, w2_scale: torch.Tensor,
                x_scale: torch.Tensor | None = None, y: torch.Tensor | None = None,
                workspace: torch.Tensor | None = None):
    """MoE expert chain on expert-grouped rows -> BF16 [R, H].

    ``x_rows`` is BF16 [R, H] (quantized inside) or int8 [R, H] with ``x_scale``.
    """
    if x_scale is None:
        _need(x_rows, torch.bfloat16, "x_rows", 2)
    else:
        _need(x_rows, torch.int8, "x_rows", 2)
        _need(x_scale, torch.float32, "x_scale", 1)
    _need(group_list, torch.int64, "group_list", 1)
    _need(w13_scale, torch.float32, "w13_scale", 2)
    _need(w2_scale, torch.float32, "w2_scale", 2)
    _need(w13_packed, torch.uint8, "w13_packed", 1)
    _need(w2_packed, torch.uint8, "w2_packed", 1)
    R, H = x_rows.shape
    E = group_list.shape[0]
    I = w13_scale.shape[1] // 2
    if tuple(w13_scale.shape) != (E, 2 * I) or tuple(w2_scale.shape) != (E, H):
        raise ValueError("scale shape mismatch")
    if w13_packed.numel() < packed_weight_bytes(E, 2 * I, H) or \
            w2_packed.numel() < packed_weight_bytes(E, H, I):
        raise ValueError("packed weights too small")
    if y is None:
        y = torch.empty((R, H), dtype=torch.bfloat16, device=x_rows.device)
    _need(y, torch.bfloat16, "y", 2)
    ws, ws_n = _workspace(moe_workspace_bytes(R, E, H, I), x_rows.device, workspace)
    _check(lib.w8a8_moe_grouped(_ptr(x_rows), _ptr(x_scale), _ptr(group_list), R, E, H, I,
                                _ptr(w13_packed), _ptr(w13_scale), _ptr(w2_packed),
                                _ptr(w2_scale), _ptr(y), _ptr(ws), ws_n, _stream()))
    return y


def moe_route(topk_ids: torch.Tensor, E: int, group_list: torch.Tensor | None = None,
              row_token: torch.Tensor | None = None, pair_row: torch.Tensor | None = None):
    """int32 expert ids [T, top_k] -> (group_list int64 [E], row_token int32 [T * top_k],
    pair_row int32 [T, top_k]); rows expert-major, pair order inside an expert."""
    _need(topk_ids, torch.int32, "topk_ids", 2)
    T, k = topk_ids.shape
    dev = topk_ids.device
    if group_list is None:
        group_list = torch.empty((E,), dtype=torch.int64, device=dev)
    if row_token is None:
        row_token = torch.empty((T * k,), dtype=torch.int32, device=dev)
    if pair_row is None:
        pair_row = torch.empty((T, k), dtype=torch.int32, device=dev)
    _need(group_list, torch.int64, "group_list", 1)
    _need(row_token, torch.int32, "row_token", 1)
    _need(pair_row, torch.int32, "pair_row", 2)
    if group_list.shape[0] != E or row_token.shape[0] != T * k or tuple(pair_row.shape) != (T, k):
        raise ValueError("route output shape mismatch")
    _check(lib.w8a8_moe_route(_ptr(topk_ids), T, k, E, _ptr(group_list), _ptr(row_token),
                              _ptr(pair_row), _stream()))
    return group_list, row_token, pair_row


def moe_gather(q: torch.Tensor, scale: torch.Tensor, row_token: torch.Tensor,
               q_rows: torch.Tensor | None = None, s_rows: torch.Tensor | None = None):
    """INT8 tokens [T, H] + scales [T] -> rows [R, H] + scales [R], row p = token row_token[p]."""
    _need(q, torch.int8, "q", 2)
    _need(scale, torch.float32, "scale", 1)
    _need(row_token, torch.int32, "row_token", 1)
    T, H = q.shape
    R = row_token.shape[0]
    if scale.shape[0] != T:
        raise ValueError("scale must have T entries")
    if q_rows is None:
        q_rows = torch.empty((R, H), dtype=torch.int8, device=q.device)
    if s_rows is None:
        s_rows = torch.empty((R,), dtype=torch.float32, device=q.device)
    _need(q_rows, torch.int8, "q_rows", 2)
    _need(s_rows, torch.float32, "s_rows", 1)
    if tuple(q_rows.shape) != (R, H) or s_rows.shape[0] != R:
        raise ValueError("gather output shape mismatch")
    _check(lib.w8a8_moe_gather(_ptr(q), _ptr(scale), T, H, _ptr(row_token), R, _ptr(q_rows),
                               _ptr(s_rows), _stream()))
    return q_rows, s_rows


def moe_combine(y_rows: torch.Tensor, pair_row: torch.Tensor, topk_weights: torch.Tensor,
                out: torch.Tensor | None = None):
    """BF16 rows [R, H] -> BF16 tokens [T, H]: weighted sum of every token's top_k rows."""
    _need(y_rows, torch.bfloat16, "y_rows", 2)
    _need(pair_row, torch.int32, "pair_row", 2)
    _need(topk_weights, torch.float32, "topk_weights", 2)
    R, H = y_rows.shape
    T, k = pair_row.shape
    if tuple(topk_weights.shape) != (T, k):
        raise ValueError("topk_weights must match pair_row")
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=y_rows.device)
    _need(out, torch.bfloat16, "out", 2)
    if tuple(out.shape) != (T, H):
        raise ValueError("out shape mismatch")
    _check(lib.w8a8_moe_combine(_ptr(y_rows), R, H, _ptr(pair_row), _ptr(topk_weights), T, k,
                                _ptr(out), _stream()))
    return out


def moe_layer_workspace_bytes(T: int, top_k: int, E: int, H: int, I: int) -> int:
    return int(lib.w8a8_moe_layer_workspace_bytes(T, top_k, E, H, I))


def moe_layer(x: torch.Tensor, topk_ids: torch.Tensor, topk_weights: torch.Tensor,
              w13_packed: torch.Tensor, w13_scale: torch.Tensor, w2_packed: torch.Tensor,
              w2_scale: torch.Tensor, out: torch.Tensor | None = None,
              workspace: torch.Tensor | None = None):
    """Whole MoE layer: BF16 tokens [T, H] -> quantize once, route, gather, W13 ->
    SwiGLU + requant -> W2, weighted combine -> BF16 [T, H]."""
    _need(x, torch.bfloat16, "x", 2)
    _need(topk_ids, torch.int32, "topk_ids", 2)
    _need(topk_weights, torch.float32, "topk_weights", 2)
    _need(w13_scale, torch.float32, "w13_scale", 2)
    _need(w2_scale, torch.float32, "w2_scale", 2)
    _need(w13_packed, torch.uint8, "w13_packed", 1)
    _need(w2_packed, torch.uint8, "w2_packed", 1)
    T, H = x.shape
    k = topk_ids.shape[1]
    E = w13_scale.shape[0]
    I = w13_scale.shape[1] // 2
    if topk_ids.shape[0] != T or tuple(topk_weights.shape) != tuple(topk_ids.shape):
        raise ValueError("topk_ids / topk_weights must be [T, top_k]")
    if tuple(w13_scale.shape) != (E, 2 * I) or tuple(w2_scale.shape) != (E, H):
        raise ValueError("scale shape mismatch")
    if w13_packed.numel() < packed_weight_bytes(E, 2 * I, H) or \
            w2_packed.numel() < packed_weight_bytes(E, H, I):
        raise ValueError("packed weights too small")
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    _need(out, torch.bfloat16, "out", 2)
    if tuple(out.shape) != (T, H):
        raise ValueError("out shape mismatch")
    ws, ws_n = _workspace(moe_layer_workspace_bytes(T, k, E, H, I), x.device, workspace)
    _check(lib.w8a8_moe_layer(_ptr(x), T, H, _ptr(topk_ids), _ptr(topk_weights), k, E, I,
                              _ptr(w13_packed), _ptr(w13_scale), _ptr(w2_packed), _ptr(w2_scale),
                              _ptr(out), _ptr(ws), ws_n, _stream()))
    return out


# ---------------------------------------------------------------------------
# MXFP8 variant
# ---------------------------------------------------------------------------

def mx_quant(x: torch.Tensor, scale_alg: int = 0, payload: torch.Tensor | None = None,
             scales: torch.Tensor | None = None):
    """BF16 [M, K] -> (E4M3 payload uint8 [M, K], E8M0 scales uint8 [M, K/32])."""
    _need(x, torch.bfloat16, "x", 2)
    M, K = x.shape
    if payload is None:
        payload = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((M, max(K // 32, 0)), dtype=torch.uint8, device=x.device)
    _need(payload, torch.uint8, "payload", 2)
    _need(scales, torch.uint8, "scales", 2)
    _check(lib.w8a8_mx_quant(_ptr(x), M, K, _ptr(payload), _ptr(scales), scale_alg, _stream()))
    return payload, scales


def mx_resolve_block_fp8(w_e4m3: torch.Tensor, scale_inv: torch.Tensor, bn: int, bk: int,
                         out: torch.Tensor | None = None) -> torch.Tensor:
    """E4M3 [N, K] with fp32 tile scales [ceil(N/bn), ceil(K/bk)] -> BF16 [N, K]."""
    _need(w_e4m3, torch.uint8, "w_e4m3", 2)
    _need(scale_inv, torch.float32, "scale_inv", 2)
    N, K = w_e4m3.shape
    if tuple(scale_inv.shape) != (-(-N // bn), -(-K // bk)):
        raise ValueError("scale_inv shape does not match the tile grid")
    if out is None:
        out = torch.empty((N, K), dtype=torch.bfloat16, device=w_e4m3.device)
    _need(out, torch.bfloat16, "out", 2)
    _check(lib.w8a8_mx_resolve_block_fp8(_ptr(w_e4m3), _ptr(scale_inv), N, K, bn, bk, _ptr(out),
                                         _stream()))
    return out


def mx_packed_bytes(N: int, K: int) -> int:
    return int(lib.w8a8_mx_packed_bytes(N, K))


def mx_prepack_weight(w_e4m3: torch.Tensor, w_e8m0: torch.Tensor,
                      out: torch.Tensor | None = None) -> torch.Tensor:
    """E4M3 [N, K] + E8M0 [N, K/32] -> packed MX weight (uint8, stable buffer)."""
    _need(w_e4m3, torch.uint8, "w_e4m3", 2)
    _need(w_e8m0, torch.uint8, "w_e8m0", 2)
    N, K = w_e4m3.shape
    if tuple(w_e8m0.shape) != (N, K // 32):
        raise ValueError("w_e8m0 must be [N, K/32]")
    nbytes = mx_packed_bytes(N, K)
    if out is None:
        out = torch.empty((nbytes,), dtype=torch.uint8, device=w_e4m3.device)
    _need(out, torch.uint8, "out", 1)
    _check(lib.w8a8_mx_prepack_weight(_ptr(w_e4m3), _ptr(w_e8m0), N, K, _ptr(out), _stream()))
    return out


def mx_linear_workspace_bytes(M: int, K: int) -> int:
    return int(lib.w8a8_mx_linear_workspace_bytes(M, K))


def mx_linear(x: torch.Tensor, w_packed: torch.Tensor, N: int, x_e8m0: torch.Tensor | None = None,
              scale_alg: int = 0, y: torch.Tensor | None = None,
              workspace: torch.Tensor | None = None) -> torch.Tensor:
    """MX block-scaled linear: BF16 x (or E4M3 x with x_e8m0) times packed MX W -> BF16 [M, N]."""
    if x_e8m0 is None:
        _need(x, torch.bfloat16, "x", 2)
    else:
        _need(x, torch.uint8, "x", 2)
        _need(x_e8m0, torch.uint8, "x_e8m0", 2)
    _need(w_packed, torch.uint8, "w_packed", 1)
    M, K = x.shape
    if w_packed.numel() < mx_packed_bytes(N, K):
        raise ValueError("w_packed too small for [N, K]")
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _need(y, torch.bfloat16, "y", 2)
    ws, ws_n = _workspace(mx_linear_workspace_bytes(M, K), x.device, workspace)
    _check(lib.w8a8_mx_linear(_ptr(x), _ptr(x_e8m0), M, K, _ptr(w_packed), N, _ptr(y), scale_alg,
                              _ptr(ws), ws_n, _stream()))
    return y


# ---------------------------------------------------------------------------
# MXFP8 MoE path
# ---------------------------------------------------------------------------
ACT_NONE, ACT_SWIGLU = 0, 1


def mx_moe_staging_bytes(N: int, K: int) -> int:
    return int(lib.w8a8_mx_moe_staging_bytes(N, K))


def mx_moe_packed_bytes(E: int, N: int, K: int) -> int:
    return int(lib.w8a8_mx_moe_packed_bytes(E, N, K))


def mx_moe_prepare(w_e4m3: torch.Tensor, scale_inv: torch.Tensor, bn: int, bk: int,
                   scale_alg: int = 0, pack: bool = True, w_e8m0: torch.Tensor | None = None,
                   packed: torch.Tensor | None = None, staging: torch.Tensor | None = None):
    """Block-FP8 expert stack -> MXFP8, one expert at a time. ``w_e4m3`` (uint8
    [E, N, K]) is overwritten with the MX payload. Returns (w_e8m0 [E, N, K/32],
    packed stack or None)."""
    _need(w_e4m3, torch.uint8, "w_e4m3", 3)
    _need(scale_inv, torch.float32, "scale_inv", 3)
    E, N, K = w_e4m3.shape
    dev = w_e4m3.device
    if tuple(scale_inv.shape) != (E, -(-N // bn), -(-K // bk)):
        raise ValueError("scale_inv must be [E, ceil(N/bn), ceil(K/bk)]")
    if w_e8m0 is None:
        w_e8m0 = torch.empty((E, N, K // 32), dtype=torch.uint8, device=dev)
    _need(w_e8m0, torch.uint8, "w_e8m0", 3)
    if pack and packed is None:
        packed = torch.empty((mx_moe_packed_bytes(E, N, K),), dtype=torch.uint8, device=dev)
    if packed is not None:
        _need(packed, torch.uint8, "packed", 1)
    st, st_n = _workspace(mx_moe_staging_bytes(N, K), dev, staging)
    _check(lib.w8a8_mx_moe_prepare(_ptr(w_e4m3), _ptr(scale_inv), E, N, K, bn, bk, scale_alg,
                                   _ptr(w_e8m0), _ptr(packed), _ptr(st), st_n, _stream()))
    return w_e8m0, packed


def mx_swiglu_quant(h: torch.Tensor, scale_alg: int = 0):
    """BF16 h [R, 2I] (gate | up) -> (E4M3 [R, I], E8M0 [R, I/32]) of BF16(SwiGLU)."""
    _need(h, torch.bfloat16, "h", 2)
    R, I2 = h.shape
    I = I2 // 2
    p = torch.empty((R, I), dtype=torch.uint8, device=h.device)
    sc = torch.empty((R, max(I // 32, 1)), dtype=torch.uint8, device=h.device)
    _check(lib.w8a8_mx_swiglu_quant(_ptr(h), R, I, scale_alg, _ptr(p), _ptr(sc), _stream()))
    return p, sc


def mx_grouped_workspace_bytes(R: int, E: int, K: int) -> int:
    return int(lib.w8a8_mx_grouped_workspace_bytes(R, E, K))


def mx_grouped_gemm(x: torch.Tensor, group_list: torch.Tensor, w_packed: torch.Tensor, N: int,
                    act: int = ACT_NONE, scale_alg: int = 0, y: torch.Tensor | None = None,
                    workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Expert-grouped BF16 rows (or [gate | up] rows with act=ACT_SWIGLU) times each
    expert's prepared MX weight -> BF16 [R, N]."""
    _need(x, torch.bfloat16, "x", 2)
    _need(group_list, torch.int64, "group_list", 1)
    _need(w_packed, torch.uint8, "w_packed", 1)
    R, Kx = x.shape
    K = Kx // 2 if act == ACT_SWIGLU else Kx
    E = group_list.shape[0]
    if w_packed.numel() < mx_moe_packed_bytes(E, N, K):
        raise ValueError("w_packed too small for [E, N, K]")
    if y is None:
        y = torch.empty((R, N), dtype=torch.bfloat16, device=x.device)
    _need(y, torch.bfloat16, "y", 2)
    ws, ws_n = _workspace(mx_grouped_workspace_bytes(R, E, K), x.device, workspace)
    _check(lib.w8a8_mx_grouped_gemm(_ptr(x), _ptr(group_list), R, E, N, K, act, _ptr(w_packed),
                                    scale_alg, _ptr(y), _ptr(ws), ws_n, _stream()))
    return y


def mx_moe_workspace_bytes(R: int, E: int, H: int, I: int) -> int:
    return int(lib.w8a8_mx_moe_workspace_bytes(R, E, H, I))


def mx_moe_grouped(x_rows: torch.Tensor, group_list: torch.Tensor, w13_packed: torch.Tensor,
                   w2_packed: torch.Tensor, I: int, scale_alg: int = 0,
                   y: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """MXFP8 expert chain on expert-grouped BF16 rows [R, H] -> BF16 [R, H]."""
    _need(x_rows, torch.bfloat16, "x_rows", 2)
    _need(group_list, torch.int64, "group_list", 1)
    _need(w13_packed, torch.uint8, "w13_packed", 1)
    _need(w2_packed, torch.uint8, "w2_packed", 1)
    R, H = x_rows.shape
    E = group_list.shape[0]
    if w13_packed.numel() < mx_moe_packed_bytes(E, 2 * I, H) or \
            w2_packed.numel() < mx_moe_packed_bytes(E, H, I):
        raise ValueError("packed expert weights too small")
    if y is None:
        y = torch.empty((R, H), dtype=torch.bfloat16, device=x_rows.device)
    _need(y, torch.bfloat16, "y", 2)
    ws, ws_n = _workspace(mx_moe_workspace_bytes(R, E, H, I), x_rows.device, workspace)
    _check(lib.w8a8_mx_moe_grouped(_ptr(x_rows), _ptr(group_list), R, E, H, I, _ptr(w13_packed),
                                   _ptr(w2_packed), scale_alg, _ptr(y), _ptr(ws), ws_n, _stream()))
    return y


# ---------------------------------------------------------------------------
# W4A16 weight variant
# ---------------------------------------------------------------------------

def w4a16_packed_bytes(N: int, K: int) -> int:
    return int(lib.w8a8_w4a16_packed_bytes(N, K))


def fp4_packed_bytes(N: int, K: int) -> int:
    return int(lib.w8a8_fp4_packed_bytes(N, K))


def w4a16_quant_weight(w: torch.Tensor, codes: bool = False, scales: bool = False,
                       pack: bool = True):
    """BF16 weight [N, K] -> (int8 codes [N, K] or None, BF16 scales [N, K/32] or
    None, packed uint8 buffer or None): INT4 per 32 input channels, scale amax / 7."""
    _need(w, torch.bfloat16, "w", 2)
    N, K = w.shape
    dev = w.device
    q = torch.empty((N, K), dtype=torch.int8, device=dev) if codes else None
    s = torch.empty((N, max(K // 32, 1)), dtype=torch.bfloat16, device=dev) if scales else None
    p = torch.empty((w4a16_packed_bytes(N, K),), dtype=torch.uint8, device=dev) if pack else None
    _check(lib.w8a8_w4a16_quant_weight(_ptr(w), N, K, _ptr(q), _ptr(s), _ptr(p), _stream()))
    return q, s, p


def w4a16_pack(q: torch.Tensor, s: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Pre-quantized int8 codes [N, K] in [-8, 7] and BF16 scales [N, K/32] -> packed."""
    _need(q, torch.int8, "q", 2)
    _need(s, torch.bfloat16, "s", 2)
    N, K = q.shape
    if tuple(s.shape) != (N, K // 32):
        raise ValueError("scales must be [N, K/32]")
    if out is None:
        out = torch.empty((w4a16_packed_bytes(N, K),), dtype=torch.uint8, device=q.device)
    _need(out, torch.uint8, "out", 1)
    _check(lib.w8a8_w4a16_pack(_ptr(q), _ptr(s), N, K, _ptr(out), _stream()))
    return out


def w4a16_linear_workspace_bytes(M: int, K: int) -> int:
    return int(lib.w8a8_w4a16_linear_workspace_bytes(M, K))


def w4a16_linear(x: torch.Tensor, w_packed: torch.Tensor, N: int,
                 y: torch.Tensor | None = None,
                 workspace: torch.Tensor | None = None) -> torch.Tensor:
    """BF16 x [M, K] times the packed INT4 weight [N, K] -> BF16 [M, N]."""
    _need(x, torch.bfloat16, "x", 2)
    _need(w_packed, torch.uint8, "w_packed", 1)
    M, K = x.shape
    if w_packed.numel() < w4a16_packed_bytes(N, K):
        raise ValueError("w_packed too small for [N, K]")
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _need(y, torch.bfloat16, "y", 2)
    ws, ws_n = _workspace(w4a16_linear_workspace_bytes(M, K), x.device, workspace)
    _check(lib.w8a8_w4a16_linear(_ptr(x), M, K, _ptr(w_packed), N, _ptr(y), _ptr(ws), ws_n,
                                 _stream()))
    return y


def fp4_quant_weight(w: torch.Tensor, codes: bool = False, scales: bool = False,
                     pack: bool = True):
    """BF16 weight [N, K] -> (E2M1 codes uint8 [N, K] or None, E8M0 bytes uint8
    [N, K/32] or None, packed uint8 buffer or None): FP4 with one E8M0 scale per 32."""
    _need(w, torch.bfloat16, "w", 2)
    N, K = w.shape
    dev = w.device
    c = torch.empty((N, K), dtype=torch.uint8, device=dev) if codes else None
    s = torch.empty((N, max(K // 32, 1)), dtype=torch.uint8, device=dev) if scales else None
    p = torch.empty((fp4_packed_bytes(N, K),), dtype=torch.uint8, device=dev) if pack else None
    _check(lib.w8a8_fp4_quant_weight(_ptr(w), N, K, _ptr(c), _ptr(s), _ptr(p), _stream()))
    return c, s, p


def fp4_linear(x: torch.Tensor, w_packed: torch.Tensor, N: int,
               y: torch.Tensor | None = None,
               workspace: torch.Tensor | None = None) -> torch.Tensor:
    """BF16 x [M, K] times the packed FP4 weight [N, K] -> BF16 [M, N]."""
    _need(x, torch.bfloat16, "x", 2)
    _need(w_packed, torch.uint8, "w_packed", 1)
    M, K = x.shape
    if w_packed.numel() < fp4_packed_bytes(N, K):
        raise ValueError("w_packed too small for [N, K]")
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _need(y, torch.bfloat16, "y", 2)
    ws, ws_n = _workspace(w4a16_linear_workspace_bytes(M, K), x.device, workspace)
    _check(lib.w8a8_fp4_linear(_ptr(x), M, K, _ptr(w_packed), N, _ptr(y), _ptr(ws), ws_n,
                               _stream()))
    return y


LOWBIT_INT4 = 0   # w4a16_quant_weight's packed layout
LOWBIT_FP4 = 1    # fp4_quant_weight's packed layout


def _lowbit_bytes(fmt: int, N: int, K: int) -> int:
    if fmt == LOWBIT_INT4:
        return w4a16_packed_bytes(N, K)
    if fmt == LOWBIT_FP4:
        return fp4_packed_bytes(N, K)
    raise ValueError(f"unknown low-bit weight format {fmt}")


def w4a16_grouped_gemm(x: torch.Tensor, group_list: torch.Tensor, w_packed: torch.Tensor, N: int,
                       fmt: int = LOWBIT_INT4, y: torch.Tensor | None = None) -> torch.Tensor:
    """Expert-grouped BF16 rows [R, K] times each expert's packed INT4 / FP4 weight
    [N, K] (experts stacked, one packed weight each) -> BF16 [R, N]."""
    _need(x, torch.bfloat16, "x", 2)
    _need(group_list, torch.int64, "group_list", 1)
    _need(w_packed, torch.uint8, "w_packed", 1)
    R, K = x.shape
    E = group_list.shape[0]
    if w_packed.numel() < E * _lowbit_bytes(fmt, N, K):
        raise ValueError("w_packed too small for [E, N, K]")
    if y is None:
        y = torch.empty((R, N), dtype=torch.bfloat16, device=x.device)
    _need(y, torch.bfloat16, "y", 2)
    _check(lib.w8a8_w4a16_grouped_gemm(fmt, _ptr(x), _ptr(group_list), R, E, N, K, _ptr(w_packed),
                                       _ptr(y), _stream()))
    return y


def w4a16_swiglu(h: torch.Tensor, a: torch.Tensor | None = None) -> torch.Tensor:
    """BF16 [R, 2I] = [gate | up] -> BF16 [R, I] = BF16(silu(gate) * up)."""
    _need(h, torch.bfloat16, "h", 2)
    R, I2 = h.shape
    if I2 % 2:
        raise ValueError("h must have an even number of columns")
    if a is None:
        a = torch.empty((R, I2 // 2), dtype=torch.bfloat16, device=h.device)
    _need(a, torch.bfloat16, "a", 2)
    _check(lib.w8a8_w4a16_swiglu(_ptr(h), R, I2 // 2, _ptr(a), _stream()))
    return a


def w4a16_moe_workspace_bytes(R: int, H: int, I: int) -> int:
    return int(lib.w8a8_w4a16_moe_workspace_bytes(R, H, I))


def w4a16_moe_grouped(x_rows: torch.Tensor, group_list: torch.Tensor, w13_packed: torch.Tensor,
                      w2_packed: torch.Tensor, I: int, fmt: int = LOWBIT_INT4,
                      y: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """Low-bit expert chain on expert-grouped BF16 rows [R, H] -> BF16 [R, H]:
    W13 -> BF16 SwiGLU -> W2, activations kept in BF16."""
    _need(x_rows, torch.bfloat16, "x_rows", 2)
    _need(group_list, torch.int64, "group_list", 1)
    _need(w13_packed, torch.uint8, "w13_packed", 1)
    _need(w2_packed, torch.uint8, "w2_packed", 1)
    R, H = x_rows.shape
    E = group_list.shape[0]
    if w13_packed.numel() < E * _lowbit_bytes(fmt, 2 * I, H) or \
            w2_packed.numel() < E * _lowbit_bytes(fmt, H, I):
        raise ValueError("packed expert weights too small")
    if y is None:
        y = torch.empty((R, H), dtype=torch.bfloat16, device=x_rows.device)
    _need(y, torch.bfloat16, "y", 2)
    ws, ws_n = _workspace(w4a16_moe_workspace_bytes(R, H, I), x_rows.device, workspace)
    _check(lib.w8a8_w4a16_moe_grouped(fmt, _ptr(x_rows), _ptr(group_list), R, E, H, I,
                                      _ptr(w13_packed), _ptr(w2_packed), _ptr(y), _ptr(ws), ws_n,
                                      _stream()))
    return y


def mx_workspace_operands(workspace: torch.Tensor, M: int, K: int):
    """(E4M3 payload in 1 KB P16x64 blocks, k-block-major E8M0 bytes) views of an
    mx_linear workspace."""
    _need(workspace, torch.uint8, "workspace", 1)
    nblk = -(-M // 16) * 16 * (-(-K // 64)) * 64
    off = -(-nblk // 256) * 256
    nsc = -(-K // 64) * (M + (M & 1)) * 2
    if workspace.numel() < off + nsc:
        raise ValueError("workspace too small")
    return workspace[:nblk], workspace[off:off + nsc]


def mx_gemm(a_e4m3: torch.Tensor, a_scale_kb: torch.Tensor, M: int, K: int,
            w_packed: torch.Tensor, N: int, y: torch.Tensor | None = None) -> torch.Tensor:
    """GEMM stage of mx_linear: E4M3 activation blocks (as mx_workspace_operands
    gives them) + k-block-major E8M0 -> BF16 [M, N]."""
    _need(a_e4m3, torch.uint8, "a_e4m3", 1)
    _need(a_scale_kb, torch.uint8, "a_scale_kb", 1)
    _need(w_packed, torch.uint8, "w_packed", 1)
    if a_e4m3.numel() < -(-M // 16) * 16 * (-(-K // 64)) * 64:
        raise ValueError("a_e4m3 too small for [M, K] in blocks")
    if a_scale_kb.numel() < -(-K // 64) * (M + (M & 1)) * 2:
        raise ValueError("a_scale_kb must hold ceil(K/64) * (M rounded up to even) * 2 bytes")
    if w_packed.numel() < mx_packed_bytes(N, K):
        raise ValueError("w_packed too small for [N, K]")
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=a_e4m3.device)
    _need(y, torch.bfloat16, "y", 2)
    _check(lib.w8a8_mx_gemm(_ptr(a_e4m3), _ptr(a_scale_kb), M, K, _ptr(w_packed), N, _ptr(y),
                            _stream()))
    return y


# ---------------------------------------------------------------------------
# static W8A8
# ---------------------------------------------------------------------------

def static_quant(x: torch.Tensor, input_scale: float, input_offset: float,
                 q: torch.Tensor | None = None) -> torch.Tensor:
    """BF16 [M, K] -> int8 [M, K] with a fixed per-tensor scale and offset."""
    _need(x, torch.bfloat16, "x", 2)
    M, K = x.shape
    if q is None:
        q = torch.empty((M, K), dtype=torch.int8, device=x.device)
    _need(q, torch.int8, "q", 2)
    if tuple(q.shape) != (M, K):
        raise ValueError("q must be [M, K]")
    _check(lib.w8a8_static_quant(_ptr(x), M, K, float(input_scale), float(input_offset), _ptr(q),
                                 _stream()))
    return q


def static_quant_packed(x: torch.Tensor, input_scale: float, input_offset: float,
                        q: torch.Tensor | None = None) -> torch.Tensor:
    """BF16 [M, K] -> int8 codes in the weight's 1 KB block layout (uint8 buffer)."""
    _need(x, torch.bfloat16, "x", 2)
    M, K = x.shape
    nbytes = packed_weight_bytes(1, M, K)
    if q is None:
        q = torch.empty((nbytes,), dtype=torch.uint8, device=x.device)
    _need(q, torch.uint8, "q", 1)
    if q.numel() < nbytes:
        raise ValueError("q too small for the packed layout")
    _check(lib.w8a8_static_quant_packed(_ptr(x), M, K, float(input_scale), float(input_offset), _ptr(q),
                                        _stream()))
    return q


def static_prepare(w: torch.Tensor, w_scale: torch.Tensor, bias: torch.Tensor | None,
                   input_scale: float, input_offset: float):
    """int8 [N, K], float [N], BF16 [N] or None -> (deq_scale float [N], quant_bias int32 [N])."""
    _need(w, torch.int8, "w", 2)
    _need(w_scale, torch.float32, "w_scale", 1)
    N, K = w.shape
    if bias is not None:
        _need(bias, torch.bfloat16, "bias", 1)
    deq = torch.empty((N,), dtype=torch.float32, device=w.device)
    qb = torch.empty((N,), dtype=torch.int32, device=w.device)
    _check(lib.w8a8_static_prepare(_ptr(w), N, K, _ptr(w_scale), _ptr(bias), float(input_scale),
                                   float(input_offset), _ptr(deq), _ptr(qb), _stream()))
    return deq, qb


def static_linear(q: torch.Tensor, w_packed: torch.Tensor, deq_scale: torch.Tensor,
                  quant_bias: torch.Tensor, N: int, out: int = OUT_BF16,
                  y: torch.Tensor | None = None, M: int | None = None,
                  K: int | None = None) -> torch.Tensor:
    """Static W8A8 matmul: int8 [M, K] codes (or, with M and K given, the uint8
    packed blocks of static_quant_packed) -> BF16 (or raw INT32) [M, N]."""
    packed = q.dtype == torch.uint8
    if packed:
        _need(q, torch.uint8, "q", 1)
        if M is None or K is None:
            raise ValueError("packed codes need M and K")
        if q.numel() < packed_weight_bytes(1, M, K):
            raise ValueError("q too small for the packed layout")
    else:
        _need(q, torch.int8, "q", 2)
        M, K = q.shape
    _need(w_packed, torch.uint8, "w_packed", 1)
    _need(deq_scale, torch.float32, "deq_scale", 1)
    _need(quant_bias, torch.int32, "quant_bias", 1)
    dt = torch.bfloat16 if out == OUT_BF16 else torch.int32
    if y is None:
        y = torch.empty((M, N), dtype=dt, device=q.device)
    _need(y, dt, "y", 2)
    flag = A_PACKED if packed else 0
    _check(lib.w8a8_static_linear(_ptr(q), M, K, _ptr(w_packed), _ptr(deq_scale), _ptr(quant_bias), N,
                                  _ptr(y), out | flag, _stream()))
    return y
