"""NumPy oracle of the MXFP8 MoE path. TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this module. It shares no code, tables or constants with the
HIP library under ``moe_token_amax_amd/``.

Page: [MXFP8] "Qwen3.8-FP8 on Ascend 950: Why Weights Become MXFP8 at Load
Time", Deep Dive 6 (MoE weights follow the same contract without a full dense
expert copy), with Deep Dives 2, 3 and 5 for the per-expert steps. What the page
fixes: the fused-MoE weights w13 and w2 go through the dense layer's contract
(source resolve -> MX re-quantization -> kernel repack) one expert at a time:
an expert is resolved, re-quantized, its MXFP8 bytes written back over its FP8
source bytes and its E8M0 scales into a separate scale buffer, before the next
expert is staged (peak staging = one dense expert); at run time the expert
buffers, their E8M0 scales and the routing metadata go to the fused expert
execution, whose activations are MX-quantized at run time as in Deep Dive 5.

Readings (the page describes the MoE apply only by what it passes along):
  * the expert chain is the one of the INT8 path ([DSV4] §三): W13 grouped
    matmul over the rows of each expert (group_list as there), SwiGLU (the
    same fixed fp32 sequence, ``w8a8_ref.swiglu``), W2 grouped matmul;
  * every matmul input is an ordinary BF16 activation MX-quantized at run time
    (Deep Dive 5): the rows of x, and the SwiGLU output rounded once to BF16;
  * each grouped matmul returns BF16 of the exact sum of the dequantized
    products (float64 here; the GPU accumulates in fp32, compared within the
    dense MX GEMM's tolerance);
  * one-expert staging is a memory property: the prepared weights equal the
    dense preparation of every expert on its own.

Parity status (tests/test_oracle_mx_moe_pins.py): the preparation pinned by the
page's worked resolve example placed in one expert, expert independence and
the MX error bound against the resolved weight; the SwiGLU MX quant by hand
rows (ties, zero groups) and the MX error bound; the grouped matmul by hand
experts, empty experts and float64 brute force; the chain by its stages and by
an unquantized float64 chain within the quantization error.
"""

from __future__ import annotations

import numpy as np

from .mx_ref import mx_dequant, mx_quant, mx_resolve
from .w8a8_ref import bf16_to_f32, f32_to_bf16, group_offsets, swiglu

__all__ = ["mx_moe_prepare", "swiglu_mx_quant", "mx_grouped_gemm", "mx_moe_grouped"]


def mx_moe_prepare(w_e4m3, scale_inv, bn: int, bk: int, scale_alg: int = 0):
    """Block-FP8 expert stack -> MXFP8, one expert at a time.

    w_e4m3 uint8 [E, N, K] (E4M3 codes), scale_inv float32 [E, ceil(N/bn),
    ceil(K/bk)]. Expert e: resolve to BF16 (Deep Dive 2), then MX-quantize the
    resolved values (Deep Dive 3). Returns (payload uint8 [E, N, K], the bytes
    that replace the source codes, and scales uint8 [E, N, K / 32]).
    """
    w = np.asarray(w_e4m3, np.uint8)
    E, N, K = w.shape
    payload = np.empty_like(w)
    scales = np.empty((E, N, K // 32), np.uint8)
    for e in range(E):                      # one dense expert staged at a time
        resolved = mx_resolve(w[e], scale_inv[e], bn, bk)
        payload[e], scales[e] = mx_quant(bf16_to_f32(resolved), scale_alg)
    return payload, scales


def swiglu_mx_quant(h_bits, inter: int, scale_alg: int = 0):
    """SwiGLU of BF16 h [R, 2I] (gate | up), rounded once to BF16, then the MX
    quant of that activation. Returns (payload [R, I], scales [R, I / 32], a_bits)."""
    a_bits = f32_to_bf16(swiglu(h_bits, inter))
    p, s = mx_quant(bf16_to_f32(a_bits), scale_alg)
    return p, s, a_bits


def mx_grouped_gemm(group_list, a_payload, a_scales, w_payload, w_scales):
    """Rows of expert e (in group order) times expert e's weight [N, K] -> BF16
    [R, N]: BF16 of the float64 sum of the dequantized products."""
    off = group_offsets(group_list)
    E, N, _ = np.asarray(w_payload).shape
    R = a_payload.shape[0]
    y = np.zeros((R, N), np.uint16)
    for e in range(E):
        a, b = int(off[e]), int(off[e + 1])
        if b == a:
            continue                        # an empty expert costs nothing
        A = mx_dequant(a_payload[a:b], a_scales[a:b])
        W = mx_dequant(w_payload[e], w_scales[e])
        y[a:b] = f32_to_bf16((A @ W.T).astype(np.float32))
    return y


def mx_moe_grouped(group_list, x_bits, w13_payload, w13_scales, w2_payload, w2_scales,
                   scale_alg: int = 0, keep: bool = False):
    """MXFP8 expert chain on expert-grouped BF16 rows x [R, H] -> BF16 [R, H]."""
    inter = w13_payload.shape[1] // 2
    q1, s1 = mx_quant(bf16_to_f32(x_bits), scale_alg)
    h = mx_grouped_gemm(group_list, q1, s1, w13_payload, w13_scales)
    q2, s2, a = swiglu_mx_quant(h, inter, scale_alg)
    y = mx_grouped_gemm(group_list, q2, s2, w2_payload, w2_scales)
    if keep:
        return dict(q1=q1, s1=s1, h=h, a=a, q2=q2, s2=s2, y=y)
    return y
