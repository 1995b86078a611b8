"""NumPy oracle of the steps on either side of the MoE chain on one GPU.
TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg
may import this module. It shares no code, tables or constants with the HIP
library under ``moe_token_amax_amd/``.

Page: [DSV4] "DeepSeek-V4 W8A8 执行链从量化权重到 Ascend INT8 算子", §三 (MoE:
DeepEP INT8 dispatch and the Ascend runner). What the page fixes: the dispatch
quantizes the local BF16 hidden states to INT8 plus one scale per token and
moves those; its output carries hidden_states, hidden_states_scale, topk_ids,
topk_weights and the number of received tokens per expert; the runner takes
the INT8 rows, their scale and the per-expert counts (expert_tokens) into W13
without quantizing again; the chain ends with the BF16 W2 output.

On one GPU the dispatch is: quantize the T tokens once, order the T x top_k
(token, slot) pairs by expert, and gather each pair's INT8 row and scale; the
combine after W2 undoes the order and sums each token's top_k rows weighted by
topk_weights.

Readings (the page names the data, not these steps' arithmetic):
  * rows of one expert keep the order of their pair index t * top_k + j
    (a stable sort by expert); pairs whose expert id lies outside [0, E) are
    dropped (no row, no contribution);
  * combine: out[t] = BF16(sum over j = 0 .. top_k - 1, in that order, of
    fl32(topk_weights[t, j] * y_row)), each product and each partial sum one
    fp32 rounding (no fused multiply-add), starting from +0.0.

Parity status (tests/test_oracle_moe_io_pins.py): route pinned by a hand
example and by counting; dispatch by its definition (quantize then gather)
against gather-then-quantize, which the page's claim makes equal; combine by a
hand example, one-hot weights and a float64 bound; moe_forward as the
composition of pinned stages.
"""

from __future__ import annotations

import numpy as np

from .w8a8_ref import bf16_to_f32, dynamic_quant, f32_to_bf16, moe_grouped

__all__ = ["route", "dispatch_int8", "combine", "moe_forward"]


def route(topk_ids, num_experts: int):
    """(token, slot) pairs -> per-expert row counts and the expert-major order.

    topk_ids int [T, top_k]. Returns (group_list int64 [E], row_token int32 [R],
    pair_row int32 [T, top_k]) with R the number of valid pairs: row p of the
    grouped input is token row_token[p]; pair (t, j) sits in row pair_row[t, j]
    (-1 for an id outside [0, E)).
    """
    ids = np.asarray(topk_ids, np.int64)
    T, k = ids.shape
    flat = ids.reshape(-1)
    valid = (flat >= 0) & (flat < num_experts)
    group_list = np.bincount(flat[valid], minlength=num_experts).astype(np.int64)
    pairs = np.nonzero(valid)[0]                               # pair indices in order
    order = pairs[np.argsort(flat[pairs], kind="stable")]      # expert-major, stable
    row_token = (order // k).astype(np.int32)
    pair_row = np.full(T * k, -1, np.int32)
    pair_row[order] = np.arange(order.size, dtype=np.int32)
    return group_list, row_token, pair_row.reshape(T, k)


def dispatch_int8(x_bits, row_token):
    """Quantize the T tokens once (per-token symmetric INT8), then gather the
    codes and scales of every routed row. Returns (q_rows int8 [R, H],
    s_rows float32 [R])."""
    q, s = dynamic_quant(x_bits)
    rt = np.asarray(row_token, np.int64)
    return q[rt], s[rt]


def combine(y_rows_bits, pair_row, topk_weights):
    """out[t] = BF16(sum_j fl32(w[t, j] * y[pair_row[t, j]])) in slot order."""
    y = bf16_to_f32(y_rows_bits)
    pr = np.asarray(pair_row, np.int64)
    w = np.asarray(topk_weights, np.float32)
    T, k = pr.shape
    acc = np.zeros((T, y.shape[1]), np.float32)
    for j in range(k):
        ok = pr[:, j] >= 0
        prod = (w[ok, j][:, None] * y[pr[ok, j]]).astype(np.float32)
        acc[ok] = (acc[ok] + prod).astype(np.float32)
    return f32_to_bf16(acc)


def moe_forward(x_bits, topk_ids, topk_weights, w13, w13_scale, w2, w2_scale, keep=False):
    """Whole MoE layer on one GPU: INT8 dispatch -> W13 -> SwiGLU + requant -> W2
    -> weighted combine. Returns out_bits [T, H] (or every stage with keep)."""
    E = w13.shape[0]
    group_list, row_token, pair_row = route(topk_ids, E)
    q_rows, s_rows = dispatch_int8(x_bits, row_token)
    y_rows = moe_grouped(group_list, w13, w13_scale, w2, w2_scale, q=q_rows, x_scale=s_rows)
    out = combine(y_rows, pair_row, topk_weights)
    if keep:
        return dict(group_list=group_list, row_token=row_token, pair_row=pair_row,
                    q_rows=q_rows, s_rows=s_rows, y_rows=y_rows, out=out)
    return out
