"""Seeded synthetic inputs for the W8A8_DYNAMIC path.

Shared by the tests, the benchmark and the oracle checks. This module holds no
step of the method itself: it draws random numbers, rounds them to BF16 with
torch's own CPU conversion, and builds the routing (top-k expert choice,
grouping rows by expert) that produces the MoE path's inputs.

Every tensor draws from its own stream ``numpy.random.default_rng([seed, tag,
index])`` so that one expert's weights can be regenerated alone.

Shapes and distributions (the five workloads):
  tiny      X BF16 [16, 256] N(0,1), 1% of entries x20; W int8 [128, 256]
            uniform [-127, 127]; w_scale U[1e-3, 1e-2]; bias BF16 N(0, 0.1)
  decode    X BF16 [64, 7168] N(0,1), 0.5% x20 (M in {1,4,16,64} takes the first
            M rows); W int8 [4096, 7168]; w_scale; no bias
  prefill   X BF16 [8192, 7168] N(0,1), 0.5% x20; W int8 [4096, 7168]; w_scale;
            bias BF16 [4096] N(0, 0.1)
  moe       T=2048 tokens, H=4096, E=256 experts, top-8, I=2048; X BF16 N(0,1);
            logits N(0,1) + per-expert bias N(0, 1.5); W13 int8 [E, 2I, H],
            W2 int8 [E, H, I]; scales U[1e-3, 1e-2]
  lowbit_moe the moe routing and activations with BF16 expert weights W13
            [E, 2I, H], W2 [E, H, I] drawn N(0, 0.02^2), quantized to INT4 or
            FP4 at load time
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

# stream tags
(_T_X, _T_W, _T_WS, _T_B, _T_LOGITS, _T_EBIAS, _T_W13, _T_W2, _T_W13S, _T_W2S, _T_MXW,
 _T_MXS, _T_MXW13, _T_MXS13, _T_MXW2, _T_MXS2, _T_LBW13, _T_LBW2) = range(18)


def rng_for(seed: int, tag: int, index: int = 0) -> np.random.Generator:
    return np.random.default_rng([seed, tag, index])


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> BF16 bits using torch's CPU conversion (round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def activations(M: int, K: int, outlier_frac: float, seed: int, index: int = 0):
    """BF16 bits [M, K]: N(0,1), then round(frac*M*K) distinct entries scaled x20."""
    r = rng_for(seed, _T_X, index)
    x = r.standard_normal((M, K), dtype=np.float32)
    n_out = int(round(outlier_frac * M * K))
    if n_out:
        idx = r.choice(M * K, size=n_out, replace=False)
        x.reshape(-1)[idx] *= np.float32(20.0)
    return to_bf16_bits(x)


def int8_weight(shape, seed: int, tag: int = _T_W, index: int = 0) -> np.ndarray:
    return rng_for(seed, tag, index).integers(-127, 128, size=shape, dtype=np.int8)


def scales(n, seed: int, tag: int = _T_WS, index: int = 0) -> np.ndarray:
    return rng_for(seed, tag, index).uniform(1e-3, 1e-2, size=n).astype(np.float32)


def bias_bf16(n: int, seed: int, sigma: float = 0.1) -> np.ndarray:
    x = rng_for(seed, _T_B).normal(0.0, sigma, size=n).astype(np.float32)
    return to_bf16_bits(x)


@dataclass
class Dense:
    name: str
    x: np.ndarray            # BF16 bits [M, K]
    w: np.ndarray            # int8 [N, K]
    w_scale: np.ndarray      # f32 [N]
    bias: np.ndarray | None  # BF16 bits [N]

    @property
    def M(self):
        return self.x.shape[0]

    @property
    def K(self):
        return self.x.shape[1]

    @property
    def N(self):
        return self.w.shape[0]


def dense(M: int, K: int, N: int, *, outlier_frac: float, bias: bool, seed: int = 0,
          name: str = "dense") -> Dense:
    return Dense(name, activations(M, K, outlier_frac, seed), int8_weight((N, K), seed),
                 scales(N, seed), bias_bf16(N, seed) if bias else None)


def tiny(seed: int = 0) -> Dense:
    return dense(16, 256, 128, outlier_frac=0.01, bias=True, seed=seed, name="tiny")


def decode(seed: int = 0, M: int = 64) -> Dense:
    d = dense(64, 7168, 4096, outlier_frac=0.005, bias=False, seed=seed, name="decode")
    d.x = d.x[:M].copy()
    return d


def prefill(seed: int = 0, M: int = 8192) -> Dense:
    d = dense(M, 7168, 4096, outlier_frac=0.005, bias=True, seed=seed, name="prefill")
    return d


# ---------------------------------------------------------------------------
# MoE routing inputs
# ---------------------------------------------------------------------------

def topk_routing(T: int, E: int, top_k: int, seed: int, ebias_sigma: float = 1.5):
    """Top-k routing inputs from logits N(0,1) + per-expert bias N(0, sigma).

    Returns (topk_ids int32 [T, top_k], topk_weights float32 [T, top_k]): the
    experts of every token by descending score (ties to the lower id) and
    weights that are the softmax of the chosen scores (an input recipe only).
    """
    logits = rng_for(seed, _T_LOGITS).standard_normal((T, E), dtype=np.float32)
    ebias = rng_for(seed, _T_EBIAS).normal(0.0, ebias_sigma, size=E).astype(np.float32)
    score = logits + ebias[None, :]
    ids = np.argsort(-score, axis=1, kind="stable")[:, :top_k]
    chosen = np.take_along_axis(score, ids, axis=1).astype(np.float64)
    wts = np.exp(chosen - chosen.max(axis=1, keepdims=True))
    wts = (wts / wts.sum(axis=1, keepdims=True)).astype(np.float32)
    return ids.astype(np.int32), wts


def route_topk(T: int, E: int, top_k: int, seed: int, ebias_sigma: float = 1.5):
    """The (token, expert) pairs of ``topk_routing`` grouped by expert, tokens
    ascending inside each expert.
    Returns (row_token [T*k], row_expert [T*k], group_list [E] int64).
    """
    ids, _ = topk_routing(T, E, top_k, seed, ebias_sigma)
    tok = np.repeat(np.arange(T, dtype=np.int64), top_k)
    exp_ = ids.reshape(-1).astype(np.int64)
    perm = np.lexsort((tok, exp_))
    row_token, row_expert = tok[perm], exp_[perm]
    group_list = np.bincount(row_expert, minlength=E).astype(np.int64)
    return row_token, row_expert, group_list


@dataclass
class MoE:
    T: int
    H: int
    I: int
    E: int
    top_k: int
    seed: int
    x_tokens: np.ndarray      # BF16 bits [T, H]
    row_token: np.ndarray     # [R]
    group_list: np.ndarray    # int64 [E]
    w13_scale: np.ndarray     # f32 [E, 2I]
    w2_scale: np.ndarray      # f32 [E, H]
    topk_ids: np.ndarray = None       # int32 [T, top_k]
    topk_weights: np.ndarray = None   # f32 [T, top_k]
    _w13: dict = field(default_factory=dict, repr=False)
    _w2: dict = field(default_factory=dict, repr=False)

    @property
    def R(self):
        return int(self.row_token.shape[0])

    def x_rows(self) -> np.ndarray:
        """Routed hidden rows, grouped by expert: BF16 bits [R, H]."""
        return self.x_tokens[self.row_token]

    def w13(self, e: int) -> np.ndarray:
        """int8 [2I, H] for expert e (drawn on demand from its own stream)."""
        if e not in self._w13:
            self._w13[e] = int8_weight((2 * self.I, self.H), self.seed, _T_W13, e)
        return self._w13[e]

    def w2(self, e: int) -> np.ndarray:
        if e not in self._w2:
            self._w2[e] = int8_weight((self.H, self.I), self.seed, _T_W2, e)
        return self._w2[e]

    def drop_cache(self):
        self._w13.clear()
        self._w2.clear()

    def w13_all(self) -> np.ndarray:
        return np.stack([int8_weight((2 * self.I, self.H), self.seed, _T_W13, e)
                         for e in range(self.E)])

    def w2_all(self) -> np.ndarray:
        return np.stack([int8_weight((self.H, self.I), self.seed, _T_W2, e)
                         for e in range(self.E)])


def moe(T: int = 2048, H: int = 4096, I: int = 2048, E: int = 256, top_k: int = 8,
        seed: int = 0, ebias_sigma: float = 1.5) -> MoE:
    x = activations(T, H, 0.0, seed)
    row_token, _, group_list = route_topk(T, E, top_k, seed, ebias_sigma)
    ids, wts = topk_routing(T, E, top_k, seed, ebias_sigma)
    w13s = np.stack([scales(2 * I, seed, _T_W13S, e) for e in range(E)])
    w2s = np.stack([scales(H, seed, _T_W2S, e) for e in range(E)])
    return MoE(T, H, I, E, top_k, seed, x, row_token, group_list, w13s, w2s, ids, wts)


# ---------------------------------------------------------------------------
# MXFP8 variant inputs
# ---------------------------------------------------------------------------

def e4m3_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> E4M3FN codes with torch's CPU conversion (values must be in range)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


@dataclass
class MX:
    x: np.ndarray            # BF16 bits [M, K]
    w_e4m3: np.ndarray       # uint8 codes [N, K] (block-FP8 checkpoint payload)
    scale_inv: np.ndarray    # f32 [ceil(N/bn), ceil(K/bk)]
    bn: int
    bk: int


def mx_block_fp8(M: int = 2048, N: int = 5120, K: int = 17408, bn: int = 128, bk: int = 128,
                 seed: int = 0) -> MX:
    """MXFP8 workload: E4M3 weight [N, K] = RNE(N(0,1)) with fp32 weight_scale_inv per
    bn x bk tile U[1e-3, 1e-2]; activations BF16 [M, K] N(0,1)."""
    w = e4m3_bits(rng_for(seed, _T_MXW).standard_normal((N, K), dtype=np.float32))
    s = rng_for(seed, _T_MXS).uniform(1e-3, 1e-2, size=(-(-N // bn), -(-K // bk))).astype(np.float32)
    return MX(activations(M, K, 0.0, seed, index=5), w, s, bn, bk)


# ---------------------------------------------------------------------------
# MXFP8 MoE inputs: block-FP8 expert stacks (E4M3 = RNE(N(0,1)), fp32
# weight_scale_inv per bn x bk tile U[1e-3, 1e-2]) on the MoE workload's shapes
# and routing
# ---------------------------------------------------------------------------

@dataclass
class MxMoE:
    T: int
    H: int
    I: int
    E: int
    top_k: int
    seed: int
    bn: int
    bk: int
    x_tokens: np.ndarray      # BF16 bits [T, H]
    row_token: np.ndarray     # [R]
    group_list: np.ndarray    # int64 [E]

    @property
    def R(self):
        return int(self.row_token.shape[0])

    def x_rows(self) -> np.ndarray:
        return self.x_tokens[self.row_token]

    def _block_fp8(self, N, K, tw, ts, e):
        w = e4m3_bits(rng_for(self.seed, tw, e).standard_normal((N, K), dtype=np.float32))
        s = rng_for(self.seed, ts, e).uniform(
            1e-3, 1e-2, size=(-(-N // self.bn), -(-K // self.bk))).astype(np.float32)
        return w, s

    def w13(self, e: int):
        """(E4M3 codes [2I, H], weight_scale_inv) of expert e."""
        return self._block_fp8(2 * self.I, self.H, _T_MXW13, _T_MXS13, e)

    def w2(self, e: int):
        """(E4M3 codes [H, I], weight_scale_inv) of expert e."""
        return self._block_fp8(self.H, self.I, _T_MXW2, _T_MXS2, e)


def mx_moe(T: int = 2048, H: int = 4096, I: int = 2048, E: int = 256, top_k: int = 8,
           seed: int = 0, bn: int = 128, bk: int = 128, ebias_sigma: float = 1.5) -> MxMoE:
    x = activations(T, H, 0.0, seed)
    row_token, _, group_list = route_topk(T, E, top_k, seed, ebias_sigma)
    return MxMoE(T, H, I, E, top_k, seed, bn, bk, x, row_token, group_list)


# ---------------------------------------------------------------------------
# low-bit (INT4 / FP4) expert weights on the MoE workload
# ---------------------------------------------------------------------------

LOWBIT_SIGMA = 0.02


@dataclass
class LowbitMoE:
    T: int
    H: int
    I: int
    E: int
    top_k: int
    seed: int
    x_tokens: np.ndarray      # BF16 bits [T, H]
    row_token: np.ndarray     # [R]
    group_list: np.ndarray    # int64 [E]

    @property
    def R(self):
        return int(self.row_token.shape[0])

    def x_rows(self) -> np.ndarray:
        return self.x_tokens[self.row_token]

    def _w(self, N, K, tag, e):
        r = rng_for(self.seed, tag, e)
        return to_bf16_bits(r.standard_normal((N, K), dtype=np.float32) * np.float32(LOWBIT_SIGMA))

    def w13(self, e: int) -> np.ndarray:
        """BF16 bits [2I, H] of expert e."""
        return self._w(2 * self.I, self.H, _T_LBW13, e)

    def w2(self, e: int) -> np.ndarray:
        """BF16 bits [H, I] of expert e."""
        return self._w(self.H, self.I, _T_LBW2, e)


def lowbit_moe(T: int = 2048, H: int = 4096, I: int = 2048, E: int = 256, top_k: int = 8,
               seed: int = 0, ebias_sigma: float = 1.5) -> LowbitMoE:
    x = activations(T, H, 0.0, seed)
    row_token, _, group_list = route_topk(T, E, top_k, seed, ebias_sigma)
    return LowbitMoE(T, H, I, E, top_k, seed, x, row_token, group_list)
