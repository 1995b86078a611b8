#!/usr/bin/env python3
"""Benchmark of the W8A8_DYNAMIC hot path on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload default|decode|prefill|moe|...]

Prints ONE JSON line. A step is one pass of the workload's whole hot path over
resident, seeded synthetic inputs. The default run reports the decode workload
as the headline (value, roofline, cpu_baseline) and, as nested objects under
"also" (each with its own value, ms_per_step, roofline and cpu_baseline), the
metric's other two parts, prefill TOPS and MoE tokens/s, plus the MXFP8
linear (TFLOPS) and the tiny latency case.
  decode   per-token quant + INT8 linear for M = 1, 4, 16 and 64 rows,
           K = 7168, N = 4096, no bias. Sixteen copies of the packed weight
           (16 x 29.4 MB) are used round-robin so that no weight read is served
           by the 256 MB MALL: every step reads its weights from HBM.
           value = algorithmic HBM bytes of the step / step time (GB/s).
  prefill  quant + INT8 linear, M = 8192, K = 7168, N = 4096, bias.
           value = 2*M*N*K / step time (TOPS).
  moe      quant -> W13 grouped GEMM -> SwiGLU + requant -> W2 grouped GEMM for
           T = 2048 tokens routed top-8 over 256 experts, H = 4096, I = 2048.
           value = tokens / step time (tokens/s).
  tiny     quant + INT8 linear, 16 x 256 x 128 with bias (latency case).
  mx       MXFP8 linear: dynamic MX quant of BF16 activations [2048, 17408] +
           block-scaled E4M3 GEMM against a weight [5120, 17408] that was
           resolved from 128 x 128-tile block FP8 and MX-requantized at load
           time (load-time prep timed once and reported in config).
           value = 2*M*N*K / step time (TFLOPS).
  copy     a plain 512 MiB device-to-device copy (torch's copy kernel): the
           measured HBM ceiling, and the reference dispatch that scales the
           FETCH_SIZE / WRITE_SIZE counters (it moves exactly 2 x 512 MiB).

Consecutive steps are captured as HIP graphs of G steps each (the C ABI calls
only enqueue kernels) and replayed, so host-side Python does not pace the GPU:
G = gcd(16, K, W), so the K timed steps are exactly K / G replays (16 with the
default K = 256, W = 32). Every step in a graph repeats the whole path; on this
GPU each graph boundary costs several microseconds of device time (decode
step 47.7 us at one step per graph against 41.7 us at 16), which a serving
loop that captures whole forward passes does not pay per layer. The average
duration of the dominant kernel comes from HIP events recorded around graphs
that hold only its launches, on the same stream.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_INT8_TOPS = 5000.0        # MI355X dense INT8 MFMA, TOP/s
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense BF16 MFMA, TFLOP/s (the MX GEMM's MFMA: it
                               # multiplies the exactly dequantized E4M3 values in BF16)
BYTES_INT8 = 1


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--workload", default="default",
                    choices=["default", "decode", "prefill", "moe", "moe_layer", "tiny", "copy", "mx",
                             "mx_moe", "static", "w4a16", "fp4", "w4a16_moe", "fp4_moe"])
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="approximate budget of the oracle timing on the host")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------

class Workload:
    """Step graphs (each holding G consecutive steps; a workload with P phases,
    e.g. rotating weight copies, runs phase i % P at step i) and, separately,
    graphs holding only launches of the dominant kernel, for its event timing."""
    name = ""
    metric = "W8A8 linear TOPS and HBM GB/s (% of peak); MoE grouped-GEMM tokens/s"
    unit = ""
    bound = "hbm"

    def __init__(self, w, torch):
        self.w = w
        self.torch = torch
        self.phases = []          # step graphs
        self.dominant_graphs = []  # (graph, launches per replay, key)

    def _graph(self, fn):
        torch = self.torch
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()                  # eager run outside capture
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        return g

    def capture(self, step_fns, dominant):
        """step_fns: callables enqueuing one step each (phase i at step i %
        len); dominant: (callable, launches, key) triples enqueuing only
        dominant-kernel launches."""
        self.step_fns = list(step_fns)
        self.dominant_graphs = [(self._graph(fn), n, key) for fn, n, key in dominant]

    def group_steps(self, g):
        """Capture the steps in graphs of g consecutive steps: graph j holds
        steps j*g .. j*g + g - 1 (mod the phase cycle)."""
        self.g = g
        self.phases = []
        for plan in graph_plan(len(self.step_fns), g):
            fns = [self.step_fns[k] for k in plan]
            self.phases.append(self._graph(lambda fns=fns: [f() for f in fns]))

    def step(self, i):
        """Step i; the graph of its group is replayed at the group's last step."""
        if i % self.g == self.g - 1:
            self.phases[(i // self.g) % len(self.phases)].replay()


def graph_plan(P, g):
    """Phases held by each step graph when P phases cycle (phase i % P at step
    i) and every graph holds g consecutive steps: graph j covers steps j*g ..
    j*g + g - 1, and replaying graphs 0, 1, .. in turn (wrapping) runs every
    step's own phase."""
    n = P // math.gcd(P, g)
    return [[(j * g + t) % P for t in range(g)] for j in range(n)]


def steps_per_graph(steps, warmup):
    """Steps per captured graph: a divisor of both counts (at most 16), so the
    warm-up and the timed region are whole graph replays."""
    return math.gcd(16, steps, warmup) if warmup else math.gcd(16, steps)


def _ev(torch):
    return torch.cuda.Event(enable_timing=True)


class DenseWorkload(Workload):
    def __init__(self, w, torch, name, Ms, K, N, bias, outlier, copies):
        super().__init__(w, torch)
        import numpy as np

        import synth
        self.name, self.Ms, self.K, self.N = name, list(Ms), K, N
        self.has_bias = bias
        self.copies = copies
        Mmax = max(self.Ms)
        if name == "decode":
            d = synth.decode(seed=0, M=Mmax)
        elif name == "prefill":
            d = synth.prefill(seed=0)
        elif name == "tiny":
            d = synth.tiny(seed=0)
        else:
            d = synth.dense(Mmax, K, N, outlier_frac=outlier, bias=bias, seed=0, name=name)
        self.d = d
        dev = "cuda"
        self.x = torch.from_numpy(d.x.view(np.int16)).to(dev).view(torch.bfloat16)
        self.w_scale = torch.from_numpy(d.w_scale).to(dev)
        self.bias = (torch.from_numpy(d.bias.view(np.int16)).to(dev).view(torch.bfloat16)
                     if d.bias is not None else None)
        packed = w.prepack_weight(torch.from_numpy(d.w).to(dev))
        nb = packed.numel()
        self.wp = torch.empty((copies, nb), dtype=torch.uint8, device=dev)
        for c in range(copies):
            self.wp[c].copy_(packed)
        del packed
        # codes in the packed block layout from 16 rows up (whole 1 KB blocks per
        # 16 rows); below that the row-major codes read fewer bytes
        self.packed = {M: M >= 16 and K % 8 == 0 for M in self.Ms}
        # BF16 straight into linear where it quantizes inside the product kernel
        # (every workgroup quantizes the rows again: up to 16 rows of at most
        # 16384 values, K % 8 == 0)
        self.fused = {M: (M <= 2 or (M <= 16 and M * K <= 16384)) and K <= 16384 and K % 8 == 0
                      for M in self.Ms}
        self.q = {M: (torch.empty((w.packed_weight_bytes(1, M, K),), dtype=torch.uint8, device=dev)
                      if self.packed[M] else torch.empty((M, K), dtype=torch.int8, device=dev))
                  for M in self.Ms}
        self.s = {M: torch.empty((M,), dtype=torch.float32, device=dev) for M in self.Ms}
        self.y = {M: torch.empty((M, N), dtype=torch.bfloat16, device=dev) for M in self.Ms}
        self.ws = {M: torch.empty((max(1, w.linear_workspace_bytes(M, N, K)),), dtype=torch.uint8,
                                  device=dev) for M in self.Ms}
        # round-robin over weight copies: phase p uses copies p*len(Ms) + j
        per = len(self.Ms)
        nphase = max(1, copies // per)
        steps = [self._make_step([(p * per + j) % copies for j in range(per)])
                 for p in range(nphase)]
        # at least 16 launches per timing graph, so that the graph launch itself
        # does not enter the per-kernel time
        nl = max(copies, 16)
        dom = [(self._make_linears(M, nl), nl, M) for M in self.Ms]
        self.capture(steps, dom)
        self.unit = "GB/s" if name != "prefill" else "TOPS"
        self.bound = "hbm" if name != "prefill" else "mfma"

    def _linear(self, M, c):
        if self.fused[M]:
            self.w.linear_bf16(self.x[:M], self.wp[c], self.w_scale, self.N, bias=self.bias,
                               y=self.y[M], workspace=self.ws[M])
        elif self.packed[M]:
            self.w.linear_packed(self.q[M], self.s[M], self.K, self.wp[c], self.w_scale, self.N,
                                 bias=self.bias, y=self.y[M], workspace=self.ws[M])
        else:
            self.w.linear(self.q[M], self.s[M], self.wp[c], self.w_scale, self.N, bias=self.bias,
                          y=self.y[M], workspace=self.ws[M])

    def _quant(self, M):
        if self.fused[M]:
            return  # inside the linear
        if self.packed[M]:
            self.w.dynamic_quant_packed(self.x[:M], self.q[M], self.s[M])
        else:
            self.w.dynamic_quant(self.x[:M], self.q[M], self.s[M])

    def _make_step(self, copy_ids):
        def fn():
            for M, c in zip(self.Ms, copy_ids):
                self._quant(M)
                self._linear(M, c)
        return fn

    def _make_linears(self, M, n):
        def fn():
            for i in range(n):
                self._linear(M, i % self.copies)
        return fn

    # algorithmic bytes / ops
    def gemm_bytes(self, M):
        """One dominant launch: weight + scales, activation in (BF16 for the fused
        quant, else INT8 codes + scales), BF16 out (+ bias)."""
        a_in = 2 * M * self.K if self.fused[M] else M * self.K + 4 * M
        b = self.N * self.K * BYTES_INT8 + 4 * self.N + a_in + 2 * M * self.N
        if self.has_bias:
            b += 2 * self.N
        return b

    def alg_bytes(self):
        """Algorithmic bytes of the dominant unit (the GEMM launches of one step)."""
        return sum(self.gemm_bytes(M) for M in self.Ms)

    def step_bytes(self):
        """External operands of the step: BF16 activations in, weight + scales
        (+ bias), BF16 out, per M (the INT8 codes are an internal intermediate)."""
        b = 0
        for M in self.Ms:
            b += 2 * M * self.K + self.N * self.K * BYTES_INT8 + 4 * self.N + 2 * M * self.N
            if self.has_bias:
                b += 2 * self.N
        return b

    def step_ops(self):
        return sum(2 * M * self.N * self.K for M in self.Ms)

    def value(self, sec_per_step):
        if self.unit == "TOPS":
            return self.step_ops() / sec_per_step / 1e12
        return self.step_bytes() / sec_per_step / 1e9

    def dominant(self, per_key_ms):
        """Roofline of the linear kernel(s): per launch algorithmic bytes / ops."""
        tot_ms = sum(per_key_ms[M] for M in self.Ms)
        if self.bound == "mfma":
            ops = sum(2 * M * self.N * self.K for M in self.Ms)
            ach = ops / (tot_ms * 1e-3) / 1e12
            return dict(bound="mfma", achieved=ach, peak=PEAK_INT8_TOPS, unit="TOP/s",
                        frac=ach / PEAK_INT8_TOPS)
        byts = sum(self.gemm_bytes(M) for M in self.Ms)
        ach = byts / (tot_ms * 1e-3) / 1e9
        return dict(bound="hbm", achieved=ach, peak=PEAK_HBM_GBS, unit="GB/s",
                    frac=ach / PEAK_HBM_GBS)

    def config(self):
        c = {"workload": self.name, "M": self.Ms if len(self.Ms) > 1 else self.Ms[0], "K": self.K,
             "N": self.N, "bias": self.has_bias, "weight_copies": self.copies,
             "packed_codes_for_M": [M for M in self.Ms if self.packed[M]],
             "fused_quant_for_M": [M for M in self.Ms if self.fused[M]],
             "x": "N(0,1) with outliers x20", "w": "int8 uniform [-127,127]"}
        return c

    def cpu_baseline(self, budget_s):
        import oracle as O
        d = self.d
        if self.name == "prefill":
            rows = 128
            xs = d.x[:rows]
            t0 = time.perf_counter()
            n = 0
            while True:
                q, s = O.dynamic_quant(xs)
                O.linear(q, s, d.w, d.w_scale, d.bias)
                n += 1
                if time.perf_counter() - t0 > budget_s:
                    break
            dt = (time.perf_counter() - t0) / n
            ops = 2 * rows * self.N * self.K
            return dict(value=ops / dt / 1e12, unit="TOPS",
                        sample=f"oracle quant + linear on the first {rows} of 8192 rows "
                               f"({n} repetitions), full N and K")
        t0 = time.perf_counter()
        n = 0
        while True:
            for M in self.Ms:
                q, s = O.dynamic_quant(d.x[:M])
                O.linear(q, s, d.w, d.w_scale, d.bias)
            n += 1
            if time.perf_counter() - t0 > budget_s:
                break
        dt = (time.perf_counter() - t0) / n
        return dict(value=self.step_bytes() / dt / 1e9, unit="GB/s",
                    sample=f"oracle quant + linear for every M of the step, {n} full steps")


class MoeWorkload(Workload):
    def __init__(self, w, torch):
        super().__init__(w, torch)
        import numpy as np

        import synth
        self.name = "moe"
        m = synth.moe(seed=0)
        self.m = m
        E, H, I = m.E, m.H, m.I
        dev = "cuda"
        per13 = w.packed_weight_bytes(1, 2 * I, H)
        per2 = w.packed_weight_bytes(1, H, I)
        self.w13p = torch.empty((E * per13,), dtype=torch.uint8, device=dev)
        self.w2p = torch.empty((E * per2,), dtype=torch.uint8, device=dev)
        for e in range(E):
            w.prepack_weight(torch.from_numpy(m.w13(e)).to(dev), out=self.w13p[e * per13:(e + 1) * per13])
            w.prepack_weight(torch.from_numpy(m.w2(e)).to(dev), out=self.w2p[e * per2:(e + 1) * per2])
            m.drop_cache()
        self.w13s = torch.from_numpy(m.w13_scale).to(dev)
        self.w2s = torch.from_numpy(m.w2_scale).to(dev)
        self.gl = torch.from_numpy(m.group_list).to(dev)
        self.x = torch.from_numpy(m.x_rows().view(np.int16)).to(dev).view(torch.bfloat16)
        R = m.R
        self.y = torch.empty((R, H), dtype=torch.bfloat16, device=dev)
        self.ws = torch.empty((w.moe_workspace_bytes(R, E, H, I),), dtype=torch.uint8, device=dev)
        # sub-stage buffers for the per-kernel timing phase
        self.q1 = torch.empty((R, H), dtype=torch.int8, device=dev)
        self.s1 = torch.empty((R,), dtype=torch.float32, device=dev)
        self.h = torch.empty((R, 2 * I), dtype=torch.bfloat16, device=dev)
        self.q2 = torch.empty((R, I), dtype=torch.int8, device=dev)
        self.s2 = torch.empty((R,), dtype=torch.float32, device=dev)
        self.unit = "tokens/s"
        self.bound = "hbm"
        self.capture([self._step], [(self._w13, 1, "w13"), (self._w2, 1, "w2")])

    def _step(self):
        """Same kernels as moe_grouped, through the sub-stage entry points."""
        w = self.w
        w.dynamic_quant(self.x, self.q1, self.s1)
        self._w13()
        w.swiglu_quant(self.h, self.q2, self.s2)
        self._w2()

    def _w13(self):
        self.w.grouped_gemm(self.q1, self.s1, self.gl, self.w13p, self.w13s, 2 * self.m.I, y=self.h)

    def _w2(self):
        self.w.grouped_gemm(self.q2, self.s2, self.gl, self.w2p, self.w2s, self.m.H, y=self.y)

    def nonempty(self):
        return int((self.m.group_list > 0).sum())

    def gemm_bytes(self, which):
        m = self.m
        ne = self.nonempty()
        R, H, I = m.R, m.H, m.I
        if which == "w13":
            return ne * (2 * I * H + 4 * 2 * I) + R * H + 4 * R + 2 * R * 2 * I + 8 * m.E
        return ne * (H * I + 4 * H) + R * I + 4 * R + 2 * R * H + 8 * m.E

    def alg_bytes(self):
        return self.gemm_bytes("w13") + self.gemm_bytes("w2")

    def value(self, sec_per_step):
        return self.m.T / sec_per_step

    def dominant(self, per_key_ms):
        byts = self.gemm_bytes("w13") + self.gemm_bytes("w2")
        tot = per_key_ms["w13"] + per_key_ms["w2"]
        ach = byts / (tot * 1e-3) / 1e9
        return dict(bound="hbm", achieved=ach, peak=PEAK_HBM_GBS, unit="GB/s",
                    frac=ach / PEAK_HBM_GBS)

    def config(self):
        m = self.m
        g = m.group_list
        return {"workload": "moe", "T": m.T, "top_k": m.top_k, "E": m.E, "H": m.H, "I": m.I,
                "R": m.R, "nonempty_experts": self.nonempty(), "max_rows_per_expert": int(g.max()),
                "experts_le4_rows": int(((g > 0) & (g <= 4)).sum()),
                "routing": "logits N(0,1) + expert bias N(0,1.5), top-8"}

    def cpu_baseline(self, budget_s):
        import numpy as np

        import oracle as O
        m = self.m
        off = O.group_offsets(m.group_list)
        xr = m.x_rows()
        t0 = time.perf_counter()
        rows = 0
        e = 0
        while time.perf_counter() - t0 < budget_s and e < m.E:
            a, b = int(off[e]), int(off[e + 1])
            if b > a:
                g1 = np.array([b - a], np.int64)
                O.moe_grouped(g1, m.w13(e)[None], m.w13_scale[e][None], m.w2(e)[None],
                              m.w2_scale[e][None], x_bits=xr[a:b])
                m.drop_cache()
                rows += b - a
            e += 1
        dt = time.perf_counter() - t0
        return dict(value=rows / m.top_k / dt, unit="tokens/s",
                    sample=f"oracle MoE chain over experts 0..{e - 1} ({rows} of {m.R} rows, "
                           f"weights drawn per expert inside the timing), tokens = rows / top_k")


class MoeLayerWorkload(MoeWorkload):
    """The MoE workload as a whole layer: BF16 tokens in, BF16 tokens out
    (quantize once, route, gather, W13 -> SwiGLU + requant -> W2, combine)."""

    def __init__(self, w, torch):
        super().__init__(w, torch)
        m = self.m
        self.name = "moe_layer"
        E, H, I, T, k = m.E, m.H, m.I, m.T, m.top_k
        dev = "cuda"
        self.xt = torch.from_numpy(m.x_tokens.view("int16")).to(dev).view(torch.bfloat16)
        self.ids = torch.from_numpy(m.topk_ids).to(dev)
        self.wts = torch.from_numpy(m.topk_weights).to(dev)
        self.out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        self.lws = torch.empty((w.moe_layer_workspace_bytes(T, k, E, H, I),), dtype=torch.uint8,
                               device=dev)
        # sub-stage buffers for the per-kernel timing of the steps around the chain
        self.gl2 = torch.empty((E,), dtype=torch.int64, device=dev)
        self.rt = torch.empty((T * k,), dtype=torch.int32, device=dev)
        self.pr = torch.empty((T, k), dtype=torch.int32, device=dev)
        self.qt = torch.empty((T, H), dtype=torch.int8, device=dev)
        self.st = torch.empty((T,), dtype=torch.float32, device=dev)
        self.phases, self.dominant_graphs = [], []
        # the short kernels are timed 16 launches per graph, so that the graph
        # launch itself does not enter their per-kernel time
        def rep(fn, n=16):
            def run():
                for _ in range(n):
                    fn()
            return run
        self.capture([self._layer], [(self._w13, 1, "w13"), (self._w2, 1, "w2"),
                                     (rep(self._route), 16, "route"),
                                     (rep(self._gather), 16, "gather"),
                                     (rep(self._combine), 16, "combine")])

    def _layer(self):
        self.w.moe_layer(self.xt, self.ids, self.wts, self.w13p, self.w13s, self.w2p, self.w2s,
                         out=self.out, workspace=self.lws)

    def _route(self):
        self.w.moe_route(self.ids, self.m.E, self.gl2, self.rt, self.pr)

    def _gather(self):
        self.w.moe_gather(self.qt, self.st, self.rt, self.q1, self.s1)

    def _combine(self):
        self.w.moe_combine(self.y, self.pr, self.wts, out=self.out)

    def alg_bytes(self):
        """Whole layer: the two grouped GEMMs plus token quant (BF16 in, INT8 +
        scale out), route (ids in; counts, rows and pair rows out), gather (INT8
        rows and scales in and out) and combine (BF16 rows and weights in, BF16
        tokens out)."""
        m = self.m
        T, k, H, R = m.T, m.top_k, m.H, m.R
        quant = T * H * 2 + T * H + 4 * T
        route = 4 * T * k + 8 * m.E + 4 * R + 4 * T * k
        gather = 4 * R + (R * H + 4 * R) * 2
        combine = 4 * T * k * 2 + 2 * R * H + 2 * T * H
        return super().alg_bytes() + quant + route + gather + combine

    def config(self):
        c = super().config()
        c["workload"] = "moe_layer"
        c["combine"] = "topk_weights = softmax of the chosen routing scores"
        return c

    def cpu_baseline(self, budget_s):
        import numpy as np

        import oracle as O
        m = self.m
        IO = O.moe_io
        t0 = time.perf_counter()
        gl, rt, pr = IO.route(m.topk_ids, m.E)
        IO.dispatch_int8(m.x_tokens, rt)
        y = np.zeros((m.R, m.H), np.uint16)
        IO.combine(y, pr, m.topk_weights)
        t_io = time.perf_counter() - t0
        chain = MoeWorkload.cpu_baseline(self, max(1.0, budget_s - t_io))
        t_chain = m.top_k / chain["value"] * m.T          # oracle chain time for all R rows
        return dict(value=m.T / (t_io + t_chain), unit="tokens/s",
                    sample=f"oracle route + INT8 dispatch + combine over all {m.T} tokens "
                           f"({t_io:.2f} s), plus the " + chain["sample"] +
                           ", scaled to all rows")


class MxMoeWorkload(Workload):
    """The MoE workload with MXFP8 experts: block-FP8 source weights prepared
    one expert at a time (resolve -> MX requant over the source bytes ->
    kernel layout), then the MX chain on the expert-grouped rows."""

    def __init__(self, w, torch):
        super().__init__(w, torch)
        import numpy as np

        import synth
        self.name = "mx_moe"
        m = synth.mx_moe(seed=0)
        self.m = m
        E, H, I = m.E, m.H, m.I
        dev = "cuda"
        s13 = w.mx_moe_packed_bytes(1, 2 * I, H)
        s2 = w.mx_moe_packed_bytes(1, H, I)
        self.w13p = torch.empty((E * s13,), dtype=torch.uint8, device=dev)
        self.w2p = torch.empty((E * s2,), dtype=torch.uint8, device=dev)
        st = torch.empty((w.mx_moe_staging_bytes(2 * I, H),), dtype=torch.uint8, device=dev)
        prep_ms = 0.0
        for e in range(E):
            (wa, sa), (wb, sb) = m.w13(e), m.w2(e)
            a_d, sa_d = torch.from_numpy(wa[None]).to(dev), torch.from_numpy(sa[None]).to(dev)
            b_d, sb_d = torch.from_numpy(wb[None]).to(dev), torch.from_numpy(sb[None]).to(dev)
            torch.cuda.synchronize()
            a, b = _ev(torch), _ev(torch)
            a.record()
            w.mx_moe_prepare(a_d, sa_d, m.bn, m.bk, packed=self.w13p[e * s13:(e + 1) * s13], staging=st)
            w.mx_moe_prepare(b_d, sb_d, m.bn, m.bk, packed=self.w2p[e * s2:(e + 1) * s2], staging=st)
            b.record()
            torch.cuda.synchronize()
            prep_ms += a.elapsed_time(b)
            if (e + 1) % 32 == 0:
                print(f"mx_moe: {e + 1} of {E} experts prepared", file=sys.stderr, flush=True)
        self.prep_ms = prep_ms
        del st
        self.gl = torch.from_numpy(m.group_list).to(dev)
        self.x = torch.from_numpy(m.x_rows().view(np.int16)).to(dev).view(torch.bfloat16)
        R = m.R
        self.y = torch.empty((R, H), dtype=torch.bfloat16, device=dev)
        self.h = torch.empty((R, 2 * I), dtype=torch.bfloat16, device=dev)
        self.ws = torch.empty((w.mx_moe_workspace_bytes(R, E, H, I),), dtype=torch.uint8, device=dev)
        self.ws13 = torch.empty((w.mx_grouped_workspace_bytes(R, E, H),), dtype=torch.uint8, device=dev)
        self.ws2 = torch.empty((w.mx_grouped_workspace_bytes(R, E, I),), dtype=torch.uint8, device=dev)
        self.unit = "tokens/s"
        self.bound = "hbm"
        self.capture([self._step], [(self._w13, 1, "w13"), (self._w2, 1, "w2")])

    def _step(self):
        self.w.mx_moe_grouped(self.x, self.gl, self.w13p, self.w2p, self.m.I, y=self.y,
                              workspace=self.ws)

    def _w13(self):
        self.w.mx_grouped_gemm(self.x, self.gl, self.w13p, 2 * self.m.I, y=self.h,
                               workspace=self.ws13)

    def _w2(self):
        self.w.mx_grouped_gemm(self.h, self.gl, self.w2p, self.m.H, act=self.w.ACT_SWIGLU,
                               y=self.y, workspace=self.ws2)

    def nonempty(self):
        return int((self.m.group_list > 0).sum())

    def stage_bytes(self, which):
        """One grouped call: the non-empty experts' MX weights (1 byte per value +
        1 scale byte per 32), the BF16 input rows (h: gate and up), the MX
        activation written and read back, the BF16 output."""
        m = self.m
        ne = self.nonempty()
        R, H, I = m.R, m.H, m.I
        if which == "w13":
            N, K, kin = 2 * I, H, H
        else:
            N, K, kin = H, I, 2 * I
        wbytes = ne * N * (K + K // 32)
        act = R * (K + K // 32)
        return wbytes + 2 * R * kin + 2 * act + 2 * R * N

    def alg_bytes(self):
        return self.stage_bytes("w13") + self.stage_bytes("w2")

    def value(self, sec_per_step):
        return self.m.T / sec_per_step

    def dominant(self, per_key_ms):
        byts = self.alg_bytes()
        tot = per_key_ms["w13"] + per_key_ms["w2"]
        ach = byts / (tot * 1e-3) / 1e9
        return dict(bound="hbm", achieved=ach, peak=PEAK_HBM_GBS, unit="GB/s",
                    frac=ach / PEAK_HBM_GBS)

    def config(self):
        m = self.m
        g = m.group_list
        return {"workload": "mx_moe", "T": m.T, "top_k": m.top_k, "E": m.E, "H": m.H, "I": m.I,
                "R": m.R, "nonempty_experts": self.nonempty(), "max_rows_per_expert": int(g.max()),
                "weights": "block-FP8 E4M3 RNE(N(0,1)), weight_scale_inv per 128x128 U[1e-3,1e-2], "
                           "prepared one expert at a time",
                "weight_prep_ms": round(self.prep_ms, 2),
                "routing": "logits N(0,1) + expert bias N(0,1.5), top-8"}

    def cpu_baseline(self, budget_s):
        import numpy as np

        import oracle as O
        m = self.m
        off = O.group_offsets(m.group_list)
        xr = m.x_rows()
        t0 = time.perf_counter()
        rows = 0
        e = 0
        while time.perf_counter() - t0 < budget_s and e < m.E:
            a, b = int(off[e]), int(off[e + 1])
            if b > a:
                (wa, sa), (wb, sb) = m.w13(e), m.w2(e)
                o13 = O.mx_moe.mx_moe_prepare(wa[None], sa[None], m.bn, m.bk)
                o2 = O.mx_moe.mx_moe_prepare(wb[None], sb[None], m.bn, m.bk)
                O.mx_moe.mx_moe_grouped(np.array([b - a], np.int64), xr[a:b], *o13, *o2)
                rows += b - a
            e += 1
        dt = time.perf_counter() - t0
        return dict(value=rows / m.top_k / dt, unit="tokens/s",
                    sample=f"oracle MX chain over experts 0..{e - 1} ({rows} of {m.R} rows, "
                           f"weights drawn and prepared per expert inside the timing), "
                           f"tokens = rows / top_k")


class W4Workload(Workload):
    """The decode-shaped linear with W4A16 weights: X BF16 [M, 7168] for M in 1,
    4, 16, 64 (0.5 % x20 outliers), the weight [4096, 7168] INT4 per 32 input
    channels with BF16 scales (fmt "int4") or FP4 E2M1 with an E8M0 scale per 32
    (fmt "fp4"), rotated over 32 packed copies (past the MALL)."""
    Ms = (1, 4, 16, 64)

    def __init__(self, w, torch, fmt="int4"):
        super().__init__(w, torch)
        import numpy as np

        import synth
        self.fmt = fmt
        self.name = "w4a16" if fmt == "int4" else "fp4"
        d = synth.decode(seed=0)
        self.K, self.N = d.x.shape[1], 4096
        dev = "cuda"
        r = np.random.default_rng([0, 44])
        wf = r.standard_normal((self.N, self.K)).astype(np.float32) * \
            r.uniform(0.005, 0.05, (self.N, 1)).astype(np.float32)
        wb = torch.from_numpy(synth.to_bf16_bits(wf).view(np.int16)).to(dev).view(torch.bfloat16)
        quant = w.w4a16_quant_weight if fmt == "int4" else w.fp4_quant_weight
        _, _, packed = quant(wb)
        del wb
        self.copies = 32
        self.wp = torch.empty((self.copies, packed.numel()), dtype=torch.uint8, device=dev)
        for c in range(self.copies):
            self.wp[c].copy_(packed)
        del packed
        self.x = torch.from_numpy(d.x.view(np.int16)).to(dev).view(torch.bfloat16)
        self.y = {M: torch.empty((M, self.N), dtype=torch.bfloat16, device=dev) for M in self.Ms}
        self.ws = {M: torch.empty((max(1, w.w4a16_linear_workspace_bytes(M, self.K)),), dtype=torch.uint8,
                                  device=dev) for M in self.Ms}
        per = len(self.Ms)
        steps = [self._make_step([(p * per + j) % self.copies for j in range(per)])
                 for p in range(self.copies // per)]
        self.capture(steps, [(self._make_linears(M, self.copies), self.copies, M) for M in self.Ms])
        self.unit = "GB/s"
        self.bound = "hbm"

    def _linear(self, M, c):
        lin = self.w.w4a16_linear if self.fmt == "int4" else self.w.fp4_linear
        lin(self.x[:M], self.wp[c], self.N, y=self.y[M], workspace=self.ws[M])

    def _make_step(self, copy_ids):
        def fn():
            for M, c in zip(self.Ms, copy_ids):
                self._linear(M, c)
        return fn

    def _make_linears(self, M, n):
        def fn():
            for i in range(n):
                self._linear(M, i % self.copies)
        return fn

    def gemm_bytes(self, M):
        """One launch: 4-bit codes (N K / 2) + scales (BF16: 2 N K / 32; E8M0:
        N K / 32), BF16 x in, BF16 y out."""
        sbytes = 2 if self.fmt == "int4" else 1
        return self.N * self.K // 2 + sbytes * self.N * self.K // 32 + 2 * M * self.K + 2 * M * self.N

    def alg_bytes(self):
        return sum(self.gemm_bytes(M) for M in self.Ms)

    def value(self, sec_per_step):
        return self.alg_bytes() / sec_per_step / 1e9

    def dominant(self, per_key_ms):
        tot_ms = sum(per_key_ms[M] for M in self.Ms)
        ach = self.alg_bytes() / (tot_ms * 1e-3) / 1e9
        return dict(bound="hbm", achieved=ach, peak=PEAK_HBM_GBS, unit="GB/s", frac=ach / PEAK_HBM_GBS)

    def config(self):
        fmt = ("INT4 per 32 input channels, BF16 scale = amax / 7" if self.fmt == "int4" else
               "FP4 E2M1 per 32 input channels, E8M0 scale 2^(floor(log2 amax) - 2)")
        return {"workload": self.name, "M": list(self.Ms), "K": self.K, "N": self.N,
                "weight": "BF16 N(0,1) x per-row U[0.005, 0.05] -> " + fmt, "copies": self.copies}

    def cpu_baseline(self, budget_s):
        import numpy as np

        import oracle as O
        import synth
        d = synth.decode(seed=0)
        r = np.random.default_rng([0, 44])
        wf = r.standard_normal((self.N, self.K)).astype(np.float32) * \
            r.uniform(0.005, 0.05, (self.N, 1)).astype(np.float32)
        if self.fmt == "int4":
            q, s = O.w4a16.w4_quant(synth.to_bf16_bits(wf))
            ref = O.w4a16.w4a16_linear_ref64
        else:
            q, s = O.w4a16.fp4_quant(synth.to_bf16_bits(wf))
            ref = O.w4a16.fp4_linear_ref64
        t0 = time.perf_counter()
        n = 0
        while time.perf_counter() - t0 < budget_s:
            for M in self.Ms:
                ref(d.x[:M], q, s)
            n += 1
        dt = (time.perf_counter() - t0) / n
        return dict(value=self.alg_bytes() / dt / 1e9, unit="GB/s",
                    sample=f"oracle dequantization + float64 product of the 4 decode linears, "
                           f"{n} whole steps (weight quantized outside the timing)")


class LowbitMoeWorkload(Workload):
    """The MoE workload (2048 tokens, top-8 of 256 experts, H 4096, I 2048,
    skewed routing) with low-bit expert weights: BF16 N(0, 0.02^2) drawn on the
    device from a seeded generator, quantized at load time to INT4 (BF16 scale
    per 32) or FP4 (E8M0 scale per 32). Step = the chain W13 -> BF16 SwiGLU ->
    W2 on the expert-grouped BF16 rows."""

    def __init__(self, w, torch, fmt="int4"):
        super().__init__(w, torch)
        import numpy as np

        import synth
        self.fmt = fmt
        self.code = w.LOWBIT_INT4 if fmt == "int4" else w.LOWBIT_FP4
        self.name = "w4a16_moe" if fmt == "int4" else "fp4_moe"
        m = synth.lowbit_moe(seed=0)
        self.m = m
        E, H, I = m.E, m.H, m.I
        dev = "cuda"
        quant = w.w4a16_quant_weight if fmt == "int4" else w.fp4_quant_weight
        nbytes = w.w4a16_packed_bytes if fmt == "int4" else w.fp4_packed_bytes
        self.b13, self.b2 = nbytes(2 * I, H), nbytes(H, I)
        self.w13p = torch.empty((E * self.b13,), dtype=torch.uint8, device=dev)
        self.w2p = torch.empty((E * self.b2,), dtype=torch.uint8, device=dev)
        gen = torch.Generator(device=dev)
        gen.manual_seed(0)
        chunk = 16   # experts per quantization call (a 512 MiB BF16 stack)
        for e0 in range(0, E, chunk):
            for N, K, buf, b in ((2 * I, H, self.w13p, self.b13), (H, I, self.w2p, self.b2)):
                wb = (torch.randn((chunk * N, K), generator=gen, device=dev) * synth.LOWBIT_SIGMA).to(torch.bfloat16)
                _, _, pk = quant(wb)
                buf[e0 * b:(e0 + chunk) * b].copy_(pk[:chunk * b])
                del wb, pk
        self.gl = torch.from_numpy(m.group_list).to(dev)
        self.x = torch.from_numpy(m.x_rows().view(np.int16)).to(dev).view(torch.bfloat16)
        R = m.R
        self.y = torch.empty((R, H), dtype=torch.bfloat16, device=dev)
        self.h = torch.empty((R, 2 * I), dtype=torch.bfloat16, device=dev)
        self.a = torch.empty((R, I), dtype=torch.bfloat16, device=dev)
        self.ws = torch.empty((w.w4a16_moe_workspace_bytes(R, H, I),), dtype=torch.uint8, device=dev)
        self.unit = "tokens/s"
        self.bound = "mfma"
        self.capture([self._step], [(self._w13, 1, "w13"), (self._w2, 1, "w2")])

    def _step(self):
        self.w.w4a16_moe_grouped(self.x, self.gl, self.w13p, self.w2p, self.m.I, fmt=self.code, y=self.y,
                                 workspace=self.ws)

    def _w13(self):
        self.w.w4a16_grouped_gemm(self.x, self.gl, self.w13p, 2 * self.m.I, fmt=self.code, y=self.h)

    def _w2(self):
        self.w.w4a16_grouped_gemm(self.a, self.gl, self.w2p, self.m.H, fmt=self.code, y=self.y)

    def nonempty(self):
        return int((self.m.group_list > 0).sum())

    def gemm_flops(self, which):
        m = self.m
        return 2 * m.R * (2 * m.I) * m.H if which == "w13" else 2 * m.R * m.H * m.I

    def gemm_bytes(self):
        """Both grouped GEMMs: weights (codes + scales) of the experts that own
        rows, BF16 rows in and out, group_list."""
        m = self.m
        R, H, I = m.R, m.H, m.I
        return self.nonempty() * (self.b13 + self.b2) + 2 * R * (H + 2 * I) + 2 * R * (I + H) + 16 * m.E

    def alg_bytes(self):
        """The GEMMs' bytes and the SwiGLU's (BF16 [R, 2I] in, [R, I] out)."""
        m = self.m
        return self.gemm_bytes() + 2 * m.R * 3 * m.I

    def value(self, sec_per_step):
        return self.m.T / sec_per_step

    def dominant(self, per_key_ms):
        fl = self.gemm_flops("w13") + self.gemm_flops("w2")
        tot = per_key_ms["w13"] + per_key_ms["w2"]
        ach = fl / (tot * 1e-3) / 1e12
        return dict(bound="mfma", achieved=ach, peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                    frac=ach / PEAK_BF16_TFLOPS,
                    gemm_hbm_gbs=self.gemm_bytes() / (tot * 1e-3) / 1e9)

    def config(self):
        m = self.m
        g = m.group_list
        fmt = ("INT4 per 32 input channels, BF16 scale = amax / 7" if self.fmt == "int4" else
               "FP4 E2M1 per 32 input channels, E8M0 scale 2^(floor(log2 amax) - 2)")
        return {"workload": self.name, "T": m.T, "top_k": m.top_k, "E": m.E, "H": m.H, "I": m.I,
                "R": m.R, "nonempty_experts": self.nonempty(), "max_rows_per_expert": int(g.max()),
                "weights": "BF16 N(0, 0.02^2) -> " + fmt,
                "routing": "logits N(0,1) + expert bias N(0,1.5), top-8"}

    def cpu_baseline(self, budget_s):
        import numpy as np

        import oracle as O
        m = self.m
        W4 = O.w4a16
        off = O.group_offsets(m.group_list)
        xr = m.x_rows()
        H, I = m.H, m.I

        def codes_scales(N, K, r):
            # seeded codes and scales of the format's ranges (the chain's cost
            # does not depend on their values; the oracle's FP4 quantizer, an
            # exhaustive nearest-value search, would take ~9 s per expert)
            if self.fmt == "int4":
                q = r.integers(-8, 8, (N, K), dtype=np.int8)
                sc = O.f32_to_bf16(r.uniform(0.004, 0.01, (N, K // 32)).astype(np.float32))
            else:
                q = r.integers(0, 16, (N, K), dtype=np.uint8)
                sc = r.integers(118, 123, (N, K // 32), dtype=np.uint8)
            return q[None], sc[None]

        timed, rows, e = 0.0, 0, 0
        while timed < budget_s and e < m.E:
            a, b = int(off[e]), int(off[e + 1])
            if b > a:
                r = np.random.default_rng([0, 77, e])
                q13, s13 = codes_scales(2 * I, H, r)
                q2, s2 = codes_scales(H, I, r)
                t0 = time.perf_counter()
                W4.lowbit_moe(self.fmt, np.array([b - a], np.int64), xr[a:b], q13, s13, q2, s2)
                timed += time.perf_counter() - t0
                rows += b - a
            e += 1
        return dict(value=rows / m.top_k / timed, unit="tokens/s",
                    sample=f"oracle low-bit MoE chain over experts 0..{e - 1} ({rows} of {m.R} rows) on "
                           f"seeded codes and scales of the format's ranges (drawn outside the timing), "
                           f"tokens = rows / top_k")


class MxWorkload(Workload):
    def __init__(self, w, torch):
        super().__init__(w, torch)
        import numpy as np

        import synth
        self.name = "mx"
        d = synth.mx_block_fp8(seed=0)
        self.d = d
        N, K = d.w_e4m3.shape
        M = d.x.shape[0]
        self.M, self.N, self.K = M, N, K
        dev = "cuda"
        w8 = torch.from_numpy(d.w_e4m3).to(dev)
        sinv = torch.from_numpy(d.scale_inv).to(dev)
        torch.cuda.synchronize()
        # load-time prep: resolve -> BF16 -> MX quant -> prepack (timed once)
        a, b = _ev(torch), _ev(torch)
        a.record()
        wb = w.mx_resolve_block_fp8(w8, sinv, d.bn, d.bk)
        wp, ws = w.mx_quant(wb)
        self.packed = w.mx_prepack_weight(wp, ws)
        b.record()
        torch.cuda.synchronize()
        self.prep_ms = a.elapsed_time(b)
        del wb, wp, ws, w8
        self.x = torch.from_numpy(d.x.view(np.int16)).to(dev).view(torch.bfloat16)
        self.y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        self.ws = torch.empty((w.mx_linear_workspace_bytes(M, K),), dtype=torch.uint8, device=dev)
        self.y2 = torch.empty_like(self.y)
        self.unit = "TFLOPS"
        self.bound = "mfma"
        self._linear()
        torch.cuda.synchronize()
        self.a_e4m3, self.a_skb = w.mx_workspace_operands(self.ws, M, K)
        self.capture([self._linear], [(self._gemm, 1, "mx_gemm")])

    def _linear(self):
        self.w.mx_linear(self.x, self.packed, self.N, y=self.y, workspace=self.ws)

    def _gemm(self):
        self.w.mx_gemm(self.a_e4m3, self.a_skb, self.M, self.K, self.packed, self.N, y=self.y2)

    def flops(self):
        return 2.0 * self.M * self.N * self.K

    def alg_bytes(self):
        """E4M3 activation + its E8M0 scales, packed weight + scales, BF16 output."""
        M, N, K = self.M, self.N, self.K
        return M * K + M * K // 32 + N * K + N * K // 32 + 2 * M * N

    def value(self, sec_per_step):
        return self.flops() / sec_per_step / 1e12

    def dominant(self, per_key_ms):
        ach = self.flops() / (per_key_ms["mx_gemm"] * 1e-3) / 1e12
        return dict(bound="mfma", achieved=ach, peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                    frac=ach / PEAK_BF16_TFLOPS)

    def config(self):
        return {"workload": "mx", "M": self.M, "N": self.N, "K": self.K, "group": 32,
                "source_block": [self.d.bn, self.d.bk], "scale_alg": 0,
                "load_prep_ms": round(self.prep_ms, 3),
                "load_prep": "resolve + MX quant + prepack of the weight, once"}

    def cpu_baseline(self, budget_s):
        import oracle as O
        d = self.d
        ns = 256                                   # weight rows in the sample
        wb = O.mx.mx_resolve(d.w_e4m3[:ns], d.scale_inv[: -(-ns // d.bn)], d.bn, d.bk)
        wp, ws = O.mx.mx_quant(O.bf16_to_f32(wb))
        rows = 16
        t0 = time.perf_counter()
        n = 0
        while True:
            r0 = (n * rows) % self.M
            ap, as_ = O.mx.mx_quant(O.bf16_to_f32(d.x[r0:r0 + rows]))
            O.mx.mx_gemm_ref64(ap, as_, wp, ws)
            n += 1
            if time.perf_counter() - t0 > budget_s:
                break
        dt = time.perf_counter() - t0
        return dict(value=n * 2.0 * rows * ns * self.K / dt / 1e12, unit="TFLOPS",
                    sample=f"oracle MX quant of {rows} activation rows + float64 GEMM against "
                           f"{ns} of the {self.N} weight rows (weight prep outside the timing), "
                           f"{n} repetitions")


class StaticWorkload(Workload):
    """Static W8A8 on the prefill shape (M = 8192, K = 7168, N = 4096, bias): a step is
    the fixed-scale activation quant + the static linear. The dequant scale, the
    integer bias and the packed weight are prepared once at setup (timed apart as
    config.load_prep_ms)."""
    SCALE, OFFSET = 6.0 / 127.0, 3.0   # fixed calibration of N(0, 1) activations

    def __init__(self, w, torch):
        super().__init__(w, torch)
        import numpy as np

        import synth
        self.name = "static"
        d = synth.prefill(seed=0)
        self.d = d
        self.M, self.K = d.x.shape
        self.N = d.w.shape[0]
        dev = "cuda"
        self.x = torch.from_numpy(d.x.view(np.int16)).to(dev).view(torch.bfloat16)
        wdev = torch.from_numpy(d.w).to(dev)
        wsc = torch.from_numpy(d.w_scale).to(dev)
        bias = torch.from_numpy(d.bias.view(np.int16)).to(dev).view(torch.bfloat16)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        self.deq, self.qb = w.static_prepare(wdev, wsc, bias, self.SCALE, self.OFFSET)
        packed = w.prepack_weight(wdev)
        torch.cuda.synchronize()
        self.load_prep_ms = (time.perf_counter() - t0) * 1e3
        self.copies = 2
        self.wp = torch.empty((self.copies, packed.numel()), dtype=torch.uint8, device=dev)
        for c in range(self.copies):
            self.wp[c].copy_(packed)
        del packed, wdev
        # codes in the weight's block layout (whole 1 KB blocks for the tiles)
        self.q = torch.empty((w.packed_weight_bytes(1, self.M, self.K),), dtype=torch.uint8,
                             device=dev)
        self.y = torch.empty((self.M, self.N), dtype=torch.bfloat16, device=dev)
        steps = [self._make_step(c) for c in range(self.copies)]
        self.capture(steps, [(self._make_linears(16), 16, "static_linear")])
        self.unit = "TOPS"
        self.bound = "mfma"

    def _linear(self, c):
        self.w.static_linear(self.q, self.wp[c], self.deq, self.qb, self.N, y=self.y, M=self.M,
                             K=self.K)

    def _make_step(self, c):
        def fn():
            self.w.static_quant_packed(self.x, self.SCALE, self.OFFSET, q=self.q)
            self._linear(c)
        return fn

    def _make_linears(self, n):
        def fn():
            for i in range(n):
                self._linear(i % self.copies)
        return fn

    def ops(self):
        return 2 * self.M * self.N * self.K

    def alg_bytes(self):
        """One static linear launch: weight, dequant scale and integer bias, INT8
        codes in, BF16 out."""
        return self.N * self.K * BYTES_INT8 + 8 * self.N + self.M * self.K + 2 * self.M * self.N

    def value(self, sec_per_step):
        return self.ops() / sec_per_step / 1e12

    def dominant(self, per_key_ms):
        ach = self.ops() / (per_key_ms["static_linear"] * 1e-3) / 1e12
        return dict(bound="mfma", achieved=ach, peak=PEAK_INT8_TOPS, unit="TOP/s",
                    frac=ach / PEAK_INT8_TOPS)

    def config(self):
        return {"workload": "static", "M": self.M, "K": self.K, "N": self.N, "bias": True,
                "scheme": "static W8A8 (per-tensor input_scale / input_offset, integer bias)",
                "input_scale": round(self.SCALE, 8), "input_offset": self.OFFSET,
                "weight_copies": self.copies, "packed_codes": True,
                "load_prep_ms": round(self.load_prep_ms, 3),
                "x": "N(0,1) with outliers x20", "w": "int8 uniform [-127,127]"}

    def cpu_baseline(self, budget_s):
        import oracle as O
        d = self.d
        deq, qb = O.static.static_prepare(d.w, d.w_scale, d.bias, self.SCALE, self.OFFSET)
        rows = 128
        t0 = time.perf_counter()
        n = 0
        while True:
            q = O.static.static_quant(d.x[:rows], self.SCALE, self.OFFSET)
            O.static.static_linear(q, d.w, deq, qb)
            n += 1
            if time.perf_counter() - t0 > budget_s:
                break
        dt = (time.perf_counter() - t0) / n
        return dict(value=2 * rows * self.N * self.K / dt / 1e12, unit="TOPS",
                    sample=f"oracle static quant + static linear on the first {rows} of "
                           f"{self.M} rows ({n} repetitions), full N and K; prepare outside")


class CopyWorkload(Workload):
    """512 MiB device copy: HBM reference, not part of the W8A8 path."""
    NBYTES = 512 << 20

    def __init__(self, w, torch):
        super().__init__(w, torch)
        self.name = "copy"
        self.src = torch.empty((self.NBYTES,), dtype=torch.uint8, device="cuda").fill_(1)
        self.dst = torch.empty_like(self.src)
        self.unit = "GB/s"
        self.bound = "hbm"
        self.capture([self._copy], [(self._copy, 1, "copy")])

    def _copy(self):
        self.dst.copy_(self.src)

    def alg_bytes(self):
        return 2 * self.NBYTES

    def value(self, sec_per_step):
        return 2 * self.NBYTES / sec_per_step / 1e9

    def dominant(self, per_key_ms):
        ach = 2 * self.NBYTES / (per_key_ms["copy"] * 1e-3) / 1e9
        return dict(bound="hbm", achieved=ach, peak=PEAK_HBM_GBS, unit="GB/s",
                    frac=ach / PEAK_HBM_GBS)

    def config(self):
        return {"workload": "copy", "bytes": self.NBYTES, "kernel": "torch device copy"}

    def cpu_baseline(self, budget_s):
        import numpy as np
        a = np.ones(self.NBYTES, np.uint8)
        b = np.empty_like(a)
        t0 = time.perf_counter()
        n = 0
        while time.perf_counter() - t0 < min(budget_s, 3.0):
            np.copyto(b, a)
            n += 1
        dt = (time.perf_counter() - t0) / n
        return dict(value=2 * self.NBYTES / dt / 1e9, unit="GB/s", sample="numpy copy of 512 MiB")


# ---------------------------------------------------------------------------

def _traffic(name):
    """HBM bytes of the dominant unit measured by rocprofv3 (profiles/pmc_traffic.md),
    or None when no figure exists or a listed kernel source changed since."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "pmc_traffic.md")
    try:
        text = open(path).read()
        blob = text[text.index("```json") + 7:]
        data = json.loads(blob[:blob.index("```")])
        rec = data[name]
        h = hashlib.sha256()
        for f in rec["sources"]:
            h.update(open(os.path.join(ROOT, f), "rb").read())
        if h.hexdigest() != rec["sha256"]:
            return None
        return float(rec["traffic_bytes"])
    except (OSError, ValueError, KeyError):
        return None


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return os.cpu_count() or 1


def _make_workload(name, w, torch):
    if name == "decode":
        return DenseWorkload(w, torch, "decode", [1, 4, 16, 64], 7168, 4096, False, 0.005, 16)
    if name == "prefill":
        return DenseWorkload(w, torch, "prefill", [8192], 7168, 4096, True, 0.005, 2)
    if name == "tiny":
        return DenseWorkload(w, torch, "tiny", [16], 256, 128, True, 0.01, 1)
    if name == "copy":
        return CopyWorkload(w, torch)
    if name == "mx":
        return MxWorkload(w, torch)
    if name == "static":
        return StaticWorkload(w, torch)
    if name == "moe_layer":
        return MoeLayerWorkload(w, torch)
    if name == "mx_moe":
        return MxMoeWorkload(w, torch)
    if name == "w4a16":
        return W4Workload(w, torch)
    if name == "fp4":
        return W4Workload(w, torch, fmt="fp4")
    if name == "w4a16_moe":
        return LowbitMoeWorkload(w, torch)
    if name == "fp4_moe":
        return LowbitMoeWorkload(w, torch, fmt="fp4")
    return MoeWorkload(w, torch)


def _run(name, w, torch, steps, warmup, cpu_seconds, cpu_baseline):
    """One workload: warm-up, K timed steps, the dominant kernel's event timing
    and (optionally) the oracle on the host. Returns the result fields."""
    wl = _make_workload(name, w, torch)
    per_graph = steps_per_graph(steps, warmup)
    wl.group_steps(per_graph)
    for i in range(warmup):
        wl.step(i)
    torch.cuda.synchronize()
    # timed region: K steps, each a replay of the step's graph
    t0 = time.perf_counter()
    for i in range(steps):
        wl.step(warmup + i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    sec = elapsed / steps

    # dominant kernel: HIP events on the launch stream around replays of graphs
    # that hold only its launches (same buffers and weight rotation as the step)
    stream = torch.cuda.current_stream()
    per_key, counts = {}, {}
    reps = max(3, min(steps, 50))
    for g, n, key in wl.dominant_graphs:
        g.replay()                                   # warm
        evs = []
        for _ in range(reps):
            a, b = _ev(torch), _ev(torch)
            a.record(stream)
            g.replay()
            b.record(stream)
            evs.append((a, b))
        torch.cuda.synchronize()
        per_key[key] = sum(a.elapsed_time(b) for a, b in evs)
        counts[key] = reps * n
    avg_ms = {k: per_key[k] / counts[k] for k in per_key}

    roof = wl.dominant(avg_ms)
    roof["traffic"] = _traffic(wl.name)
    roof["algorithmic_bytes"] = wl.alg_bytes()
    roof["kernel_avg_us"] = {str(k): round(v * 1e3, 3) for k, v in avg_ms.items()}
    out = {
        "value": round(wl.value(sec), 3),
        "unit": wl.unit,
        "ms_per_step": round(sec * 1e3, 5),
        "steps_per_graph": per_graph,
        "dtype": {"mx": "bf16 (E4M3 x 2^E operands)", "mx_moe": "bf16 (E4M3 x 2^E operands)",
                  "w4a16": "bf16 (int4 weights)", "fp4": "bf16 (fp4 weights)",
                  "w4a16_moe": "bf16 (int4 weights)", "fp4_moe": "bf16 (fp4 weights)"}.get(wl.name, "int8"),
        "config": wl.config(),
        "roofline": {k: (round(v, 4) if isinstance(v, float) else v) for k, v in roof.items()},
    }
    if cpu_baseline:
        cb = wl.cpu_baseline(cpu_seconds)
        cb.update(cores=_blas_threads(), kind="oracle", host=platform.processor() or platform.machine())
        cb["value"] = round(cb["value"], 4)
        out["cpu_baseline"] = cb
    del wl
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def main():
    args = _args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1 "
                                   "(the multi-GPU sharding is described, not built)"}))
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(3)
    torch.cuda.set_device(0)
    import moe_token_amax_amd as w

    headline = "decode" if args.workload == "default" else args.workload
    res = _run(headline, w, torch, args.steps, args.warmup, args.cpu_seconds, not args.no_cpu_baseline)
    out = {
        "metric": Workload.metric,
        "value": res.pop("value"),
        "unit": res.pop("unit"),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res.pop("ms_per_step"),
        "steps_per_graph": res.pop("steps_per_graph"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": res.pop("dtype"),
        "data": "synthetic (seeded numpy; see synth/)",
    }
    out.update(res)
    if args.workload == "default":
        # the metric's other parts on their own workloads: prefill-shaped
        # linear TOPS, MoE grouped-GEMM tokens/s, and the other two configs of
        # the metric (the MXFP8 linear, the tiny latency case), each with its
        # roofline and oracle timing (at most 48 timed steps and 16 warm-up)
        extra = {}
        for name in ("prefill", "moe", "mx", "tiny"):
            r = _run(name, w, torch, min(args.steps, 48), min(args.warmup, 16), args.cpu_seconds,
                     not args.no_cpu_baseline)
            r["steps"] = min(args.steps, 48)
            r["warmup"] = min(args.warmup, 16)
            extra[name] = r
        out["also"] = extra
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
