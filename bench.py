#!/usr/bin/env python3
"""Benchmark of the MoE expert feed-forward layer on one MI355X.

One step = the whole forward hot path over one batch of synthetic tokens:
router top-k -> permutation into expert groups -> grouped gate_up GEMM with
ScaledSwiGLU -> grouped down GEMM -> unpermute/combine, at the Mixtral-8x7B
layer shape (T=8192, H=4096, I=14336, E=8, top-2, bf16). A second measurement
runs forward + backward at T=4096. Throughput is the algorithmic GEMM work
(6*R*H*I per forward, twice that per backward) over the wall time of the
timed steps, inputs already resident in HBM.

Prints one JSON line. The oracle's CPU time on a bounded sample of the same
workload is reported beside it (cpu_baseline).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
HBM_PEAK_GBPS = 8000.0      # MI355X HBM3E, published
FP32_PEAK_TFLOPS = 157.3    # MI355X fp32 vector, published
METRIC = "grouped-MLP TFLOP/s fwd and fwd+bwd, Mixtral-8x7B layer; % MFMA peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gate_up_traffic.json")
# the gate_up kernel's source: its file and the headers whose device code it inlines
KERNEL_SRCS = [os.path.join(ROOT, "grouped_expert_gemm_amd", "csrc", f)
               for f in ("gemm_fwd.hip", "gemm_common.h", "common.h", "gemm_bf16.h")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def dev_bf16(torch, np, bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


class Layer:
    """Device buffers and the C calls of one forward (and optionally backward) step."""

    def __init__(self, w, inp, backward: bool, mx: bool = False, prequant: bool = False, fp8: bool = False):
        import numpy as np
        import torch

        import grouped_expert_gemm_amd as moe
        from grouped_expert_gemm_amd import _lib

        self.torch, self.moe, self.L = torch, moe, moe.lib()
        self.w = w
        T, H, I, E, k = w.T, w.H, w.I, w.E, w.k
        R = T * k
        self.R = R
        dev = torch.device("cuda", 0)
        bf = torch.bfloat16
        self.logits = torch.from_numpy(inp.logits).cuda()
        self.x = dev_bf16(torch, np, inp.bits["x"])
        self.w1 = dev_bf16(torch, np, inp.bits["w1"])
        self.w2 = dev_bf16(torch, np, inp.bits["w2"])
        self.idx = torch.empty((T, k), dtype=torch.int32, device=dev)
        self.prob = torch.empty((T, k), dtype=torch.float32, device=dev)
        self.x_perm = torch.empty((R, H), dtype=bf, device=dev)
        self.prob_perm = torch.empty(R, dtype=torch.float32, device=dev)
        self.split = torch.empty(E, dtype=torch.int32, device=dev)
        self.offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
        self.rmap = torch.empty(R, dtype=torch.int32, device=dev)
        self.src = torch.empty(R, dtype=torch.int32, device=dev)
        self.ws_perm = torch.empty(max(1, moe.workspace_size(_lib.MOE_OP_PERMUTE, None, 0, T, E, k)),
                                   dtype=torch.uint8, device=dev)
        self.ws_gemm = moe.gemm_workspace(dev)
        self.h = torch.empty((R, I), dtype=bf, device=dev)
        self.z = torch.empty((R, 2 * I), dtype=bf, device=dev) if backward else None
        self.y = torch.empty((R, H), dtype=bf, device=dev)
        self.out = torch.empty((T, H), dtype=bf, device=dev)
        self.t1, self._k1 = _lib.ptr_table([self.w1[e].data_ptr() for e in range(E)])
        self.t2, self._k2 = _lib.ptr_table([self.w2[e].data_ptr() for e in range(E)])
        self.backward = backward
        if backward:
            self.dout = dev_bf16(torch, np, inp.bits["dout"])
            self.dy = torch.empty((R, H), dtype=bf, device=dev)
            self.dx_perm = torch.empty((R, H), dtype=bf, device=dev)
            self.dx = torch.empty((T, H), dtype=bf, device=dev)
            self.dw1 = torch.empty_like(self.w1)
            self.dw2 = torch.empty_like(self.w2)
            self.dprob_perm = torch.empty(R, dtype=torch.float32, device=dev)
            self.dprob = torch.empty(R, dtype=torch.float32, device=dev)
            self.d1, self._k3 = _lib.ptr_table([self.dw1[e].data_ptr() for e in range(E)])
            self.d2, self._k4 = _lib.ptr_table([self.dw2[e].data_ptr() for e in range(E)])
            comp = _lib.MOE_FP8 if fp8 else (_lib.MOE_MXFP8 if mx else _lib.MOE_BF16)
            self.desc = _lib.MlpDesc(E, H, I, comp, _lib.MOE_BF16, _lib.MOE_BF16, 1)
            self.ws_bwd = torch.empty(moe.workspace_size(_lib.MOE_OP_MLP_BWD, self.desc, R), dtype=torch.uint8,
                                      device=dev)
        self.mx = mx or fp8
        self.fs1 = self.fs2 = None
        self.wq_step = None
        if (mx or fp8) and backward:
            # the forward's and the backward's weight layouts from one two-layout call per
            # weight tensor: once outside the timed steps (prequant), or at the start of
            # every step from the bf16 master weights (as a step after an optimizer update)
            quant = moe.fp8_tensor_quantize_weights if fp8 else moe.mxfp8_quantize_weights
            self.q1, qs1, self.pk1 = quant(self.w1)
            self.q2, qs2, self.pk2 = quant(self.w2)
            self.qs1, self.qs2 = qs1, qs2
            t = lambda ts: _lib.ptr_table([x.data_ptr() for x in ts])
            self.t1, self._k1 = t([self.q1[e] for e in range(E)])
            self.t2, self._k2 = t([self.q2[e] for e in range(E)])
            if fp8:
                self.fs1, self._k5 = _lib.ptr_table([qs1.data_ptr() + 4 * e for e in range(E)])
                self.fs2, self._k6 = _lib.ptr_table([qs2.data_ptr() + 4 * e for e in range(E)])
            else:
                self.fs1, self._k5 = t([qs1[e] for e in range(E)])
                self.fs2, self._k6 = t([qs2[e] for e in range(E)])
            self.b1, self._k7 = t([self.pk1[e] for e in range(E)])
            self.b2, self._k8 = t([self.pk2[e] for e in range(E)])
            if not prequant:
                w1t, k9 = t([self.w1[e] for e in range(E)])
                w2t, k10 = t([self.w2[e] for e in range(E)])
                self._k9 = (k9, k10)
                if fp8:  # the factors: one float32 array per weight tensor
                    f1, f2 = ctypes.c_void_p(qs1.data_ptr()), ctypes.c_void_p(qs2.data_ptr())
                    self.wq_step = [(self.L.fp8_tensor_quantize_weights, E, w1t, 2 * I, H, self.t1, f1, self.b1),
                                    (self.L.fp8_tensor_quantize_weights, E, w2t, H, I, self.t2, f2, self.b2)]
                else:
                    self.wq_step = [(self.L.mxfp8_quantize_weights, E, w1t, 2 * I, H, self.t1, self.fs1, self.b1),
                                    (self.L.mxfp8_quantize_weights, E, w2t, H, I, self.t2, self.fs2, self.b2)]
            comp = _lib.MOE_FP8 if fp8 else _lib.MOE_MXFP8
            self.desc = _lib.MlpDesc(E, H, I, comp, _lib.MOE_BF16, comp, 1)
            self.ws_bwd = torch.empty(moe.workspace_size(_lib.MOE_OP_MLP_BWD, self.desc, R), dtype=torch.uint8,
                                      device=dev)
            self.desc_fwd = _lib.MlpDesc(E, H, I, comp, _lib.MOE_BF16, comp, 1)
            self.ws_fwd = torch.empty(moe.workspace_size(_lib.MOE_OP_MLP_FWD, self.desc_fwd, R), dtype=torch.uint8,
                                      device=dev)
        elif fp8:  # the grouped MLP forward in per-tensor FP8 (one call)
            wt = _lib.MOE_BF16
            if prequant:
                # weights quantised once, outside the timed steps: codes and one factor per expert
                wt = _lib.MOE_FP8
                q1 = [moe.fp8_tensor_quantize(self.w1[e]) for e in range(E)]
                q2 = [moe.fp8_tensor_quantize(self.w2[e]) for e in range(E)]
                self._q = (q1, q2)
                self.t1, self._k1 = _lib.ptr_table([c.data_ptr() for c, _ in q1])
                self.t2, self._k2 = _lib.ptr_table([c.data_ptr() for c, _ in q2])
                self.fs1, self._k5 = _lib.ptr_table([f.data_ptr() for _, f in q1])
                self.fs2, self._k6 = _lib.ptr_table([f.data_ptr() for _, f in q2])
            self.desc_fwd = _lib.MlpDesc(E, H, I, _lib.MOE_FP8, _lib.MOE_BF16, wt, 0)
            self.ws_fwd = torch.empty(moe.workspace_size(_lib.MOE_OP_MLP_FWD, self.desc_fwd, R), dtype=torch.uint8,
                                      device=dev)
        elif mx:  # the grouped MLP forward in MXFP8 (one call)
            wt = _lib.MOE_BF16
            if prequant:
                # weights quantised once, outside the timed steps, by rows (the forward's layout)
                wt = _lib.MOE_MXFP8
                self.q1, self.qs1 = moe.mxfp8_quantize(self.w1)
                self.q2, self.qs2 = moe.mxfp8_quantize(self.w2)
                self.t1, self._k1 = _lib.ptr_table([self.q1[e].data_ptr() for e in range(E)])
                self.t2, self._k2 = _lib.ptr_table([self.q2[e].data_ptr() for e in range(E)])
                self.fs1, self._k5 = _lib.ptr_table([self.qs1[e].data_ptr() for e in range(E)])
                self.fs2, self._k6 = _lib.ptr_table([self.qs2[e].data_ptr() for e in range(E)])
            self.desc_fwd = _lib.MlpDesc(E, H, I, _lib.MOE_MXFP8, _lib.MOE_BF16, wt, 0)
            self.ws_fwd = torch.empty(moe.workspace_size(_lib.MOE_OP_MLP_FWD, self.desc_fwd, R), dtype=torch.uint8,
                                      device=dev)
        if not ((mx or fp8) and backward):
            self.b1, self.b2 = self.t1, self.t2
        self.stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        self.ev = []

    def step(self, time_gate_up=False):
        from grouped_expert_gemm_amd import _lib
        L, w, s, p = self.L, self.w, self.stream, (lambda t: ctypes.c_void_p(t.data_ptr()))
        T, H, I, E, k, R = w.T, w.H, w.I, w.E, w.k, self.R
        BF = _lib.MOE_BF16
        c = _lib.check
        c("route", L.moe_route_topk(p(self.logits), T, E, k, 1, p(self.idx), p(self.prob), s))
        c("permute", L.moe_permute(p(self.x), None, BF, T, H, E, k, p(self.idx), p(self.prob), 0, p(self.x_perm),
                                   None, p(self.prob_perm), p(self.split), p(self.offsets), p(self.rmap),
                                   p(self.src), p(self.ws_perm), self.ws_perm.numel(), s))
        if self.wq_step:  # bf16 master weights -> both layouts, every step
            for fn, *args in self.wq_step:
                c("weight quantisation", fn(*args, s))
        if self.mx:
            c("mlp fwd", L.moe_grouped_mlp_fwd(ctypes.byref(self.desc_fwd), R, p(self.x_perm), None, self.t1, self.t2,
                                               self.fs1, self.fs2, p(self.offsets), p(self.prob_perm), p(self.y),
                                               p(self.z) if self.z is not None else None, p(self.h),
                                               p(self.ws_fwd), self.ws_fwd.numel(), s))
        else:
            if time_gate_up:
                e0 = self.torch.cuda.Event(enable_timing=True)
                e1 = self.torch.cuda.Event(enable_timing=True)
                e0.record()
            c("gate_up", L.moe_grouped_gate_up_swiglu(E, R, H, I, BF, p(self.x_perm), None, self.t1, None,
                                                      p(self.offsets), p(self.prob_perm), p(self.h), None,
                                                      p(self.z) if self.z is not None else None, p(self.ws_gemm),
                                                      self.ws_gemm.numel(), s))
            if time_gate_up:
                e1.record()
                self.ev.append((e0, e1))
            c("down", L.moe_grouped_linear(E, R, I, H, BF, p(self.h), self.t2, p(self.offsets), p(self.y),
                                           p(self.ws_gemm), self.ws_gemm.numel(), s))
        c("combine", L.moe_unpermute_combine(p(self.y), BF, p(self.rmap), None, T, H, k, p(self.out), s))
        if self.backward:
            c("dOut gather", L.moe_permute(p(self.dout), None, BF, T, H, E, k, None, None, 1, p(self.dy), None,
                                           None, None, None, p(self.rmap), None, None, 0, s))
            c("mlp bwd", L.moe_grouped_mlp_bwd(ctypes.byref(self.desc), R, p(self.dy), p(self.x_perm), p(self.z),
                                               p(self.h), p(self.prob_perm), self.b1, self.b2, p(self.offsets),
                                               p(self.dx_perm), self.d1, self.d2, p(self.dprob_perm),
                                               p(self.ws_bwd), self.ws_bwd.numel(), s))
            c("dx combine", L.moe_unpermute_combine(p(self.dx_perm), BF, p(self.rmap), None, T, H, k, p(self.dx),
                                                    s))
            # dprob[t, j] = dprob_perm[row_id_map[t*k + j]]: a gather, i.e. a combine with k = 1
            c("dprob gather", L.moe_unpermute_combine(p(self.dprob_perm), _lib.MOE_F32, p(self.rmap), None, R, 1,
                                                      1, p(self.dprob), s))

    def gate_up_ms(self):
        self.torch.cuda.synchronize()
        ts = [a.elapsed_time(b) for a, b in self.ev]
        return sum(ts) / len(ts)


def time_steps(layer, steps, warmup):
    torch = layer.torch
    for _ in range(warmup):
        layer.step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        layer.step(time_gate_up=True)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


FP8_PEAK_TFLOPS = 5000.0    # MI355X dense fp8 MFMA, published
FLUSH_BYTES = 512 << 20     # twice the 256 MB Infinity Cache


_flush_buf = None


def timed_flushed(f, reps):
    """Average time of f() (ms) over `reps` calls, each timed alone with events on the
    current stream right after a 512 MB device write, which evicts the Infinity Cache
    and L2: a memory-bound call then reads its inputs from HBM, not from a cache that
    the previous call warmed."""
    import torch
    global _flush_buf
    if _flush_buf is None:
        _flush_buf = torch.empty(FLUSH_BYTES // 4, dtype=torch.int32, device="cuda")
    f()
    total = 0.0
    for i in range(reps):
        _flush_buf.fill_(i)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        f()
        b.record()
        b.synchronize()
        total += a.elapsed_time(b)
    return total / reps


def extra_forward(w, inp, steps, warmup, compute="bf16", prequant=False):
    """One forward layer step through the Python binding (route, permute, grouped MLP,
    combine) on another workload or precision; returns its throughput record."""
    import numpy as np
    import torch

    import grouped_expert_gemm_amd as moe

    dev_logits = torch.from_numpy(inp.logits).cuda()
    x = dev_bf16(torch, np, inp.bits["x"])
    w1 = dev_bf16(torch, np, inp.bits["w1"])
    w2 = dev_bf16(torch, np, inp.bits["w2"])
    s1 = s2 = None
    if prequant and compute == "fp8":
        # master weights quantised once (one scale per expert weight), outside the timed steps
        q1 = [moe.fp8_tensor_quantize(w1[e]) for e in range(w.E)]
        q2 = [moe.fp8_tensor_quantize(w2[e]) for e in range(w.E)]
        w1, s1 = [c for c, _ in q1], [sc for _, sc in q1]
        w2, s2 = [c for c, _ in q2], [sc for _, sc in q2]
    elif prequant:
        # master weights quantised once, outside the timed steps
        E, twoI, H = w1.shape
        q1, s1 = moe.mxfp8_quantize(w1.reshape(E * twoI, H))
        q2, s2 = moe.mxfp8_quantize(w2.reshape(E * H, w.I))
        w1, s1 = q1.reshape(E, twoI, H), s1.reshape(E, twoI, H // 32)
        w2, s2 = q2.reshape(E, H, w.I), s2.reshape(E, H, w.I // 32)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")

    def step():
        nonlocal ws
        idx, p = moe.moe_route_topk(dev_logits, w.k)
        r = moe.moe_permute(x, idx, p, w.E)
        y = moe.moe_grouped_mlp_fwd(r["x_perm"], w1, w2, r["offsets"], r["prob_perm"], compute=compute,
                                    w_gate_up_scale=s1, w_down_scale=s2, workspace=ws)
        moe.moe_unpermute_combine(y, r["row_id_map"], w.T, w.k)

    from grouped_expert_gemm_amd import _lib
    desc = _lib.MlpDesc(w.E, w.H, w.I, moe._COMPUTE[compute], _lib.MOE_BF16,
                        moe._COMPUTE[compute] if prequant else _lib.MOE_BF16, 0)
    ws = torch.empty(max(1, moe.workspace_size(_lib.MOE_OP_MLP_FWD, desc, w.R)), dtype=torch.uint8, device="cuda")
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    v = w.gemm_flop_fwd() / (ms * 1e-3) / 1e12
    peak = FP8_PEAK_TFLOPS if compute in ("mxfp8", "fp8") else BF16_PEAK_TFLOPS
    rec = {"workload": w.name, "T": w.T, "H": w.H, "I": w.I, "E": w.E, "k": w.k, "compute": compute,
           "value": round(v, 2), "unit": "TFLOP/s", "ms_per_step": round(ms, 4),
           "pct_of_peak": round(100 * v / peak, 2), "peak": peak}
    if compute in ("mxfp8", "fp8"):
        rec["weights"] = (f"{compute.upper()}, quantised once outside the step" if prequant
                          else "bf16 master weights, quantised inside every step")
    log(f"{w.name} {compute}{' prequant' if prequant else ''}: {ms:.3f} ms -> {v:.1f} TFLOP/s")
    return rec


def router_measure(w, inp, reps=20):
    """The router gate linear (bf16 MFMA; HBM-bound at small E), the top-k gating
    backward and the gate linear's backward (float32 VALU) at a workload's shape, each
    timed with events around single calls after a cache flush (timed_flushed); returns
    one record per op with its roofline."""
    import numpy as np
    import torch

    import grouped_expert_gemm_amd as moe

    T, H, E, k = w.T, w.H, w.E, w.k
    x = dev_bf16(torch, np, inp.bits["x"])
    g = torch.Generator(device="cuda").manual_seed(w.seed)
    wr = (0.02 * torch.randn((E, H), generator=g, device="cuda")).to(torch.bfloat16)
    logits = torch.from_numpy(inp.logits).cuda()
    idx, prob = moe.moe_route_topk(logits, k)
    dprob = torch.randn((T, k), generator=g, device="cuda")
    dlog = moe.moe_route_topk_bwd(idx, prob, dprob, E)
    dx = torch.empty_like(x)

    def timed(f):
        return timed_flushed(f, reps)

    out = {"workload": w.name, "T": T, "H": H, "E": E, "k": k}
    ms = timed(lambda: moe.moe_router_logits(x, wr))
    nbytes = T * H * 2 + E * H * 2 + T * E * 4
    out["router_logits"] = {"ms": round(ms, 4), "bound": "hbm", "achieved_GBps": round(nbytes / ms / 1e6, 1),
                            "peak_GBps": HBM_PEAK_GBPS, "frac": round(nbytes / ms / 1e6 / HBM_PEAK_GBPS, 4),
                            "tflops": round(2.0 * T * H * E / ms / 1e9, 2)}
    ms = timed(lambda: moe.moe_route_topk_bwd(idx, prob, dprob, E))
    nbytes = T * k * 12 + T * E * 4
    out["route_topk_bwd"] = {"ms": round(ms, 4), "bound": "hbm", "achieved_GBps": round(nbytes / ms / 1e6, 1),
                             "peak_GBps": HBM_PEAK_GBPS, "frac": round(nbytes / ms / 1e6 / HBM_PEAK_GBPS, 4)}
    ms = timed(lambda: moe.moe_router_bwd(x, wr, dlog, dx_in=dx, dx=dx))
    # x read, dx read and written, d_logits read, dW written: whichever of the fp32
    # vector rate and HBM takes longer bounds the op
    flops = 4.0 * T * H * E
    nbytes = 3 * T * H * 2 + T * E * 4 + E * H * 4
    if flops / FP32_PEAK_TFLOPS / 1e12 >= nbytes / HBM_PEAK_GBPS / 1e9:
        out["router_bwd"] = {"ms": round(ms, 4), "bound": "alu", "achieved_TFLOPs": round(flops / ms / 1e9, 2),
                             "peak_TFLOPs": FP32_PEAK_TFLOPS, "frac": round(flops / ms / 1e9 / FP32_PEAK_TFLOPS, 4)}
    else:
        out["router_bwd"] = {"ms": round(ms, 4), "bound": "hbm", "achieved_GBps": round(nbytes / ms / 1e6, 1),
                             "peak_GBps": HBM_PEAK_GBPS, "frac": round(nbytes / ms / 1e6 / HBM_PEAK_GBPS, 4)}
    log(f"router {w.name}: logits {out['router_logits']['ms']:.3f} ms, topk bwd {out['route_topk_bwd']['ms']:.3f} ms, "
        f"gate bwd {out['router_bwd']['ms']:.3f} ms")
    return out


def colwise_measure(reps=20):
    """Column-wise MXFP8 quantisation (per expert, along the token axis; the operand
    layout of MXFP8 weight gradients) of the Mixtral backward's dY [R, H] and h [R, I]
    (T=4096, top-2), pad 256, each call timed after a cache flush: HBM-bound."""
    import torch

    import grouped_expert_gemm_amd as moe
    from moe_inputs import WORKLOADS, make_inputs, scaled

    w = WORKLOADS["mixtral_fwd_bwd"]
    inp = make_inputs(scaled(w, H=32, I=32), want_float=False)  # the routing depends on the logits only
    idx, p = moe.moe_route_topk(torch.from_numpy(inp.logits).cuda(), w.k)
    r = moe.moe_permute(torch.zeros((w.T, 32), dtype=torch.bfloat16, device="cuda"), idx, p, w.E)
    off = r["offsets"]
    R = w.T * w.k
    g = torch.Generator(device="cuda").manual_seed(w.seed)
    recs = []
    for name, C in (("dY", w.H), ("h", w.I)):
        x = torch.randn((R, C), generator=g, device="cuda").to(torch.bfloat16)
        codes, scales, kofs = moe.mxfp8_quantize_colwise(x, off, 256)  # allocates the outputs once
        kcap = codes.shape[1]
        L = moe.lib()
        vp = ctypes.c_void_p
        args = (vp(x.data_ptr()), R, C, w.E, vp(off.data_ptr()), 256, kcap, vp(codes.data_ptr()),
                vp(scales.data_ptr()), vp(kofs.data_ptr()), vp(torch.cuda.current_stream().cuda_stream))
        # the C entry point on the same buffers (no allocation), each call after a cache flush
        ms = timed_flushed(lambda: L.mxfp8_quantize_colwise(*args), reps)
        ktot = int(kofs[-1].item())
        nbytes = R * C * 2 + C * ktot + C * ktot // 32
        recs.append({"tensor": name, "rows": R, "cols": C, "padded_rows": ktot, "ms": round(ms, 4), "bound": "hbm",
                     "achieved_GBps": round(nbytes / ms / 1e6, 1), "peak_GBps": HBM_PEAK_GBPS,
                     "frac": round(nbytes / ms / 1e6 / HBM_PEAK_GBPS, 4)})
        log(f"mxfp8 colwise {name} [{R}, {C}]: {ms:.3f} ms -> {nbytes / ms / 1e6:.0f} GB/s")
    return recs


def memory_bound_measure(w, inp, reps=20):
    """The permutation (count, scan and gather of x into expert order, with the maps)
    and the combine at a forward workload's shape, each call timed alone after a cache
    flush. Algorithmic bytes: permute T*H*2 (x) + R*H*2 (x_perm) + T*k*8 (ids and
    probabilities) + R*16 (four maps and prob_perm); combine R*H*2 + T*H*2 + T*k*4."""
    import numpy as np
    import torch

    import grouped_expert_gemm_amd as moe
    from grouped_expert_gemm_amd import _lib

    T, H, E, k = w.T, w.H, w.E, w.k
    R = T * k
    x = dev_bf16(torch, np, inp.bits["x"])
    idx, prob = moe.moe_route_topk(torch.from_numpy(inp.logits).cuda(), k)
    r = moe.moe_permute(x, idx, prob, E)
    y = torch.randn((R, H), device="cuda").to(torch.bfloat16)
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(max(1, moe.workspace_size(_lib.MOE_OP_PERMUTE, None, 0, T, E, k)), dtype=torch.uint8,
                     device="cuda")
    L = moe.lib()
    vp = lambda t: ctypes.c_void_p(t.data_ptr())
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def permute():
        _lib.check("permute", L.moe_permute(vp(x), None, _lib.MOE_BF16, T, H, E, k, vp(idx), vp(prob), 0,
                                            vp(r["x_perm"]), None, vp(r["prob_perm"]), vp(r["split_sizes"]),
                                            vp(r["offsets"]), vp(r["row_id_map"]), vp(r["src_token"]), vp(ws),
                                            ws.numel(), s))

    def combine():
        _lib.check("combine", L.moe_unpermute_combine(vp(y), _lib.MOE_BF16, vp(r["row_id_map"]), None, T, H, k,
                                                      vp(out), s))

    recs = {"workload": w.name, "T": T, "H": H, "E": E, "k": k, "cache": "flushed (512 MB write) before each call"}
    for name, f, nbytes in (("permute", permute, T * H * 2 + R * H * 2 + T * k * 8 + R * 16),
                            ("combine", combine, R * H * 2 + T * H * 2 + T * k * 4)):
        ms = timed_flushed(f, reps)
        recs[name] = {"ms": round(ms, 4), "bound": "hbm", "achieved_GBps": round(nbytes / ms / 1e6, 1),
                      "peak_GBps": HBM_PEAK_GBPS, "frac": round(nbytes / ms / 1e6 / HBM_PEAK_GBPS, 4),
                      "bytes": nbytes}
        log(f"{name} {w.name}: {ms:.4f} ms -> {nbytes / ms / 1e6:.0f} GB/s")
    return recs


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def kernel_sha256():
    """sha256 over the gate_up kernel's source files, in a fixed order."""
    h = hashlib.sha256()
    for f in KERNEL_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def traffic_record():
    """HBM bytes per gate_up launch from the committed rocprofv3 counter runs, or None
    if they were taken on a different version of the kernel source."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
        sha = kernel_sha256()
        if rec.get("kernel_sha256") != sha:
            return None
        return rec.get("bytes_per_launch")
    except (OSError, ValueError):
        return None


def cpu_baseline(inp, w, seconds):
    """The oracle (float64 numpy, per-expert loop) on the same workload, expert by expert
    in index order until about `seconds` of host time have passed (at least one expert):
    route, permute, then the grouped MLP of each expert on all of its rows."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle
    from moe_inputs import bf16_bits_to_f32

    idx, p = oracle.route_topk(inp.logits, w.k)
    m = oracle.permute(idx, w.E)
    pp = p.ravel()[m["src_token"] * w.k + m["src_slot"]]
    t_all = 0.0
    rows = 0
    experts = 0
    for e in range(w.E):
        a, b = int(m["offsets"][e]), int(m["offsets"][e + 1])
        x = bf16_bits_to_f32(inp.bits["x"][m["src_token"][a:b]])
        w1 = bf16_bits_to_f32(inp.bits["w1"][e:e + 1])
        w2 = bf16_bits_to_f32(inp.bits["w2"][e:e + 1])
        t0 = time.perf_counter()
        oracle.grouped_mlp_forward(x, w1, w2, np.array([0, b - a]), pp[a:b])
        t_all += time.perf_counter() - t0
        rows += b - a
        experts += 1
        if t_all >= seconds:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    flop = 6.0 * rows * w.H * w.I
    return {"value": round(flop / t_all / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"float64 numpy oracle, grouped MLP forward (gate_up, ScaledSwiGLU, down) of experts "
                      f"0..{experts - 1} of the {w.name} workload on all their rows ({rows} of {w.R} rows, "
                      f"H={w.H}, I={w.I}); {t_all:.1f} s of oracle time, {os.cpu_count()} host CPUs visible"}


_FWD_BWD_INPUTS = None


def fwd_bwd_measure(steps, warmup, mx=False, prequant=False, fp8=False):
    """The whole layer forward + backward step (route ... combine, dOut gather, grouped
    MLP backward, dx combine, dprob gather) at the Mixtral fwd+bwd shape; mx: the grouped
    MLP forward and backward in MXFP8 (the forward saving z and h in bf16); fp8: the same
    in per-tensor FP8. The low-precision steps start from the bf16 master weights: one
    call per weight tensor writes the forward's and the backward's layouts at the start
    of every step, or once outside the timed steps with prequant."""
    global _FWD_BWD_INPUTS
    from moe_inputs import WORKLOADS, make_inputs

    wb = WORKLOADS["mixtral_fwd_bwd"]
    if _FWD_BWD_INPUTS is None:   # the same seeded inputs for every fwd+bwd measurement
        t0 = time.perf_counter()
        _FWD_BWD_INPUTS = make_inputs(wb, want_float=False)
        log(f"inputs {wb.name}: {time.perf_counter() - t0:.1f} s")
    lb = Layer(wb, _FWD_BWD_INPUTS, backward=True, mx=mx, prequant=prequant, fp8=fp8)
    msb = time_steps(lb, steps, warmup)
    flopb = 3.0 * wb.gemm_flop_fwd()
    vb = flopb / (msb * 1e-3) / 1e12
    peak = FP8_PEAK_TFLOPS if (mx or fp8) else BF16_PEAK_TFLOPS
    tag = " (FP8)" if fp8 else (" (MXFP8)" if mx else "")
    log(f"fwd+bwd step{tag}{' prequant' if prequant else ''} {msb:.3f} ms -> {vb:.1f} TFLOP/s")
    rec = {"workload": "mixtral_fwd_bwd", "T": wb.T, "value": round(vb, 2), "unit": "TFLOP/s",
           "ms_per_step": round(msb, 4), "flop_per_step": flopb}
    if fp8:
        rec.update(compute="fp8", pct_of_fp8_peak=round(100 * vb / peak, 2),
                   weights=("FP8, quantised once outside the step (codes and factors for the forward, transposed "
                            "packs for the backward)" if prequant else
                            "bf16 master weights, quantised inside every step (one factor per tensor; "
                            "fp8_tensor_quantize_weights: the forward's codes and the backward's packs together)"))
    elif mx:
        rec.update(compute="mxfp8", pct_of_fp8_peak=round(100 * vb / peak, 2),
                   weights=("MXFP8, quantised once outside the step (row-wise for the forward, packed for the "
                            "backward)" if prequant else
                            "bf16 master weights, quantised inside every step (mxfp8_quantize_weights: row-wise "
                            "for the forward and packed for the backward from one read)"))
    else:
        rec["pct_of_bf16_peak"] = round(100 * vb / peak, 2)
    return rec


def bwd_measure(reps=10):
    """The grouped MLP backward call alone at the Mixtral fwd+bwd shape (T=4096, top-2),
    bf16 and MXFP8, on the saved z and h of one bf16 forward. Work: the four backward
    GEMMs, 2x the forward's GEMM flop."""
    import torch
    from grouped_expert_gemm_amd import _lib
    import grouped_expert_gemm_amd as moe
    from moe_inputs import WORKLOADS, make_inputs

    wb = WORKLOADS["mixtral_fwd_bwd"]
    lb = Layer(wb, make_inputs(wb, want_float=False), backward=True)
    lb.step()
    torch.cuda.synchronize()
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    flop = 2.0 * wb.gemm_flop_fwd()
    out = []
    for name, comp in (("bf16", _lib.MOE_BF16), ("mxfp8", _lib.MOE_MXFP8), ("fp8", _lib.MOE_FP8)):
        desc = _lib.MlpDesc(wb.E, wb.H, wb.I, comp, _lib.MOE_BF16, _lib.MOE_BF16, 1)
        ws = torch.empty(moe.workspace_size(_lib.MOE_OP_MLP_BWD, desc, lb.R), dtype=torch.uint8, device="cuda")

        def call():
            _lib.check("mlp bwd", lb.L.moe_grouped_mlp_bwd(
                ctypes.byref(desc), lb.R, p(lb.dy), p(lb.x_perm), p(lb.z), p(lb.h), p(lb.prob_perm), lb.t1, lb.t2,
                p(lb.offsets), p(lb.dx_perm), lb.d1, lb.d2, p(lb.dprob_perm), p(ws), ws.numel(), lb.stream))

        for _ in range(2):
            call()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            call()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        v = flop / (ms * 1e-3) / 1e12
        peak = BF16_PEAK_TFLOPS if name == "bf16" else 2 * BF16_PEAK_TFLOPS
        log(f"grouped MLP backward {name}: {ms:.3f} ms -> {v:.1f} TFLOP/s ({100 * v / peak:.1f}% of {peak:.0f})")
        out.append({"workload": "mixtral_fwd_bwd", "compute": name, "ms": round(ms, 4), "value": round(v, 2),
                    "unit": "TFLOP/s", "pct_of_peak": round(100 * v / peak, 2), "flop": flop})
        del ws
    return out


def only_measurement(which, steps, warmup):
    """One measurement on its own (for kernel traces of that workload)."""
    from moe_inputs import WORKLOADS, make_inputs

    if which == "fwd_bwd":
        return fwd_bwd_measure(steps, warmup)
    if which == "mx_fwd_bwd":
        return fwd_bwd_measure(steps, warmup, mx=True)
    if which == "mx_fwd_bwd_pre":
        return fwd_bwd_measure(steps, warmup, mx=True, prequant=True)
    if which == "fp8_fwd_bwd":
        return fwd_bwd_measure(steps, warmup, fp8=True)
    if which == "fp8_fwd_bwd_pre":
        return fwd_bwd_measure(steps, warmup, fp8=True, prequant=True)
    if which == "bwd":
        return bwd_measure(steps)
    if which == "qwen3":
        wq = WORKLOADS["qwen3_fwd"]
        return extra_forward(wq, make_inputs(wq, want_float=False), steps, warmup)
    w = WORKLOADS["mixtral_fwd"]
    inp = make_inputs(w, want_float=False)
    if which == "mxfp8":
        w8 = WORKLOADS["mixtral_mxfp8_fwd"]
        return [extra_forward(w8, inp, steps, warmup, compute="mxfp8"),
                extra_forward(w8, inp, steps, warmup, compute="mxfp8", prequant=True)]
    if which == "colwise":
        return colwise_measure(steps)
    if which == "permute":
        wq = WORKLOADS["qwen3_fwd"]
        return [memory_bound_measure(w, inp, steps), memory_bound_measure(wq, make_inputs(wq, want_float=False), steps)]
    if which == "fp8":
        w8 = WORKLOADS["mixtral_mxfp8_fwd"]
        return [extra_forward(w8, inp, steps, warmup, compute="fp8"),
                extra_forward(w8, inp, steps, warmup, compute="fp8", prequant=True)]
    wq = WORKLOADS["qwen3_fwd"]
    return [router_measure(w, inp, steps), router_measure(wq, make_inputs(wq, want_float=False), steps)]


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-fwd-bwd", action="store_true", help="skip the forward+backward measurement")
    ap.add_argument("--quick", action="store_true", help="skip the MXFP8 and Qwen3 measurements")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--only", choices=["fwd_bwd", "mx_fwd_bwd", "mx_fwd_bwd_pre", "fp8_fwd_bwd", "fp8_fwd_bwd_pre", "bwd", "qwen3", "mxfp8", "fp8", "router", "colwise", "permute"],
                    help="run one measurement and print its record (kernel traces of that workload)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (HBM counter calibration)")
    args = ap.parse_args()
    if args.calibrate_copy:
        import torch
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": 1 << 30, "copy_bytes_written": 1 << 30, "launches": 5}))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the MoE layer here runs all experts on a single MI355X "
              "(no expert parallelism across GPUs is built); run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    from moe_inputs import WORKLOADS, make_inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)

    if args.only:
        print(json.dumps(only_measurement(args.only, args.steps, args.warmup)), flush=True)
        return

    w = WORKLOADS["mixtral_fwd"]
    t0 = time.perf_counter()
    inp = make_inputs(w, want_float=False)
    log(f"inputs {w.name}: {time.perf_counter() - t0:.1f} s")
    layer = Layer(w, inp, backward=False)
    ms = time_steps(layer, args.steps, args.warmup)
    gate_ms = layer.gate_up_ms()
    flop = w.gemm_flop_fwd()
    value = flop / (ms * 1e-3) / 1e12
    R = w.R
    gate_flop = 4.0 * R * w.H * w.I
    achieved = gate_flop / (gate_ms * 1e-3) / 1e12
    log(f"fwd step {ms:.3f} ms -> {value:.1f} TFLOP/s; gate_up {gate_ms:.3f} ms -> {achieved:.1f} TFLOP/s")
    traffic = traffic_record()
    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "mixtral_fwd", "T": w.T, "H": w.H, "I": w.I, "E": w.E, "k": w.k,
                   "step": "route + permute + gate_up/ScaledSwiGLU + down + combine (forward)",
                   "flop_per_step": flop},
        "pct_of_bf16_peak": round(100 * value / BF16_PEAK_TFLOPS, 2),
        "roofline": {"kernel": "grouped gate_up + ScaledSwiGLU (grouped_gemm_fwd_kernel<EPI_SWIGLU>)",
                     "bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
                     "avg_launch_ms": round(gate_ms, 4), "traffic": traffic},
    }
    del layer
    torch.cuda.empty_cache()

    if not args.quick:
        # MXFP8 on the same Mixtral tensors (the MXFP8 workload draws the same inputs)
        w8 = WORKLOADS["mixtral_mxfp8_fwd"]
        result["mxfp8_fwd"] = extra_forward(w8, inp, max(3, args.steps // 2), args.warmup, compute="mxfp8")
        result["mxfp8_fwd_prequantised"] = extra_forward(w8, inp, max(3, args.steps // 2), args.warmup,
                                                          compute="mxfp8", prequant=True)
        torch.cuda.empty_cache()
        # per-tensor FP8 on the same tensors (one scale per tensor; h goes through bf16)
        result["fp8_tensor_fwd"] = extra_forward(w8, inp, max(3, args.steps // 2), args.warmup, compute="fp8")
        result["fp8_tensor_fwd_prequantised"] = extra_forward(w8, inp, max(3, args.steps // 2), args.warmup,
                                                              compute="fp8", prequant=True)
        torch.cuda.empty_cache()
        wq = WORKLOADS["qwen3_fwd"]
        t0 = time.perf_counter()
        inpq = make_inputs(wq, want_float=False)
        log(f"inputs {wq.name}: {time.perf_counter() - t0:.1f} s")
        result["qwen3_fwd"] = extra_forward(wq, inpq, max(3, args.steps // 2), args.warmup)
        result["router"] = [router_measure(w, inp), router_measure(wq, inpq)]
        result["permute_combine"] = [memory_bound_measure(w, inp), memory_bound_measure(wq, inpq)]
        result["mxfp8_colwise"] = colwise_measure()
        del inpq
        torch.cuda.empty_cache()

    if not args.no_fwd_bwd:
        result["fwd_bwd"] = fwd_bwd_measure(max(3, args.steps // 2), args.warmup)
        torch.cuda.empty_cache()
        result["mxfp8_fwd_bwd"] = fwd_bwd_measure(max(3, args.steps // 2), args.warmup, mx=True)
        torch.cuda.empty_cache()
        result["mxfp8_fwd_bwd_prequantised"] = fwd_bwd_measure(max(3, args.steps // 2), args.warmup, mx=True,
                                                               prequant=True)
        torch.cuda.empty_cache()
        result["fp8_tensor_fwd_bwd"] = fwd_bwd_measure(max(3, args.steps // 2), args.warmup, fp8=True)
        torch.cuda.empty_cache()
        result["fp8_tensor_fwd_bwd_prequantised"] = fwd_bwd_measure(max(3, args.steps // 2), args.warmup,
                                                                    fp8=True, prequant=True)
        torch.cuda.empty_cache()
        result["mlp_bwd"] = bwd_measure()
        torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        t0 = time.perf_counter()
        result["cpu_baseline"] = cpu_baseline(inp, w, args.cpu_seconds)
        log(f"cpu baseline: {time.perf_counter() - t0:.1f} s")
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
