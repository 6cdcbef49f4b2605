"""Seeded synthetic inputs for the MoE expert feed-forward layer.

This module is shared by the CPU oracle and the HIP path's tests and benchmark,
and by nothing else. It holds no arithmetic of the method itself: only the
workload table, the random draws, and the float32 -> bfloat16 rounding that
turns a draw into a bf16 input tensor.

Workloads stand in for the layers the pages train (Mixtral-8x7B in
"Efficient MoE Training for Biological Foundation Models", Results; Qwen3 MoE
30B in the DGX H100 table of the PyTorch-native MoE library article). Their
datasets and weights are not available, so activations are N(0,1), weights
N(0, 0.02^2), router logits N(0,1), drawn from numpy SeedSequence streams.

Stream layout for a seed s: ``SeedSequence(s).spawn(6)`` gives six
generators g0..g5, used as
  g0: hidden_states x [T, H]
  g1: gate_up weights, expert by expert, each [2I, H] (rows [0, I) gate)
  g2: down weights, expert by expert, each [H, I]
  g3: router logits [T, E]
  g4: Zipf load skew: a permutation of expert ranks 1..E
  g5: upstream gradient dOut [T, H]
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    T: int
    H: int
    I: int
    E: int
    k: int
    dtype: str          # "f32", "bf16" or "mxfp8" (mxfp8: bf16 inputs quantised in the path)
    zipf: float = 0.0   # >0: add -zipf*ln(rank_e) to expert e's logit
    backward: bool = False
    note: str = ""

    @property
    def R(self) -> int:
        return self.T * self.k

    def gemm_flop_fwd(self) -> float:
        # gate_up (2*R*H*2I) + down (2*R*I*H)
        return 6.0 * self.R * self.H * self.I


WORKLOADS = {
    "tiny": Workload("tiny", 0, 256, 128, 256, 8, 2, "f32",
                     note="tiny MoE FFN, fp32, forward"),
    "mixtral_fwd": Workload("mixtral_fwd", 1, 8192, 4096, 14336, 8, 2, "bf16",
                            note="Mixtral-8x7B layer, 4x2048 tokens, bf16, forward"),
    "qwen3_fwd": Workload("qwen3_fwd", 5, 16384, 2048, 768, 128, 8, "bf16", zipf=1.2,
                          note="Qwen3-MoE-30B-A3B layer, Zipf(1.2)-skewed load, bf16, forward"),
    "mixtral_mxfp8_fwd": Workload("mixtral_mxfp8_fwd", 1, 8192, 4096, 14336, 8, 2, "mxfp8",
                                  note="Mixtral-8x7B layer, MXFP8 (E4M3 + E8M0 per 32 K), forward"),
    "mixtral_fwd_bwd": Workload("mixtral_fwd_bwd", 4, 4096, 4096, 14336, 8, 2, "bf16",
                                backward=True,
                                note="Mixtral-8x7B layer, bf16, forward + backward"),
}


def scaled(w: Workload, **over) -> Workload:
    """A copy of ``w`` with some fields replaced (smaller parity shapes)."""
    d = dict(w.__dict__)
    d.update(over)
    return Workload(**d)


# ---------------------------------------------------------------------------
# bfloat16 bit patterns (round to nearest, ties to even) kept as uint16 arrays.
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    return ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Inputs:
    """Host-side inputs. Floating tensors are float32 arrays; for bf16/mxfp8
    workloads they hold bf16-exact values and ``*_bits`` holds the uint16 patterns."""
    w: Workload
    x: np.ndarray
    w1: np.ndarray
    w2: np.ndarray
    logits: np.ndarray
    dout: np.ndarray | None = None
    bits: dict = field(default_factory=dict)


def _round_bf16(a: np.ndarray):
    b = f32_to_bf16_bits(a)
    return bf16_bits_to_f32(b), b


def make_inputs(w: Workload, want_float=True) -> Inputs:
    """Draw the workload's tensors. With ``want_float=False`` the large float32
    copies of bf16 tensors are dropped (only the bf16 bit patterns are kept)."""
    g = [np.random.default_rng(c) for c in np.random.SeedSequence(w.seed).spawn(6)]
    lowp = w.dtype in ("bf16", "mxfp8")
    bits = {}

    x = g[0].standard_normal((w.T, w.H), np.float32)
    w1 = np.empty((w.E, 2 * w.I, w.H), np.uint16 if lowp else np.float32)
    w2 = np.empty((w.E, w.H, w.I), np.uint16 if lowp else np.float32)
    for e in range(w.E):
        a = np.float32(0.02) * g[1].standard_normal((2 * w.I, w.H), np.float32)
        w1[e] = f32_to_bf16_bits(a) if lowp else a
    for e in range(w.E):
        a = np.float32(0.02) * g[2].standard_normal((w.H, w.I), np.float32)
        w2[e] = f32_to_bf16_bits(a) if lowp else a
    logits = g[3].standard_normal((w.T, w.E), np.float32)
    if w.zipf > 0:
        rank = g[4].permutation(w.E) + 1
        logits += (-w.zipf * np.log(rank)).astype(np.float32)[None, :]
    dout = g[5].standard_normal((w.T, w.H), np.float32) if w.backward else None

    if lowp:
        x, bits["x"] = _round_bf16(x)
        bits["w1"], bits["w2"] = w1, w2
        w1 = bf16_bits_to_f32(w1) if want_float else None
        w2 = bf16_bits_to_f32(w2) if want_float else None
        if dout is not None:
            dout, bits["dout"] = _round_bf16(dout)
    return Inputs(w, x, w1, w2, logits, dout, bits)


def make_grad(shape, seed: int, lowp: bool = True):
    """An extra N(0,1) tensor for op-level tests (e.g. an upstream gradient on
    permuted rows). Returns (float32 values, bf16 bits or None)."""
    a = np.random.default_rng(np.random.SeedSequence(seed)).standard_normal(shape, np.float32)
    if lowp:
        return _round_bf16(a)
    return a, None
