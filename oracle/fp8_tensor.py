"""Per-tensor FP8 (E4M3) quantisation and the grouped MLP forward on it, as a plain CPU
reference (test infrastructure only).

"Efficient MoE Training for Biological Foundation Models", Challenge 2 contrasts FP8,
where one scaling factor covers a whole tensor, with MXFP8's one factor per 32 values.
The pages give no FP8 scale rule; the reading used here ("current scaling"):

* the scale of a tensor is s = amax / 448 in float32 (amax = max |x| over the whole
  tensor; s = 1 for an all-zero tensor), so the largest magnitude maps to E4M3's 448;
* an element's code is the OCP E4M3 code (rule of mxfp8.e4m3_encode: round to nearest,
  ties to even, saturating, sign kept) of the float32 quotient x / s;
* in the grouped MLP forward, x_perm is one tensor and each expert's W1_e and W2_e is
  one tensor; h is materialised in bf16 (its scale needs the whole tensor's amax first)
  and quantised from that bf16 value as one tensor; GEMM products are exact, sums
  float64 here; y = (h_q W2_e,q^T) s_h s_w2,e.

All arithmetic is float64 except the float32 scale and quotient, which fix the codes.
"""
from __future__ import annotations

import numpy as np

from .mxfp8 import E4M3_MAX, e4m3_decode, e4m3_encode

__all__ = ["fp8_tensor_scale", "fp8_tensor_quantize", "fp8_tensor_qdq", "bf16_round", "BF16_MAX", "grouped_mlp_forward_fp8_tensor"]


def fp8_tensor_scale(x) -> np.float32:
    """float32 scale amax / 448 of a whole tensor (1 for an all-zero or empty tensor)."""
    a = np.asarray(x, np.float32)
    amax = np.float32(np.max(np.abs(a))) if a.size else np.float32(0.0)
    return np.float32(amax / np.float32(E4M3_MAX)) if amax > 0 else np.float32(1.0)


def fp8_tensor_quantize(x, scale=None):
    """(codes uint8, scale float32) of a whole tensor; scale: use this float32 scale
    instead of the tensor's own (for a part of a larger tensor)."""
    a = np.asarray(x, np.float32)
    s = fp8_tensor_scale(a) if scale is None else np.float32(scale)
    q = (a / s).astype(np.float32)      # the float32 quotient decides the code
    return e4m3_encode(q.astype(np.float64)), s


def fp8_tensor_qdq(x, scale=None, chunk: int = 1 << 22) -> np.ndarray:
    """Quantise then dequantise a whole tensor. The factor needs the whole tensor; the
    codes are elementwise, so tensors of more than `chunk` elements are encoded in
    chunks on host threads (numpy releases the interpreter lock in its array loops):
    the same bits as one call on the whole tensor."""
    a = np.asarray(x, np.float32)
    if a.size <= chunk:
        codes, s = fp8_tensor_quantize(a, scale)
        return e4m3_decode(codes) * np.float64(s)
    import os
    from concurrent.futures import ThreadPoolExecutor
    s = fp8_tensor_scale(a) if scale is None else np.float32(scale)
    flat = a.reshape(-1)
    out = np.empty(flat.size, np.float64)

    def one(i):
        codes, _ = fp8_tensor_quantize(flat[i:i + chunk], s)
        out[i:i + chunk] = e4m3_decode(codes) * np.float64(s)

    with ThreadPoolExecutor(max_workers=min(16, len(os.sched_getaffinity(0)))) as ex:
        list(ex.map(one, range(0, flat.size, chunk)))
    return out.reshape(a.shape)


BF16_MAX = float.fromhex("0x1.fep127")   # largest finite bfloat16: (2 - 2^-7) * 2^127


def bf16_round(a):
    """float64 -> the nearest bfloat16 value, ties to the even significand, as float64.

    bfloat16 keeps 8 significant bits and float32's exponent range: values in
    [2^e, 2^(e+1)) with e >= -126 are spaced 2^(e-7), values below 2^-126 are
    multiples of 2^-133 (subnormals). The value is divided by its spacing (exact: a
    power of two), rounded half to even by np.rint, and scaled back (exact). Results
    beyond the largest finite value become +-inf (IEEE rounding of an overflow);
    zeros, infinities and NaN pass through. There is no float32 step in between, so
    no double rounding. Large inputs are rounded in chunks on host threads (the
    rounding is elementwise: the same bits)."""
    a = np.asarray(a, np.float64)
    if a.size > (1 << 22):
        import os
        from concurrent.futures import ThreadPoolExecutor
        flat = a.reshape(-1)
        res = np.empty_like(flat)
        step = 1 << 22

        def one(i):
            res[i:i + step] = _bf16_round_flat(flat[i:i + step])

        with ThreadPoolExecutor(max_workers=min(16, len(os.sched_getaffinity(0)))) as ex:
            list(ex.map(one, range(0, flat.size, step)))
        return res.reshape(a.shape)
    return _bf16_round_flat(a)


def _bf16_round_flat(a):
    out = np.array(a, dtype=np.float64, copy=True)
    fin = np.isfinite(a) & (a != 0)
    v = a[fin]
    _, ex = np.frexp(np.abs(v))              # |v| = m * 2^ex, m in [0.5, 1)
    e = np.maximum(ex - 1, -126)             # exponent of the binade, subnormals at -126
    step = np.ldexp(1.0, e - 7)
    r = np.rint(v / step) * step
    r = np.where(np.abs(r) > BF16_MAX, np.copysign(np.inf, r), r)
    out[fin] = r
    return out


def grouped_mlp_forward_fp8_tensor(x_perm, w_gate_up, w_down, offsets, prob_perm, x_scale=None, return_zh=False):
    """y_perm [R, H] of the grouped MLP with every GEMM operand quantised per tensor.
    x_scale: x_perm's scale when x_perm is part of a larger tensor (default: its own).
    return_zh: also return z [R, 2I] (the gate_up product of the quantised operands)
    and h [R, I] (the bf16 value of h that is quantised), as (y, z, h)."""
    x = np.asarray(x_perm, np.float64)
    w1 = np.asarray(w_gate_up, np.float64)
    w2 = np.asarray(w_down, np.float64)
    p = np.asarray(prob_perm, np.float64)
    E, twoI, H = w1.shape
    I = twoI // 2
    R = x.shape[0]
    xq = fp8_tensor_qdq(x, x_scale)
    h = np.zeros((R, I))
    z_all = np.zeros((R, 2 * I))
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b == a:
            continue
        z = xq[a:b] @ fp8_tensor_qdq(w1[e]).T
        z_all[a:b] = z
        g, u = z[:, :I], z[:, I:]
        h[a:b] = g / (1.0 + np.exp(-g)) * u * p[a:b, None]
    hb = bf16_round(h)
    hq = fp8_tensor_qdq(hb)
    y = np.zeros((R, H))
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            y[a:b] = hq[a:b] @ fp8_tensor_qdq(w2[e]).T
    return (y, z_all, hb) if return_zh else y
