"""MXFP8 block quantisation, as a plain CPU reference (test infrastructure only).

"Efficient MoE Training for Biological Foundation Models", Challenge 2: MXFP8
gives every block of 32 consecutive values its own scaling factor and stores
each value in 8 bits; Challenge 3: bf16 master weights and activations are
converted to MXFP8 before the low-precision GEMM and the result is converted
back. The pages do not give the element format or the scale rule; the
readings used here are:

* elements are OCP FP8 E4M3 ("FN" variant): sign, 4 exponent bits with bias 7,
  3 mantissa bits, no infinities, 0x7F/0xFF are NaN, largest finite 448,
  smallest normal 2^-6, subnormal step 2^-9;
* the scale is an E8M0 power of two 2^s stored as the byte s + 127, one per
  32 contiguous values along the GEMM reduction (K) axis;
* s is the smallest integer with max|block| <= 448 * 2^s, clamped to
  [-127, 127]; an all-zero block gets s = -127 (byte 0);
* an element's code is E4M3 round-to-nearest, ties to the even mantissa, of
  x / 2^s (an exact division), keeping the sign bit of x.
"""
from __future__ import annotations

import os

import numpy as np

__all__ = [
    "E4M3_MAX", "e4m3_encode", "e4m3_decode", "e8m0_scale_exponent",
    "mxfp8_quantize", "mxfp8_dequantize", "mxfp8_qdq", "mxfp8_quantize_colwise",
]

E4M3_MAX = 448.0
_BLOCK = 32


def e4m3_encode(v) -> np.ndarray:
    """Round float64 values (|v| <= 448 expected) to E4M3 codes, RNE, saturating."""
    v = np.asarray(v, dtype=np.float64)
    sign = np.signbit(v).astype(np.uint8)
    a = np.minimum(np.abs(v), E4M3_MAX)
    mant, ex = np.frexp(a)            # a = mant * 2^ex, mant in [0.5, 1)
    e_unb = ex - 1                    # a = (2*mant) * 2^e_unb, 2*mant in [1, 2)
    normal = a >= 2.0 ** -6
    # normal range: 3 fractional mantissa bits at exponent e_unb
    q_norm = np.rint((2.0 * mant - 1.0) * 8.0)          # 0..8 (8: carry into exponent)
    e_field = e_unb + 7 + (q_norm == 8)
    m_field = np.where(q_norm == 8, 0, q_norm)
    # subnormal range: multiples of 2^-9
    q_sub = np.rint(a * 512.0)                           # 0..8 (8: smallest normal)
    code_sub = q_sub                                     # 8 -> exponent field 1, mantissa 0 = 0x08
    code_norm = e_field * 8 + m_field
    code = np.where(normal, code_norm, code_sub).astype(np.int64)
    code = np.minimum(code, 0x7E)                        # saturate to 448
    return (code.astype(np.uint8) | (sign << 7)).astype(np.uint8)


def e4m3_decode(c) -> np.ndarray:
    c = np.asarray(c, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((e == 0xF) & (m == 0x7), np.nan, val)
    return s * val


def e8m0_scale_exponent(amax) -> np.ndarray:
    """Smallest integer s with amax <= 448 * 2^s, found by exact comparisons,
    clamped to [-127, 127]; amax == 0 gives -127."""
    a = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(np.where(a > 0, a / E4M3_MAX, 1.0))
    s = ex.astype(np.int64)                 # first guess, within one of the answer
    for _ in range(3):
        too_small = a > E4M3_MAX * np.exp2(s.astype(np.float64))
        s = s + too_small
    for _ in range(3):
        smaller_ok = a <= E4M3_MAX * np.exp2(s.astype(np.float64) - 1.0)
        s = s - smaller_ok
    s = np.where(a > 0, s, -127)
    return np.clip(s, -127, 127)


def mxfp8_quantize(x):
    """x [rows, C] (C % 32 == 0) -> (E4M3 codes uint8 [rows, C], E8M0 bytes uint8 [rows, C/32])."""
    x = np.asarray(x, dtype=np.float64)
    rows, C = x.shape
    assert C % _BLOCK == 0
    blk = x.reshape(rows, C // _BLOCK, _BLOCK)
    s = e8m0_scale_exponent(np.abs(blk).max(axis=2))
    scaled = blk / np.exp2(s.astype(np.float64))[:, :, None]
    codes = e4m3_encode(scaled).reshape(rows, C)
    return codes, (s + 127).astype(np.uint8)


def mxfp8_dequantize(codes, scales) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8)
    rows, C = codes.shape
    v = e4m3_decode(codes).reshape(rows, C // _BLOCK, _BLOCK)
    s = np.asarray(scales, dtype=np.int64) - 127
    return (v * np.exp2(s.astype(np.float64))[:, :, None]).reshape(rows, C)


def mxfp8_qdq(x, rows_per_chunk: int = 2048) -> np.ndarray:
    """Quantise then dequantise (the naive separate-op path of Challenge 3).

    Every 32-value block lies inside one row, so rows are independent: inputs with
    more than rows_per_chunk rows are done in chunks of rows on host threads (numpy
    releases the interpreter lock in its array loops). The result is the same bits
    as one call on the whole array."""
    x = np.asarray(x, dtype=np.float64)
    if x.shape[0] <= rows_per_chunk:
        return mxfp8_dequantize(*mxfp8_quantize(x))
    from concurrent.futures import ThreadPoolExecutor
    out = np.empty_like(x)

    def one(r0):
        out[r0:r0 + rows_per_chunk] = mxfp8_dequantize(*mxfp8_quantize(x[r0:r0 + rows_per_chunk]))

    with ThreadPoolExecutor(max_workers=min(16, len(os.sched_getaffinity(0)))) as ex:
        list(ex.map(one, range(0, x.shape[0], rows_per_chunk)))
    return out


def mxfp8_quantize_colwise(x, offsets, pad, kcap):
    """MXFP8 along the token axis, expert by expert: the operand layout of a weight
    gradient, whose reduction runs over each expert's rows (the backward GEMMs take
    their operands in MXFP8 along their own K axis, Challenge 3's matching backward).

    x [R, C]; expert e owns rows [offsets[e], offsets[e+1]). Its rows, zero-padded to a
    multiple of `pad` (a multiple of 32), become columns [kofs[e], kofs[e+1]) of the
    transposed output and are quantised in blocks of 32 along that axis by the rule of
    mxfp8_quantize (all-padding blocks: scale byte 0, codes 0).
    Returns (codes [C, kcap] uint8, scales [C, kcap / 32] uint8, kofs [E + 1] int32);
    entries at and past kofs[E] are 0.
    """
    x = np.asarray(x, dtype=np.float64)
    R, C = x.shape
    offsets = np.asarray(offsets, dtype=np.int64)
    E = len(offsets) - 1
    assert pad % _BLOCK == 0 and kcap % _BLOCK == 0
    kofs = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        m = int(offsets[e + 1] - offsets[e])
        kofs[e + 1] = kofs[e] + -(-m // pad) * pad
    assert kofs[E] <= kcap
    codes = np.zeros((C, kcap), dtype=np.uint8)
    scales = np.zeros((C, kcap // _BLOCK), dtype=np.uint8)
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        kp = int(kofs[e + 1] - kofs[e])
        if kp == 0:
            continue
        seg = np.zeros((kp, C))
        seg[: b - a] = x[a:b]
        cq, sq = mxfp8_quantize(seg.T)
        codes[:, kofs[e]:kofs[e + 1]] = cq
        scales[:, kofs[e] // _BLOCK:kofs[e + 1] // _BLOCK] = sq
    return codes, scales, kofs.astype(np.int32)
