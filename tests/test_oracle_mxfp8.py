"""Pins for the oracle's MXFP8 quantiser (CPU only): fixed E4M3 code points,
a brute-force nearest-codebook search, the scale rule's bounds, scale
equivariance, exact round trips and idempotence."""
import json
import os

import numpy as np
import pytest

import oracle
from moe_inputs import bf16_bits_to_f32, f32_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _codebook():
    """All finite E4M3 values from the bit fields: sign, exponent (bias 7), mantissa."""
    vals = {}
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            continue
        mag = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
        vals[c] = -mag if s else mag
    return vals


def test_e4m3_fixed_points():
    g = json.load(open(os.path.join(GOLDEN, "e4m3_codes.json")))
    for case in g["codes"]:
        assert int(oracle.e4m3_encode(case["value"])) == case["code"], case
        assert float(oracle.e4m3_decode(case["code"])) == case["value"]
    for c in g["nan_codes"]:
        assert np.isnan(oracle.e4m3_decode(c))


def test_e4m3_decode_matches_codebook():
    cb = _codebook()
    codes = np.array(sorted(cb), np.uint8)
    np.testing.assert_array_equal(oracle.e4m3_decode(codes), [cb[int(c)] for c in codes])


def test_e4m3_encode_brute_force_nearest_ties_to_even():
    cb = _codebook()
    pos = sorted((v, c) for c, v in cb.items() if c < 128)      # non-negative codes
    grid = set(np.linspace(0, 448, 20001).tolist())
    for (a, _), (b, _) in zip(pos, pos[1:]):
        grid.update([(a + b) / 2, a, b, np.nextafter((a + b) / 2, 0), np.nextafter((a + b) / 2, 1e9)])
    grid = np.array(sorted(grid))
    vals = np.array([v for v, _ in pos])
    codes = np.array([c for _, c in pos])
    expect = []
    for x in grid:
        d = np.abs(vals - x)
        best = np.flatnonzero(d == d.min())
        if len(best) > 1:                       # a tie: the even mantissa wins
            best = [b for b in best if codes[b] % 2 == 0]
        expect.append(codes[best[0]])
    got = oracle.e4m3_encode(grid)
    np.testing.assert_array_equal(got, expect)
    np.testing.assert_array_equal(oracle.e4m3_encode(-grid[1:]), np.array(expect[1:]) | 0x80)


def test_e8m0_scale_brute_force():
    rng = np.random.default_rng(0)
    amax = np.concatenate([np.exp2(rng.uniform(-140, 125, 3000)),
                           448 * np.exp2(np.arange(-20, 20, dtype=np.float64)),
                           np.nextafter(448 * np.exp2(np.arange(-5, 5.0)), np.inf)])
    s = oracle.e8m0_scale_exponent(amax)
    for a, si in zip(amax, s):
        want = next(t for t in range(-127, 128) if a <= 448 * 2.0 ** t) if a <= 448 * 2.0 ** 127 else 127
        assert si == want
    assert oracle.e8m0_scale_exponent(0.0) == -127


def _bf16_blocks(rows=64, cols=256, seed=0, spread=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    if spread:
        x *= np.exp2(rng.integers(-30, 30, (rows, cols // 32))).repeat(32, 1).astype(np.float32)
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


def test_quantize_scale_bounds_and_zero_block():
    x = _bf16_blocks()
    x[3, 32:64] = 0.0
    codes, scales = oracle.mxfp8_quantize(x)
    amax = np.abs(x.reshape(64, 8, 32)).max(2)
    scale = np.exp2(scales.astype(np.float64) - 127)
    nz = amax > 0
    assert (amax[nz] / scale[nz] <= 448).all()
    assert (amax[nz] / scale[nz] > 224).all()            # smallest such power of two
    assert scales[3, 1] == 0 and not codes[3, 32:64].any()
    # no code is NaN and the largest element of each block lands in the top binade
    assert not np.isnan(oracle.e4m3_decode(codes)).any()


def test_quantize_equivariance_roundtrip_idempotence():
    x = _bf16_blocks(seed=1)
    codes, scales = oracle.mxfp8_quantize(x)
    for j in (-7, 1, 12):
        c2, s2 = oracle.mxfp8_quantize(x * 2.0 ** j)
        np.testing.assert_array_equal(c2, codes)
        np.testing.assert_array_equal(s2.astype(int), scales.astype(int) + j)
    dq = oracle.mxfp8_dequantize(codes, scales)
    # already representable: the values survive a second pass unchanged; the codes
    # too, except where the block maximum rounded down to 224 * scale, which moves
    # the block one binade down (same values, scale one smaller)
    c3, s3 = oracle.mxfp8_quantize(dq)
    np.testing.assert_array_equal(oracle.mxfp8_dequantize(c3, s3), dq)
    amax_dq = np.abs(dq.reshape(dq.shape[0], -1, 32)).max(2)
    same = amax_dq > 224 * np.exp2(scales.astype(np.float64) - 127)
    np.testing.assert_array_equal(s3[same], scales[same])
    np.testing.assert_array_equal(s3[~same].astype(int), scales[~same].astype(int) - 1)
    np.testing.assert_array_equal(c3.reshape(dq.shape[0], -1, 32)[same], codes.reshape(dq.shape[0], -1, 32)[same])
    np.testing.assert_array_equal(oracle.mxfp8_qdq(dq), dq)
    # relative error of a normal-range element is at most half an E4M3 ulp (2^-4)
    big = np.abs(dq) >= np.exp2(scales.astype(float) - 127 - 6).repeat(32, 1)
    rel = np.abs(dq - x)[big] / np.abs(x)[big]
    assert rel.max() <= 2.0 ** -4 + 1e-12


def test_quantize_commutes_with_row_permutation():
    x = _bf16_blocks(seed=2)
    perm = np.random.default_rng(3).permutation(x.shape[0])
    c, s = oracle.mxfp8_quantize(x)
    cp, sp = oracle.mxfp8_quantize(x[perm])
    np.testing.assert_array_equal(cp, c[perm])
    np.testing.assert_array_equal(sp, s[perm])


def test_mxfp8_mlp_equals_exact_mlp_on_representable_inputs():
    """With x, W1, W2 already MX-representable only h is rounded: the MXFP8
    reference then equals the exact MLP run on the rounded h."""
    from moe_inputs import WORKLOADS, make_inputs, scaled
    inp = make_inputs(scaled(WORKLOADS["tiny"], T=40, H=64, I=64, E=4, k=2, seed=3, dtype="bf16"))
    x = oracle.mxfp8_qdq(inp.x)
    w1 = np.stack([oracle.mxfp8_qdq(w) for w in inp.w1])
    w2 = np.stack([oracle.mxfp8_qdq(w) for w in inp.w2])
    idx, p = oracle.route_topk(inp.logits, 2)
    m = oracle.permute(idx, 4)
    xp = oracle.gather_rows(x, m["src_token"])
    pp = p.ravel()[m["src_token"] * 2 + m["src_slot"]]
    y8, h = oracle.grouped_mlp_forward_mxfp8(xp, w1, w2, m["offsets"], pp)
    _, z_exact, h_exact = oracle.grouped_mlp_forward(xp, w1, w2, m["offsets"], pp)
    np.testing.assert_allclose(h, h_exact, rtol=1e-13, atol=1e-16)
    # the gate_up product it returns on request is the exact one too, and asking for it
    # changes nothing else
    y8z, hz, z8 = oracle.grouped_mlp_forward_mxfp8(xp, w1, w2, m["offsets"], pp, return_z=True)
    np.testing.assert_allclose(z8, z_exact, rtol=1e-13, atol=1e-14)
    assert np.array_equal(y8z, y8) and np.array_equal(hz, h)
    y_ref = np.zeros_like(y8)
    hq = oracle.mxfp8_qdq(h)
    for e in range(4):
        a, b = m["offsets"][e], m["offsets"][e + 1]
        y_ref[a:b] = hq[a:b] @ w2[e].T
    np.testing.assert_allclose(y8, y_ref, rtol=1e-12, atol=1e-14)


def test_colwise_brute_force_tiny():
    """Column-wise (per expert, along the token axis) quantisation against a direct
    per-element construction: blocks of 32 along each expert's zero-padded rows, the
    scale by search over exponents, every code by the nearest codebook value."""
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((45, 3)) * np.exp2(rng.integers(-8, 8, (45, 3)))).astype(np.float32)
    x[10, 1] = -0.0
    off = np.array([0, 7, 7, 45])
    codes, scales, kofs = oracle.mxfp8_quantize_colwise(x, off, 32, 128)
    assert list(kofs) == [0, 32, 32, 96]      # 7 and 38 rows padded to 32 and 64
    cb = _codebook()
    items = sorted(cb.items())
    for c in range(3):
        for e in range(3):
            col = np.zeros(int(kofs[e + 1] - kofs[e]))
            col[: off[e + 1] - off[e]] = x[off[e]:off[e + 1], c]
            for blk in range(len(col) // 32):
                v = col[32 * blk: 32 * blk + 32]
                a = np.abs(v).max()
                s = -127 if a == 0 else next(t for t in range(-127, 128) if a <= 448 * 2.0 ** t)
                assert scales[c, kofs[e] // 32 + blk] == s + 127
                for i, xv in enumerate(v):
                    q = xv / 2.0 ** s
                    d = [(abs(val - q), code) for code, val in items if (code >> 7) == (1 if np.signbit(xv) else 0)]
                    dmin = min(dd for dd, _ in d)
                    best = [code for dd, code in d if dd == dmin]
                    if len(best) > 1:
                        best = [b for b in best if b % 2 == 0]
                    assert codes[c, kofs[e] + 32 * blk + i] == best[0], (c, e, blk, i)
    assert not codes[:, 96:].any() and not scales[:, 3:].any()


def test_colwise_padding_and_segment_independence():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((300, 64)).astype(np.float32)
    off = np.array([0, 40, 40, 300])
    codes, scales, kofs = oracle.mxfp8_quantize_colwise(x, off, 256, 1024)
    assert list(kofs) == [0, 256, 256, 768]   # 40 and 260 rows padded to 256 and 512
    # expert 0 has 40 rows: blocks 2..7 of its padded range are all padding
    assert not scales[:, 2:8].any() and not codes[:, 64:256].any()
    assert not codes[:, 40:64].any()          # the padded tail of block 1 is code 0
    # changing expert 0's rows leaves expert 2's columns alone
    y = x.copy()
    y[:40] *= 3.0
    c2, s2, _ = oracle.mxfp8_quantize_colwise(y, off, 256, 1024)
    assert np.array_equal(c2[:, 256:], codes[:, 256:]) and np.array_equal(s2[:, 8:], scales[:, 8:])


def _bwd_case(seed=5, sizes=(37, 0, 70), H=64, I=64):
    """Small backward inputs: saved z = x W1^T and h = silu(G) U p from the exact forward."""
    rng = np.random.default_rng(seed)
    E = len(sizes)
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    R = int(off[-1])
    x = rng.standard_normal((R, H))
    w1 = 0.1 * rng.standard_normal((E, 2 * I, H))
    w2 = 0.1 * rng.standard_normal((E, H, I))
    p = rng.uniform(0.1, 1.0, R)
    dy = rng.standard_normal((R, H))
    _, z, h = oracle.grouped_mlp_forward(x, w1, w2, off, p)
    return dict(dy_perm=dy, x_perm=x, z_save=z, h_save=h, w_gate_up=w1, w_down=w2, offsets=off, prob_perm=p)


def test_mxfp8_backward_without_quantisation_is_the_exact_backward():
    """Dropping every quantiser leaves the bf16 backward's formulas (which recompute z
    from x and W1): the two must agree to float64 round-off, with zero weight gradients
    for the empty expert."""
    c = _bwd_case()
    got = oracle.grouped_mlp_backward_mxfp8(**c, quantize=False)
    ref = oracle.grouped_mlp_backward(c["dy_perm"], c["x_perm"], c["w_gate_up"], c["w_down"], c["offsets"],
                                      c["prob_perm"])
    for k in ref:
        np.testing.assert_allclose(got[k], ref[k], rtol=1e-11, atol=1e-12)
    assert not got["dw_gate_up"][1].any() and not got["dw_down"][1].any()


def test_mxfp8_backward_quantises_each_gemm_along_its_reduction_axis():
    """Power-of-two rescalings that MX quantisation along the stated axis carries through
    exactly (a block's scale absorbs them) but quantisation along the other axis would
    not: K-blocks of the dH GEMM (dY's columns and W2's rows in one 32-block of H, in
    opposite directions), one column of W1 (the dx GEMM quantises W1 along 2I), one
    column of x, dY or h (the weight-gradient GEMMs quantise along the expert's rows)."""
    c = _bwd_case()
    base = oracle.grouped_mlp_backward_mxfp8(**c)
    # 1. dH = Q_H(dY) Q_H(W2): a 32-block of H scaled by 2^5 in dY and 2^-5 in W2
    c1 = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in c.items()}
    c1["dy_perm"][:, 32:64] *= 2.0 ** 5
    c1["w_down"][:, 32:64, :] *= 2.0 ** -5
    r1 = oracle.grouped_mlp_backward_mxfp8(**c1)
    np.testing.assert_array_equal(r1["dprob_perm"], base["dprob_perm"])
    np.testing.assert_array_equal(r1["dx_perm"], base["dx_perm"])
    np.testing.assert_array_equal(r1["dw_gate_up"], base["dw_gate_up"])
    # the same rescaling over a block that straddles two K-blocks does change dH
    c1b = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in c.items()}
    c1b["dy_perm"][:, 16:48] *= 2.0 ** 5
    c1b["w_down"][:, 16:48, :] *= 2.0 ** -5
    assert not np.array_equal(oracle.grouped_mlp_backward_mxfp8(**c1b)["dprob_perm"], base["dprob_perm"])
    # 2. dx = Q_2I(dZ) Q_2I(W1): column 7 of every W1 scaled by 2^3 scales column 7 of dx
    c2 = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in c.items()}
    c2["w_gate_up"][:, :, 7] *= 8.0
    r2 = oracle.grouped_mlp_backward_mxfp8(**c2)
    want = base["dx_perm"].copy()
    want[:, 7] *= 8.0
    np.testing.assert_array_equal(r2["dx_perm"], want)
    # 3. dW1 = Q_tok(dZ)^T Q_tok(x): column 5 of x scaled by 2^4 scales column 5 of dW1
    c3 = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in c.items()}
    c3["x_perm"][:, 5] *= 16.0
    r3 = oracle.grouped_mlp_backward_mxfp8(**c3)
    want = base["dw_gate_up"].copy()
    want[:, :, 5] *= 16.0
    np.testing.assert_array_equal(r3["dw_gate_up"], want)
    # 4. dW2 = Q_tok(dY)^T Q_tok(h): column 9 of h scales column 9 of dW2; column 3 of dY
    #    scales row 3 of dW2 (dY also feeds dH, whose blocks it changes: not checked here)
    c4 = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in c.items()}
    c4["h_save"][:, 9] *= 4.0
    c4["dy_perm"][:, 3] *= 0.5
    r4 = oracle.grouped_mlp_backward_mxfp8(**c4)
    want = base["dw_down"].copy()
    want[:, :, 9] *= 4.0
    want[:, 3, :] *= 0.5
    np.testing.assert_array_equal(r4["dw_down"], want)


def test_mxfp8_backward_token_blocks_start_at_each_expert():
    """The token-axis blocks of the weight gradients restart at every expert's first
    row: moving rows from expert 0 to expert 2's range through an empty expert must not
    change expert 2's gradient when its own rows and their order are unchanged, and an
    expert's gradient equals a one-expert call on its rows alone."""
    c = _bwd_case(sizes=(37, 0, 70))
    base = oracle.grouped_mlp_backward_mxfp8(**c)
    a, b = 37, 107
    solo = {k: (v[a:b] if k in ("dy_perm", "x_perm", "z_save", "h_save", "prob_perm") else v)
            for k, v in c.items()}
    solo["offsets"] = np.array([0, 0, 0, b - a])
    r = oracle.grouped_mlp_backward_mxfp8(**solo)
    np.testing.assert_array_equal(r["dw_down"][2], base["dw_down"][2])
    np.testing.assert_array_equal(r["dw_gate_up"][2], base["dw_gate_up"][2])


def test_qdq_row_chunks_give_the_same_bits():
    # quantisation blocks lie within rows: the threaded row-chunked qdq must equal one
    # pass over the whole array, bit for bit (negative zeros and all-zero blocks included)
    rng = np.random.default_rng(31)
    x = rng.standard_normal((300, 96)) * np.exp2(rng.integers(-20, 20, (300, 1)))
    x[5] = 0.0
    x[7, :32] = -0.0
    whole = oracle.mxfp8_qdq(x, rows_per_chunk=1 << 30)
    for chunk in (1, 7, 64, 299):
        got = oracle.mxfp8_qdq(x, rows_per_chunk=chunk)
        assert np.array_equal(got.view(np.uint64), whole.view(np.uint64)), chunk
