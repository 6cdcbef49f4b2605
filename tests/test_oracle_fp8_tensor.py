"""Pins for the oracle's per-tensor FP8 quantisation and the grouped MLP forward on it
(CPU only): the scale rule at the tensor maximum, the round-off bound of E4M3, exact
power-of-two equivariance, identity on representable tensors, and per-expert weight
scales (an expert with small weights keeps its accuracy next to a large one)."""
import numpy as np
import pytest

import oracle


def _e4m3_half_ulp(v):
    """Half the E4M3 spacing at |v| (|v| <= 448)."""
    a = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    return 0.5 * np.where(a >= 2.0 ** -6, 2.0 ** (e - 3), 2.0 ** -9)


def test_tensor_maximum_maps_to_448():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((37, 19)).astype(np.float32)
    codes, s = oracle.fp8_tensor_quantize(x)
    i = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert codes[i] & 0x7F == 0x7E
    assert s == np.float32(np.float32(np.abs(x).max()) / np.float32(448.0))


def test_round_off_bound():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(5000) * np.exp(rng.uniform(-6, 3, 5000))).astype(np.float32)
    codes, s = oracle.fp8_tensor_quantize(x)
    q = x.astype(np.float64) / np.float64(s)
    err = np.abs(oracle.e4m3_decode(codes) - np.minimum(np.abs(q), 448.0) * np.sign(q))
    assert np.all(err <= _e4m3_half_ulp(q) * (1 + 2.0 ** -20) + 1e-12)


@pytest.mark.parametrize("k", [-3, 5])
def test_power_of_two_equivariance(k):
    rng = np.random.default_rng(2)
    x = rng.standard_normal((64, 33)).astype(np.float32)
    a = oracle.fp8_tensor_qdq(x)
    b = oracle.fp8_tensor_qdq(x * np.float32(2.0 ** k))
    assert np.array_equal(b, a * 2.0 ** k)


def test_zero_tensor():
    codes, s = oracle.fp8_tensor_quantize(np.zeros((4, 8), np.float32))
    assert s == 1.0 and not codes.any()


def test_identity_on_representable_tensors():
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 256, (40, 24)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x10          # no NaN codes
    x = oracle.e4m3_decode(codes) * 2.0 ** -3
    x[0, 0] = 448.0 * 2.0 ** -3                     # amax / 448 = 2^-3 exactly
    assert np.array_equal(oracle.fp8_tensor_qdq(x.astype(np.float32)), x)


def test_forward_close_to_bf16_forward_and_per_expert_weight_scales():
    rng = np.random.default_rng(4)
    E, H, I = 3, 32, 16
    sizes = [9, 0, 14]
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    R = int(off[-1])
    x = rng.standard_normal((R, H))
    w1 = 0.1 * rng.standard_normal((E, 2 * I, H))
    w2 = 0.1 * rng.standard_normal((E, H, I))
    w2[2] *= 1e-5   # expert 2's down weights: below E4M3's range under a scale shared with expert 0
    p = rng.uniform(0.1, 1.0, R)
    y = oracle.grouped_mlp_forward_fp8_tensor(x, w1, w2, off, p)
    ref, _, _ = oracle.grouped_mlp_forward(x, w1, w2, off, p)
    for e in range(E):
        a, b = off[e], off[e + 1]
        if b > a:   # one scale per expert weight keeps every expert within FP8 accuracy
            rel = np.abs(y[a:b] - ref[a:b]).max() / np.abs(ref[a:b]).max()
            assert rel <= 8e-2, (e, rel)


# ---------------------------------------------------------------------------------
# grouped MLP backward with per-tensor FP8 operands
# ---------------------------------------------------------------------------------

def _representable(rng, shape, k):
    """A tensor whose per-tensor FP8 quantisation is the identity: E4M3 values times
    2^k, with one element at 448 * 2^k so that amax / 448 = 2^k exactly."""
    codes = rng.integers(0, 256, shape).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38            # no NaN codes (0x38 = 1.0)
    x = oracle.e4m3_decode(codes) * 2.0 ** k
    if x.size:
        x.flat[0] = 448.0 * 2.0 ** k
    return x


def _brute_tensor_qdq(t):
    """Per-tensor E4M3 quantisation by search over the 256 codes: the float32 factor
    amax / 448, the float32 quotient, then the nearest codebook value (ties: the value
    with an even code), times the factor."""
    t32 = np.asarray(t, np.float32)
    amax = np.float32(np.abs(t32).max())
    s = np.float32(amax / np.float32(448.0)) if amax > 0 else np.float32(1.0)
    q = (t32 / s).astype(np.float64).ravel()
    codes = np.arange(256)
    vals = oracle.e4m3_decode(codes.astype(np.uint8))
    ok = ~np.isnan(vals)
    codes, vals = codes[ok], vals[ok]
    out = np.empty_like(q)
    for i, v in enumerate(q):
        d = np.abs(vals - v)
        best = np.flatnonzero(d == d.min())
        if len(best) > 1:                               # a tie: keep the even code
            best = best[(codes[best] & 1) == 0]
            best = best[np.argmin(np.abs(vals[best]))] if len(best) > 1 else best[0]
        else:
            best = best[0]
        out[i] = vals[best] * np.float64(s)
    return out.reshape(np.shape(t))


def _fp8_bwd_case(seed=11, sizes=(23, 0, 31), H=32, I=16):
    rng = np.random.default_rng(seed)
    E = len(sizes)
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    R = int(off[-1])
    x = _representable(rng, (R, H), -2)
    dy = _representable(rng, (R, H), -4)
    # per-expert weight factors differ (2^-7, 2^-5, 2^-9): one factor shared by the
    # experts would not leave every expert's weight representable
    w1 = np.stack([_representable(rng, (2 * I, H), k) for k in (-7, -5, -9)])
    w2 = np.stack([_representable(rng, (H, I), k) for k in (-8, -6, -10)])
    p = rng.uniform(0.1, 1.0, R)
    _, z, h = oracle.grouped_mlp_forward(x, w1, w2, off, p)
    h = _representable(rng, (R, I), -3)                 # the saved h, taken as given
    return dict(dy_perm=dy, x_perm=x, z_save=z, h_save=h, w_gate_up=w1, w_down=w2, offsets=off, prob_perm=p)


def test_fp8_backward_without_quantisation_is_the_exact_backward():
    """Dropping every quantiser leaves the bf16 backward's formulas (which recompute z
    from x and W1 and h from z): equal to float64 round-off when the saved z and h are
    the exact forward's, with zero weight gradients for the empty expert."""
    rng = np.random.default_rng(5)
    sizes = (37, 0, 70)
    E, H, I = 3, 64, 64
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    R = int(off[-1])
    x = rng.standard_normal((R, H))
    w1 = 0.1 * rng.standard_normal((E, 2 * I, H))
    w2 = 0.1 * rng.standard_normal((E, H, I))
    p = rng.uniform(0.1, 1.0, R)
    dy = rng.standard_normal((R, H))
    _, z, h = oracle.grouped_mlp_forward(x, w1, w2, off, p)
    got = oracle.grouped_mlp_backward_fp8_tensor(dy, x, z, h, w1, w2, off, p, quantize=False)
    ref = oracle.grouped_mlp_backward(dy, x, w1, w2, off, p)
    for k in ref:
        np.testing.assert_allclose(got[k], ref[k], rtol=1e-11, atol=1e-12)
    assert not got["dw_gate_up"][1].any() and not got["dw_down"][1].any()


def test_fp8_backward_quantises_each_tensor_once_with_one_factor():
    """On operands that per-tensor FP8 represents exactly (per-expert weight factors
    that differ), the quantised backward without the bf16 roundings equals the
    unquantised one wherever dZ does not enter (dprob, dW2), and dx, dW1 equal the
    unquantised dZ passed through a brute-force per-tensor quantiser over all rows (one
    factor, not one per expert) times the exact W1 and x."""
    c = _fp8_bwd_case()
    got = oracle.grouped_mlp_backward_fp8_tensor(**c, round_bf16=False)
    ref = oracle.grouped_mlp_backward_fp8_tensor(**c, quantize=False)
    np.testing.assert_array_equal(got["dprob_perm"], ref["dprob_perm"])
    np.testing.assert_array_equal(got["dw_down"], ref["dw_down"])
    dzq = _brute_tensor_qdq(ref["dz_perm"])
    off = c["offsets"]
    for e in range(3):
        a, b = int(off[e]), int(off[e + 1])
        if a == b:
            assert not got["dw_gate_up"][e].any() and not got["dw_down"][e].any()
            continue
        np.testing.assert_allclose(got["dx_perm"][a:b], dzq[a:b] @ c["w_gate_up"][e], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(got["dw_gate_up"][e], dzq[a:b].T @ c["x_perm"][a:b], rtol=1e-12, atol=1e-14)
    # the experts' dZ magnitudes differ, so a factor per expert would quantise differently
    amax = [np.abs(ref["dz_perm"][off[e]:off[e + 1]]).max() for e in (0, 2)]
    assert max(amax) > 2 * min(amax)


def test_fp8_backward_rounds_dh_and_dz_to_bf16():
    """With round_bf16 the dZ that is quantised is a bf16 value and differs from the
    unrounded one; both readings stay within FP8 accuracy of the exact gradients."""
    c = _fp8_bwd_case(seed=12)
    r1 = oracle.grouped_mlp_backward_fp8_tensor(**c)
    r0 = oracle.grouped_mlp_backward_fp8_tensor(**c, round_bf16=False)
    ex = oracle.grouped_mlp_backward_fp8_tensor(**c, quantize=False)
    dz = r1["dz_perm"]
    assert np.array_equal(oracle.bf16_round(dz), dz) and not np.array_equal(r0["dz_perm"], dz)
    for r in (r0, r1):
        for k in ("dx_perm", "dw_gate_up", "dprob_perm"):
            rel = np.abs(r[k] - ex[k]).max() / np.abs(ex[k]).max()
            assert rel < 0.1, (k, rel)


def test_fp8_backward_no_rows():
    c = _fp8_bwd_case(sizes=(0, 0, 0))
    r = oracle.grouped_mlp_backward_fp8_tensor(**c)
    for k in ("dx_perm", "dw_gate_up", "dw_down", "dprob_perm"):
        assert not r[k].any()


def test_fp8_backward_matches_brute_force_quantisation_on_generic_operands():
    """Generic (not representable) operands: the quantised backward without the bf16
    roundings equals the unquantised backward run on operands that a brute-force
    per-tensor quantiser has already quantised (dY, x, h over all rows; W1_e, W2_e per
    expert) wherever dZ does not enter, and dx, dW1 are its own dZ quantised the same
    way times those operands."""
    rng = np.random.default_rng(13)
    sizes = (19, 0, 26, 7)
    E, H, I = len(sizes), 32, 16
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    R = int(off[-1])
    x = rng.standard_normal((R, H)).astype(np.float32).astype(np.float64)
    dy = rng.standard_normal((R, H)).astype(np.float32).astype(np.float64)
    w1 = (np.stack([s * rng.standard_normal((2 * I, H)) for s in (0.1, 0.02, 0.3, 0.05)])).astype(np.float32).astype(np.float64)
    w2 = (np.stack([s * rng.standard_normal((H, I)) for s in (0.07, 0.4, 0.01, 0.2)])).astype(np.float32).astype(np.float64)
    p = rng.uniform(0.1, 1.0, R)
    _, z, h = oracle.grouped_mlp_forward(x, w1, w2, off, p)
    h = h.astype(np.float32).astype(np.float64)
    got = oracle.grouped_mlp_backward_fp8_tensor(dy, x, z, h, w1, w2, off, p, round_bf16=False)
    qw1 = np.stack([_brute_tensor_qdq(w) for w in w1])
    qw2 = np.stack([_brute_tensor_qdq(w) for w in w2])
    qx = _brute_tensor_qdq(x)
    pre = oracle.grouped_mlp_backward_fp8_tensor(_brute_tensor_qdq(dy), qx, z, _brute_tensor_qdq(h), qw1, qw2, off, p,
                                                 quantize=False)
    np.testing.assert_array_equal(got["dprob_perm"], pre["dprob_perm"])
    np.testing.assert_array_equal(got["dw_down"], pre["dw_down"])
    dzq = _brute_tensor_qdq(got["dz_perm"].astype(np.float32))
    for e in range(E):
        a, b = int(off[e]), int(off[e + 1])
        if a == b:
            continue
        np.testing.assert_allclose(got["dx_perm"][a:b], dzq[a:b] @ qw1[e], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(got["dw_gate_up"][e], dzq[a:b].T @ qx[a:b], rtol=1e-12, atol=1e-14)


def test_qdq_chunks_give_the_same_bits():
    # the factor is the whole tensor's; the threaded chunked encoding equals one call
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((300, 70)) * np.exp(rng.uniform(-8, 4, (300, 70)))).astype(np.float32)
    whole = oracle.fp8_tensor_qdq(x)
    assert np.array_equal(oracle.fp8_tensor_qdq(x, chunk=1000), whole)
    assert np.array_equal(oracle.fp8_tensor_qdq(x, scale=np.float32(0.5), chunk=777),
                          oracle.fp8_tensor_qdq(x, scale=np.float32(0.5)))
