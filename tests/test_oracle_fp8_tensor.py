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
