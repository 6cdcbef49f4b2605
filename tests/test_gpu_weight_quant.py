"""GPU parity of the weight quantisers that write the forward's and the backward's
operand layouts from one read of each bf16 weight (mxfp8_quantize_weights,
fp8_tensor_quantize_weights): bit for bit against the oracle's quantisers, and byte for
byte against the library's single-layout calls; then a training step on those weights
against the same step on the bf16 master weights quantised inside the calls.

Source: "Efficient MoE Training for Biological Foundation Models", Challenge 2 (MXFP8:
32-value blocks; FP8: one factor per tensor) and Challenge 3 (quantisation as separate
ops is the overhead the fused recipe removes)."""
import numpy as np
import pytest
import torch

import oracle
from moe_inputs import WORKLOADS, bf16_bits_to_f32, f32_to_bf16_bits, make_inputs, scaled

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import grouped_expert_gemm_amd as g
    g.lib()
    return g


from gpu_util import dev_bf16, dev_f32, oracle_perm  # noqa: E402


def _bits(a):
    return f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def _weights(n, rows, cols, seed):
    """n weights with magnitudes that change by powers of two every 32 rows and every
    32 columns (so the row blocks and the column blocks take different scales), some
    all-zero blocks, negative zeros and values at the top of bf16's range."""
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((n, rows, cols))
    w *= np.exp2(rng.integers(-8, 8, (n, rows // 32, 1, 1))).repeat(32, 1).reshape(n, rows, 1)
    w *= np.exp2(rng.integers(-4, 4, (n, 1, cols // 32, 1))).repeat(32, 2).reshape(n, 1, cols)
    w[:, :32, :32] = 0.0
    w[0, rows - 1, cols - 32:] = -0.0
    w[-1, rows // 2, 5] = 3.0e38
    return _bits(w)


# (n, rows, cols): one weight; several; more than one tensor table (16 per launch); an
# odd number of 64-column blocks (a workgroup's item pairs straddle row groups)
MX_CASES = [(1, 128, 64), (3, 512, 384), (17, 256, 128), (2, 384, 192)]


@pytest.mark.parametrize("n,rows,cols", MX_CASES)
def test_mxfp8_quantize_weights_bits(moe, n, rows, cols):
    wb = _weights(n, rows, cols, n * 1000 + rows + cols)
    w = dev_bf16(wb)
    print(f"mxfp8_quantize_weights n={n} rows={rows} cols={cols}", flush=True)
    codes, scales, packed = moe.mxfp8_quantize_weights(w)
    torch.cuda.synchronize()
    c, s, p = codes.cpu().numpy(), scales.cpu().numpy(), packed.cpu().numpy()
    for i in range(n):
        wf = bf16_bits_to_f32(wb[i])
        oc, os_ = oracle.mxfp8_quantize(wf)
        assert np.array_equal(c[i], oc), i
        assert np.array_equal(s[i], os_), i
        tc, ts, _ = oracle.mxfp8_quantize_colwise(wf, np.array([0, rows]), 32, rows)
        assert np.array_equal(p[i, :rows * cols].reshape(cols, rows), tc), i
        sm = ts.reshape(cols, rows // 128, 4).transpose(1, 0, 2).reshape(-1)   # step-major words
        assert np.array_equal(p[i, rows * cols:], sm), i
    # byte for byte the single-layout calls
    for i in (0, n - 1):
        rc, rs = moe.mxfp8_quantize(w[i])
        assert torch.equal(rc, codes[i]) and torch.equal(rs, scales[i])
        assert torch.equal(moe.mxfp8_pack_weight_bwd(w[i]), packed[i])


# (n, rows, cols): one weight; several; more than one tensor table (64 per launch); an
# odd number of 64-column blocks
FP8_CASES = [(1, 32, 64), (3, 512, 384), (65, 64, 128), (2, 96, 192)]


@pytest.mark.parametrize("n,rows,cols", FP8_CASES)
def test_fp8_tensor_quantize_weights_bits(moe, n, rows, cols):
    wb = _weights(n, rows, cols, n * 7 + rows + cols)
    if n > 1:
        wb[1] = _bits(np.zeros((rows, cols)))     # an all-zero weight: factor 1, codes 0
    w = dev_bf16(wb)
    print(f"fp8_tensor_quantize_weights n={n} rows={rows} cols={cols}", flush=True)
    codes, scale, packed = moe.fp8_tensor_quantize_weights(w)
    torch.cuda.synchronize()
    c, f, p = codes.cpu().numpy(), scale.cpu().numpy(), packed.cpu().numpy()
    for i in range(n):
        oc, of = oracle.fp8_tensor_quantize(bf16_bits_to_f32(wb[i]))
        assert f[i] == of, i
        assert np.array_equal(c[i], oc), i
        assert np.array_equal(p[i, :rows * cols].reshape(cols, rows), oc.T), i
        assert p[i, rows * cols:rows * cols + 4].view(np.float32)[0] == of, i
    for i in (0, n - 1):
        rc, rf = moe.fp8_tensor_quantize(w[i])
        assert torch.equal(rc, codes[i]) and torch.equal(rf[0], scale[i])
        assert torch.equal(moe.fp8_tensor_pack_weight_bwd(w[i])[:rows * cols + 4], packed[i, :rows * cols + 4])


@pytest.mark.parametrize("compute", ["mxfp8", "fp8"])
def test_training_step_on_quantised_weights(moe, compute):
    """Forward and backward on the weights quantised by the two-layout call give the same
    bits as on the bf16 master weights quantised inside each call."""
    T, H, I, E, k = 600, 512, 256, 5, 2
    w = scaled(WORKLOADS["mixtral_fwd_bwd"], T=T, H=H, I=I, E=E, k=k, zipf=1.2, seed=45)
    inp = make_inputs(w)
    idx, p, m, pp = oracle_perm(inp, k, E)
    R = T * k
    xp = dev_bf16(inp.bits["x"][m["src_token"]])
    off = torch.from_numpy(m["offsets"].astype(np.int32)).cuda()
    prob = dev_f32(pp.astype(np.float32))
    w1, w2 = dev_bf16(inp.bits["w1"]), dev_bf16(inp.bits["w2"])
    dy = dev_bf16(_bits(np.random.default_rng(3).standard_normal((R, H))))
    print(f"{compute} step on two-layout weights: R={R} H={H} I={I} E={E}", flush=True)
    y0, z0, h0 = moe.moe_grouped_mlp_fwd(xp, w1, w2, off, prob, compute=compute, save_for_bwd=True)
    g0 = moe.moe_grouped_mlp_bwd(dy, xp, z0, h0, prob, w1, w2, off, compute=compute)
    if compute == "mxfp8":
        q1, s1, p1 = moe.mxfp8_quantize_weights(w1)
        q2, s2, p2 = moe.mxfp8_quantize_weights(w2)
    else:
        q1, s1, p1 = moe.fp8_tensor_quantize_weights(w1)
        q2, s2, p2 = moe.fp8_tensor_quantize_weights(w2)
        s1, s2 = [s1[e:e + 1] for e in range(E)], [s2[e:e + 1] for e in range(E)]
    y1, z1, h1 = moe.moe_grouped_mlp_fwd(xp, q1, q2, off, prob, compute=compute, save_for_bwd=True,
                                         w_gate_up_scale=s1, w_down_scale=s2)
    g1 = moe.moe_grouped_mlp_bwd(dy, xp, z1, h1, prob, [p1[e] for e in range(E)], [p2[e] for e in range(E)], off,
                                 compute=compute)
    torch.cuda.synchronize()
    for name, a, b in zip(("y", "z", "h"), (y1, z1, h1), (y0, z0, h0)):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), name
    for name, a, b in zip(("dx", "dw_gate_up", "dw_down", "dprob"), g1, g0):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), name
