"""GPU parity of per-tensor FP8 (E4M3, one float32 scale per tensor, current scaling):

  * fp8_tensor_quantize: codes and scale bit-exact with the oracle's quantiser;
  * the grouped MLP forward with compute="fp8" against the oracle's FP8-emulated
    forward (x_perm, each expert's W1 and W2, and h quantised per tensor): max rel
    error <= 6e-2, the bound used for the block-scaled MXFP8 forward;
  * pre-quantised operands (codes + scales from fp8_tensor_quantize) give the same bits
    as the fused path, which quantises them inside the call;
  * at the Mixtral layer shape, the layer in the benchmark's launch configuration.
"""
import numpy as np
import pytest
import torch

import oracle
from conftest import max_rel_err
from moe_inputs import WORKLOADS, bf16_bits_to_f32, f32_to_bf16_bits, make_inputs, scaled

pytestmark = pytest.mark.gpu

FP8_TOL = 6e-2


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import grouped_expert_gemm_amd as g
    g.lib()
    return g


from gpu_util import dev_bf16, dev_f32, host, oracle_perm  # noqa: E402


@pytest.mark.parametrize("shape,mag", [((1000, 136), 1.0), ((3, 8), 1e-30), ((4096, 520), 3e4), ((64, 40), 2e-38),
                                       ((8192, 512), 2.0 ** 100)])
def test_quantize_bit_exact(moe, shape, mag):
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(shape) * mag).astype(np.float32)
    bits = (x.view(np.uint32) + 0x7FFF + ((x.view(np.uint32) >> 16) & 1)) >> 16
    bits = bits.astype(np.uint16)
    print(f"fp8_tensor_quantize {shape} x{mag:g}", flush=True)
    codes, scale = moe.fp8_tensor_quantize(dev_bf16(bits))
    torch.cuda.synchronize()
    rc, rs = oracle.fp8_tensor_quantize(bf16_bits_to_f32(bits))
    assert scale.cpu().numpy()[0] == rs
    assert np.array_equal(codes.cpu().numpy(), rc)


def test_quantize_zero_and_empty(moe):
    codes, scale = moe.fp8_tensor_quantize(torch.zeros((16, 64), dtype=torch.bfloat16, device="cuda"))
    torch.cuda.synchronize()
    assert scale.item() == 1.0 and not codes.any()
    codes, scale = moe.fp8_tensor_quantize(torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda"))
    torch.cuda.synchronize()
    assert scale.item() == 1.0 and codes.numel() == 0


def test_quantize_keeps_sign_of_zero(moe):
    """-0 inputs get code 0x80 (the E4M3 code of the quotient -0 / s, sign kept) in every
    per-tensor FP8 quantiser: by rows, along the token axis and in the weight packs; also
    in a tensor that is all -0 (factor 1)."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((64, 128)).astype(np.float32)
    x[::3, ::5] = -0.0
    x[5] = -0.0
    bits = f32_to_bf16_bits(x)
    rc, rs = oracle.fp8_tensor_quantize(bf16_bits_to_f32(bits))
    assert (rc[5] == 0x80).all()
    xd = dev_bf16(bits)
    codes, scale = moe.fp8_tensor_quantize(xd)
    packed = moe.fp8_tensor_pack_weight_bwd(xd)
    off = torch.tensor([0, 64], dtype=torch.int32, device="cuda")
    tcodes, tscale, _ = moe.fp8_tensor_quantize_colwise(xd, off, 32)
    neg = dev_bf16(f32_to_bf16_bits(np.full((32, 64), -0.0, np.float32)))
    ncodes, nscale = moe.fp8_tensor_quantize(neg)
    torch.cuda.synchronize()
    assert scale.item() == rs and tscale.item() == rs
    assert np.array_equal(codes.cpu().numpy(), rc)
    assert np.array_equal(packed.cpu().numpy()[:64 * 128].reshape(128, 64), rc.T)
    assert np.array_equal(tcodes.cpu().numpy()[:, :64], rc.T)
    assert nscale.item() == 1.0 and (ncodes.cpu().numpy() == 0x80).all()


SHAPES = [
    # name, T, H, I, E, k, zipf, empty experts
    ("ragged", 1500, 512, 512, 4, 2, 0.0, ()),
    ("skewed_empty", 900, 256, 256, 16, 4, 1.2, (2, 7)),
    ("many_experts", 700, 256, 256, 80, 4, 1.2, (3, 70)),   # expert tables in two launches of 64
]


def _setup(name, T, H, I, E, k, zipf, empty):
    w = scaled(WORKLOADS["mixtral_mxfp8_fwd"], T=T, H=H, I=I, E=E, k=k, zipf=zipf, seed=37)
    inp = make_inputs(w)
    if empty:
        inp.logits[:, list(empty)] -= 100.0
    idx, p, m, pp = oracle_perm(inp, k, E)
    for e in empty:
        assert m["split_sizes"][e] == 0
    return w, inp, m, pp


@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_fp8_forward(moe, shape):
    w, inp, m, pp = _setup(*shape)
    xp_bits = inp.bits["x"][m["src_token"]]
    off = torch.from_numpy(m["offsets"].astype(np.int32)).cuda()
    prob = dev_f32(pp.astype(np.float32))
    print(f"fp8 fwd {shape[0]}: R={w.R} H={w.H} I={w.I} E={w.E}", flush=True)
    w1b, w2b = dev_bf16(inp.bits["w1"]), dev_bf16(inp.bits["w2"])
    y = moe.moe_grouped_mlp_fwd(dev_bf16(xp_bits), w1b, w2b, off, prob, compute="fp8")
    torch.cuda.synchronize()
    ref = oracle.grouped_mlp_forward_fp8_tensor(bf16_bits_to_f32(xp_bits), inp.w1, inp.w2, m["offsets"], pp)
    err = max_rel_err(host(y), ref)
    print(f"  max rel err {err:.3e}", flush=True)
    assert err <= FP8_TOL
    # pre-quantised operands: the same codes and scales, so the same bits
    E = w.E
    xq, xs = moe.fp8_tensor_quantize(dev_bf16(xp_bits))
    q1 = [moe.fp8_tensor_quantize(w1b[e]) for e in range(E)]
    q2 = [moe.fp8_tensor_quantize(w2b[e]) for e in range(E)]
    y_pre = moe.moe_grouped_mlp_fwd(xq, [c for c, _ in q1], [c for c, _ in q2], off, prob, compute="fp8",
                                    x_perm_scale=xs, w_gate_up_scale=[s for _, s in q1],
                                    w_down_scale=[s for _, s in q2])
    torch.cuda.synchronize()
    assert torch.equal(y_pre, y)
    # mixed storage: codes for x with bf16 master weights, and bf16 x with weight codes
    y_xq = moe.moe_grouped_mlp_fwd(xq, w1b, w2b, off, prob, compute="fp8", x_perm_scale=xs)
    y_wq = moe.moe_grouped_mlp_fwd(dev_bf16(xp_bits), [c for c, _ in q1], [c for c, _ in q2], off, prob,
                                   compute="fp8", w_gate_up_scale=[s for _, s in q1], w_down_scale=[s for _, s in q2])
    torch.cuda.synchronize()
    assert torch.equal(y_xq, y) and torch.equal(y_wq, y)
    # a second call on the same inputs: same bits (the h maximum is an order-free max)
    y2 = moe.moe_grouped_mlp_fwd(dev_bf16(xp_bits), w1b, w2b, off, prob, compute="fp8")
    torch.cuda.synchronize()
    assert torch.equal(y2, y)


@pytest.mark.slow
def test_fp8_forward_mixtral_shape(moe):
    """The Mixtral layer (T=8192, H=4096, I=14336, E=8, top-2) in FP8. x's scale and the
    sampled expert's weight scales are the oracle's exact ones; h's scale needs all of h,
    whose oracle would quantise every expert's weights (minutes of host work and tens of GB), so the
    oracle's h scale here is the maximum over the sampled expert's h. A smaller scale
    only moves h's quantisation grid: the bound is the same E4M3 round-off."""
    w = WORKLOADS["mixtral_mxfp8_fwd"]
    inp = make_inputs(w, want_float=False)
    print(f"mixtral fp8 fwd: T={w.T} H={w.H} I={w.I}", flush=True)
    idx, p = moe.moe_route_topk(dev_f32(inp.logits), w.k)
    r = moe.moe_permute(dev_bf16(inp.bits["x"]), idx, p, w.E)
    y = moe.moe_grouped_mlp_fwd(r["x_perm"], dev_bf16(inp.bits["w1"]), dev_bf16(inp.bits["w2"]), r["offsets"],
                                r["prob_perm"], compute="fp8")
    torch.cuda.synchronize()
    ridx, rp = oracle.route_topk(inp.logits, w.k)
    m = oracle.permute(ridx, w.E)
    assert np.array_equal(r["offsets"].cpu().numpy(), m["offsets"])
    pp = rp.ravel()[m["src_token"] * w.k + m["src_slot"]]
    x_all = bf16_bits_to_f32(inp.bits["x"])
    s_x = oracle.fp8_tensor_scale(x_all)
    e = int(np.argmax(np.diff(m["offsets"])))
    a, b = int(m["offsets"][e]), int(m["offsets"][e + 1])
    x = bf16_bits_to_f32(inp.bits["x"][m["src_token"][a:b]])
    W1 = bf16_bits_to_f32(inp.bits["w1"][e:e + 1])
    W2 = bf16_bits_to_f32(inp.bits["w2"][e:e + 1])
    ref = oracle.grouped_mlp_forward_fp8_tensor(x, W1, W2, np.array([0, b - a]), pp[a:b], x_scale=s_x)
    err = max_rel_err(host(y)[a:b], ref)
    print(f"  expert {e}: rows {b - a}, max rel err {err:.2e}", flush=True)
    assert err <= FP8_TOL
