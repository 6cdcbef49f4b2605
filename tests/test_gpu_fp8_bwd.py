"""GPU parity of the per-tensor FP8 grouped MLP backward against the oracle's
(grouped_mlp_backward_fp8_tensor: one factor per tensor for dY, dZ, h and x over all
rows and for each expert's W1 and W2). Tolerance 6e-2, the FP8 forward's bound, on dx,
dW1, dW2 and dprob; experts without rows get exactly zero weight gradients.

The saved forward tensors z and h are the oracle's exact forward rounded to bf16: both
sides take the same bits. dY, h and x are bf16 on both sides, so their factors and
codes agree bit for bit; dH and dZ come from float32 GEMMs here and float64 ones in the
oracle, so an element on a bf16 or E4M3 rounding boundary can take the neighbouring
code. The transposed per-tensor codes are compared bit for bit with the row-major
quantiser's (the codes of one tensor under one factor)."""
import numpy as np
import pytest
import torch

import oracle
from conftest import max_rel_err, record_parity
from moe_inputs import WORKLOADS, bf16_bits_to_f32, f32_to_bf16_bits, make_grad, make_inputs, scaled

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

SHAPES = [
    # name, T, H, I, E, k, zipf, empty experts
    ("ragged", 700, 512, 256, 4, 2, 0.0, ()),
    ("skewed_empty", 900, 256, 512, 8, 2, 1.2, (5,)),
    # several 256-row K steps per expert, more weight-gradient tiles than CUs
    ("many_tiles", 1500, 1024, 1024, 16, 2, 1.2, (4, 11)),
]


def _bits(a):
    return f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def _check_both_readings(got, dy, x, z, h, w1, w2, offsets, pp, group):
    """Against the oracle with dH and dZ rounded to bf16 after their GEMMs and without
    those roundings: both must hold the FP8 bound."""
    for rounded in (True, False):
        ref = oracle.grouped_mlp_backward_fp8_tensor(dy, x, z, h, w1, w2, offsets, pp, round_bf16=rounded)
        errs = dict(dx=max_rel_err(got["dx"], ref["dx_perm"]), dw1=max_rel_err(got["dw1"], ref["dw_gate_up"]),
                    dw2=max_rel_err(got["dw2"], ref["dw_down"]), dprob=max_rel_err(got["dprob"], ref["dprob_perm"]))
        print(f"  max rel err ({'with' if rounded else 'without'} the dH, dZ bf16 roundings) "
              + " ".join(f"{k2} {v:.2e}" for k2, v in errs.items()), flush=True)
        record_parity(group + (", dH/dZ rounded to bf16" if rounded else ", no dH/dZ rounding"), **errs)
        for k2, v in errs.items():
            assert v <= FP8_TOL, (k2, rounded)


@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_fp8_backward(moe, shape):
    name, T, H, I, E, k, zipf, empty = shape
    w = scaled(WORKLOADS["mixtral_fwd_bwd"], T=T, H=H, I=I, E=E, k=k, zipf=zipf, seed=51)
    inp = make_inputs(w)
    if empty:
        inp.logits[:, list(empty)] -= 100.0
    idx, p, m, pp = oracle_perm(inp, k, E)
    for e in empty:
        assert m["split_sizes"][e] == 0
    R = T * k
    xp_bits = inp.bits["x"][m["src_token"]]
    xp = bf16_bits_to_f32(xp_bits)
    _, z, h = oracle.grouped_mlp_forward(xp, inp.w1, inp.w2, m["offsets"], pp)
    z_bits, h_bits = _bits(z), _bits(h)
    dyf, dyb = make_grad((R, H), 87)
    off = torch.from_numpy(m["offsets"].astype(np.int32)).cuda()
    dw1 = torch.full((E, 2 * I, H), float("nan"), dtype=torch.bfloat16, device="cuda")
    dw2 = torch.full((E, H, I), float("nan"), dtype=torch.bfloat16, device="cuda")
    print(f"fp8 bwd {name}: R={R} H={H} I={I} E={E}", flush=True)
    dx, dw1, dw2, dprob = moe.moe_grouped_mlp_bwd(
        dev_bf16(dyb), dev_bf16(xp_bits), dev_bf16(z_bits), dev_bf16(h_bits), dev_f32(pp.astype(np.float32)),
        dev_bf16(inp.bits["w1"]), dev_bf16(inp.bits["w2"]), off, compute="fp8", dw_gate_up=dw1, dw_down=dw2)
    torch.cuda.synchronize()
    got = dict(dx=host(dx), dw1=host(dw1), dw2=host(dw2), dprob=dprob.cpu().numpy())
    zf, hf = bf16_bits_to_f32(z_bits), bf16_bits_to_f32(h_bits)
    _check_both_readings(got, dyf, xp, zf, hf, inp.w1, inp.w2, m["offsets"], pp, "FP8 backward small shapes")
    for e in empty:
        assert not got["dw1"][e].any() and not got["dw2"][e].any(), "idle expert must get zero weight gradients"
    # the quantisation is visible: the result is not the unquantised backward's
    ref = oracle.grouped_mlp_backward_fp8_tensor(dyf, xp, zf, hf, inp.w1, inp.w2, m["offsets"], pp)
    exact = oracle.grouped_mlp_backward_fp8_tensor(dyf, xp, zf, hf, inp.w1, inp.w2, m["offsets"], pp, quantize=False)
    assert max_rel_err(ref["dw_down"], exact["dw_down"]) > 1e-3


def test_fp8_training_step(moe):
    """The per-tensor FP8 forward saving z and h, then the FP8 backward on them, against
    the oracle's FP8 forward (its z, and its bf16 h) and FP8 backward: a whole layer
    step's GEMMs in FP8. Saving does not change y."""
    T, H, I, E, k = 900, 512, 256, 8, 2
    w = scaled(WORKLOADS["mixtral_fwd_bwd"], T=T, H=H, I=I, E=E, k=k, zipf=1.2, seed=53)
    inp = make_inputs(w)
    inp.logits[:, [6]] -= 100.0
    idx, p, m, pp = oracle_perm(inp, k, E)
    assert m["split_sizes"][6] == 0
    R = T * k
    xp_bits = inp.bits["x"][m["src_token"]]
    xp = bf16_bits_to_f32(xp_bits)
    off = torch.from_numpy(m["offsets"].astype(np.int32)).cuda()
    prob = dev_f32(pp.astype(np.float32))
    w1, w2 = dev_bf16(inp.bits["w1"]), dev_bf16(inp.bits["w2"])
    print(f"fp8 training step: R={R} H={H} I={I} E={E}", flush=True)
    y, z, h = moe.moe_grouped_mlp_fwd(dev_bf16(xp_bits), w1, w2, off, prob, compute="fp8", save_for_bwd=True)
    y0 = moe.moe_grouped_mlp_fwd(dev_bf16(xp_bits), w1, w2, off, prob, compute="fp8")
    dyf, dyb = make_grad((R, H), 88)
    dx, dw1, dw2, dprob = moe.moe_grouped_mlp_bwd(dev_bf16(dyb), dev_bf16(xp_bits), z, h, prob, w1, w2, off,
                                                  compute="fp8")
    torch.cuda.synchronize()
    assert torch.equal(y, y0), "saving z and h must not change y"
    y_ref, z_ref, h_ref = oracle.grouped_mlp_forward_fp8_tensor(xp, inp.w1, inp.w2, m["offsets"], pp, return_zh=True)
    ey, ez, eh = max_rel_err(host(y), y_ref), max_rel_err(host(z), z_ref), max_rel_err(host(h), h_ref)
    print(f"  y {ey:.2e}, saved z {ez:.2e}, saved h {eh:.2e}", flush=True)
    assert ey <= FP8_TOL and ez <= 1e-2 and eh <= 1e-2
    zb, hb = bf16_bits_to_f32(_bits(z_ref)), bf16_bits_to_f32(_bits(h_ref))
    got = dict(dx=host(dx), dw1=host(dw1), dw2=host(dw2), dprob=dprob.cpu().numpy())
    _check_both_readings(got, dyf, xp, zb, hb, inp.w1, inp.w2, m["offsets"], pp, "FP8 training step")
    assert not got["dw1"][6].any() and not got["dw2"][6].any()


def test_fp8_backward_degenerate(moe):
    """No routed rows at all (every weight gradient exactly zero, weights prefilled with
    NaN to show they are written), and every row on one expert of four."""
    E, H, I = 4, 256, 256
    rng = np.random.default_rng(6)
    w1b = _bits(0.02 * rng.standard_normal((E, 2 * I, H)))
    w2b = _bits(0.02 * rng.standard_normal((E, H, I)))
    w1, w2 = dev_bf16(w1b), dev_bf16(w2b)
    dev = torch.device("cuda")
    empty = lambda *shape: torch.empty(shape, dtype=torch.bfloat16, device=dev)
    dw1 = torch.full((E, 2 * I, H), float("nan"), dtype=torch.bfloat16, device=dev)
    dw2 = torch.full((E, H, I), float("nan"), dtype=torch.bfloat16, device=dev)
    off = torch.zeros(E + 1, dtype=torch.int32, device=dev)
    print("fp8 bwd: R = 0", flush=True)
    dx, dw1, dw2, dprob = moe.moe_grouped_mlp_bwd(empty(0, H), empty(0, H), empty(0, 2 * I), empty(0, I),
                                                  torch.empty(0, dtype=torch.float32, device=dev), w1, w2, off,
                                                  compute="fp8", dw_gate_up=dw1, dw_down=dw2)
    torch.cuda.synchronize()
    assert dx.shape == (0, H) and dprob.numel() == 0
    assert not host(dw1).any() and not host(dw2).any()
    R = 300
    xb = _bits(rng.standard_normal((R, H)))
    dyb = _bits(rng.standard_normal((R, H)))
    zb = _bits(rng.standard_normal((R, 2 * I)))
    hb = _bits(0.3 * rng.standard_normal((R, I)))
    pp = rng.uniform(0.2, 1.0, R).astype(np.float32)
    offs = np.array([0, 0, 0, R, R], np.int32)
    print("fp8 bwd: one busy expert", flush=True)
    dx, dw1, dw2, dprob = moe.moe_grouped_mlp_bwd(dev_bf16(dyb), dev_bf16(xb), dev_bf16(zb), dev_bf16(hb), dev_f32(pp),
                                                  w1, w2, torch.from_numpy(offs).cuda(), compute="fp8")
    torch.cuda.synchronize()
    ref = oracle.grouped_mlp_backward_fp8_tensor(bf16_bits_to_f32(dyb), bf16_bits_to_f32(xb), bf16_bits_to_f32(zb),
                                                 bf16_bits_to_f32(hb), bf16_bits_to_f32(w1b), bf16_bits_to_f32(w2b),
                                                 offs, pp)
    for k2, got in (("dx_perm", host(dx)), ("dw_gate_up", host(dw1)), ("dw_down", host(dw2)),
                    ("dprob_perm", dprob.cpu().numpy())):
        err = max_rel_err(got, ref[k2])
        print(f"  {k2} {err:.2e}", flush=True)
        assert err <= FP8_TOL, k2
    for e in (0, 1, 3):
        assert not host(dw1)[e].any() and not host(dw2)[e].any()


@pytest.mark.parametrize("sizes,C,mag", [((37, 0, 70, 128), 128, 1.0), ((300, 5), 192, 3e-3), ((1,), 64, 40.0)])
def test_fp8_colwise_codes_bit_exact(moe, sizes, C, mag):
    """fp8_tensor_quantize_colwise: the factor and codes of the oracle's per-tensor
    quantiser, bit for bit, transposed with each expert's rows zero-padded (an idle
    expert takes no columns)."""
    rng = np.random.default_rng(7)
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    R = int(off[-1])
    xb = _bits(mag * rng.standard_normal((R, C)))
    codes, scale, kofs = moe.fp8_tensor_quantize_colwise(dev_bf16(xb), torch.from_numpy(off).cuda(), pad=256)
    torch.cuda.synchronize()
    ref_codes, ref_scale = oracle.fp8_tensor_quantize(bf16_bits_to_f32(xb))
    assert scale.cpu().numpy()[0] == ref_scale
    kofs = kofs.cpu().numpy()
    want_kofs = np.concatenate([[0], np.cumsum([(m + 255) // 256 * 256 for m in sizes])])
    assert np.array_equal(kofs, want_kofs)
    got = codes.cpu().numpy()
    for e, m in enumerate(sizes):
        a = int(off[e])
        block = got[:, kofs[e]:kofs[e + 1]]
        assert np.array_equal(block[:, :m], ref_codes[a:a + m].T), e
        assert not block[:, m:].any(), e


@pytest.mark.parametrize("rows,cols", [(512, 384), (32, 64), (1024, 1536)])
def test_fp8_pack_weight_bwd_bits(moe, rows, cols):
    """fp8_tensor_pack_weight_bwd: the oracle's per-tensor codes of w, transposed, then
    its float32 factor, bit for bit."""
    rng = np.random.default_rng(rows + cols)
    w = 0.05 * rng.standard_normal((rows, cols))
    w[:3, :5] = 0.0
    wb = _bits(w)
    packed = moe.fp8_tensor_pack_weight_bwd(dev_bf16(wb))
    torch.cuda.synchronize()
    got = packed.cpu().numpy()
    codes, factor = oracle.fp8_tensor_quantize(bf16_bits_to_f32(wb))
    assert np.array_equal(got[:rows * cols].reshape(cols, rows), codes.T)
    assert got[rows * cols:rows * cols + 4].view(np.float32)[0] == factor


def test_fp8_backward_with_packed_weights(moe):
    """The FP8 backward on weights packed once by fp8_tensor_pack_weight_bwd gives the
    same bits as on the bf16 master weights quantised inside the call."""
    T, H, I, E, k = 700, 512, 256, 4, 2
    w = scaled(WORKLOADS["mixtral_fwd_bwd"], T=T, H=H, I=I, E=E, k=k, seed=57)
    inp = make_inputs(w)
    idx, p, m, pp = oracle_perm(inp, k, E)
    R = T * k
    xp_bits = inp.bits["x"][m["src_token"]]
    rng = np.random.default_rng(8)
    zb = _bits(rng.standard_normal((R, 2 * I)))
    hb = _bits(0.3 * rng.standard_normal((R, I)))
    dyf, dyb = make_grad((R, H), 89)
    off = torch.from_numpy(m["offsets"].astype(np.int32)).cuda()
    w1, w2 = dev_bf16(inp.bits["w1"]), dev_bf16(inp.bits["w2"])
    args = (dev_bf16(dyb), dev_bf16(xp_bits), dev_bf16(zb), dev_bf16(hb), dev_f32(pp.astype(np.float32)))
    print("fp8 bwd: packed weights", flush=True)
    a = moe.moe_grouped_mlp_bwd(*args, w1, w2, off, compute="fp8")
    p1 = [moe.fp8_tensor_pack_weight_bwd(w1[e]) for e in range(E)]
    p2 = [moe.fp8_tensor_pack_weight_bwd(w2[e]) for e in range(E)]
    b = moe.moe_grouped_mlp_bwd(*args, p1, p2, off, compute="fp8")
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
