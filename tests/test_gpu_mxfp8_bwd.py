"""GPU parity of the MXFP8 grouped MLP backward against the oracle's MXFP8 backward
(every GEMM operand quantised along that GEMM's reduction axis; the weight gradients
along each expert's rows). Tolerance 6e-2, the MXFP8 forward's bound, on dx, dW1, dW2
and dprob; experts without rows get exactly zero weight gradients.

The saved forward tensors z and h are the oracle's exact forward rounded to bf16: both
sides take the same bits. Both round dH and dZ to bf16 before quantising them; the
library computes them in float32, the oracle in float64, so an element whose value
sits on a bf16 or E4M3 rounding boundary can take the neighbouring code."""
import numpy as np
import pytest
import torch

import oracle
from conftest import max_rel_err, record_parity
from moe_inputs import WORKLOADS, bf16_bits_to_f32, f32_to_bf16_bits, make_grad, make_inputs, scaled

pytestmark = pytest.mark.gpu

MX_TOL = 6e-2


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


def _check_both_readings(got, dy, x, z, h, w1, w2, offsets, pp):
    """The GPU gradients against the oracle's MXFP8 backward twice: with dH and dZ rounded
    to bf16 after their GEMMs (the recipe returns a low-precision GEMM's result to bf16)
    and without those two roundings (every quantiser kept). Both must hold the MXFP8
    bound, so parity does not rest on the oracle mirroring the kernel's bf16 storage."""
    for rounded in (True, False):
        ref = oracle.grouped_mlp_backward_mxfp8(dy, x, z, h, w1, w2, offsets, pp, round_bf16=rounded)
        errs = dict(dx=max_rel_err(got["dx"], ref["dx_perm"]), dw1=max_rel_err(got["dw1"], ref["dw_gate_up"]),
                    dw2=max_rel_err(got["dw2"], ref["dw_down"]), dprob=max_rel_err(got["dprob"], ref["dprob_perm"]))
        print(f"  max rel err ({'with' if rounded else 'without'} the dH, dZ bf16 roundings) "
              + " ".join(f"{k2} {v:.2e}" for k2, v in errs.items()), flush=True)
        record_parity("MXFP8 backward small shapes, " + ("dH/dZ rounded to bf16" if rounded else "no dH/dZ rounding"),
                      **errs)
        for k2, v in errs.items():
            assert v <= MX_TOL, (k2, rounded)


@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_mxfp8_backward(moe, shape):
    name, T, H, I, E, k, zipf, empty = shape
    w = scaled(WORKLOADS["mixtral_fwd_bwd"], T=T, H=H, I=I, E=E, k=k, zipf=zipf, seed=41)
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
    dyf, dyb = make_grad((R, H), 77)
    off = torch.from_numpy(m["offsets"].astype(np.int32)).cuda()
    print(f"mxfp8 bwd {name}: R={R} H={H} I={I} E={E}", flush=True)
    dx, dw1, dw2, dprob = moe.moe_grouped_mlp_bwd(
        dev_bf16(dyb), dev_bf16(xp_bits), dev_bf16(z_bits), dev_bf16(h_bits), dev_f32(pp.astype(np.float32)),
        dev_bf16(inp.bits["w1"]), dev_bf16(inp.bits["w2"]), off, compute="mxfp8")
    torch.cuda.synchronize()
    got = dict(dx=host(dx), dw1=host(dw1), dw2=host(dw2), dprob=dprob.cpu().numpy())
    _check_both_readings(got, dyf, xp, bf16_bits_to_f32(z_bits), bf16_bits_to_f32(h_bits), inp.w1, inp.w2,
                         m["offsets"], pp)
    ref = oracle.grouped_mlp_backward_mxfp8(dyf, xp, bf16_bits_to_f32(z_bits), bf16_bits_to_f32(h_bits), inp.w1,
                                            inp.w2, m["offsets"], pp)
    for e in empty:
        assert not host(dw1)[e].any() and not host(dw2)[e].any(), "idle expert must get zero weight gradients"
    # the quantisation is visible: the result is not the exact bf16-free backward
    exact = oracle.grouped_mlp_backward_mxfp8(dyf, xp, bf16_bits_to_f32(z_bits), bf16_bits_to_f32(h_bits), inp.w1,
                                              inp.w2, m["offsets"], pp, quantize=False)
    assert max_rel_err(ref["dw_down"], exact["dw_down"]) > 1e-3


def test_mxfp8_training_step(moe):
    """An MXFP8 forward that saves z and h, then the MXFP8 backward on them, against the
    oracle's MXFP8 forward (its z and h rounded to bf16) and MXFP8 backward. Saving does
    not change y; the saved tensors match the oracle's to bf16-level error (the GEMM of
    identical MX operands, float32 against float64 accumulation)."""
    T, H, I, E, k = 900, 512, 256, 8, 2
    w = scaled(WORKLOADS["mixtral_fwd_bwd"], T=T, H=H, I=I, E=E, k=k, zipf=1.2, seed=43)
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
    print(f"mxfp8 training step: R={R} H={H} I={I} E={E}", flush=True)
    y, z, h = moe.moe_grouped_mlp_fwd(dev_bf16(xp_bits), w1, w2, off, prob, compute="mxfp8", save_for_bwd=True)
    y0 = moe.moe_grouped_mlp_fwd(dev_bf16(xp_bits), w1, w2, off, prob, compute="mxfp8")
    dyf, dyb = make_grad((R, H), 78)
    dx, dw1, dw2, dprob = moe.moe_grouped_mlp_bwd(dev_bf16(dyb), dev_bf16(xp_bits), z, h, prob, w1, w2, off,
                                                  compute="mxfp8")
    torch.cuda.synchronize()
    assert torch.equal(y, y0), "saving z and h must not change y"
    y_ref, h_ref, z_ref = oracle.grouped_mlp_forward_mxfp8(xp, inp.w1, inp.w2, m["offsets"], pp, return_z=True)
    ez, eh = max_rel_err(host(z), z_ref), max_rel_err(host(h), h_ref)
    print(f"  saved z {ez:.2e}, saved h {eh:.2e}", flush=True)
    assert ez <= 1e-2 and eh <= 1e-2
    zb, hb = bf16_bits_to_f32(_bits(z_ref)), bf16_bits_to_f32(_bits(h_ref))
    got = dict(dx=host(dx), dw1=host(dw1), dw2=host(dw2), dprob=dprob.cpu().numpy())
    _check_both_readings(got, dyf, xp, zb, hb, inp.w1, inp.w2, m["offsets"], pp)
    assert not host(dw1)[6].any() and not host(dw2)[6].any()


def test_mxfp8_backward_degenerate(moe):
    """No routed rows at all (every weight gradient exactly zero, weights prefilled with
    NaN to show they are written), and every row on one expert of four."""
    E, H, I = 4, 256, 256
    rng = np.random.default_rng(5)
    w1b = _bits(0.02 * rng.standard_normal((E, 2 * I, H)))
    w2b = _bits(0.02 * rng.standard_normal((E, H, I)))
    w1, w2 = dev_bf16(w1b), dev_bf16(w2b)
    dev = torch.device("cuda")
    empty = lambda *shape: torch.empty(shape, dtype=torch.bfloat16, device=dev)
    dw1 = torch.full((E, 2 * I, H), float("nan"), dtype=torch.bfloat16, device=dev)
    dw2 = torch.full((E, H, I), float("nan"), dtype=torch.bfloat16, device=dev)
    off = torch.zeros(E + 1, dtype=torch.int32, device=dev)
    print("mxfp8 bwd: R = 0", flush=True)
    dx, dw1, dw2, dprob = moe.moe_grouped_mlp_bwd(empty(0, H), empty(0, H), empty(0, 2 * I), empty(0, I),
                                                  torch.empty(0, dtype=torch.float32, device=dev), w1, w2, off,
                                                  compute="mxfp8", dw_gate_up=dw1, dw_down=dw2)
    torch.cuda.synchronize()
    assert dx.shape == (0, H) and dprob.numel() == 0
    assert not host(dw1).any() and not host(dw2).any()
    # all rows on expert 2
    R = 300
    xb = _bits(rng.standard_normal((R, H)))
    dyb = _bits(rng.standard_normal((R, H)))
    zb = _bits(rng.standard_normal((R, 2 * I)))
    hb = _bits(0.3 * rng.standard_normal((R, I)))
    pp = rng.uniform(0.2, 1.0, R).astype(np.float32)
    offs = np.array([0, 0, 0, R, R], np.int32)
    print("mxfp8 bwd: one busy expert", flush=True)
    dx, dw1, dw2, dprob = moe.moe_grouped_mlp_bwd(dev_bf16(dyb), dev_bf16(xb), dev_bf16(zb), dev_bf16(hb), dev_f32(pp),
                                                  w1, w2, torch.from_numpy(offs).cuda(), compute="mxfp8")
    torch.cuda.synchronize()
    ref = oracle.grouped_mlp_backward_mxfp8(bf16_bits_to_f32(dyb), bf16_bits_to_f32(xb), bf16_bits_to_f32(zb),
                                            bf16_bits_to_f32(hb), bf16_bits_to_f32(w1b), bf16_bits_to_f32(w2b), offs,
                                            pp)
    for k2, got in (("dx_perm", host(dx)), ("dw_gate_up", host(dw1)), ("dw_down", host(dw2)),
                    ("dprob_perm", dprob.cpu().numpy())):
        err = max_rel_err(got, ref[k2])
        print(f"  {k2} {err:.2e}", flush=True)
        assert err <= MX_TOL, k2
    for e in (0, 1, 3):
        assert not host(dw1)[e].any() and not host(dw2)[e].any()


@pytest.mark.parametrize("rows,cols", [(512, 384), (128, 64), (1024, 1536)])
def test_mxfp8_pack_weight_bwd_bits(moe, rows, cols):
    """mxfp8_pack_weight_bwd: the codes of w^T quantised along w's rows (32-value blocks)
    and the step-major scales, bit for bit against the oracle's column-wise quantiser
    (one expert of `rows` rows, 32-row padding, which is none here)."""
    rng = np.random.default_rng(rows + cols)
    w = (rng.standard_normal((rows, cols)) * np.exp2(rng.integers(-6, 6, (rows // 32, 1)).repeat(32, 0))).astype(np.float32)
    w[:32, :5] = 0.0                              # all-zero blocks
    wb = _bits(w)
    print(f"pack weight rows={rows} cols={cols}", flush=True)
    packed = moe.mxfp8_pack_weight_bwd(dev_bf16(wb)).cpu().numpy()
    codes, scales, _ = oracle.mxfp8_quantize_colwise(bf16_bits_to_f32(wb), np.array([0, rows]), 32, rows)
    assert np.array_equal(packed[:rows * cols].reshape(cols, rows), codes)
    # step-major: the 4 scales of rows [128 k, 128 k + 128) of column c form word k * cols + c
    sm = scales.reshape(cols, rows // 128, 4).transpose(1, 0, 2).reshape(-1)
    assert np.array_equal(packed[rows * cols:], sm)


def test_mxfp8_backward_with_packed_weights(moe):
    """The MXFP8 backward on weights packed once (mxfp8_pack_weight_bwd) gives the same
    bits as on the bf16 master weights quantised inside the call."""
    T, H, I, E, k = 700, 512, 256, 6, 2
    w = scaled(WORKLOADS["mixtral_fwd_bwd"], T=T, H=H, I=I, E=E, k=k, zipf=1.2, seed=44)
    inp = make_inputs(w)
    inp.logits[:, [2]] -= 100.0
    idx, p, m, pp = oracle_perm(inp, k, E)
    assert m["split_sizes"][2] == 0
    R = T * k
    xp = dev_bf16(inp.bits["x"][m["src_token"]])
    gen = np.random.default_rng(9)
    z = dev_bf16(_bits(gen.standard_normal((R, 2 * I))))
    h = dev_bf16(_bits(0.3 * gen.standard_normal((R, I))))
    dy = dev_bf16(_bits(gen.standard_normal((R, H))))
    off = torch.from_numpy(m["offsets"].astype(np.int32)).cuda()
    prob = dev_f32(pp.astype(np.float32))
    w1, w2 = dev_bf16(inp.bits["w1"]), dev_bf16(inp.bits["w2"])
    print(f"mxfp8 bwd with packed weights: R={R} H={H} I={I} E={E}", flush=True)
    ref = moe.moe_grouped_mlp_bwd(dy, xp, z, h, prob, w1, w2, off, compute="mxfp8")
    p1 = [moe.mxfp8_pack_weight_bwd(w1[e]) for e in range(E)]
    p2 = [moe.mxfp8_pack_weight_bwd(w2[e]) for e in range(E)]
    got = moe.moe_grouped_mlp_bwd(dy, xp, z, h, prob, p1, p2, off, compute="mxfp8")
    torch.cuda.synchronize()
    for name, a, b in zip(("dx", "dw_gate_up", "dw_down", "dprob"), got, ref):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), name
