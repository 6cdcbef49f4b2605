"""GPU parity with one expert holding more than 16 row tiles of 256 rows. The GEMMs take
an expert's row tiles in groups of at most 16 (row tiles fastest inside a group), so
such an expert is split into several groups: every grouped GEMM (bf16, MXFP8 and
per-tensor FP8 forward; the bf16, MXFP8 and FP8 data gradients) runs that order here,
checked against the oracle. Expert 0 is chosen by every token (its logit raised), so it
holds T rows; the other experts share the second slots.

Tolerances as in the other parity tests: bf16 2e-2 (float32 accumulation of bf16
products), MXFP8 and per-tensor FP8 6e-2 (the quantised forwards' bound)."""
import numpy as np
import pytest
import torch

import oracle
from conftest import max_rel_err
from moe_inputs import WORKLOADS, bf16_bits_to_f32, f32_to_bf16_bits, make_grad, make_inputs, scaled

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
LOWP_TOL = 6e-2


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import grouped_expert_gemm_amd as g
    g.lib()
    return g


from gpu_util import dev_bf16, dev_f32, host, oracle_perm  # noqa: E402

# (T, row tiles of expert 0): 18 tiles (two groups of 9), 35 tiles (three groups)
CASES = [(4600, 18), (8800, 35)]
H, I, E, K = 256, 256, 4, 2


def _setup(T, seed):
    w = scaled(WORKLOADS["mixtral_fwd_bwd"], T=T, H=H, I=I, E=E, k=K, zipf=0.0, seed=seed)
    inp = make_inputs(w)
    inp.logits[:, 0] += 100.0
    idx, p, m, pp = oracle_perm(inp, K, E)
    return inp, m, pp


def _bits(a):
    return f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


@pytest.mark.parametrize("T,tiles", CASES)
def test_long_expert_bf16(moe, T, tiles):
    inp, m, pp = _setup(T, 61)
    assert -(-int(m["split_sizes"][0]) // 256) == tiles
    xp_bits = inp.bits["x"][m["src_token"]]
    xp = dev_bf16(xp_bits)
    w1, w2 = dev_bf16(inp.bits["w1"]), dev_bf16(inp.bits["w2"])
    off = torch.from_numpy(m["offsets"].astype(np.int32)).cuda()
    prob = dev_f32(pp.astype(np.float32))
    R = T * K
    dyf, dyb = make_grad((R, H), 63)
    print(f"long expert bf16: T={T} expert 0 rows {m['split_sizes'][0]} ({tiles} row tiles)", flush=True)
    y, z, h = moe.moe_grouped_mlp_fwd(xp, w1, w2, off, prob, compute="bf16", save_for_bwd=True)
    dx, dw1, dw2, dprob = moe.moe_grouped_mlp_bwd(dev_bf16(dyb), xp, z, h, prob, w1, w2, off)
    torch.cuda.synchronize()
    xf = inp.x[m["src_token"]]
    ry, rz, rh = oracle.grouped_mlp_forward(xf, inp.w1, inp.w2, m["offsets"], pp)
    assert max_rel_err(host(y), ry) <= BF16_TOL
    assert max_rel_err(host(h), rh) <= BF16_TOL
    ref = oracle.grouped_mlp_backward(dyf, xf, inp.w1, inp.w2, m["offsets"], pp)
    assert max_rel_err(host(dx), ref["dx_perm"]) <= BF16_TOL
    assert max_rel_err(host(dw1), ref["dw_gate_up"]) <= BF16_TOL
    assert max_rel_err(host(dw2), ref["dw_down"]) <= BF16_TOL
    assert max_rel_err(dprob.cpu().numpy(), ref["dprob_perm"]) <= BF16_TOL


@pytest.mark.parametrize("T,tiles", CASES)
@pytest.mark.parametrize("compute", ["mxfp8", "fp8"])
def test_long_expert_low_precision(moe, T, tiles, compute):
    inp, m, pp = _setup(T, 62)
    assert -(-int(m["split_sizes"][0]) // 256) == tiles
    xp_bits = inp.bits["x"][m["src_token"]]
    xf = bf16_bits_to_f32(xp_bits)
    xp = dev_bf16(xp_bits)
    w1, w2 = dev_bf16(inp.bits["w1"]), dev_bf16(inp.bits["w2"])
    off = torch.from_numpy(m["offsets"].astype(np.int32)).cuda()
    prob = dev_f32(pp.astype(np.float32))
    R = T * K
    print(f"long expert {compute}: T={T} expert 0 rows {m['split_sizes'][0]} ({tiles} row tiles)", flush=True)
    y = moe.moe_grouped_mlp_fwd(xp, w1, w2, off, prob, compute=compute)
    # the backward on the oracle's exact forward rounded to bf16 (both sides take the same z, h)
    _, z, h = oracle.grouped_mlp_forward(xf, inp.w1, inp.w2, m["offsets"], pp)
    z_bits, h_bits = _bits(z), _bits(h)
    dyf, dyb = make_grad((R, H), 64)
    dx, dw1, dw2, dprob = moe.moe_grouped_mlp_bwd(dev_bf16(dyb), xp, dev_bf16(z_bits), dev_bf16(h_bits), prob, w1, w2,
                                                  off, compute=compute)
    torch.cuda.synchronize()
    zf, hf = bf16_bits_to_f32(z_bits), bf16_bits_to_f32(h_bits)
    if compute == "mxfp8":
        ry = oracle.grouped_mlp_forward_mxfp8(xf, inp.w1, inp.w2, m["offsets"], pp)[0]
        ref = oracle.grouped_mlp_backward_mxfp8(dyf, xf, zf, hf, inp.w1, inp.w2, m["offsets"], pp)
    else:
        ry = oracle.grouped_mlp_forward_fp8_tensor(xf, inp.w1, inp.w2, m["offsets"], pp)
        ref = oracle.grouped_mlp_backward_fp8_tensor(dyf, xf, zf, hf, inp.w1, inp.w2, m["offsets"], pp)
    assert max_rel_err(host(y), ry) <= LOWP_TOL
    assert max_rel_err(host(dx), ref["dx_perm"]) <= LOWP_TOL
    assert max_rel_err(host(dw1), ref["dw_gate_up"]) <= LOWP_TOL
    assert max_rel_err(host(dw2), ref["dw_down"]) <= LOWP_TOL
    assert max_rel_err(dprob.cpu().numpy(), ref["dprob_perm"]) <= LOWP_TOL
