"""GPU parity of the grouped MLP (forward, backward) and of the whole layer
against the CPU oracle, at multi-tile shapes with ragged expert groups, empty
experts, and the tiny float32 workload. Tolerance: max|a-b| / max|b| <= 2e-2
for bf16 outputs with float32 accumulation (the float32 path is held to 1e-4)."""
import numpy as np
import pytest
import torch

import oracle
from conftest import max_rel_err, record_parity
from moe_inputs import WORKLOADS, make_grad, make_inputs, scaled

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
F32_TOL = 1e-4


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import grouped_expert_gemm_amd as g
    g.lib()
    return g


from gpu_util import dev_bf16, dev_f32, host, oracle_perm  # noqa: E402


def _setup(w, zero_experts=()):
    inp = make_inputs(w)
    if zero_experts:
        inp.logits[:, list(zero_experts)] -= 100.0
    idx, p, m, pp = oracle_perm(inp, w.k, w.E)
    for e in zero_experts:
        assert m["split_sizes"][e] == 0
    return inp, idx, p, m, pp


def _dev_inputs(inp, m, pp):
    xp_bits = inp.bits["x"][m["src_token"]]
    return (dev_bf16(xp_bits), dev_bf16(inp.bits["w1"]), dev_bf16(inp.bits["w2"]),
            torch.from_numpy(m["offsets"].astype(np.int32)).cuda(), dev_f32(pp.astype(np.float32)))


FWD_SHAPES = [
    # name, T, H, I, E, k, zipf, empty experts
    ("ragged", 1500, 512, 384, 4, 2, 0.0, ()),
    ("skewed", 1200, 256, 128, 16, 4, 1.2, (3, 9)),
    ("one_expert", 300, 256, 256, 1, 1, 0.0, ()),
    ("tiny_groups", 37, 256, 128, 8, 2, 0.0, (0,)),
    ("max_experts", 300, 256, 256, 256, 2, 0.0, ()),   # E = 256: experts of 0-3 rows, many idle
]


@pytest.mark.parametrize("shape", FWD_SHAPES, ids=[s[0] for s in FWD_SHAPES])
def test_grouped_mlp_fwd_bf16(moe, shape):
    name, T, H, I, E, k, zipf, empty = shape
    w = scaled(WORKLOADS["mixtral_fwd"], T=T, H=H, I=I, E=E, k=k, zipf=zipf, seed=11)
    inp, idx, p, m, pp = _setup(w, empty)
    xp, w1, w2, off, prob = _dev_inputs(inp, m, pp)
    print(f"mlp fwd bf16 {name}: R={T * k} H={H} I={I} E={E}", flush=True)
    y, z, h = moe.moe_grouped_mlp_fwd(xp, w1, w2, off, prob, compute="bf16", save_for_bwd=True)
    y2 = moe.moe_grouped_mlp_fwd(xp, w1, w2, off, prob, compute="bf16")
    torch.cuda.synchronize()
    ry, rz, rh = oracle.grouped_mlp_forward(inp.x[m["src_token"]], inp.w1, inp.w2, m["offsets"], pp)
    assert max_rel_err(host(y), ry) <= BF16_TOL
    assert max_rel_err(host(z), rz) <= BF16_TOL
    assert max_rel_err(host(h), rh) <= BF16_TOL
    assert torch.equal(y, y2), "saving z/h must not change y"


BWD_SHAPES = [
    ("ragged", 700, 512, 256, 4, 2, 0.0, ()),
    ("skewed_empty", 900, 256, 256, 8, 2, 1.2, (5,)),
    # more weight-gradient tiles than CUs (dW1: 16 experts x 8 x 4 tiles): each workgroup
    # runs several, issuing the next tile's first copies before its stores; skewed
    # expert sizes give both long and short K loops, and idle experts in the chain
    ("many_tiles", 1200, 1024, 1024, 16, 2, 1.2, (4, 11)),
    ("max_experts", 300, 256, 256, 256, 2, 0.0, ()),   # E = 256, many idle experts
]


@pytest.mark.parametrize("shape", BWD_SHAPES, ids=[s[0] for s in BWD_SHAPES])
def test_grouped_mlp_bwd_bf16(moe, shape):
    name, T, H, I, E, k, zipf, empty = shape
    w = scaled(WORKLOADS["mixtral_fwd_bwd"], T=T, H=H, I=I, E=E, k=k, zipf=zipf, seed=12)
    inp, idx, p, m, pp = _setup(w, empty)
    xp, w1, w2, off, prob = _dev_inputs(inp, m, pp)
    R = T * k
    dyf, dyb = make_grad((R, H), 99)
    print(f"mlp bwd bf16 {name}: R={R} H={H} I={I} E={E}", flush=True)
    y, z, h = moe.moe_grouped_mlp_fwd(xp, w1, w2, off, prob, compute="bf16", save_for_bwd=True)
    dx, dw1, dw2, dprob = moe.moe_grouped_mlp_bwd(dev_bf16(dyb), xp, z, h, prob, w1, w2, off)
    torch.cuda.synchronize()
    ref = oracle.grouped_mlp_backward(dyf, inp.x[m["src_token"]], inp.w1, inp.w2, m["offsets"], pp)
    assert max_rel_err(host(dx), ref["dx_perm"]) <= BF16_TOL
    assert max_rel_err(host(dw1), ref["dw_gate_up"]) <= BF16_TOL
    assert max_rel_err(host(dw2), ref["dw_down"]) <= BF16_TOL
    assert max_rel_err(dprob.cpu().numpy(), ref["dprob_perm"]) <= BF16_TOL
    for e in empty:
        assert not host(dw1)[e].any() and not host(dw2)[e].any(), "idle expert must get zero weight gradients"


def test_tiny_layer_f32_forward_and_backward(moe):
    """The tiny workload end to end in float32: route -> permute -> grouped MLP -> combine,
    against the per-expert loop; then the backward against the loop's backward."""
    w = WORKLOADS["tiny"]
    inp = make_inputs(w)
    T, H, E, k = w.T, w.H, w.E, w.k
    idx, p = moe.moe_route_topk(dev_f32(inp.logits), k)
    x = dev_f32(inp.x)
    r = moe.moe_permute(x, idx, p, E)
    w1, w2 = dev_f32(inp.w1), dev_f32(inp.w2)
    y, z, h = moe.moe_grouped_mlp_fwd(r["x_perm"], w1, w2, r["offsets"], r["prob_perm"], compute="f32",
                                      save_for_bwd=True)
    out = moe.moe_unpermute_combine(y, r["row_id_map"], T, k)
    ridx, rp = oracle.route_topk(inp.logits, k)
    ref = oracle.moe_ffn_forward(inp.x, inp.w1, inp.w2, ridx, rp)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert max_rel_err(out.cpu().numpy(), ref) <= F32_TOL

    dout = np.random.default_rng(7).standard_normal((T, H)).astype(np.float32)
    dyp = moe.moe_permute(dev_f32(dout), idx, None, E, row_id_map=r["row_id_map"])["x_perm"]
    dx_perm, dw1, dw2, dprob_perm = moe.moe_grouped_mlp_bwd(dyp, r["x_perm"], z, h, r["prob_perm"], w1, w2,
                                                            r["offsets"], compute="f32")
    dx = moe.moe_unpermute_combine(dx_perm, r["row_id_map"], T, k)
    g = oracle.moe_ffn_backward(inp.x, inp.w1, inp.w2, ridx, rp, dout)
    assert max_rel_err(dx.cpu().numpy(), g["dx"]) <= F32_TOL
    assert max_rel_err(dw1.cpu().numpy(), g["dw_gate_up"]) <= F32_TOL
    assert max_rel_err(dw2.cpu().numpy(), g["dw_down"]) <= F32_TOL
    # dprob [T, k] gathered on the GPU (a one-slot combine of one-column rows)
    dprob = moe.moe_unpermute_combine(dprob_perm.view(T * k, 1), r["row_id_map"], T * k, 1).view(T, k)
    assert max_rel_err(dprob.cpu().numpy(), g["drouting_weights"]) <= F32_TOL


# (T, H, I, E, k): H and I off the 32 and 64 grids of the float32 tiles (64 x 64, K in
# steps of 32), experts spanning several 64-row tiles with ragged ends, the last
# expert idle
F32_RAGGED = [(300, 100, 72, 5, 2), (400, 33, 130, 3, 1)]


@pytest.mark.parametrize("T,H,I,E,k", F32_RAGGED)
def test_f32_ragged_shapes(moe, T, H, I, E, k):
    """The float32 grouped GEMMs at sizes that are not multiples of their tiles: the
    MLP forward and backward, the grouped linear and the fused gate_up, against the
    oracle."""
    w = scaled(WORKLOADS["tiny"], T=T, H=H, I=I, E=E, k=k, seed=T + H + I)
    inp = make_inputs(w)
    inp.logits[:, E - 1] -= 100.0
    idx, p, m, pp = oracle_perm(inp, k, E)
    assert m["split_sizes"][E - 1] == 0 and max(m["split_sizes"]) > 128
    xf = inp.x[m["src_token"]]
    xp = dev_f32(xf)
    w1, w2 = dev_f32(inp.w1), dev_f32(inp.w2)
    off = torch.from_numpy(m["offsets"].astype(np.int32)).cuda()
    prob = dev_f32(pp)
    R = T * k
    dyf = np.random.default_rng(5).standard_normal((R, H)).astype(np.float32)
    print(f"f32 ragged: T={T} H={H} I={I} E={E} k={k} rows per expert {m['split_sizes'].tolist()}", flush=True)
    y, z, h = moe.moe_grouped_mlp_fwd(xp, w1, w2, off, prob, compute="f32", save_for_bwd=True)
    dx, dw1, dw2, dprob = moe.moe_grouped_mlp_bwd(dev_f32(dyf), xp, z, h, prob, w1, w2, off, compute="f32")
    lin = moe.moe_grouped_linear(xp, w1, off)
    h2, z2 = moe.moe_grouped_gate_up_swiglu(xp, w1, off, prob, save_z=True)
    torch.cuda.synchronize()
    ry, rz, rh = oracle.grouped_mlp_forward(xf, inp.w1, inp.w2, m["offsets"], pp)
    assert max_rel_err(host(y), ry) <= F32_TOL
    assert max_rel_err(host(z), rz) <= F32_TOL
    assert max_rel_err(host(h), rh) <= F32_TOL
    assert np.array_equal(host(h2), host(h)) and np.array_equal(host(z2), host(z))
    assert max_rel_err(host(lin), oracle.grouped_linear(xf, inp.w1, m["offsets"])) <= F32_TOL
    ref = oracle.grouped_mlp_backward(dyf, xf, inp.w1, inp.w2, m["offsets"], pp)
    assert max_rel_err(host(dx), ref["dx_perm"]) <= F32_TOL
    assert max_rel_err(host(dw1), ref["dw_gate_up"]) <= F32_TOL
    assert max_rel_err(host(dw2), ref["dw_down"]) <= F32_TOL
    assert max_rel_err(dprob.cpu().numpy(), ref["dprob_perm"]) <= F32_TOL
    assert not host(dw1)[E - 1].any() and not host(dw2)[E - 1].any(), "idle expert must get zero weight gradients"


def test_f32_one_row_tiny_sizes(moe):
    """The float32 path at its smallest: one routed row, H = 5 and I = 3 (K below one
    32-wide stage, one partial tile everywhere), the second expert idle."""
    T, H, I, E, k = 1, 5, 3, 2, 1
    w = scaled(WORKLOADS["tiny"], T=T, H=H, I=I, E=E, k=k, seed=77)
    inp = make_inputs(w)
    inp.logits[:, 1] -= 100.0
    idx, p, m, pp = oracle_perm(inp, k, E)
    assert list(m["split_sizes"]) == [1, 0]
    xf = inp.x[m["src_token"]]
    xp, w1, w2 = dev_f32(xf), dev_f32(inp.w1), dev_f32(inp.w2)
    off = torch.from_numpy(m["offsets"].astype(np.int32)).cuda()
    prob = dev_f32(pp)
    dyf = np.random.default_rng(6).standard_normal((T * k, H)).astype(np.float32)
    print("f32 one row: H=5 I=3 E=2", flush=True)
    y, z, h = moe.moe_grouped_mlp_fwd(xp, w1, w2, off, prob, compute="f32", save_for_bwd=True)
    dx, dw1, dw2, dprob = moe.moe_grouped_mlp_bwd(dev_f32(dyf), xp, z, h, prob, w1, w2, off, compute="f32")
    torch.cuda.synchronize()
    ry, _, rh = oracle.grouped_mlp_forward(xf, inp.w1, inp.w2, m["offsets"], pp)
    assert max_rel_err(host(y), ry) <= F32_TOL and max_rel_err(host(h), rh) <= F32_TOL
    ref = oracle.grouped_mlp_backward(dyf, xf, inp.w1, inp.w2, m["offsets"], pp)
    assert max_rel_err(host(dx), ref["dx_perm"]) <= F32_TOL
    assert max_rel_err(host(dw1), ref["dw_gate_up"]) <= F32_TOL
    assert max_rel_err(host(dw2), ref["dw_down"]) <= F32_TOL
    assert max_rel_err(dprob.cpu().numpy(), ref["dprob_perm"]) <= F32_TOL


def test_layer_bf16_end_to_end(moe):
    """route -> permute -> grouped MLP -> combine in bf16 against the per-expert loop."""
    w = scaled(WORKLOADS["qwen3_fwd"], T=2000, H=512, I=256, E=32, k=4, seed=21)
    inp = make_inputs(w)
    idx, p = moe.moe_route_topk(dev_f32(inp.logits), w.k)
    r = moe.moe_permute(dev_bf16(inp.bits["x"]), idx, p, w.E)
    y = moe.moe_grouped_mlp_fwd(r["x_perm"], dev_bf16(inp.bits["w1"]), dev_bf16(inp.bits["w2"]), r["offsets"],
                                r["prob_perm"], compute="bf16")
    out = moe.moe_unpermute_combine(y, r["row_id_map"], w.T, w.k)
    ridx, rp = oracle.route_topk(inp.logits, w.k)
    ref = oracle.moe_ffn_forward(inp.x, inp.w1, inp.w2, ridx, rp)
    assert max_rel_err(host(out), ref) <= BF16_TOL


@pytest.mark.parametrize("shape", [("mixtral_like", 600, 512, 256, 8, 2, 0.0), ("qwen_like", 700, 256, 256, 32, 8, 1.2)],
                         ids=["mixtral_like", "qwen_like"])
def test_layer_bf16_forward_backward_with_gpu_gathers(moe, shape):
    """The bf16 layer forward and backward exactly as the benchmark runs it: the output
    gradient gathered onto the routed rows, the grouped MLP backward, dx combined over
    each token's k rows and dprob [T, k] gathered from the routed rows, all on the GPU;
    against the per-expert loop's backward (dx, the weight gradients, and the gradient
    w.r.t. the routing probabilities)."""
    name, T, H, I, E, k, zipf = shape
    w = scaled(WORKLOADS["mixtral_fwd_bwd"], T=T, H=H, I=I, E=E, k=k, zipf=zipf, seed=13)
    inp = make_inputs(w)
    R = T * k
    print(f"layer bf16 fwd+bwd {name}: T={T} H={H} I={I} E={E} k={k}", flush=True)
    idx, p = moe.moe_route_topk(dev_f32(inp.logits), k)
    r = moe.moe_permute(dev_bf16(inp.bits["x"]), idx, p, E)
    w1, w2 = dev_bf16(inp.bits["w1"]), dev_bf16(inp.bits["w2"])
    y, z, h = moe.moe_grouped_mlp_fwd(r["x_perm"], w1, w2, r["offsets"], r["prob_perm"], save_for_bwd=True)
    out = moe.moe_unpermute_combine(y, r["row_id_map"], T, k)
    dyp = moe.moe_permute(dev_bf16(inp.bits["dout"]), idx, None, E, row_id_map=r["row_id_map"])["x_perm"]
    dxp, dw1, dw2, dprob_perm = moe.moe_grouped_mlp_bwd(dyp, r["x_perm"], z, h, r["prob_perm"], w1, w2, r["offsets"])
    dx = moe.moe_unpermute_combine(dxp, r["row_id_map"], T, k)
    dprob = moe.moe_unpermute_combine(dprob_perm.view(R, 1), r["row_id_map"], R, 1).view(T, k)
    torch.cuda.synchronize()
    ridx, rp = oracle.route_topk(inp.logits, k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    ref = oracle.moe_ffn_forward(inp.x, inp.w1, inp.w2, ridx, rp)
    g = oracle.moe_ffn_backward(inp.x, inp.w1, inp.w2, ridx, rp, inp.dout)
    errs = dict(out=max_rel_err(host(out), ref), dx=max_rel_err(host(dx), g["dx"]),
                dw_gate_up=max_rel_err(host(dw1), g["dw_gate_up"]), dw_down=max_rel_err(host(dw2), g["dw_down"]),
                dprob=max_rel_err(dprob.cpu().numpy(), g["drouting_weights"]))
    print("  " + ", ".join(f"{k2} {v:.2e}" for k2, v in errs.items()), flush=True)
    record_parity("layer bf16 fwd+bwd with GPU gathers", **errs)
    for k2, v in errs.items():
        assert v <= BF16_TOL, k2
    # the gather moves bits: each dprob[t, j] is the dprob_perm entry of its row
    assert torch.equal(dprob.view(-1), dprob_perm[r["row_id_map"].long()])
