"""GPU parity of the split-K tail of the forward grouped GEMM (GroupedLinear and the
fused gate_up + ScaledSwiGLU): when the last round of tiles would leave most CUs idle,
its tiles are cut along K into float32 partial tiles and summed by a second kernel.

Small cases are shaped so that the launch grid (the host's tile bound) is at least
twice the tile count, which forces the split whatever the CU count; the workspace's
header (tail tile count, chunks per tile) shows that it happened. Larger cases have
full rounds plus a ragged tail on a 256-CU GPU. Every case is checked against the
oracle with the bf16 tolerance (max|a-b| / max|b| <= 2e-2), with and without a
workspace.
"""
import numpy as np
import pytest
import torch

import oracle
from conftest import max_rel_err
from moe_inputs import bf16_bits_to_f32, f32_to_bf16_bits

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import grouped_expert_gemm_amd as g
    g.lib()
    return g


from gpu_util import dev_bf16, dev_f32, host  # noqa: E402


def _bf16(rng, shape, scale):
    bits = f32_to_bf16_bits((scale * rng.standard_normal(shape)).astype(np.float32))
    return bits, bf16_bits_to_f32(bits).astype(np.float64)


def _offsets(sizes):
    return np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)


def _split_header(ws):
    head = ws[:16].cpu().numpy().view(np.int32)
    return int(head[0]), int(head[1])


LINEAR = [
    # name, expert sizes, K, N, split expected
    ("two_experts", [150, 150], 1024, 256, True),
    ("mostly_empty", [0, 200, 0, 0, 57, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0], 512, 512, True),
    ("rounds_and_tail", [4352], 512, 4096, False),
    ("ragged_rounds", [1000, 3000, 17], 256, 2048, False),
]


@pytest.mark.parametrize("case", LINEAR, ids=[c[0] for c in LINEAR])
def test_grouped_linear_split_tail(moe, case):
    name, sizes, K, N, must_split = case
    rng = np.random.default_rng(101)
    E = len(sizes)
    off = _offsets(sizes)
    R = int(off[-1])
    xb, x = _bf16(rng, (R, K), 1.0)
    wb, w = _bf16(rng, (E, N, K), 0.02)
    print(f"grouped linear split {name}: R={R} K={K} N={N} E={E}", flush=True)
    ref = oracle.grouped_linear(x, w, off)
    ws = moe.gemm_workspace("cuda")
    ws.fill_(0xFF)  # the kernels must not rely on a cleared workspace
    d_off = torch.from_numpy(off).cuda()
    y = moe.moe_grouped_linear(dev_bf16(xb), dev_bf16(wb), d_off, workspace=ws)
    y0 = moe.moe_grouped_linear(dev_bf16(xb), dev_bf16(wb), d_off)
    torch.cuda.synchronize()
    n_tail, split = _split_header(ws)
    print(f"  tail tiles {n_tail}, chunks {split}", flush=True)
    if must_split:
        assert n_tail > 0 and split >= 2
    assert max_rel_err(host(y), ref) <= BF16_TOL
    assert max_rel_err(host(y0), ref) <= BF16_TOL


GATE_UP = [
    # name, expert sizes, H, I, split expected
    ("two_experts", [150, 150], 1024, 128, True),
    ("rounds_and_tail", [4352], 512, 2048, False),
]


@pytest.mark.parametrize("case", GATE_UP, ids=[c[0] for c in GATE_UP])
def test_gate_up_swiglu_split_tail(moe, case):
    name, sizes, H, I, must_split = case
    rng = np.random.default_rng(202)
    E = len(sizes)
    off = _offsets(sizes)
    R = int(off[-1])
    xb, x = _bf16(rng, (R, H), 1.0)
    wb, w1 = _bf16(rng, (E, 2 * I, H), 0.02)
    prob = rng.uniform(0.1, 1.0, R)
    print(f"gate_up split {name}: R={R} H={H} I={I} E={E}", flush=True)
    _, rz, rh = oracle.grouped_mlp_forward(x, w1, np.zeros((E, H, I)), off, prob)
    ws = moe.gemm_workspace("cuda")
    ws.fill_(0xFF)
    d_off = torch.from_numpy(off).cuda()
    h, z = moe.moe_grouped_gate_up_swiglu(dev_bf16(xb), dev_bf16(wb), d_off, dev_f32(prob), save_z=True,
                                          workspace=ws)
    h0 = moe.moe_grouped_gate_up_swiglu(dev_bf16(xb), dev_bf16(wb), d_off, dev_f32(prob))
    torch.cuda.synchronize()
    n_tail, split = _split_header(ws)
    print(f"  tail tiles {n_tail}, chunks {split}", flush=True)
    if must_split:
        assert n_tail > 0 and split >= 2
    assert max_rel_err(host(h), rh) <= BF16_TOL
    assert max_rel_err(host(z), rz) <= BF16_TOL
    assert max_rel_err(host(h0), rh) <= BF16_TOL
