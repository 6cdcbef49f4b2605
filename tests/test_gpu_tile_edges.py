"""GPU parity of the forward grouped GEMM at expert sizes on every row-tile boundary:
0, 1, a 32-row sub-tile, 64 / 65, 128 / 129, 192 / 193 rows past a multiple of the 256-row tile
(the boundaries of the forward kernel's active row sub-tile counts 1-4),
and whole tiles (the last tile of an expert is mostly rows past it, which the copies'
range check turns into zeros and the stores skip). Outputs start as NaN so a row no
kernel writes fails the check; both the plain-store (GroupedLinear) and the ScaledSwiGLU
epilogue (with z saved) are compared with the oracle at the bf16 tolerance
max|a-b| / max|b| <= 2e-2, with and without the split-K workspace, at a long and a
short K range.
"""
import numpy as np
import pytest
import torch

import oracle
from conftest import max_rel_err
from moe_inputs import bf16_bits_to_f32, f32_to_bf16_bits

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2

SIZES = [0, 1, 31, 64, 65, 100, 128, 129, 192, 193, 255, 256, 257, 300, 384, 385, 449, 576]


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


@pytest.mark.parametrize("use_ws,K", [(False, 512), (True, 512), (False, 192)])
def test_grouped_linear_tile_edges(moe, use_ws, K):
    rng = np.random.default_rng(11)
    E, N = len(SIZES), 512
    off = _offsets(SIZES)
    R = int(off[-1])
    xb, x = _bf16(rng, (R, K), 1.0)
    wb, w = _bf16(rng, (E, N, K), 0.02)
    print(f"grouped linear tile edges: R={R} K={K} N={N} E={E} workspace={use_ws}", flush=True)
    ref = oracle.grouped_linear(x, w, off)
    y = torch.full((R, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = moe.gemm_workspace("cuda") if use_ws else None
    moe.moe_grouped_linear(dev_bf16(xb), dev_bf16(wb), torch.from_numpy(off).cuda(), out=y, workspace=ws)
    torch.cuda.synchronize()
    yh = host(y)
    for e in range(E):
        a, b = off[e], off[e + 1]
        if b > a:
            assert max_rel_err(yh[a:b], ref[a:b]) <= BF16_TOL, (e, SIZES[e])


@pytest.mark.parametrize("use_ws", [False, True])
def test_gate_up_swiglu_tile_edges(moe, use_ws):
    rng = np.random.default_rng(12)
    E, H, I = len(SIZES), 512, 256
    off = _offsets(SIZES)
    R = int(off[-1])
    xb, x = _bf16(rng, (R, H), 1.0)
    wb, w1 = _bf16(rng, (E, 2 * I, H), 0.02)
    prob = rng.uniform(0.1, 1.0, R)
    print(f"gate_up tile edges: R={R} H={H} I={I} E={E} workspace={use_ws}", flush=True)
    _, rz, rh = oracle.grouped_mlp_forward(x, w1, np.zeros((E, H, I)), off, prob)
    ws = moe.gemm_workspace("cuda") if use_ws else None
    h = torch.full((R, I), float("nan"), dtype=torch.bfloat16, device="cuda")
    res = moe.moe_grouped_gate_up_swiglu(dev_bf16(xb), dev_bf16(wb), torch.from_numpy(off).cuda(), dev_f32(prob),
                                         save_z=True, out=h, workspace=ws)
    z = res[1]
    torch.cuda.synchronize()
    hh, zh = host(h), host(z)
    for e in range(E):
        a, b = off[e], off[e + 1]
        if b > a:
            assert max_rel_err(hh[a:b], rh[a:b]) <= BF16_TOL, (e, SIZES[e])
            assert max_rel_err(zh[a:b], rz[a:b]) <= BF16_TOL, (e, SIZES[e])


@pytest.mark.parametrize("compute", ["mxfp8", "fp8"])
def test_fp8_forward_tile_edges(moe, compute):
    """The MXFP8 and per-tensor FP8 grouped MLP forwards at the same expert sizes, against
    the oracle's quantise -> dequantise forwards (max rel error <= 6e-2)."""
    rng = np.random.default_rng(13)
    E, H, I = len(SIZES), 256, 256
    off = _offsets(SIZES)
    R = int(off[-1])
    xb, x = _bf16(rng, (R, H), 1.0)
    w1b, w1 = _bf16(rng, (E, 2 * I, H), 0.02)
    w2b, w2 = _bf16(rng, (E, H, I), 0.02)
    prob = rng.uniform(0.1, 1.0, R)
    print(f"{compute} forward tile edges: R={R} H={H} I={I} E={E}", flush=True)
    if compute == "mxfp8":
        ref, _ = oracle.grouped_mlp_forward_mxfp8(x, w1, w2, off, prob)
    else:
        ref = oracle.grouped_mlp_forward_fp8_tensor(x, w1, w2, off, prob)
    y = torch.full((R, H), float("nan"), dtype=torch.bfloat16, device="cuda")
    moe.moe_grouped_mlp_fwd(dev_bf16(xb), dev_bf16(w1b), dev_bf16(w2b), torch.from_numpy(off).cuda(),
                            dev_f32(prob), compute=compute, out=y)
    torch.cuda.synchronize()
    yh = host(y)
    assert not np.isnan(yh).any()
    assert max_rel_err(yh, ref) <= 6e-2
