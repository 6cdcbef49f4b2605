"""GPU parity of the router gate linear and the backward of top-k gating against the
CPU oracle: logits (bf16 products, float32 sums), d_logits (float32) and the gate
linear's input and weight gradients, at sizes with ragged token counts, every expert
sub-tile width, the token-chunked weight gradient, and at the Mixtral and Qwen3 layer
shapes."""
import numpy as np
import pytest
import torch

import oracle
from conftest import max_rel_err
from moe_inputs import bf16_bits_to_f32, f32_to_bf16_bits

pytestmark = pytest.mark.gpu

F32_SUM_TOL = 1e-5   # float32 sums of exact bf16 products, against float64
BF16_TOL = 2e-2      # bf16 outputs


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import grouped_expert_gemm_amd as g
    g.lib()
    return g


from gpu_util import dev_bf16, dev_f32, host  # noqa: E402


def _bf16(rng, shape, scale=1.0):
    bits = f32_to_bf16_bits((scale * rng.standard_normal(shape)).astype(np.float32))
    return bits, bf16_bits_to_f32(bits).astype(np.float64)


LOGITS = [
    # T, H, E
    (300, 256, 8),      # Mixtral's expert count, ragged token tile
    (1, 64, 1),
    (97, 128, 33),      # two expert sub-tiles, the second almost empty
    (64, 512, 128),     # Qwen3's expert count
    (40, 192, 256),
    (8192, 4096, 8),    # Mixtral-8x7B layer
    (16384, 2048, 128), # Qwen3-MoE-30B-A3B layer
]


@pytest.mark.parametrize("T,H,E", LOGITS, ids=[f"T{t}_H{h}_E{e}" for t, h, e in LOGITS])
def test_router_logits(moe, T, H, E):
    rng = np.random.default_rng(T + H + E)
    xb, x = _bf16(rng, (T, H))
    wb, w = _bf16(rng, (E, H), 0.02)
    print(f"router logits T={T} H={H} E={E}", flush=True)
    got = host(moe.moe_router_logits(dev_bf16(xb), dev_bf16(wb)))
    ref = oracle.router_logits(x, w)
    assert max_rel_err(got, ref) <= F32_SUM_TOL


BWD = [
    # T, E, k, renormalize
    (257, 8, 2, True), (257, 8, 2, False), (100, 128, 8, True), (100, 128, 8, False),
    (33, 256, 16, True), (33, 256, 16, False), (50, 6, 6, True), (7, 1, 1, True), (7, 1, 1, False),
    (65, 65, 3, False),
]


@pytest.mark.parametrize("T,E,k,renorm", BWD, ids=[f"T{a}_E{b}_k{c}_{'renorm' if d else 'full'}" for a, b, c, d in BWD])
def test_route_topk_bwd(moe, T, E, k, renorm):
    rng = np.random.default_rng(T * 7 + E + k)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    g = rng.standard_normal((T, k)).astype(np.float32)
    idx, p = oracle.route_topk(logits, k, renorm)
    print(f"route bwd T={T} E={E} k={k} renorm={renorm}", flush=True)
    d = moe.moe_route_topk_bwd(torch.from_numpy(idx).cuda(), dev_f32(p), dev_f32(g), E, renorm,
                               logits=dev_f32(logits))
    ref = oracle.route_topk_backward(logits, idx, g, renorm)
    got = host(d)
    assert max_rel_err(got, ref) <= F32_SUM_TOL
    if renorm:   # experts that were not chosen get exactly zero
        mask = np.ones((T, E), bool)
        np.put_along_axis(mask, idx, False, axis=1)
        assert np.all(got[mask] == 0.0)


ROUTER_BWD = [
    # T, H, E, with dx_in
    (300, 256, 8, False),
    (300, 264, 8, True),     # H not a multiple of 64
    (2500, 128, 128, True),  # three token chunks of the weight gradient
    (1, 64, 3, False),
    (1025, 4096, 8, True),   # Mixtral width, two chunks
    (333, 264, 72, False),   # 9 expert groups of 8, ragged columns and tokens
    (70, 8, 64, True),       # one column block of 8
    (5000, 2048, 128, False),  # the Qwen3 width, several token chunks
]


@pytest.mark.parametrize("T,H,E,acc", ROUTER_BWD, ids=[f"T{a}_H{b}_E{c}_{'acc' if d else 'new'}" for a, b, c, d in ROUTER_BWD])
def test_router_bwd(moe, T, H, E, acc):
    rng = np.random.default_rng(T + 3 * H + E)
    xb, x = _bf16(rng, (T, H))
    wb, w = _bf16(rng, (E, H), 0.02)
    dl = (0.1 * rng.standard_normal((T, E))).astype(np.float32)
    print(f"router bwd T={T} H={H} E={E} dx_in={acc}", flush=True)
    dinb, din = _bf16(rng, (T, H), 0.01) if acc else (None, 0.0)
    dx, dw = moe.moe_router_bwd(dev_bf16(xb), dev_bf16(wb), dev_f32(dl),
                                dx_in=dev_bf16(dinb) if acc else None)
    rdx, rdw = oracle.router_backward(x, w, dl)
    assert max_rel_err(host(dx), rdx + din) <= BF16_TOL
    assert max_rel_err(host(dw), rdw) <= F32_SUM_TOL


def test_router_bwd_no_tokens(moe):
    x = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    w = torch.ones((8, 128), dtype=torch.bfloat16, device="cuda")
    dl = torch.empty((0, 8), dtype=torch.float32, device="cuda")
    dx, dw = moe.moe_router_bwd(x, w, dl)
    torch.cuda.synchronize()
    assert dx.shape == (0, 128)
    assert torch.count_nonzero(dw).item() == 0
