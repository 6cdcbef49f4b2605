"""The layer's training step captured into a HIP graph (torch.cuda.CUDAGraph) and
replayed: every library call only launches kernels on the caller's stream (no host
synchronisation, no allocation, no memset), so the whole step (route, permute, grouped
MLP forward, combine, dOut gather, grouped MLP backward, dx combine) can be captured
once and replayed. Each replay runs on new inputs copied into the captured buffers,
with the program's own eager work and synchronisations between replays, and is
compared bit for bit with the same step run eagerly on those inputs. Also
moe_permute_noalloc under capture against moe_permute."""
import ctypes

import pytest
import torch

pytestmark = pytest.mark.gpu

T, H, I, E, K = 512, 512, 512, 8, 2


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import grouped_expert_gemm_amd as g
    g.lib()
    return g


def _step(moe, logits, x, w1, w2, dout, compute):
    idx, prob = moe.moe_route_topk(logits, K)
    r = moe.moe_permute(x, idx, prob, E)
    y, z, h = moe.moe_grouped_mlp_fwd(r["x_perm"], w1, w2, r["offsets"], r["prob_perm"], compute=compute,
                                      save_for_bwd=True)
    out = moe.moe_unpermute_combine(y, r["row_id_map"], T, K)
    dy = moe.moe_permute(dout, idx, None, E, row_id_map=r["row_id_map"])["x_perm"]
    dx_perm, dw1, dw2, dprob = moe.moe_grouped_mlp_bwd(dy, r["x_perm"], z, h, r["prob_perm"], w1, w2, r["offsets"],
                                                       compute=compute)
    dx = moe.moe_unpermute_combine(dx_perm, r["row_id_map"], T, K)
    return out, dx, dw1, dw2, dprob


def _inputs(seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    logits = torch.randn((T, E), generator=g, device="cuda")
    x = torch.randn((T, H), generator=g, device="cuda").to(torch.bfloat16)
    dout = torch.randn((T, H), generator=g, device="cuda").to(torch.bfloat16)
    return logits, x, dout


@pytest.mark.parametrize("compute", ["bf16", "mxfp8", "fp8"])
def test_training_step_graph_replays(moe, compute):
    g = torch.Generator(device="cuda").manual_seed(7)
    w1 = (0.05 * torch.randn((E, 2 * I, H), generator=g, device="cuda")).to(torch.bfloat16)
    w2 = (0.05 * torch.randn((E, H, I), generator=g, device="cuda")).to(torch.bfloat16)
    logits, x, dout = _inputs(100)            # the captured step's input buffers
    print(f"{compute} training step under graph capture: T={T} H={H} I={I} E={E} k={K}", flush=True)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):             # warm-up outside the capture
        for _ in range(2):
            _step(moe, logits, x, w1, w2, dout, compute)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        static_out = _step(moe, logits, x, w1, w2, dout, compute)
    torch.cuda.synchronize()
    names = ("out", "dx", "dw_gate_up", "dw_down", "dprob")
    prev = None
    for rep in range(3):
        new = _inputs(200 + rep)
        for dst, src in zip((logits, x, dout), new):
            dst.copy_(src)
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in static_out]
        ref = _step(moe, *new[:2], w1, w2, new[2], compute)   # eager, on the same inputs
        torch.cuda.synchronize()
        for n, a, b in zip(names, got, ref):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {rep}: {n}"
        if prev is not None:   # the replay computed on its own inputs, not the captured ones
            assert not torch.equal(got[0], prev)
        prev = got[0]


def test_permute_noalloc_under_capture(moe):
    from grouped_expert_gemm_amd import _lib
    L = moe.lib()
    logits, x, _ = _inputs(300)
    R = T * K
    idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
    prob = torch.empty((T, K), dtype=torch.float32, device="cuda")
    xp = torch.empty((R, H), dtype=torch.bfloat16, device="cuda")
    pp = torch.empty(R, dtype=torch.float32, device="cuda")
    split = torch.empty(E, dtype=torch.int32, device="cuda")
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    rmap = torch.empty(R, dtype=torch.int32, device="cuda")
    src = torch.empty(R, dtype=torch.int32, device="cuda")
    p = lambda t: ctypes.c_void_p(t.data_ptr())

    def run():
        s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        _lib.check("route", L.moe_route_topk(p(logits), T, E, K, 1, p(idx), p(prob), s))
        _lib.check("permute_noalloc", L.moe_permute_noalloc(p(x), None, _lib.MOE_BF16, T, H, E, K, p(idx), p(prob), 0,
                                                            p(xp), None, p(pp), p(split), p(off), p(rmap), p(src), s))

    print(f"moe_permute_noalloc under graph capture: T={T} H={H} E={E} k={K}", flush=True)
    run()                                      # first call on the device looks up the scratch array
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for rep in range(3):
        nl, nx, _ = _inputs(400 + rep)
        logits.copy_(nl)
        x.copy_(nx)
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (xp, pp, split, off, rmap, src)]
        i2, p2 = moe.moe_route_topk(nl, K)
        ref = moe.moe_permute(nx, i2, p2, E)
        torch.cuda.synchronize()
        for n, a, b in zip(("x_perm", "prob_perm", "split_sizes", "offsets", "row_id_map", "src_token"), got,
                           (ref["x_perm"], ref["prob_perm"], ref["split_sizes"], ref["offsets"], ref["row_id_map"],
                            ref["src_token"])):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {rep}: {n}"
