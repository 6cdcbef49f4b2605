"""moe_permute_noalloc (the allocation-free variant of moe_permute, for callers that
cannot allocate: its count/scan scratch is a static device array) against moe_permute
with a caller-owned workspace, through the C ABI: two calls in a row, the second with
fewer tokens, experts and slots than the first, every output compared bit for bit."""
import ctypes

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from grouped_expert_gemm_amd import _lib
    return _lib.lib()


def _route(T, E, k, seed):
    g = np.random.default_rng(seed)
    idx = np.stack([g.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    prob = g.uniform(0.05, 1.0, (T, k)).astype(np.float32)
    x = torch.from_numpy(g.standard_normal((T, 128)).astype(np.float32)).to(torch.bfloat16).cuda()
    return x, torch.from_numpy(idx).cuda(), torch.from_numpy(prob).cuda()


def _outputs(T, H, E, k, dev):
    R = T * k
    return dict(x_perm=torch.full((R, H), -1.0, dtype=torch.bfloat16, device=dev),
                prob_perm=torch.full((R,), -1.0, device=dev),
                split=torch.full((E,), -1, dtype=torch.int32, device=dev),
                offsets=torch.full((E + 1,), -1, dtype=torch.int32, device=dev),
                rmap=torch.full((R,), -2, dtype=torch.int32, device=dev),
                src=torch.full((R,), -2, dtype=torch.int32, device=dev))


def _call(L, fn, x, idx, prob, E, o, ws):
    from grouped_expert_gemm_amd import _lib
    T, H = x.shape
    k = idx.shape[1]
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    args = [p(x), None, _lib.MOE_BF16, T, H, E, k, p(idx), p(prob), 0, p(o["x_perm"]), None, p(o["prob_perm"]),
            p(o["split"]), p(o["offsets"]), p(o["rmap"]), p(o["src"])]
    if fn == "moe_permute":
        args += [p(ws), ws.numel()]
    _lib.check(fn, getattr(L, fn)(*args, s))


@pytest.mark.parametrize("first,second", [((5000, 16, 4), (300, 8, 2)), ((20000, 128, 8), (3, 4, 2))])
def test_noalloc_permute_matches_workspace_permute(L, first, second):
    from grouped_expert_gemm_amd import _lib
    import grouped_expert_gemm_amd as moe
    for n, (T, E, k) in enumerate((first, second)):
        print(f"noalloc permute call {n}: T={T} E={E} k={k}", flush=True)
        x, idx, prob = _route(T, E, k, 100 + n)
        ws = torch.empty(max(1, moe.workspace_size(_lib.MOE_OP_PERMUTE, None, 0, T, E, k)), dtype=torch.uint8,
                         device="cuda")
        a = _outputs(T, 128, E, k, "cuda")
        b = _outputs(T, 128, E, k, "cuda")
        _call(L, "moe_permute", x, idx, prob, E, a, ws)
        _call(L, "moe_permute_noalloc", x, idx, prob, E, b, None)
        torch.cuda.synchronize()
        for key in a:
            if a[key].dtype == torch.bfloat16:
                assert torch.equal(a[key].view(torch.int16), b[key].view(torch.int16)), key
            else:
                assert torch.equal(a[key], b[key]), key
        assert int(b["offsets"][-1]) == T * k
