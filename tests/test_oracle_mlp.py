"""Pins for the oracle's expert MLP forward and backward (CPU only).

The oracle's per-expert loop is checked against: a dense brute force that
runs every expert on every token and masks to the top-k (torch, float64), the
k = E full mixture, the E = 1 / k = 1 textbook SwiGLU MLP, a closed form with
H = I = 1 (which also fixes which half of gate_up is the gate), token-shuffle
equivariance, central finite differences, torch.autograd, and two exact
identities from linearity.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from moe_inputs import WORKLOADS, make_inputs, scaled


def _tiny(T=48, H=16, I=24, E=6, k=2, seed=0, zipf=0.0):
    w = scaled(WORKLOADS["tiny"], T=T, H=H, I=I, E=E, k=k, seed=seed, zipf=zipf)
    return make_inputs(w)


def _dense_brute_force(x, w1, w2, logits, k):
    """Every expert on every token (torch float64), weighted by a mask that holds
    the renormalised top-k softmax weight and zero elsewhere."""
    X = torch.from_numpy(x).double()
    L = torch.from_numpy(logits).double()
    E = w1.shape[0]
    I = w1.shape[1] // 2
    probs = torch.softmax(L, dim=1)
    vals, pos = torch.topk(L, k, dim=1)         # ties do not occur for continuous draws
    mask = torch.zeros_like(probs).scatter(1, pos, 1.0)
    wts = probs * mask
    wts = wts / wts.sum(1, keepdim=True)
    out = torch.zeros_like(X)
    for e in range(E):
        W1 = torch.from_numpy(w1[e]).double()
        W2 = torch.from_numpy(w2[e]).double()
        hidden = F.silu(F.linear(X, W1[:I])) * F.linear(X, W1[I:])
        out += wts[:, e:e + 1] * F.linear(hidden, W2)
    return out.numpy()


@pytest.mark.parametrize("E,k", [(6, 2), (8, 3), (4, 1)])
def test_forward_matches_dense_brute_force(E, k):
    inp = _tiny(E=E, k=k, seed=E * 10 + k)
    idx, p = oracle.route_topk(inp.logits, k)
    out = oracle.moe_ffn_forward(inp.x, inp.w1, inp.w2, idx, p)
    ref = _dense_brute_force(inp.x, inp.w1, inp.w2, inp.logits, k)
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)


def test_k_equals_E_is_full_softmax_mixture():
    inp = _tiny(E=5, k=5, seed=7)
    idx, p = oracle.route_topk(inp.logits, 5)
    out = oracle.moe_ffn_forward(inp.x, inp.w1, inp.w2, idx, p)
    X = torch.from_numpy(inp.x).double()
    probs = torch.softmax(torch.from_numpy(inp.logits).double(), 1)
    I = inp.w1.shape[1] // 2
    ref = torch.zeros_like(X)
    for e in range(5):
        W1 = torch.from_numpy(inp.w1[e]).double()
        W2 = torch.from_numpy(inp.w2[e]).double()
        ref += probs[:, e:e + 1] * F.linear(F.silu(F.linear(X, W1[:I])) * F.linear(X, W1[I:]), W2)
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-10, atol=1e-12)


def test_single_expert_is_plain_swiglu_mlp():
    inp = _tiny(E=1, k=1, seed=8)
    idx, p = oracle.route_topk(inp.logits, 1)
    assert np.all(p == 1.0)
    out = oracle.moe_ffn_forward(inp.x, inp.w1, inp.w2, idx, p)
    X = torch.from_numpy(inp.x).double()
    W1 = torch.from_numpy(inp.w1[0]).double()
    W2 = torch.from_numpy(inp.w2[0]).double()
    gate, up = F.linear(X, W1).chunk(2, dim=1)
    ref = F.linear(F.silu(gate) * up, W2)
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-14)


def test_closed_form_one_by_one():
    """H = I = 1, E = 2, k = 2: out = sum_e p_e * d_e * silu(g_e x) * (u_e x)."""
    x = np.array([[0.7], [-1.3]])
    w1 = np.array([[[2.0], [0.5]], [[-1.0], [3.0]]])     # [E, 2I=2, H=1]: row 0 gate, row 1 up
    w2 = np.array([[[1.5]], [[-0.25]]])                   # [E, H=1, I=1]
    logits = np.array([[0.2, -0.4], [1.0, 1.5]], np.float32)
    idx, p = oracle.route_topk(logits, 2)
    out = oracle.moe_ffn_forward(x, w1, w2, idx, p)
    for t in range(2):
        ex = [math.exp(float(v)) for v in logits[t]]
        wt = [v / sum(ex) for v in ex]
        s = 0.0
        for e in range(2):
            g = w1[e, 0, 0] * x[t, 0]
            u = w1[e, 1, 0] * x[t, 0]
            s += wt[e] * w2[e, 0, 0] * (g / (1.0 + math.exp(-g))) * u
        assert out[t, 0] == pytest.approx(s, rel=1e-13)


def test_token_shuffle_equivariance():
    inp = _tiny(seed=9)
    idx, p = oracle.route_topk(inp.logits, 2)
    out = oracle.moe_ffn_forward(inp.x, inp.w1, inp.w2, idx, p)
    perm = np.random.default_rng(1).permutation(inp.x.shape[0])
    out2 = oracle.moe_ffn_forward(inp.x[perm], inp.w1, inp.w2, idx[perm], p[perm])
    np.testing.assert_allclose(out2, out[perm], rtol=1e-13, atol=1e-15)


def test_grouped_form_equals_loop():
    """Permute -> grouped MLP with the probability inside SwiGLU -> unweighted
    combine gives the loop's output (probability applied after the expert)."""
    inp = _tiny(E=8, k=3, seed=10, zipf=1.2)
    T, k, E = inp.x.shape[0], 3, 8
    idx, p = oracle.route_topk(inp.logits, k)
    m = oracle.permute(idx, E)
    xp = oracle.gather_rows(inp.x, m["src_token"])
    pp = p.ravel()[m["src_token"] * k + m["src_slot"]]
    y, z, h = oracle.grouped_mlp_forward(xp, inp.w1, inp.w2, m["offsets"], pp)
    out = oracle.unpermute_combine(y, m["row_id_map"], T, k)
    ref = oracle.moe_ffn_forward(inp.x, inp.w1, inp.w2, idx, p)
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-13)
    # p == 1 reduces ScaledSwiGLU to plain SwiGLU
    y1, _, h1 = oracle.grouped_mlp_forward(xp, inp.w1, inp.w2, m["offsets"], np.ones_like(pp))
    np.testing.assert_allclose(h, h1 * pp[:, None], rtol=1e-13, atol=1e-16)


# ---------------------------------------------------------------------------
# backward
# ---------------------------------------------------------------------------

def _loss(inp, w1, w2, p, idx, dout, x=None):
    x = inp.x if x is None else x
    return float((oracle.moe_ffn_forward(x, w1, w2, idx, p) * dout).sum())


def test_backward_finite_differences():
    inp = _tiny(T=12, H=6, I=5, E=4, k=2, seed=12)
    idx, p = oracle.route_topk(inp.logits, 2)
    dout = np.random.default_rng(2).standard_normal(inp.x.shape)
    w1 = inp.w1.astype(np.float64) * 20     # larger weights: curvature of silu matters
    w2 = inp.w2.astype(np.float64) * 20
    x = inp.x.astype(np.float64)
    g = oracle.moe_ffn_backward(x, w1, w2, idx, p, dout)
    eps = 1e-6
    rng = np.random.default_rng(3)

    def fd(arr, name):
        for _ in range(6):
            pos = tuple(rng.integers(0, s) for s in arr.shape)
            old = arr[pos]
            arr[pos] = old + eps
            lp = _loss(inp, w1, w2, p, idx, dout, x)
            arr[pos] = old - eps
            lm = _loss(inp, w1, w2, p, idx, dout, x)
            arr[pos] = old
            num = (lp - lm) / (2 * eps)
            assert g[name][pos] == pytest.approx(num, rel=1e-6, abs=1e-9), (name, pos)

    fd(x, "dx")
    fd(w1, "dw_gate_up")
    fd(w2, "dw_down")
    fd(p, "drouting_weights")


def test_backward_matches_torch_autograd():
    inp = _tiny(T=40, H=12, I=10, E=5, k=2, seed=13)
    idx, p = oracle.route_topk(inp.logits, 2)
    dout = np.random.default_rng(4).standard_normal(inp.x.shape)
    g = oracle.moe_ffn_backward(inp.x, inp.w1, inp.w2, idx, p, dout)

    X = torch.from_numpy(inp.x.astype(np.float64)).requires_grad_()
    W1 = torch.from_numpy(inp.w1.astype(np.float64)).requires_grad_()
    W2 = torch.from_numpy(inp.w2.astype(np.float64)).requires_grad_()
    P = torch.from_numpy(p.copy()).requires_grad_()
    I = inp.w1.shape[1] // 2
    out = torch.zeros_like(X)
    for t in range(X.shape[0]):
        for j in range(2):
            e = int(idx[t, j])
            hid = F.silu(W1[e, :I] @ X[t]) * (W1[e, I:] @ X[t])
            out = out.index_add(0, torch.tensor([t]), (P[t, j] * (W2[e] @ hid))[None])
    (out * torch.from_numpy(dout)).sum().backward()
    np.testing.assert_allclose(g["dx"], X.grad.numpy(), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(g["dw_gate_up"], W1.grad.numpy(), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(g["dw_down"], W2.grad.numpy(), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(g["drouting_weights"], P.grad.numpy(), rtol=1e-10, atol=1e-13)


def test_backward_linearity_identities_and_idle_experts():
    inp = _tiny(T=64, H=16, I=20, E=8, k=2, seed=14)
    logits = inp.logits.copy()
    logits[:, 6:] -= 50.0                    # experts 6 and 7 never chosen
    idx, p = oracle.route_topk(logits, 2)
    dout = np.random.default_rng(5).standard_normal(inp.x.shape)
    out = oracle.moe_ffn_forward(inp.x, inp.w1, inp.w2, idx, p)
    g = oracle.moe_ffn_backward(inp.x, inp.w1, inp.w2, idx, p, dout)
    ref = float((dout * out).sum())
    # out is linear in p and in W2, so <grad, value> = <dout, out> for each
    assert float((g["drouting_weights"] * p).sum()) == pytest.approx(ref, rel=1e-11)
    assert float((g["dw_down"] * inp.w2).sum()) == pytest.approx(ref, rel=1e-11)
    assert not g["dw_gate_up"][6:].any() and not g["dw_down"][6:].any()


def test_grouped_backward_equals_loop_backward():
    inp = _tiny(T=50, H=16, I=12, E=6, k=3, seed=15, zipf=1.2)
    T, k, E = 50, 3, 6
    idx, p = oracle.route_topk(inp.logits, k)
    dout = np.random.default_rng(6).standard_normal(inp.x.shape)
    m = oracle.permute(idx, E)
    xp = oracle.gather_rows(inp.x, m["src_token"])
    pp = p.ravel()[m["src_token"] * k + m["src_slot"]]
    dyp = oracle.gather_rows(dout, m["src_token"])        # combine's gradient gathers
    gb = oracle.grouped_mlp_backward(dyp, xp, inp.w1, inp.w2, m["offsets"], pp)
    gl = oracle.moe_ffn_backward(inp.x, inp.w1, inp.w2, idx, p, dout)
    dx = oracle.unpermute_combine(gb["dx_perm"], m["row_id_map"], T, k)
    np.testing.assert_allclose(dx, gl["dx"], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(gb["dw_gate_up"], gl["dw_gate_up"], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(gb["dw_down"], gl["dw_down"], rtol=1e-11, atol=1e-13)
    dp = gb["dprob_perm"][m["row_id_map"]].reshape(T, k)
    np.testing.assert_allclose(dp, gl["drouting_weights"], rtol=1e-11, atol=1e-13)


def test_grouped_linear_brute_force_and_down_projection():
    """GroupedLinear: a triple loop on a tiny ragged case with an empty expert, and
    the down projection inside the grouped MLP (y = h W2^T per expert)."""
    rng = np.random.default_rng(7)
    E, N, K = 3, 5, 4
    sizes = [2, 0, 3]
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    x = rng.standard_normal((off[-1], K))
    w = rng.standard_normal((E, N, K))
    y = oracle.grouped_linear(x, w, off)
    for e in range(E):
        for r in range(off[e], off[e + 1]):
            for n in range(N):
                acc = 0.0
                for kk in range(K):
                    acc += x[r, kk] * w[e, n, kk]
                assert abs(y[r, n] - acc) <= 1e-12 * max(1.0, abs(acc))
    inp = _tiny()
    idx, p = oracle.route_topk(inp.logits, 2)
    m = oracle.permute(idx, 6)
    pp = p.ravel()[m["src_token"] * 2 + m["src_slot"]]
    yf, z, h = oracle.grouped_mlp_forward(inp.x[m["src_token"]], inp.w1, inp.w2, m["offsets"], pp)
    assert np.allclose(oracle.grouped_linear(h, inp.w2, m["offsets"]), yf, rtol=0, atol=1e-12)
    # the gate_up projection is GroupedLinear with the [2I, H] weight
    assert np.allclose(oracle.grouped_linear(inp.x[m["src_token"]], inp.w1, m["offsets"]), z, rtol=0, atol=1e-12)
