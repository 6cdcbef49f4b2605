"""Pins for the oracle's router gate linear and top-k gating backward (CPU only).

Each check ties the oracle to something other than its own formula: central finite
differences of the forward gating, brute-force loops, and invariants of a softmax
gradient.
"""
import numpy as np
import pytest

import oracle


def _fd_grad(f, a, eps=1e-6):
    """Central differences of the scalar f at every entry of a (float64)."""
    a = np.array(a, np.float64)
    g = np.zeros_like(a)
    it = np.nditer(a, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        ap, am = a.copy(), a.copy()
        ap[i] += eps
        am[i] -= eps
        g[i] = (f(ap) - f(am)) / (2 * eps)
    return g


@pytest.mark.parametrize("renorm", [True, False])
@pytest.mark.parametrize("E,k", [(8, 2), (6, 6), (16, 5), (5, 1)])
def test_route_backward_matches_finite_differences(E, k, renorm):
    rng = np.random.default_rng(E * 10 + k)
    T = 7
    logits = rng.standard_normal((T, E)) * 2.0   # distinct logits: the chosen set is stable under eps
    g = rng.standard_normal((T, k))
    idx, _ = oracle.route_topk(logits, k, renorm)

    def loss(l):
        i2, p = oracle.route_topk(l, k, renorm)
        assert np.array_equal(i2, idx)   # the selection did not move
        return float((p * g).sum())

    fd = _fd_grad(loss, logits)
    d = oracle.route_topk_backward(logits, idx, g, renorm)
    np.testing.assert_allclose(d, fd, rtol=1e-6, atol=1e-8)


@pytest.mark.parametrize("renorm", [True, False])
def test_route_backward_invariants(renorm):
    rng = np.random.default_rng(3)
    T, E, k = 50, 12, 3
    logits = rng.standard_normal((T, E))
    g = rng.standard_normal((T, k))
    idx, p = oracle.route_topk(logits, k, renorm)
    d = oracle.route_topk_backward(logits, idx, g, renorm)
    # adding a constant to a row of logits changes no probability: rows sum to zero
    np.testing.assert_allclose(d.sum(axis=1), 0.0, atol=1e-12)
    if renorm:
        # experts that were not chosen get no gradient
        mask = np.zeros((T, E), bool)
        np.put_along_axis(mask, idx, True, axis=1)
        assert np.all(d[~mask] == 0.0)
    # an upstream gradient equal for every slot moves nothing when the k probabilities
    # sum to one (renormalised)
    if renorm:
        d1 = oracle.route_topk_backward(logits, idx, np.ones((T, k)), True)
        np.testing.assert_allclose(d1, 0.0, atol=1e-12)


def test_route_backward_k_equals_e_is_the_softmax_jacobian():
    # k = E: both modes are the full softmax; its Jacobian is diag(P) - P P^T
    rng = np.random.default_rng(4)
    T, E = 5, 6
    logits = rng.standard_normal((T, E))
    g = rng.standard_normal((T, E))
    for renorm in (True, False):
        idx, p = oracle.route_topk(logits, E, renorm)
        d = oracle.route_topk_backward(logits, idx, g, renorm)
        for t in range(T):
            P = np.exp(logits[t] - logits[t].max())
            P /= P.sum()
            J = np.diag(P) - np.outer(P, P)
            G = np.zeros(E)
            G[idx[t]] = g[t]
            np.testing.assert_allclose(d[t], J @ G, rtol=1e-12, atol=1e-14)


def test_router_logits_brute_force():
    rng = np.random.default_rng(5)
    T, H, E = 4, 9, 3
    x = rng.standard_normal((T, H))
    w = rng.standard_normal((E, H))
    ref = np.zeros((T, E))
    for t in range(T):
        for e in range(E):
            for h in range(H):
                ref[t, e] += x[t, h] * w[e, h]
    np.testing.assert_allclose(oracle.router_logits(x, w), ref, rtol=1e-13)


def test_router_backward_brute_force_and_finite_differences():
    rng = np.random.default_rng(6)
    T, H, E = 5, 7, 4
    x = rng.standard_normal((T, H))
    w = rng.standard_normal((E, H))
    G = rng.standard_normal((T, E))
    dx, dw = oracle.router_backward(x, w, G)
    bx = np.zeros((T, H))
    bw = np.zeros((E, H))
    for t in range(T):
        for e in range(E):
            for h in range(H):
                bx[t, h] += G[t, e] * w[e, h]
                bw[e, h] += G[t, e] * x[t, h]
    np.testing.assert_allclose(dx, bx, rtol=1e-12)
    np.testing.assert_allclose(dw, bw, rtol=1e-12)
    # the loss sum(logits * G) is linear: central differences are exact up to rounding
    fx = _fd_grad(lambda a: float((oracle.router_logits(a, w) * G).sum()), x, eps=1e-3)
    fw = _fd_grad(lambda a: float((oracle.router_logits(x, a) * G).sum()), w, eps=1e-3)
    np.testing.assert_allclose(dx, fx, rtol=1e-8, atol=1e-10)
    np.testing.assert_allclose(dw, fw, rtol=1e-8, atol=1e-10)
