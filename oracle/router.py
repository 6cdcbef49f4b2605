"""Router gate linear and the backward of top-k gating (test infrastructure only).

The pages never show the router. Reading (the same as the forward gating's): the
gate is a bias-free linear map hidden -> E applied to each token, logits[t, e] =
sum_h x[t, h] * w_router[e, h] (the [out, in] weight layout of the pages'
GroupedLinear weights), followed by the top-k gating of ``route_topk``. Its
backward is the chain rule through that gating: the selection itself is piecewise
constant in the logits, so only the probabilities carry a gradient.

All arithmetic is float64; inputs are upcast exactly.
"""
from __future__ import annotations

import numpy as np

__all__ = ["router_logits", "route_topk_backward", "router_backward"]

f64 = np.float64


def router_logits(x, w_router):
    """logits [T, E] = x [T, H] times w_router [E, H] transposed."""
    return np.asarray(x, f64) @ np.asarray(w_router, f64).T


def _softmax_rows(a):
    a = np.asarray(a, f64)
    z = np.exp(a - a.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def route_topk_backward(logits, topk_idx, d_topk_prob, renormalize: bool = True):
    """d_logits [T, E] from the gradient d_topk_prob [T, k] of route_topk's output.

    With ``renormalize`` the k probabilities are a softmax over the k chosen logits,
    p_j = exp(l_{i_j}) / sum_j' exp(l_{i_j'}), so d l_{i_j} = p_j * (g_j - sum_j' p_j' g_j')
    and the other experts get zero. Otherwise p_j = P[i_j] with P the softmax over all
    E logits, and d l_e = P_e * (G_e - sum_j P[i_j] g_j), G_e = g_j where e = i_j and 0
    elsewhere.
    """
    l = np.asarray(logits, f64)
    idx = np.asarray(topk_idx)
    g = np.asarray(d_topk_prob, f64)
    T, E = l.shape
    d = np.zeros((T, E), f64)
    for t in range(T):
        sel = l[t, idx[t]]
        if renormalize:
            p = np.exp(sel - sel.max())
            p /= p.sum()
            s = float(np.dot(p, g[t]))
            for j, e in enumerate(idx[t]):
                d[t, e] = p[j] * (g[t, j] - s)
        else:
            P = _softmax_rows(l[t:t + 1])[0]
            G = np.zeros(E, f64)
            for j, e in enumerate(idx[t]):
                G[e] = g[t, j]
            s = float(np.dot(P[idx[t]], g[t]))
            d[t] = P * (G - s)
    return d


def router_backward(x, w_router, d_logits):
    """(dx [T, H], dw_router [E, H]) of logits = x w_router^T: dx = d_logits w_router,
    dw_router = d_logits^T x."""
    dl = np.asarray(d_logits, f64)
    return dl @ np.asarray(w_router, f64), dl.T @ np.asarray(x, f64)
