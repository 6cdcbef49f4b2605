"""Plain CPU reference for the MoE expert feed-forward layer (test infrastructure only).

Source: "Efficient MoE Training for Biological Foundation Models"
  * Challenge 1 (Fragmented expert kernels): the naive baseline visits the experts
    one after another; each expert takes the (token, slot) pairs the router sent to
    it, runs its MLP on those tokens, scales each result by the pair's routing
    weight and adds it into the token's output. GroupedLinear instead takes
    per-expert token counts (split_sizes), and each expert's gate_up weight is
    [2 * intermediate, hidden].
  * Challenge 3: ScaledSwiGLU multiplies the routing probability into the
    SwiGLU output, and the grouped MLP is GroupedLinear(gate_up) ->
    ScaledSwiGLU -> GroupedLinear(down), with a matching backward.

Readings where the pages are silent (each is listed with its reason in the
design notes):
  * routing: softmax over the experts, keep the k largest, renormalise the k
    kept probabilities to sum to 1; selection compares the logits, larger
    first, lower expert index first on equal logits;
  * rows of an expert are ordered by ascending token (the order the loop
    visits them when the routing mask is laid out [token, slot]);
  * gate is rows [0, I) of the gate_up weight, up is rows [I, 2I);
    SwiGLU(g, u) = silu(g) * u with silu(g) = g / (1 + exp(-g)); no biases;
  * the probability is applied once: after the expert here (as the loop does),
    inside ScaledSwiGLU in the grouped form; both are equal in exact arithmetic.

All arithmetic is float64; inputs are upcast exactly.
"""
from __future__ import annotations

import numpy as np

from .fp8_tensor import bf16_round, fp8_tensor_qdq
from .mxfp8 import mxfp8_qdq

__all__ = [
    "route_topk", "permute", "silu", "expert_ffn", "moe_ffn_forward",
    "grouped_mlp_forward",
    "grouped_linear", "grouped_mlp_forward_mxfp8", "unpermute_combine",
    "grouped_mlp_backward", "moe_ffn_backward", "gather_rows", "grouped_mlp_backward_mxfp8",
    "grouped_mlp_backward_fp8_tensor",
]

f64 = np.float64


def silu(g):
    return g / (1.0 + np.exp(-g))


def _sigmoid(g):
    return 1.0 / (1.0 + np.exp(-g))


# ---------------------------------------------------------------------------
# Router gating: routing_weights [T, k] and the chosen experts [T, k]
# ---------------------------------------------------------------------------

def route_topk(logits, k: int, renormalize: bool = True):
    """Top-k router gating.

    Returns (topk_idx int32 [T, k], topk_prob float64 [T, k]). Slot j holds the
    j-th largest logit (ties: lower expert index first). With ``renormalize``
    the k probabilities are the softmax restricted to the chosen experts;
    otherwise they are the full softmax's entries for those experts.
    """
    l = np.asarray(logits, dtype=f64)
    T, E = l.shape
    assert 1 <= k <= E
    # a stable sort of the negated logits keeps equal logits in index order
    order = np.argsort(-l, axis=1, kind="stable")[:, :k]
    sel = np.take_along_axis(l, order, axis=1)
    m = sel[:, :1]                                    # the largest logit of the row
    num = np.exp(sel - m)
    if renormalize:
        den = num.sum(axis=1, keepdims=True)
    else:
        den = np.exp(l - m).sum(axis=1, keepdims=True)
    return order.astype(np.int32), num / den


# ---------------------------------------------------------------------------
# Token permutation into per-expert groups (split_sizes)
# ---------------------------------------------------------------------------

def permute(topk_idx, E: int):
    """Group the T*k (token, slot) pairs by expert.

    Expert e's pairs are listed in ascending token order (the order a row-major scan
    of the [T, k] choice table meets them); the lists of experts 0..E-1 are laid end
    to end. Returns dict with
      split_sizes [E], offsets [E+1], row_id_map [T*k] ((t, j) -> row; -1 for a pair
      that names no expert in [0, E)), src_token [T*k] (row -> t), src_slot [T*k]
      (row -> j); only the first offsets[E] entries of the last two are filled.
    """
    choice = np.asarray(topk_idx)
    T, k = choice.shape
    split_sizes = np.zeros(E, np.int64)
    row_id_map = np.full(T * k, -1, np.int64)
    src_token = np.empty(T * k, np.int64)
    src_slot = np.empty(T * k, np.int64)
    next_row = 0
    for e in range(E):
        tok, slot = np.nonzero(choice == e)          # row-major: ascending token
        rows = next_row + np.arange(tok.size)
        split_sizes[e] = tok.size
        row_id_map[tok * k + slot] = rows
        src_token[rows] = tok
        src_slot[rows] = slot
        next_row += tok.size
    offsets = np.concatenate([[0], np.cumsum(split_sizes)])
    return dict(split_sizes=split_sizes, offsets=offsets, row_id_map=row_id_map,
                src_token=src_token, src_slot=src_slot)


def gather_rows(x, src_token):
    """x_perm[r] = x[src_token[r]]."""
    return np.asarray(x)[np.asarray(src_token)]


# ---------------------------------------------------------------------------
# The expert MLP and the per-expert loop
# ---------------------------------------------------------------------------

def expert_ffn(X, w_gate_up, w_down):
    """One expert: Z = X W1^T, A = silu(Z[:, :I]) * Z[:, I:], Y = A W2^T.
    Returns (Y, Z, A), all float64."""
    X = np.asarray(X, dtype=f64)
    W1 = np.asarray(w_gate_up, dtype=f64)
    W2 = np.asarray(w_down, dtype=f64)
    I = W1.shape[0] // 2
    Z = X @ W1.T
    A = silu(Z[:, :I]) * Z[:, I:]
    return A @ W2.T, Z, A


def moe_ffn_forward(x, w_gate_up, w_down, topk_idx, topk_prob):
    """Layer output [T, H] by the naive per-expert loop (float64).

    For each expert in turn: the tokens that chose it, their expert MLP output, each
    weighted by the probability of the slot that chose the expert, accumulated into
    those tokens' outputs. w_gate_up [E, 2I, H], w_down [E, H, I]."""
    x = np.asarray(x, dtype=f64)
    choice = np.asarray(topk_idx)
    prob = np.asarray(topk_prob, dtype=f64)
    T, H = x.shape
    out = np.zeros((T, H), f64)
    for e in range(w_gate_up.shape[0]):
        tok, slot = np.nonzero(choice == e)
        if tok.size:
            y_e, _, _ = expert_ffn(x[tok], w_gate_up[e], w_down[e])
            np.add.at(out, tok, prob[tok, slot][:, None] * y_e)
    return out


def grouped_mlp_forward(x_perm, w_gate_up, w_down, offsets, prob_perm):
    """The grouped form on permuted rows: for expert e, rows
    [offsets[e], offsets[e+1]) go through gate_up, ScaledSwiGLU (probability
    folded in) and down.

    Returns (y_perm [R, H], z [R, 2I], h [R, I]) in float64, where
    h = silu(gate) * up * prob and y_perm = h W2^T.
    """
    x = np.asarray(x_perm, dtype=f64)
    p = np.asarray(prob_perm, dtype=f64)
    off = np.asarray(offsets, dtype=np.int64)
    E, twoI, H = w_gate_up.shape
    I = twoI // 2
    R = x.shape[0]
    y = np.zeros((R, H), f64)
    z = np.zeros((R, twoI), f64)
    h = np.zeros((R, I), f64)
    for e in range(E):
        a, b = int(off[e]), int(off[e + 1])
        if a == b:
            continue
        W1 = np.asarray(w_gate_up[e], dtype=f64)
        W2 = np.asarray(w_down[e], dtype=f64)
        Z = x[a:b] @ W1.T
        Hs = silu(Z[:, :I]) * Z[:, I:] * p[a:b, None]
        y[a:b] = Hs @ W2.T
        z[a:b] = Z
        h[a:b] = Hs
    return y, z, h


def grouped_linear(x_perm, w, offsets):
    """GroupedLinear (Challenge 1): for expert e, y[r] = x[r] W_e^T for the rows
    r in [offsets[e], offsets[e+1]); one weight [N, K] per expert. float64."""
    x = np.asarray(x_perm, dtype=f64)
    off = np.asarray(offsets, dtype=np.int64)
    E, N, K = w.shape
    y = np.zeros((x.shape[0], N), f64)
    for e in range(E):
        a, b = int(off[e]), int(off[e + 1])
        if a < b:
            y[a:b] = x[a:b] @ np.asarray(w[e], dtype=f64).T
    return y


def grouped_mlp_forward_mxfp8(x_perm, w_gate_up, w_down, offsets, prob_perm, return_z=False):
    """Grouped MLP with the naive quantise -> dequantise steps of Challenge 3
    around both GEMMs: x (along H), W1 (along H), h (along I) and W2 (along I)
    each pass through MXFP8 before their GEMM; gate_up accumulators stay
    unrounded. Returns (y_perm, h_before_quantisation) in float64, and the
    gate_up product z [R, 2I] as a third value with return_z."""
    x = mxfp8_qdq(np.asarray(x_perm, dtype=f64)) if len(x_perm) else np.zeros((0, w_gate_up.shape[2]))
    p = np.asarray(prob_perm, dtype=f64)
    off = np.asarray(offsets, dtype=np.int64)
    E, twoI, H = w_gate_up.shape
    I = twoI // 2
    R = x.shape[0]
    y = np.zeros((R, H), f64)
    h = np.zeros((R, I), f64)
    z = np.zeros((R, 2 * I), f64)
    for e in range(E):
        a, b = int(off[e]), int(off[e + 1])
        if a == b:
            continue
        W1 = mxfp8_qdq(np.asarray(w_gate_up[e], dtype=f64))
        W2 = mxfp8_qdq(np.asarray(w_down[e], dtype=f64))
        Z = x[a:b] @ W1.T
        z[a:b] = Z
        Hs = silu(Z[:, :I]) * Z[:, I:] * p[a:b, None]
        h[a:b] = Hs
        y[a:b] = mxfp8_qdq(Hs) @ W2.T
    return (y, h, z) if return_z else (y, h)


def unpermute_combine(y_perm, row_id_map, T: int, k: int, weights=None):
    """out[t] = sum over slots j (ascending) of w[t, j] * y_perm[row_id_map[t*k + j]];
    w = 1 when the probability was already folded in (weights=None)."""
    y = np.asarray(y_perm, dtype=f64)
    rmap = np.asarray(row_id_map).reshape(T, k)
    out = np.zeros((T, y.shape[1]), f64)
    for j in range(k):
        contrib = y[rmap[:, j]]
        if weights is not None:
            contrib = contrib * np.asarray(weights, dtype=f64).reshape(T, k)[:, j:j + 1]
        out += contrib
    return out


# ---------------------------------------------------------------------------
# Backward (the "matching fused backward" of Challenge 3, as explicit formulas)
# ---------------------------------------------------------------------------

def grouped_mlp_backward(dy_perm, x_perm, w_gate_up, w_down, offsets, prob_perm):
    """Gradients of y_perm = (silu(G) * U * p) W2^T with (G, U) = x W1^T, per expert.

    dy_perm [R, H] is the upstream gradient on the permuted rows. Returns dict
    dx_perm [R, H], dw_gate_up [E, 2I, H], dw_down [E, H, I], dprob_perm [R].
    Experts with no rows get exactly zero weight gradients.
    """
    dy = np.asarray(dy_perm, dtype=f64)
    x = np.asarray(x_perm, dtype=f64)
    p = np.asarray(prob_perm, dtype=f64)
    off = np.asarray(offsets, dtype=np.int64)
    E, twoI, H = w_gate_up.shape
    I = twoI // 2
    R = x.shape[0]
    dx = np.zeros((R, H), f64)
    dw1 = np.zeros((E, twoI, H), f64)
    dw2 = np.zeros((E, H, I), f64)
    dprob = np.zeros(R, f64)
    for e in range(E):
        a, b = int(off[e]), int(off[e + 1])
        if a == b:
            continue
        W1 = np.asarray(w_gate_up[e], dtype=f64)
        W2 = np.asarray(w_down[e], dtype=f64)
        X, dY, pe = x[a:b], dy[a:b], p[a:b, None]
        Z = X @ W1.T
        G, U = Z[:, :I], Z[:, I:]
        sg = _sigmoid(G)
        A = G * sg * U                      # SwiGLU before the probability
        Hs = A * pe
        dw2[e] = dY.T @ Hs
        dHs = dY @ W2
        dprob[a:b] = (dHs * A).sum(axis=1)
        dA = dHs * pe
        dG = dA * U * sg * (1.0 + G * (1.0 - sg))
        dU = dA * G * sg
        dZ = np.concatenate([dG, dU], axis=1)
        dx[a:b] = dZ @ W1
        dw1[e] = dZ.T @ X
    return dict(dx_perm=dx, dw_gate_up=dw1, dw_down=dw2, dprob_perm=dprob)


def moe_ffn_backward(x, w_gate_up, w_down, topk_idx, topk_prob, d_out):
    """Gradients of moe_ffn_forward's output against d_out, by the same per-expert loop
    run backwards. Returns dict dx [T, H], dw_gate_up, dw_down, drouting_weights [T, k]
    (gradient w.r.t. the routing probabilities themselves)."""
    x = np.asarray(x, dtype=f64)
    choice = np.asarray(topk_idx)
    prob = np.asarray(topk_prob, dtype=f64)
    g = np.asarray(d_out, dtype=f64)
    E, twoI, H = w_gate_up.shape
    I = twoI // 2
    dx = np.zeros_like(x)
    dw1 = np.zeros((E, twoI, H), f64)
    dw2 = np.zeros((E, H, I), f64)
    dprob = np.zeros_like(prob)
    for e in range(E):
        tok, slot = np.nonzero(choice == e)
        if tok.size == 0:
            continue
        W1 = np.asarray(w_gate_up[e], dtype=f64)
        W2 = np.asarray(w_down[e], dtype=f64)
        y_e, Z, A = expert_ffn(x[tok], W1, W2)
        g_e = g[tok]                                 # the forward accumulated into these tokens
        dprob[tok, slot] = (g_e * y_e).sum(axis=1)
        dY = g_e * prob[tok, slot][:, None]
        dw2[e] = dY.T @ A
        dA = dY @ W2
        G, U = Z[:, :I], Z[:, I:]
        sg = _sigmoid(G)
        dZ = np.concatenate([dA * U * sg * (1.0 + G * (1.0 - sg)), dA * G * sg], axis=1)
        np.add.at(dx, tok, dZ @ W1)
        dw1[e] = dZ.T @ x[tok]
    return dict(dx=dx, dw_gate_up=dw1, dw_down=dw2, drouting_weights=dprob)


def _qdq_rows_per_expert(x, a, b):
    """x[a:b] quantised through MXFP8 along the token axis: 32-row blocks starting at the
    expert's first row, the last block zero-padded (padding rows do not change a block's
    maximum and are dropped again)."""
    seg = np.asarray(x, dtype=f64)[a:b]
    m = b - a
    padded = np.zeros((-(-m // 32) * 32, seg.shape[1]), f64)
    padded[:m] = seg
    return mxfp8_qdq(padded.T).T[:m]


def grouped_mlp_backward_mxfp8(dy_perm, x_perm, z_save, h_save, w_gate_up, w_down, offsets, prob_perm,
                               quantize=True, round_bf16=True):
    """The grouped MLP backward with every GEMM operand passed through MXFP8 along that
    GEMM's own reduction (K) axis (Challenge 2's 32-value blocks; Challenge 3 puts the
    backward GEMMs in MXFP8 as it does the forward ones):

      dH     = Q_H(dY) Q_H(W2_e)                      (K = H: dY along its rows' H, W2 along H)
      dprob, dA, dG, dU from dH, the saved z = [G, U] and prob, as in grouped_mlp_backward
      dx     = Q_2I(dZ) Q_2I(W1_e)                    (K = 2I)
      dW2_e  = Q_tok(dY_e)^T Q_tok(h_e)               (K = the expert's rows)
      dW1_e  = Q_tok(dZ_e)^T Q_tok(x_e)

    Q_tok blocks start at each expert's first row (the padded layout of
    mxfp8_quantize_colwise). The recipe of Challenge 3 converts a low-precision GEMM's
    result back to bf16 and keeps activations (and so their gradients) in bf16: dH and
    dZ are rounded to bf16 (nearest, ties to even) before they are used. z_save [R, 2I]
    and h_save [R, I] are the forward's saved tensors, taken as given. quantize=False
    drops every Q and both roundings and gives the bf16 backward's formulas evaluated on
    the saved z and h; round_bf16=False keeps every Q but drops the two bf16 roundings
    (dH and dZ enter dprob, dSwiGLU and their quantisers unrounded)."""
    q = mxfp8_qdq if quantize else (lambda t: np.asarray(t, dtype=f64))
    rnd = bf16_round if (quantize and round_bf16) else (lambda t: t)
    qt = _qdq_rows_per_expert if quantize else (lambda t, a, b: np.asarray(t, dtype=f64)[a:b])
    dy = np.asarray(dy_perm, dtype=f64)
    x = np.asarray(x_perm, dtype=f64)
    z = np.asarray(z_save, dtype=f64)
    h = np.asarray(h_save, dtype=f64)
    p = np.asarray(prob_perm, dtype=f64)
    off = np.asarray(offsets, dtype=np.int64)
    E, twoI, H = w_gate_up.shape
    I = twoI // 2
    R = x.shape[0]
    dx = np.zeros((R, H), f64)
    dw1 = np.zeros((E, twoI, H), f64)
    dw2 = np.zeros((E, H, I), f64)
    dprob = np.zeros(R, f64)
    dyq = q(dy) if R else dy
    for e in range(E):
        a, b = int(off[e]), int(off[e + 1])
        if a == b:
            continue
        W1 = np.asarray(w_gate_up[e], dtype=f64)
        W2 = np.asarray(w_down[e], dtype=f64)
        G, U = z[a:b, :I], z[a:b, I:]
        sg = _sigmoid(G)
        A = G * sg * U
        pe = p[a:b, None]
        dHs = rnd(dyq[a:b] @ q(W2.T).T)
        dprob[a:b] = (dHs * A).sum(axis=1)
        dA = dHs * pe
        dZ = rnd(np.concatenate([dA * U * sg * (1.0 + G * (1.0 - sg)), dA * G * sg], axis=1))
        dx[a:b] = q(dZ) @ q(W1.T).T
        dw2[e] = qt(dy, a, b).T @ qt(h, a, b)
        dw1[e] = qt(dZ, 0, b - a).T @ qt(x, a, b)
    return dict(dx_perm=dx, dw_gate_up=dw1, dw_down=dw2, dprob_perm=dprob)


def grouped_mlp_backward_fp8_tensor(dy_perm, x_perm, z_save, h_save, w_gate_up, w_down, offsets, prob_perm,
                                    quantize=True, round_bf16=True):
    """The grouped MLP backward with every GEMM operand quantised per tensor (Challenge
    2's FP8: one scaling factor for a whole tensor; the factor is amax / 448 as in
    fp8_tensor_quantize). The tensors are those of the forward: dY, dZ, h and x each over
    all routed rows, W1_e and W2_e each per expert.

      dH_e  = Q(dY)_e Q(W2_e)
      dprob, dA, dG, dU from dH, the saved z = [G, U] and prob, as in grouped_mlp_backward
      dx_e  = Q(dZ)_e Q(W1_e)
      dW2_e = Q(dY)_e^T Q(h)_e
      dW1_e = Q(dZ)_e^T Q(x)_e

    One factor per tensor does not depend on the axis a GEMM reduces over, so each
    tensor is quantised once and serves both GEMMs it enters; dZ's factor needs every
    expert's dZ first. As in the MXFP8 backward, dH and dZ are rounded to bf16 (the
    recipe keeps activations and their gradients in bf16) unless round_bf16 is False.
    z_save [R, 2I] and h_save [R, I] are the forward's saved tensors, taken as given.
    quantize=False drops every Q and both roundings. Also returns dz_perm, the dZ that
    was quantised (bf16-rounded when round_bf16)."""
    q = fp8_tensor_qdq if quantize else (lambda t: np.asarray(t, dtype=f64))
    rnd = bf16_round if (quantize and round_bf16) else (lambda t: t)
    dy = np.asarray(dy_perm, dtype=f64)
    x = np.asarray(x_perm, dtype=f64)
    z = np.asarray(z_save, dtype=f64)
    h = np.asarray(h_save, dtype=f64)
    p = np.asarray(prob_perm, dtype=f64)
    off = np.asarray(offsets, dtype=np.int64)
    E, twoI, H = w_gate_up.shape
    I = twoI // 2
    R = x.shape[0]
    dx = np.zeros((R, H), f64)
    dw1 = np.zeros((E, twoI, H), f64)
    dw2 = np.zeros((E, H, I), f64)
    dprob = np.zeros(R, f64)
    dz = np.zeros((R, twoI), f64)
    if R == 0:
        return dict(dx_perm=dx, dw_gate_up=dw1, dw_down=dw2, dprob_perm=dprob, dz_perm=dz)
    dyq, hq, xq = q(dy), q(h), q(x)
    for e in range(E):           # dH, dprob, dZ; the down weight gradient
        a, b = int(off[e]), int(off[e + 1])
        if a == b:
            continue
        W2 = q(np.asarray(w_down[e], dtype=f64))
        G, U = z[a:b, :I], z[a:b, I:]
        sg = _sigmoid(G)
        A = G * sg * U
        dHs = rnd(dyq[a:b] @ W2)
        dprob[a:b] = (dHs * A).sum(axis=1)
        dA = dHs * p[a:b, None]
        dz[a:b] = rnd(np.concatenate([dA * U * sg * (1.0 + G * (1.0 - sg)), dA * G * sg], axis=1))
        dw2[e] = dyq[a:b].T @ hq[a:b]
    dzq = q(dz)                   # one factor over every expert's rows
    for e in range(E):           # dx and the gate_up weight gradient
        a, b = int(off[e]), int(off[e + 1])
        if a == b:
            continue
        W1 = q(np.asarray(w_gate_up[e], dtype=f64))
        dx[a:b] = dzq[a:b] @ W1
        dw1[e] = dzq[a:b].T @ xq[a:b]
    return dict(dx_perm=dx, dw_gate_up=dw1, dw_down=dw2, dprob_perm=dprob, dz_perm=dz)
