"""Pins for the oracle's router gating, permutation and combine (CPU only).

Each check ties the oracle to something other than itself: hand-worked
values, a brute-force selection loop, a library sort, or invariants.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special

import oracle
from moe_inputs import WORKLOADS, make_inputs, scaled

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _brute_topk(row, k):
    """Pick the largest remaining logit k times; on equal logits the lower index wins."""
    chosen = []
    for _ in range(k):
        best = None
        for e, v in enumerate(row):
            if e in chosen:
                continue
            if best is None or v > row[best]:
                best = e
        chosen.append(best)
    return chosen


def test_route_golden():
    g = json.load(open(os.path.join(GOLDEN, "route_permute_worked.json")))
    for case in g["route"]:
        idx, p = oracle.route_topk(np.array(case["logits"], np.float32), case["k"])
        assert idx.tolist() == case["topk_idx"], case["comment"]
        np.testing.assert_allclose(p, case["topk_prob"], rtol=1e-6)


def test_route_brute_force_selection():
    rng = np.random.default_rng(11)
    for E, k in [(8, 2), (16, 5), (128, 8), (5, 5)]:
        logits = rng.standard_normal((40, E)).astype(np.float32)
        logits[::7, 1] = logits[::7, 3]             # exact ties
        logits[::5, :] = np.round(logits[::5, :])   # many ties
        idx, p = oracle.route_topk(logits, k)
        for t in range(logits.shape[0]):
            assert idx[t].tolist() == _brute_topk(logits[t].tolist(), k)
        # renormalised weights: sum to one, descending, ratios are exp of logit gaps
        np.testing.assert_allclose(p.sum(1), 1.0, rtol=0, atol=1e-12)
        assert (np.diff(p, axis=1) <= 0).all()
        sel = np.take_along_axis(logits.astype(np.float64), idx.astype(np.int64), 1)
        np.testing.assert_allclose(p[:, 1:] / p[:, :1], np.exp(sel[:, 1:] - sel[:, :1]), rtol=1e-12)


def test_route_k_equals_E_is_full_softmax():
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((30, 8)).astype(np.float32)
    idx, p = oracle.route_topk(logits, 8)
    full = scipy.special.softmax(logits.astype(np.float64), axis=1)
    np.testing.assert_allclose(np.take_along_axis(full, idx.astype(np.int64), 1), p, rtol=1e-12)


def test_route_without_renormalisation_is_softmax_entries():
    rng = np.random.default_rng(4)
    logits = rng.standard_normal((30, 16)).astype(np.float32)
    idx, p = oracle.route_topk(logits, 3, renormalize=False)
    full = scipy.special.softmax(logits.astype(np.float64), axis=1)
    np.testing.assert_allclose(np.take_along_axis(full, idx.astype(np.int64), 1), p, rtol=1e-12)
    # renormalising the kept entries gives the default weights
    _, pr = oracle.route_topk(logits, 3)
    np.testing.assert_allclose(p / p.sum(1, keepdims=True), pr, rtol=1e-12)


def test_permute_golden():
    g = json.load(open(os.path.join(GOLDEN, "route_permute_worked.json")))["permute"]
    m = oracle.permute(np.array(g["topk_idx"]), g["E"])
    for key in ("split_sizes", "offsets", "row_id_map", "src_token"):
        assert m[key].tolist() == g[key], key


@pytest.mark.parametrize("T,E,k", [(256, 8, 2), (97, 16, 4), (300, 128, 8), (1, 4, 1)])
def test_permute_matches_stable_sort(T, E, k):
    rng = np.random.default_rng(T + E)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    idx, _ = oracle.route_topk(logits, k)
    m = oracle.permute(idx, E)
    flat = idx.ravel()
    order = np.argsort(flat, kind="stable")               # library routine
    assert (m["src_token"] == order // k).all()
    assert (m["src_slot"] == order % k).all()
    assert (m["split_sizes"] == np.bincount(flat, minlength=E)).all()
    assert m["split_sizes"].sum() == T * k
    assert (np.diff(m["offsets"]) >= 0).all() and m["offsets"][0] == 0
    # row_id_map is a bijection onto [0, R) and inverts src_token/src_slot
    assert np.array_equal(np.sort(m["row_id_map"]), np.arange(T * k))
    r = m["row_id_map"]
    assert (m["src_token"][r] == np.arange(T * k) // k).all()
    # every row of expert e's group really went to e
    for e in range(E):
        a, b = m["offsets"][e], m["offsets"][e + 1]
        assert (idx.ravel()[m["src_token"][a:b] * k + m["src_slot"][a:b]] == e).all()
    # gathering moves bits unchanged
    x = rng.standard_normal((T, 8)).astype(np.float32)
    xp = oracle.gather_rows(x, m["src_token"])
    assert np.array_equal(xp[r.reshape(T, k)[:, -1]], x)


def test_combine_is_index_add_and_inverse_permutation():
    rng = np.random.default_rng(5)
    T, E, k, H = 64, 8, 3, 16
    idx, p = oracle.route_topk(rng.standard_normal((T, E)).astype(np.float32), k)
    m = oracle.permute(idx, E)
    y = rng.standard_normal((T * k, H))
    out = oracle.unpermute_combine(y, m["row_id_map"], T, k, weights=p)
    ref = np.zeros((T, H))
    w = p.ravel()[m["src_token"] * k + m["src_slot"]]
    np.add.at(ref, m["src_token"], y * w[:, None])       # index_add_
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-13)
    # k = 1 with unit weights is the inverse permutation, exactly
    idx1, _ = oracle.route_topk(rng.standard_normal((T, E)).astype(np.float32), 1)
    m1 = oracle.permute(idx1, E)
    x = rng.standard_normal((T, H)).astype(np.float32)
    back = oracle.unpermute_combine(oracle.gather_rows(x, m1["src_token"]), m1["row_id_map"], T, 1)
    assert np.array_equal(back, x.astype(np.float64))


def test_qwen3_workload_has_idle_experts():
    """The skewed workload must leave at least one expert without tokens."""
    w = WORKLOADS["qwen3_fwd"]
    # the logits come from their own stream, so smaller H and I leave them unchanged
    inp = make_inputs(scaled(w, H=32, I=32), want_float=False)
    idx, _ = oracle.route_topk(inp.logits, w.k)
    sizes = np.bincount(idx.ravel(), minlength=w.E)
    assert (sizes == 0).sum() >= 1
    assert sizes.max() > 8 * sizes.mean()
