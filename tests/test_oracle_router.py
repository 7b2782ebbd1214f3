"""Pins for the oracle router and dispatch: hand-derived fixture, closed forms,
brute force over all k-subsets, the library stable sort, and the per-expert
mask-gather order of the layer loop in 'Xiaohongshu dots3 note Open Source Deep
Dive', §3.1."""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
from moe_inputs import config, generate

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
L3 = math.log(3.0)


def _golden():
    return json.load(open(os.path.join(GOLDEN, "tiny_layer_by_hand.json")))


def test_router_golden_by_hand():
    g = _golden()
    r = oracle.route(np.array(g["x"], float), np.array(g["w_router_in_units_of_ln3"]) * L3,
                     np.array(g["bias"]), g["dims"]["k"])
    ex = g["expected"]
    np.testing.assert_allclose(r.scores, ex["scores"], rtol=0, atol=1e-15)
    np.testing.assert_array_equal(r.idx, ex["idx"])
    np.testing.assert_allclose(r.w, ex["w"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(r.gap_sel, ex["gap_sel"], atol=1e-15)
    np.testing.assert_allclose(r.gap_ord, ex["gap_ord"], atol=1e-15)


def test_dispatch_golden_by_hand():
    g = _golden()
    ex = g["expected"]
    d = oracle.dispatch(np.array(ex["idx"]), g["dims"]["E"])
    for key in ("counts", "offsets", "perm", "inv"):
        np.testing.assert_array_equal(getattr(d, key), ex[key])


def _c0_routing():
    cfg = config(0)
    inp = generate(cfg)
    return cfg, inp, oracle.route_inputs(cfg, inp)


def test_router_invariants_c0():
    cfg, inp, r = _c0_routing()
    assert r.idx.shape == (cfg.T, cfg.k) and r.idx.dtype == np.int32
    assert np.all((r.idx >= 0) & (r.idx < cfg.E))
    assert all(len(set(row)) == cfg.k for row in r.idx.tolist())
    np.testing.assert_allclose(r.w.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(r.w > 0)
    chosen = np.take_along_axis(r.keys, r.idx.astype(np.int64), 1)
    assert np.all(np.diff(chosen, axis=1) <= 0)             # slot order: key descending
    # every unchosen key is at most the k-th chosen key
    mask = np.ones_like(r.keys, bool)
    np.put_along_axis(mask, r.idx.astype(np.int64), False, 1)
    assert np.all(np.where(mask, r.keys, -np.inf).max(1) <= chosen[:, -1])


def test_router_zero_weight_closed_form():
    """W_router = 0: every score is sigmoid(0) = 1/2, so the choice is the top-k
    of the bias alone (lower index first on equal bias) and every weight is 1/k."""
    rng = np.random.default_rng(5)
    E, k, T, H = 16, 4, 7, 32
    bias = np.round(rng.uniform(-0.01, 0.01, E), 3)          # rounding makes equal biases
    bias[3] = bias[9]
    r = oracle.route(rng.normal(size=(T, H)), np.zeros((E, H)), bias, k)
    assert np.all(r.scores == 0.5)
    expect = sorted(range(E), key=lambda e: (-bias[e], e))[:k]
    for t in range(T):
        assert r.idx[t].tolist() == expect
    assert np.all(r.w == 1.0 / k)


def test_router_bruteforce_subsets():
    """The chosen set maximises the sum of keys over all C(E, k) subsets."""
    rng = np.random.default_rng(6)
    E, k, T, H = 9, 3, 40, 16
    x = rng.normal(size=(T, H))
    wr = rng.normal(0, 0.3, size=(E, H))
    b = rng.uniform(-0.1, 0.1, E)
    r = oracle.route(x, wr, b, k)
    s_ref = 1.0 / (1.0 + np.exp(-(x @ wr.T)))
    np.testing.assert_allclose(r.scores, s_ref, rtol=1e-15)
    for t in range(T):
        c = s_ref[t] + b
        best = max(itertools.combinations(range(E), k), key=lambda sub: sum(c[list(sub)]))
        assert set(r.idx[t].tolist()) == set(best)
        # weights renormalise the UNBIASED scores of the chosen experts
        sel = s_ref[t, r.idx[t]]
        np.testing.assert_allclose(r.w[t], sel / sel.sum(), rtol=1e-14)


def test_router_flags_and_scaling():
    rng = np.random.default_rng(7)
    x, wr, b = rng.normal(size=(5, 8)), rng.normal(size=(6, 8)), np.zeros(6)
    r0 = oracle.route(x, wr, b, 2, norm_topk_prob=False, routed_scaling_factor=2.5)
    sel = np.take_along_axis(r0.scores, r0.idx.astype(np.int64), 1)
    np.testing.assert_allclose(r0.w, 2.5 * sel, rtol=1e-15)
    r1 = oracle.route(x, wr, b, 2, routed_scaling_factor=2.5)
    np.testing.assert_allclose(r1.w.sum(1), 2.5, rtol=1e-14)
    r6 = oracle.route(x, wr, b, 6)          # k = E: every expert, no selection gap
    assert np.all(np.isinf(r6.gap_sel))
    assert sorted(r6.idx[0].tolist()) == list(range(6))


def test_dispatch_invariants_and_library_sort():
    cfg, inp, r = _c0_routing()
    d = oracle.dispatch(r.idx, cfg.E)
    R = cfg.T * cfg.k
    assert d.counts.sum() == R
    np.testing.assert_array_equal(d.offsets[1:] - d.offsets[:-1], d.counts)
    np.testing.assert_array_equal(np.sort(d.perm), np.arange(R))      # bijection
    np.testing.assert_array_equal(d.inv[d.perm], np.arange(R))
    np.testing.assert_array_equal(d.perm, np.argsort(r.idx.ravel(), kind="stable"))
    np.testing.assert_array_equal(d.counts, np.bincount(r.idx.ravel(), minlength=cfg.E))


def test_dispatch_matches_mask_gather_order():
    """The layer loop visits experts in index order and gathers x[mask], i.e.
    the tokens that picked expert e in ascending token order.  The sorted rows
    of expert e must be those tokens in that order."""
    rng = np.random.default_rng(8)
    E, k, T = 12, 3, 50
    idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    d = oracle.dispatch(idx, E)
    for e in range(E):
        mask_tokens = [t for t in range(T) if e in idx[t]]
        rows = d.perm[d.offsets[e]:d.offsets[e + 1]]
        assert (rows // k).tolist() == mask_tokens
        assert all(idx[f // k, f % k] == e for f in rows)


def test_dispatch_empty_experts():
    idx = np.array([[5, 2], [2, 5], [5, 7]], dtype=np.int32)
    d = oracle.dispatch(idx, 9)
    assert d.counts.tolist() == [0, 0, 2, 0, 0, 3, 0, 1, 0]
    assert d.offsets.tolist() == [0, 0, 0, 2, 2, 2, 5, 5, 6, 6]
    assert d.perm.tolist() == [1, 2, 0, 3, 4, 5]


def test_zipf_workload_skew():
    """The skewed workload must leave some experts empty and give some more than
    10x the mean number of rows (its stated purpose), under the oracle router."""
    cfg = config(3)
    inp = generate(cfg, weights=False)
    r = oracle.route_inputs(cfg, inp)
    counts = np.bincount(r.idx.ravel(), minlength=cfg.E)
    mean = cfg.T * cfg.k / cfg.E
    assert counts.max() >= 10 * mean
    assert (counts == 0).sum() >= 1
