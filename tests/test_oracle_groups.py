"""Pins for the oracle's group-limited router (n_group experts groups, the
topk_group best groups by group score, then the top-k inside them; field
table «MoE 路由与专家相关字段» of the Transformers dots.llm1 article):
a hand-derived fixture, brute force over all group and expert subsets, and
the special cases that reduce to the plain top-k."""
import itertools
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _fixture():
    return json.load(open(os.path.join(GOLDEN, "grouped_router_by_hand.json")))


def _route_scores(s, bias, d):
    s = np.asarray(s, float)
    x = np.log(s / (1.0 - s))                 # logits whose sigmoid is s
    return oracle.route(x, np.eye(d["E"]), np.asarray(bias, float), d["k"],
                        n_group=d["n_group"], topk_group=d["topk_group"])


def test_grouped_router_golden_by_hand():
    g = _fixture()
    d, ex = g["dims"], g["expected"]
    r = _route_scores(g["scores"], g["bias"], d)
    np.testing.assert_array_equal(r.idx, ex["idx"])
    np.testing.assert_allclose(r.w, ex["w"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(r.gap_sel, ex["gap_sel"], atol=1e-14)
    np.testing.assert_allclose(r.gap_ord, ex["gap_ord"], atol=1e-14)
    np.testing.assert_allclose(r.gap_grp, ex["gap_grp"], atol=1e-14)


def test_grouped_router_bias_moves_the_group_choice():
    g = _fixture()
    d = g["dims"]
    r = _route_scores(g["scores"][:1], g["with_bias"]["bias"], d)
    assert r.idx[0, 0] == 6 and r.idx[0, 1] in (4, 7)
    s2 = {4: 0.70, 7: 0.20}[int(r.idx[0, 1])]
    np.testing.assert_allclose(r.w[0], [0.30 / (0.30 + s2), s2 / (0.30 + s2)], atol=1e-14)


def _brute(c, n_group, topk_group, k):
    """All topk_group-subsets of groups (group score by brute force over
    pairs), then all k-subsets of the allowed experts."""
    E = c.size
    G = E // n_group
    gs = []
    for g in range(n_group):
        vals = c[g * G:(g + 1) * G]
        gs.append(vals[0] if G == 1 else max(vals[a] + vals[b]
                                              for a, b in itertools.combinations(range(G), 2)))
    best_groups = max(itertools.combinations(range(n_group), topk_group),
                      key=lambda sub: sum(gs[g] for g in sub))
    allowed = [e for e in range(E) if e // G in best_groups]
    best = max(itertools.combinations(allowed, k), key=lambda sub: sum(c[e] for e in sub))
    return sorted(best, key=lambda e: -c[e])


@pytest.mark.parametrize("E,n_group,topk_group,k", [(8, 4, 2, 2), (12, 3, 2, 3), (8, 8, 3, 3),
                                                    (16, 4, 1, 2), (6, 2, 2, 4)])
def test_grouped_router_brute_force(E, n_group, topk_group, k):
    rng = np.random.default_rng(E * 100 + n_group * 10 + k)
    T, H = 40, 16
    x = rng.standard_normal((T, H))
    w = rng.standard_normal((E, H)) * 0.5
    b = rng.uniform(-0.05, 0.05, E)
    r = oracle.route(x, w, b, k, n_group=n_group, topk_group=topk_group)
    c = oracle.sigmoid(x @ w.T) + b
    for t in range(T):
        assert list(r.idx[t]) == _brute(c[t], n_group, topk_group, k), t
    chosen = np.take_along_axis(oracle.sigmoid(x @ w.T), r.idx.astype(np.int64), 1)
    np.testing.assert_allclose(r.w, chosen / chosen.sum(1, keepdims=True), rtol=1e-15)


@pytest.mark.parametrize("n_group", [1, 2, 4, 8])
def test_all_groups_kept_is_plain_top_k(n_group):
    rng = np.random.default_rng(7)
    x = rng.standard_normal((64, 32))
    w = rng.standard_normal((16, 32)) * 0.3
    b = rng.uniform(-0.01, 0.01, 16)
    plain_c = oracle.sigmoid(x @ w.T) + b
    r = oracle.route(x, w, b, 4, n_group=n_group, topk_group=n_group)
    for t in range(64):
        ref = sorted(range(16), key=lambda e: (-plain_c[t, e], e))[:4]
        assert list(r.idx[t]) == ref
    assert np.all(np.isinf(r.gap_grp))


def test_group_scores_definition():
    c = np.array([[0.1, 0.9, 0.5, 0.3, 0.2, 0.2]])
    np.testing.assert_allclose(oracle.group_scores(c, 2), [[1.4, 0.5]])   # {0.9, 0.5}, {0.3, 0.2}
    np.testing.assert_allclose(oracle.group_scores(c, 3), [[1.0, 0.8, 0.4]])
    np.testing.assert_allclose(oracle.group_scores(c, 6), c)                # one expert per group
