"""Pins of the oracle's routing: selection against a library stable sort,
weights against the softmax-over-selected closed form, hand-worked ties."""

import numpy as np
import pytest
from scipy.special import softmax

import oracle


def lexsort_topk(logits, k):
    """First k of a stable full sort by (logit desc, index asc) via numpy."""
    out = []
    for row in logits:
        order = np.lexsort((np.arange(len(row)), -row.astype(np.float64)))
        out.append(order[:k])
    return np.array(out)


@pytest.mark.parametrize("m,e,k", [(1, 16, 2), (4, 512, 8), (3, 64, 64), (2, 33, 1)])
def test_topk_equals_full_sort_random(m, e, k):
    rng = np.random.default_rng(10 + e)
    logits = rng.standard_normal((m, e)).astype(np.float32)
    ids, w = oracle.route_topk(logits, k)
    np.testing.assert_array_equal(ids, lexsort_topk(logits, k))


@pytest.mark.parametrize("seed", range(5))
def test_topk_equals_full_sort_tie_heavy(seed):
    rng = np.random.default_rng(seed)
    logits = rng.choice(np.float32([-1.0, 0.0, -0.0, 1.0]), size=(4, 512))
    for k in (1, 8, 32, 512):
        ids, _ = oracle.route_topk(logits, k)
        np.testing.assert_array_equal(ids, lexsort_topk(logits, k))


def test_topk_hand_worked_ties(golden):
    for case in golden("route_ties.json")["cases"]:
        lg = np.array([case["logits"]], dtype=np.float32)
        ids, _ = oracle.route_topk(lg, case["k"])
        assert ids[0].tolist() == case["ids"], case


def test_weights_closed_form():
    rng = np.random.default_rng(7)
    logits = (rng.standard_normal((4, 512)) * 3).astype(np.float32)
    ids, w = oracle.route_topk(logits, 8)
    for m in range(4):
        sel = logits[m, ids[m]].astype(np.float64)
        np.testing.assert_allclose(w[m], softmax(sel), rtol=1e-13, atol=0)
        assert abs(w[m].sum() - 1.0) < 1e-14
        assert (np.diff(w[m]) <= 0).all()      # ordered like the logits


def test_k1_weight_is_one():
    logits = np.random.default_rng(8).standard_normal((3, 20)).astype(np.float32)
    ids, w = oracle.route_topk(logits, 1)
    assert (w == 1.0).all()
    np.testing.assert_array_equal(ids[:, 0], np.argmax(logits, axis=1))


def test_dispatch_table_groups_tokens():
    ids = np.array([[3, 1], [1, 7], [5, 3]], dtype=np.int32)
    w = np.array([[0.6, 0.4], [0.9, 0.1], [0.7, 0.3]])
    experts, masks, weights = oracle.dispatch_table(ids, w, 16)
    assert experts.tolist() == [1, 3, 5, 7, 16]
    assert masks.tolist() == [0b011, 0b101, 0b100, 0b010, 0b111]
    np.testing.assert_array_equal(weights[0], [0.4, 0.9, 0.0])
    np.testing.assert_array_equal(weights[1], [0.6, 0.0, 0.3])
    np.testing.assert_array_equal(weights[4], [1.0, 1.0, 1.0])


def test_dispatch_bound_verify_window():
    rng = np.random.default_rng(9)
    for _ in range(20):
        logits = rng.standard_normal((4, 512)).astype(np.float32)
        ids, w = oracle.route_topk(logits, 8)
        experts, masks, weights = oracle.dispatch_table(ids, w, 512)
        assert len(experts) - 1 <= 32          # at most 32 routed experts per verify
        # every (token, choice) appears exactly once
        assert sum(bin(int(mk)).count("1") for mk in masks[:-1]) == 32
        np.testing.assert_allclose(weights[:-1].sum(axis=0), 1.0, rtol=1e-14)


def test_router_logits_hand_worked():
    # W_router [E=3][H=2], x [M=1][H=2], worked by hand:
    # e0: 1*2 + 2*(-1) = 0;  e1: -1*2 + 0.5*(-1) = -2.5;  e2: 0*2 + 3*(-1) = -3
    w = np.array([[1.0, 2.0], [-1.0, 0.5], [0.0, 3.0]])
    x = np.array([[2.0, -1.0]])
    np.testing.assert_array_equal(oracle.router_logits(w, x), [[0.0, -2.5, -3.0]])


def test_router_logits_one_hot_selects_a_column_and_zero_input():
    rng = np.random.default_rng(11)
    w = rng.standard_normal((5, 7))           # E = 5 experts, H = 7
    for j in range(7):
        x = np.zeros((1, 7))
        x[0, j] = 1.0
        np.testing.assert_array_equal(oracle.router_logits(w, x)[0], w[:, j])
    np.testing.assert_array_equal(oracle.router_logits(w, np.zeros((2, 7))), np.zeros((2, 5)))


def test_router_logits_linear_in_x():
    rng = np.random.default_rng(12)
    w = rng.integers(-8, 8, size=(6, 16)).astype(np.float64)     # integer values: sums exact
    x1 = rng.integers(-8, 8, size=(3, 16)).astype(np.float64)
    x2 = rng.integers(-8, 8, size=(3, 16)).astype(np.float64)
    np.testing.assert_array_equal(oracle.router_logits(w, x1 + x2),
                                  oracle.router_logits(w, x1) + oracle.router_logits(w, x2))


def test_expert_groups_hand_worked(golden):
    case = golden("expert_groups.json")
    groups = oracle.expert_groups(np.array(case["ids"]), case["n_experts"])
    assert [g.tolist() for g in groups] == case["groups"]
    assert [len(g) for g in groups] == case["counts"]


@pytest.mark.parametrize("m,e,k", [(4, 512, 8), (32, 16, 2), (7, 33, 5)])
def test_expert_groups_match_dispatch_table(m, e, k):
    rng = np.random.default_rng(40 + m)
    ids, w = oracle.route_topk(rng.standard_normal((m, e)).astype(np.float32), k)
    groups = oracle.expert_groups(ids, e)
    experts, masks, _ = oracle.dispatch_table(ids, w, e)
    active = [x for x in range(e) if len(groups[x])]
    assert active == experts[:-1].tolist()
    for x, mask in zip(experts, masks):
        assert groups[x].tolist() == [t for t in range(m) if (int(mask) >> t) & 1]


def test_expert_groups_counting_invariants():
    rng = np.random.default_rng(41)
    t_tokens, e, k = 1000, 512, 8
    ids, _ = oracle.route_topk(rng.standard_normal((t_tokens, e)).astype(np.float32), k)
    groups = oracle.expert_groups(ids, e)
    assert len(groups) == e + 1
    assert sum(len(g) for g in groups) == t_tokens * k + t_tokens
    assert groups[e].tolist() == list(range(t_tokens))
    seen = np.zeros((t_tokens, e), dtype=np.int64)
    for x in range(e):
        assert (np.diff(groups[x]) > 0).all()            # ascending, no repeats
        seen[groups[x], x] += 1
    for t in range(t_tokens):
        assert np.nonzero(seen[t])[0].tolist() == sorted(ids[t].tolist())
