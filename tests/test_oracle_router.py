"""Pins for the oracle's router (oracle_route_topk): a hand-worked example, brute
force against numpy's stable argsort and scipy's softmax, and the invariants the
definition implies (shift invariance, the bias steering the choice only,
relabelling, topk = all experts)."""
import numpy as np
import pytest
from scipy.special import softmax

import oracle


def brute(logits, topk, bias=None):
    """numpy / scipy: stable descending argsort of the fp32 score, softmax of the chosen raw logits."""
    lg = np.asarray(logits, np.float32)
    score = lg if bias is None else (lg + np.asarray(bias, np.float32)).astype(np.float32)
    ids = np.argsort(-score, axis=1, kind="stable")[:, :topk].astype(np.int32)
    chosen = np.take_along_axis(lg.astype(np.float64), ids, axis=1)
    return ids, softmax(chosen, axis=1)


def test_hand_example():
    # scores 0, 1, 1, -2: the tie between experts 1 and 2 goes to the lower id first
    ids, w = oracle.route_topk(np.array([[0.0, 1.0, 1.0, -2.0]], np.float32), 2)
    assert ids.tolist() == [[1, 2]]
    np.testing.assert_allclose(w, [[0.5, 0.5]], rtol=0, atol=1e-15)
    # with a bias of 3 on expert 3 its score is 1: it ties with 1 and 2 and has the highest id
    ids, w = oracle.route_topk(np.array([[0.0, 1.0, 1.0, -2.0]], np.float32), 3,
                               bias=np.array([0, 0, 0, 3], np.float32))
    assert ids.tolist() == [[1, 2, 3]]
    e = np.exp([1.0, 1.0, -2.0])
    np.testing.assert_allclose(w, [e / e.sum()], rtol=1e-14)


@pytest.mark.parametrize("seed", range(6))
def test_brute_force(seed):
    rng = np.random.default_rng(seed)
    T, Eg, k = 40, [8, 48, 384][seed % 3], [1, 2, 8][seed % 3]
    lg = rng.standard_normal((T, Eg)).astype(np.float32)
    if seed % 2:
        lg = np.round(lg * 2) / 2  # many exact ties
    bias = rng.standard_normal(Eg).astype(np.float32) if seed >= 3 else None
    ids, w = oracle.route_topk(lg, k, bias=bias)
    bi, bw = brute(lg, k, bias)
    np.testing.assert_array_equal(ids, bi)
    np.testing.assert_allclose(w, bw, rtol=1e-13)


def test_weights_are_a_distribution_in_score_order():
    rng = np.random.default_rng(7)
    lg = rng.standard_normal((64, 384)).astype(np.float32)
    ids, w = oracle.route_topk(lg, 8)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-14)
    assert np.all(np.diff(w, axis=1) <= 0)  # without a bias the order of ids is the order of weights
    assert all(len(set(r)) == 8 for r in ids.tolist())


def test_shift_invariance():
    # integer logits and shifts keep every fp32 score exact
    rng = np.random.default_rng(3)
    lg = rng.integers(-20, 20, size=(30, 48)).astype(np.float32)
    bias = rng.integers(-5, 5, size=48).astype(np.float32)
    ids, w = oracle.route_topk(lg, 8, bias=bias)
    ids2, w2 = oracle.route_topk(lg + 7.0, 8, bias=bias)  # every logit of every token
    np.testing.assert_array_equal(ids, ids2)
    np.testing.assert_allclose(w, w2, rtol=1e-13)
    ids3, w3 = oracle.route_topk(lg, 8, bias=bias - 3.0)  # every bias
    np.testing.assert_array_equal(ids, ids3)
    np.testing.assert_allclose(w, w3, rtol=0, atol=0)


def test_bias_steers_the_choice_only():
    rng = np.random.default_rng(11)
    lg = rng.standard_normal((20, 48)).astype(np.float32)
    bias = np.zeros(48, np.float32)
    bias[[5, 17]] = 1e6
    ids, w = oracle.route_topk(lg, 4, bias=bias)
    assert np.all(np.sort(ids[:, :2], axis=1) == [5, 17])
    # weights: softmax over the chosen *raw* logits
    chosen = np.take_along_axis(lg.astype(np.float64), ids, axis=1)
    np.testing.assert_allclose(w, softmax(chosen, axis=1), rtol=1e-13)
    # without the bias, experts 5 and 17 are chosen only where their logits rank
    plain, _ = oracle.route_topk(lg, 4)
    both = [(5 in r) and (17 in r) for r in plain.tolist()]
    assert sum(both) < len(both)


def test_relabelling():
    rng = np.random.default_rng(5)
    lg = rng.standard_normal((25, 48)).astype(np.float32)  # distinct scores
    bias = rng.standard_normal(48).astype(np.float32)
    perm = rng.permutation(48)  # new label of old expert e is perm[e]
    lg_p = np.empty_like(lg)
    lg_p[:, perm] = lg
    bias_p = np.empty_like(bias)
    bias_p[perm] = bias
    ids, w = oracle.route_topk(lg, 8, bias=bias)
    ids_p, w_p = oracle.route_topk(lg_p, 8, bias=bias_p)
    np.testing.assert_array_equal(ids_p, perm[ids])
    np.testing.assert_allclose(w_p, w, rtol=0, atol=0)


def test_all_experts_and_errors():
    lg = np.array([[3.0, -1.0, 2.0, 0.5]], np.float32)
    ids, w = oracle.route_topk(lg, 4)
    assert ids.tolist() == [[0, 2, 3, 1]]
    np.testing.assert_allclose(w[0], softmax(np.array([3.0, 2.0, 0.5, -1.0])), rtol=1e-14)
    with pytest.raises(ValueError):
        oracle.route_topk(lg, 5)
    with pytest.raises(ValueError):
        oracle.route_topk(lg, 0)
