"""Pins of the oracle's router (orc_route) on the CPU.

The router is the step before the routed-expert path: softmax over the experts, the k most
probable experts in descending order with ties to the lower id, and their probabilities
renormalised to sum to one (summed in selection order).  The oracle is checked against a
brute force written here with Python's sorted() and math.exp, against closed forms (two
experts: the logistic function), and against invariants that hold for any correct router
(weights sum to one, selection in descending logit order, shift invariance, k = E gives a
permutation).
"""
import math

import numpy as np
import pytest

import oracle
from workload import gen_logits


def brute_route(logits, k):
    """Python reference: selection by (descending logit, ascending id); p from math.exp."""
    ids, ws = [], []
    for row in np.asarray(logits, dtype=np.float32):
        vals = [float(v) for v in row]
        m = max(vals)
        ex = [math.exp(v - m) for v in vals]
        z = 0.0
        for v in ex:
            z += v
        p = [v / z for v in ex]
        sel = sorted(range(len(vals)), key=lambda e: (-vals[e], e))[:k]
        s = 0.0
        for e in sel:
            s += p[e]
        ids.append(sel)
        ws.append([p[e] / s for e in sel])
    return np.array(ids, np.int32), np.array(ws, np.float64)


@pytest.mark.parametrize("T,E,k", [(40, 8, 2), (25, 37, 5), (12, 512, 10), (6, 1024, 16), (9, 13, 13)])
def test_route_matches_brute_force(T, E, k):
    lg = gen_logits(T, E, seed=100 + E)
    ids, w = oracle.route(lg, k)
    bids, bw = brute_route(lg, k)
    assert np.array_equal(ids, bids)
    np.testing.assert_allclose(w, bw, rtol=1e-12, atol=0)


def test_route_ties_go_to_the_lower_id():
    rng = np.random.default_rng(7)
    lg = rng.integers(-2, 3, size=(50, 20)).astype(np.float32)  # many equal logits per row
    ids, w = oracle.route(lg, 6)
    bids, bw = brute_route(lg, 6)
    assert np.array_equal(ids, bids)
    np.testing.assert_allclose(w, bw, rtol=1e-12)
    # equal logits in one row get equal weights
    for t in range(lg.shape[0]):
        for a in range(6):
            for b in range(6):
                if lg[t, ids[t, a]] == lg[t, ids[t, b]]:
                    assert w[t, a] == w[t, b]


def test_route_two_experts_closed_form():
    lg = np.array([[0.25, -1.5], [3.0, 3.0], [-2.0, 1.0]], np.float32)
    ids, w = oracle.route(lg, 1)
    assert ids.ravel().tolist() == [0, 0, 1] and np.all(w == 1.0)
    ids, w = oracle.route(lg, 2)
    assert ids.tolist() == [[0, 1], [0, 1], [1, 0]]
    for t in range(3):
        a, b = float(lg[t, ids[t, 0]]), float(lg[t, ids[t, 1]])
        assert w[t, 0] == pytest.approx(1.0 / (1.0 + math.exp(b - a)), rel=1e-14)
        assert w[t, 1] == pytest.approx(1.0 / (1.0 + math.exp(a - b)), rel=1e-14)


def test_route_invariants():
    lg = gen_logits(64, 512, seed=5)
    ids, w = oracle.route(lg, 10)
    # weights sum to one, are positive and follow the selection (non-increasing)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-14)
    assert np.all(w > 0) and np.all(np.diff(w, axis=1) <= 0)
    # selection in descending logit order, distinct ids, none better left out
    sel = np.take_along_axis(lg, ids, axis=1)
    assert np.all(np.diff(sel, axis=1) <= 0)
    assert all(len(set(r)) == 10 for r in ids.tolist())
    rest = lg.copy()
    np.put_along_axis(rest, ids, -np.inf, axis=1)
    assert np.all(rest.max(axis=1) <= sel[:, -1])
    # shift invariance: on logits that are multiples of 2^-10 with |l| < 8, adding 64 is exact
    # in fp32, so the selection is identical and the weights agree to double rounding
    lq = (np.round(lg * 1024.0) / 1024.0).astype(np.float32)
    idq, wq = oracle.route(lq, 10)
    ids2, w2 = oracle.route(lq + np.float32(64.0), 10)
    assert np.array_equal(ids2, idq)
    np.testing.assert_allclose(w2, wq, rtol=1e-13)


def test_route_k_equals_e_is_a_permutation():
    lg = gen_logits(10, 13, seed=9)
    ids, w = oracle.route(lg, 13)
    assert np.all(np.sort(ids, axis=1) == np.arange(13))
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-14)


def test_route_rejects_bad_shapes():
    lg = gen_logits(2, 4, seed=1)
    with pytest.raises(ValueError):
        oracle.route(lg, 5)
    with pytest.raises(ValueError):
        oracle.route(lg, 0)
