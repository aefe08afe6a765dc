"""Pins of the oracle's DFlash 2 path selector ([DF] section 7.1, Problem 1) to facts other
than its own formula: candidate order against a stable library sort, the greedy limit when
the pair term vanishes, and a hand-built "successor" model whose pair term is lambda when
b = a + 1 (one-hot embeddings, A = identity, B = shift, H = lambda), where the walk's
result is known without evaluating S."""
import numpy as np

import oracle as O

V = 8


def _successor_model(lam):
    E = np.eye(V)                                  # one-hot token embeddings, D = V
    w_a = np.eye(V)                                # A(a) = e_a
    w_b = np.zeros((V, V))
    for b in range(V):
        w_b[b, (b - 1) % V] = 1.0                  # B(b) = e_{b-1}
    w_h = np.full((V, V), lam / V)                 # H(norm(1)) = lam * 1
    h = np.ones((V, V))                            # rmsnorm(1) = 1 with unit gains
    return E, w_a, w_b, w_h, h


def _select(z, h, anchor, E, w_a, w_b, w_h, k):
    return O.select_path(z, h, anchor, E, np.ones(E.shape[1]), 0.0, w_a, w_b, w_h, top_k=k, dt=np.float64)


def test_candidates_follow_a_stable_descending_sort():
    rng = np.random.default_rng(3)
    z = rng.integers(0, 6, size=(5, 40)).astype(np.float64)     # many ties
    for k in (1, 4, 16, 40):
        got = O.topk_lowest(z, k)
        want = np.argsort(-z, axis=-1, kind="stable")[:, :k]
        assert np.array_equal(got, want)


def test_no_pair_term_is_the_greedy_argmax():
    rng = np.random.default_rng(4)
    z = rng.standard_normal((7, 50))
    h = rng.standard_normal((7, 12))
    E = rng.standard_normal((50, 12))
    w_a = np.zeros((12, 6))
    w_b = rng.standard_normal((12, 6))
    w_h = rng.standard_normal((12, 6))
    ids, cand, _ = O.select_path(z, h, 3, E, np.ones(12), 1e-6, w_a, w_b, w_h, top_k=16, dt=np.float64)
    assert np.array_equal(ids, O.argmax_lowest(z))
    assert np.array_equal(cand[:, 0], O.argmax_lowest(z))
    # a single candidate per position is the greedy argmax whatever the pair weights
    ids1, _, _ = O.select_path(z, h, 3, E, np.ones(12), 1e-6, rng.standard_normal((12, 6)), w_b, w_h,
                               top_k=1, dt=np.float64)
    assert np.array_equal(ids1, O.argmax_lowest(z))


def test_strong_successor_term_walks_from_the_anchor():
    rng = np.random.default_rng(5)
    E, w_a, w_b, w_h, h = _successor_model(lam=100.0)
    z = rng.random((6, V))
    for anchor in (0, 5):
        ids, _, _ = _select(z, h[:6], anchor, E, w_a, w_b, w_h, V)
        assert list(ids) == [(anchor + t) % V for t in range(1, 7)]


def test_the_walk_follows_its_own_choices_not_the_argmax():
    # top-2 candidates; the successor of the previous choice wins when it is a candidate,
    # otherwise the higher logit of the two
    E, w_a, w_b, w_h, h = _successor_model(lam=100.0)
    z = np.zeros((4, V))
    z[0, [1, 6]] = [1.0, 2.0]    # successor of anchor 0 is 1: a candidate, chosen over 6
    z[1, [4, 5]] = [2.0, 1.0]    # successor 2 is not a candidate: the higher logit, 4
    z[2, [5, 3]] = [1.0, 2.0]    # successor of 4 is 5 (lower logit) - chosen
    z[3, [6, 7]] = [1.0, 2.0]    # successor of 5 is 6
    ids, _, _ = _select(z, h[:4], 0, E, w_a, w_b, w_h, 2)
    assert list(ids) == [1, 4, 5, 6]
    # the plain argmax walk would differ at positions 1, 3 and 4
    assert list(O.argmax_lowest(z)) == [6, 4, 3, 7]


def test_a_negative_gate_avoids_the_successor():
    E, w_a, w_b, w_h, h = _successor_model(lam=-100.0)
    z = np.zeros((3, V))
    z[:, :] = np.arange(V)[None, :] * 0.01
    z[0, 3] = 5.0                # the successor of anchor 2 has the best logit ...
    ids, _, _ = _select(z, h[:3], 2, E, w_a, w_b, w_h, V)
    assert ids[0] != 3           # ... but the gate pushes it below every other candidate
    assert ids[0] == V - 1       # the best remaining logit
