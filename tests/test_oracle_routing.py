"""Pins of the oracle's routing and dispatch (CPU only).

Each check ties the oracle to something other than itself: exhaustive subset
enumeration, a comparison sort, closed forms, scipy's softmax, and the
invariants the MoonEP page states for dispatch (S*K rows; cu_seqlens offsets).
"""
import itertools

import numpy as np
import pytest
import scipy.special

import oracle



def _beats(l, i, j):
    """Expert i ranks above expert j: larger logit, or equal logit and lower index."""
    return l[i] > l[j] or (l[i] == l[j] and i < j)


def _bruteforce_topk(l, K):
    """The unique K-subset whose every member ranks above every non-member, best first."""
    E = len(l)
    found = []
    for T in itertools.combinations(range(E), K):
        rest = [j for j in range(E) if j not in T]
        if all(_beats(l, i, j) for i in T for j in rest):
            found.append(T)
    assert len(found) == 1
    T = list(found[0])
    # position of i inside T = how many members rank above it
    pos = {i: sum(_beats(l, j, i) for j in T if j != i) for i in T}
    return [i for i, _ in sorted(pos.items(), key=lambda kv: kv[1])]


@pytest.mark.parametrize("seed", range(6))
def test_topk_matches_subset_enumeration_with_ties(seed):
    rng = np.random.default_rng(seed)
    for _ in range(40):
        E = int(rng.integers(2, 9))
        K = int(rng.integers(1, E + 1))
        # integer logits in [-2, 2] force many ties; some zeros become -0.0
        l = rng.integers(-2, 3, size=E).astype(np.float32)
        l[(l == 0) & (rng.random(E) < 0.5)] = -0.0
        got = oracle.topk_experts(l[None, :], K)[0].tolist()
        assert got == _bruteforce_topk(l, K), (l, K)


def test_topk_uniform_logits_pick_lowest_indices():
    l = np.full((3, 10), 0.75, np.float32)
    assert oracle.topk_experts(l, 4).tolist() == [[0, 1, 2, 3]] * 3


def test_topk_negative_zero_equals_positive_zero():
    l = np.array([[-0.0, 0.0, -1.0]], np.float32)
    assert oracle.topk_experts(l, 2).tolist() == [[0, 1]]
    l = np.array([[0.0, -0.0, -1.0]], np.float32)
    assert oracle.topk_experts(l, 2).tolist() == [[0, 1]]


def test_topk_nan_ranks_last():
    l = np.array([[np.nan, -np.inf, 1.0, np.nan]], np.float32)
    assert oracle.topk_experts(l, 4).tolist() == [[2, 1, 0, 3]]


def test_gates_closed_form():
    # logits ln(1..4): p = (1,2,3,4)/10; top-2 = experts 3, 2
    l = np.log(np.array([[1.0, 2.0, 3.0, 4.0]])).astype(np.float32)
    idx = oracle.topk_experts(l, 2)
    assert idx.tolist() == [[3, 2]]
    np.testing.assert_allclose(oracle.gate_weights(l, idx, renorm=False)[0], [0.4, 0.3], rtol=1e-6)
    np.testing.assert_allclose(oracle.gate_weights(l, idx, renorm=True)[0], [4 / 7, 3 / 7], rtol=1e-6)


def test_gates_raw_full_k_is_scipy_softmax():
    rng = np.random.default_rng(1)
    l = (rng.standard_normal((16, 7)) * 3).astype(np.float32)
    idx = np.tile(np.arange(7, dtype=np.int32), (16, 1))
    np.testing.assert_allclose(oracle.gate_weights(l, idx, renorm=False),
                               scipy.special.softmax(l.astype(np.float64), axis=1), rtol=1e-13)


def test_gates_two_experts_top1_raw_is_sigmoid_of_gap():
    rng = np.random.default_rng(2)
    l = (rng.standard_normal((32, 2)) * 4).astype(np.float32)
    idx = oracle.topk_experts(l, 1)
    g = oracle.gate_weights(l, idx, renorm=False)[:, 0]
    sel = np.take_along_axis(l, idx, 1)[:, 0].astype(np.float64)
    other = np.take_along_axis(l, 1 - idx, 1)[:, 0].astype(np.float64)
    np.testing.assert_allclose(g, scipy.special.expit(sel - other), rtol=1e-13)


def test_gates_renorm_sum_to_one_and_shift_invariant():
    rng = np.random.default_rng(3)
    l = (rng.standard_normal((50, 12)) * 2).astype(np.float32)
    idx = oracle.topk_experts(l, 3)
    g = oracle.gate_weights(l, idx, renorm=True)
    np.testing.assert_allclose(g.sum(1), 1.0, atol=1e-14)
    g2 = oracle.gate_weights(l + np.float32(8.0), idx, renorm=True)
    np.testing.assert_allclose(g, g2, rtol=1e-5)  # logits re-rounded to float32 after the shift
    assert np.all(np.diff(g, axis=1) <= 1e-15)      # best first => non-increasing gates


def test_router_logits_against_integer_closed_form():
    # small integers: every product and sum is exact in float32 and float64
    rng = np.random.default_rng(4)
    x = rng.integers(-3, 4, size=(5, 6)).astype(np.float32)
    Wg = rng.integers(-3, 4, size=(6, 4)).astype(np.float32)
    b = np.array([0.5, -1.0, 2.0, 0.0], np.float32)
    want = np.array([[sum(int(x[s, h]) * int(Wg[h, e]) for h in range(6)) + b[e] for e in range(4)]
                     for s in range(5)], np.float32)
    np.testing.assert_array_equal(oracle.router_logits(x, Wg, b), want)


def test_dispatch_hand_worked_example():
    # S=3, K=2, E=3; counting by hand: expert 0 gets tokens 0 (k=1), 1 (k=0);
    # expert 1 gets tokens 1 (k=1), 2 (k=1); expert 2 gets tokens 0 (k=0), 2 (k=0).
    idx = np.array([[2, 0], [0, 1], [2, 1]], np.int32)
    counts, cu = oracle.expert_counts(idx, 3)
    assert counts.tolist() == [2, 2, 2] and cu.tolist() == [0, 2, 4, 6]
    row_of, tok_of = oracle.dispatch_permutation(idx, 3)
    assert row_of.tolist() == [4, 0, 1, 2, 5, 3]
    assert tok_of.tolist() == [0, 1, 1, 2, 0, 2]


def _random_routing(rng, S, E, K):
    l = rng.standard_normal((S, E)).astype(np.float32)
    l += np.float32(2.0) * (np.arange(E) % 3 == 0)   # skew: some experts hot
    return oracle.topk_experts(l, K)


@pytest.mark.parametrize("S,E,K", [(1, 1, 1), (7, 5, 5), (64, 8, 2), (300, 33, 4), (129, 64, 8)])
def test_dispatch_invariants_and_comparison_sort(S, E, K):
    rng = np.random.default_rng(S * 31 + E)
    idx = _random_routing(rng, S, E, K)
    counts, cu = oracle.expert_counts(idx, E)
    np.testing.assert_array_equal(counts, np.bincount(idx.ravel(), minlength=E))
    assert cu[0] == 0 and cu[-1] == S * K and np.all(np.diff(cu) >= 0)
    assert np.all(counts <= S)
    row_of, tok_of = oracle.dispatch_permutation(idx, E)
    # bijection on [0, S*K)
    assert sorted(row_of.tolist()) == list(range(S * K))
    p = np.arange(S * K)
    np.testing.assert_array_equal(tok_of[row_of], p // K)
    # each pair lands in its expert's block; tokens strictly ascend inside a block
    e_of_pair = idx.ravel()
    assert np.all(row_of >= cu[e_of_pair]) and np.all(row_of < cu[e_of_pair + 1])
    for e in range(E):
        blk = tok_of[cu[e]:cu[e + 1]]
        assert np.all(np.diff(blk) > 0)
    # same permutation from a comparison sort of the pairs by (expert, token)
    pairs = sorted(range(S * K), key=lambda q: (int(e_of_pair[q]), q // K))
    want = np.empty(S * K, np.int64)
    want[np.array(pairs)] = np.arange(S * K)
    np.testing.assert_array_equal(row_of, want)
    # dispatch copies every token bit for bit into each of its rows
    x = rng.standard_normal((S, 16)).astype(np.float32)
    xd = oracle.dispatch_rows(x, tok_of)
    np.testing.assert_array_equal(xd[row_of], np.repeat(x, K, axis=0))


def test_maxvio_definition():
    assert oracle.maxvio([4, 4, 4, 4]) == 0.0
    assert oracle.maxvio([16, 0, 0, 0]) == pytest.approx(3.0)


def test_load_entropy_closed_forms():
    # balanced load: ln E; one expert takes every pair: 0; a 3:1 split of two
    # experts: ln 4 - (3/4) ln 3 (worked by hand: -(3/4) ln(3/4) - (1/4) ln(1/4))
    assert oracle.load_entropy([5, 5, 5, 5, 5, 5, 5, 5]) == pytest.approx(np.log(8), rel=1e-14)
    assert oracle.load_entropy([0, 0, 12, 0]) == 0.0
    assert oracle.load_entropy([3, 0, 1]) == pytest.approx(np.log(4) - 0.75 * np.log(3), rel=1e-14)
    assert oracle.load_entropy([0, 0, 0]) == 0.0
    # invariant under relabelling the experts and under scaling every count
    rng = np.random.default_rng(3)
    c = rng.integers(0, 50, size=37)
    assert oracle.load_entropy(c) == pytest.approx(oracle.load_entropy(rng.permutation(c)), rel=1e-13)
    assert oracle.load_entropy(c) == pytest.approx(oracle.load_entropy(7 * c), rel=1e-13)
    # between 0 and ln(#experts with load)
    assert 0.0 <= oracle.load_entropy(c) <= np.log(np.count_nonzero(c)) + 1e-12
