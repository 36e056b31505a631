"""Pins of the CPU oracle against facts fixed outside the oracle itself.

The AdaFuse summary pages print no worked example, so every pin here is a closed
form, a hand-derived exact example, brute force over tiny inputs, an invariant the
method must satisfy, or a special case that reduces to a textbook routine.  Each is
chosen so that a plausible slip in the oracle (a dropped term, a wrong sign or index,
a transposed operand, the wrong softmax pool) fails at least one of them.
"""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import expit, softmax

from oracle import adafuse as O


def distinct_logits(rng, E, gap=1e-3):
    while True:
        z = rng.standard_normal(E)
        s = np.sort(z)
        if E == 1 or np.min(np.diff(s)) >= gap:
            return z


# ---------------------------------------------------------------- top-k selection


@pytest.mark.parametrize("E", range(1, 9))
def test_topk_is_the_argmax_subset_by_brute_force(E):
    """The selected set is the unique k-subset with the largest score sum, listed in
    descending score order (exhaustive over all C(E, k) subsets)."""
    rng = np.random.default_rng(100 + E)
    for trial in range(20):
        z = distinct_logits(rng, E)
        for k in range(1, E + 1):
            idx = O.select_topk(z, k)
            best = max(itertools.combinations(range(E), k), key=lambda c: sum(z[i] for i in c))
            assert set(idx.tolist()) == set(best)
            vals = [z[i] for i in idx]
            assert all(vals[i] > vals[i + 1] for i in range(k - 1))


@pytest.mark.parametrize("E", range(1, 7))
def test_topk_over_every_permutation(E):
    """For every ordering of E distinct scores, the j-th selected index holds the j-th
    largest score (exhaustive over all E! permutations)."""
    base = np.linspace(-1.5, 2.0, E) if E > 1 else np.array([0.3])
    desc = sorted(base.tolist(), reverse=True)
    for perm in itertools.permutations(range(E)):
        z = base[list(perm)]
        for k in range(1, E + 1):
            idx = O.select_topk(z, k)
            assert [z[i] for i in idx] == desc[:k]


def test_topk_ties_go_to_the_lower_index():
    assert O.select_topk([1.0, 3.0, 3.0, 2.0], 2).tolist() == [1, 2]
    assert O.select_topk([0.5, 0.5, 0.5, 0.5], 3).tolist() == [0, 1, 2]
    assert O.select_topk([2.0, 1.0, 2.0, 2.0], 2).tolist() == [0, 2]
    # brute force: with many ties, the stable rule equals lexicographic (-z, e) order
    rng = np.random.default_rng(7)
    for _ in range(200):
        E = int(rng.integers(1, 9))
        z = rng.integers(0, 3, size=E).astype(float)
        k = int(rng.integers(1, E + 1))
        expect = [e for _, e in sorted((-z[e], e) for e in range(E))][:k]
        assert O.select_topk(z, k).tolist() == expect


def test_topk_decides_in_fp32():
    """Scores closer than fp32 resolution tie, and the tie goes to the lower index."""
    z = np.array([1.0, 1.0 + 1e-12])
    assert O.select_topk(z, 1).tolist() == [0]


# ---------------------------------------------------------------- gates


def test_gates_closed_forms():
    rng = np.random.default_rng(1)
    for _ in range(50):
        E = int(rng.integers(1, 17))
        z = distinct_logits(rng, E) * 3
        for k in range(1, E + 1):
            idx = O.select_topk(z, k)
            g = O.gate_weights(z, idx, renorm=True)
            assert abs(g.sum() - 1.0) < 1e-14
            assert np.all(np.diff(g) < 0) or k == 1
            # shifting every logit leaves the gates unchanged
            g2 = O.gate_weights(z + 123.25, idx, renorm=True)
            np.testing.assert_allclose(g2, g, rtol=1e-12)
        # k = E: the textbook softmax, in selection order
        idx = O.select_topk(z, E)
        np.testing.assert_allclose(O.gate_weights(z, idx), softmax(z)[idx], rtol=1e-13)
        # k = 1: a single gate of exactly one
        assert O.gate_weights(z, O.select_topk(z, 1)).tolist() == [1.0]


def test_top2_gate_is_the_logistic_of_the_logit_gap():
    rng = np.random.default_rng(2)
    for _ in range(100):
        z = distinct_logits(rng, 8) * 2
        idx = O.select_topk(z, 2)
        g = O.gate_weights(z, idx)
        assert abs(g[0] - expit(z[idx[0]] - z[idx[1]])) < 1e-14
        assert abs(g[1] - expit(z[idx[1]] - z[idx[0]])) < 1e-14


def test_gates_without_renormalisation_are_full_softmax_entries():
    rng = np.random.default_rng(3)
    z = distinct_logits(rng, 8)
    idx = O.select_topk(z, 3)
    np.testing.assert_allclose(O.gate_weights(z, idx, renorm=False), softmax(z)[idx], rtol=1e-13)
    assert O.gate_weights(z, idx, renorm=False).sum() < 1.0


def test_router_logits_by_loops():
    rng = np.random.default_rng(4)
    R = rng.standard_normal((5, 7))
    h = rng.standard_normal(7)
    z = O.router_logits(h, R)
    for e in range(5):
        acc = 0.0
        for j in range(7):
            acc += R[e, j] * h[j]
        assert abs(z[e] - acc) < 1e-12


# ---------------------------------------------------------------- hand-derived example

# E = 3 experts of rank 1 over d_in = 3, d_out = 2, s = 2, router over d = 2.
# R h = [ln 3, 0, -1]: top-2 picks experts [0, 1]; softmax over {ln 3, 0} gives
# gates [3/4, 1/4], so the coefficients s*g are [3/2, 1/2].
#   B0 A0 = [1,-1]^T [1,0,2] = [[1,0,2],[-1,0,-2]]
#   B1 A1 = [2, 0]^T [0,1,1] = [[0,2,2],[ 0,0, 0]]
#   delta = 3/2 B0A0 + 1/2 B1A1 = [[3/2, 1, 4], [-3/2, 0, -3]]
#   W'    = [[1,2,3],[4,5,6]] + delta = [[5/2, 3, 7], [5/2, 5, 3]]
# With x = [1,1,1]: W' x = [25/2, 21/2]; the routed form gives W x = [6, 15],
#   A0 x = 3, A1 x = 2, s(3/4 B0*3 + 1/4 B1*2) = [13/2, -9/2], sum [25/2, 21/2].
HAND = dict(
    h=[1.0, 0.0],
    R=[[math.log(3.0), 0.0], [0.0, 0.0], [-1.0, 0.0]],
    W=[[1, 2, 3], [4, 5, 6]],
    A=[[[1, 0, 2]], [[0, 1, 1]], [[5, 5, 5]]],
    B=[[[1], [-1]], [[2], [0]], [[7], [7]]],
    s=2.0,
    idx=[0, 1],
    gate=[Fraction(3, 4), Fraction(1, 4)],
    merged=[[Fraction(5, 2), 3, 7], [Fraction(5, 2), 5, 3]],
    x=[1, 1, 1],
    y=[Fraction(25, 2), Fraction(21, 2)],
)


def test_hand_derived_example():
    idx, g = O.pregate(HAND["h"], HAND["R"], 2)
    assert idx.tolist() == HAND["idx"]
    np.testing.assert_allclose(g, [float(v) for v in HAND["gate"]], rtol=1e-15)
    Wm = O.merge(HAND["W"], HAND["A"], HAND["B"], idx, g, HAND["s"])
    np.testing.assert_allclose(Wm, [[float(v) for v in row] for row in HAND["merged"]], rtol=1e-15, atol=1e-15)
    y = O.gemv(Wm, HAND["x"])
    np.testing.assert_allclose(y, [float(v) for v in HAND["y"]], rtol=1e-15)
    yb = O.routed_lora_forward(HAND["W"], HAND["A"], HAND["B"], idx, g, HAND["s"], HAND["x"])
    np.testing.assert_allclose(yb, [float(v) for v in HAND["y"]], rtol=1e-15)
    back = O.unmerge(Wm, HAND["A"], HAND["B"], idx, g, HAND["s"])
    np.testing.assert_allclose(back, HAND["W"], atol=1e-15)


# ---------------------------------------------------------------- merge


def loop_merge(W, A, B, idx, coef):
    """Merged weights by explicit loops over (row, col, slot, rank)."""
    d_out, d_in = len(W), len(W[0])
    r = len(A[0])
    out = [[float(W[i][j]) for j in range(d_in)] for i in range(d_out)]
    for e, c in zip(idx, coef):
        if c == 0:
            continue
        for i in range(d_out):
            for j in range(d_in):
                acc = 0.0
                for t in range(r):
                    acc += float(B[e][i][t]) * float(A[e][t][j])
                out[i][j] += c * acc
    return np.array(out)


def test_merge_matches_explicit_loops():
    rng = np.random.default_rng(5)
    E, r, d_out, d_in = 4, 3, 5, 7
    W = rng.standard_normal((d_out, d_in))
    A = rng.standard_normal((E, r, d_in))
    B = rng.standard_normal((E, d_out, r))
    idx, g, s = [2, 0, 3], [0.5, 0.3, 0.2], 1.75
    got = O.merge(W, A, B, idx, g, s)
    ref = loop_merge(W.tolist(), A.tolist(), B.tolist(), idx, [s * v for v in g])
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-13)


def test_merge_places_a_rank1_update_at_row_of_B_and_column_of_A():
    """Unit vectors: B_e = unit row 3, A_e = unit column 5  ->  only W'[3, 5] changes.
    A transposed operand or swapped factor would move the update."""
    E, r, d_out, d_in = 3, 1, 6, 8
    W = np.zeros((d_out, d_in))
    A = np.zeros((E, r, d_in))
    B = np.zeros((E, d_out, r))
    A[1, 0, 5] = 1.0
    B[1, 3, 0] = 1.0
    A[0, 0, 2] = 1.0   # expert 0 must stay unused
    B[0, 1, 0] = 1.0
    got = O.merge(W, A, B, [1], [1.0], 2.5)
    expect = np.zeros((d_out, d_in))
    expect[3, 5] = 2.5
    assert np.array_equal(got, expect)


def test_k1_unit_gate_is_the_static_lora_merge():
    """k = 1, g = 1 reduces to the static LoRA fusion W + s B A (explicit loops)."""
    rng = np.random.default_rng(6)
    E, r, d_out, d_in = 3, 4, 6, 5
    W = rng.standard_normal((d_out, d_in))
    A = rng.standard_normal((E, r, d_in))
    B = rng.standard_normal((E, d_out, r))
    got = O.merge(W, A, B, [2], [1.0], 2.0)
    ref = W.copy()
    for i in range(d_out):
        for j in range(d_in):
            ref[i, j] += 2.0 * sum(B[2, i, t] * A[2, t, j] for t in range(r))
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-14)


def test_zero_gates_leave_w_bit_identical_and_are_dropped():
    rng = np.random.default_rng(8)
    W = rng.standard_normal((4, 6))
    W[0, 0] = -0.0
    A = rng.standard_normal((3, 2, 6))
    B = rng.standard_normal((3, 4, 2))
    A[1, 0, 0] = np.inf            # a dropped slot must never touch it (0 * inf = nan)
    out = O.merge(W, A, B, [1, 2], [0.0, 0.0], 2.0)
    assert out.tobytes() == W.tobytes()
    out = O.merge(W, A, B, [1, 2], [0.0, 1.0], 2.0)
    assert np.all(np.isfinite(out))
    np.testing.assert_allclose(out, W + 2.0 * B[2] @ A[2], rtol=1e-14)


def test_linearity_merged_gemv_equals_routed_lora():
    """(W + delta) x == W x + s sum_j g_j B_j (A_j x) in fp64."""
    rng = np.random.default_rng(9)
    E, r, d_out, d_in = 8, 16, 48, 40
    W = rng.standard_normal((d_out, d_in)) * 0.02
    A = rng.standard_normal((E, r, d_in)) / np.sqrt(d_in)
    B = rng.standard_normal((E, d_out, r)) * 0.01
    h, R = rng.standard_normal(d_in), rng.standard_normal((E, d_in))
    idx, g = O.pregate(h, R, 3)
    x = rng.standard_normal(d_in)
    lhs = O.gemv(O.merge(W, A, B, idx, g, 2.0), x)
    rhs = O.routed_lora_forward(W, A, B, idx, g, 2.0, x)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-14)
    # and a dropped expert is visible at this scale
    lhs_missing = O.gemv(O.merge(W, A, B, idx[:2], g[:2], 2.0), x)
    assert np.max(np.abs(lhs_missing - rhs)) > 1e-6


def test_unmerge_undoes_merge_and_switch_equals_remerge():
    rng = np.random.default_rng(10)
    E, r, d_out, d_in = 6, 4, 10, 12
    W = rng.standard_normal((d_out, d_in))
    A = rng.standard_normal((E, r, d_in))
    B = rng.standard_normal((E, d_out, r))
    p = (np.array([4, 1]), np.array([0.6, 0.4]))
    c = (np.array([0, 5, 2]), np.array([0.5, 0.3, 0.2]))
    Wm = O.merge(W, A, B, *p, 2.0)
    back = O.unmerge(Wm, A, B, *p, 2.0)
    np.testing.assert_allclose(back, W, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(O.switch(Wm, A, B, p, c, 2.0), O.merge(W, A, B, *c, 2.0), rtol=1e-13, atol=1e-13)


def test_expert_relabelling_is_invisible():
    """Permuting the expert banks together with the router rows gives the same result."""
    rng = np.random.default_rng(11)
    E, r, d = 6, 4, 16
    W = rng.standard_normal((d, d))
    A = rng.standard_normal((E, r, d))
    B = rng.standard_normal((E, d, r))
    h, R = rng.standard_normal(d), rng.standard_normal((E, d))
    idx, g = O.pregate(h, R, 3)
    ref = O.merge(W, A, B, idx, g, 2.0)
    perm = rng.permutation(E)
    idx2, g2 = O.pregate(h, R[perm], 3)
    assert perm[idx2].tolist() == idx.tolist()
    # BLAS may block the relabelled router product differently: equal to rounding
    np.testing.assert_allclose(O.merge(W, A[perm], B[perm], idx2, g2, 2.0), ref, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- gemv


def test_gemv_by_loops_and_identity():
    rng = np.random.default_rng(12)
    W = rng.standard_normal((5, 9))
    x = rng.standard_normal(9)
    y = O.gemv(W, x)
    for i in range(5):
        assert abs(y[i] - sum(W[i, j] * x[j] for j in range(9))) < 1e-12
    assert np.array_equal(O.gemv(np.eye(4), [1.0, -2.0, 3.5, 0.25]), np.array([1.0, -2.0, 3.5, 0.25]))


def test_shape_errors_are_loud():
    with pytest.raises(ValueError):
        O.router_logits(np.zeros(3), np.zeros((2, 4)))
    with pytest.raises(ValueError):
        O.select_topk(np.zeros(3), 4)
    with pytest.raises(ValueError):
        O.adapter_delta(np.zeros((2, 3, 4)), np.zeros((2, 5, 2)), [0], [1.0])
