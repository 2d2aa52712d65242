"""CPU tests of the fp64 oracle against what the pages and mathematics fix."""
import numpy as np
import pytest
import scipy.linalg

import oracle
from oracle import alt
from tests import oracle_pins as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    errs = pin(oracle.recurrent)
    assert not errs, errs


def _case(seed, lengths, Nqk, Nv, dk=8, dv=8):
    return pins._rand_case(seed, lengths, Nqk, Nv, dk, dv)


def test_linear_in_values_and_state():
    q, k, v, g, beta, s0, cu = _case(1, [6, 3], 1, 2)
    rng = np.random.default_rng(2)
    v2 = rng.standard_normal(v.shape)
    s2 = rng.standard_normal(s0.shape)
    a, b = 0.7, -1.3
    o1, t1 = oracle.recurrent(q, k, v, g, beta, s0, cu, 0.5)
    o2, t2 = oracle.recurrent(q, k, v2, g, beta, s2, cu, 0.5)
    o3, t3 = oracle.recurrent(q, k, a * v + b * v2, g, beta, a * s0 + b * s2, cu, 0.5)
    assert pins._rel(o3, a * o1 + b * o2) < 1e-13
    assert pins._rel(t3, a * t1 + b * t2) < 1e-13


def test_split_sequence_equals_whole():
    """Carrying state_out into the next call reproduces one long call."""
    q, k, v, g, beta, s0, cu = _case(3, [40], 2, 4)
    o, st = oracle.recurrent(q, k, v, g, beta, s0, cu, 0.4)
    cut = 17
    oa, sa = oracle.recurrent(q[:cut], k[:cut], v[:cut], g[:cut], beta[:cut], s0,
                              np.array([0, cut], np.int32), 0.4)
    ob, sb = oracle.recurrent(q[cut:], k[cut:], v[cut:], g[cut:], beta[cut:], sa,
                              np.array([0, 40 - cut], np.int32), 0.4)
    assert pins._rel(np.concatenate([oa, ob]), o) < 1e-14
    assert pins._rel(sb, st) < 1e-14


def test_packed_equals_separate():
    lengths = [5, 0, 9, 1]
    q, k, v, g, beta, s0, cu = _case(4, lengths, 1, 2)
    o, st = oracle.recurrent(q, k, v, g, beta, s0, cu, 0.4)
    for b in range(len(lengths)):
        t0, t1 = cu[b], cu[b + 1]
        ob, sb = oracle.recurrent(q[t0:t1], k[t0:t1], v[t0:t1], g[t0:t1], beta[t0:t1], s0[b:b + 1],
                                  np.array([0, t1 - t0], np.int32), 0.4)
        assert np.array_equal(ob, o[t0:t1])
        assert np.array_equal(sb[0], st[b])
    # a zero-length sequence returns its initial state
    assert np.array_equal(st[1], s0[1])


def test_gqa_equals_repeated_heads():
    q, k, v, g, beta, s0, cu = _case(5, [11, 4], 2, 6)
    o, st = oracle.recurrent(q, k, v, g, beta, s0, cu, 0.4)
    qr = np.repeat(q, 3, axis=1)
    kr = np.repeat(k, 3, axis=1)
    o2, st2 = oracle.recurrent(qr, kr, v, g, beta, s0, cu, 0.4)
    assert np.array_equal(o, o2) and np.array_equal(st, st2)


def test_value_permutation():
    q, k, v, g, beta, s0, cu = _case(6, [12], 1, 1)
    perm = np.random.default_rng(0).permutation(v.shape[2])
    o, st = oracle.recurrent(q, k, v, g, beta, s0, cu, 0.4)
    o2, st2 = oracle.recurrent(q, k, v[:, :, perm], g, beta, s0[:, :, perm, :], cu, 0.4)
    assert np.array_equal(o[:, :, perm], o2)
    assert np.array_equal(st[:, :, perm, :], st2)


def test_scale_is_linear():
    q, k, v, g, beta, s0, cu = _case(7, [10], 1, 1)
    o1, _ = oracle.recurrent(q, k, v, g, beta, s0, cu, 1.0)
    o2, _ = oracle.recurrent(q, k, v, g, beta, s0, cu, 0.125)
    assert pins._rel(o2, 0.125 * o1) < 1e-15


def test_state_not_symmetric_sensitive():
    """Transposing the initial state changes the result (orientation is pinned)."""
    q, k, v, g, beta, s0, cu = _case(8, [6], 1, 1)
    o1, _ = oracle.recurrent(q, k, v, g, beta, s0, cu, 0.4)
    o2, _ = oracle.recurrent(q, k, v, g, beta, np.swapaxes(s0, -1, -2).copy(), cu, 0.4)
    assert pins._rel(o1, o2) > 1e-3


# ---- facts about the chunkwise building blocks (blog post section 5(1)d, e) ----

def test_row_recurrence_inverse_matches_library():
    rng = np.random.default_rng(9)
    n = 37
    L = np.tril(rng.standard_normal((n, n)) * 0.3, -1)
    T = alt.unit_lower_inverse_rows(-L)          # (I + L)^-1
    ref = scipy.linalg.solve_triangular(np.eye(n) + L, np.eye(n), lower=True, unit_diagonal=True)
    assert np.max(np.abs(T - ref)) < 1e-12
    assert np.max(np.abs((np.eye(n) + L) @ T - np.eye(n))) < 1e-12


def test_nilpotent_series():
    rng = np.random.default_rng(10)
    n = 8
    L = np.tril(rng.standard_normal((n, n)), -1)
    series = sum(np.linalg.matrix_power(-L, p) for p in range(n))
    assert np.allclose(series, np.linalg.inv(np.eye(n) + L), atol=1e-10, rtol=1e-10)
    assert np.count_nonzero(np.linalg.matrix_power(L, n)) == 0


def test_similarity_identity():
    """(I + D L0 D^-1)^-1 D Kb = D (I + L0)^-1 Kb: one inverse serves U and W."""
    rng = np.random.default_rng(12)
    n, d = 16, 5
    gam = np.exp(np.cumsum(-rng.uniform(0, 0.5, n)))
    Dm = np.diag(gam)
    Kb = rng.standard_normal((n, d))
    K = rng.standard_normal((n, d))
    L0 = np.tril(Kb @ K.T, -1)
    lhs = np.linalg.inv(np.eye(n) + Dm @ L0 @ np.linalg.inv(Dm)) @ Dm @ Kb
    rhs = Dm @ np.linalg.inv(np.eye(n) + L0) @ Kb
    assert np.allclose(lhs, rhs, atol=1e-10)


def test_oracle_threads_reported():
    assert oracle.threads(2) == 2


def test_without_normalisation_matches_prenormalised():
    """l2norm=False on pre-normalised q, k equals l2norm=True with eps = 0."""
    q, k, v, g, beta, s0, cu = _case(13, [9], 1, 2)
    qn = q / np.linalg.norm(q, axis=-1, keepdims=True)
    kn = k / np.linalg.norm(k, axis=-1, keepdims=True)
    o1, s1 = oracle.recurrent(qn, kn, v, g, beta, s0, cu, 0.4, l2norm=False)
    o2, s2 = oracle.recurrent(q, k, v, g, beta, s0, cu, 0.4, eps=0.0)
    assert pins._rel(o1, o2) < 1e-14 and pins._rel(s1, s2) < 1e-14
    o3, _ = oracle.recurrent(q, k, v, g, beta, s0, cu, 0.4, l2norm=False)
    assert pins._rel(o3, o1) > 1e-2


def test_rel_l2_hand_values():
    """The checker every parity test relies on, on values worked by hand:
    |(1,2,2) - (1,2,4)| = 2 and |(1,2,4)| = sqrt(21); a zero reference gives
    the absolute error; equal arrays give 0; the error is symmetric in sign."""
    import math
    assert oracle.rel_l2([1.0, 2.0, 2.0], [1.0, 2.0, 4.0]) == pytest.approx(2 / math.sqrt(21), rel=1e-15)
    assert oracle.rel_l2([[3.0], [4.0]], [[0.0], [0.0]]) == pytest.approx(5.0, rel=1e-15)
    assert oracle.rel_l2(np.ones((3, 4)), np.ones((3, 4))) == 0.0
    assert oracle.rel_l2([0.0, 0.0], [3.0, 4.0]) == pytest.approx(1.0, rel=1e-15)
    assert oracle.rel_l2([-1.0, 2.0], [1.0, 2.0]) == pytest.approx(2 / math.sqrt(5), rel=1e-15)
