"""Pins for the oracle's per-row functions.

Each check compares the oracle with something other than itself: scipy's
logsumexp / softmax (library routines), numpy's first-occurrence argmax,
the total-variation identity for the acceptance rate, and brute force over
the 2^-24 uniform grid for the inverse-CDF draws.
"""
import numpy as np
import pytest
from scipy.special import logsumexp, softmax

GRID = 2 ** 24


def rows(seed, V, scale=2.0, n=2):
    rng = np.random.default_rng(seed)
    return (scale * rng.standard_normal((n, V))).astype(np.float32)


@pytest.mark.parametrize("T", [0.25, 0.6, 1.0, 1.7])
@pytest.mark.parametrize("V", [1, 7, 32, 1000])
def test_log_normalizer_matches_logsumexp(svo, T, V):
    x = rows(V, V, 3.0)[0]
    ref = logsumexp(x.astype(np.float64) / np.float64(np.float32(T)))
    assert svo.log_normalizer(x, np.float32(T)) == pytest.approx(ref, rel=1e-14, abs=1e-13)


def test_prob_matches_softmax(svo):
    x = rows(1, 50)[0]
    T = float(np.float32(0.6))
    p = softmax(x.astype(np.float64) / T)
    for y in (0, 3, 49):
        assert svo.prob(x, T, y) == pytest.approx(p[y], rel=1e-13)


def test_masked_vocabulary(svo):
    x = rows(2, 16)[0]
    x[[1, 5, 9]] = -np.inf
    p = softmax(np.where(np.isinf(x), -np.inf, x.astype(np.float64)))
    for y in range(16):
        assert svo.prob(x, 1.0, y) == pytest.approx(p[y], rel=1e-13, abs=0)
    assert svo.prob(x, 1.0, 5) == 0.0


@pytest.mark.parametrize("T", [0.6, 1.0])
@pytest.mark.parametrize("seed", range(5))
def test_alpha_is_one_minus_total_variation(svo, T, seed):
    P, Q = rows(seed, 64, 2.0)
    Td = float(np.float32(T))
    p = softmax(P.astype(np.float64) / Td)
    q = softmax(Q.astype(np.float64) / Td)
    tv = 0.5 * np.abs(p - q).sum()
    a = svo.alpha(P, Q, Td)
    assert a == pytest.approx(1.0 - tv, abs=1e-14)
    # and the acceptance probability of a draft drawn from q
    acc = sum(q[y] * min(1.0, p[y] / q[y]) for y in range(64))
    assert a == pytest.approx(acc, abs=1e-14)


def test_alpha_special_cases(svo):
    P = rows(9, 40)[0]
    assert svo.alpha(P, P, 1.0) == pytest.approx(1.0, abs=1e-15)
    A = np.full(8, -np.inf, dtype=np.float32)
    Bq = np.full(8, -np.inf, dtype=np.float32)
    A[:4] = 0.0
    Bq[4:] = 0.0
    assert svo.alpha(A, Bq, 1.0) == 0.0


def test_argmax_first_occurrence(svo):
    rng = np.random.default_rng(3)
    for _ in range(200):
        V = int(rng.integers(1, 300))
        # coarse values give many exact ties
        x = rng.integers(-3, 4, size=V).astype(np.float32)
        if rng.random() < 0.3:
            x[rng.integers(0, V, size=V // 3)] = -np.inf
        if np.all(np.isinf(x)):
            x[0] = 0.0
        assert svo.argmax(x) == int(np.argmax(x))


def test_row_valid(svo):
    assert svo.row_valid(np.array([0.0, -np.inf], dtype=np.float32))
    assert not svo.row_valid(np.array([-np.inf, -np.inf], dtype=np.float32))
    assert not svo.row_valid(np.array([0.0, np.nan], dtype=np.float32))
    assert not svo.row_valid(np.array([0.0, np.inf], dtype=np.float32))
    assert svo.row_valid(np.array([3e38, -3e38], dtype=np.float32))


def grid_intervals(fn, V):
    """For a function u -> token that is non-decreasing in u on the 2^-24
    grid, return the number of grid points mapping to each token."""
    counts = np.zeros(V, dtype=np.int64)
    lo = 0
    while lo < GRID:
        y = fn(lo / GRID)
        a, b = lo, GRID - 1
        if fn(b / GRID) == y:
            hi = GRID
        else:
            while b - a > 1:  # fn(a) == y, fn(b) != y
                mid = (a + b) // 2
                if fn(mid / GRID) == y:
                    a = mid
                else:
                    b = mid
            hi = b
        counts[y] += hi - lo
        lo = hi
    return counts


@pytest.mark.parametrize("T", [0.6, 1.0, 2.0])
@pytest.mark.parametrize("seed", range(3))
def test_sample_target_grid_mass(svo, T, seed):
    V = 6
    P = rows(seed, V, 2.0)[0]
    Td = float(np.float32(T))
    p = softmax(P.astype(np.float64) / Td)
    counts = grid_intervals(lambda u: svo.sample_target(P, Td, u)[0], V)
    assert np.all(np.abs(counts / GRID - p) <= 2.0 / GRID)


@pytest.mark.parametrize("T", [0.6, 1.0])
@pytest.mark.parametrize("seed", range(3))
def test_sample_residual_grid_mass(svo, T, seed):
    V = 6
    P, Q = rows(seed + 10, V, 2.0)
    Td = float(np.float32(T))
    p = softmax(P.astype(np.float64) / Td)
    q = softmax(Q.astype(np.float64) / Td)
    w = np.maximum(p - q, 0.0)
    counts = grid_intervals(lambda u: svo.sample_residual(P, Q, Td, u)[0], V)
    assert np.all(np.abs(counts / GRID - w / w.sum()) <= 2.0 / GRID)
    assert np.all(counts[w == 0] == 0)
    _, _, R = svo.sample_residual(P, Q, Td, 0.5)
    assert R == pytest.approx(w.sum(), abs=1e-14)


def test_residual_zero_falls_back_to_target(svo):
    P = rows(4, 5)[0]
    p = softmax(P.astype(np.float64))
    counts = grid_intervals(lambda u: svo.sample_residual(P, P, 1.0, u)[0], 5)
    assert np.all(np.abs(counts / GRID - p) <= 2.0 / GRID)


def test_draw_margin_is_distance_to_cdf_boundary(svo):
    P = rows(5, 9)[0]
    p = softmax(P.astype(np.float64))
    c = np.cumsum(p)
    for u in (0.0, 0.1, 0.5, 0.77, 1 - 2 ** -24):
        y, m = svo.sample_target(P, 1.0, u)
        assert y == int(np.searchsorted(c, u, side="right"))
        lo = u - (c[y - 1] if y > 0 else 0.0)
        hi = c[y] - u
        assert m == pytest.approx(min(lo, hi), abs=1e-15)


def test_accept_ratio(svo):
    P, Q = rows(6, 20, 2.0)
    p = softmax(P.astype(np.float64))
    q = softmax(Q.astype(np.float64))
    for d in range(20):
        keep, ratio = svo.accept(P, Q, 1.0, d, 0.5)
        assert ratio == pytest.approx(p[d] / q[d], rel=1e-13)
        assert keep == (0.5 < p[d] / q[d])
    # u = 0 is always kept when p(d) > 0; q(d) = 0 < p(d) is kept; p(d) = 0 never
    assert svo.accept(P, Q, 1.0, 3, 0.0)[0]
    Qm = Q.copy()
    Qm[2] = -np.inf
    keep, ratio = svo.accept(P, Qm, 1.0, 2, 1 - 2 ** -24)
    assert keep and np.isinf(ratio)
    Pm = P.copy()
    Pm[2] = -np.inf
    assert not svo.accept(Pm, Q, 1.0, 2, 0.0)[0]
