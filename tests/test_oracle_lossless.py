"""Losslessness of the oracle's verification, by exhaustive enumeration.

The pages state that speculative verification only emits what the target
would have sampled (ai.thesatyajit.com, intro; tradepoint.io, "Why one
universal drafter underperforms": lossless rejection sampling; newx.sg,
Abstract: the target distribution is unchanged).  For a target whose rows do
not depend on the prefix, that means: given that position k is reached with
any prefix h, the token emitted at k is distributed as p_k.

The enumeration drives the oracle's composed per-request function with every
draft tuple (weighted by prod q_k(d_k), computed here with scipy) and every
outcome of the uniforms on the 2^-24 grid (each accept test and each draw is
monotone in its uniform, so exact grid counts come from binary search).
Probabilities are therefore exact up to the 2^-24 grid.
"""
import itertools

import numpy as np
import pytest
from scipy.special import softmax

GRID = 2 ** 24


def instance(seed, n, V, scale=1.5):
    rng = np.random.default_rng(seed)
    P = (scale * rng.standard_normal((n + 1, V))).astype(np.float32)
    Q = (P[:n] + rng.standard_normal((n, V))).astype(np.float32)
    return P, Q


def accept_count(svo, P, Q, T, d):
    """Number of grid uniforms for which the draft token d is kept."""
    lo, hi = 0, GRID  # keep(u) is true on [0, a) of the grid
    if not svo.accept(P, Q, T, d, 0.0)[0]:
        return 0
    if svo.accept(P, Q, T, d, (GRID - 1) / GRID)[0]:
        return GRID
    while hi - lo > 1:  # keep(lo) true, keep(hi) false
        mid = (lo + hi) // 2
        if svo.accept(P, Q, T, d, mid / GRID)[0]:
            lo = mid
        else:
            hi = mid
    return hi


def grid_intervals(fn):
    out = {}
    lo = 0
    while lo < GRID:
        y = fn(lo / GRID)
        if fn((GRID - 1) / GRID) == y:
            hi = GRID
        else:
            a, b = lo, GRID - 1
            while b - a > 1:
                mid = (a + b) // 2
                if fn(mid / GRID) == y:
                    a = mid
                else:
                    b = mid
            hi = b
        out[y] = out.get(y, 0) + (hi - lo)
        lo = hi
    return out


def enumerate_outputs(svo, P, Q, T):
    """Exact grid probability of every emitted sequence of the composed
    per-request function."""
    n, V = Q.shape
    q = [softmax(Q[k].astype(np.float64) / T) for k in range(n)]
    acc = np.array([[accept_count(svo, P[k], Q[k], T, d) for d in range(V)] for k in range(n)],
                   dtype=np.float64)
    probs = {}
    for d in itertools.product(range(V), repeat=n):
        wd = float(np.prod([q[k][d[k]] for k in range(n)])) if n else 1.0
        if wd == 0.0:
            continue
        for j in range(n + 1):
            pr = wd
            for k in range(j):
                pr *= acc[k][d[k]] / GRID
            if j < n:
                pr *= 1.0 - acc[j][d[j]] / GRID
            if pr == 0.0:
                continue
            ua = np.zeros(max(n, 1))
            if j < n:
                ua[j] = acc[j][d[j]] / GRID  # first grid uniform that rejects

            def last_token(us_j, j=j, d=d, ua=ua):
                us = np.zeros(n + 1)
                us[j] = us_j
                tau, out, _, _, _ = svo.verify_request(P, Q, np.array(d), T, ua, us)
                assert tau == j
                assert list(out[:j]) == list(d[:j])
                return int(out[j])

            for y, cnt in grid_intervals(last_token).items():
                seq = tuple(d[:j]) + (y,)
                probs[seq] = probs.get(seq, 0.0) + pr * cnt / GRID
    return probs


CASES = [(3, 4, 1.0, 0), (3, 3, 0.6, 1), (2, 8, 1.0, 2), (2, 6, 1.7, 3), (1, 8, 0.6, 4),
         (0, 5, 1.0, 5), (3, 2, 1.0, 6)]


@pytest.mark.parametrize("n,V,T,seed", CASES)
def test_enumeration_emits_target_distribution(svo, n, V, T, seed):
    T = float(np.float32(T))
    P, Q = instance(seed, n, V)
    p = [softmax(P[k].astype(np.float64) / T) for k in range(n + 1)]
    probs = enumerate_outputs(svo, P, Q, T)
    tol = 4.0 * (n + 2) / GRID
    assert sum(probs.values()) == pytest.approx(1.0, abs=tol)
    # For every position k and reached prefix h, the emitted token ~ p_k.
    for k in range(n + 1):
        for h in itertools.product(range(V), repeat=k):
            m = np.zeros(V)
            for seq, pr in probs.items():
                if len(seq) > k and tuple(seq[:k]) == h:
                    m[seq[k]] += pr
            reach = m.sum()
            assert np.all(np.abs(m - reach * p[k]) <= tol), (k, h)
    # The chance of reaching position k is prod_{i<k} alpha_i (alpha = 1 - TV),
    # and the mean number of accepted drafts is sum_m prod_{i<=m} alpha_i.
    alphas = [svo.alpha(P[i], Q[i], T) for i in range(n)]
    for k in range(n + 1):
        reach_k = sum(pr for seq, pr in probs.items() if len(seq) > k)
        assert reach_k == pytest.approx(float(np.prod(alphas[:k])), abs=tol)
    mean_tau = sum(pr * (len(seq) - 1) for seq, pr in probs.items())
    assert mean_tau == pytest.approx(svo.expected_accepted(alphas), abs=tol * (n + 1))


def test_c1_position_marginals(svo):
    """The tiny exhaustive workload (2 requests x 3 drafts, V = 32, fp32,
    P ~ N(0, 2^2), Q = P + N(0, 1), T = 1): per position, the emitted token
    given the position is reached is distributed as p_k, from the oracle's
    accept and draw functions over every draft token and grid uniform."""
    rng = np.random.default_rng(100)
    T = 1.0
    for _ in range(2):
        P = (2.0 * rng.standard_normal((4, 32))).astype(np.float32)
        Q = (P[:3] + rng.standard_normal((3, 32))).astype(np.float32)
        for k in range(3):
            p = softmax(P[k].astype(np.float64))
            q = softmax(Q[k].astype(np.float64))
            acc = np.array([accept_count(svo, P[k], Q[k], T, d) for d in range(32)]) / GRID
            res = grid_intervals(lambda u: svo.sample_residual(P[k], Q[k], T, u)[0])
            resv = np.zeros(32)
            for y, c in res.items():
                resv[y] = c / GRID
            reject = float(np.sum(q * (1.0 - acc)))
            emitted = q * acc + reject * resv
            assert np.all(np.abs(emitted - p) <= 4.0 / GRID)
            assert float(np.sum(q * acc)) == pytest.approx(svo.alpha(P[k], Q[k], T), abs=2.0 / GRID)
        bonus = grid_intervals(lambda u: svo.sample_target(P[3], T, u)[0])
        pb = softmax(P[3].astype(np.float64))
        for y in range(32):
            assert abs(bonus.get(y, 0) / GRID - pb[y]) <= 2.0 / GRID
