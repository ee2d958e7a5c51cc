"""Pins for the oracle's drafter confidence and D-cut keep-ratio choice
("AngelSpec: specialize the drafter...", section "D-cut": Figure 3 panels 1
and 2, equations A-hat and K_rho, and the budget widget).  Each pin checks the
oracle against something other than itself: a library softmax, invariants of
a probability, hand-computed interpolation values, or a brute force over
every prefix-closed allocation."""
import itertools
import math

import numpy as np
import pytest
from scipy.special import softmax


def rows(rng, n, V, scale=3.0):
    return (rng.normal(size=(n, V)) * scale).astype(np.float32)


# ---- drafter confidence ------------------------------------------------------

def test_confidence_matches_library_softmax(svo):
    """conf[r, k] = softmax(row / T)[d] with the row found through draft_row0
    (rows are distinct, so a wrong row or token index fails)."""
    rng = np.random.default_rng(1)
    B, D, V = 3, 4, 97
    X = rows(rng, 20, V)
    dr0 = np.array([0, 7, 13])
    tok = rng.integers(0, V, size=(B, D)).astype(np.int32)
    T = np.array([1.0, 0.6, 1.7], dtype=np.float32)
    conf = svo.draft_confidence(X, dr0, tok, T)
    for r in range(B):
        for k in range(D):
            ref = softmax(X[dr0[r] + k].astype(np.float64) / float(T[r]))[tok[r, k]]
            assert conf[r, k] == pytest.approx(ref, rel=1e-6)


def test_confidence_sums_to_one_over_tokens(svo):
    """Scoring every token of one row gives a probability distribution."""
    rng = np.random.default_rng(2)
    V = 64
    X = rows(rng, 1, V)
    tok = np.arange(V, dtype=np.int32).reshape(V, 1)
    dr0 = np.zeros(V, dtype=np.int64)
    conf = svo.draft_confidence(X, dr0, tok, np.full(V, 0.8, np.float32))
    assert float(conf.astype(np.float64).sum()) == pytest.approx(1.0, abs=1e-6)


def test_confidence_greedy_drafter_reads_t_as_one(svo):
    rng = np.random.default_rng(3)
    X = rows(rng, 4, 50)
    tok = np.array([[3, 9, 11, 40]], dtype=np.int32)
    c0 = svo.draft_confidence(X, [0], tok, np.array([0.0], np.float32))
    c1 = svo.draft_confidence(X, [0], tok, np.array([1.0], np.float32))
    assert np.array_equal(c0, c1)


def test_confidence_shift_invariant_and_uniform_row(svo):
    rng = np.random.default_rng(4)
    X = rows(rng, 2, 40)
    tok = np.array([[5, 6]], dtype=np.int32)
    T = np.array([1.3], np.float32)
    a = svo.draft_confidence(X, [0], tok, T)
    b = svo.draft_confidence(X + np.float32(8.0), [0], tok, T)
    assert np.allclose(a, b, rtol=1e-6)
    U = np.zeros((1, 40), np.float32)
    u = svo.draft_confidence(U, [0], np.array([[17]], np.int32), np.array([0.5], np.float32))
    assert u[0, 0] == pytest.approx(1.0 / 40, rel=1e-7)


def test_confidence_masks_depth_and_invalid_inputs(svo):
    V = 16
    X = np.zeros((8, V), np.float32)
    X[0, 3] = -np.inf                      # a masked token: probability 0
    X[1, :] = -np.inf                      # every token masked: invalid row
    X[2, 4] = np.nan                       # NaN: invalid row
    X[3, 5] = np.inf                       # +inf: invalid row
    tok = np.array([[3, 0, 0, 0], [1, 99, 0, 0]], dtype=np.int32)
    T = np.array([1.0, 1.0], np.float32)
    conf = svo.draft_confidence(X, [0, 4], tok, T, depth=np.array([4, 2]))
    assert conf[0, 0] == 0.0
    assert np.isnan(conf[0, 1]) and np.isnan(conf[0, 2]) and np.isnan(conf[0, 3])
    assert conf[1, 0] == pytest.approx(1.0 / V, rel=1e-7)
    assert np.isnan(conf[1, 1])            # token out of range
    assert conf[1, 2] == 0.0 and conf[1, 3] == 0.0   # past the depth
    bad = svo.draft_confidence(X, [0, 4], tok, np.array([-1.0, np.nan], np.float32))
    assert np.isnan(bad).all()
    bad_depth = svo.draft_confidence(X, [0, 4], tok, T, depth=np.array([5, -1]))
    assert np.isnan(bad_depth).all()


# ---- keep-ratio choice -------------------------------------------------------

def test_table_latency_interpolation_hand_values(svo):
    tb = [8, 32, 64]
    tl = [[1.0, 2.0], [4.0, 8.0], [10.0, 20.0]]
    # below, at and above the ends, and a third of the way from 8 to 32 (B = 16)
    assert svo.table_latency(tb, tl, 0, 1) == 1.0
    assert svo.table_latency(tb, tl, 1, 8) == 2.0
    assert svo.table_latency(tb, tl, 1, 100) == 20.0
    assert svo.table_latency(tb, tl, 0, 16) == pytest.approx(2.0, rel=1e-15)
    assert svo.table_latency(tb, tl, 1, 48) == pytest.approx(14.0, rel=1e-15)


def prefix_scores(conf):
    return np.cumprod(np.clip(conf, 0, 1).astype(np.float32), axis=1, dtype=np.float32)


def brute_choice(conf, ratios, lat):
    """Independent reading of the choice: for each ratio, the best utility
    over every prefix-closed allocation that keeps exactly K positions."""
    B, D = conf.shape
    s = prefix_scores(conf).astype(np.float64)
    best_j, best_tp, Ks = -1, 0.0, []
    for j, rho in enumerate(ratios):
        K = math.ceil(rho * B * D)
        Ks.append(K)
        u = max(sum(s[r, :a[r]].sum() for r in range(B))
                for a in itertools.product(range(D + 1), repeat=B) if sum(a) == K)
        tp = (B + u) / lat[j]
        if best_j < 0 or tp > best_tp:
            best_j, best_tp = j, tp
    return best_j, Ks


def test_ratio_choice_brute_force(svo):
    rng = np.random.default_rng(5)
    ratios = [0.25, 0.5, 0.75, 1.0]
    for _ in range(40):
        B, D = int(rng.integers(1, 4)), int(rng.integers(1, 5))
        conf = rng.uniform(0, 1, size=(B, D)).astype(np.float32)
        lat = rng.uniform(1.0, 3.0, size=4)
        lat.sort()                         # costlier with a larger budget
        res = svo.select_budget_ratio(conf, ratios, [B], lat.reshape(1, 4).astype(np.float32))
        j, Ks = brute_choice(conf, ratios, lat.astype(np.float32).astype(np.float64))
        assert res["choice"] == j
        assert res["K"] == Ks[j]
        assert int(res["depth"].sum()) == Ks[j]


def test_ratio_choice_special_cases(svo):
    rng = np.random.default_rng(6)
    conf = rng.uniform(0.2, 1, size=(6, 8)).astype(np.float32)
    ratios = [0.25, 0.5, 0.75, 1.0]
    # equal latencies: more budget never lowers the projected tokens
    res = svo.select_budget_ratio(conf, ratios, [6], [[2.0, 2.0, 2.0, 2.0]])
    assert res["choice"] == 3 and res["K"] == 48
    # the budget widget's shape: 6 requests x 8 positions at rho = 1/2 keep 24
    res = svo.select_budget_ratio(conf, [0.5], [6], [[1.0]])
    assert res["K"] == 24 and int(res["depth"].sum()) == 24
    # zero confidence: every ratio projects B tokens; the cheapest wins, and
    # on a tie the first listed
    z = np.zeros((6, 8), np.float32)
    res = svo.select_budget_ratio(z, ratios, [6], [[3.0, 1.0, 1.0, 2.0]])
    assert res["choice"] == 1
    assert res["projected"][1] == pytest.approx(6.0, rel=1e-15)
    # depth limits bound N
    res = svo.select_budget_ratio(conf, [1.0], [6], [[1.0]], max_depth=np.array([0, 1, 2, 3, 4, 5]))
    assert res["K"] == 15 and list(res["depth"]) == [0, 1, 2, 3, 4, 5]


def test_ratio_choice_rejects_bad_tables(svo):
    conf = np.ones((2, 2), np.float32)
    with pytest.raises(ValueError):
        svo.select_budget_ratio(conf, [0.5, 1.5], [2], [[1.0, 1.0]])
    with pytest.raises(ValueError):
        svo.select_budget_ratio(conf, [0.5], [4, 2], [[1.0], [1.0]])
    with pytest.raises(ValueError):
        svo.select_budget_ratio(conf, [0.5], [2], [[0.0]])
