"""Pins for the oracle's verification budget (ai.thesatyajit.com, section
"D-cut": Figure 3, equations A-hat and K_rho, and the budget widget)."""
import itertools
import os

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def golden(name):
    with open(os.path.join(HERE, "golden", name)) as f:
        return [l.split() for l in f if l.strip() and not l.startswith("#")]


def test_k_rho_hand_values(svo):
    for B, D, rho, K in golden("k_rho.txt"):
        assert svo.k_rho(int(B), int(D), float(rho)) == int(K)


def scores(conf):
    # prefix products in float32, left to right (numpy's cumprod, a library
    # routine, accumulates in the array's dtype)
    return np.cumprod(np.clip(np.nan_to_num(conf, nan=0.0), 0, 1).astype(np.float32), axis=1,
                      dtype=np.float32)


def lexsort_selection(conf, K, max_depth=None):
    B, D = conf.shape
    s = scores(conf)
    md = np.full(B, D) if max_depth is None else np.asarray(max_depth)
    rr, kk = np.meshgrid(np.arange(B), np.arange(D), indexing="ij")
    valid = kk < md[:, None]
    sv, rv, kv = s[valid], rr[valid], kk[valid]
    order = np.lexsort((kv, rv, -sv.astype(np.float64)))
    K = max(0, min(K, sv.size))
    depth = np.bincount(rv[order[:K]], minlength=B)
    return depth, float(sv[order[:K]].astype(np.float64).sum()), float(
        sv.astype(np.float64).sum())


def test_topk_equals_library_sort_selection(svo):
    rng = np.random.default_rng(20)
    for trial in range(300):
        B = int(rng.integers(1, 9))
        D = int(rng.integers(1, 9))
        conf = rng.beta(2, 2, size=(B, D)).astype(np.float32)
        # exact ties: confidence 1 repeats a score, 0 zeroes the tail
        conf[rng.random((B, D)) < 0.15] = 1.0
        conf[rng.random((B, D)) < 0.05] = 0.0
        if trial % 3 == 0:  # identical requests tie across requests
            conf[:] = conf[0]
        K = int(rng.integers(0, B * D + 3))
        md = rng.integers(0, D + 1, size=B).astype(np.int32) if trial % 4 == 1 else None
        res = svo.allocate_budget(conf, K, md)
        depth, kept, total = lexsort_selection(conf, K, md)
        assert list(res["depth"]) == list(depth)
        assert res["utility"][0] == pytest.approx(kept, rel=1e-12, abs=1e-30)
        assert res["utility"][1] == pytest.approx(total, rel=1e-12, abs=1e-30)
        assert list(res["draft_row0"]) == list(np.concatenate([[0], np.cumsum(depth)[:-1]]))
        assert list(res["target_row0"]) == list(
            np.concatenate([[0], np.cumsum(depth + 1)[:-1]]))


def test_topk_maximises_retained_utility_brute_force(svo):
    """Among every allocation that keeps a prefix of each request and spends
    exactly K positions, the global top-K attains the largest sum of
    prefix-confidence products (equation A-hat summed over the batch)."""
    rng = np.random.default_rng(21)
    for _ in range(60):
        B = int(rng.integers(1, 5))
        D = int(rng.integers(1, 5))
        conf = rng.uniform(0, 1, size=(B, D)).astype(np.float32)
        s = scores(conf).astype(np.float64)
        for K in range(0, B * D + 1):
            best = -1.0
            for alloc in itertools.product(range(D + 1), repeat=B):
                if sum(alloc) != K:
                    continue
                best = max(best, sum(s[r, :alloc[r]].sum() for r in range(B)))
            res = svo.allocate_budget(conf, K)
            assert res["utility"][0] == pytest.approx(best, rel=1e-12)
            assert res["depth"].sum() == K


def test_budget_invariants(svo):
    rng = np.random.default_rng(22)
    B, D = 64, 16
    conf = np.empty((B, D), np.float32)
    conf[:32] = rng.beta(8, 2, size=(32, D))
    conf[32:] = rng.beta(3, 3, size=(32, D))
    for K in (0, 1, 63, 64, 256, 512, 1023, 1024, 5000, -5):
        res = svo.allocate_budget(conf, K)
        assert res["depth"].sum() == min(max(K, 0), B * D)
        assert np.all((res["depth"] >= 0) & (res["depth"] <= D))
        fixed = svo.fixed_depth(B, D, min(max(K, 0), B * D))
        s = scores(conf).astype(np.float64)
        u_fixed = sum(s[r, :fixed[r]].sum() for r in range(B))
        assert res["utility"][0] >= u_fixed - 1e-12
    full = svo.allocate_budget(conf, B * D)
    assert np.all(full["depth"] == D)
    # prefix closure in score order: every kept position outranks every cut one
    res = svo.allocate_budget(conf, 256)
    s = scores(conf)
    kept_min = min(s[r, k] for r in range(B) for k in range(res["depth"][r]))
    cut_max = max([s[r, k] for r in range(B) for k in range(res["depth"][r], D)] + [0.0])
    assert kept_min >= cut_max
    # code-like requests (high confidence) keep more depth than chat-like ones
    assert res["depth"][:32].mean() > res["depth"][32:].mean()


def test_budget_float32_products_and_denormals(svo):
    # products that underflow into float32 subnormals and to zero still order
    # by value, then by request and position
    conf = np.array([[1e-20, 1e-20, 1e-5, 0.5], [1e-19, 1e-19, 1.0, 1.0]], np.float32)
    s = scores(conf)
    assert s[0, 1] == np.float32(1e-20) * np.float32(1e-20)  # 0 in float32
    for K in range(9):
        res = svo.allocate_budget(conf, K)
        depth, _, _ = lexsort_selection(conf, K)
        assert list(res["depth"]) == list(depth)


def test_clamping_of_bad_confidences(svo):
    conf = np.array([[np.nan, 0.9], [1.5, -0.2], [0.5, 0.5]], np.float32)
    res = svo.allocate_budget(conf, 3)
    # row 0 scores (0, 0), row 1 scores (1, 0), row 2 scores (0.5, 0.25)
    assert list(res["depth"]) == [0, 1, 2]


def test_widget_global_beats_fixed(svo):
    """Budget widget: 6 requests x 8 positions, K = 24 of 48.  The page
    prints 72.6% (global) vs 66.5% (fixed) retained utility but not the
    confidences behind them, so those two values are parity unpinned; the
    ordering global >= fixed holds for any confidences."""
    rng = np.random.default_rng(23)
    for _ in range(50):
        conf = np.concatenate([rng.beta(8, 2, size=(3, 8)), rng.beta(3, 3, size=(3, 8))]).astype(
            np.float32)
        res = svo.allocate_budget(conf, 24)
        fixed = svo.fixed_depth(6, 8, 24)
        s = scores(conf).astype(np.float64)
        assert res["utility"][0] >= sum(s[r, :fixed[r]].sum() for r in range(6)) - 1e-12


def test_fixed_depth_hand_values(svo):
    """The fixed-depth baseline against hand values (tests/golden/fixed_depth.txt):
    the remainder goes to the first K mod B requests, K past B D clamps to D,
    K <= 0 keeps nothing, B = 0 is empty."""
    for row in golden("fixed_depth.txt"):
        B, D, K = int(row[0]), int(row[1]), int(row[2])
        want = [int(x) for x in row[4:]]
        assert list(svo.fixed_depth(B, D, K)) == want, row
        if B > 0:
            res = svo.fixed_depth_budget(np.full((B, D), 0.5, np.float32), K)
            assert list(res["depth"]) == want
            assert list(res["draft_row0"]) == list(np.concatenate([[0], np.cumsum(want)[:-1]]))
            assert list(res["target_row0"]) == list(
                np.concatenate([[0], np.cumsum(np.asarray(want) + 1)[:-1]]))


def test_fixed_and_global_utility_hand_values(svo):
    conf = np.array([[0.75, 0.75, 0.5], [0.25, 1.0, 1.0]], np.float32)
    for K, kind, d0, d1, kept, total in golden("fixed_vs_global_utility.txt"):
        res = (svo.fixed_depth_budget if kind == "fixed" else svo.allocate_budget)(conf, int(K))
        assert list(res["depth"]) == [int(d0), int(d1)]
        assert res["utility"][0] == float(kept)
        assert res["utility"][1] == float(total)


def test_fixed_depth_utility_against_library_products(svo):
    """Kept and total utility of the fixed baseline equal sums of numpy's
    float32 cumprod over the kept prefixes; retained utility global >= fixed."""
    rng = np.random.default_rng(24)
    for _ in range(100):
        B = int(rng.integers(1, 12))
        D = int(rng.integers(1, 12))
        conf = rng.beta(3, 2, size=(B, D)).astype(np.float32)
        conf[rng.random((B, D)) < 0.05] = np.nan
        K = int(rng.integers(-2, B * D + 4))
        res = svo.fixed_depth_budget(conf, K)
        s = scores(conf).astype(np.float64)
        want = svo.fixed_depth(B, D, K)
        assert list(res["depth"]) == list(want)
        assert res["utility"][0] == pytest.approx(sum(s[r, :want[r]].sum() for r in range(B)),
                                                  rel=1e-12, abs=1e-30)
        assert res["utility"][1] == pytest.approx(s.sum(), rel=1e-12, abs=1e-30)
        glob = svo.allocate_budget(conf, K)
        assert glob["utility"][0] >= res["utility"][0] - 1e-12


def test_accept_accumulate_hand_values(svo):
    rows = {r[0]: [float(x) for x in r[1:]] for r in golden("accept_accumulate.txt")}
    depth = np.array([3, 3, 2, 0], np.int32)
    tau = np.array([0, 3, 1, 0], np.int32)
    alpha = np.array([[0.5, 0.5, 0.5], [1, 1, 1], [0.5, 1, 0], [0, 0, 0]], np.float64)
    acc, summ = svo.accept_accumulate(depth, alpha, tau, 3)
    assert list(acc) == rows["accum1"]
    assert list(summ) == rows["summary"]
    acc, summ = svo.accept_accumulate(depth, alpha, tau, 3, acc)
    assert list(acc) == rows["accum2"]
    assert list(summ) == rows["summary"]


def test_accept_accumulate_printed_mal_relation(svo):
    """With every request verified at depth D, MAL = 1 + D x mean acceptance
    and MAL = 1 + sum of the position-wise acceptances, the relation of the
    printed pairs 2.58 / 52.8% and 2.99 / 66.4% at D = 3 ([T] "The MTP
    path"; tests/golden/mtp_ttt_mal.txt)."""
    rng = np.random.default_rng(25)
    D = 3
    acc = None
    for _ in range(50):
        B = int(rng.integers(1, 40))
        tau = rng.integers(0, D + 1, size=B).astype(np.int32)
        acc, summ = svo.accept_accumulate(np.full(B, D, np.int32), None, tau, D, acc)
    assert summ[0] == pytest.approx(1 + D * summ[2], rel=1e-12)
    assert summ[0] == pytest.approx(1 + summ[3:].sum(), rel=1e-12)
    assert np.all(np.diff(summ[3:]) <= 0)     # P(tau >= k) does not increase with k
