"""Pins for the oracle's batch function: the T = 0 arg-max chain, special
cases with closed forms, composition with the Philox stream, the expected
accepted length by Monte Carlo, and the statistics definitions against the
figures the pages print."""
import os

import numpy as np
import pytest
from scipy.special import softmax

HERE = os.path.dirname(os.path.abspath(__file__))


def padded_batch(rng, B, D, V, scale=2.0, noise=1.0):
    P = (scale * rng.standard_normal((B, D + 1, V))).astype(np.float32)
    Q = (P[:, :D] + noise * rng.standard_normal((B, D, V))).astype(np.float32)
    tr0 = np.arange(B, dtype=np.int64) * (D + 1)
    dr0 = np.arange(B, dtype=np.int64) * D
    return P, Q, tr0, dr0


# ---- T = 0 ----------------------------------------------------------------

def test_t0_emits_target_argmax_chain(svo):
    """At T = 0 (the pages' greedy setting, tradepoint.io "The MTP path") the
    emitted block is [argmax P_0, ..., argmax P_tau] with tau the first
    position whose draft differs from the target arg max (numpy's
    first-occurrence argmax on tie-heavy rows)."""
    rng = np.random.default_rng(7)
    B, D, V = 40, 6, 50
    P = rng.integers(-4, 5, size=(B, D + 1, V)).astype(np.float32)  # many ties
    Q = P[:, :D].copy()
    tr0 = np.arange(B, dtype=np.int64) * (D + 1)
    dr0 = np.arange(B, dtype=np.int64) * D
    am = np.argmax(P, axis=-1)
    tokens = am[:, :D].astype(np.int32).copy()
    # perturb some drafts so that mismatches happen at varied positions
    flip = rng.random((B, D)) < 0.25
    tokens[flip] = (tokens[flip] + 1 + rng.integers(0, V - 1, size=flip.sum())) % V
    depth = rng.integers(0, D + 1, size=B).astype(np.int32)
    res = svo.verify_batch(P.reshape(-1, V), Q.reshape(-1, V), tr0, dr0, tokens, depth,
                           np.zeros(B, np.float32), D_max=D)
    for r in range(B):
        n = depth[r]
        mism = [k for k in range(n) if tokens[r, k] != am[r, k]]
        tau = mism[0] if mism else n
        assert res["accepted_len"][r] == tau
        assert res["num_out"][r] == tau + 1
        assert list(res["out_tokens"][r, : tau + 1]) == list(am[r, : tau + 1])
        assert np.all(res["out_tokens"][r, tau + 1:] == -1)
        assert list(res["alpha"][r, :n]) == [1.0 if tokens[r, k] == am[r, k] else 0.0
                                            for k in range(n)]
    assert np.all(res["draws"] == 0)


def test_t0_draft_rows_not_needed(svo):
    rng = np.random.default_rng(8)
    B, D, V = 3, 2, 10
    P = rng.standard_normal((B * (D + 1), V)).astype(np.float32)
    tr0 = np.arange(B, dtype=np.int64) * (D + 1)
    tokens = np.argmax(P.reshape(B, D + 1, V)[:, :D], -1).astype(np.int32)
    res = svo.verify_batch(P, None, tr0, None, tokens, np.full(B, D, np.int32),
                           np.zeros(B, np.float32), D_max=D)
    assert np.all(res["accepted_len"] == D)


def test_sampling_request_without_draft_rows_is_invalid(svo):
    """Draft rows may be absent only when no request samples: a T > 0 request
    with drafted positions is then reported as an invalid row (nothing
    emitted), while greedy requests and bonus-only requests (depth 0, which
    read no draft row) are verified as usual."""
    rng = np.random.default_rng(9)
    B, D, V = 3, 2, 10
    P = rng.standard_normal((B * (D + 1), V)).astype(np.float32)
    tr0 = np.arange(B, dtype=np.int64) * (D + 1)
    tokens = np.argmax(P.reshape(B, D + 1, V)[:, :D], -1).astype(np.int32)
    depth = np.array([D, D, 0], np.int32)
    res = svo.verify_batch(P, None, tr0, None, tokens, depth,
                           np.array([0.0, 1.0, 1.0], np.float32), D_max=D)
    assert res["bits"].tolist() == [0, svo.BIT_BAD_ROW, 0]
    assert res["accepted_len"][0] == D and res["num_out"][0] == D + 1
    assert res["num_out"][1] == 0 and np.all(res["out_tokens"][1] == -1)
    assert res["accepted_len"][2] == 0 and res["num_out"][2] == 1
    assert 0 <= res["out_tokens"][2, 0] < V


# ---- closed-form special cases --------------------------------------------

def test_identical_draft_accepts_everything(svo):
    """q = p: every test passes (u < 1 <= p/q), alpha = 1, tau = n, and the
    block ends with a bonus draw from the last target row."""
    rng = np.random.default_rng(9)
    B, D, V = 5, 4, 33
    P = (2.0 * rng.standard_normal((B, D + 1, V))).astype(np.float32)
    Q = P[:, :D].copy()
    tr0 = np.arange(B, dtype=np.int64) * (D + 1)
    dr0 = np.arange(B, dtype=np.int64) * D
    tokens = rng.integers(0, V, size=(B, D)).astype(np.int32)
    for seed in range(5):
        res = svo.verify_batch(P.reshape(-1, V), Q.reshape(-1, V), tr0, dr0, tokens,
                               np.full(B, D, np.int32), np.ones(B, np.float32), seed=seed,
                               D_max=D)
        assert np.all(res["accepted_len"] == D)
        assert np.allclose(res["alpha"], 1.0, atol=1e-15)
        for r in range(B):
            assert list(res["out_tokens"][r, :D]) == list(tokens[r])
            _, us = svo.uniforms(seed, r, 0, D)
            y, _ = svo.sample_target(P[r, D], 1.0, us)
            assert res["out_tokens"][r, D] == y


def test_disjoint_supports_reject_first_position(svo):
    """p and q on disjoint supports: alpha = 0, the first draft is always
    rejected and the correction is drawn from p itself (max(0, p - q) = p)."""
    B, D, V = 4, 3, 12
    P = np.full((B, D + 1, V), -np.inf, np.float32)
    Q = np.full((B, D, V), -np.inf, np.float32)
    rng = np.random.default_rng(10)
    P[:, :, :6] = rng.standard_normal((B, D + 1, 6))
    Q[:, :, 6:] = rng.standard_normal((B, D, 6))
    tokens = np.full((B, D), 7, np.int32)
    tr0 = np.arange(B, dtype=np.int64) * (D + 1)
    dr0 = np.arange(B, dtype=np.int64) * D
    res = svo.verify_batch(P.reshape(-1, V), Q.reshape(-1, V), tr0, dr0, tokens,
                           np.full(B, D, np.int32), np.ones(B, np.float32), D_max=D)
    assert np.all(res["accepted_len"] == 0)
    assert np.all(res["alpha"] == 0.0)
    for r in range(B):
        _, us = svo.uniforms(0, r, 0, 0)
        p = softmax(P[r, 0, :6].astype(np.float64))
        y = int(np.searchsorted(np.cumsum(p), us * p.sum(), side="right"))
        assert res["out_tokens"][r, 0] == y


def test_zero_depth_is_bonus_only(svo):
    rng = np.random.default_rng(11)
    B, D, V = 3, 4, 20
    P, Q, tr0, dr0 = padded_batch(rng, B, D, V)
    tokens = rng.integers(0, V, size=(B, D)).astype(np.int32)
    res = svo.verify_batch(P.reshape(-1, V), Q.reshape(-1, V), tr0, dr0, tokens,
                           np.zeros(B, np.int32), np.ones(B, np.float32), D_max=D)
    assert np.all(res["accepted_len"] == 0)
    assert np.all(res["num_out"] == 1)
    for r in range(B):
        _, us = svo.uniforms(0, r, 0, 0)
        assert res["out_tokens"][r, 0] == svo.sample_target(P[r, 0], 1.0, us)[0]


def test_one_hot_target_is_deterministic(svo):
    """A target row with one finite logit: any T > 0 emits that token."""
    B, D, V = 2, 2, 9
    P = np.full((B, D + 1, V), -np.inf, np.float32)
    P[:, :, 4] = 0.0
    Q = np.zeros((B, D, V), np.float32)
    tokens = np.full((B, D), 4, np.int32)
    tr0 = np.arange(B, dtype=np.int64) * (D + 1)
    dr0 = np.arange(B, dtype=np.int64) * D
    for seed in range(10):
        res = svo.verify_batch(P.reshape(-1, V), Q.reshape(-1, V), tr0, dr0, tokens,
                               np.full(B, D, np.int32), np.full(B, 0.7, np.float32),
                               seed=seed, D_max=D)
        assert np.all(res["out_tokens"][:, : D + 1] == 4)


def test_invalid_inputs_are_flagged(svo):
    import oracle
    rng = np.random.default_rng(12)
    B, D, V = 4, 2, 8
    P, Q, tr0, dr0 = padded_batch(rng, B, D, V)
    tokens = rng.integers(0, V, size=(B, D)).astype(np.int32)
    tokens[0, 1] = V          # bad token
    P[1, 2, 3] = np.nan       # bad target (bonus) row
    Q[2, 0, :] = -np.inf      # all -inf draft row
    depth = np.array([2, 2, 2, 3], np.int32)  # depth 3 > D_max
    res = svo.verify_batch(P.reshape(-1, V), Q.reshape(-1, V), tr0, dr0, tokens, depth,
                           np.ones(B, np.float32), D_max=D)
    assert res["bits"][0] == oracle.BIT_BAD_TOKEN
    assert res["bits"][1] == oracle.BIT_BAD_ROW
    assert res["bits"][2] == oracle.BIT_BAD_ROW
    assert res["bits"][3] == oracle.BIT_BAD_DEPTH
    assert np.all(res["num_out"] == 0)
    assert np.all(res["out_tokens"] == -1)


def test_temperature_domain_scaled_maximum(svo):
    """T > 0 is in the verifier's domain while every verified row's maximum m
    has |m * fl(log2(e)/T)| < 2^24 in float32.  Hand values: at T = 1e-5,
    fl(log2(e)/T) = 144269.5..., so a row maximum of 100 scales to 1.4427e7
    (valid) and 120 to 1.7312e7 (past 2^24 = 16777216); T = 1e-37 puts any
    maximum above 1.2e-30 past it.  Greedy T = 0 has no such limit."""
    import oracle
    B, D, V = 6, 2, 16
    P = np.zeros((B, D + 1, V), np.float32)
    Q = np.zeros((B, D, V), np.float32)
    P[:, :, 3] = 100.0
    Q[:, :, 3] = 100.0
    P[1, 2, 5] = 120.0          # r1: the bonus row's maximum scales past 2^24
    Q[2, 1, 6] = -120.0         # r2: a draft row's minimum does not matter ...
    Q[3, 1, :] = -120.0         # r3: ... but an all -120 draft row's maximum does
    temps = np.array([1e-5, 1e-5, 1e-5, 1e-5, 1e-37, 1e-37], np.float32)
    P[5] = 1e-31                # r5: maxima of 1e-31 stay inside at T = 1e-37
    Q[5] = 1e-31
    P[5, :, 3] = 2e-31
    Q[5, :, 3] = 2e-31
    tokens = np.full((B, D), 3, np.int32)
    tr0 = np.arange(B, dtype=np.int64) * (D + 1)
    dr0 = np.arange(B, dtype=np.int64) * D
    res = svo.verify_batch(P.reshape(-1, V), Q.reshape(-1, V), tr0, dr0, tokens,
                           np.full(B, D, np.int32), temps, D_max=D)
    assert list(res["bits"]) == [0, oracle.BIT_BAD_TEMPERATURE, 0, oracle.BIT_BAD_TEMPERATURE,
                                 oracle.BIT_BAD_TEMPERATURE, 0]
    # inside the domain the peaked rows verify as the greedy chain would
    for r in (0, 2, 5):
        assert res["accepted_len"][r] == D and list(res["out_tokens"][r]) == [3] * (D + 1)
    assert np.all(res["out_tokens"][[1, 3, 4]] == -1)
    # the same rows at T = 0 are valid whatever their scale
    res0 = svo.verify_batch(P.reshape(-1, V), Q.reshape(-1, V), tr0, dr0, tokens,
                            np.full(B, D, np.int32), np.zeros(B, np.float32), D_max=D)
    assert np.all(res0["bits"] == 0)


# ---- composition with the Philox stream -----------------------------------

def test_batch_uses_per_request_philox_stream(svo):
    """The batch function is the per-request function fed with the uniforms
    of counter (position, request_id, step, 0); a request's outcome does not
    depend on the other requests in the batch."""
    rng = np.random.default_rng(13)
    B, D, V = 6, 4, 24
    P, Q, tr0, dr0 = padded_batch(rng, B, D, V, noise=1.5)
    tokens = rng.integers(0, V, size=(B, D)).astype(np.int32)
    depth = np.array([4, 0, 2, 4, 1, 3], np.int32)
    rid = np.array([10, 3, 77, 5, 1000, 2], np.uint32)
    T = np.array([1.0, 0.6, 1.0, 1.3, 0.6, 1.0], np.float32)
    res = svo.verify_batch(P.reshape(-1, V), Q.reshape(-1, V), tr0, dr0, tokens, depth, T,
                           seed=99, step=4, request_id=rid, D_max=D)
    for r in range(B):
        n = depth[r]
        u = [svo.uniforms(99, int(rid[r]), 4, k) for k in range(n + 1)]
        tau, out, _, _, _ = svo.verify_request(P[r, : n + 1], Q[r, :n], tokens[r, :n], T[r],
                                               [a for a, _ in u[:n]], [s for _, s in u])
        assert res["accepted_len"][r] == tau
        assert list(res["out_tokens"][r, : tau + 1]) == list(out)
        # the same request alone in a batch of one
        one = svo.verify_batch(P[r].reshape(-1, V), Q[r].reshape(-1, V), [0], [0],
                               tokens[r:r + 1], depth[r:r + 1], T[r:r + 1], seed=99, step=4,
                               request_id=rid[r:r + 1], D_max=D)
        assert one["accepted_len"][0] == tau
        assert list(one["out_tokens"][0]) == list(res["out_tokens"][r])


def test_expected_accepted_length_monte_carlo(svo):
    """Mean tau over many Philox seeds matches sum_m prod_{k<=m} alpha_k
    (equation L_e2e, ai.thesatyajit.com "MTP: fix position 2 and 3") within
    4 standard errors, and position k is reached with frequency
    prod_{i<k} alpha_i."""
    rng = np.random.default_rng(14)
    D, V = 3, 16
    P = (2.0 * rng.standard_normal((D + 1, V))).astype(np.float32)
    Q = (P[:D] + 0.8 * rng.standard_normal((D, V))).astype(np.float32)
    alphas = [svo.alpha(P[k], Q[k], 1.0) for k in range(D)]
    e_tau = svo.expected_accepted(alphas)
    q = [softmax(Q[k].astype(np.float64)) for k in range(D)]
    draft_rng = np.random.default_rng(15)
    N = 6000
    taus = np.empty(N)
    first = np.empty(N, dtype=np.int64)
    for i in range(N):
        tokens = np.array([[draft_rng.choice(V, p=q[k]) for k in range(D)]], np.int32)
        res = svo.verify_batch(P, Q, [0], [0], tokens, [D], [1.0], seed=i, D_max=D)
        taus[i] = res["accepted_len"][0]
        first[i] = res["out_tokens"][0, 0]
    se = taus.std() / np.sqrt(N)
    assert abs(taus.mean() - e_tau) < 4 * se
    for k in range(1, D + 1):
        frac = np.mean(taus >= k)
        pk = float(np.prod(alphas[:k]))
        assert abs(frac - pk) < 4 * np.sqrt(pk * (1 - pk) / N) + 1e-12
    # the first emitted token is always distributed as p_0
    p0 = softmax(P[0].astype(np.float64))
    counts = np.bincount(first, minlength=V)
    chi2 = ((counts - N * p0) ** 2 / (N * p0)).sum()
    assert chi2 < (V - 1) + 6 * np.sqrt(2 * (V - 1))


# ---- statistics -------------------------------------------------------------

def load_golden(name):
    rows = []
    with open(os.path.join(HERE, "golden", name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def test_mal_and_mean_acceptance_match_printed_figures(svo):
    """With depth 3, the printed mean acceptance 52.8% / 66.4% and mean
    accepted length 2.58 / 2.99 satisfy MAL = 1 + D * mean acceptance: the
    oracle's empirical MAL counts the +1 token and its mean acceptance is
    sum tau / sum n."""
    for D, acc, mal in load_golden("mtp_ttt_mal.txt"):
        D, acc, mal = int(D), float(acc), float(mal)
        B = 125                                  # 125 * 3 * acc is an integer
        total = round(B * D * acc)
        assert total == pytest.approx(B * D * acc)
        taus = np.zeros(B, np.int32)
        for i in range(total):                   # spread tau over requests, each <= D
            taus[i % B] += 1
        st = svo.accept_stats(np.full(B, D, np.int32), None, taus, D)
        assert st["summary"][2] == pytest.approx(acc, abs=1e-12)
        assert round(st["summary"][0], 2) == mal
        assert st["summary"][3] == B * D


def test_accept_stats_definitions(svo):
    depth = np.array([3, 3, 1, 0], np.int32)
    tau = np.array([3, 1, 0, 0], np.int32)
    alpha = np.array([[0.5, 0.5, 0.5], [1.0, 0.25, 1.0], [0.3, 0, 0], [0, 0, 0]])
    st = svo.accept_stats(depth, alpha, tau, 3)
    assert list(st["expected_len"]) == pytest.approx([0.875, 1.5, 0.3, 0.0])
    assert list(st["per_depth"][0]) == [3, 2, 1]   # tested at k
    assert list(st["per_depth"][1]) == [2, 1, 1]   # kept at k
    assert list(st["per_depth"][2]) == pytest.approx([0.6, 0.375, 0.75])
    s = st["summary"]
    assert s[0] == pytest.approx(1 + 4 / 4)
    assert s[1] == pytest.approx(1 + (0.875 + 1.5 + 0.3) / 4)
    assert s[2] == pytest.approx(4 / 7)
    assert s[3] == 7


def test_accept_stats_clamps_depth(svo):
    """A depth outside [0, D_max] counts as the nearest end: the request with
    depth 5 at D_max = 3 has three positions (its prefix products stop at the
    row's end), the one with depth -2 has none; nothing past a row is read."""
    depth = np.array([5, -2, 2], np.int32)
    tau = np.array([0, 0, 2], np.int32)
    alpha = np.array([[0.5, 0.5, 0.5], [0.9, 0.9, 0.9], [1.0, 0.25, 0.7]])
    st = svo.accept_stats(depth, alpha, tau, 3)
    assert list(st["expected_len"]) == pytest.approx([0.875, 0.0, 1.25])
    assert list(st["per_depth"][0]) == [2, 1, 0]   # tested at k (tau >= k)
    assert list(st["per_depth"][1]) == [1, 1, 0]   # kept at k (tau > k)
    assert list(st["per_depth"][2]) == pytest.approx([0.75, 0.375, 0.5])
    s = st["summary"]
    assert s[0] == pytest.approx(1 + 2 / 3)
    assert s[1] == pytest.approx(1 + (0.875 + 1.25) / 3)
    assert s[2] == pytest.approx(2 / 5)
    assert s[3] == 5
