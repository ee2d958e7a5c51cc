"""Pins for the oracle's multi-step decode loop on a synthetic Markov target
([T] "The MTP path": MAL measured over whole generations; [A] "MTP": blocks of
drafts verified in one pass).  Lossless verification makes the emitted
sequence a sample of the target chain whatever the drafter: the transition
frequencies of the emitted tokens match softmax(P[prev] / T) (chi-square), a
drafter equal to the target is always accepted, and at T = 0 the output is
the target's greedy chain."""
import numpy as np
import pytest
from scipy.stats import chi2
from scipy.special import softmax


def tables(rng, V, noise):
    P = (1.5 * rng.standard_normal((V, V))).astype(np.float32)
    Q = (P + noise * rng.standard_normal((V, V))).astype(np.float32)
    return P, Q


def stream(res, r, start):
    seq = [start]
    for step in res["emitted"]:
        seq.extend(step[r])
    return seq


def test_draft_uniform_is_word_two(svo):
    for seed, rid, step, pos in [(0, 0, 0, 0), (7, 3, 5, 2), ((5 << 32) | 9, 1, 2, 3)]:
        w = svo.philox([pos, rid, step, 0], [seed & 0xFFFFFFFF, seed >> 32])
        assert svo.draft_uniform(seed, rid, step, pos) == (int(w[2]) >> 8) * 2.0 ** -24
        u0, u1 = svo.uniforms(seed, rid, step, pos)
        assert u0 == (int(w[0]) >> 8) * 2.0 ** -24 and u1 == (int(w[1]) >> 8) * 2.0 ** -24


@pytest.mark.parametrize("T", [1.0, 0.7])
def test_emitted_chain_follows_the_target(svo, T):
    rng = np.random.default_rng(31)
    V, B, D = 4, 4, 3
    P, Q = tables(rng, V, noise=1.5)
    start = [0, 1, 2, 3]
    res = svo.markov_decode(P, Q, start, D, [T] * B, steps=700, seed=5)
    counts = np.zeros((V, V))
    for r in range(B):
        seq = stream(res, r, start[r])
        for a, b in zip(seq[:-1], seq[1:]):
            counts[a, b] += 1
    stat, dof = 0.0, 0
    for a in range(V):
        n = counts[a].sum()
        expect = n * softmax(P[a].astype(np.float64) / T)
        stat += float(((counts[a] - expect) ** 2 / expect).sum())
        dof += V - 1
    assert counts.sum() > 4000
    assert chi2.sf(stat, dof) > 1e-4, (stat, dof)
    # a drafter that differs from the target is rejected sometimes
    taus = np.array(res["tau"])
    assert 0 < taus.mean() < D


def test_drafter_equal_to_target_is_always_accepted(svo):
    rng = np.random.default_rng(32)
    V, B, D = 8, 3, 4
    P, _ = tables(rng, V, noise=0.0)
    res = svo.markov_decode(P, P, [1, 2, 3], D, [1.0, 0.5, 2.0], steps=40, seed=9)
    for step, taus in zip(res["emitted"], res["tau"]):
        assert taus == [D] * B
        assert all(len(e) == D + 1 for e in step)
    # and each step's drafts are its first D emitted tokens
    for em, dr in zip(res["emitted"], res["drafts"]):
        for r in range(B):
            assert em[r][:D] == dr[r]


def test_greedy_decoding_is_the_argmax_chain(svo):
    rng = np.random.default_rng(33)
    V, B, D = 16, 2, 3
    P, Q = tables(rng, V, noise=2.0)
    start = [4, 11]
    res = svo.markov_decode(P, Q, start, D, [0.0, 0.0], steps=25, seed=1)
    for r in range(B):
        seq = stream(res, r, start[r])
        for a, b in zip(seq[:-1], seq[1:]):
            assert b == int(np.argmax(P[a]))
