"""Pins of the oracle's sampling (runs without a GPU).

Philox4x32-10 against the known-answer vectors published with the generator (Salmon et al.,
"Parallel random numbers: as easy as 1, 2, 3", SC 2011; the Random123 distribution's
known-answer tests for philox4x32_10).  The sampler against scipy's softmax (counts of a
stratified grid of draws), closed-form nucleus boundaries, ties broken by index, and the greedy
limits of small top_p and small temperature.
"""
import numpy as np
import pytest
import scipy.special

import oracle

PHILOX_KAT = [
    ((0x00000000, 0x00000000, 0x00000000, 0x00000000), (0x00000000, 0x00000000),
     (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF), (0xFFFFFFFF, 0xFFFFFFFF),
     (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


@pytest.mark.parametrize("ctr,key,want", PHILOX_KAT)
def test_philox_known_answers(ctr, key, want):
    assert tuple(int(x) for x in oracle.philox4x32_10(ctr, key)) == want


def test_uniform_draw_is_in_range_and_spread():
    us = np.array([oracle.sample_uniform(1234, p) for p in range(20000)])
    assert us.min() >= 0.0 and us.max() < 1.0
    assert abs(us.mean() - 0.5) < 0.01 and abs(np.mean(us < 0.25) - 0.25) < 0.01
    assert oracle.sample_uniform(1234, 7) == oracle.sample_uniform(1234, 7)
    assert oracle.sample_uniform(1234, 7) != oracle.sample_uniform(1235, 7)
    # 24-bit resolution: every draw is a multiple of 2^-24
    assert np.all(np.floor(us * 2**24) == us * 2**24)


def test_draws_follow_the_tempered_softmax():
    rng = np.random.default_rng(3)
    z = rng.standard_normal(50) * 2.0
    temp, N = 0.7, 20000
    p = scipy.special.softmax(z / temp)
    counts = np.zeros(50, dtype=np.int64)
    for k in range(N):
        tok, nsize, nmass = oracle.sample(z, temp, 1.0, (k + 0.5) / N)
        counts[tok] += 1
    assert nsize == 50 and abs(nmass - 1.0) < 1e-12
    # an inverse CDF over a stratified grid gives each token floor or ceil of N p_i draws
    assert np.all(np.abs(counts - N * p) <= 1.0 + 1e-9)


@pytest.mark.parametrize("top_p,size", [(0.4, 1), (0.79, 2), (0.81, 3), (0.96, 4), (1.0, 4)])
def test_nucleus_boundaries_closed_form(top_p, size):
    probs = np.array([0.15, 0.5, 0.05, 0.3])      # order by p: 1, 3, 0, 2
    z = np.log(probs)
    members = {1: [1], 2: [1, 3], 3: [1, 3, 0], 4: [1, 3, 0, 2]}[size]
    tok, nsize, nmass = oracle.sample(z, 1.0, top_p, 0.0)
    assert nsize == size
    assert abs(nmass - probs[members].sum()) < 1e-12
    # u = 0 draws the lowest-index member; u -> 1 the highest
    assert tok == min(members)
    tok_hi, _, _ = oracle.sample(z, 1.0, top_p, 1.0 - 1e-12)
    assert tok_hi == max(members)


def test_ties_are_ordered_by_index():
    z = np.zeros(10)                               # ten tokens of 0.1
    seen = set()
    for k in range(400):
        tok, nsize, nmass = oracle.sample(z, 1.0, 0.35, (k + 0.5) / 400)
        seen.add(tok)
        assert nsize == 4 and abs(nmass - 0.4) < 1e-12
    assert seen == {0, 1, 2, 3}


def test_greedy_limits():
    rng = np.random.default_rng(8)
    z = rng.standard_normal(1000)
    am = int(np.argmax(z))
    for u in (0.0, 0.3, 0.999):
        assert oracle.sample(z, 1.0, 1e-9, u)[0] == am      # nucleus of one token
        assert oracle.sample(z, 1e-4, 0.9, u)[0] == am      # all mass on the maximum
    # a very high temperature flattens the distribution: the nucleus holds about top_p of them
    _, nsize, _ = oracle.sample(z, 1e4, 0.5, 0.5)
    assert 490 <= nsize <= 510
