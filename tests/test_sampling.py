"""Pins of the oracle's sampler (train_gpt2.cu, sample_softmax): inverse-CDF
draws checked against closed forms and exact counts, independent of its code."""

import math

import numpy as np

import oracle


def test_uniform_logits_give_floor_of_coin_times_v():
    V = 1000
    z = np.full(V, 0.7)
    for k in (0, 1, 499, 998, 999):
        assert oracle.sample_softmax(z, V, (k + 0.5) / V) == k


def test_two_tokens_split_at_the_sigmoid():
    a, b = 1.3, -0.4
    p0 = 1.0 / (1.0 + math.exp(b - a))
    z = np.array([a, b])
    assert oracle.sample_softmax(z, 2, p0 * (1 - 1e-9)) == 0
    assert oracle.sample_softmax(z, 2, p0 * (1 + 1e-9)) == 1
    assert oracle.sample_softmax(z, 2, 0.0) == 0


def test_dominant_logit_wins():
    z = np.zeros(100)
    z[37] = 60.0
    for c in (1e-6, 0.3, 0.999999):
        assert oracle.sample_softmax(z, 100, c) == 37


def test_counts_on_a_coin_grid_match_the_probabilities():
    # coins (k + 1/2) / N: token i is drawn for the coins in [cdf_{i-1}, cdf_i),
    # so its count is N p_i to within one
    rng = np.random.default_rng(3)
    z = rng.normal(0, 2, 50)
    p = np.exp(z - z.max())
    p /= p.sum()
    N = 100000
    counts = np.bincount([oracle.sample_softmax(z, 50, (k + 0.5) / N) for k in range(N)], minlength=50)
    assert np.all(np.abs(counts - N * p) <= 1.0 + 1e-9)


def test_padded_columns_are_never_drawn():
    z = np.concatenate([np.zeros(10), np.full(6, 100.0)])
    assert all(oracle.sample_softmax(z, 10, c) < 10 for c in (0.0, 0.5, 1.0 - 2 ** -24, 1.0))
    assert oracle.sample_softmax(z, 10, 1.0) == 9  # no crossing: the last valid index
