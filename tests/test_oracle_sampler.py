"""Pins for the oracle's top-k sampler ("a 1-bit llm, from scratch", section
"the interesting bit": the next token comes from the k largest of 4096
logits, kept in a size-k min-heap rather than a full sort; "ultragraph-1bit
0.12.0" README, "A whole ternary GPT": generate() with temperature and
top_k).  The reading: rank by logit (larger first, equal values by lower
index), weight rank r by exp((l_r - l_1) / T), and return the first rank
whose cumulative weight exceeds u times the total."""
import math

import numpy as np

import oracle


def test_k1_is_argmax():
    rng = np.random.default_rng(80)
    x = rng.standard_normal((20, 4096), dtype=np.float32)
    x[3, 100] = x[3, 7] = np.float32(50.0)  # a tie at the top: the lower index wins
    tok, idx, _, cdf = oracle.sample_topk(x, 1, 0.7, rng.random(20, dtype=np.float32))
    assert np.array_equal(tok, np.argmax(x, axis=1).astype(np.int32))
    assert tok[3] == 7 and np.all(cdf == 1.0)


def test_ranking_matches_a_stable_sort():
    """The kept set, in order, is what a stable sort of the negated logits
    gives (equal values stay in index order), ties and repeated values
    included."""
    rng = np.random.default_rng(81)
    x = np.round(rng.standard_normal((8, 4096)) * 4).astype(np.float32)  # many ties
    for k in (1, 40, 100, 256):
        _, idx, val, _ = oracle.sample_topk(x, k, 1.0, np.zeros(8, np.float32))
        want = np.argsort(-x, axis=1, kind="stable")[:, :k].astype(np.int32)
        assert np.array_equal(idx, want)
        assert np.array_equal(val, np.take_along_axis(x, want, axis=1))


def test_u_zero_takes_the_top_rank():
    rng = np.random.default_rng(82)
    x = rng.standard_normal((5, 1000), dtype=np.float32)
    tok, idx, _, _ = oracle.sample_topk(x, 100, 1.3, np.zeros(5, np.float32))
    assert np.array_equal(tok, idx[:, 0])


def test_uniform_limit_of_a_huge_temperature():
    """T -> infinity makes every kept weight 1: rank floor(u k)."""
    rng = np.random.default_rng(83)
    x = rng.standard_normal((1, 500), dtype=np.float32)
    k = 40
    for u in (0.01, 0.26, 0.5, 0.77, 0.999):
        tok, idx, _, cdf = oracle.sample_topk(x, k, 1e30, [u])
        assert np.allclose(cdf[0], np.arange(1, k + 1) / k, rtol=0, atol=1e-12)
        assert tok[0] == idx[0, int(math.floor(u * k))]


def test_two_kept_logits_with_temperature():
    """Two kept logits l_1 > l_2: rank 1 has weight 1 / (1 + e^{-(l_1-l_2)/T}),
    so u just below it gives rank 1 and u just above gives rank 2.  A
    temperature multiplied in instead of divided moves the threshold."""
    x = np.full((1, 64), -100.0, np.float32)
    x[0, 9], x[0, 30] = 2.0, 0.5
    for T in (0.5, 1.0, 3.0):
        p1 = 1.0 / (1.0 + math.exp(-(2.0 - 0.5) / T))
        lo, hi = np.float32(p1 - 1e-6), np.float32(p1 + 1e-6)
        assert oracle.sample_topk(x, 2, T, [lo])[0][0] == 9
        assert oracle.sample_topk(x, 2, T, [hi])[0][0] == 30
        wrong = 1.0 / (1.0 + math.exp(-(2.0 - 0.5) * T))
        if abs(wrong - p1) > 1e-3:
            mid = np.float32((p1 + wrong) / 2)
            want = 9 if mid < p1 else 30
            assert oracle.sample_topk(x, 2, T, [mid])[0][0] == want


def test_sampling_frequencies_follow_the_softmax():
    """Evenly spaced u over [0, 1) hit each kept rank in proportion to its
    softmax probability (to within one step of u)."""
    rng = np.random.default_rng(84)
    x = rng.standard_normal((1, 300), dtype=np.float32)
    k, T, N = 10, 0.8, 20000
    us = ((np.arange(N) + 0.5) / N).astype(np.float32)
    toks = np.array([oracle.sample_topk(x, k, T, [u])[0][0] for u in us[::10]])
    _, idx, val, _ = oracle.sample_topk(x, k, T, [0.0])
    w = np.exp((val[0].astype(np.float64) - val[0, 0]) / T)
    p = w / w.sum()
    freq = np.array([(toks == i).mean() for i in idx[0]])
    assert np.all(np.abs(freq - p) <= 2.0 / (N / 10))
