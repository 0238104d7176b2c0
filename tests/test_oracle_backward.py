"""Pins for the oracle's straight-through backward ("ultragraph - when the
graph is the 1-bit LLM, part 2", section "autograd on a byte-graph": the
estimator pretends the quantizers and the per-row scale are the identity,
so dL/dx = g W, dL/dW = g^T x, dL/db = sum g, with W the fp32 masters).

The estimator's gradient is the exact gradient of the unquantized layer
y = x W^T + b.  The loss L = sum(g * y) is linear in each of x, W and b, so
a finite difference of L is exact up to the rounding of L itself: the
checks below are finite differences (as the pages' autograd is grad-checked
against them), one-hot upstream gradients, and a transposition guard."""
import math

import numpy as np

import oracle


def _loss(g, x, W, b):
    """L = sum_{m,n} g[m,n] (x W^T + b)[m,n], exactly (math.fsum of float64
    products of fp32 values, each exact)."""
    y = x.astype(np.float64) @ W.astype(np.float64).T + b.astype(np.float64)
    return math.fsum((g.astype(np.float64) * y).ravel().tolist())


def test_finite_differences_of_the_unquantized_layer():
    rng = np.random.default_rng(70)
    M, N, K = 5, 7, 6
    g = rng.standard_normal((M, N), dtype=np.float32)
    x = rng.standard_normal((M, K), dtype=np.float32)
    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    b = rng.standard_normal(N, dtype=np.float32)
    r = oracle.bitlinear_backward(g, x, W)
    h = 0.5  # L is linear: any step gives the derivative (a power of two keeps it exact)
    L0 = _loss(g, x, W, b)
    for m in range(M):
        for k in range(K):
            x2 = x.copy()
            x2[m, k] += np.float32(h)
            fd = (_loss(g, x2, W, b) - L0) / h
            assert abs(r["dx"][m, k] - fd) <= 1e-6 * (1 + abs(fd))
    for n in range(N):
        for k in range(K):
            W2 = W.copy()
            W2[n, k] += np.float32(h)
            fd = (_loss(g, x, W2, b) - L0) / h
            assert abs(r["dW"][n, k] - fd) <= 1e-6 * (1 + abs(fd))
        b2 = b.copy()
        b2[n] += np.float32(h)
        fd = (_loss(g, x, W, b2) - L0) / h
        assert abs(r["db"][n] - fd) <= 1e-6 * (1 + abs(fd))


def test_one_hot_upstream_gradient():
    """g = e_{m,n}: dx has W's row n in row m, dW has x's row m in row n,
    db = e_n, bit for bit."""
    rng = np.random.default_rng(71)
    M, N, K = 4, 9, 13
    x = rng.standard_normal((M, K), dtype=np.float32)
    W = rng.standard_normal((N, K), dtype=np.float32)
    for (m, n) in ((0, 0), (3, 8), (2, 5)):
        g = np.zeros((M, N), np.float32)
        g[m, n] = 1.0
        r = oracle.bitlinear_backward(g, x, W)
        want_dx = np.zeros((M, K), np.float32)
        want_dx[m] = W[n]
        want_dW = np.zeros((N, K), np.float32)
        want_dW[n] = x[m]
        assert np.array_equal(r["dx"], want_dx)
        assert np.array_equal(r["dW"], want_dW)
        assert np.array_equal(r["db"], np.eye(N, dtype=np.float32)[n])


def test_sums_of_exact_products():
    """Small-integer inputs: every product and partial sum is exact in fp32
    and double, so the results equal integer matrix products exactly."""
    rng = np.random.default_rng(72)
    M, N, K = 11, 6, 8
    g = rng.integers(-3, 4, (M, N)).astype(np.float32)
    x = rng.integers(-3, 4, (M, K)).astype(np.float32)
    W = rng.integers(-1, 2, (N, K)).astype(np.float32)
    r = oracle.bitlinear_backward(g, x, W)
    gi, xi, Wi = g.astype(np.int64), x.astype(np.int64), W.astype(np.int64)
    assert np.array_equal(r["dx"], (gi @ Wi).astype(np.float32))
    assert np.array_equal(r["dW"], (gi.T @ xi).astype(np.float32))
    assert np.array_equal(r["db"], gi.sum(axis=0).astype(np.float32))
