"""The straight-through backward on the GPU (ug_bitlinear_backward):
"ultragraph - when the graph is the 1-bit LLM, part 2", section "autograd on
a byte-graph": dL/dx = g W, dL/dW = g^T x, dL/db = sum g, with W the fp32
masters.  Compared with the oracle's double-precision sums within the fp32
rounding bound: a sum of n products, computed with one rounding per product
and per addition in any association (pieces of the contraction added at the
end included: no term passes through more than n roundings), is within
gamma(n) sum |a_i b_i| of the exact value; with the oracle's own fp32
rounding u |exact| and some slack the test allows gamma(n+8) sum |a_i b_i|."""
import numpy as np
import pytest

import oracle
from bitlinear_matmul_amd import ug
from gpu_util import host, pitched

pytestmark = pytest.mark.gpu
U = 2.0 ** -24


def _case(*a):
    print("case:", *a, flush=True)


def gam(n):
    # n roundings on any term's path, the oracle's own rounding, and slack
    return (n + 8) * U / (1 - (n + 8) * U)


def _within(got, ref, absterms, n, what):
    err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    tol = gam(n) * absterms
    bad = err > tol
    print("%s: max error %.3g, max error / bound %.3g" % (what, err.max(),
                                                         (err / np.maximum(tol, 1e-300)).max()),
          flush=True)
    assert not bad.any(), (what, int(bad.sum()), np.argwhere(bad)[0])


def _data(seed, M, N, K):
    rng = np.random.default_rng(seed)
    g = rng.standard_normal((M, N), dtype=np.float32) * np.float32(1e-2)
    x = rng.standard_normal((M, K), dtype=np.float32)
    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    return g, x, W


@pytest.mark.parametrize("M,N,K", [(64, 96, 80), (130, 257, 33), (1, 1, 1), (7, 300, 129),
                                   (300, 5, 1000), (256, 384, 1536),
                                   (200, 2100, 131),   # dx cut into contraction pieces, K % 4 != 0
                                   (640, 4100, 300),   # dx in pieces with a ragged last piece
                                   # (on 256 CUs) dx: 30 tiles in 16 pieces each; dW: 600
                                   # tiles 3 steps deep, too shallow to cut
                                   (48, 2560, 3840),
                                   # dx: 32 tiles in 16 pieces; dW: 1024 tiles, one
                                   # whole round
                                   (16, 4096, 4096)])
def test_backward_parity(dev, M, N, K):
    _case("backward", M, N, K)
    g, x, W = _data([95, M, N, K], M, N, K)
    got = ug.ug_bitlinear_backward(pitched(g), pitched(x), pitched(W))
    ref = oracle.bitlinear_backward(g, x, W)
    g64, x64, W64 = (a.astype(np.float64) for a in (g, x, W))
    _within(host(got["dx"]), ref["dx"], np.abs(g64) @ np.abs(W64), N, "dx")
    _within(host(got["dW"]), ref["dW"], np.abs(g64).T @ np.abs(x64), M, "dW")
    _within(host(got["db"]), ref["db"], np.abs(g64).sum(axis=0), M, "db")


def test_backward_stack_shape_sampled(dev):
    """The stack workload's up projection at M = 2048 tokens (W 6912 x 2560):
    the whole GPU result, checked on 48 sampled rows of dx and 48 sampled
    rows of dW (the oracle computes those rows on their own: dx row m needs
    only g's row m; dW row n only g's column n) and every db entry."""
    M, N, K = 2048, 6912, 2560
    g, x, W = _data(96, M, N, K)
    got = ug.ug_bitlinear_backward(pitched(g), pitched(x), pitched(W))
    dx, dW, db = host(got["dx"]), host(got["dW"]), host(got["db"])
    rng = np.random.default_rng(97)
    ms = np.sort(rng.choice(M, 48, replace=False))
    ns = np.sort(rng.choice(N, 48, replace=False))
    rx = oracle.bitlinear_backward(g[ms], x[ms], W, want=("dx",))
    _within(dx[ms], rx["dx"], np.abs(g[ms].astype(np.float64)) @ np.abs(W.astype(np.float64)),
            N, "dx rows")
    rw = oracle.bitlinear_backward(np.ascontiguousarray(g[:, ns]), x, W[ns], want=("dW", "db"))
    _within(dW[ns], rw["dW"],
            np.abs(g[:, ns].astype(np.float64)).T @ np.abs(x.astype(np.float64)), M, "dW rows")
    rb = oracle.bitlinear_backward(g, x[:, :4].copy(), W[:, :4].copy(), want=("db",))
    _within(db, rb["db"], np.abs(g.astype(np.float64)).sum(axis=0), M, "db")


def test_backward_outputs_one_at_a_time(dev):
    """Each output alone (the others NULL) gives the same bits as all
    three together."""
    g, x, W = _data(98, 70, 140, 210)
    gd, xd, Wd = pitched(g), pitched(x), pitched(W)
    allr = {k: host(v) for k, v in ug.ug_bitlinear_backward(gd, xd, Wd).items()}
    for name in ("dx", "dW", "db"):
        one = ug.ug_bitlinear_backward(gd, xd, Wd, want=(name,))
        assert np.array_equal(host(one[name]).view(np.uint32), allr[name].view(np.uint32))


def test_backward_repeat_and_junk_workspace(dev):
    """A workspace full of junk, and the same workspace again on the next
    call, give the same bits as a fresh one: every partial tile is written
    before it is read (on 256 CUs: dx's 64 tiles in 16 pieces each; dW's 32
    tiles beyond a whole round of blocks in 2 pieces each).  Sampled rows
    of both products against the oracle."""
    import torch
    M, N, K = 256, 4224, 4096
    g, x, W = _data(99, M, N, K)
    gd, xd, Wd = pitched(g), pitched(x), pitched(W)
    first = {k: host(v) for k, v in ug.ug_bitlinear_backward(gd, xd, Wd).items()}
    ws = torch.full((ug.lib().ug_bitlinear_backward_workspace_size(M, N, K),), 0xA5,
                    dtype=torch.uint8, device=gd.device)
    for rep in range(3):
        again = ug.ug_bitlinear_backward(gd, xd, Wd, ws=ws)
        for name in ("dx", "dW", "db"):
            assert np.array_equal(host(again[name]).view(np.uint32),
                                  first[name].view(np.uint32)), (rep, name)
    rng = np.random.default_rng(100)
    ms = np.sort(rng.choice(M, 24, replace=False))
    rx = oracle.bitlinear_backward(g[ms], x[ms], W, want=("dx",))
    _within(first["dx"][ms], rx["dx"],
            np.abs(g[ms].astype(np.float64)) @ np.abs(W.astype(np.float64)), N, "dx rows")
    ns = np.concatenate([np.arange(N - 8, N), rng.choice(N - 8, 16, replace=False)])
    ns = np.sort(ns)
    rw = oracle.bitlinear_backward(np.ascontiguousarray(g[:, ns]), x, W[ns], want=("dW",))
    _within(first["dW"][ns], rw["dW"],
            np.abs(g[:, ns].astype(np.float64)).T @ np.abs(x.astype(np.float64)), M, "dW rows")
