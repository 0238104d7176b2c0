"""Top-k sampling on the GPU (ug_sample_topk): "a 1-bit llm, from scratch",
section "the interesting bit" (the next token from the k largest of 4096
logits, without sorting them all) and the "ultragraph-1bit 0.12.0" README,
"A whole ternary GPT" (temperature and top_k).

Which indices are kept and in which order is decided by comparisons only:
bit-exact against the oracle.  The draw goes through expf and fp32 sums, so
for each row the test derives a band around the oracle's (double precision)
cumulative weights: a token is valid if u lies in its rank's interval
widened by that band, and must equal the oracle's token whenever u is
farther than the band from every boundary."""
import numpy as np
import pytest
import torch

import oracle
from bitlinear_matmul_amd import ug
from gpu_util import assert_bits_equal, host, pitched, vec

pytestmark = pytest.mark.gpu
U = 2.0 ** -24


def _case(*a):
    print("case:", *a, flush=True)


def _band(val, T):
    """Each weight e_r = expf(fl(fl(l_r - l_1) / T)): two roundings of its
    argument a_r (2u |a_r| after the exp) and expf's own error (<= 2 ulp,
    4u); each running sum C_r is a fixed tree of depth <= 9 (at most 10u);
    the threshold fl(u C_k) one more.  A boundary C_r / C_k so moves by at
    most 2 (2u max|a| + 4u + 10u) + u <= (4 max|a| + 32) u."""
    a = np.abs((val.astype(np.float64) - val[:, :1]) / T).max(axis=1)
    return (4 * a + 32) * U


def _check(logits, k, T, u):
    B = logits.shape[0]
    x = pitched(logits)  # rows padded to a multiple of 4 floats
    tok, idx, val, prob = ug.ug_sample_topk(x, k, T, vec(u), want_topk=True)
    tok, idx, val, prob = host(tok), host(idx), host(val), host(prob)
    r_tok, r_idx, r_val, r_cdf = oracle.sample_topk(logits, k, T, u)
    assert_bits_equal(idx, r_idx, "kept indices")
    assert_bits_equal(val, r_val, "kept logits")
    band = _band(r_val, T)
    lo = np.concatenate([np.zeros((B, 1)), r_cdf[:, :-1]], axis=1)
    for b in range(B):
        r = int(np.nonzero(idx[b] == tok[b])[0][0])
        hi = r_cdf[b, r] if r < k - 1 else 2.0
        assert lo[b, r] - band[b] <= u[b] < hi + band[b], (b, r, float(u[b]))
        clear = np.all(np.abs(r_cdf[b, :-1] - u[b]) > band[b])
        if clear:
            assert tok[b] == r_tok[b], (b, tok[b], r_tok[b])
    # the probabilities, within the same band
    p_ref = np.diff(np.concatenate([np.zeros((B, 1)), r_cdf], axis=1), axis=1)
    assert np.all(np.abs(prob - p_ref) <= 2 * band[:, None] + 1e-30)
    return tok


@pytest.mark.parametrize("B,V,k,T,kind", [
    (1, 4096, 100, 0.8, "normal"),     # the page's case: 100 of 4096
    (64, 4096, 40, 1.0, "normal"),     # the README's top_k = 40
    (7, 256, 40, 0.8, "normal"),       # byte-level vocabulary
    (3, 50000, 100, 1.0, "normal"),    # a row longer than the register path
    (5, 4097, 256, 2.0, "normal"),
    (9, 300, 1, 1.0, "normal"),        # k = 1: the argmax
    (4, 100, 100, 1.0, "normal"),      # k = V
    (16, 4096, 100, 1.0, "ties"),      # many equal logits around the cut
    (3, 1000, 50, 1.0, "constant"),    # every logit equal
    (6, 2000, 64, 1.0, "zeros"),       # -0 and +0 mixed
    (4, 4096, 100, 1e30, "normal"),    # uniform over the kept ranks
    (64, 4096, 150, 1.0, "normal"),    # candidates near 256: rows take either selection
    (4, 4096, 100, 1.0, "ascending"),  # the largest logits packed into the last threads
    (4, 4096, 100, 1.0, "descending"),
])
def test_sampler_parity(dev, B, V, k, T, kind):
    """Rows whose large logits are spread over the block's threads select
    from the keys above a per-wave threshold; tied, constant, sorted and
    large-k rows (more than 256 keys above it) take the radix select."""
    _case("sampler", B, V, k, T, kind)
    rng = np.random.default_rng([90, B, V, k])
    x = rng.standard_normal((B, V), dtype=np.float32) * np.float32(3.0)
    if kind == "ties":
        x = np.round(x).astype(np.float32)
    elif kind == "constant":
        x[:] = np.float32(0.25)
    elif kind in ("ascending", "descending"):
        x = np.sort(x, axis=1)
        if kind == "descending":
            x = np.ascontiguousarray(x[:, ::-1])
    elif kind == "zeros":
        x = np.where(rng.random((B, V)) < 0.5, np.float32(-0.0), np.float32(0.0)).astype(np.float32)
        x[:, ::7] = rng.standard_normal((B, (V + 6) // 7), dtype=np.float32)
    u = rng.random(B, dtype=np.float32)
    u[0] = 0.0
    _check(x, k, T, u)


@pytest.mark.parametrize("B,V,k,kind", [
    (8, 1000, 3, "normal"),         # k not a multiple of 4: each wave's 1st largest
    (8, 777, 13, "normal"),         # ragged: the last threads and waves hold no logits
    (8, 130, 5, "normal"),          # one logit per thread; waves 3 and 4 empty: x = 0
    (8, 4096, 100, "one_thread"),   # the 16 largest logits in one thread's span
    (8, 4096, 100, "one_wave"),     # the 1024 largest in one wave's threads
    (8, 4096, 7, "spikes"),         # a few huge logits far above the rest
    (8, 4096, 256, "normal"),       # the largest k: x is the least thread maximum
])
def test_sampler_threshold_edges(dev, B, V, k, kind):
    """Rows where the candidate threshold (each wave's ceil(k/4)-th largest
    thread maximum, the least of the four) is tight, degenerate or lets in
    many keys: the kept indices and their order stay exact."""
    _case("sampler edges", B, V, k, kind)
    rng = np.random.default_rng([92, B, V, k])
    x = rng.standard_normal((B, V), dtype=np.float32)
    per = -(-V // 256)
    if kind == "one_thread":
        t0 = 97 * per
        x[:, t0:t0 + per] += np.float32(50.0)
    elif kind == "one_wave":
        w0 = 2 * 64 * per
        x[:, w0:w0 + 64 * per] += np.float32(50.0)
    elif kind == "spikes":
        for b in range(B):
            x[b, rng.choice(V, 5, replace=False)] = np.float32(1e4) * rng.random(5, dtype=np.float32)
    u = rng.random(B, dtype=np.float32)
    _check(x, k, 1.0, u)


def test_sampler_frequencies(dev):
    """20000 rows of the same logits with evenly spaced draws: each kept
    rank is drawn in proportion to its softmax weight."""
    rng = np.random.default_rng(91)
    B, V, k, T = 20000, 4096, 100, 0.7
    x = np.tile(rng.standard_normal((1, V), dtype=np.float32) * np.float32(2.0), (B, 1))
    u = ((np.arange(B) + 0.5) / B).astype(np.float32)
    tok = _check(x, k, T, u)
    _, idx, _, cdf = oracle.sample_topk(x[:1], k, T, u[:1])
    p = np.diff(np.concatenate([[0.0], cdf[0]]))
    freq = np.array([(tok == i).mean() for i in idx[0]])
    assert np.all(np.abs(freq - p) <= 2.0 / B)
