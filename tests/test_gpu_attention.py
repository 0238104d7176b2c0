"""Causal attention over a key/value cache on the GPU (ug_attention_cached):
"ultragraph - when the graph is the 1-bit LLM, part 2", section "attention,
as graph ops" (softmax(Q K^T / sqrt(d_h) + mask) V per head) and the
"ultragraph-1bit 0.12.0" README, "A whole ternary GPT" (decoding with a
per-layer K/V cache whose cached steps reproduce the full forward).

Parity: against the oracle's double-precision attention, within a bound
derived from the fp32 arithmetic of the kernels (below).  Invariants, bit
for bit on the GPU itself: a one-row decode call at position t equals row t
of a full-forward call; keys after a query's position never touch it."""
import math

import numpy as np
import pytest
import torch

import oracle
from bitlinear_matmul_amd import ug
from gpu_util import assert_bits_equal, host, pitched, scalar_dev, vec

pytestmark = pytest.mark.gpu
U = 2.0 ** -24


def _case(*a):
    print("case:", *a, flush=True)


def _inputs(seed, T, H, dh, M):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((M, H * dh), dtype=np.float32)
    k = rng.standard_normal((T, H * dh), dtype=np.float32)
    v = rng.standard_normal((T, H * dh), dtype=np.float32)
    return q, k, v


def _bound(q, k, v, pos0, H):
    """Per-element error bound of the fp32 kernels against exact attention.
    A score is a sum of dh products (partials of 4 products, then dh/4
    partials in order: at most dh + dh/4 <= dh + 64 roundings) and one
    division: |d score_j| <= E_j = gamma(dh + 66) * sum_d |q_d k_jd| /
    sqrt(dh).  A weight a_j = e^{s_j} / sum e^{s_i} then moves by at most
    2 max_j E_j relative, plus the roundings of its exp (two, with the chunk
    rescale), of the sums (at most 64 keys in order within a chunk and a
    fold of at most 8 row sums, up to 16 chunks in order per wave of the
    combine, then two levels) and of the products: at most 256 u relative
    to sum_j a_j |v_jd| all told.  So |out_d - exact_d| <=
    (2 max E + 256 u) sum_j a_j |v_jd|."""
    M, HD = q.shape
    dh = HD // H
    tol = np.empty((M, HD))
    gam = (dh + 66) * U / (1 - (dh + 66) * U)
    for m in range(M):
        p = pos0 + m
        for h in range(H):
            s = slice(h * dh, (h + 1) * dh)
            qh = q[m, s].astype(np.float64)
            kh = k[:p + 1, s].astype(np.float64)
            vh = v[:p + 1, s].astype(np.float64)
            sc = kh @ qh / math.sqrt(dh)
            E = gam * (np.abs(kh) @ np.abs(qh)).max() / math.sqrt(dh)
            a = np.exp(sc - sc.max())
            a /= a.sum()
            tol[m, s] = (2 * E + 256 * U) * (a @ np.abs(vh))
    return tol


def _gpu(q, k, v, pos0, H):
    return host(ug.ug_attention_cached(pitched(q), pitched(k), pitched(v), pos0, H))


@pytest.mark.parametrize("T,H,dh,M,pos0", [
    (4096, 20, 128, 1, 4095),   # decode at 4096 tokens, 2B-class heads (2560 = 20 x 128)
    (256, 4, 32, 1, 255),       # decode, the README's small GPT (d_model 128, 4 heads)
    (700, 2, 64, 1, 699),       # ragged last chunk
    (300, 1, 256, 1, 299),
    (9, 3, 64, 1, 0),           # a single key
    (257, 2, 32, 1, 256),       # second chunk of one key
    (300, 3, 64, 300, 0),       # full forward over 300 tokens
    (520, 2, 128, 8, 512),      # a few rows after a long prefix
])
def test_attention_parity(dev, T, H, dh, M, pos0):
    _case("attention", T, H, dh, M, pos0)
    q, k, v = _inputs([61, T, H, dh, M], T, H, dh, M)
    got = _gpu(q, k, v, pos0, H)
    ref = oracle.attention(q, k, v, pos0, H)
    tol = _bound(q, k, v, pos0, H)
    err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    print("max error %.3g, max error / bound %.3g" % (err.max(), (err / tol).max()), flush=True)
    bad = err > tol
    assert not bad.any(), (int(bad.sum()), np.argwhere(bad)[0])


def test_cached_step_equals_full_forward_row(dev):
    """README "A whole ternary GPT": a cached decoding step gives the bits of
    the full forward at that position.  Row t of one call over 600 query rows
    against single-row calls at position t, across chunk boundaries."""
    T, H, dh = 600, 2, 64
    q, k, v = _inputs(62, T, H, dh, T)
    full = _gpu(q, k, v, 0, H)
    for t in (0, 1, 255, 256, 257, 511, 512, 599):
        _case("cached vs full", t)
        one = _gpu(q[t:t + 1], k, v, t, H)
        assert_bits_equal(one[0], full[t], "row %d" % t)


def test_attention_is_causal_on_gpu(dev):
    """"attention, as graph ops": an earlier position must not see later
    ones.  Keys and values after position t changed wildly: row t keeps its
    bits."""
    T, H, dh, t = 800, 2, 128, 300
    q, k, v = _inputs(63, T, H, dh, 1)
    base = _gpu(q, k, v, t, H)
    k2, v2 = k.copy(), v.copy()
    k2[t + 1:] *= np.float32(50.0)
    v2[t + 1:] = np.float32(1e6)
    assert_bits_equal(_gpu(q, k2, v2, t, H), base, "after changing the future")
    v3 = v.copy()
    v3[t] += np.float32(1.0)
    assert not np.array_equal(_gpu(q, k, v3, t, H), base)


def test_decode_step_around_the_gemv(dev):
    """One decode step of an attention block with BitLinear projections:
    grouped GEMV for q, k, v (fp32 token quantized in the launch, biases),
    whose k and v outputs land straight in the cache row of the new
    position; attention over the cache; grouped GEMV for the output
    projection of the context.  q/k/v and the projection bit-exact against
    the oracle (the projection fed the GPU's context), the context within
    the attention bound."""
    rng = np.random.default_rng(64)
    d, H, dh, prev = 256, 4, 64, 37
    T = prev + 1
    x = rng.standard_normal((1, d), dtype=np.float32)
    Ws = [rng.standard_normal((d, d), dtype=np.float32) * np.float32(0.02) for _ in range(4)]
    bs = [rng.standard_normal(d, dtype=np.float32) * np.float32(0.1) for _ in range(4)]
    kc = ug.empty_pitched(T, d, torch.float32, dev)
    vc = ug.empty_pitched(T, d, torch.float32, dev)
    kc[:prev] = torch.from_numpy(rng.standard_normal((prev, d), dtype=np.float32)).to(dev)
    vc[:prev] = torch.from_numpy(rng.standard_normal((prev, d), dtype=np.float32)).to(dev)
    qbuf = ug.empty_pitched(1, d, torch.float32, dev)
    packed, betas, refs = [], [], []
    for W, b in zip(Ws, bs):
        wq, beta = oracle.quant_weight_absmean(W)
        packed.append(pitched(oracle.pack_trits(wq)[0]))
        betas.append(scalar_dev(beta))
    xd = pitched(x)
    outs = [qbuf, kc[prev:prev + 1], vc[prev:prev + 1]]
    plan = ug.ug_gemv_plan_init([dict(x=xd, w=packed[i], wfmt=ug.UG_W_PACK5, beta=betas[i], K=d,
                                      bias=vec(bs[i]), y=outs[i]) for i in range(3)])
    ug.ug_bitlinear_gemv_grouped(plan)
    for i in range(3):
        r = oracle.bitlinear(x, Ws[i], bias=bs[i])
        assert_bits_equal(host(outs[i]), r["y"], "projection %d" % i)
    ctx = ug.ug_attention_cached(qbuf, kc, vc, prev, H)
    qh, kh, vh = host(qbuf), host(kc), host(vc)
    ref = oracle.attention(qh, kh, vh, prev, H)
    tol = _bound(qh, kh, vh, prev, H)
    assert np.all(np.abs(host(ctx).astype(np.float64) - ref) <= tol)
    y = ug.empty_pitched(1, d, torch.float32, dev)
    plan_o = ug.ug_gemv_plan_init([dict(x=ctx, w=packed[3], wfmt=ug.UG_W_PACK5, beta=betas[3],
                                        K=d, bias=vec(bs[3]), y=y)])
    ug.ug_bitlinear_gemv_grouped(plan_o)
    r = oracle.bitlinear(host(ctx), Ws[3], bias=bs[3])
    assert_bits_equal(host(y), r["y"], "output projection")
