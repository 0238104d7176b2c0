"""Pins for the oracle's causal attention over a key/value cache
("ultragraph - when the graph is the 1-bit LLM, part 2", section
"attention, as graph ops": scores = Q K^T / sqrt(d_h), a causal mask,
A = softmax(scores + M), ctx = A V, per head; "ultragraph-1bit 0.12.0"
README, "A whole ternary GPT": decoding keeps a per-layer K/V cache).

Each pin is a closed form or an invariant the page states, chosen so that a
plausible slip (no 1/sqrt(d_h), 1/d_h instead, an off-by-one in the causal
range, the wrong head's columns, a missing normalization) fails one."""
import math

import numpy as np

import oracle


def _rand(rng, T, H, dh, M=1):
    q = rng.standard_normal((M, H * dh), dtype=np.float32)
    k = rng.standard_normal((T, H * dh), dtype=np.float32)
    v = rng.standard_normal((T, H * dh), dtype=np.float32)
    return q, k, v


def test_attention_single_key_returns_its_value():
    """Position 0 sees one key: its softmax weight is exactly 1 and the
    output is that key's value row, bit for bit."""
    rng = np.random.default_rng(50)
    q, k, v = _rand(rng, 5, 3, 32)
    out = oracle.attention(q, k, v, 0, 3)
    assert np.array_equal(out[0], v[0])


def test_attention_equal_keys_average_the_values():
    """Every key equal: all scores equal, uniform weights 1/n, so the output
    is the mean of the n value rows (n = position + 1)."""
    rng = np.random.default_rng(51)
    H, dh, T = 2, 64, 40
    q, _, v = _rand(rng, T, H, dh)
    k = np.tile(rng.standard_normal((1, H * dh), dtype=np.float32), (T, 1))
    for pos in (0, 7, 39):
        out = oracle.attention(q, k, v, pos, H)
        for d in range(H * dh):
            want = math.fsum(v[:pos + 1, d].astype(np.float64).tolist()) / (pos + 1)
            assert abs(out[0, d] - want) <= 2e-7 * (1 + abs(want))


def test_attention_two_keys_closed_form_with_root_dh_scale():
    """Two keys whose dot products with q are exact: the weights are
    1 / (1 + e^{-D}) and e^{-D} / (1 + e^{-D}) with D = (s0 - s1) / sqrt(d_h).
    A missing 1/sqrt(d_h), or 1/d_h, gives other weights."""
    for dh in (32, 64, 128):
        H = 1
        q = np.zeros((1, dh), np.float32)
        k = np.zeros((2, dh), np.float32)
        v = np.zeros((2, dh), np.float32)
        q[0, 3] = 2.0
        k[0, 3] = 1.5   # s0 = 3
        k[1, 3] = -0.5  # s1 = -1
        v[0] = 1.0
        v[1] = -2.0
        out = oracle.attention(q, k, v, 1, H)
        D = (3.0 - (-1.0)) / math.sqrt(dh)
        w0 = 1.0 / (1.0 + math.exp(-D))
        want = w0 * 1.0 + (1.0 - w0) * -2.0
        assert abs(out[0, 0] - want) <= 1e-6
        for wrong in (4.0, 4.0 / dh):  # no scale; 1/d_h
            w0b = 1.0 / (1.0 + math.exp(-wrong))
            assert abs(out[0, 0] - (w0b - 2.0 * (1 - w0b))) > 1e-3


def test_attention_is_causal():
    """The page's own check: perturbing keys and values after a query's
    position leaves its output bit-identical; perturbing one at or before
    it changes the output."""
    rng = np.random.default_rng(52)
    H, dh, T, pos = 2, 32, 30, 11
    q, k, v = _rand(rng, T, H, dh)
    base = oracle.attention(q, k, v, pos, H)
    k2, v2 = k.copy(), v.copy()
    k2[pos + 1:] = rng.standard_normal(k2[pos + 1:].shape, dtype=np.float32) * np.float32(9)
    v2[pos + 1:] = 1e3
    assert np.array_equal(oracle.attention(q, k2, v2, pos, H), base)
    v3 = v.copy()
    v3[pos] += np.float32(1.0)
    assert not np.array_equal(oracle.attention(q, k, v3, pos, H), base)


def test_attention_heads_are_independent():
    """Head h reads only its own d_h columns of q, K and V."""
    rng = np.random.default_rng(53)
    H, dh, T, pos = 4, 32, 20, 19
    q, k, v = _rand(rng, T, H, dh)
    base = oracle.attention(q, k, v, pos, H)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    sl = slice(2 * dh, 3 * dh)  # head 2
    q2[:, sl] *= np.float32(-3)
    k2[:, sl] += np.float32(1)
    v2[:, sl] = 7.0
    out = oracle.attention(q2, k2, v2, pos, H)
    for h in (0, 1, 3):
        s = slice(h * dh, (h + 1) * dh)
        assert np.array_equal(out[:, s], base[:, s])
    assert np.allclose(out[:, sl], 7.0, rtol=0, atol=1e-6)


def test_attention_dominant_key():
    """One key whose score exceeds every other by far takes all the weight."""
    rng = np.random.default_rng(54)
    H, dh, T = 1, 64, 50
    q, k, v = _rand(rng, T, H, dh)
    k *= np.float32(0.01)
    k[17] = q[0] * np.float32(4.0)  # score ~ 4 |q|^2 / 8
    out = oracle.attention(q, k, v, 49, H)
    assert np.allclose(out[0], v[17], rtol=0, atol=1e-6)


def test_attention_rows_are_the_single_row_results():
    """Query rows are independent: row m of a call over M rows at pos0 is,
    bit for bit, the single-row call at position pos0 + m (the README's
    cached-decoding claim, for the oracle itself)."""
    rng = np.random.default_rng(55)
    H, dh, T = 3, 32, 70
    q, k, v = _rand(rng, T, H, dh, M=70)
    full = oracle.attention(q, k, v, 0, H)
    for t in (0, 1, 33, 69):
        one = oracle.attention(q[t:t + 1], k, v, t, H)
        assert np.array_equal(one[0], full[t])
