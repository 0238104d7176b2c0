"""Pins for the CPU oracle: checks of it against what the pages and the
mathematics fix -- hand-worked examples (tests/golden), closed forms,
invariants, special cases and brute force on tiny inputs -- chosen so that a
plausible slip in the oracle (wrong rounding rule, dropped term, wrong index,
transposed operand, wrong clip range) fails at least one of them.

Page references: "ultragraph - when the graph is the 1-bit LLM, part 2"
(sections "the bytes", "autograd on a byte-graph", "attention, as graph
ops"), "ultragraph-1bit 0.12.0" README (sections "A whole ternary GPT",
"Layout"), "a 1-bit llm, from scratch" (its tl;dr: 31% zeros).
"""
import math
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
from bitlinear_matmul_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
EPS32 = np.float32(1e-5)
U = 2.0 ** -24  # unit roundoff of binary32


def _read_kv(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split(":", 1)
            out[k.strip()] = v.split()
    return out


def _round_half_even_f64(v):
    return np.round(v)  # numpy rounds half to even


# ---------------------------------------------------------------------------
# Activation quantization ("the bytes": s = max|x|/127 + eps,
# x_q = clip(round(x/s), -127, 127))
# ---------------------------------------------------------------------------
def test_act_quant_golden_ties():
    g = _read_kv("act_quant_ties.txt")
    scale = np.float32(2.0 ** int(g["scale_pow2"][0]))
    ratios = np.array([float(v) for v in g["ratios"]], np.float64)
    x = (ratios * float(scale)).astype(np.float32)[None, :]
    assert np.all(x.astype(np.float64) == ratios * float(scale))  # exact inputs
    xq, s = oracle.quant_act(x, float(g["eps"][0]))
    assert s[0] == scale * np.float32(float(g["s_over_scale"][0]))
    assert xq[0].tolist() == [int(v) for v in g["x_q"]]


def test_act_quant_range_and_sign_invariants():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((64, 333), dtype=np.float32) * np.float32(3.0)
    x[5] *= np.float32(1e-3)
    x[7, :] = 0.0
    x[9, 17] = np.float32(-40.0)  # negative arg-max
    xq, s = oracle.quant_act(x)
    assert xq.min() >= -127 and xq.max() <= 127
    # sign(x_q) is sign(x) or 0
    sx, sq = np.sign(x), np.sign(xq)
    assert np.all((sq == 0) | (sq == sx))
    # all-zero row: s = eps, x_q = 0
    assert s[7] == EPS32 and np.all(xq[7] == 0)
    # negative arg-max maps to exactly -127 (never -128)
    assert xq[9, 17] == -127
    # arg-max of every row with max|x| >= 0.3213 maps to +-127
    a = np.abs(x).max(axis=1)
    for m in range(x.shape[0]):
        if a[m] >= 0.3213:
            k = int(np.argmax(np.abs(x[m])))
            assert abs(int(xq[m, k])) == 127
    # monotone within a row
    for m in range(0, 64, 9):
        order = np.argsort(x[m], kind="stable")
        assert np.all(np.diff(xq[m, order].astype(np.int32)) >= 0)


def test_act_quant_float64_brute_force():
    """x_q agrees with a float64 evaluation except within 1e-5 of a .5 tie;
    s agrees with float64 a/127 + eps to two roundings."""
    rng = np.random.default_rng(12)
    x = rng.standard_normal((40, 257), dtype=np.float32)
    x[:, 3] *= np.float32(20.0)
    xq, s = oracle.quant_act(x)
    a = np.abs(x.astype(np.float64)).max(axis=1)
    s64 = a / 127.0 + 1e-5
    assert np.all(np.abs(s.astype(np.float64) - s64) <= 2.5 * U * s64)
    q64 = x.astype(np.float64) / s64[:, None]
    ref = np.clip(_round_half_even_f64(q64), -127, 127)
    near_tie = np.abs(np.abs(q64 - np.floor(q64)) - 0.5) < 1e-5
    mism = (xq != ref) & ~near_tie
    assert not mism.any()
    # dequantization error of every element is at most s/2 (plus rounding)
    err = np.abs(x.astype(np.float64) - s.astype(np.float64)[:, None] * xq)
    assert np.all(err <= s.astype(np.float64)[:, None] * (0.5 + 4 * U))


def test_act_quant_rows_independent():
    """The pages' causality check: perturbing one row (token) leaves every
    other row's x_q and s bit-identical ("attention, as graph ops")."""
    rng = np.random.default_rng(13)
    x = rng.standard_normal((16, 100), dtype=np.float32)
    xq0, s0 = oracle.quant_act(x)
    x2 = x.copy()
    x2[6] *= np.float32(50.0)
    x2[6, 3] = np.float32(1e4)
    xq1, s1 = oracle.quant_act(x2)
    keep = np.arange(16) != 6
    assert np.array_equal(xq0[keep], xq1[keep]) and np.array_equal(s0[keep], s1[keep])
    assert not np.array_equal(xq0[6], xq1[6])


# ---------------------------------------------------------------------------
# RMSNorm ("attention, as graph ops": x / sqrt(mean x^2 + eps) * g)
# ---------------------------------------------------------------------------
def test_rmsnorm_constant_row_quantizes_to_full_scale():
    for c in (0.75, -3.0, 1e-2):
        x = np.full((2, 300), np.float32(c), np.float32)
        xn = oracle.rmsnorm(x)
        r = math.sqrt(c * c + 1e-5)
        assert np.allclose(xn, c / r, rtol=4 * U, atol=0)
        xq, _ = oracle.rmsnorm_quant_act(x)
        assert np.all(xq == (127 if c > 0 else -127))


def test_rmsnorm_float64_bound_and_gain():
    rng = np.random.default_rng(14)
    for K in (7, 384, 1536, 2560, 6912):
        x = rng.standard_normal((5, K), dtype=np.float32)
        g = (np.float32(1.0) + rng.standard_normal(K, dtype=np.float32) * np.float32(0.1))
        xn = oracle.rmsnorm(x, g)
        x64 = x.astype(np.float64)
        r64 = np.sqrt((x64 * x64).mean(axis=1) + 1e-5)
        ref = x64 / r64[:, None] * g.astype(np.float64)
        depth = math.ceil(K / 1024) + 8
        bound = (depth / 2 + 6) * U
        assert np.all(np.abs(xn - ref) <= bound * np.abs(ref) + 1e-30)


def test_row_sum_squares_exact_cases():
    # a single non-zero anywhere: every order gives x^2 exactly (catches a
    # dropped or misplaced element)
    K = 6912
    for pos in (0, 1, 3, 4, 1023, 1024, 4095, 4096, 5000, K - 1):
        x = np.zeros(K, np.float32)
        x[pos] = np.float32(3.0)
        assert oracle.row_sum_squares(x) == np.float32(9.0)
    # all ones: integer partial sums are exact, T = K
    for K in (1, 5, 1024, 1025, 6912):
        assert oracle.row_sum_squares(np.ones(K, np.float32)) == np.float32(K)
    # fsum bound on random data
    rng = np.random.default_rng(15)
    x = rng.standard_normal(6912, dtype=np.float32)
    sq = (x * x).astype(np.float64)  # fl(x*x) is exact in float64
    exact = math.fsum((x.astype(np.float64) ** 2).tolist())
    d = math.ceil(6912 / 1024) + 8
    assert abs(float(oracle.row_sum_squares(x)) - exact) <= d * U / (1 - d * U) * sq.sum() + U * sq.sum()


def test_rmsnorm_rows_independent():
    rng = np.random.default_rng(16)
    x = rng.standard_normal((8, 2560), dtype=np.float32)
    a, sa = oracle.rmsnorm_quant_act(x)
    x[2] *= np.float32(7.0)
    b, sb = oracle.rmsnorm_quant_act(x)
    keep = np.arange(8) != 2
    assert np.array_equal(a[keep], b[keep]) and np.array_equal(sa[keep], sb[keep])


def test_rmsnorm_quant_equals_quant_of_rmsnorm():
    rng = np.random.default_rng(17)
    x = rng.standard_normal((6, 1000), dtype=np.float32)
    g = rng.random(1000, dtype=np.float32) + np.float32(0.5)
    xq, s = oracle.rmsnorm_quant_act(x, g)
    xq2, s2 = oracle.quant_act(oracle.rmsnorm(x, g))
    assert np.array_equal(xq, xq2) and np.array_equal(s, s2)


# ---------------------------------------------------------------------------
# Absmean ("the bytes": beta = (1/n) sum |W_i| + eps)
# ---------------------------------------------------------------------------
def _depth(n):
    nchunks = -(-n // 8192)
    return 8 + 2 + 8 + math.ceil(nchunks / 256) + 8


def test_absmean_sum_within_fsum_bound():
    for (N, K, seed) in ((512, 128, 0), (1152, 384, 1), (300, 7, 2), (6912, 2560, 3)):
        rng = np.random.default_rng(seed)
        W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
        T = oracle.absmean_sum(W)
        a = np.abs(W).astype(np.float64).ravel()
        exact = math.fsum(a.tolist())
        d = _depth(N * K)
        gam = d * U / (1 - d * U)
        assert abs(float(T) - exact) <= gam * exact


def test_absmean_single_nonzero_anywhere():
    """One non-zero element at any flat position: the sum is that value
    exactly, so no element is dropped or double counted, including in the
    padded last chunk and past the first 256 chunks."""
    N, K = 2600, 1000  # n = 2.6e6, 318 chunks, ragged tail
    n = N * K
    W = np.zeros((N, K), np.float32)
    for e in (0, 1, 3, 4, 1023, 1024, 8191, 8192, 256 * 8192 + 5, n - 8191, n - 1):
        W.flat[e] = np.float32(-0.125)
        assert oracle.absmean_sum(W) == np.float32(0.125), e
        W.flat[e] = 0.0


def test_absmean_sum_is_not_sequential():
    """2^25 ones: any left-to-right fp32 sum stalls at 2^24, while the fixed
    two-stage pairwise order keeps every partial sum an exact integer below
    2^24 and returns 2^25 exactly."""
    W = np.ones((4096, 8192), np.float32)
    assert oracle.absmean_sum(W) == np.float32(2.0 ** 25)
    wq, beta = oracle.quant_weight_absmean(W)
    assert beta == np.float32(1.0) + EPS32 and np.all(wq == 1)


def test_absmean_closed_forms():
    # constant tensor c: beta = |c| + eps (sums of 0.25 are exact here)
    W = np.full((256, 256), np.float32(-0.25), np.float32)
    wq, beta = oracle.quant_weight_absmean(W)
    assert beta == np.float32(0.25) + EPS32
    assert np.all(wq == -1)
    # all zeros: beta = eps, W_q = 0
    wq, beta = oracle.quant_weight_absmean(np.zeros((64, 96), np.float32))
    assert beta == EPS32 and np.all(wq == 0)


def test_absmean_gaussian_expectation_and_zero_fraction():
    """For W ~ N(0, sigma^2): E|W| = sigma sqrt(2/pi), and the zero fraction
    is P(|W| <= beta/2) = erf(1/(2 sqrt(pi))) = 0.31006 -- the 31% of exactly
    zero weights reported on "a 1-bit llm, from scratch" (tl;dr)."""
    x, W = inputs.tiny_layer()
    wq, beta = oracle.quant_weight_absmean(W)
    n = W.size
    sigma = 0.02
    e_beta = sigma * math.sqrt(2 / math.pi) + 1e-5
    sd = sigma * math.sqrt(1 - 2 / math.pi) / math.sqrt(n)
    assert abs(float(beta) - e_beta) < 5 * sd
    p0 = math.erf(1 / (2 * math.sqrt(math.pi)))
    assert abs(p0 - 0.31006) < 1e-5
    frac = float((wq == 0).mean())
    assert abs(frac - p0) < 5 * math.sqrt(p0 * (1 - p0) / n)
    assert abs(frac - 0.31) < 0.01


# ---------------------------------------------------------------------------
# Ternary quantization (W_q = clip(round(W/beta), -1, 1))
# ---------------------------------------------------------------------------
def test_ternary_golden_ties():
    g = _read_kv("ternary_ties.txt")
    scale = 2.0 ** int(g["scale_pow2"][0])
    ratios = np.array([float(v) for v in g["ratios"]], np.float64)
    W = (ratios * scale).astype(np.float32)[None, :]
    wq, beta = oracle.quant_weight_absmean(W, float(g["eps"][0]))
    assert beta == np.float32(scale * float(g["beta_over_scale"][0]))
    assert wq[0].tolist() == [int(v) for v in g["w_q"]]


def test_ternary_threshold_form():
    """clip(round(q), -1, 1) with round half to even is sign(q)[|q| > 1/2]."""
    rng = np.random.default_rng(21)
    W = rng.standard_normal((700, 333), dtype=np.float32) * np.float32(0.02)
    wq, beta = oracle.quant_weight_absmean(W)
    q = W / beta  # binary32 division, correctly rounded
    ref = np.sign(q) * (np.abs(q) > np.float32(0.5))
    assert np.array_equal(wq, ref.astype(np.int8))
    assert set(np.unique(wq).tolist()) == {-1, 0, 1}


# ---------------------------------------------------------------------------
# Five trits per byte (README "A whole ternary GPT" / "Layout": pack.py)
# ---------------------------------------------------------------------------
def _all_tuples():
    t = np.array(np.meshgrid(*[[-1, 0, 1]] * 5, indexing="ij")).reshape(5, -1).T
    return np.ascontiguousarray(t.astype(np.int8))  # [243, 5]


def test_pack_golden_codes():
    rows, codes = [], []
    with open(os.path.join(GOLDEN, "pack_codes.txt")) as f:
        for line in f:
            if line.startswith("#") or "->" not in line:
                continue
            a, b = line.split("->")
            rows.append([int(v) for v in a.split()])
            codes.append(int(b))
    packed, bad = oracle.pack_trits(np.array(rows, np.int8), ldp=1)
    assert bad == 0
    assert packed[:, 0].tolist() == codes


def test_pack_exhaustive_bijection_and_roundtrip():
    t = _all_tuples()
    packed, bad = oracle.pack_trits(t, ldp=1)
    assert bad == 0
    codes = packed[:, 0].astype(np.int64)
    assert sorted(codes.tolist()) == list(range(243))
    # negation maps code b to 242 - b
    pneg, _ = oracle.pack_trits((-t).astype(np.int8), ldp=1)
    assert np.array_equal(pneg[:, 0].astype(np.int64), 242 - codes)
    back, bad = oracle.unpack_trits(packed, 5)
    assert bad == 0 and np.array_equal(back, t)


def test_unpack_all_256_codes():
    b = np.arange(256, dtype=np.uint8)[:, None]
    wq, bad = oracle.unpack_trits(b, 5)
    assert bad == 13  # codes 243..255
    assert np.all(wq[243:] == 0)
    repacked, _ = oracle.pack_trits(wq[:243], ldp=1)
    assert np.array_equal(repacked[:, 0], np.arange(243, dtype=np.uint8))


def test_pack_tail_padding_and_bad_entries():
    rng = np.random.default_rng(22)
    K = 7  # groups: [0..4], [5, 6, pad, pad, pad]
    wq = rng.integers(-1, 2, size=(9, K)).astype(np.int8)
    packed, bad = oracle.pack_trits(wq, ldp=16)
    assert bad == 0
    assert np.all(packed[:, 2:] == 121)  # pad bytes
    # the tail byte only carries trits 5 and 6
    exp = 121 + wq[:, 5].astype(np.int64) + 3 * wq[:, 6].astype(np.int64)
    assert np.array_equal(packed[:, 1].astype(np.int64), exp)
    back, bad = oracle.unpack_trits(packed, K)
    assert bad == 0 and np.array_equal(back, wq)
    # out-of-range entries are counted and clamped
    wbad = wq.copy()
    wbad[0, 0], wbad[3, 6], wbad[8, 2] = 2, -5, 127
    pb, bad = oracle.pack_trits(wbad, ldp=16)
    assert bad == 3
    pc, _ = oracle.pack_trits(np.clip(wbad, -1, 1).astype(np.int8), ldp=16)
    assert np.array_equal(pb, pc)


def test_pack_density():
    """3^5 = 243 <= 256 < 3^6: five is the most trits a byte holds; 8/5 = 1.6
    bits per trit against log2(3) = 1.585 ("the bytes"; README "A whole
    ternary GPT": ~1.6 bits/weight)."""
    assert 3 ** 5 <= 256 < 3 ** 6
    assert abs(math.log2(3) - 1.58496) < 1e-5
    assert 8 / 5 == 1.6 and 1.6 / math.log2(3) > 0.99
    K = 2560
    wq = np.zeros((3, K), np.int8)
    packed, _ = oracle.pack_trits(wq, ldp=oracle.packed_pitch(K, align=1))
    assert packed.shape[1] == K // 5


# ---------------------------------------------------------------------------
# Integer matmul and rescale ("autograd on a byte-graph": y = (x_q W_q^T)(s b))
# ---------------------------------------------------------------------------
def test_matmul_brute_force_tiny():
    rng = np.random.default_rng(31)
    vals = np.array([-127, -1, 0, 1, 127], np.int8)
    for (M, N, K) in ((1, 1, 1), (2, 3, 5), (4, 4, 10), (3, 2, 7)):
        xq = rng.choice(vals, size=(M, K)).astype(np.int8)
        wq = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
        acc = oracle.matmul_i32(xq, wq)
        for m in range(M):
            for n in range(N):
                ref = 0
                for k in range(K):
                    ref += int(xq[m, k]) * int(wq[n, k])
                assert acc[m, n] == ref


def test_matmul_special_cases():
    rng = np.random.default_rng(32)
    K = 37
    xq = rng.integers(-127, 128, size=(5, K)).astype(np.int8)
    eye = np.eye(K, dtype=np.int8)
    assert np.array_equal(oracle.matmul_i32(xq, eye), xq.astype(np.int32))
    ones = np.ones((3, K), np.int8)
    rs = xq.astype(np.int64).sum(axis=1)
    assert np.array_equal(oracle.matmul_i32(xq, ones), np.repeat(rs[:, None], 3, 1))
    assert np.array_equal(oracle.matmul_i32(xq, -ones), -np.repeat(rs[:, None], 3, 1))
    wq = rng.integers(-1, 2, size=(11, K)).astype(np.int8)
    e = np.zeros((1, K), np.int8)
    e[0, 13] = 1
    assert np.array_equal(oracle.matmul_i32(e, wq)[0], wq[:, 13].astype(np.int32))
    # |acc| <= 127 * nnz(W_q[n])
    acc = oracle.matmul_i32(xq, wq)
    assert np.all(np.abs(acc) <= 127 * (wq != 0).sum(axis=1)[None, :])


def test_matmul_pairs_match_and_linearity():
    rng = np.random.default_rng(33)
    xq = rng.integers(-127, 128, size=(9, 200)).astype(np.int8)
    xq2 = rng.integers(-60, 61, size=(9, 200)).astype(np.int8)
    wq = rng.integers(-1, 2, size=(13, 200)).astype(np.int8)
    acc = oracle.matmul_i32(xq, wq)
    mi = rng.integers(0, 9, 50)
    ni = rng.integers(0, 13, 50)
    assert np.array_equal(oracle.matmul_i32_pairs(xq, wq, mi, ni), acc[mi, ni])
    # integer linearity in x
    s = (xq2.astype(np.int16) - xq.astype(np.int16) // 2)
    ok = (s >= -127) & (s <= 127)
    s = np.where(ok, s, 0).astype(np.int8)
    lhs = oracle.matmul_i32(s, wq)
    rhs = oracle.matmul_i32(xq2, wq) - oracle.matmul_i32(np.where(ok, xq.astype(np.int16) // 2, 0).astype(np.int8), wq)
    # rows where every entry stayed in range obey exact linearity
    rows = ok.all(axis=1)
    assert np.array_equal(lhs[rows], rhs[rows])


def test_matmul_not_transposed():
    """A non-square case where x_q W_q (instead of x_q W_q^T) would not even
    have the right shape, plus a direction check."""
    xq = np.array([[1, 2, 3]], np.int8)
    wq = np.array([[1, 0, 0], [0, 0, -1]], np.int8)
    assert oracle.matmul_i32(xq, wq).tolist() == [[1, -3]]


def test_epilogue_float64_bound():
    rng = np.random.default_rng(34)
    acc = rng.integers(-300000, 300000, size=(7, 50)).astype(np.int32)
    acc[0, 0] = 0
    s = rng.random(7, dtype=np.float32) + np.float32(0.01)
    beta = np.float32(0.0159)
    y = oracle.epilogue(acc, s, beta)
    ref = acc.astype(np.float64) * s.astype(np.float64)[:, None] * float(beta)
    assert np.all(np.abs(y - ref) <= 2.5 * U * np.abs(ref))
    assert y[0, 0] == 0.0
    # within the 1e-6 relative output tolerance by a wide margin
    nz = ref != 0
    assert np.max(np.abs(y[nz] - ref[nz]) / np.abs(ref[nz])) < 1e-6


def test_packed_and_byte_formats_agree():
    """Running from the packed bytes gives the same integers as running from
    one byte per trit (README "A whole ternary GPT": deployed logits are
    byte-exact)."""
    x, W = inputs.tiny_layer()
    r = oracle.bitlinear(x, W)
    packed, _ = oracle.pack_trits(r["wq"])
    wq2, _ = oracle.unpack_trits(packed, W.shape[1])
    assert np.array_equal(oracle.matmul_i32(r["xq"], wq2), r["acc"])


def test_batch_invariance():
    """Row m of the batched result equals the result for row m alone
    (README "A whole ternary GPT": cached decoding must reproduce the
    full-forward bits)."""
    x, W = inputs.tiny_layer()
    full = oracle.bitlinear(x, W)
    for m in (0, 13, 31):
        one = oracle.bitlinear(x[m:m + 1], W)
        assert np.array_equal(one["acc"][0], full["acc"][m])
        assert np.array_equal(one["y"][0], full["y"][m])


def test_oracle_thread_count_invariance():
    code = (
        "import sys, hashlib, numpy as np; sys.path.insert(0, %r);"
        "import oracle; from bitlinear_matmul_amd import inputs;"
        "x, W = inputs.sweep_inputs(2, 16); r = oracle.bitlinear(x, W);"
        "xr = oracle.rmsnorm_quant_act(x);"
        "h = hashlib.sha256();"
        "[h.update(np.ascontiguousarray(v).tobytes()) for v in (r['xq'], r['s'], r['wq'], r['beta'], r['acc'], r['y'], xr[0], xr[1])];"
        "print(h.hexdigest())" % os.path.dirname(GOLDEN).rsplit(os.sep, 1)[0]
    )
    outs = []
    for nt in ("1", "4"):
        env = dict(os.environ, OMP_NUM_THREADS=nt)
        outs.append(subprocess.run([sys.executable, "-c", code], env=env, check=True,
                                   capture_output=True, text=True).stdout.strip())
    assert outs[0] == outs[1] and len(outs[0]) == 64


# ---------------------------------------------------------------------------
# Order-sensitive and rounding-sensitive fixtures (tests/golden/*_order.txt,
# rounding_cases.txt).  The bounds above hold for any summation order and
# either rounding of a quotient; these cases hold for the stated ones only.
# ---------------------------------------------------------------------------
from fractions import Fraction  # noqa: E402


def f32_rne(v):
    """The binary32 value nearest to the exact rational v, ties to even
    (normal and subnormal range; no overflow handling is needed here)."""
    v = Fraction(v)
    if v == 0:
        return np.float32(0.0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    q = max(e - 23, -149)  # weight of the last significand bit
    scaled = a / (Fraction(2) ** q)
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return np.float32(sign * float(n * Fraction(2) ** q))


def rne_int(v):
    """Round an exact rational to the nearest integer, ties to even."""
    v = Fraction(v)
    n = v.numerator // v.denominator
    rem = v - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return n


def half_away_int(v):
    v = Fraction(v)
    n = int(abs(v) + Fraction(1, 2))
    return n if v >= 0 else -n


def F(x):
    return Fraction(float(x))


def _read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            if line.startswith("#") or "|" not in line:
                continue
            rows.append([c.strip() for c in line.split("|")])
    return rows


def test_f32_rne_helper():
    """The test's own rounding agrees with numpy's binary32 arithmetic on
    sums, products and quotients (each correctly rounded by IEEE 754)."""
    rng = np.random.default_rng(40)
    a = rng.standard_normal(2000, dtype=np.float32) * np.float32(37.0)
    b = rng.standard_normal(2000, dtype=np.float32) + np.float32(0.01)
    for x, y in zip(a[:400], b[:400]):
        assert f32_rne(F(x) + F(y)) == np.float32(x + y)
        assert f32_rne(F(x) * F(y)) == np.float32(x * y)
        assert f32_rne(F(x) / F(y)) == np.float32(x / y)
    assert f32_rne(Fraction(2 ** 24 + 1)) == np.float32(2 ** 24)
    assert f32_rne(Fraction(2 ** 24 + 3)) == np.float32(2 ** 24 + 4)
    assert f32_rne(Fraction(1, 2 ** 149)) == np.float32(2.0 ** -149)


def test_absmean_stated_order_fixtures():
    """tests/golden/absmean_order.txt: every lane, fold level and stage-2
    assignment of the stated two-stage order, each case hand-worked."""
    for name, shape, sets, expect, _why in _read_table("absmean_order.txt"):
        N, K = (int(v) for v in shape.split())
        W = np.zeros((N, K), np.float32)
        for kv in sets.split():
            pos, val = kv.split("=")
            W.flat[int(pos)] = np.float32(float(val))
        T = oracle.absmean_sum(W)
        assert T == np.float32(float(expect)), (name, float(T))
        # beta = fl(fl(T / n) + eps) on the same tensor
        _, beta = oracle.quant_weight_absmean(W)
        assert beta == f32_rne(F(f32_rne(F(T) / (N * K))) + F(EPS32)), name


def test_row_sum_squares_stated_order_fixtures():
    """tests/golden/row_order.txt: the slot map, the in-slot order and every
    fold level of the RMSNorm sum of squares, each case hand-worked."""
    for name, K, sets, expect, _why in _read_table("row_order.txt"):
        x = np.zeros(int(K), np.float32)
        for kv in sets.split():
            pos, val = kv.split("=")
            x[int(pos)] = np.float32(float(val))
        T = oracle.row_sum_squares(x)
        assert T == np.float32(float(expect)), (name, float(T))
        # the RMSNorm built on it: r = sqrt(fl(fl(T/K) + eps)), x_n = fl(x/r)
        xn = oracle.rmsnorm(x[None, :])
        ms = f32_rne(F(T) / int(K))
        r = np.sqrt(np.float32(f32_rne(F(ms) + F(EPS32))))  # binary32 sqrt, correctly rounded
        assert xn[0, 0] == f32_rne(F(x[0]) / F(r)), name


def _rounding_rows(kind):
    out = []
    with open(os.path.join(GOLDEN, "rounding_cases.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            parts = line.split()
            if parts[0] == kind:
                out.append(parts[1:])
    return out


def test_act_quant_true_division_cases():
    """Activation code by the correctly rounded quotient and round half to
    even ("the bytes"), on rows where a reciprocal product or rounding half
    away from zero gives a different code."""
    rows = _rounding_rows("act")
    assert len(rows) >= 5
    for a_s, x_s, *_ in rows:
        a, x = np.float32(float.fromhex(a_s)), np.float32(float.fromhex(x_s))
        xq, s = oracle.quant_act(np.array([[a, x]], np.float32))
        s_exp = f32_rne(F(f32_rne(F(a) / 127)) + F(EPS32))
        assert s[0] == s_exp
        q = f32_rne(F(x) / F(s_exp))
        code = max(-127, min(127, rne_int(F(q))))
        assert int(xq[0, 1]) == code, (a_s, x_s)
        # the case separates the stated reading from at least one other
        q_rcp = f32_rne(F(x) * F(f32_rne(Fraction(1) / F(s_exp))))
        others = {max(-127, min(127, rne_int(F(q_rcp)))),
                  max(-127, min(127, half_away_int(F(q))))}
        assert others != {code}, (a_s, x_s)


def test_act_scale_divides_by_127():
    """s = fl(fl(a / 127) + eps) exactly, over many row maxima, and the
    alternative fl(a * fl(1/127)) differs on some of them."""
    rng = np.random.default_rng(41)
    a = np.abs(rng.standard_normal(3000, dtype=np.float32)) * np.float32(9.0)
    a = np.maximum(a, np.float32(1e-3))
    _, s = oracle.quant_act(a[:, None])
    r127 = f32_rne(Fraction(1, 127))
    differs = 0
    for ai, si in zip(a, s):
        assert si == f32_rne(F(f32_rne(F(ai) / 127)) + F(EPS32))
        differs += f32_rne(F(ai) * F(r127)) != f32_rne(F(ai) / 127)
    assert differs > 0


def test_ternary_true_division_cases():
    rows = _rounding_rows("tern")
    assert len(rows) >= 3
    for A_s, w_s, *_ in rows:
        A, w = np.float32(float.fromhex(A_s)), np.float32(float.fromhex(w_s))
        wq, beta = oracle.quant_weight_absmean(np.array([[A, w]], np.float32))
        T = f32_rne(abs(F(A)) + abs(F(w)))
        b_exp = f32_rne(F(f32_rne(F(T) / 2)) + F(EPS32))
        assert beta == b_exp
        q = f32_rne(F(w) / F(b_exp))
        code = max(-1, min(1, rne_int(F(q))))
        assert int(wq[0, 1]) == code, (A_s, w_s)
        q_rcp = f32_rne(F(w) * F(f32_rne(Fraction(1) / F(b_exp))))
        others = {max(-1, min(1, rne_int(F(q_rcp)))), max(-1, min(1, half_away_int(F(q))))}
        assert others != {code}, (A_s, w_s)


def test_epilogue_grouping_cases():
    """y = fl(float(acc) * fl(s * beta)): the grouping of the forward
    formula ("autograd on a byte-graph"), on inputs where both other
    groupings round differently."""
    rows = _rounding_rows("epi")
    assert len(rows) >= 3
    for acc_s, s_s, b_s in rows:
        acc = int(acc_s)
        s, b = np.float32(float.fromhex(s_s)), np.float32(float.fromhex(b_s))
        y = oracle.epilogue(np.array([[acc]], np.int32), np.array([s], np.float32), b)
        exp = f32_rne(acc * F(f32_rne(F(s) * F(b))))
        assert y[0, 0] == exp, acc_s
        assert f32_rne(F(f32_rne(acc * F(s))) * F(b)) != exp
        assert f32_rne(F(f32_rne(acc * F(b))) * F(s)) != exp


def test_rmsnorm_exact_given_sum():
    """Given the row's sum of squares T (whose order the fixtures above pin),
    every RMSNorm output is r = sqrt(fl(fl(T/K) + eps)) correctly rounded and
    x_n = fl(fl(x / r) * g) ("attention, as graph ops": divide by the root,
    then the fp32 gain), checked with exact rationals."""
    rng = np.random.default_rng(42)
    for K in (5, 300, 2560):
        x = rng.standard_normal((3, K), dtype=np.float32) * np.float32(2.5)
        g = np.float32(1.0) + rng.standard_normal(K, dtype=np.float32) * np.float32(0.2)
        xn = oracle.rmsnorm(x, g)
        for m in range(3):
            T = oracle.row_sum_squares(x[m])
            v = f32_rne(F(f32_rne(F(T) / K)) + F(EPS32))
            r = f32_rne(Fraction(math.sqrt(float(v))))  # float64 sqrt, then binary32
            # r is the correctly rounded binary32 root of v: (r -+ half ulp)^2 bracket v
            ulp = F(np.spacing(r))
            assert (F(r) - ulp / 2) ** 2 <= F(v) <= (F(r) + ulp / 2) ** 2
            for k in range(0, K, max(1, K // 97)):
                assert xn[m, k] == f32_rne(F(f32_rne(F(x[m, k]) / F(r))) * F(g[k])), (K, m, k)


def test_epilogue_bias_cases():
    """With the bias of the deployed forward ("autograd on a byte-graph":
    y = (x_q W_q^T)(s beta) + b): the rescale is rounded, then b is added
    and rounded, on inputs where one fused multiply-add would round
    differently; and a zero bias changes no bit."""
    rows = _rounding_rows("bias")
    assert len(rows) >= 3
    for acc_s, s_s, b_s, c_s in rows:
        acc = int(acc_s)
        s, b, c = (np.float32(float.fromhex(v)) for v in (s_s, b_s, c_s))
        y = oracle.epilogue(np.array([[acc]], np.int32), np.array([s], np.float32), b,
                            np.array([c], np.float32))
        sc = f32_rne(F(s) * F(b))
        exp = f32_rne(F(f32_rne(acc * F(sc))) + F(c))
        assert y[0, 0] == exp, acc_s
        assert f32_rne(acc * F(sc) + F(c)) != exp
    rng = np.random.default_rng(43)
    acc = rng.integers(-30000, 30000, size=(5, 40)).astype(np.int32)
    sv = rng.random(5, dtype=np.float32) + np.float32(0.01)
    y0 = oracle.epilogue(acc, sv, np.float32(0.02))
    y1 = oracle.epilogue(acc, sv, np.float32(0.02), np.zeros(40, np.float32))
    assert np.array_equal(y0.view(np.uint32), y1.view(np.uint32))
    bias = rng.standard_normal(40, dtype=np.float32)
    y2 = oracle.epilogue(acc, sv, np.float32(0.02), bias)
    assert np.array_equal(y2, (y0 + bias[None, :]).astype(np.float32))

