"""Op-level parity of the HIP path against the CPU oracle, called through
the C ABI, on seeded inputs spanning several tiles, ragged tails and the
degenerate cases of each step.  Bit-exact for x_q, s, beta, W_q, packed
bytes and int32 accumulators; fp32 y within 1e-6 relative (expected exact).
"""
import numpy as np
import pytest
import torch

import oracle
from bitlinear_matmul_amd import ug
from gpu_util import (assert_bits_equal, assert_y_close, host, pitched, scalar_dev, vec)

pytestmark = pytest.mark.gpu


def _print_case(*a):
    print("case:", *a, flush=True)


# ---------------------------------------------------------------------------
# activation quantization
# ---------------------------------------------------------------------------
ACT_SHAPES = [(32, 128), (1, 384), (1, 1536), (7, 13), (3, 1), (5, 4097), (3, 40000),
              (64, 6912), (513, 2560), (2, 1024), (9, 1023),
              # rows walked several per block, the next row's loads in flight
              (1700, 6912), (900, 3001), (1540, 1025), (770, 8192), (769, 8193)]


@pytest.mark.parametrize("M,K", ACT_SHAPES)
def test_quant_act_parity(dev, M, K):
    _print_case("quant_act", M, K)
    rng = np.random.default_rng([100, M, K])
    x = rng.standard_normal((M, K), dtype=np.float32)
    if K > 8:
        x[:, rng.choice(K, max(1, K // 100), replace=False)] *= np.float32(20)
    if M > 2:
        x[1] = 0.0                                          # all-zero row
        x[2] *= np.float32(1e-39)                           # subnormal row
    xq_d, s_d = ug.ug_quant_act(pitched(x), 1e-5)
    xq_r, s_r = oracle.quant_act(x, 1e-5)
    assert_bits_equal(host(s_d), s_r, "s")
    assert_bits_equal(host(xq_d), xq_r, "x_q")


def test_quant_act_golden_ties(dev):
    scale = np.float32(2.0 ** 20)
    ratios = np.array([127, 2.5, 3.5, -0.5, 0.5, -1.5, 126.5, -2.5, 1, 0, -127, 64.5])
    x = (ratios * float(scale)).astype(np.float32)[None, :]
    xq_d, s_d = ug.ug_quant_act(pitched(x), 1e-5)
    assert host(s_d)[0] == scale
    assert host(xq_d)[0].tolist() == [127, 2, 4, 0, 0, -2, 126, -2, 1, 0, -127, 64]


@pytest.mark.parametrize("K", [64, 2560, 6912])
def test_quant_act_near_ties(dev, K):
    """Values whose quotient x/s sits on, or a few ulps either side of, every
    half-integer k + 1/2 (|k| <= 127), for row scales of several binades:
    the kernels round through a reciprocal and form the exact quotient only
    near such points, so this is where a wrong tie band would show."""
    rng = np.random.default_rng([105, K])
    rows = []
    for amax in (127.0, 1.0, 3.0e-3, 6.5e4, 0.7):
        a = np.float32(amax)
        s = np.float32(np.float32(a / np.float32(127)) + np.float32(1e-5))
        halves = np.arange(-127, 127, dtype=np.float64) + 0.5
        base = (halves * np.float64(s)).astype(np.float32)
        cand = [base]
        for d in (1, 2, 3, 5, 8):
            cand.append(np.nextafter(base, np.float32(np.inf)))
            cand.append(np.nextafter(base, np.float32(-np.inf)))
            base = cand[-2]
        vals = np.concatenate(cand)
        vals = vals[np.abs(vals) <= a]
        row = rng.choice(vals, size=K).astype(np.float32)
        row[0] = a                                           # fixes the row max
        rows.append(row)
    x = np.stack(rows)
    xq_d, s_d = ug.ug_quant_act(pitched(x), 1e-5)
    xq_r, s_r = oracle.quant_act(x, 1e-5)
    assert_bits_equal(host(s_d), s_r, "s")
    assert_bits_equal(host(xq_d), xq_r, "x_q")
    g = np.ones(K, np.float32)
    xq_n, s_n = ug.ug_rmsnorm_quant_act(pitched(x), vec(g))
    xq_nr, s_nr = oracle.rmsnorm_quant_act(x, g)
    assert_bits_equal(host(s_n), s_nr, "s (rmsnorm)")
    assert_bits_equal(host(xq_n), xq_nr, "x_q (rmsnorm)")


def test_quant_act_rows_independent(dev):
    rng = np.random.default_rng(101)
    x = rng.standard_normal((16, 2560), dtype=np.float32)
    a, sa = ug.ug_quant_act(pitched(x))
    x[5] *= np.float32(100)
    b, sb = ug.ug_quant_act(pitched(x))
    a, b, sa, sb = host(a), host(b), host(sa), host(sb)
    keep = np.arange(16) != 5
    assert np.array_equal(a[keep], b[keep]) and np.array_equal(sa[keep], sb[keep])


# ---------------------------------------------------------------------------
# RMSNorm + quantization
# ---------------------------------------------------------------------------
RMS_SHAPES = [(4, 2560), (3, 6912), (5, 1001), (2, 9000), (6, 1), (8, 384), (2048, 2560),
              (1600, 6912), (800, 3001), (1540, 1025), (769, 8192)]


@pytest.mark.parametrize("M,K", RMS_SHAPES)
@pytest.mark.parametrize("with_gain", [False, True])
def test_rmsnorm_quant_parity(dev, M, K, with_gain):
    _print_case("rmsnorm_quant", M, K, with_gain)
    rng = np.random.default_rng([102, M, K])
    x = rng.standard_normal((M, K), dtype=np.float32) * np.float32(3)
    if M > 2:
        x[1] = np.float32(0.75)                              # constant row
    g = None
    if with_gain:
        g = np.float32(1) + rng.standard_normal(K, dtype=np.float32) * np.float32(0.1)
    xq_d, s_d = ug.ug_rmsnorm_quant_act(pitched(x), vec(g) if g is not None else None)
    xq_r, s_r = oracle.rmsnorm_quant_act(x, g)
    assert_bits_equal(host(s_d), s_r, "s")
    assert_bits_equal(host(xq_d), xq_r, "x_q")


def test_rmsnorm_quant_extreme_rows(dev):
    """RMSNorm's division x / r runs as a corrected product with 1 / r where
    quotient and input are normal, and as the division itself elsewhere:
    rows whose values, sums of squares or quotients are tiny, huge, subnormal,
    zero or overflowing must give the oracle's bits either way (900 rows:
    several per block)."""
    rng = np.random.default_rng(103)
    M, K = 900, 2560
    x = rng.standard_normal((M, K), dtype=np.float32)
    scales = [1e-30, 1e-20, 1e-12, 1e12, 1e18, 1e19, 1e20, 1e30, 1e-38, 3e-39, 0.0]
    for i, sc in enumerate(scales):
        x[7 * i] *= np.float32(sc)
    x[100, ::3] = 0.0
    x[101, :5] = np.float32(1e25)
    x[102, 7] = np.float32(3e-45)
    g = np.float32(1) + rng.standard_normal(K, dtype=np.float32) * np.float32(0.1)
    with np.errstate(over="ignore", under="ignore"):
        for gain in (None, g):
            xq_d, s_d = ug.ug_rmsnorm_quant_act(pitched(x), vec(gain) if gain is not None else None)
            xq_r, s_r = oracle.rmsnorm_quant_act(x, gain)
            assert_bits_equal(host(s_d), s_r, "s")
            assert_bits_equal(host(xq_d), xq_r, "x_q")


# ---------------------------------------------------------------------------
# absmean ternary quantization
# ---------------------------------------------------------------------------
W_SHAPES = [(512, 128), (1152, 384), (384, 1536), (6912, 2560), (2560, 6912), (300, 7), (1, 1),
            (2600, 1000), (3, 8193)]


@pytest.mark.parametrize("N,K", W_SHAPES)
def test_absmean_parity(dev, N, K):
    _print_case("absmean", N, K)
    rng = np.random.default_rng([103, N, K])
    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    wq_d, beta_d = ug.ug_quant_weight_absmean(pitched(W))
    wq_r, beta_r = oracle.quant_weight_absmean(W)
    assert_bits_equal(host(beta_d), np.array([beta_r], np.float32), "beta")
    assert_bits_equal(host(wq_d), wq_r, "W_q")


def test_absmean_pitched_input(dev):
    """A row pitch larger than K takes the strided path; same bits."""
    rng = np.random.default_rng(104)
    N, K = 700, 1000
    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    Wd = ug.empty_pitched(N, K, torch.float32, torch.device("cuda:0"), 64)  # ld = 1008
    Wd.copy_(torch.from_numpy(W))
    assert Wd.stride(0) != K
    wq_d, beta_d = ug.ug_quant_weight_absmean(Wd)
    wq_r, beta_r = oracle.quant_weight_absmean(W)
    assert host(beta_d)[0] == beta_r
    assert_bits_equal(host(wq_d), wq_r, "W_q")


def test_absmean_one_read_limits_and_shared_workspace(dev):
    """Back-to-back calls that share one workspace (the previous call's
    chunk sums still there), over tensors of 25,165,824 elements (3072
    chunks of 8192) and one more row, and the 2B-class shapes: every beta
    and W_q bit-exact."""
    rng = np.random.default_rng(106)
    dev_ = torch.device("cuda:0")
    ws = torch.empty(ug.ug_quant_weight_absmean_workspace_size(6145, 4096), dtype=torch.uint8,
                     device=dev_)
    for (N, K) in [(6144, 4096), (6145, 4096), (2560, 6912), (6912, 2560), (384, 1152)]:
        _print_case("absmean shared ws", N, K)
        W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
        W[rng.integers(0, N), :] *= np.float32(30.0)
        wq_d, beta_d = ug.ug_quant_weight_absmean(pitched(W), ws=ws)
        wq_r, beta_r = oracle.quant_weight_absmean(W)
        assert_bits_equal(host(beta_d), np.array([beta_r], np.float32), "beta %dx%d" % (N, K))
        assert_bits_equal(host(wq_d), wq_r, "W_q %dx%d" % (N, K))


def test_absmean_special_cases(dev):
    # 2^25 ones: exact 2^25 in the fixed order
    W = torch.ones((4096, 8192), dtype=torch.float32, device="cuda:0")
    wq, beta = ug.ug_quant_weight_absmean(W)
    assert host(beta)[0] == np.float32(1.0) + np.float32(1e-5)
    assert bool((wq == 1).all())
    del W, wq
    # zeros -> beta = eps, W_q = 0
    wq, beta = ug.ug_quant_weight_absmean(torch.zeros((64, 96), dtype=torch.float32,
                                                      device="cuda:0"))
    assert host(beta)[0] == np.float32(1e-5) and bool((wq == 0).all())
    # ties: W/beta = +-0.5 -> 0, +-1.5 -> +-1
    r = np.array([0.5, -0.5, 1.5, -1.5, 1, -1, 0, 2])
    W = (r * 2.0 ** 20).astype(np.float32)[None, :]
    wq, beta = ug.ug_quant_weight_absmean(pitched(W))
    assert host(beta)[0] == np.float32(2.0 ** 20)
    assert host(wq)[0].tolist() == [0, 0, 1, -1, 1, -1, 0, 1]


# ---------------------------------------------------------------------------
# pack / unpack
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("N,K", [(243, 5), (512, 128), (6912, 2560), (2560, 6912), (9, 7),
                                 (5, 1), (33, 81)])
def test_pack_parity(dev, N, K):
    _print_case("pack", N, K)
    rng = np.random.default_rng([105, N, K])
    wq = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    if N == 243 and K == 5:
        wq = np.array(np.meshgrid(*[[-1, 0, 1]] * 5, indexing="ij")).reshape(5, -1).T.astype(
            np.int8)
    bad = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    pk_d = ug.ug_pack_trits(pitched(wq), bad_count=bad)
    pk_r, bad_r = oracle.pack_trits(wq, ldp=pk_d.shape[1])
    assert_bits_equal(host(pk_d), pk_r, "packed")
    assert host(bad)[0] == bad_r == 0
    un_d = ug.ug_unpack_trits(pk_d, K, bad_count=bad)
    assert_bits_equal(host(un_d), wq, "unpacked")
    assert host(bad)[0] == 0


@pytest.mark.parametrize("N,K", [(7, 2559), (5, 2561), (3, 5121), (11, 13), (4, 7680)])
def test_pack_unpack_row_pads(dev, N, K):
    """Rows a span boundary away from K, in pitched buffers whose pads hold
    junk: pack ignores the trit bytes past K (0x55 there is no trit), unpack
    reads no pad byte of the packed rows (0xff there is no code) and writes
    none past K."""
    _print_case("pack pads", N, K)
    rng = np.random.default_rng([107, N, K])
    wq = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    ldq = -(-K // 16) * 16 + 16
    src = torch.full((N, ldq), 0x55, dtype=torch.int8, device="cuda:0")
    src[:, :K] = torch.from_numpy(wq).to(dev)
    bad = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    pk = ug.ug_pack_trits(src[:, :K], bad_count=bad)
    pk_r, _ = oracle.pack_trits(wq, ldp=pk.shape[1])
    assert_bits_equal(host(pk), pk_r, "packed")
    assert host(bad)[0] == 0
    groups = -(-K // 5)
    ldp = -(-groups // 16) * 16 + 32
    pin = torch.full((N, ldp), 0xff, dtype=torch.uint8, device="cuda:0")
    pin[:, :groups] = pk[:, :groups]
    out = torch.full((N, ldq), 0x33, dtype=torch.int8, device="cuda:0")
    ug.ug_unpack_trits(pin[:, :groups], K, wq=out[:, :K], bad_count=bad)
    assert host(bad)[0] == 0
    o = host(out)
    assert_bits_equal(o[:, :K], wq, "unpacked")
    assert bool((o[:, K:] == 0x33).all()), "unpack wrote past K"


def test_pack_every_byte_value(dev):
    """Every int8 value as a trit byte, at every position of a 5-trit group
    and of a 4-byte word: 253 of the 256 are bad, each clamped to -1 or 1."""
    vals = np.arange(-128, 128, dtype=np.int16).astype(np.int8)
    rng = np.random.default_rng(108)
    rows = [np.roll(vals, r) for r in range(20)] + [rng.permutation(vals) for _ in range(12)]
    wq = np.stack(rows)
    bad = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    pk = ug.ug_pack_trits(pitched(wq), bad_count=bad)
    pk_r, bad_r = oracle.pack_trits(wq, ldp=pk.shape[1])
    assert bad_r == 253 * wq.shape[0] and host(bad)[0] == bad_r
    assert_bits_equal(host(pk), pk_r, "packed")


def test_pack_bad_entries_and_unpack_bad_codes(dev):
    rng = np.random.default_rng(106)
    wq = rng.integers(-1, 2, size=(40, 37)).astype(np.int8)
    wq[0, 0], wq[3, 36], wq[39, 5], wq[7, 7] = 2, -5, 127, -128
    bad = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    pk = ug.ug_pack_trits(pitched(wq), bad_count=bad)
    pk_r, bad_r = oracle.pack_trits(wq, ldp=pk.shape[1])
    assert bad_r == 4 and host(bad)[0] == 4
    assert_bits_equal(host(pk), pk_r, "packed")
    # all 256 codes
    codes = np.arange(256, dtype=np.uint8).reshape(1, 256)
    codes_p = np.full((1, 256), 121, np.uint8)
    codes_p[:] = codes
    bad.zero_()
    K = 5 * 256
    un = ug.ug_unpack_trits(pitched(codes_p), K, bad_count=bad)
    un_r, bad_r = oracle.unpack_trits(codes_p, K)
    assert bad_r == 13 and host(bad)[0] == 13
    assert_bits_equal(host(un), un_r, "unpacked")


# ---------------------------------------------------------------------------
# GEMV / GEMM
# ---------------------------------------------------------------------------
def _rand_problem(rng, M, N, K):
    xq = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    wq = (rng.integers(-1, 2, size=(N, K))).astype(np.int8)
    s = (rng.random(M, dtype=np.float32) * np.float32(0.05) + np.float32(1e-3))
    beta = np.float32(0.0159)
    return xq, wq, s, beta


GEMV_CASES = [(1, 6912, 2560), (1, 2560, 6912), (4, 1152, 384), (3, 385, 1001), (5, 64, 7),
              (16, 512, 128), (64, 300, 2560), (2, 17, 81), (1, 4096, 384), (33, 1000, 160),
              (20, 700, 2560), (32, 129, 6912), (64, 64, 6912), (16, 2560, 6912),
              (1, 40, 20000), (7, 8000, 1536)]


@pytest.mark.parametrize("M,N,K", GEMV_CASES)
@pytest.mark.parametrize("fmt", [ug.UG_W_PACK5, ug.UG_W_I8])
def test_gemv_parity(dev, M, N, K, fmt):
    _print_case("gemv", M, N, K, fmt)
    rng = np.random.default_rng([107, M, N, K])
    xq, wq, s, beta = _rand_problem(rng, M, N, K)
    if fmt == ug.UG_W_PACK5:
        pk, _ = oracle.pack_trits(wq)
        w = pitched(pk)
    else:
        w = pitched(wq)
    acc_d, y_d = ug.ug_bitlinear_gemv(pitched(xq), vec(s), w, fmt, scalar_dev(beta), K=K,
                                      want_acc=True)
    acc_r = oracle.matmul_i32(xq, wq)
    y_r = oracle.epilogue(acc_r, s, beta)
    assert_bits_equal(host(acc_d), acc_r, "acc")
    assert_y_close(host(y_d), y_r, "y")
    assert_bits_equal(host(y_d), y_r, "y bits")


def test_gemv_invalid_codes_and_garbage_pad(dev):
    """Pad bytes past ceil(K/5) (here garbage, invalid codes included) and
    trits past K never change the result; a row holding an invalid code
    (243..255) among its data bytes leaves every other row exact."""
    rng = np.random.default_rng(108)
    M, N, K = 3, 70, 101  # 21 bytes used per row, pitch 32
    xq, wq, s, beta = _rand_problem(rng, M, N, K)
    pk, _ = oracle.pack_trits(wq)
    pk[:, 21:] = rng.integers(0, 256, size=(N, pk.shape[1] - 21))  # garbage pad
    # last data byte: keep its trit at k = 100, random trits at k = 101..104 (past K)
    pk[:, 20] = (pk[:, 20].astype(np.int64) % 3 + 3 * rng.integers(0, 81, N)).astype(np.uint8)
    wq_eff, bad = oracle.unpack_trits(pk, K)
    assert bad == 0
    bad_rows = [5, 9]
    pk[5, 3] = 250                                                   # invalid codes
    pk[9, 0] = 243
    for fmt_call in (ug.ug_bitlinear_gemv, ug.ug_bitlinear_gemm):
        _, y_d = fmt_call(pitched(xq), vec(s), pitched(pk), ug.UG_W_PACK5, scalar_dev(beta),
                          K=K)
        acc_r = oracle.matmul_i32(xq, wq_eff)
        y_r = oracle.epilogue(acc_r, s, beta)
        keep = np.setdiff1d(np.arange(N), bad_rows)
        assert_bits_equal(host(y_d)[:, keep], y_r[:, keep], "y")


# the last four use the 256 x 256-tile kernel (M, N >= 512), with ragged M, N
# and K edges and the XCD tile order over a grid that is not a multiple of 8
GEMM_CASES = [(1, 64, 64), (33, 129, 100), (128, 512, 128), (300, 64, 2560), (257, 1000, 1536),
              (200, 2560, 6912), (512, 6912, 2560), (600, 700, 197), (1100, 1300, 1000),
              (2048, 2560, 6912)]


@pytest.mark.parametrize("M,N,K", GEMM_CASES)
@pytest.mark.parametrize("fmt", [ug.UG_W_I8, ug.UG_W_PACK5])
def test_gemm_parity(dev, M, N, K, fmt):
    _print_case("gemm", M, N, K, fmt)
    rng = np.random.default_rng([109, M, N, K])
    xq, wq, s, beta = _rand_problem(rng, M, N, K)
    w = pitched(oracle.pack_trits(wq)[0]) if fmt == ug.UG_W_PACK5 else pitched(wq)
    acc_d, y_d = ug.ug_bitlinear_gemm(pitched(xq), vec(s), w, fmt, scalar_dev(beta), K=K,
                                      want_acc=True)
    acc_r = oracle.matmul_i32(xq, wq)
    y_r = oracle.epilogue(acc_r, s, beta)
    assert_bits_equal(host(acc_d), acc_r, "acc")
    assert_y_close(host(y_d), y_r, "y")
    assert_bits_equal(host(y_d), y_r, "y bits")


@pytest.mark.parametrize("M,N,K,splits", [(2048, 2560, 6912, None), (512, 6912, 2560, None),
                                          (1100, 1300, 1000, 2), (1100, 1300, 1000, 5),
                                          (600, 700, 197, 4), (512, 512, 64, 1)])
def test_gemm_split_matches_whole_tiles(dev, M, N, K, splits):
    """K-split launches (a tile's K steps shared by several blocks, finished
    by the last one in) give the same bits as one whole tile per block, and
    leave the shared workspace ready: a second, smaller call through the
    same workspace is right too.  splits=None keeps the library's choice;
    otherwise ug_bitlinear_gemm_tiled asks for that many (odd counts, counts
    that do not divide the K steps, one K step per split with the K tail in
    the last one)."""
    _print_case("gemm split", M, N, K, splits)
    rng = np.random.default_rng([113, M, N, K])
    xq, wq, s, beta = _rand_problem(rng, M, N, K)
    args = (pitched(xq), vec(s), pitched(wq), ug.UG_W_I8, scalar_dev(beta))
    acc_s, y_s = ug.ug_bitlinear_gemm(*args, want_acc=True, k_splits=splits)
    acc_w, y_w = ug.ug_bitlinear_gemm(*args, want_acc=True, split=False)
    assert_bits_equal(host(acc_s), host(acc_w), "acc split vs whole")
    assert_bits_equal(host(y_s), host(y_w), "y split vs whole")
    acc_r = oracle.matmul_i32(xq, wq)
    assert_bits_equal(host(acc_s), acc_r, "acc")
    m2, n2 = max(512, M // 2 + 3), max(512, N // 2 + 5)
    acc2, y2 = ug.ug_bitlinear_gemm(pitched(xq[:m2]), vec(s[:m2]), pitched(wq[:n2]), ug.UG_W_I8,
                                    scalar_dev(beta), want_acc=True)
    assert_bits_equal(host(acc2), acc_r[:m2, :n2], "acc second call")
    assert_bits_equal(host(y2), oracle.epilogue(acc_r[:m2, :n2], s[:m2], beta), "y second call")


@pytest.mark.parametrize("shape", [0, 1])
@pytest.mark.parametrize("M,N,K,splits", [(600, 700, 197, 1), (1100, 1300, 1000, 1),
                                          (1100, 1300, 1000, 3), (512, 2560, 6912, 2)])
def test_gemm_tile_shapes(dev, shape, M, N, K, splits):
    """Each large-tile shape (256 x 256 and 256 x 160 output tiles),
    whole or K-split, against the oracle: ragged M, N and K edges, partial
    tiles of every column-piece width in the output pass."""
    _print_case("gemm shape", shape, M, N, K, splits)
    rng = np.random.default_rng([127, M, N, K])
    xq, wq, s, beta = _rand_problem(rng, M, N, K)
    acc_d, y_d = ug.ug_bitlinear_gemm(pitched(xq), vec(s), pitched(wq), ug.UG_W_I8,
                                      scalar_dev(beta), want_acc=True, tile=shape,
                                      k_splits=splits)
    acc_r = oracle.matmul_i32(xq, wq)
    assert_bits_equal(host(acc_d), acc_r, "acc")
    assert_bits_equal(host(y_d), oracle.epilogue(acc_r, s, beta), "y")


def test_gemm_split_after_packed_calls(dev):
    """Packed-weight calls that decode weights into the shared workspace
    (one too large to split, one that splits) must leave the split counters
    alone: a split call afterwards still matches one whole tile per block."""
    rng = np.random.default_rng(117)
    xb, wb, sb, bb = _rand_problem(rng, 2048, 6912, 640)
    pk = pitched(oracle.pack_trits(wb)[0])
    _, yb = ug.ug_bitlinear_gemm(pitched(xb), vec(sb), pk, ug.UG_W_PACK5, scalar_dev(bb), K=640)
    _, yb8 = ug.ug_bitlinear_gemm(pitched(xb), vec(sb), pitched(wb), ug.UG_W_I8, scalar_dev(bb))
    assert_bits_equal(host(yb), host(yb8), "large packed vs bytes")
    xq, wq, s, beta = _rand_problem(rng, 512, 6912, 2560)
    pk2 = pitched(oracle.pack_trits(wq)[0])
    acc5, _ = ug.ug_bitlinear_gemm(pitched(xq), vec(s), pk2, ug.UG_W_PACK5, scalar_dev(beta),
                                   K=2560, want_acc=True)
    args = (pitched(xq), vec(s), pitched(wq), ug.UG_W_I8, scalar_dev(beta))
    acc_s, _ = ug.ug_bitlinear_gemm(*args, want_acc=True)
    acc_w, _ = ug.ug_bitlinear_gemm(*args, want_acc=True, split=False)
    assert_bits_equal(host(acc5), host(acc_w), "packed split vs whole")
    assert_bits_equal(host(acc_s), host(acc_w), "split vs whole after packed calls")


def test_gemm_split_any_workspace_contents(dev):
    """The split counters carry the launch they belong to (a 56-bit launch
    number that starts at random per process), so a workspace full of
    arbitrary bytes, of counter words of small launch numbers (those of
    launches 1..400 of any process), or of decoded trits (00/01/FF bytes)
    is fine; and a packed-weight call that decodes into a workspace too
    small for the split area leaves the counter bytes alone."""
    rng = np.random.default_rng(119)
    M, N, K = 1024, 1024, 1536
    xq, wq, s, beta = _rand_problem(rng, M, N, K)
    need = ug.ug_bitlinear_gemm_workspace_size(M, N, K, ug.UG_W_I8)
    g = torch.Generator(device="cpu").manual_seed(5)
    ws = torch.randint(0, 256, (need,), dtype=torch.uint8, generator=g).to("cuda:0")
    args = (pitched(xq), vec(s), pitched(wq), ug.UG_W_I8, scalar_dev(beta))
    acc_r = oracle.matmul_i32(xq, wq)
    n_words = ug.UG_GEMM_COUNTER_BYTES // 8
    fills = {
        "random bytes": lambda: torch.randint(0, 256, (ug.UG_GEMM_COUNTER_BYTES,),
                                              dtype=torch.uint8, generator=g),
        "small epochs": lambda: torch.from_numpy(
            ((np.arange(n_words, dtype=np.int64) % 400 + 1) << 8
             | rng.integers(0, 8, n_words)).astype(np.int64)).view(torch.uint8),
        "trit bytes": lambda: torch.from_numpy(
            rng.choice(np.array([0, 1, 255], np.uint8), ug.UG_GEMM_COUNTER_BYTES)),
    }
    for name, fill in fills.items():
        for rep in range(2):
            ws[:ug.UG_GEMM_COUNTER_BYTES] = fill().to("cuda:0")
            acc_s, _ = ug.ug_bitlinear_gemm(*args, want_acc=True, ws=ws, k_splits=3)
            assert_bits_equal(host(acc_s), acc_r, "acc, %s, call %d" % (name, rep))
    # a packed call whose decoded weights do not leave room for the split
    # area: they go after the counter bytes, which stay as they were
    before = ws[:ug.UG_GEMM_COUNTER_BYTES].clone()
    xs, ws5, ss, bs = _rand_problem(rng, 300, 700, 1000)
    pk = pitched(oracle.pack_trits(ws5)[0])
    small = ws[:ug.UG_GEMM_COUNTER_BYTES + 700 * 1008]
    acc5, _ = ug.ug_bitlinear_gemm(pitched(xs), vec(ss), pk, ug.UG_W_PACK5, scalar_dev(bs),
                                   K=1000, want_acc=True, ws=small)
    assert_bits_equal(host(acc5), oracle.matmul_i32(xs, ws5), "packed acc, small workspace")
    assert torch.equal(ws[:ug.UG_GEMM_COUNTER_BYTES], before)
    acc_s, _ = ug.ug_bitlinear_gemm(*args, want_acc=True, ws=ws, k_splits=3)
    assert_bits_equal(host(acc_s), acc_r, "acc after the packed call")


def test_gemm_extreme_values(dev):
    """|acc| at its largest: x_q = +-127 everywhere against all +-1 rows."""
    M, N, K = 64, 64, 6912
    xq = np.full((M, K), 127, np.int8)
    xq[1::2] = -127
    wq = np.ones((N, K), np.int8)
    wq[::3] = -1
    s = np.full(M, np.float32(0.5))
    acc_d, _ = ug.ug_bitlinear_gemm(pitched(xq), vec(s), pitched(wq), ug.UG_W_I8,
                                    scalar_dev(np.float32(1)), want_acc=True)
    assert_bits_equal(host(acc_d), oracle.matmul_i32(xq, wq), "acc")
    acc_v, _ = ug.ug_bitlinear_gemv(pitched(xq), vec(s), pitched(wq), ug.UG_W_I8,
                                    scalar_dev(np.float32(1)), want_acc=True)
    assert_bits_equal(host(acc_v), oracle.matmul_i32(xq, wq), "acc gemv")


@pytest.mark.parametrize("M,N,K,fmt,path", [
    (1, 1152, 384, 1, "gemv"), (4, 700, 333, 0, "gemv"), (16, 2560, 6912, 1, "gemv"),
    (64, 2560, 2560, 1, "gemv"), (33, 1000, 640, 0, "gemv"),
    (32, 512, 128, 0, "gemm"), (300, 700, 197, 0, "gemm"), (2048, 2560, 6912, 0, "gemm"),
    (4096, 6912, 2560, 0, "gemm"), (600, 1300, 1000, 1, "gemm")])
def test_bias_epilogue(dev, M, N, K, fmt, path):
    """The deployed forward with its bias ("autograd on a byte-graph":
    y = (x_q W_q^T)(s beta) + b): y bit-exact against the oracle's
    fl(fl(acc * fl(s * beta)) + b[n]); acc unchanged by the bias; every
    matmul kernel (fine, stream and chunked GEMV splits; small, large and
    K-split GEMM tiles; ragged edges)."""
    _print_case("bias", M, N, K, fmt, path)
    rng = np.random.default_rng([131, M, N, K])
    xq, wq, s, beta = _rand_problem(rng, M, N, K)
    bias = rng.standard_normal(N, dtype=np.float32)
    w = pitched(oracle.pack_trits(wq)[0]) if fmt == ug.UG_W_PACK5 else pitched(wq)
    fn = ug.ug_bitlinear_gemv if path == "gemv" else ug.ug_bitlinear_gemm
    acc_d, y_d = fn(pitched(xq), vec(s), w, fmt, scalar_dev(beta), K=K, want_acc=True,
                    bias=vec(bias))
    acc_r = oracle.matmul_i32(xq, wq)
    assert_bits_equal(host(acc_d), acc_r, "acc")
    assert_bits_equal(host(y_d), oracle.epilogue(acc_r, s, beta, bias), "y with bias")


# ---------------------------------------------------------------------------
# matrix-core rate probe (a measurement helper)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("kind", [0, 1])
def test_mfma_rate_probe_runs_and_repeats(dev, kind):
    """The probe's operands come from the block and thread index only, so
    two calls write the same words, and different waves different ones."""
    blocks = 8
    a = torch.zeros(4 * blocks, dtype=torch.int32, device="cuda:0")
    b = torch.ones(4 * blocks, dtype=torch.int32, device="cuda:0")
    ops = ug.ug_mfma_rate_probe(kind, blocks, 3, a)
    ug.ug_mfma_rate_probe(kind, blocks, 3, b)
    torch.cuda.synchronize()
    assert ops == 4 * blocks * 3 * 16 * (65536 if kind == 0 else 2048)
    assert torch.equal(a, b)
    assert len(set(host(a).tolist())) > 1


# HBM read-rate probe (a measurement helper)
@pytest.mark.parametrize("walk", [0, 1])
@pytest.mark.parametrize("words,blocks", [(4, 1), (4, 3), (1000 * 4, 3), (262144 * 4 + 12, 2048),
                                          (262144 * 4 + 12, 1000)])
def test_hbm_read_probe_reads_every_word(dev, words, blocks, walk):
    """The XOR of the probe's sink words is the XOR of every 32-bit word of
    the buffer (ragged tails, blocks with empty ranges: each word read once)."""
    rng = np.random.default_rng([540, words])
    host_words = rng.integers(0, 2 ** 32, size=words, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(host_words.view(np.int32)).to(dev)
    sink = torch.zeros(4 * blocks, dtype=torch.int32, device=dev)
    n = ug.ug_hbm_read_probe(buf, blocks, sink, walk=walk)
    assert n == 4 * words
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host_words)
