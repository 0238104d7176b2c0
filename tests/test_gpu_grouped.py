"""Grouped decode GEMV (ug_gemv_plan_init + ug_bitlinear_gemv_grouped):
several independent problems in one launch, optionally quantizing fp32
activations inside the launch.  Every problem is compared with the CPU
oracle: x_q, s, int32 accumulators bit-exact, y within 1e-6 relative."""
import numpy as np
import pytest
import torch

import oracle
from bitlinear_matmul_amd import inputs, ug
from gpu_util import assert_bits_equal, assert_y_close, host, pitched, scalar_dev, vec

pytestmark = pytest.mark.gpu


def _case(*a):
    print("case:", *a, flush=True)


def test_decode_stack_one_launch_fused_quant(dev):
    """All 33 matrices of the batch-1 decode pass, fp32 activations in, one
    launch: act quant + GEMV."""
    probs, refs = [], []
    for (layer, mi, name, K, N) in inputs.decode_stack_shapes():
        x, W = inputs.decode_stack_matrix(layer, mi, K, N)
        wq_r, beta_r = oracle.quant_weight_absmean(W)
        pk_r, _ = oracle.pack_trits(wq_r)
        p = dict(x=pitched(x), w=pitched(pk_r), wfmt=ug.UG_W_PACK5, beta=scalar_dev(beta_r),
                 K=K, xq=ug.empty_pitched(1, K, torch.int8, dev),
                 s=torch.empty(1, dtype=torch.float32, device=dev),
                 y=ug.empty_pitched(1, N, torch.float32, dev),
                 acc=ug.empty_pitched(1, N, torch.int32, dev))
        probs.append(p)
        xq_r, s_r = oracle.quant_act(x)
        acc_r = oracle.matmul_i32(xq_r, wq_r)
        refs.append((xq_r, s_r, acc_r, oracle.epilogue(acc_r, s_r, beta_r)))
    plan = ug.ug_gemv_plan_init(probs)
    assert plan.info.count == 33
    ug.ug_bitlinear_gemv_grouped(plan)
    for i, (p, (xq_r, s_r, acc_r, y_r)) in enumerate(zip(probs, refs)):
        assert_bits_equal(host(p["xq"]), xq_r, "x_q %d" % i)
        assert_bits_equal(host(p["s"]), s_r, "s %d" % i)
        assert_bits_equal(host(p["acc"]), acc_r, "acc %d" % i)
        assert_y_close(host(p["y"]), y_r, "y %d" % i)
        assert_bits_equal(host(p["y"]), y_r, "y bits %d" % i)
    # replay: same bits
    y0 = [host(p["y"]).copy() for p in probs]
    ug.ug_bitlinear_gemv_grouped(plan)
    for p, a in zip(probs, y0):
        assert_bits_equal(host(p["y"]), a, "replay")


@pytest.mark.parametrize("M,shapes", [(1, [(1152, 384), (384, 384), (1536, 384), (384, 1536)]),
                                      (4, [(6912, 2560), (2560, 2560)]),
                                      (1, [(6912, 2560), (2560, 6912)] * 8)])
def test_grouped_bias_fused(dev, M, shapes):
    """Grouped launches with a bias per problem (the deployed forward's
    "+ b", "autograd on a byte-graph"), fp32 activations quantized in the
    launch: the fine split (the decode pass) and the stream split."""
    rng = np.random.default_rng([311, M, len(shapes)])
    probs, refs = [], []
    for i, (N, K) in enumerate(shapes):
        _case("grouped bias", M, i, N, K)
        x = rng.standard_normal((M, K), dtype=np.float32)
        W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
        b = rng.standard_normal(N, dtype=np.float32) * np.float32(0.1)
        wq_r, beta_r = oracle.quant_weight_absmean(W)
        pk_r, _ = oracle.pack_trits(wq_r)
        p = dict(x=pitched(x), w=pitched(pk_r), wfmt=ug.UG_W_PACK5, beta=scalar_dev(beta_r),
                 K=K, bias=vec(b), y=ug.empty_pitched(M, N, torch.float32, dev),
                 acc=ug.empty_pitched(M, N, torch.int32, dev))
        probs.append(p)
        xq_r, s_r = oracle.quant_act(x)
        acc_r = oracle.matmul_i32(xq_r, wq_r)
        refs.append((acc_r, oracle.epilogue(acc_r, s_r, beta_r, b)))
    plan = ug.ug_gemv_plan_init(probs)
    ug.ug_bitlinear_gemv_grouped(plan)
    for i, (p, (acc_r, y_r)) in enumerate(zip(probs, refs)):
        assert_bits_equal(host(p["acc"]), acc_r, "acc %d" % i)
        assert_bits_equal(host(p["y"]), y_r, "y with bias %d" % i)


def _staged_kp(wfmt, M, K):
    rb = -(-K // 5) if wfmt == ug.UG_W_PACK5 else K
    cls = 0 if M <= 16 else (1 if M <= 32 else 2)
    u = (2, 2, 1)[cls] if wfmt == ug.UG_W_PACK5 else (4, 4, 2)[cls]
    steps = -(-rb // 64)
    return (320 if wfmt == ug.UG_W_PACK5 else 64) * u * -(-steps // u)


GROUPS = [
    # (wfmt, M, list of (N, K)) -- M fixes the activation-row class
    (ug.UG_W_PACK5, 1, [(6912, 2560), (2560, 6912), (2560, 2560), (17, 7), (100, 81)]),
    (ug.UG_W_PACK5, 4, [(6912, 2560), (2560, 6912), (1000, 1001)]),
    (ug.UG_W_PACK5, 16, [(512, 384), (2560, 6912), (33, 1536)]),
    (ug.UG_W_PACK5, 20, [(300, 2560), (64, 3000)]),
    (ug.UG_W_PACK5, 64, [(256, 1280), (100, 320), (16, 7)]),
    (ug.UG_W_I8, 1, [(512, 128), (2560, 4000), (70, 33)]),
    (ug.UG_W_I8, 16, [(1000, 1024), (64, 4096)]),
    (ug.UG_W_I8, 33, [(128, 640), (99, 100)]),
]


@pytest.mark.parametrize("gi", range(len(GROUPS)))
@pytest.mark.parametrize("fused", [False, True])
def test_grouped_parity(dev, gi, fused):
    wfmt, M, shapes = GROUPS[gi]
    _case("grouped", gi, wfmt, M, fused)
    rng = np.random.default_rng([300, gi, int(fused)])
    probs, refs = [], []
    for (N, K) in shapes:
        if fused and M * _staged_kp(wfmt, M, K) > 65536:   # the documented staging limit
            continue
        x = rng.standard_normal((M, K), dtype=np.float32)
        wq = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
        beta = np.float32(0.015 + 0.001 * len(probs))
        xq_r, s_r = oracle.quant_act(x)
        w = pitched(oracle.pack_trits(wq)[0]) if wfmt == ug.UG_W_PACK5 else pitched(wq)
        p = dict(w=w, wfmt=wfmt, beta=scalar_dev(beta), K=K,
                 y=ug.empty_pitched(M, N, torch.float32, dev),
                 acc=ug.empty_pitched(M, N, torch.int32, dev))
        if fused:
            p.update(x=pitched(x), xq=ug.empty_pitched(M, K, torch.int8, dev),
                     s=torch.empty(M, dtype=torch.float32, device=dev))
        else:
            p.update(xq=pitched(xq_r), s=vec(s_r))
        probs.append(p)
        acc_r = oracle.matmul_i32(xq_r, wq)
        refs.append((xq_r, s_r, acc_r, oracle.epilogue(acc_r, s_r, beta)))
    if not probs:
        pytest.skip("no problem small enough for fused quantization")
    plan = ug.ug_gemv_plan_init(probs)
    ug.ug_bitlinear_gemv_grouped(plan)
    for i, (p, (xq_r, s_r, acc_r, y_r)) in enumerate(zip(probs, refs)):
        if fused:
            assert_bits_equal(host(p["xq"]), xq_r, "x_q %d" % i)
            assert_bits_equal(host(p["s"]), s_r, "s %d" % i)
        assert_bits_equal(host(p["acc"]), acc_r, "acc %d" % i)
        assert_y_close(host(p["y"]), y_r, "y %d" % i)


# (M, N, K, fused, short, tiny): one problem each; plan.info.variant bit 8 =
# fine split, bit 10 = its short variant (at most 4 pieces and 2 activation
# tiles per wave), bit 12 = the tiny one (with bit 10: at most 3 pieces and 1
# tile per wave).
FINE_VARIANTS = [
    (1, 2560, 2560, True, True, False),     # decode-sized: 10 fp32 tiles per block
    (4, 1000, 384, True, True, False),      # 12 fp32 tiles: 2 per wave
    (1, 16, 20000, False, False, False),    # one item of 63 steps: 8 pieces per wave
    (16, 6912, 2560, False, False, False),  # 48 x_q tiles: 6 per wave
    (16, 512, 2560, True, False, False),    # 160 fp32 tiles: 20 per wave (3 batches)
    (1, 4096, 384, True, True, True),       # 3 fp32 tiles, 2 pieces per block
    (1, 2560, 2560, False, True, True),     # 3 x_q tiles, 8 pieces per block
]


@pytest.mark.parametrize("ci", range(len(FINE_VARIANTS)))
def test_fine_variants(dev, ci):
    M, N, K, fused, short, tiny = FINE_VARIANTS[ci]
    _case("fine variant", M, N, K, fused, short, tiny)
    rng = np.random.default_rng([303, ci])
    x = rng.standard_normal((M, K), dtype=np.float32)
    wq = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    beta = np.float32(0.02)
    xq_r, s_r = oracle.quant_act(x)
    p = dict(w=pitched(oracle.pack_trits(wq)[0]), wfmt=ug.UG_W_PACK5, beta=scalar_dev(beta),
             K=K, y=ug.empty_pitched(M, N, torch.float32, dev),
             acc=ug.empty_pitched(M, N, torch.int32, dev))
    if fused:
        p.update(x=pitched(x), xq=ug.empty_pitched(M, K, torch.int8, dev),
                 s=torch.empty(M, dtype=torch.float32, device=dev))
    else:
        p.update(xq=pitched(xq_r), s=vec(s_r))
    plan = ug.ug_gemv_plan_init([p])
    assert (plan.info.variant >> 8) & 1 == 1, "fine split"
    assert bool((plan.info.variant >> 10) & 1) == short, "variant %#x" % plan.info.variant
    assert bool((plan.info.variant >> 12) & 1) == tiny, "variant %#x" % plan.info.variant
    ug.ug_bitlinear_gemv_grouped(plan)
    if fused:
        assert_bits_equal(host(p["xq"]), xq_r, "x_q")
        assert_bits_equal(host(p["s"]), s_r, "s")
    acc_r = oracle.matmul_i32(xq_r, wq)
    assert_bits_equal(host(p["acc"]), acc_r, "acc")
    assert_y_close(host(p["y"]), oracle.epilogue(acc_r, s_r, beta), "y")


# (wfmt, M, list of (N, K)): groups with a problem whose activation rows do
# not fit the stream split's 80 KB staging area, so the launch stages them chunk by chunk
# (plan.info.variant bit 11); every row class and both weight formats, ragged
# N and K, a staged problem in the same launch.
CHUNKED = [
    (ug.UG_W_PACK5, 1, [(300, 90001), (100, 640)]),
    (ug.UG_W_PACK5, 16, [(777, 6912), (50, 333)]),
    (ug.UG_W_PACK5, 17, [(600, 5000), (33, 4321)]),
    (ug.UG_W_PACK5, 64, [(513, 2560), (40, 1283)]),
    (ug.UG_W_I8, 16, [(300, 5200)]),
    (ug.UG_W_I8, 64, [(200, 1400), (31, 77)]),
]


@pytest.mark.parametrize("ci", range(len(CHUNKED)))
def test_chunked_parity(dev, ci):
    wfmt, M, shapes = CHUNKED[ci]
    _case("chunked", ci, wfmt, M)
    rng = np.random.default_rng([304, ci])
    probs, refs = [], []
    for (N, K) in shapes:
        x = rng.standard_normal((M, K), dtype=np.float32)
        wq = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
        beta = np.float32(0.01 + 0.002 * len(probs))
        xq_r, s_r = oracle.quant_act(x)
        w = pitched(oracle.pack_trits(wq)[0]) if wfmt == ug.UG_W_PACK5 else pitched(wq)
        probs.append(dict(w=w, wfmt=wfmt, beta=scalar_dev(beta), K=K, xq=pitched(xq_r), s=vec(s_r),
                          y=ug.empty_pitched(M, N, torch.float32, dev),
                          acc=ug.empty_pitched(M, N, torch.int32, dev)))
        acc_r = oracle.matmul_i32(xq_r, wq)
        refs.append((acc_r, oracle.epilogue(acc_r, s_r, beta)))
    plan = ug.ug_gemv_plan_init(probs)
    assert (plan.info.variant >> 11) & 1 == 1, "variant %#x" % plan.info.variant
    ug.ug_bitlinear_gemv_grouped(plan)
    for i, (p, (acc_r, y_r)) in enumerate(zip(probs, refs)):
        assert_bits_equal(host(p["acc"]), acc_r, "acc %d" % i)
        assert_y_close(host(p["y"]), y_r, "y %d" % i)


# (M, list of (N, K), fused, spread): stream-split groups (more 16-row
# pieces than the fine split takes).  Five trits per byte at M <= 16 take
# the spread staging (each packed byte's five activations in 8 staged bytes,
# plan.info.variant bit 13) when every problem's staged rows fit the 80 KB
# staging area: the spread rows alone when x_q is given, the K-order rows
# and the spread rows when the launch quantizes fp32 activations; otherwise
# the permuted staging.  Ragged K (tail bytes with fewer than five trits),
# ragged N, fp32 activations quantized in the launch or x_q given.
SPREAD = [
    (1, [(6912, 2560)] * 4 + [(2560, 6913), (77, 5), (300, 81)], False, True),
    (1, [(6912, 2560)] * 4 + [(2560, 6912), (513, 7)], True, True),
    (2, [(6912, 2560)] * 5 + [(100, 1001)], False, True),
    (3, [(6912, 2560)] * 5 + [(64, 3000)], True, True),
    (16, [(131200, 640), (77, 333)], False, True),
    (4, [(6912, 2560)] * 4 + [(2560, 6912)], False, True),
    (8, [(6912, 2560)] * 4 + [(2560, 6912)], False, False),  # 8 rows of 6912: too long to spread
    (16, [(6912, 2560)] * 5 + [(33, 2557)], False, True),
    (16, [(6912, 2560)] * 5, True, False),  # fused: K-order and spread rows do not both fit
]


@pytest.mark.parametrize("si", range(len(SPREAD)))
def test_stream_spread_staging(dev, si):
    M, shapes, fused, spread = SPREAD[si]
    _case("spread", si, M, fused, spread)
    rng = np.random.default_rng([306, si])
    probs, refs = [], []
    for i, (N, K) in enumerate(shapes):
        x = rng.standard_normal((M, K), dtype=np.float32)
        wq = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
        beta = np.float32(0.02 + 0.001 * i)
        xq_r, s_r = oracle.quant_act(x)
        p = dict(w=pitched(oracle.pack_trits(wq)[0]), wfmt=ug.UG_W_PACK5, beta=scalar_dev(beta),
                 K=K, y=ug.empty_pitched(M, N, torch.float32, dev),
                 acc=ug.empty_pitched(M, N, torch.int32, dev))
        if fused:
            p.update(x=pitched(x), xq=ug.empty_pitched(M, K, torch.int8, dev),
                     s=torch.empty(M, dtype=torch.float32, device=dev))
        else:
            p.update(xq=pitched(xq_r), s=vec(s_r))
        probs.append(p)
        acc_r = oracle.matmul_i32(xq_r, wq)
        refs.append((xq_r, s_r, acc_r, oracle.epilogue(acc_r, s_r, beta)))
    plan = ug.ug_gemv_plan_init(probs)
    v = plan.info.variant
    assert (v >> 8) & 1 == 0 and (v >> 11) & 1 == 0, "stream split expected, variant %#x" % v
    assert bool((v >> 13) & 1) == spread, "variant %#x" % v
    ug.ug_bitlinear_gemv_grouped(plan)
    for i, (p, (xq_r, s_r, acc_r, y_r)) in enumerate(zip(probs, refs)):
        if fused:
            assert_bits_equal(host(p["xq"]), xq_r, "x_q %d" % i)
            assert_bits_equal(host(p["s"]), s_r, "s %d" % i)
        assert_bits_equal(host(p["acc"]), acc_r, "acc %d" % i)
        assert_bits_equal(host(p["y"]), y_r, "y %d" % i)


@pytest.mark.parametrize("M", [1, 4, 16])
def test_stream_cache_line_pitch(dev, M):
    """Packed rows on a 128-byte pitch (ug.stream_pitch: 1408 bytes for the
    1383-byte rows of K = 6912) through the stream split and, at M = 16, the
    chunked split; the pad bytes hold junk, which meets zero activations."""
    _case("stream pitch", M)
    rng = np.random.default_rng([307, M])
    K, N, G = 6912, 2560, 7
    ldp = ug.stream_pitch(K)
    assert ldp == 1408
    probs, refs = [], []
    for i in range(G):
        wq = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
        x = rng.standard_normal((M, K), dtype=np.float32)
        xq_r, s_r = oracle.quant_act(x)
        pk = np.full((N, ldp), 0xA7, dtype=np.uint8)
        pk[:, :-(-K // 5)] = oracle.pack_trits(wq)[0][:, :-(-K // 5)]
        beta = np.float32(0.02 + 0.001 * i)
        probs.append(dict(xq=pitched(xq_r), s=vec(s_r), w=torch.from_numpy(pk).to(dev),
                          wfmt=ug.UG_W_PACK5, beta=scalar_dev(beta), K=K,
                          y=ug.empty_pitched(M, N, torch.float32, dev),
                          acc=ug.empty_pitched(M, N, torch.int32, dev)))
        acc_r = oracle.matmul_i32(xq_r, wq)
        refs.append((acc_r, oracle.epilogue(acc_r, s_r, beta)))
    plan = ug.ug_gemv_plan_init(probs)
    assert (plan.info.variant >> 8) & 1 == 0, "variant %#x" % plan.info.variant
    ug.ug_bitlinear_gemv_grouped(plan)
    for i, (p, (acc_r, y_r)) in enumerate(zip(probs, refs)):
        assert_bits_equal(host(p["acc"]), acc_r, "acc %d" % i)
        assert_bits_equal(host(p["y"]), y_r, "y %d" % i)


def test_grouped_many_problems_multi_item_blocks(dev):
    """A group large enough that every block walks several items."""
    rng = np.random.default_rng(301)
    K, N, G = 2560, 6912, 48
    wq = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    pk = pitched(oracle.pack_trits(wq)[0])
    xs = [rng.standard_normal((1, K), dtype=np.float32) for _ in range(G)]
    probs = [dict(x=pitched(x), w=pk, wfmt=ug.UG_W_PACK5, beta=scalar_dev(np.float32(0.02)),
                  K=K, y=ug.empty_pitched(1, N, torch.float32, dev)) for x in xs]
    plan = ug.ug_gemv_plan_init(probs)
    assert plan.info.grid < plan.info.total_items
    ug.ug_bitlinear_gemv_grouped(plan)
    for i in range(G):
        xq_r, s_r = oracle.quant_act(xs[i])
        y_r = oracle.epilogue(oracle.matmul_i32(xq_r, wq), s_r, np.float32(0.02))
        assert_bits_equal(host(probs[i]["y"]), y_r, "y %d" % i)


def test_grouped_stream_uneven_problems(dev):
    """Stream-split block ranges are cut by cost (weight bytes plus a set-up
    per problem a block enters), so blocks start and end at uneven places:
    problems of very different sizes (1 item to hundreds), some blocks
    crossing several problems, every output checked.  (The 21000-long rows
    have more steps than the fine split takes per item: the stream split
    runs.)"""
    rng = np.random.default_rng(305)
    shapes = [(6912, 2560), (16, 384), (40, 77), (2560, 6912), (33, 5), (4096, 1536),
              (100, 2560), (1, 1), (6912, 2560), (512, 21000)]
    probs, refs = [], []
    for i, (N, K) in enumerate(shapes):
        wq = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
        x = rng.standard_normal((1, K), dtype=np.float32)
        xq_r, s_r = oracle.quant_act(x)
        beta = np.float32(0.02 + 0.001 * i)
        probs.append(dict(xq=pitched(xq_r), s=vec(s_r), w=pitched(oracle.pack_trits(wq)[0]),
                          wfmt=ug.UG_W_PACK5, beta=scalar_dev(beta), K=K,
                          y=ug.empty_pitched(1, N, torch.float32, dev),
                          acc=ug.empty_pitched(1, N, torch.int32, dev)))
        acc_r = oracle.matmul_i32(xq_r, wq)
        refs.append((acc_r, oracle.epilogue(acc_r, s_r, beta)))
    plan = ug.ug_gemv_plan_init(probs)
    assert (plan.info.variant >> 8) & 1 == 0, "stream split expected"
    ug.ug_bitlinear_gemv_grouped(plan)
    for i, (p, (acc_r, y_r)) in enumerate(zip(probs, refs)):
        assert_bits_equal(host(p["acc"]), acc_r, "acc %d" % i)
        assert_y_close(host(p["y"]), y_r, "y %d" % i)


def test_grouped_plan_rejects(dev):
    rng = np.random.default_rng(302)
    wq = rng.integers(-1, 2, size=(64, 256)).astype(np.int8)
    x = pitched(rng.standard_normal((1, 256), dtype=np.float32))
    y = ug.empty_pitched(1, 64, torch.float32, dev)
    b = scalar_dev(np.float32(0.02))
    p8 = dict(x=x, w=pitched(wq), wfmt=ug.UG_W_I8, beta=b, y=y)
    p5 = dict(x=x, w=pitched(oracle.pack_trits(wq)[0]), wfmt=ug.UG_W_PACK5, beta=b, K=256, y=y)
    with pytest.raises(ug.UgError) as e:
        ug.ug_gemv_plan_init([p8, p5])   # mixed formats
    assert e.value.status == ug.UG_ERR_INVALID_ARG
    big = dict(x=pitched(rng.standard_normal((17, 4000), dtype=np.float32)),
               w=pitched(rng.integers(-1, 2, size=(8, 4000)).astype(np.int8)), wfmt=ug.UG_W_I8,
               beta=b, y=ug.empty_pitched(17, 8, torch.float32, dev))
    with pytest.raises(ug.UgError) as e:
        ug.ug_gemv_plan_init([big])      # fused quant with M*K > 65536
    assert e.value.status == ug.UG_ERR_UNSUPPORTED
