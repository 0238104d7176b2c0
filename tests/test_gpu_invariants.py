"""Invariants the pages state, checked on the GPU path itself (plus the
oracle where a reference value is needed):
  - batch invariance: row m of the GEMM equals the GEMV on row m alone
    (README "A whole ternary GPT": cached decoding must reproduce the
    full-forward bits), and GEMV at M rows equals GEMV per row;
  - format invariance: 5-trits-per-byte weights give the same integers as
    one trit per byte (README: deployed logits are byte-exact);
  - row independence of the quantizers ("attention, as graph ops");
  - determinism: two runs give identical bits (no atomics on values).
"""
import numpy as np
import pytest
import torch

import oracle
from bitlinear_matmul_amd import inputs, ug
from gpu_util import assert_bits_equal, host, pitched, scalar_dev, vec

pytestmark = pytest.mark.gpu


def test_gemm_rows_equal_gemv_rows(dev):
    x, W = inputs.sweep_inputs(0, 64)
    xq, s = ug.ug_quant_act(pitched(x))
    wq, beta = ug.ug_quant_weight_absmean(pitched(W))
    pk = ug.ug_pack_trits(wq)
    acc_g, y_g = ug.ug_bitlinear_gemm(xq, s, wq, ug.UG_W_I8, beta, want_acc=True)
    acc_v, y_v = ug.ug_bitlinear_gemv(xq, s, pk, ug.UG_W_PACK5, beta, K=x.shape[1],
                                      want_acc=True)
    assert_bits_equal(host(acc_v), host(acc_g), "gemv(64) vs gemm")
    assert_bits_equal(host(y_v), host(y_g), "y gemv(64) vs gemm")
    for m in (0, 17, 63):
        a1, y1 = ug.ug_bitlinear_gemv(xq[m:m + 1], s[m:m + 1], pk, ug.UG_W_PACK5, beta,
                                      K=x.shape[1], want_acc=True)
        assert_bits_equal(host(a1)[0], host(acc_g)[m], "row %d" % m)
        assert_bits_equal(host(y1)[0], host(y_g)[m], "y row %d" % m)


@pytest.mark.parametrize("use_gemm", [False, True])
def test_packed_equals_byte_format(dev, use_gemm):
    x, W = inputs.sweep_inputs(1, 16)
    xq, s = ug.ug_quant_act(pitched(x))
    wq, beta = ug.ug_quant_weight_absmean(pitched(W))
    pk = ug.ug_pack_trits(wq)
    fn = ug.ug_bitlinear_gemm if use_gemm else ug.ug_bitlinear_gemv
    a8, y8 = fn(xq, s, wq, ug.UG_W_I8, beta, want_acc=True)
    a5, y5 = fn(xq, s, pk, ug.UG_W_PACK5, beta, K=x.shape[1], want_acc=True)
    assert_bits_equal(host(a5), host(a8), "acc pack5 vs i8")
    assert_bits_equal(host(y5), host(y8), "y pack5 vs i8")


def test_rmsnorm_rows_independent(dev):
    rng = np.random.default_rng(200)
    x = rng.standard_normal((32, 6912), dtype=np.float32)
    a, sa = ug.ug_rmsnorm_quant_act(pitched(x))
    x[31] *= np.float32(-9)
    x[30, 100] = np.float32(1e6)
    b, sb = ug.ug_rmsnorm_quant_act(pitched(x))
    a, b, sa, sb = host(a), host(b), host(sa), host(sb)
    assert np.array_equal(a[:30], b[:30]) and np.array_equal(sa[:30], sb[:30])


def test_deterministic_repeat(dev):
    x, W, _ = inputs.prefill_inputs(0, M=512)
    outs = []
    for _ in range(2):
        xq, s = ug.ug_quant_act(pitched(x))
        wq, beta = ug.ug_quant_weight_absmean(pitched(W))
        pk = ug.ug_pack_trits(wq)
        _, yg = ug.ug_bitlinear_gemm(xq, s, wq, ug.UG_W_I8, beta)
        _, yv = ug.ug_bitlinear_gemv(xq[:8], s[:8], pk, ug.UG_W_PACK5, beta, K=x.shape[1])
        outs.append([host(t) for t in (xq, s, wq, beta, pk, yg, yv)])
    for a, b in zip(*outs):
        assert_bits_equal(a, b, "repeat")


def test_stream_ordering_on_side_stream(dev):
    """The whole chain enqueued on a non-default stream gives the same bits."""
    x, W = inputs.tiny_layer()
    side = torch.cuda.Stream()
    xd, Wd = pitched(x), pitched(W)
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        xq, s = ug.ug_quant_act(xd, stream=side)
        wq, beta = ug.ug_quant_weight_absmean(Wd, stream=side)
        _, y = ug.ug_bitlinear_gemm(xq, s, wq, ug.UG_W_I8, beta, stream=side)
    side.synchronize()
    ref = oracle.bitlinear(x, W)
    assert_bits_equal(host(y), ref["y"], "y on side stream")
