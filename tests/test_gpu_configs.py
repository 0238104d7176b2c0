"""Parity of the whole path on the five workloads, at their full sizes, in
the launch configurations the benchmark times.  Every stage is compared with
the CPU oracle on the same seeded inputs: x_q, s, beta, W_q, packed bytes and
int32 accumulators bit-exact, y within 1e-6 relative (expected exact).
"""
import numpy as np
import pytest
import torch

import oracle
from bitlinear_matmul_amd import inputs, ug
from gpu_util import assert_bits_equal, assert_y_close, host, pitched

pytestmark = pytest.mark.gpu


def _case(*a):
    print("case:", *a, flush=True)


def _gpu_layer(x, W, fmt, use_gemm, want_acc=True):
    """GPU path: act quant, absmean, (pack), matmul. Returns host arrays."""
    xq_d, s_d = ug.ug_quant_act(pitched(x))
    wq_d, beta_d = ug.ug_quant_weight_absmean(pitched(W))
    w = wq_d
    pk_d = None
    if fmt == ug.UG_W_PACK5:
        pk_d = ug.ug_pack_trits(wq_d)
        w = pk_d
    fn = ug.ug_bitlinear_gemm if use_gemm else ug.ug_bitlinear_gemv
    acc_d, y_d = fn(xq_d, s_d, w, fmt, beta_d, K=x.shape[1], want_acc=want_acc)
    out = dict(xq=host(xq_d), s=host(s_d), wq=host(wq_d), beta=host(beta_d)[0], y=host(y_d))
    if acc_d is not None:
        out["acc"] = host(acc_d)
    if pk_d is not None:
        out["packed"] = host(pk_d)
    return out


def _check_layer(got, x, W, fmt, full_acc=True, pairs=None):
    ref_xq, ref_s = oracle.quant_act(x)
    ref_wq, ref_beta = oracle.quant_weight_absmean(W)
    assert_bits_equal(got["s"], ref_s, "s")
    assert_bits_equal(got["xq"], ref_xq, "x_q")
    assert got["beta"].view(np.uint32) == np.float32(ref_beta).view(np.uint32), "beta"
    assert_bits_equal(got["wq"], ref_wq, "W_q")
    if fmt == ug.UG_W_PACK5:
        ref_pk, _ = oracle.pack_trits(ref_wq, ldp=got["packed"].shape[1])
        assert_bits_equal(got["packed"], ref_pk, "packed")
    if full_acc:
        acc = oracle.matmul_i32(ref_xq, ref_wq)
        assert_bits_equal(got["acc"], acc, "acc")
        y = oracle.epilogue(acc, ref_s, ref_beta)
        assert_y_close(got["y"], y, "y")
        assert_bits_equal(got["y"], y, "y bits")
    else:
        mi, ni = pairs
        acc = oracle.matmul_i32_pairs(ref_xq, ref_wq, mi, ni)
        assert_bits_equal(got["acc"][mi, ni], acc, "acc (sampled)")
        y = (acc.astype(np.float32) * (ref_s[mi] * np.float32(ref_beta))).astype(np.float32)
        assert_y_close(got["y"][mi, ni], y, "y (sampled)")


def test_tiny_layer_full_path(dev):
    """x [32,128], W [512,128] (1 trit/byte), seed 0: GEMV and GEMM."""
    x, W = inputs.tiny_layer()
    for use_gemm in (False, True):
        _case("tiny", "gemm" if use_gemm else "gemv")
        got = _gpu_layer(x, W, ug.UG_W_I8, use_gemm)
        _check_layer(got, x, W, ug.UG_W_I8)
    zero_frac = float((got["wq"] == 0).mean())
    assert 0.28 < zero_frac < 0.34


def test_decode_stack_all_matrices(dev):
    """Batch-1 decode stack: 8 x {qkv, o, up, down} + head, 5 trits/byte."""
    for (layer, mi, name, K, N) in inputs.decode_stack_shapes():
        _case("decode_stack", layer, name, K, N)
        x, W = inputs.decode_stack_matrix(layer, mi, K, N)
        got = _gpu_layer(x, W, ug.UG_W_PACK5, use_gemm=False)
        _check_layer(got, x, W, ug.UG_W_PACK5)


@pytest.mark.parametrize("j", [0, 1])
def test_prefill_full_size(dev, j):
    """M=4096 GEMM on both 2B-class shapes, 1% outlier channels x20; the
    whole int32 accumulator matrix is compared."""
    K, N = inputs.PREFILL_SHAPES[j]
    _case("prefill", j, K, N)
    x, W, _ = inputs.prefill_inputs(j)
    got = _gpu_layer(x, W, ug.UG_W_I8, use_gemm=True)
    _check_layer(got, x, W, ug.UG_W_I8)


@pytest.mark.parametrize("shape_idx", [0, 1, 2])
def test_sweep_all_points(dev, shape_idx):
    for M in inputs.SWEEP_MS:
        K, N = inputs.SWEEP_SHAPES[shape_idx]
        _case("sweep", shape_idx, M, K, N)
        x, W = inputs.sweep_inputs(shape_idx, M)
        got = _gpu_layer(x, W, ug.UG_W_PACK5, use_gemm=False)
        _check_layer(got, x, W, ug.UG_W_PACK5)


def _stack_rows(M):
    """Rows of the stack workload whose chain the oracle follows: the first
    two, the middle, the last, and 60 seeded others."""
    rng = np.random.default_rng(777)
    extra = rng.choice(np.arange(2, M - 1), size=60, replace=False)
    return np.unique(np.concatenate([[0, 1, M // 2 - 1, M - 1], extra])).astype(np.int64)


@pytest.mark.timeout(900)
def test_stack_full_depth_chained(dev):
    """The whole stack step at M = 2048, as the benchmark runs it: all 60 fp32
    masters requantized (absmean + ternary) and compared in full (beta and
    every W_q); then the 60 x (RMSNorm + act quant + GEMM) chain.  Rows are
    independent ("attention, as graph ops": one scale per token), so at every
    layer the oracle takes the GPU's own input rows for a sample of 64 rows
    and checks s, x_q, the whole accumulator row and y bit for bit; the
    oracle also runs its own chain from x0 on those rows, which must end on
    the GPU's bits."""
    M = inputs.STACK_M
    rows = _stack_rows(M)
    rows_d = torch.from_numpy(rows).to("cuda:0")
    dev_ = torch.device("cuda:0")
    # requantization of every master first (the benchmark's order)
    ws = torch.empty(max(ug.ug_quant_weight_absmean_workspace_size(N, K)
                         for (K, N) in inputs.STACK_SHAPES), dtype=torch.uint8, device=dev_)
    mats = []
    for layer in range(inputs.STACK_LAYERS):
        for which in (0, 1):
            _case("stack requant", layer, which)
            K, N = inputs.STACK_SHAPES[which]
            W = inputs.stack_master(layer, which)
            wq_d = ug.empty_pitched(N, K, torch.int8, dev_)
            beta_d = torch.empty(1, dtype=torch.float32, device=dev_)
            ug.ug_quant_weight_absmean(pitched(W), wq=wq_d, beta=beta_d, ws=ws)
            ref_wq, ref_beta = oracle.quant_weight_absmean(W)
            assert host(beta_d)[0].view(np.uint32) == np.float32(ref_beta).view(np.uint32), \
                ("beta", layer, which)
            assert_bits_equal(host(wq_d), ref_wq, "W_q layer %d/%d" % (layer, which))
            mats.append((K, N, wq_d, beta_d, ref_wq, ref_beta))
    x0 = inputs.stack_x0()
    x_d = torch.from_numpy(x0).to(dev_)
    own = x0[rows]  # the oracle's own chain on the sampled rows
    for li, (K, N, wq_d, beta_d, ref_wq, ref_beta) in enumerate(mats):
        _case("stack chain", li // 2, li % 2, K, N)
        xq_d, s_d = ug.ug_rmsnorm_quant_act(x_d)
        acc_d, y_d = ug.ug_bitlinear_gemm(xq_d, s_d, wq_d, ug.UG_W_I8, beta_d, want_acc=True)
        x_in = host(x_d.index_select(0, rows_d))
        ref_xq, ref_s = oracle.rmsnorm_quant_act(x_in)
        assert_bits_equal(host(s_d.index_select(0, rows_d)), ref_s, "s %d" % li)
        assert_bits_equal(host(xq_d.index_select(0, rows_d)), ref_xq, "x_q %d" % li)
        acc = oracle.matmul_i32(ref_xq, ref_wq)
        assert_bits_equal(host(acc_d.index_select(0, rows_d)), acc, "acc %d" % li)
        y = oracle.epilogue(acc, ref_s, ref_beta)
        assert_bits_equal(host(y_d.index_select(0, rows_d)), y, "y %d" % li)
        oq, os_ = oracle.rmsnorm_quant_act(own)
        own = oracle.epilogue(oracle.matmul_i32(oq, ref_wq), os_, ref_beta)
        x_d = y_d
    assert_bits_equal(host(x_d.index_select(0, rows_d)), own, "end of the oracle's own chain")
