"""Requantization straight to five trits per byte
(ug_quant_weight_absmean_pack5): the fp32 masters go to PACK5 bytes in one
pass after the absmean sum ("ultragraph ... part 2", "training the thing":
requantize after every optimizer step; README "A whole ternary GPT": five
ternary values per byte).  Bit for bit the same beta and bytes as the
oracle's pack_trits(quant_weight_absmean(W)), at the pitch asked for."""
import numpy as np
import pytest
import torch

import oracle
from bitlinear_matmul_amd import inputs, ug
from gpu_util import assert_bits_equal, host, pitched

pytestmark = pytest.mark.gpu


def _case(*a):
    print("case:", *a, flush=True)


def _check(W, ldp=None, w_pad=0):
    N, K = W.shape
    ldp = ldp or ug.packed_pitch(K)
    if w_pad:
        # a weight pitch wider than the row: the pad holds large values that
        # must not reach beta or the bytes
        Wp = np.full((N, K + w_pad), np.float32(1e6), np.float32)
        Wp[:, :K] = W
        W_d = torch.from_numpy(Wp).to("cuda:0")[:, :K]
    else:
        W_d = pitched(W)
    packed = torch.empty((N, ldp), dtype=torch.uint8, device="cuda:0")
    pk_d, beta_d = ug.ug_quant_weight_absmean_pack5(W_d, packed=packed)
    ref_wq, ref_beta = oracle.quant_weight_absmean(W)
    ref_pk, bad = oracle.pack_trits(ref_wq, ldp=ldp)
    assert bad == 0
    assert host(beta_d)[0].view(np.uint32) == np.float32(ref_beta).view(np.uint32), "beta"
    assert_bits_equal(host(pk_d), ref_pk, "packed")
    return host(pk_d)


@pytest.mark.parametrize("N,K", [(512, 128), (1152, 384), (384, 1536), (6912, 2560),
                                 (2560, 6912), (33, 7), (5, 21), (17, 1), (3, 1000),
                                 (101, 19), (7, 20), (9, 85)])
def test_requant_pack5_parity(dev, N, K):
    _case("requant pack5", N, K)
    rng = np.random.default_rng([701, N, K])
    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    _check(W)


@pytest.mark.parametrize("N,K,extra,w_pad", [(64, 2560, 32, 0), (40, 6912, 16, 12),
                                             (9, 23, 48, 5)])
def test_requant_pack5_pitches(dev, N, K, extra, w_pad):
    """Row pitches beyond the minimum: pad bytes are 121; the weights' own
    row pad is never read into a result."""
    _case("requant pack5 pitches", N, K, extra, w_pad)
    rng = np.random.default_rng([703, N, K])
    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    got = _check(W, ldp=ug.packed_pitch(K) + extra, w_pad=w_pad)
    assert np.all(got[:, -(-K // 5):] == 121)


def test_requant_pack5_special_tensors(dev):
    """All zero: beta = eps, every byte 121 (five zero trits); a constant
    tensor c: beta = |c| + eps and every trit sign(c) (bytes 242 or 0 in full
    groups); the stack workload's first master."""
    z = _check(np.zeros((20, 333), np.float32))
    assert np.all(z == 121)
    c = _check(np.full((8, 100), np.float32(-0.25), np.float32))
    assert np.all(c[:, :20] == 0)
    c = _check(np.full((8, 100), np.float32(0.25), np.float32))
    assert np.all(c[:, :20] == 242)
    _check(inputs.stack_master(0, 1))


def test_requant_pack5_feeds_the_gemv(dev):
    """The bytes go straight into the decode GEMV: same accumulators as the
    oracle's quantize-pack-multiply."""
    rng = np.random.default_rng(705)
    K, N = 2560, 2560
    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    x = rng.standard_normal((4, K), dtype=np.float32)
    pk_d, beta_d = ug.ug_quant_weight_absmean_pack5(pitched(W))
    xq_d, s_d = ug.ug_quant_act(pitched(x))
    acc_d, _ = ug.ug_bitlinear_gemv(xq_d, s_d, pk_d, ug.UG_W_PACK5, beta_d, K=K, want_acc=True)
    r = oracle.bitlinear(x, W)
    assert_bits_equal(host(acc_d), r["acc"], "acc")
