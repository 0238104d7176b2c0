"""The allocation-free absmean entry point (ug_quant_weight_absmean_static),
called through the C ABI, gives the same beta bits and W_q bytes as
ug_quant_weight_absmean with a caller workspace, on two calls in a row (the
second smaller, so stale chunk sums from the first sit in the static array
past the second's chunks), and both agree with the oracle."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from bitlinear_matmul_amd import ug
from gpu_util import assert_bits_equal, host, pitched

pytestmark = pytest.mark.gpu


def _static(W_d, wq_d, beta_d):
    L = ug.lib()
    N, K = W_d.shape
    st = L.ug_quant_weight_absmean_static(
        ctypes.c_void_p(W_d.data_ptr()), ug._ld(W_d), N, K, ctypes.c_float(1e-5),
        ctypes.c_void_p(wq_d.data_ptr()), ug._ld(wq_d), ctypes.c_void_p(beta_d.data_ptr()),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == ug.UG_OK, ug.status_string(st)


@pytest.mark.parametrize("shapes", [((6912, 2560), (1152, 384)), ((2560, 6912), (33, 100))])
def test_static_absmean_matches_workspace_entry(dev, shapes):
    rng = np.random.default_rng([901, shapes[0][0]])
    for (N, K) in shapes:
        print("case: absmean static", N, K, flush=True)
        W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
        W_d = pitched(W)
        wq_s = ug.empty_pitched(N, K, torch.int8, dev)
        beta_s = torch.empty(1, dtype=torch.float32, device=dev)
        _static(W_d, wq_s, beta_s)
        wq_w, beta_w = ug.ug_quant_weight_absmean(W_d)
        assert host(beta_s).view(np.uint32)[0] == host(beta_w).view(np.uint32)[0]
        assert_bits_equal(host(wq_s), host(wq_w), "W_q static vs workspace")
        ref_wq, ref_beta = oracle.quant_weight_absmean(W)
        assert host(beta_s)[0].view(np.uint32) == np.float32(ref_beta).view(np.uint32)
        assert_bits_equal(host(wq_s), ref_wq, "W_q static vs oracle")
