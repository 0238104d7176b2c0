"""Steps captured as HIP graphs and replayed.  One decode step of a small
ternary transformer block: grouped GEMV for q, k and v (the fp32 token quantized in
the launch; k and v written straight into the cache row of the new
position, "ultragraph-1bit 0.12.0" README, "A whole ternary GPT"), causal
attention over the cache ("ultragraph ... part 2", "attention, as graph
ops"), grouped GEMV for the output projection and then for a vocabulary
head, and the top-k sampler ("a 1-bit llm, from scratch", "the interesting
bit").  Between replays the test does eager work of its own (new inputs,
host reads, synchronizations); every replay must give the bits of the same
calls made eagerly.  And one layer step of training-time work (below).
None of these calls records a memset."""
import numpy as np
import pytest
import torch

import oracle
from bitlinear_matmul_amd import ug
from gpu_util import assert_bits_equal, host, pitched, scalar_dev, vec

pytestmark = pytest.mark.gpu


def test_decode_step_graph_replays_match_eager(dev):
    rng = np.random.default_rng(71)
    d, H, prev, V, k = 256, 4, 37, 512, 20
    T = prev + 1
    mats = [rng.standard_normal((d, d), dtype=np.float32) * np.float32(0.02) for _ in range(4)]
    mats.append(rng.standard_normal((V, d), dtype=np.float32) * np.float32(0.02))
    biases = [rng.standard_normal(w.shape[0], dtype=np.float32) * np.float32(0.1) for w in mats]
    packed, betas = [], []
    for W in mats:
        wq, beta = oracle.quant_weight_absmean(W)
        packed.append(pitched(oracle.pack_trits(wq)[0]))
        betas.append(scalar_dev(beta))
    x = ug.empty_pitched(1, d, torch.float32, dev)
    kc = ug.empty_pitched(T, d, torch.float32, dev)
    vc = ug.empty_pitched(T, d, torch.float32, dev)
    kc[:prev] = torch.from_numpy(rng.standard_normal((prev, d), dtype=np.float32)).to(dev)
    vc[:prev] = torch.from_numpy(rng.standard_normal((prev, d), dtype=np.float32)).to(dev)
    qbuf = ug.empty_pitched(1, d, torch.float32, dev)
    ctx = ug.empty_pitched(1, d, torch.float32, dev)
    yo = ug.empty_pitched(1, d, torch.float32, dev)
    logits = ug.empty_pitched(1, V, torch.float32, dev)
    u = torch.empty(1, dtype=torch.float32, device=dev)
    tok = torch.empty(1, dtype=torch.int32, device=dev)
    attn_ws = torch.empty(ug.ug_attention_workspace_size(1, prev, H, d // H), dtype=torch.uint8,
                          device=dev)
    outs = [qbuf, kc[prev:prev + 1], vc[prev:prev + 1]]
    plan_qkv = ug.ug_gemv_plan_init([dict(x=x, w=packed[i], wfmt=ug.UG_W_PACK5, beta=betas[i],
                                          K=d, bias=vec(biases[i]), y=outs[i]) for i in range(3)])
    plan_o = ug.ug_gemv_plan_init([dict(x=ctx, w=packed[3], wfmt=ug.UG_W_PACK5, beta=betas[3],
                                        K=d, bias=vec(biases[3]), y=yo)])
    plan_head = ug.ug_gemv_plan_init([dict(x=yo, w=packed[4], wfmt=ug.UG_W_PACK5, beta=betas[4],
                                           K=d, bias=vec(biases[4]), y=logits)])

    def step():
        ug.ug_bitlinear_gemv_grouped(plan_qkv)
        ug.ug_attention_cached(qbuf, kc, vc, prev, H, out=ctx, ws=attn_ws)
        ug.ug_bitlinear_gemv_grouped(plan_o)
        ug.ug_bitlinear_gemv_grouped(plan_head)
        ug.ug_sample_topk(logits, k, 0.8, u, tokens=tok)

    def snapshot():
        return [host(t).copy() for t in (qbuf, kc[prev:prev + 1], vc[prev:prev + 1], ctx, yo,
                                         logits, tok)]

    names = ("q", "k row", "v row", "context", "projection", "logits", "token")
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        x.copy_(torch.from_numpy(rng.standard_normal((1, d), dtype=np.float32)))
        u.fill_(0.5)
        step()  # warm-up outside the capture
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.synchronize()
    for r in range(4):
        xr = rng.standard_normal((1, d), dtype=np.float32) * np.float32(1 + r)
        ur = float(rng.random())
        x.copy_(torch.from_numpy(xr))
        u.fill_(ur)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        replayed = snapshot()
        x.copy_(torch.from_numpy(xr))
        u.fill_(ur)
        step()
        eager = snapshot()
        for name, a, b in zip(names, replayed, eager):
            assert_bits_equal(a, b, "replay %d: %s" % (r, name))
        # the replay's own projection of q matches the oracle, bias included
        ref = oracle.bitlinear(xr, mats[0], bias=biases[0])
        assert_bits_equal(replayed[0], ref["y"], "replay %d: q vs oracle" % r)


def test_layer_step_graph_replays_match_eager(dev):
    """One training-time layer step as a HIP graph: requantization of the
    fp32 master (absmean sum, then the ternary pass), RMSNorm + act quant of
    the layer input, and the prefill GEMM, at M = 2048, 2560 -> 2560 (few
    output tiles: the GEMM splits each tile's K steps over several blocks
    that hand partial tiles over through tagged counters, which a replay of
    the same launch must leave reusable).  Masters and inputs change
    between replays; every replay is bit-identical to the eager calls and
    its W_q and beta to the oracle."""
    rng = np.random.default_rng(72)
    M, K, N = 2048, 2560, 2560
    W = ug.empty_pitched(N, K, torch.float32, dev)
    x = ug.empty_pitched(M, K, torch.float32, dev)
    wq = ug.empty_pitched(N, K, torch.int8, dev)
    beta = torch.empty(1, dtype=torch.float32, device=dev)
    xq = ug.empty_pitched(M, K, torch.int8, dev)
    s = torch.empty(M, dtype=torch.float32, device=dev)
    y = ug.empty_pitched(M, N, torch.float32, dev)
    aws = torch.empty(ug.ug_quant_weight_absmean_workspace_size(N, K), dtype=torch.uint8,
                      device=dev)
    gws = torch.empty(ug.ug_bitlinear_gemm_workspace_size(M, N, K, ug.UG_W_I8),
                      dtype=torch.uint8, device=dev)

    def step():
        ug.ug_quant_weight_absmean(W, wq=wq, beta=beta, ws=aws)
        ug.ug_rmsnorm_quant_act(x, xq=xq, s=s)
        ug.ug_bitlinear_gemm(xq, s, wq, ug.UG_W_I8, beta, y=y, ws=gws)

    def snapshot():
        return [host(t).copy() for t in (wq, beta, xq, s, y)]

    def fill(r):
        Wr = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02 * (1 + r))
        xr = rng.standard_normal((M, K), dtype=np.float32)
        W.copy_(torch.from_numpy(Wr))
        x.copy_(torch.from_numpy(xr))
        return Wr

    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        fill(0)
        step()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=st):
            step()
    torch.cuda.synchronize()
    names = ("W_q", "beta", "x_q", "s", "y")
    for r in range(1, 4):
        Wr = fill(r)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        replayed = snapshot()
        step()
        eager = snapshot()
        for name, a, b in zip(names, replayed, eager):
            assert_bits_equal(a, b, "replay %d: %s" % (r, name))
        wq_r, beta_r = oracle.quant_weight_absmean(Wr)
        assert_bits_equal(replayed[0], wq_r, "replay %d: W_q vs oracle" % r)
        assert_bits_equal(replayed[1], np.array([beta_r], np.float32), "replay %d: beta" % r)
