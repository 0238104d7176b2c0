"""One decode step of a small ternary transformer block, captured as a HIP
graph and replayed: grouped GEMV for q, k and v (the fp32 token quantized in
the launch; k and v written straight into the cache row of the new
position, "ultragraph-1bit 0.12.0" README, "A whole ternary GPT"), causal
attention over the cache ("ultragraph ... part 2", "attention, as graph
ops"), grouped GEMV for the output projection and then for a vocabulary
head, and the top-k sampler ("a 1-bit llm, from scratch", "the interesting
bit").  Between replays the test does eager work of its own (new inputs,
host reads, synchronizations); every replay must give the bits of the same
calls made eagerly.  None of these calls records a memset."""
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
