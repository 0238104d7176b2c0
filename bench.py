"""Benchmark of the BitLinear forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Prints ONE JSON line.  Workloads (default: decode_stack):
  decode_stack  batch-1 decode pass over 8 x {384->1152, 384->384,
                384->1536, 1536->384} + a 384->4096 head, weights 5 trits per
                byte; a step = per-row int8 quantization of each matrix's input
                plus the GEMV of every matrix (33 x); each step reads its own
                copy of the weights so they stream from HBM (cold).
                value = packed-weight GB/s.
  sweep         decode GEMV at M in {1,4,16,64} x the three 2B-class shapes
                (cold, cycling weight copies); value = weight GB/s over all
                12 points.
  prefill       M=4096 act quant + int8 MFMA GEMM for 2560->6912 and
                6912->2560; value = int8 TOP/s.
  stack         30 layers x {2560->6912, 6912->2560}: requantize the fp32
                masters, RMSNorm + act quant + GEMM chained at M=2048;
                value = int8 TOP/s of the whole step.
  tiny          x[32,128] W[512,128]: the full path incl. weight quant.

Inputs are seeded synthetic tensors (bitlinear_matmul_amd.inputs) already
resident in HBM when timing starts.  Timing: W untimed steps, then K steps
between torch.cuda.synchronize() calls (HIP events on the stream the
kernels run on).  The dominant kernel's roofline fraction uses algorithmic
bytes (or ops) per launch over its average launch duration, measured here
with HIP events.  The CPU oracle is timed on a bounded sample of the same
workload on the host cores.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "BitLinear GEMV weight GB/s (decode) and GEMM int8 TOPS (prefill), % roofline"
HBM_PEAK_GBS = 8000.0
INT8_PEAK_TOPS = 5000.0
COLD_BYTES = 2 << 30  # weight copies to cycle through: >= 8x the 256 MB MALL


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None)
    p.add_argument("--warmup", type=int, default=None)
    p.add_argument("--workload", default="decode_stack",
                   choices=["decode_stack", "sweep", "prefill", "stack", "tiny"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--sweep-point", default=None, metavar="M,SHAPE",
                   help="sweep: run only the point with M rows and shape index SHAPE "
                        "(0: 2560->6912, 1: 6912->2560, 2: 2560->2560), e.g. for profiling")
    p.add_argument("--copy-probe", action="store_true",
                   help="first run one plain 256 MiB device copy (a known-size kernel that "
                        "calibrates the FETCH_SIZE / WRITE_SIZE counters of a profiled run)")
    return p.parse_args()


# HBM traffic of the dominant kernel per launch, from two rocprofv3 --pmc runs
# of this script (FETCH_SIZE, then WRITE_SIZE), each scaled by the reading of
# the same counter for a plain 256 MiB copy in the same run (--copy-probe).
# Valid only for the kernel sources they were taken on: `src_sha` is the
# SHA-256 of the kernel's source file; any other source reports null.
TRAFFIC = {
    # profiles/gemv_fine_grouped_decode_stack.md: 1990.9 KiB fetched x 1.9997,
    # 146.4 KiB written x 1.0000
    "decode_stack": dict(src="bitlinear_matmul_amd/csrc/gemv_mfma.hip",
                         src_sha="1aae82af7e9516601044d9b7a23aec2baef46e0964b8951dc49212bf55f17d0a",
                         bytes_per_launch=4226741),
    # profiles/gemv_stream_grouped_sweep_m1.md: M=1 2560->6912, 37 problems per
    # launch: 64217.2 KiB fetched x 1.9997, 697.6 KiB written x 1.0000
    "sweep": dict(src="bitlinear_matmul_amd/csrc/gemv_mfma.hip",
                  src_sha="1aae82af7e9516601044d9b7a23aec2baef46e0964b8951dc49212bf55f17d0a",
                  bytes_per_launch=132214235),
    # profiles/gemm_i8_large_prefill.md: mean of both shapes, 60190.6 KiB
    # fetched x 1.9997, 75776.0 KiB written x 1.0000
    "prefill": dict(src="bitlinear_matmul_amd/csrc/gemm.hip",
                    src_sha="11ab35c8fe414afb87b67a3d95e82774ae246e31de0d9e609a3908b361837e64",
                    bytes_per_launch=200846379),
}


def source_sha(relpath):
    import hashlib
    with open(os.path.join(ROOT, relpath), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def traffic_for(workload):
    t = TRAFFIC.get(workload)
    if t is None or source_sha(t["src"]) != t["src_sha"]:
        return None
    return t["bytes_per_launch"]


def copy_probe(torch):
    n = 256 << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    log("copy probe: %d bytes read, %d bytes written" % (n, n))
    del a, b
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# timing helpers
# ---------------------------------------------------------------------------
def time_graph(torch, g, stream):
    """Replay a captured graph once between events on its stream; ms."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1)


def capture(torch, fn):
    """Capture fn() (which launches libug kernels on the current stream)
    into a HIP graph."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fn()
    torch.cuda.synchronize()
    return g


# ---------------------------------------------------------------------------
# decode_stack
# ---------------------------------------------------------------------------
def setup_decode_stack(torch, ug, inputs, n_copies):
    """Quantize + pack every matrix once (deployed weights), then make
    n_copies copies of the packed set and one grouped plan per copy: a plan
    quantizes the 33 fp32 inputs and runs the 33 GEMVs in one launch."""
    dev = torch.device("cuda:0")
    mats = []
    for (layer, mi, name, K, N) in inputs.decode_stack_shapes():
        x, W = inputs.decode_stack_matrix(layer, mi, K, N)
        wq, beta = ug.ug_quant_weight_absmean(torch.from_numpy(W).to(dev))
        pk = ug.ug_pack_trits(wq)
        mats.append(dict(K=K, N=N, x=torch.from_numpy(x).to(dev), pk=pk, beta=beta,
                         xq=ug.empty_pitched(1, K, torch.int8, dev),
                         s=torch.empty(1, dtype=torch.float32, device=dev),
                         y=ug.empty_pitched(1, N, torch.float32, dev), W=W, x_host=x))
        del wq
    plans = []
    for c in range(n_copies):
        probs = []
        for m in mats:
            w = m["pk"] if c == 0 else m["pk"].clone()
            probs.append(dict(x=m["x"], w=w, wfmt=ug.UG_W_PACK5, beta=m["beta"], K=m["K"],
                              y=m["y"], xq=m["xq"], s=m["s"]))
        plans.append(ug.ug_gemv_plan_init(probs))
    torch.cuda.synchronize()
    per_pass_bytes = sum(m["N"] * (-(-m["K"] // 5)) for m in mats)
    return mats, plans, per_pass_bytes


def gemv_alg_bytes(M, N, K, packed=True, fp32_x=False):
    """Algorithmic bytes of one GEMV: packed (or 1 B/trit) weights, the
    activations (fp32 when quantized in the launch, else int8 + scales),
    beta and the fp32 output."""
    wb = N * (-(-K // 5)) if packed else N * K
    xb = 4 * M * K if fp32_x else M * K + 4 * M
    return wb + xb + 4 + 4 * M * N


def cpu_decode_stack(oracle, mats, seconds):
    # oracle state: quantized weights of each matrix (setup, untimed)
    prep = []
    for m in mats:
        wq, beta = oracle.quant_weight_absmean(m["W"])
        pk, _ = oracle.pack_trits(wq)
        prep.append((m["x_host"], pk, m["K"], beta))
    passes = 0
    t0 = time.perf_counter()
    while True:
        for (x, pk, K, beta) in prep:
            xq, s = oracle.quant_act(x)
            wq, _ = oracle.unpack_trits(pk, K)
            oracle.epilogue(oracle.matmul_i32(xq, wq), s, beta)
        passes += 1
        if time.perf_counter() - t0 >= seconds:
            break
    return passes, time.perf_counter() - t0


def run_decode_stack(args, torch, ug, inputs):
    steps = args.steps if args.steps is not None else 200
    warm = args.warmup if args.warmup is not None else 20
    per_copy = sum(N * ug.packed_pitch(K) for (_, _, _, K, N) in inputs.decode_stack_shapes())
    n_copies = min(max(1, COLD_BYTES // per_copy), warm + steps)
    mats, plans, per_pass_bytes = setup_decode_stack(torch, ug, inputs, n_copies)
    log("decode_stack: %d matrices, %d packed weight bytes per pass, %d copies, grid %d"
        % (len(mats), per_pass_bytes, n_copies, plans[0].info.grid))
    g_warm = capture(torch, lambda: [ug.ug_bitlinear_gemv_grouped(plans[c % n_copies])
                                     for c in range(warm)])
    g_run = capture(torch, lambda: [ug.ug_bitlinear_gemv_grouped(plans[(warm + c) % n_copies])
                                    for c in range(steps)])
    stream = torch.cuda.current_stream()
    time_graph(torch, g_warm, stream)
    ms = time_graph(torch, g_run, stream)
    log("decode_stack: %d steps in %.3f ms" % (steps, ms))
    # hot regime: one weight copy, resident in L2 / MALL (the realistic
    # regime for a 3 MB model); reported beside the cold value
    g_hot = capture(torch, lambda: [ug.ug_bitlinear_gemv_grouped(plans[0]) for _ in range(steps)])
    time_graph(torch, g_hot, stream)
    ms_hot = time_graph(torch, g_hot, stream)
    del g_hot
    # The step is one launch of the grouped kernel, so the kernel's average
    # launch duration is the step time (inter-launch gap included).
    alg = sum(gemv_alg_bytes(1, m["N"], m["K"], fp32_x=True) for m in mats)
    avg_launch_s = ms / 1e3 / steps
    achieved = alg / avg_launch_s / 1e9
    value = per_pass_bytes * steps / (ms / 1e3) / 1e9
    out = dict(value=value, unit="GB/s", ms_per_step=ms / steps, steps=steps, warmup=warm,
               dtype="i8 (int32 accumulate)",
               config={"workload": "decode_stack", "batch": 1, "matrices": len(mats),
                       "weight_format": "pack5", "packed_weight_bytes_per_step": per_pass_bytes,
                       "launches_per_step": 1, "weight_copies_cycled": n_copies,
                       "regime": "cold (each step reads its own weight copy from HBM)",
                       "us_per_token_pass": ms * 1e3 / steps,
                       "hot_us_per_token_pass": ms_hot * 1e3 / steps,
                       "hot_weight_GBps": per_pass_bytes * steps / (ms_hot / 1e3) / 1e9},
               roofline=dict(bound="hbm", kernel="gemv_fine_grouped<PACK5, fused, tiny>",
                             achieved=achieved, peak=HBM_PEAK_GBS, unit="GB/s",
                             frac=achieved / HBM_PEAK_GBS, traffic=traffic_for("decode_stack"),
                             avg_launch_us=avg_launch_s * 1e6, alg_bytes_per_launch=alg))
    if not args.no_cpu_baseline:
        import oracle
        passes, secs = cpu_decode_stack(oracle, mats, args.cpu_seconds)
        out["cpu_baseline"] = dict(value=per_pass_bytes * passes / secs / 1e9, unit="GB/s",
                                   cores=oracle.num_threads(), kind="oracle",
                                   sample="%d full decode passes (33 x quant + unpack + int "
                                          "matmul + rescale) in %.1f s" % (passes, secs))
    return out


# ---------------------------------------------------------------------------
# sweep: decode GEMV at M in {1,4,16,64} x three 2B-class shapes
# ---------------------------------------------------------------------------
def run_sweep(args, torch, ug, inputs):
    """Per point: (a) one GEMV call, cold, latency per call; (b) streaming:
    a grouped launch over G distinct weight copies (G * bytes >= 128 MB),
    steps cycling through enough copies to exceed the MALL."""
    steps = args.steps if args.steps is not None else 10
    warm = args.warmup if args.warmup is not None else 2
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    points = []
    tot_bytes = 0.0
    tot_s = 0.0
    dom = None
    only = tuple(int(v) for v in args.sweep_point.split(",")) if args.sweep_point else None
    for si, (K, N) in enumerate(inputs.SWEEP_SHAPES):
        if only is not None and only[1] != si:
            continue
        x64, W = inputs.sweep_inputs(si, 64)
        wq, beta = ug.ug_quant_weight_absmean(torch.from_numpy(W).to(dev))
        pk = ug.ug_pack_trits(wq)
        del wq
        wbytes = N * (-(-K // 5))
        G = max(1, (128 << 20) // (N * ug.packed_pitch(K)))
        n_sets = max(2, min(warm + steps, (COLD_BYTES // (G * N * ug.packed_pitch(K))) + 1))
        copies = [[pk.clone() for _ in range(G)] for _ in range(n_sets)]
        for M in inputs.SWEEP_MS:
            if only is not None and only[0] != M:
                continue
            xq, s = ug.ug_quant_act(torch.from_numpy(x64[:M].copy()).to(dev))
            y = ug.empty_pitched(M, N, torch.float32, dev)
            try:
                plans = [ug.ug_gemv_plan_init([dict(xq=xq, s=s, w=w, wfmt=ug.UG_W_PACK5,
                                                    beta=beta, K=K, y=y) for w in cs])
                         for cs in copies]
            except ug.UgError:
                plans = None
            if plans is not None:
                g = capture(torch, lambda: [ug.ug_bitlinear_gemv_grouped(plans[c % n_sets])
                                            for c in range(warm + steps)])
                ms = time_graph(torch, g, stream)
                launch_us = ms * 1e3 / (warm + steps)
                gbs = wbytes * G / (launch_us * 1e-6) / 1e9
                alg = gemv_alg_bytes(M, N, K) * G
                del g
            else:
                launch_us, gbs, alg = None, None, None
            # single-call latency, cold copies
            g1 = capture(torch, lambda: [ug.ug_bitlinear_gemv(
                xq, s, copies[c % n_sets][c % G], ug.UG_W_PACK5, beta, K=K, y=y)
                for c in range(warm + steps)])
            ms1 = time_graph(torch, g1, stream)
            del g1
            call_us = ms1 * 1e3 / (warm + steps)
            pt = {"M": M, "K": K, "N": N, "call_us": call_us,
                  "call_weight_GBps": wbytes / (call_us * 1e-6) / 1e9,
                  "grouped_G": G if plans else 0, "grouped_launch_us": launch_us,
                  "grouped_weight_GBps": gbs}
            log("sweep", pt)
            points.append(pt)
            if plans is not None:
                tot_bytes += wbytes * G
                tot_s += launch_us * 1e-6
                if M == 1 and si == 0:
                    dom = dict(bound="hbm", kernel="gemv_stream_grouped<PACK5, 1>",
                               achieved=alg / (launch_us * 1e-6) / 1e9, peak=HBM_PEAK_GBS,
                               unit="GB/s", frac=alg / (launch_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                               traffic=traffic_for("sweep"), avg_launch_us=launch_us,
                               alg_bytes_per_launch=alg,
                               point="M=1 K=2560 N=6912, %d copies per launch" % G)
        del copies
        torch.cuda.empty_cache()
    value = tot_bytes / tot_s / 1e9
    return dict(value=value, unit="GB/s", ms_per_step=tot_s * 1e3 / len(points), steps=steps,
                warmup=warm, dtype="i8 (int32 accumulate)",
                config={"workload": "sweep", "points": points, "weight_format": "pack5",
                        "regime": "cold; value = grouped streaming over all points"},
                roofline=dom)


# ---------------------------------------------------------------------------
# prefill
# ---------------------------------------------------------------------------
def run_prefill(args, torch, ug, inputs):
    steps = args.steps if args.steps is not None else 20
    warm = args.warmup if args.warmup is not None else 3
    dev = torch.device("cuda:0")
    layers = []
    for j in (0, 1):
        x, W, _ = inputs.prefill_inputs(j)
        K, N = inputs.PREFILL_SHAPES[j]
        wq, beta = ug.ug_quant_weight_absmean(torch.from_numpy(W).to(dev))
        layers.append(dict(K=K, N=N, x=torch.from_numpy(x).to(dev), wq=wq, beta=beta,
                           xq=ug.empty_pitched(x.shape[0], K, torch.int8, dev),
                           s=torch.empty(x.shape[0], dtype=torch.float32, device=dev),
                           y=ug.empty_pitched(x.shape[0], N, torch.float32, dev),
                           x_host=x, W=W))
    M = inputs.PREFILL_M
    ops_per_step = sum(2 * M * l["N"] * l["K"] for l in layers)

    def step():
        for l in layers:
            ug.ug_quant_act(l["x"], 1e-5, xq=l["xq"], s=l["s"])
            ug.ug_bitlinear_gemm(l["xq"], l["s"], l["wq"], ug.UG_W_I8, l["beta"], y=l["y"])

    stream = torch.cuda.current_stream()
    for _ in range(warm):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    # GEMM alone
    e0.record(stream)
    for _ in range(steps):
        for l in layers:
            ug.ug_bitlinear_gemm(l["xq"], l["s"], l["wq"], ug.UG_W_I8, l["beta"], y=l["y"])
    e1.record(stream)
    torch.cuda.synchronize()
    gemm_ms = e0.elapsed_time(e1) / (2 * steps)
    achieved = ops_per_step / 2 / (gemm_ms / 1e3) / 1e12
    out = dict(value=ops_per_step * steps / (ms / 1e3) / 1e12, unit="TOP/s",
               ms_per_step=ms / steps, steps=steps, warmup=warm, dtype="i8 (int32 accumulate)",
               config={"workload": "prefill", "M": M, "shapes_KxN": [[l["K"], l["N"]]
                                                                     for l in layers],
                       "weight_format": "i8"},
               roofline=dict(bound="mfma", kernel="gemm_i8_large", achieved=achieved,
                             peak=INT8_PEAK_TOPS, unit="TOP/s", frac=achieved / INT8_PEAK_TOPS,
                             traffic=traffic_for("prefill"), avg_launch_us=gemm_ms * 1e3,
                             alg_ops_per_launch=ops_per_step / 2))
    if not args.no_cpu_baseline:
        import oracle
        # bounded sample: the first rows of each layer's x through the oracle
        rows = 0
        t0 = time.perf_counter()
        ops = 0
        prep = [(l["x_host"], oracle.quant_weight_absmean(l["W"])) for l in layers]
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < args.cpu_seconds and rows < M:
            for (x, (wq, beta)) in prep:
                xq, s = oracle.quant_act(x[rows:rows + 64])
                oracle.epilogue(oracle.matmul_i32(xq, wq), s, beta)
                ops += 2 * xq.shape[0] * wq.shape[0] * wq.shape[1]
            rows += 64
        secs = time.perf_counter() - t0
        out["cpu_baseline"] = dict(value=ops / secs / 1e12, unit="TOP/s",
                                   cores=oracle.num_threads(), kind="oracle",
                                   sample="first %d of 4096 rows of both layers (quant + int "
                                          "matmul + rescale) in %.1f s" % (rows, secs))
    return out


# ---------------------------------------------------------------------------
# stack: 30 layers x {2560->6912, 6912->2560} at M=2048 with requantization
# ---------------------------------------------------------------------------
def run_stack(args, torch, ug, inputs):
    """One step: requantize all 60 fp32 masters (absmean + ternary), then the
    chain of 60 x (RMSNorm + act quant + int8 GEMM) from x0."""
    steps = args.steps if args.steps is not None else 3
    warm = args.warmup if args.warmup is not None else 1
    dev = torch.device("cuda:0")
    M = inputs.STACK_M
    mats = []
    for layer in range(inputs.STACK_LAYERS):
        for which in (0, 1):
            K, N = inputs.STACK_SHAPES[which]
            W = torch.from_numpy(inputs.stack_master(layer, which)).to(dev)
            mats.append(dict(K=K, N=N, W=W, wq=ug.empty_pitched(N, K, torch.int8, dev),
                             beta=torch.empty(1, dtype=torch.float32, device=dev),
                             xq=ug.empty_pitched(M, K, torch.int8, dev),
                             s=torch.empty(M, dtype=torch.float32, device=dev),
                             y=ug.empty_pitched(M, N, torch.float32, dev)))
    ws = torch.empty(max(ug.ug_quant_weight_absmean_workspace_size(m["N"], m["K"]) for m in mats),
                     dtype=torch.uint8, device=dev)
    x0 = torch.from_numpy(inputs.stack_x0()).to(dev)
    ops_per_step = sum(2 * M * m["N"] * m["K"] for m in mats)
    log("stack: %d BitLinears, %.3g int8 ops per step" % (len(mats), ops_per_step))

    def requant():
        for m in mats:
            ug.ug_quant_weight_absmean(m["W"], wq=m["wq"], beta=m["beta"], ws=ws)

    def chain(gemm_only=False):
        x = x0
        for m in mats:
            if not gemm_only:
                ug.ug_rmsnorm_quant_act(x, xq=m["xq"], s=m["s"])
            ug.ug_bitlinear_gemm(m["xq"], m["s"], m["wq"], ug.UG_W_I8, m["beta"], y=m["y"])
            x = m["y"]

    stream = torch.cuda.current_stream()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    for _ in range(warm):
        requant()
        chain()
    torch.cuda.synchronize()
    t_req = t_chain = 0.0
    e_all0, e_all1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e_all0.record(stream)
    for _ in range(steps):
        e[0].record(stream)
        requant()
        e[1].record(stream)
        chain()
        e[2].record(stream)
        torch.cuda.synchronize()
        t_req += e[0].elapsed_time(e[1])
        t_chain += e[1].elapsed_time(e[2])
    e_all1.record(stream)
    torch.cuda.synchronize()
    ms = t_req + t_chain
    # the GEMMs alone (the dominant kernel), same chain of operands
    e[0].record(stream)
    for _ in range(steps):
        chain(gemm_only=True)
    e[1].record(stream)
    torch.cuda.synchronize()
    gemm_ms = e[0].elapsed_time(e[1]) / (steps * len(mats))
    req_bytes = sum(9 * m["N"] * m["K"] for m in mats)
    act_bytes = sum(4 * M * m["K"] + M * m["K"] + 4 * M for m in mats)
    achieved = ops_per_step / len(mats) / (gemm_ms / 1e3) / 1e12
    out = dict(value=ops_per_step * steps / (ms / 1e3) / 1e12, unit="TOP/s",
               ms_per_step=ms / steps, steps=steps, warmup=warm, dtype="i8 (int32 accumulate)",
               config={"workload": "stack", "layers": inputs.STACK_LAYERS, "M": M,
                       "shapes_KxN": [list(x) for x in inputs.STACK_SHAPES],
                       "weight_format": "i8", "requant_ms_per_step": t_req / steps,
                       "requant_GBps": req_bytes * steps / (t_req / 1e3) / 1e9,
                       "chain_ms_per_step": t_chain / steps,
                       "gemm_us_per_launch": gemm_ms * 1e3,
                       "act_quant_alg_bytes_per_step": act_bytes},
               roofline=dict(bound="mfma", kernel="gemm_i8_large", achieved=achieved,
                             peak=INT8_PEAK_TOPS, unit="TOP/s", frac=achieved / INT8_PEAK_TOPS,
                             traffic=traffic_for("stack"), avg_launch_us=gemm_ms * 1e3,
                             alg_ops_per_launch=ops_per_step / len(mats)))
    if not args.no_cpu_baseline:
        import oracle
        # bounded sample: layer 0 (both BitLinears) at the first rows of x0,
        # including the requantization of its two masters
        x = inputs.stack_x0()
        masters = [inputs.stack_master(0, w) for w in (0, 1)]
        rows, ops = 0, 0
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < args.cpu_seconds and rows < M:
            xr = x[rows:rows + 64]
            for Wm in masters:
                wq, beta = oracle.quant_weight_absmean(Wm)
                xq, s = oracle.rmsnorm_quant_act(xr)
                xr = oracle.epilogue(oracle.matmul_i32(xq, wq), s, beta)
                ops += 2 * xq.shape[0] * wq.shape[0] * wq.shape[1]
            rows += 64
        secs = time.perf_counter() - t0
        out["cpu_baseline"] = dict(value=ops / secs / 1e12, unit="TOP/s",
                                   cores=oracle.num_threads(), kind="oracle",
                                   sample="layer 0 (requant of both masters + RMSNorm/quant + "
                                          "int matmul + rescale, both BitLinears) on %d of "
                                          "2048 rows per pass, %.1f s" % (rows, secs))
    return out


# ---------------------------------------------------------------------------
# tiny: x[32,128], W[512,128], one trit per byte, the whole path
# ---------------------------------------------------------------------------
def run_tiny(args, torch, ug, inputs):
    steps = args.steps if args.steps is not None else 200
    warm = args.warmup if args.warmup is not None else 20
    dev = torch.device("cuda:0")
    x, W = inputs.tiny_layer()
    xd, Wd = torch.from_numpy(x).to(dev), torch.from_numpy(W).to(dev)
    M, K = x.shape
    N = W.shape[0]
    wq = ug.empty_pitched(N, K, torch.int8, dev)
    beta = torch.empty(1, dtype=torch.float32, device=dev)
    ws = torch.empty(ug.ug_quant_weight_absmean_workspace_size(N, K), dtype=torch.uint8, device=dev)
    xq = ug.empty_pitched(M, K, torch.int8, dev)
    s = torch.empty(M, dtype=torch.float32, device=dev)
    y = ug.empty_pitched(M, N, torch.float32, dev)

    def step():
        ug.ug_quant_weight_absmean(Wd, wq=wq, beta=beta, ws=ws)
        ug.ug_quant_act(xd, 1e-5, xq=xq, s=s)
        ug.ug_bitlinear_gemm(xq, s, wq, ug.UG_W_I8, beta, y=y)

    stream = torch.cuda.current_stream()
    g = capture(torch, lambda: [step() for _ in range(steps)])
    time_graph(torch, g, stream)
    ms = time_graph(torch, g, stream)
    g2 = capture(torch, lambda: [ug.ug_bitlinear_gemm(xq, s, wq, ug.UG_W_I8, beta, y=y)
                                 for _ in range(steps)])
    time_graph(torch, g2, stream)
    gemm_ms = time_graph(torch, g2, stream) / steps
    ops = 2 * M * N * K
    out = dict(value=ops * steps / (ms / 1e3) / 1e12, unit="TOP/s", ms_per_step=ms / steps,
               steps=steps, warmup=warm, dtype="i8 (int32 accumulate)",
               config={"workload": "tiny", "M": M, "K": K, "N": N, "weight_format": "i8",
                       "launches_per_step": 4, "us_per_step": ms * 1e3 / steps,
                       "regime": "launch-bound (a parity-sized layer)"},
               roofline=dict(bound="mfma", kernel="gemm_i8_kernel",
                             achieved=ops / (gemm_ms / 1e3) / 1e12, peak=INT8_PEAK_TOPS,
                             unit="TOP/s", frac=ops / (gemm_ms / 1e3) / 1e12 / INT8_PEAK_TOPS,
                             traffic=None, avg_launch_us=gemm_ms * 1e3, alg_ops_per_launch=ops))
    if not args.no_cpu_baseline:
        import oracle
        n = 0
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < min(args.cpu_seconds, 5.0):
            wq_r, b_r = oracle.quant_weight_absmean(W)
            xq_r, s_r = oracle.quant_act(x)
            oracle.epilogue(oracle.matmul_i32(xq_r, wq_r), s_r, b_r)
            n += 1
        secs = time.perf_counter() - t0
        out["cpu_baseline"] = dict(value=ops * n / secs / 1e12, unit="TOP/s",
                                   cores=oracle.num_threads(), kind="oracle",
                                   sample="%d whole steps (weight quant + act quant + matmul + "
                                          "rescale) in %.1f s" % (n, secs))
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(use --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch

    from bitlinear_matmul_amd import inputs, ug
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    ug.lib()
    if args.copy_probe:
        copy_probe(torch)
    runners = {"decode_stack": run_decode_stack, "prefill": run_prefill, "sweep": run_sweep,
               "stack": run_stack, "tiny": run_tiny}
    res = runners[args.workload](args, torch, ug, inputs)
    line = {"metric": METRIC, "value": res["value"], "unit": res["unit"], "n_gpus": 1,
            "steps": res["steps"], "warmup": res["warmup"], "ms_per_step": res["ms_per_step"],
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": res["dtype"], "data": "synthetic (seeded numpy, shapes of the workload)",
            "config": res["config"], "roofline": res["roofline"]}
    if "cpu_baseline" in res:
        line["cpu_baseline"] = res["cpu_baseline"]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
