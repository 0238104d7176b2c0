"""Benchmark of the BitLinear forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Prints ONE JSON line.  Workloads (default: decode_stack):
  decode_stack  batch-1 decode pass over 8 x {384->1152, 384->384,
                384->1536, 1536->384} + a 384->4096 head, weights 5 trits per
                byte; a step = per-row int8 quantization of each matrix's input
                plus the GEMV of every matrix (33 x), one launch.  Every step
                reads its own copy of the weights, the copies span >= 2 GiB,
                and a 1 GiB write evicts the caches before each timed region,
                so weights stream from HBM (cold).  value = packed-weight GB/s.
                The same line also carries, each with its own roofline: the
                prefill GEMM (4096 x 2560 -> 6912 and 4096 x 6912 -> 2560,
                int8 TOP/s) as "prefill_gemm"; the streaming decode GEMV at
                M = 1, 2560 -> 6912 (weight GB/s) as "stream_m1"; the
                requantization of a 6912 x 2560 fp32 master straight to five
                trits per byte as "requant_pack5"; and one decode step of
                causal attention over a 4096-position K/V cache (20 heads x
                128) as "attention_decode"; top-100-of-4096 sampling as
                "sampler"; the straight-through backward (dx, dW, db) of a
                2048-token 6912 x 2560 layer as "backward".
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
resident in HBM when timing starts.  Timing: W untimed steps, then exactly K
steps between torch.cuda.synchronize() calls, timed with HIP events on the
stream the kernels run on.  The dominant kernel's roofline fraction uses
algorithmic bytes (or ops) per launch over its average launch duration in
that timed region; the median over at least 50 further launches is reported
beside it.  The CPU oracle is timed on a bounded sample of the same
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
FLUSH_BYTES = 1 << 30  # written before a timed region: evicts L2 and the MALL
STAT_LAUNCHES = 60     # launches behind each reported median


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


class Flusher:
    """A 1 GiB device buffer whose rewrite evicts the weights from L2 and
    the MALL before a timed region (the write itself is never timed)."""

    def __init__(self, torch):
        self.torch = torch
        self.buf = torch.empty(FLUSH_BYTES // 4, dtype=torch.int32, device="cuda:0")
        self.n = 0

    def __call__(self):
        self.n += 1
        self.buf.fill_(self.n)


def median(v):
    v = sorted(v)
    n = len(v)
    return v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])


def launch_stats(torch, launch, stream, count=STAT_LAUNCHES, flush=None, per=1):
    """Per-launch durations (us) of `count` timed calls of launch(i) (each
    runs `per` back-to-back kernel launches), each between HIP events on
    `stream`, optionally after a cache flush; returns (median, p10, p90)."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(count)]
    torch.cuda.synchronize()
    for i in range(count):
        if flush is not None:
            flush()
        ev[i][0].record(stream)
        launch(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    us = sorted(a.elapsed_time(b) * 1e3 / per for a, b in ev)
    return median(us), us[len(us) // 10], us[(9 * len(us)) // 10]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None)
    p.add_argument("--warmup", type=int, default=None)
    p.add_argument("--workload", default="decode_stack",
                   choices=["decode_stack", "sweep", "prefill", "stack", "tiny"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-marginal", action="store_true",
                   help="stream_m1: skip the launches of twice the problems (profiling)")
    p.add_argument("--no-extra", action="store_true",
                   help="decode_stack: skip the extra measurement points")
    p.add_argument("--only", default=None,
                   choices=["prefill_gemm", "vendor_int8_gemm", "hbm_copy_rate", "hbm_read_rate",
                            "stream_m1",
                            "pack", "requant_pack5", "attention_decode", "sampler",
                            "backward", "mfma_sustained"],
                   help="run just this one of the decode_stack line's extra points and print "
                        "its JSON object (for profiling a single kernel)")
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
    # HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE (KiB per
    # dispatch, medians), calibrated by a 256 MiB copy: bytes = FETCH x 1024 x
    # 1.99977 + WRITE x 1024.  A record holds only while the kernel sources
    # it was taken on are unchanged.
    # profiles/gemv_fine_grouped_decode_stack.md: 1772.2 KiB / 146.4 KiB
    "decode_stack": dict(src={"bitlinear_matmul_amd/csrc/gemv_mfma.hip":
                              "5a7201909a6c70fc24447ce66b28b5bb130889ea0c88c05aeb51149d3e4516d8",
                              "bitlinear_matmul_amd/csrc/api.hip":
                              "fc7393bcd0906b1442f9491311fb3f3f27b63ac92f6563fd8603fae300f9762c"},
                         bytes_per_launch=3779031),
    # profiles/gemv_stream_grouped_sweep_m1.md: M=1 2560->6912, 37 problems per
    # launch, spread staging: 64107.3 KiB / 191.3 KiB
    "sweep": dict(src={"bitlinear_matmul_amd/csrc/gemv_mfma.hip":
                       "5a7201909a6c70fc24447ce66b28b5bb130889ea0c88c05aeb51149d3e4516d8"},
                  bytes_per_launch=131466773),
    # profiles/gemm_i8_large_prefill.md: mean of the two shapes' launches
    "prefill": dict(src={"bitlinear_matmul_amd/csrc/gemm.hip":
                         "02b27e9db0529ba1b218003a0d600a96eb02f97bdc7bbbc8ef0ed0e7862fabf3"},
                    bytes_per_launch=200752978),
    # profiles/gemm_i8_large_stack.md: mean of the two shapes' launches
    "stack": dict(src={"bitlinear_matmul_amd/csrc/gemm.hip":
                       "02b27e9db0529ba1b218003a0d600a96eb02f97bdc7bbbc8ef0ed0e7862fabf3"},
                  bytes_per_launch=143287088),
    # profiles/pack_unpack_6912x2560.md: mean of the pack and unpack calls
    "pack": dict(src={"bitlinear_matmul_amd/csrc/pack.hip":
                      "a752a31dc60e320f1f3841a49c54afa110a55e65614c559d94983a25d7c60f6c"},
                 bytes_per_launch=21286585),
    # profiles/absmean_ternary_pack5_requant.md: stage 1 + fused pass per call
    "requant_pack5": dict(src={"bitlinear_matmul_amd/csrc/absmean.hip":
                               "a69523d80a0c82173d06857320485e02857481b5810e490f22fae63e67d95234"},
                          bytes_per_launch=145415161),
    # profiles/attention_decode_4096.md: partials + combine per call
    "attention_decode": dict(src={"bitlinear_matmul_amd/csrc/attention.hip":
                                  "d056702cf7f6a76a59cc97c7e0e992b33c28afa64e7f83209459662ea53b9377"},
                             bytes_per_launch=85617150),
    # profiles/topk_sample_batch4096.md: the 4096-row launch
    "sampler": dict(src={"bitlinear_matmul_amd/csrc/sampler.hip":
                         "5626fcf9f96f214c619bce97c12f84286293f235fe296ac41c7771d47261fa0e"},
                    bytes_per_launch=67639194),
    # profiles/gemm_f32_backward.md: mean of the dx call and the dW call (each
    # a GEMM and the sum of its cut tiles' pieces)
    "backward": dict(src={"bitlinear_matmul_amd/csrc/backward.hip":
                          "2582b06d5a06e5dab55f20cf6a235e3908523f6ce3d4c8a9e2384ec04333e669"},
                     bytes_per_launch=835617886),
}


def source_sha(relpath):
    import hashlib
    with open(os.path.join(ROOT, relpath), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def traffic_for(workload):
    t = TRAFFIC.get(workload)
    if t is None or any(source_sha(f) != h for f, h in t["src"].items()):
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
    """Replay a captured graph once between events on its stream; ms.  (A
    graph's first replay also pays one-time set-up: callers replay it once
    untimed first.)"""
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
                         y=ug.empty_pitched(1, N, torch.float32, dev)))
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


def cpu_decode_stack(oracle, inputs, seconds):
    # oracle state: quantized + packed weights of each matrix (set-up, untimed)
    prep = []
    for (layer, mi, name, K, N) in inputs.decode_stack_shapes():
        x, W = inputs.decode_stack_matrix(layer, mi, K, N)
        wq, beta = oracle.quant_weight_absmean(W)
        pk, _ = oracle.pack_trits(wq)
        prep.append((x, pk, K, beta))
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
    # every launch of the warm-up and the timed region reads its own copy,
    # and the copies span at least COLD_BYTES whatever the step count
    n_copies = max(warm + steps, -(-COLD_BYTES // per_copy))
    mats, plans, per_pass_bytes = setup_decode_stack(torch, ug, inputs, n_copies)
    flush = Flusher(torch)
    log("decode_stack: %d matrices, %d packed weight bytes per pass, %d copies (%.2f GiB), "
        "grid %d" % (len(mats), per_pass_bytes, n_copies, n_copies * per_copy / 2 ** 30,
                     plans[0].info.grid))
    g_warm = capture(torch, lambda: [ug.ug_bitlinear_gemv_grouped(plans[c]) for c in range(warm)])
    g_run = capture(torch, lambda: [ug.ug_bitlinear_gemv_grouped(plans[warm + c])
                                    for c in range(steps)])
    stream = torch.cuda.current_stream()
    time_graph(torch, g_warm, stream)
    # the timed graph's first replay, untimed (its one-time set-up: a
    # graph's first replay runs ~1 us per launch slower), then the caches
    # are flushed again, so the timed replay still reads every copy cold
    time_graph(torch, g_run, stream)
    flush()
    ms = time_graph(torch, g_run, stream)
    log("decode_stack: %d steps in %.3f ms" % (steps, ms))
    # per-launch spread: STAT_LAUNCHES single cold launches (caches flushed
    # before each), each on a copy the timed region did not use
    c0 = (warm + steps) % n_copies
    med, p10, p90 = launch_stats(
        torch, lambda i: ug.ug_bitlinear_gemv_grouped(plans[(c0 + i) % n_copies]), stream,
        flush=flush)
    # hot regime: one weight copy, resident in L2 / MALL (the realistic
    # regime for a 3 MB model); reported beside the cold value
    g_hot = capture(torch, lambda: [ug.ug_bitlinear_gemv_grouped(plans[0]) for _ in range(steps)])
    time_graph(torch, g_hot, stream)
    ms_hot = time_graph(torch, g_hot, stream)
    del g_hot, g_warm, g_run
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
                       "weight_copy_bytes_cycled": n_copies * per_copy,
                       "regime": "cold: each step reads its own weight copy, the copies span "
                                 ">= 2 GiB, and 1 GiB is written just before the timed region",
                       "us_per_token_pass": ms * 1e3 / steps,
                       "cold_launch_us_median": med, "cold_launch_us_p10": p10,
                       "cold_launch_us_p90": p90, "cold_launches_in_median": STAT_LAUNCHES,
                       "hot_us_per_token_pass": ms_hot * 1e3 / steps,
                       "hot_weight_GBps": per_pass_bytes * steps / (ms_hot / 1e3) / 1e9},
               roofline=dict(bound="hbm", kernel="gemv_fine_grouped<PACK5, fused, tiny>",
                             achieved=achieved, peak=HBM_PEAK_GBS, unit="GB/s",
                             frac=achieved / HBM_PEAK_GBS, traffic=traffic_for("decode_stack"),
                             avg_launch_us=avg_launch_s * 1e6, median_launch_us=med,
                             alg_bytes_per_launch=alg))
    del plans, mats, flush
    torch.cuda.empty_cache()
    if not args.no_extra:
        out["mfma_sustained"] = measure_mfma_sustained(torch, ug)
        torch.cuda.empty_cache()
        out["prefill_gemm"] = measure_prefill_gemm(torch, ug, inputs)
        torch.cuda.empty_cache()
        out["vendor_int8_gemm"] = measure_vendor_gemm(torch, ug, inputs)
        torch.cuda.empty_cache()
        out["hbm_copy_rate"] = measure_copy_rate(torch)
        torch.cuda.empty_cache()
        out["hbm_read_rate"] = measure_hbm_read(torch, ug)
        torch.cuda.empty_cache()
        out["stream_m1"] = measure_stream_m1(torch, ug, inputs, read=out["hbm_read_rate"])
        torch.cuda.empty_cache()
        out["pack"] = measure_pack(torch, ug, inputs)
        torch.cuda.empty_cache()
        out["requant_pack5"] = measure_requant_pack5(torch, ug, inputs)
        torch.cuda.empty_cache()
        out["attention_decode"] = measure_attention_decode(torch, ug)
        torch.cuda.empty_cache()
        out["sampler"] = measure_sampler(torch, ug)
        torch.cuda.empty_cache()
        out["backward"] = measure_backward(torch, ug)
        torch.cuda.empty_cache()
        # each HBM-bound point against a plain read of its algorithmic bytes
        attach_plain_read(torch, ug, out["roofline"], out["roofline"]["median_launch_us"])
        for k in ("stream_m1", "pack", "requant_pack5", "attention_decode", "sampler"):
            r = out[k]["roofline"]
            attach_plain_read(torch, ug, r, r["median_launch_us"])
        torch.cuda.empty_cache()
        # the matrix-core kernels against what the matrix cores sustain
        ms = out["mfma_sustained"]
        out["prefill_gemm"]["roofline"]["frac_of_sustained"] = (
            out["prefill_gemm"]["roofline"]["achieved"] / ms["int8_TOPs"])
        out["backward"]["roofline"]["frac_of_sustained"] = (
            out["backward"]["roofline"]["achieved"] / ms["fp32_TFLOPs"])
    if not args.no_cpu_baseline:
        import oracle
        passes, secs = cpu_decode_stack(oracle, inputs, args.cpu_seconds)
        out["cpu_baseline"] = dict(value=per_pass_bytes * passes / secs / 1e9, unit="GB/s",
                                   cores=oracle.num_threads(), cpu_model=cpu_model(),
                                   kind="oracle",
                                   sample="%d full decode passes (33 x quant + unpack + int "
                                          "matmul + rescale) in %.1f s" % (passes, secs))
    return out


def measure_prefill_gemm(torch, ug, inputs):
    """The int8 MFMA GEMM of the prefill workload (M = 4096; 2560 -> 6912 and
    6912 -> 2560, I8 weights), alone: per shape, the median over STAT_LAUNCHES
    samples of 5 back-to-back launches, each sample between HIP events on
    the launch stream."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    per_shape = []
    for j in (0, 1):
        x, W, _ = inputs.prefill_inputs(j)
        K, N = inputs.PREFILL_SHAPES[j]
        M = x.shape[0]
        wq, beta = ug.ug_quant_weight_absmean(torch.from_numpy(W).to(dev))
        xq, s = ug.ug_quant_act(torch.from_numpy(x).to(dev))
        y = ug.empty_pitched(M, N, torch.float32, dev)
        del x, W
        for _ in range(3):
            ug.ug_bitlinear_gemm(xq, s, wq, ug.UG_W_I8, beta, y=y)
        # a prefill runs its GEMMs back to back: each sample is 5 launches in
        # a row, per-launch time = their time / 5
        med, p10, p90 = launch_stats(
            torch, lambda i: [ug.ug_bitlinear_gemm(xq, s, wq, ug.UG_W_I8, beta, y=y)
                              for _ in range(5)], stream, per=5)
        ops = 2 * M * N * K
        per_shape.append(dict(M=M, K=K, N=N, ops=ops, median_us=med, p10_us=p10, p90_us=p90,
                              TOPs=ops / (med * 1e-6) / 1e12))
        log("prefill gemm", per_shape[-1])
        del wq, xq, s, y
    ops = sum(p["ops"] for p in per_shape) / 2
    us = sum(p["median_us"] for p in per_shape) / 2
    achieved = ops / (us * 1e-6) / 1e12
    return dict(value=achieved, unit="TOP/s", shapes=per_shape,
                roofline=dict(bound="mfma", kernel="gemm_i8_large", achieved=achieved,
                              peak=INT8_PEAK_TOPS, unit="TOP/s", frac=achieved / INT8_PEAK_TOPS,
                              traffic=traffic_for("prefill"), median_launch_us=us,
                              alg_ops_per_launch=ops))


def measure_vendor_gemm(torch, ug, inputs):
    """Context, not this library: the vendor BLAS's int8 GEMM (torch._int_mm,
    hipBLASLt on ROCm) on the prefill shapes and the same quantized operands,
    int32 output (no rescale, so less output work than ours), timed as
    prefill_gemm is: medians of samples of 5 back-to-back launches."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    per_shape = []
    for j in (0, 1):
        x, W, _ = inputs.prefill_inputs(j)
        K, N = inputs.PREFILL_SHAPES[j]
        M = x.shape[0]
        wq, _beta = ug.ug_quant_weight_absmean(torch.from_numpy(W).to(dev))
        xq, _s = ug.ug_quant_act(torch.from_numpy(x).to(dev))
        a = xq[:, :K].contiguous()
        bt = wq[:, :K].contiguous().t()  # K x N, column-major: x_q W_q^T
        del x, W, xq, wq
        out = torch._int_mm(a, bt)
        for _ in range(3):
            torch._int_mm(a, bt, out=out)
        med, p10, p90 = launch_stats(
            torch, lambda i: [torch._int_mm(a, bt, out=out) for _ in range(5)], stream, per=5)
        ops = 2 * M * N * K
        per_shape.append(dict(M=M, K=K, N=N, median_us=med, p10_us=p10, p90_us=p90,
                              TOPs=ops / (med * 1e-6) / 1e12))
        log("vendor int8 gemm", per_shape[-1])
        del a, bt, out
    us = sum(p["median_us"] for p in per_shape) / 2
    ops = 2 * per_shape[0]["M"] * per_shape[0]["N"] * per_shape[0]["K"]
    return dict(value=ops / (us * 1e-6) / 1e12, unit="TOP/s", library="torch._int_mm",
                note="context only: the vendor library on the same operands, int32 output",
                shapes=per_shape, median_launch_us=us,
                frac_of_int8_peak=ops / (us * 1e-6) / 1e12 / INT8_PEAK_TOPS)


def measure_copy_rate(torch):
    """Context, not this library: the HBM rate of a plain device-to-device
    copy on this GPU (torch's copy_, 128 MiB read + 128 MiB written per call,
    sources spanning >= 2 GiB cycled so every call reads cold); bytes read
    plus written per second, the median over STAT_LAUNCHES calls."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    n = 128 << 20
    n_copies = -(-COLD_BYTES // n) + 1
    srcs = [torch.ones(n, dtype=torch.uint8, device=dev) for _ in range(n_copies)]
    dst = torch.empty(n, dtype=torch.uint8, device=dev)
    for i in range(2):
        dst.copy_(srcs[i])
    med, p10, p90 = launch_stats(torch, lambda i: dst.copy_(srcs[(i + 2) % n_copies]), stream)
    res = dict(value=2 * n / (med * 1e-6) / 1e9, unit="GB/s", library="torch copy_",
               note="context only: a vendor copy of 128 MiB per call (read + written), cold",
               median_call_us=med, p10_call_us=p10, p90_call_us=p90,
               frac_of_hbm_peak=2 * n / (med * 1e-6) / 1e9 / HBM_PEAK_GBS)
    log("copy rate", res)
    del srcs, dst
    return res


def measure_hbm_read(torch, ug):
    """The measured streaming-read ceiling (ug_hbm_read_probe: every wave
    load reads 1 KB contiguous, eight loads in flight per thread): calls of
    128 MiB and of 256 MiB, each region read once in a cycle spanning
    >= 2 GiB (cold); the difference of the medians gives the marginal read
    rate and the fixed cost per call, as for the streaming GEMV.  A few walks
    and grid sizes are timed (more loads in flight is not faster: one block
    of four waves per CU with a grid stride measured best); the fastest
    per-call configuration is the ceiling."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    configs = [(0, cus), (0, 2 * cus), (1, 2 * cus), (1, 16 * cus)]
    sink = torch.zeros(4 * 16 * cus, dtype=torch.int32, device=dev)
    n1 = 128 << 20
    span = COLD_BYTES + 2 * n1
    buf = torch.ones(span // 4, dtype=torch.int32, device=dev)

    def timed(n, walk, blocks):
        regions = span // n
        views = [buf[i * (n // 4):(i + 1) * (n // 4)] for i in range(regions)]
        for i in range(2):
            ug.ug_hbm_read_probe(views[i], blocks, sink, walk=walk)
        return launch_stats(torch, lambda i: ug.ug_hbm_read_probe(
            views[(i + 2) % regions], blocks, sink, walk=walk), stream)

    tried = []
    for walk, blocks in configs:
        med, p10, p90 = timed(n1, walk, blocks)
        med2 = timed(2 * n1, walk, blocks)[0]
        tried.append(dict(walk=walk, blocks=blocks, median_call_us=med, p10_call_us=p10,
                          p90_call_us=p90, median_call_us_2x=med2))
    best = min(tried, key=lambda t: t["median_call_us"])
    med, med2 = best["median_call_us"], best["median_call_us_2x"]
    rate = n1 / (med * 1e-6) / 1e9
    marginal = n1 / ((med2 - med) * 1e-6) / 1e9 if med2 > med else None
    res = dict(value=rate, unit="GB/s", kernel="hbm_read_kernel (ug_hbm_read_probe)",
               note="measured streaming-read ceiling: 128 MiB read per call, cold",
               walk=best["walk"], blocks=best["blocks"], median_call_us=med,
               p10_call_us=best["p10_call_us"], p90_call_us=best["p90_call_us"],
               median_call_us_2x=med2, marginal_GBps=marginal, fixed_us_per_call=2 * med - med2,
               frac_of_hbm_peak=rate / HBM_PEAK_GBS,
               marginal_frac_of_hbm_peak=marginal / HBM_PEAK_GBS if marginal else None,
               configs=[{k: (round(v, 2) if isinstance(v, float) else v) for k, v in t.items()}
                        for t in tried])
    log("read rate", res)
    del buf, sink
    return res


def plain_read_us(torch, ug, nbytes):
    """Median time (us, over STAT_LAUNCHES cold calls) of a plain streaming
    read of nbytes (ug_hbm_read_probe, one block of four waves per CU, the
    fastest configuration of the read-rate point), regions cycled over
    >= 2 GiB: what moving a point's algorithmic bytes costs when nothing
    else is done, fixed launch cost included."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    blocks = torch.cuda.get_device_properties(dev).multi_processor_count
    n = max(16, int(nbytes) // 16 * 16)
    regions = max(2, COLD_BYTES // n + 1)
    buf = torch.ones(regions * n // 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(4 * blocks, dtype=torch.int32, device=dev)
    views = [buf[i * (n // 4):(i + 1) * (n // 4)] for i in range(regions)]
    for i in range(2):
        ug.ug_hbm_read_probe(views[i], blocks, sink, walk=0)
    med = launch_stats(torch, lambda i: ug.ug_hbm_read_probe(views[(i + 2) % regions], blocks,
                                                             sink, walk=0), stream)[0]
    del views, buf, sink
    torch.cuda.empty_cache()
    return med


def attach_plain_read(torch, ug, roof, launch_us):
    """Adds to an HBM-bound point's roofline the time of a plain read of its
    algorithmic bytes and the ratio of the two (both single cold calls)."""
    us = plain_read_us(torch, ug, roof["alg_bytes_per_launch"])
    roof["plain_read_same_bytes_us"] = us
    roof["frac_of_plain_read"] = us / launch_us


def measure_mfma_sustained(torch, ug, iters=4000):
    """Context for the matrix-core rooflines: the rate the matrix cores
    sustain with every CU busy (ug_mfma_rate_probe: one block of four waves
    per CU, back-to-back int8 32x32x32 or fp32 16x16x4 instructions on
    register operands that change every instruction, ~1 ms per call, so the
    clock settles where the board's power limit holds it).  Medians over
    STAT_LAUNCHES calls of each kind."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    blocks = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.empty(4 * blocks, dtype=torch.int32, device=dev)
    res = dict(blocks=blocks, iters=iters,
               note="context: register-only matrix instructions on every CU; the published "
                    "peaks assume the 2.4 GHz peak clock")
    for kind, name, peak in ((0, "int8", INT8_PEAK_TOPS), (1, "fp32", FP32_MFMA_PEAK_TFLOPS)):
        ops = ug.ug_mfma_rate_probe(kind, blocks, iters, sink)
        med, p10, p90 = launch_stats(torch, lambda i: ug.ug_mfma_rate_probe(kind, blocks, iters,
                                                                            sink), stream)
        rate = ops / (med * 1e-6) / 1e12
        res[name + ("_TOPs" if kind == 0 else "_TFLOPs")] = rate
        res[name + "_frac_of_peak"] = rate / peak
        res[name + "_median_call_us"] = med
    log("mfma sustained", res)
    return res


def measure_pack(torch, ug, inputs):
    """Five trits per byte and back (the pack and unpack steps) on a 2B-class
    matrix (6912 x 2560, the stack workload's up projection): one-trit-per-
    byte codes -> PACK5, and PACK5 -> codes; inputs cycle through >= 2 GiB
    of copies (each read cold); medians over STAT_LAUNCHES calls."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    K, N = inputs.STACK_SHAPES[0]
    W0 = torch.from_numpy(inputs.stack_master(0, 0)).to(dev)
    wq, _beta = ug.ug_quant_weight_absmean(W0)
    del W0
    pk = ug.ug_pack_trits(wq)
    n_q = -(-COLD_BYTES // (N * ug.packed_pitch(K) * 5)) + 1
    wqs = [wq] + [wq.clone() for _ in range(n_q - 1)]
    pks = [pk] + [pk.clone() for _ in range(n_q - 1)]
    pk_out = torch.empty_like(pk)
    wq_out = torch.empty_like(wq)
    for i in range(2):
        ug.ug_pack_trits(wqs[i], packed=pk_out)
        ug.ug_unpack_trits(pks[i], K, wq=wq_out)
    pmed, pp10, pp90 = launch_stats(
        torch, lambda i: ug.ug_pack_trits(wqs[(i + 2) % n_q], packed=pk_out), stream)
    umed, up10, up90 = launch_stats(
        torch, lambda i: ug.ug_unpack_trits(pks[(i + 2) % n_q], K, wq=wq_out), stream)
    alg = N * K + N * (-(-K // 5))  # codes one way, packed bytes the other
    res = dict(value=2 * alg / ((pmed + umed) * 1e-6) / 1e9, unit="GB/s",
               point="W_q [%d, %d] int8 <-> PACK5 [%d, %d]; %d copies of each cycled"
                     % (N, K, N, ug.packed_pitch(K), n_q),
               pack_us_median=pmed, pack_us_p10=pp10, pack_us_p90=pp90,
               pack_GBps=alg / (pmed * 1e-6) / 1e9,
               unpack_us_median=umed, unpack_us_p10=up10, unpack_us_p90=up90,
               unpack_GBps=alg / (umed * 1e-6) / 1e9,
               roofline=dict(bound="hbm", kernel="pack_kernel + unpack_kernel",
                             achieved=2 * alg / ((pmed + umed) * 1e-6) / 1e9, peak=HBM_PEAK_GBS,
                             unit="GB/s",
                             frac=2 * alg / ((pmed + umed) * 1e-6) / 1e9 / HBM_PEAK_GBS,
                             traffic=traffic_for("pack"), median_launch_us=(pmed + umed) / 2,
                             alg_bytes_per_launch=alg))
    log("pack", res)
    del wqs, pks
    return res


def measure_requant_pack5(torch, ug, inputs):
    """Requantization of a 2B-class fp32 master (6912 x 2560, the stack
    workload's up projection) straight to five trits per byte: the absmean
    sum, then the fused ternary + pack pass.  Calls cycle through >= 2 GiB of
    master copies (each read cold); the median over STAT_LAUNCHES calls."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    K, N = inputs.STACK_SHAPES[0]
    W0 = torch.from_numpy(inputs.stack_master(0, 0)).to(dev)
    n_copies = -(-COLD_BYTES // (4 * N * K))
    masters = [W0] + [W0.clone() for _ in range(n_copies - 1)]
    packed = torch.empty((N, ug.packed_pitch(K)), dtype=torch.uint8, device=dev)
    beta = torch.empty(1, dtype=torch.float32, device=dev)
    ws = torch.empty(ug.ug_quant_weight_absmean_workspace_size(N, K), dtype=torch.uint8,
                     device=dev)
    for i in range(2):
        ug.ug_quant_weight_absmean_pack5(masters[i], packed=packed, beta=beta, ws=ws)
    med, p10, p90 = launch_stats(
        torch, lambda i: ug.ug_quant_weight_absmean_pack5(masters[(i + 2) % n_copies],
                                                          packed=packed, beta=beta, ws=ws),
        stream)
    # the sum reads W, the fused pass reads it again and writes the bytes
    alg = 4 * N * K + 4 * N * K + N * (-(-K // 5)) + 4
    achieved = alg / (med * 1e-6) / 1e9
    out = dict(value=achieved, unit="GB/s",
               point="W fp32 [%d, %d] -> PACK5 [%d, %d] + beta; %d master copies (%.2f GiB) "
                     "cycled" % (N, K, N, ug.packed_pitch(K), n_copies,
                                 n_copies * 4 * N * K / 2 ** 30),
               median_call_us=med, p10_call_us=p10, p90_call_us=p90,
               roofline=dict(bound="hbm", kernel="absmean_stage1 + ternary_pack5",
                             achieved=achieved, peak=HBM_PEAK_GBS, unit="GB/s",
                             frac=achieved / HBM_PEAK_GBS, traffic=traffic_for("requant_pack5"),
                             median_launch_us=med, alg_bytes_per_launch=alg))
    log("requant pack5", out)
    del masters
    return out


def measure_attention_decode(torch, ug, T=4096, H=20, dh=128):
    """One decode step of causal attention over a K/V cache of T positions
    with 2B-class heads (d_model 2560 = 20 x 128): the new token's query
    against every cached key and value (fp32).  Calls cycle through >= 2 GiB
    of cache copies (each read cold); the median over STAT_LAUNCHES calls."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    d = H * dh
    g = torch.Generator(device="cuda:0").manual_seed(7)
    q = torch.randn((1, d), device=dev, generator=g)
    kv_bytes = 2 * T * d * 4
    n_copies = -(-COLD_BYTES // kv_bytes)
    caches = [(torch.randn((T, d), device=dev, generator=g),
               torch.randn((T, d), device=dev, generator=g)) for _ in range(n_copies)]
    out = torch.empty((1, d), device=dev)
    ws = torch.empty(ug.ug_attention_workspace_size(1, T - 1, H, dh), dtype=torch.uint8,
                     device=dev)
    for i in range(2):
        ug.ug_attention_cached(q, caches[i][0], caches[i][1], T - 1, H, out=out, ws=ws)
    med, p10, p90 = launch_stats(
        torch, lambda i: ug.ug_attention_cached(q, caches[(i + 2) % n_copies][0],
                                                caches[(i + 2) % n_copies][1], T - 1, H,
                                                out=out, ws=ws), stream)
    alg = kv_bytes + 4 * d + 4 * d  # the cache, the query, the context
    achieved = alg / (med * 1e-6) / 1e9
    res = dict(value=achieved, unit="GB/s",
               point="M=1 at position %d, %d heads x %d, fp32 K/V cache; %d cache copies "
                     "(%.2f GiB) cycled" % (T - 1, H, dh, n_copies,
                                           n_copies * kv_bytes / 2 ** 30),
               median_call_us=med, p10_call_us=p10, p90_call_us=p90,
               roofline=dict(bound="hbm", kernel="attn_partial<128> + attn_combine<128>",
                             achieved=achieved, peak=HBM_PEAK_GBS, unit="GB/s",
                             frac=achieved / HBM_PEAK_GBS, traffic=traffic_for("attention_decode"),
                             median_launch_us=med,
                             alg_bytes_per_launch=alg))
    log("attention decode", res)
    del caches
    return res


def measure_sampler(torch, ug, V=4096, k=100, B=4096):
    """Top-k sampling of the next token, 100 of 4096 logits ("a 1-bit llm,
    from scratch"): one row (the latency of a batch-1 decode step) and a
    batch of B rows (whole-chip throughput, bounded by reading the logits).
    Batches cycle through >= 2 GiB of logit copies; medians over
    STAT_LAUNCHES calls."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    g = torch.Generator(device="cuda:0").manual_seed(11)
    n_copies = max(2, -(-COLD_BYTES // (B * V * 4)))
    rows = [torch.randn((B, V), device=dev, generator=g) * 3.0 for _ in range(n_copies)]
    u = torch.rand(B, device=dev, generator=g)
    tok = torch.empty(B, dtype=torch.int32, device=dev)
    for i in range(2):
        ug.ug_sample_topk(rows[i], k, 0.8, u, tokens=tok)
    one_med, one_p10, one_p90 = launch_stats(
        torch, lambda i: ug.ug_sample_topk(rows[i % n_copies][:1], k, 0.8, u[:1], tokens=tok[:1]),
        stream)
    med, p10, p90 = launch_stats(
        torch, lambda i: ug.ug_sample_topk(rows[(i + 1) % n_copies], k, 0.8, u, tokens=tok),
        stream)
    alg = B * V * 4 + B * 4 + B * 4  # the logits, the draws, the tokens
    achieved = alg / (med * 1e-6) / 1e9
    res = dict(value=achieved, unit="GB/s",
               point="top-%d of %d logits, temperature 0.8: batch of %d rows (%d copies, "
                     "%.2f GiB, cycled) and a single row" % (k, V, B, n_copies,
                                                            n_copies * B * V * 4 / 2 ** 30),
               single_row_us_median=one_med, single_row_us_p10=one_p10,
               single_row_us_p90=one_p90, batch_us_median=med, batch_us_p10=p10,
               batch_us_p90=p90,
               roofline=dict(bound="hbm", kernel="topk_sample<true>", achieved=achieved,
                             peak=HBM_PEAK_GBS, unit="GB/s", frac=achieved / HBM_PEAK_GBS,
                             traffic=traffic_for("sampler"), median_launch_us=med, alg_bytes_per_launch=alg))
    log("sampler", res)
    del rows
    return res


FP32_MFMA_PEAK_TFLOPS = 157.3


def measure_backward(torch, ug, M=2048, N=6912, K=2560):
    """The straight-through backward of the stack workload's up projection
    (M = 2048 tokens, W 6912 x 2560): dx = g W and dW = g^T x on the fp32
    matrix cores (2 M N K flops each) and db; medians over STAT_LAUNCHES
    calls of each."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    gen = torch.Generator(device="cuda:0").manual_seed(13)
    g = torch.randn((M, N), device=dev, generator=gen) * 0.01
    x = torch.randn((M, K), device=dev, generator=gen)
    W = torch.randn((N, K), device=dev, generator=gen) * 0.02
    outs = {}
    ws = torch.empty(ug.lib().ug_bitlinear_backward_workspace_size(M, N, K), dtype=torch.uint8,
                     device=dev)
    # untimed load first: in a fresh process the first tens of milliseconds
    # of these products measured about 10% slower than the rest
    warm = ug.ug_bitlinear_backward(g, x, W, want=("dx", "dW"), ws=ws)
    for _ in range(40):
        ug.ug_bitlinear_backward(g, x, W, want=("dx", "dW"), ws=ws, **warm)
    torch.cuda.synchronize()
    for name in ("dx", "dW", "db"):
        res = ug.ug_bitlinear_backward(g, x, W, want=(name,), ws=ws)
        res["ws"] = ws
        med, p10, p90 = launch_stats(
            torch, lambda i: ug.ug_bitlinear_backward(g, x, W, want=(name,), **res), stream)
        outs[name] = (med, p10, p90)
    flops = 2 * M * N * K
    tf = {k: flops / (outs[k][0] * 1e-6) / 1e12 for k in ("dx", "dW")}
    achieved = 2 * flops / ((outs["dx"][0] + outs["dW"][0]) * 1e-6) / 1e12
    res = dict(value=achieved, unit="TFLOP/s",
               point="g [%d, %d], x [%d, %d], W [%d, %d] fp32" % (M, N, M, K, N, K),
               dx_us_median=outs["dx"][0], dx_TFLOPs=tf["dx"], dW_us_median=outs["dW"][0],
               dW_TFLOPs=tf["dW"], db_us_median=outs["db"][0],
               roofline=dict(bound="mfma", kernel="gemm_f32 (v_mfma_f32_16x16x4f32)",
                             achieved=achieved, peak=FP32_MFMA_PEAK_TFLOPS, unit="TFLOP/s",
                             frac=achieved / FP32_MFMA_PEAK_TFLOPS, traffic=traffic_for("backward"),
                             median_launch_us=(outs["dx"][0] + outs["dW"][0]) / 2,
                             alg_flops_per_launch=flops))
    log("backward", res)
    return res


def measure_stream_m1(torch, ug, inputs, M=1, si=0, marginal=True, read=None):
    """The streaming decode GEMV at one sweep point (default M = 1,
    2560 -> 6912, PACK5): grouped launches of G distinct weight copies
    (>= 128 MB each), launch sets cycling through >= 2 GiB of copies (cold);
    the median over STAT_LAUNCHES launches."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    K, N = inputs.SWEEP_SHAPES[si]
    x64, W = inputs.sweep_inputs(si, 64)
    wq, beta = ug.ug_quant_weight_absmean(torch.from_numpy(W).to(dev))
    pk = ug.ug_pack_trits(wq, packed=torch.empty((N, ug.stream_pitch(K)), dtype=torch.uint8,
                                                  device=dev))
    del wq, W
    G = max(1, (128 << 20) // (N * ug.stream_pitch(K)))
    xq, s = ug.ug_quant_act(torch.from_numpy(x64[:M].copy()).to(dev))
    y = ug.empty_pitched(M, N, torch.float32, dev)

    def timed(g):
        """Median launch time of groups of g weight copies, cold."""
        n_sets = max(2, COLD_BYTES // (g * N * ug.stream_pitch(K)) + 1)
        copies = [[pk.clone() for _ in range(g)] for _ in range(n_sets)]
        plans = [ug.ug_gemv_plan_init([dict(xq=xq, s=s, w=w, wfmt=ug.UG_W_PACK5, beta=beta, K=K,
                                             y=y) for w in cs]) for cs in copies]
        for i in range(2):
            ug.ug_bitlinear_gemv_grouped(plans[i % n_sets])
        r = launch_stats(
            torch, lambda i: ug.ug_bitlinear_gemv_grouped(plans[(i + 2) % n_sets]), stream)
        variant = plans[0].info.variant
        del plans, copies
        torch.cuda.empty_cache()
        return r, n_sets, variant

    (med, p10, p90), n_sets, variant = timed(G)
    # the same with twice the copies per launch: the difference is the
    # streaming time of G problems, the rest the launch's fixed cost
    med2 = timed(2 * G)[0][0] if marginal else med
    wbytes = N * (-(-K // 5)) * G
    alg = gemv_alg_bytes(M, N, K) * G
    achieved = alg / (med * 1e-6) / 1e9
    rate2 = alg / ((med2 - med) * 1e-6) / 1e9 if med2 > med else None
    kernel = "gemv_stream_grouped<PACK5, 1%s>" % (", spread" if (variant >> 13) & 1 else "")
    out = dict(value=wbytes / (med * 1e-6) / 1e9, unit="GB/s",
               point="M=%d K=%d N=%d, PACK5, %d weight copies per launch, %d launch sets "
                     "(%.2f GiB) cycled" % (M, K, N, G, n_sets,
                                           n_sets * G * N * ug.stream_pitch(K) / 2 ** 30),
               median_launch_us=med, p10_launch_us=p10, p90_launch_us=p90,
               median_launch_us_2x=med2 if marginal else None,
               marginal_GBps=rate2, fixed_us_per_launch=2 * med - med2 if marginal else None,
               roofline=dict(bound="hbm", kernel=kernel,
                             achieved=achieved, peak=HBM_PEAK_GBS, unit="GB/s",
                             frac=achieved / HBM_PEAK_GBS,
                             frac_marginal=rate2 / HBM_PEAK_GBS if rate2 else None,
                             # against the measured streaming-read ceiling
                             # (ug_hbm_read_probe, same size per call)
                             frac_of_read_ceiling=achieved / read["value"] if read else None,
                             marginal_frac_of_read_ceiling=(
                                 rate2 / read["marginal_GBps"]
                                 if read and rate2 and read["marginal_GBps"] else None),
                             traffic=traffic_for("sweep") if (M, si) == (1, 0) else None,
                             median_launch_us=med, alg_bytes_per_launch=alg))
    log("stream", out)
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
    flush = Flusher(torch)
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
        # rows of at least 1 KB start on a cache line (ug.stream_pitch)
        pk = ug.ug_pack_trits(wq, packed=torch.empty((N, ug.stream_pitch(K)), dtype=torch.uint8,
                                                      device=dev))
        del wq
        wbytes = N * (-(-K // 5))
        G = max(1, (128 << 20) // (N * ug.stream_pitch(K)))
        n_sets = max(2, COLD_BYTES // (G * N * ug.stream_pitch(K)) + 1)
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
                time_graph(torch, g, stream)  # first replay untimed (one-time set-up)
                flush()
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
            time_graph(torch, g1, stream)
            flush()
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
                    spread = (plans[0].info.variant >> 13) & 1
                    dom = dict(bound="hbm",
                               kernel="gemv_stream_grouped<PACK5, 1%s>" % (", spread" * spread),
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
                                   cores=oracle.num_threads(), cpu_model=cpu_model(), kind="oracle",
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
    # requantization straight to five trits per byte (the deployed format)
    # of the same 60 masters, timed on its own
    pk_bufs = {K: torch.empty((N, ug.packed_pitch(K)), dtype=torch.uint8, device=dev)
               for (K, N) in inputs.STACK_SHAPES}
    e[0].record(stream)
    for _ in range(steps):
        for m in mats:
            ug.ug_quant_weight_absmean_pack5(m["W"], packed=pk_bufs[m["K"]], beta=m["beta"], ws=ws)
    e[1].record(stream)
    torch.cuda.synchronize()
    t_req5 = e[0].elapsed_time(e[1]) / steps
    req5_bytes = sum(8 * m["N"] * m["K"] + m["N"] * (-(-m["K"] // 5)) for m in mats)
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
                       "requant_pack5_ms_per_step": t_req5,
                       "requant_pack5_GBps": req5_bytes / (t_req5 / 1e3) / 1e9,
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
                                   cores=oracle.num_threads(), cpu_model=cpu_model(), kind="oracle",
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
                                   cores=oracle.num_threads(), cpu_model=cpu_model(), kind="oracle",
                                   sample="%d whole steps (weight quant + act quant + matmul + "
                                          "rescale) in %.1f s" % (n, secs))
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
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
    if args.only is not None:
        fn = {"prefill_gemm": lambda: measure_prefill_gemm(torch, ug, inputs),
              "vendor_int8_gemm": lambda: measure_vendor_gemm(torch, ug, inputs),
              "hbm_copy_rate": lambda: measure_copy_rate(torch),
              "pack": lambda: measure_pack(torch, ug, inputs),
              "stream_m1": lambda: measure_stream_m1(torch, ug, inputs,
                                                     marginal=not args.no_marginal),
              "hbm_read_rate": lambda: measure_hbm_read(torch, ug),
              "requant_pack5": lambda: measure_requant_pack5(torch, ug, inputs),
              "attention_decode": lambda: measure_attention_decode(torch, ug),
              "sampler": lambda: measure_sampler(torch, ug),
              "backward": lambda: measure_backward(torch, ug),
              "mfma_sustained": lambda: measure_mfma_sustained(torch, ug)}[args.only]
        print(json.dumps({"point": args.only, **fn()}), flush=True)
        return
    runners = {"decode_stack": run_decode_stack, "prefill": run_prefill, "sweep": run_sweep,
               "stack": run_stack, "tiny": run_tiny}
    res = runners[args.workload](args, torch, ug, inputs)
    line = {"metric": METRIC, "value": res["value"], "unit": res["unit"], "n_gpus": 1,
            "steps": res["steps"], "warmup": res["warmup"], "ms_per_step": res["ms_per_step"],
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": res["dtype"], "data": "synthetic (seeded numpy, shapes of the workload)",
            "config": res["config"], "roofline": res["roofline"]}
    for k in ("mfma_sustained", "prefill_gemm", "vendor_int8_gemm", "hbm_copy_rate",
              "hbm_read_rate", "stream_m1",
              "pack", "requant_pack5", "attention_decode", "sampler", "backward",
              "cpu_baseline"):
        if k in res:
            line[k] = res[k]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
