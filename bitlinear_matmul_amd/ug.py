"""Python binding of libug (``include/ug.h``): argument marshalling only.

Each function has the name of the C entry point it calls.  Tensors are
torch tensors on the GPU; the binding reads their pointers, shapes and row
pitches, allocates outputs with torch when the caller passes none (torch is
the device-memory and stream provider), and calls the C ABI on torch's
current stream.  Every step of the computation runs in libug's HIP kernels;
there is no fallback: if ``libug.so`` is missing or a call fails, this raises.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libug.so")

UG_OK = 0
UG_ERR_INVALID_ARG = 1
UG_ERR_UNSUPPORTED = 2
UG_ERR_WORKSPACE = 3
UG_ERR_HIP = 4

UG_W_I8 = 0
UG_W_PACK5 = 1

UG_MAX_K = 132104
UG_GEMV_MAX_M = 64

# Every symbol the header declares, with (restype, argtypes).
_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_f32 = ctypes.c_float
_sz = ctypes.c_size_t
SIGNATURES = {
    "ug_version": (_i32, []),
    "ug_status_string": (ctypes.c_char_p, [_i32]),
    "ug_last_hip_error": (_i32, []),
    "ug_quant_act": (_i32, [_vp, _i64, _i64, _i64, _f32, _vp, _i64, _vp, _vp]),
    "ug_rmsnorm_quant_act": (_i32, [_vp, _i64, _vp, _i64, _i64, _f32, _f32, _vp, _i64, _vp, _vp]),
    "ug_quant_weight_absmean_workspace_size": (_sz, [_i64, _i64]),
    "ug_quant_weight_absmean": (_i32, [_vp, _i64, _i64, _i64, _f32, _vp, _i64, _vp, _vp, _sz,
                                       _vp]),
    "ug_quant_weight_absmean_pack5": (_i32, [_vp, _i64, _i64, _i64, _f32, _vp, _i64, _vp, _vp,
                                             _sz, _vp]),
    "ug_quant_weight_absmean_static": (_i32, [_vp, _i64, _i64, _i64, _f32, _vp, _i64, _vp,
                                              _vp]),
    "ug_pack_trits": (_i32, [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _vp]),
    "ug_unpack_trits": (_i32, [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _vp]),
    "ug_bitlinear_gemv": (_i32, [_vp, _i64, _vp, _vp, _i32, _i64, _vp, _vp, _i64, _i64, _i64,
                                 _vp, _i64, _vp, _i64, _vp]),
    "ug_bitlinear_gemm_workspace_size": (_sz, [_i64, _i64, _i64, _i32]),
    "ug_gemv_plan_size": (_sz, [_i32]),
    "ug_gemv_plan_init": (_i32, [_vp, _i32, _vp, _sz, _vp]),
    "ug_bitlinear_gemv_grouped": (_i32, [_vp, _vp, _vp]),
    "ug_bitlinear_gemm": (_i32, [_vp, _i64, _vp, _vp, _i32, _i64, _vp, _vp, _i64, _i64, _i64,
                                 _vp, _i64, _vp, _i64, _vp, _sz, _vp]),
    "ug_bitlinear_gemm_tiled": (_i32, [_vp, _i64, _vp, _vp, _i32, _i64, _vp, _vp, _i64, _i64,
                                       _i64, _vp, _i64, _vp, _i64, _vp, _sz, _i32, _i32, _vp]),
    "ug_bitlinear_backward_workspace_size": (_sz, [_i64, _i64, _i64]),
    "ug_bitlinear_backward": (_i32, [_vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _i64, _vp,
                                     _i64, _vp, _i64, _vp, _vp, _sz, _vp]),
    "ug_sample_topk": (_i32, [_vp, _i64, _i64, _i64, _i64, _f32, _vp, _vp, _vp, _i64, _vp, _i64,
                              _vp, _i64, _vp]),
    "ug_attention_workspace_size": (_sz, [_i64, _i64, _i64, _i64]),
    "ug_attention_cached": (_i32, [_vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _i64, _i64, _vp,
                                   _i64, _vp, _sz, _vp]),
    "ug_mfma_rate_probe": (_i32, [_i32, _i32, _i32, _vp, _vp]),
    "ug_hbm_read_probe": (_i32, [_vp, _sz, _i32, _i32, _vp, _vp]),
}

UG_GEMM_COUNTER_BYTES = 2048

_lib = None


class GemvProblem(ctypes.Structure):
    """ug_gemv_problem (include/ug.h)."""
    _fields_ = [("x", _vp), ("ldx", _i64), ("eps", _f32), ("xq", _vp), ("ldxq", _i64),
                ("s", _vp), ("w", _vp), ("wfmt", _i32), ("ldw", _i64), ("beta", _vp),
                ("bias", _vp), ("M", _i64), ("N", _i64), ("K", _i64), ("acc", _vp), ("ldacc", _i64),
                ("y", _vp), ("ldy", _i64)]


class GemvPlanInfo(ctypes.Structure):
    """ug_gemv_plan_info (include/ug.h)."""
    _fields_ = [("count", _i32), ("total_items", _i32), ("variant", _i32), ("grid", _i32)]


class UgError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = "%s failed: %s" % (where, status_string(status))
        if status == UG_ERR_HIP:
            msg += " (hipError %d)" % lib().ug_last_hip_error()
        super().__init__(msg)


def lib():
    """The loaded libug.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libug.so is not built (%s); run __graft_entry__.build()"
                               % LIB_PATH)
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


def status_string(st):
    return lib().ug_status_string(int(st)).decode()


def _check(st, where):
    if st != UG_OK:
        raise UgError(st, where)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _p(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _ld(t):
    """Row pitch (elements) of a 2-D tensor with unit column stride."""
    if t.dim() != 2 or (t.stride(1) != 1 and t.shape[1] > 1):
        raise ValueError("expected a 2-D tensor with contiguous rows")
    return t.stride(0) if t.shape[0] > 1 else max(t.stride(0), t.shape[1])


def round_up(a, b):
    return -(-a // b) * b


def empty_pitched(rows, cols, dtype, device, align_bytes=16):
    """[rows, cols] view of a [rows, ld] allocation, ld*itemsize a multiple of
    align_bytes (the pitches the ABI wants)."""
    item = torch.empty((), dtype=dtype).element_size()
    ld = round_up(cols * item, align_bytes) // item
    return torch.empty((rows, ld), dtype=dtype, device=device)[:, :cols]


def packed_pitch(K):
    """Smallest valid UG_W_PACK5 row pitch (bytes) for K inputs."""
    return round_up(-(-K // 5), 16)


def stream_pitch(K):
    """UG_W_PACK5 row pitch for weights the GEMV streams: rows of at least
    1 KB start on a 128-byte cache line (at most 1/8 more bytes), so no
    64-byte piece of a row straddles two lines; shorter rows keep the
    smallest pitch."""
    rb = -(-K // 5)
    return round_up(rb, 128) if rb >= 1024 else packed_pitch(K)


def ug_version():
    return lib().ug_version()


def ug_last_hip_error():
    return lib().ug_last_hip_error()


def ug_quant_act(x, eps=1e-5, xq=None, s=None, stream=None):
    """Per-row absmax int8 quantization.  x fp32 [M,K] -> (xq int8 [M,K],
    s fp32 [M])."""
    M, K = x.shape
    if xq is None:
        xq = empty_pitched(M, K, torch.int8, x.device)
    if s is None:
        s = torch.empty(M, dtype=torch.float32, device=x.device)
    _check(lib().ug_quant_act(_p(x), _ld(x), M, K, eps, _p(xq), _ld(xq), _p(s), _stream(stream)),
           "ug_quant_act")
    return xq, s


def ug_rmsnorm_quant_act(x, g=None, eps_norm=1e-5, eps=1e-5, xq=None, s=None, stream=None):
    """RMSNorm (fp32 gain g, None = ones) fused with per-row quantization."""
    M, K = x.shape
    if xq is None:
        xq = empty_pitched(M, K, torch.int8, x.device)
    if s is None:
        s = torch.empty(M, dtype=torch.float32, device=x.device)
    _check(lib().ug_rmsnorm_quant_act(_p(x), _ld(x), _p(g), M, K, eps_norm, eps, _p(xq), _ld(xq),
                                      _p(s), _stream(stream)), "ug_rmsnorm_quant_act")
    return xq, s


def ug_quant_weight_absmean_workspace_size(N, K):
    return lib().ug_quant_weight_absmean_workspace_size(N, K)


def ug_quant_weight_absmean(W, eps=1e-5, wq=None, beta=None, ws=None, stream=None):
    """Absmean ternary quantization.  W fp32 [N,K] -> (wq int8 [N,K],
    beta fp32 [1] on the device)."""
    N, K = W.shape
    if wq is None:
        wq = empty_pitched(N, K, torch.int8, W.device)
    if beta is None:
        beta = torch.empty(1, dtype=torch.float32, device=W.device)
    need = ug_quant_weight_absmean_workspace_size(N, K)
    if ws is None:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=W.device)
    _check(lib().ug_quant_weight_absmean(_p(W), _ld(W), N, K, eps, _p(wq), _ld(wq), _p(beta),
                                         _p(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "ug_quant_weight_absmean")
    return wq, beta


def ug_quant_weight_absmean_pack5(W, eps=1e-5, packed=None, beta=None, ws=None, stream=None):
    """Absmean ternary quantization written straight as 5 trits per byte.
    W fp32 [N,K] -> (packed uint8 [N, ldp] full pitched rows, beta fp32 [1])."""
    N, K = W.shape
    if packed is None:
        packed = torch.empty((N, packed_pitch(K)), dtype=torch.uint8, device=W.device)
    if beta is None:
        beta = torch.empty(1, dtype=torch.float32, device=W.device)
    need = ug_quant_weight_absmean_workspace_size(N, K)
    if ws is None:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=W.device)
    _check(lib().ug_quant_weight_absmean_pack5(_p(W), _ld(W), N, K, eps, _p(packed),
                                               _ld(packed), _p(beta), _p(ws),
                                               ws.numel() * ws.element_size(), _stream(stream)),
           "ug_quant_weight_absmean_pack5")
    return packed, beta


def ug_quant_weight_absmean_static(W, eps=1e-5, wq=None, beta=None, stream=None):
    """ug_quant_weight_absmean through the library's static scratch array
    (the C call allocates nothing and takes no workspace).  Pass wq and beta
    to keep this call free of allocations too."""
    N, K = W.shape
    if wq is None:
        wq = empty_pitched(N, K, torch.int8, W.device)
    if beta is None:
        beta = torch.empty(1, dtype=torch.float32, device=W.device)
    _check(lib().ug_quant_weight_absmean_static(_p(W), _ld(W), N, K, eps, _p(wq), _ld(wq),
                                                _p(beta), _stream(stream)),
           "ug_quant_weight_absmean_static")
    return wq, beta


def ug_pack_trits(wq, packed=None, bad_count=None, stream=None):
    """One trit per byte -> five trits per byte.  Returns packed uint8
    [N, ldp] (the full pitched rows)."""
    N, K = wq.shape
    if packed is None:
        packed = torch.empty((N, packed_pitch(K)), dtype=torch.uint8, device=wq.device)
    _check(lib().ug_pack_trits(_p(wq), _ld(wq), N, K, _p(packed), _ld(packed), _p(bad_count),
                               _stream(stream)), "ug_pack_trits")
    return packed


def ug_unpack_trits(packed, K, wq=None, bad_count=None, stream=None):
    """Five trits per byte -> one trit per byte, int8 [N, K]."""
    N = packed.shape[0]
    if wq is None:
        wq = empty_pitched(N, K, torch.int8, packed.device)
    _check(lib().ug_unpack_trits(_p(packed), _ld(packed), N, K, _p(wq), _ld(wq), _p(bad_count),
                                 _stream(stream)), "ug_unpack_trits")
    return wq


def _weight_args(w, wfmt, K):
    if wfmt == UG_W_PACK5:
        return w.shape[0], _ld(w)
    if w.shape[1] != K:
        raise ValueError("int8 weight must be [N, K]")
    return w.shape[0], _ld(w)


def ug_bitlinear_gemv(xq, s, w, wfmt, beta, K=None, acc=None, y=None, want_acc=False,
                      want_y=True, bias=None, stream=None):
    """Decode GEMV: xq int8 [M,K] (M <= 64), w int8 [N,K] or packed uint8
    [N,ldp] -> (acc int32 [M,N] or None, y fp32 [M,N] or None); bias: fp32
    [N] added to y, or None."""
    M = xq.shape[0]
    K = xq.shape[1] if K is None else K
    N, ldw = _weight_args(w, wfmt, K)
    if want_acc and acc is None:
        acc = empty_pitched(M, N, torch.int32, xq.device)
    if want_y and y is None:
        y = empty_pitched(M, N, torch.float32, xq.device)
    _check(lib().ug_bitlinear_gemv(_p(xq), _ld(xq), _p(s), _p(w), wfmt, ldw, _p(beta), _p(bias),
                                   M, N, K, _p(acc), _ld(acc) if acc is not None else 0, _p(y),
                                   _ld(y) if y is not None else 0, _stream(stream)),
           "ug_bitlinear_gemv")
    return acc, y


def ug_bitlinear_gemm_workspace_size(M, N, K, wfmt):
    return lib().ug_bitlinear_gemm_workspace_size(M, N, K, wfmt)


_gemm_ws_cache = {}


def gemm_workspace(need, device):
    """The per-device GEMM workspace, grown on demand.  One buffer serves
    all calls that do not overlap in time; calls running concurrently on
    different streams must each pass their own buffer."""
    key = (device.type, device.index)
    t = _gemm_ws_cache.get(key)
    if t is None or t.numel() < need:
        t = torch.empty(need, dtype=torch.uint8, device=device)
        _gemm_ws_cache[key] = t
    return t


def ug_bitlinear_gemm(xq, s, w, wfmt, beta, K=None, acc=None, y=None, want_acc=False,
                      want_y=True, ws=None, split=True, tile=None, k_splits=None, bias=None,
                      stream=None):
    """Prefill GEMM (int8 MFMA): same arguments as the GEMV, any M.
    ws: workspace (default: the shared per-device one); split=False passes
    only what UG_W_PACK5 decoding needs, so every block computes whole
    tiles.  tile / k_splits (ug_bitlinear_gemm_tiled): force the tile shape
    (0: 256 x 256, 1: 256 x 160) and the K-split count."""
    M = xq.shape[0]
    K = xq.shape[1] if K is None else K
    N, ldw = _weight_args(w, wfmt, K)
    if want_acc and acc is None:
        acc = empty_pitched(M, N, torch.int32, xq.device)
    if want_y and y is None:
        y = empty_pitched(M, N, torch.float32, xq.device)
    need = ug_bitlinear_gemm_workspace_size(M, N, K, wfmt)
    if not split:
        # a private buffer with room for the decoded weights only (they
        # follow the counter bytes), too small for the split area
        need = UG_GEMM_COUNTER_BYTES + N * (-(-K // 16) * 16) if wfmt == UG_W_PACK5 else 0
        if ws is None and need:
            ws = torch.empty(need, dtype=torch.uint8, device=xq.device)
    if ws is None and need:
        ws = gemm_workspace(need, xq.device)
    # the whole buffer: the library lays it out by its size alone
    ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    args = [_p(xq), _ld(xq), _p(s), _p(w), wfmt, ldw, _p(beta), _p(bias), M, N, K,
            _p(acc), _ld(acc) if acc is not None else 0, _p(y), _ld(y) if y is not None else 0,
            _p(ws) if ws_bytes else None, ws_bytes]
    if tile is None and k_splits is None:
        _check(lib().ug_bitlinear_gemm(*args, _stream(stream)), "ug_bitlinear_gemm")
    else:
        _check(lib().ug_bitlinear_gemm_tiled(*args, -1 if tile is None else tile,
                                             -1 if k_splits is None else k_splits,
                                             _stream(stream)), "ug_bitlinear_gemm_tiled")
    return acc, y


class GemvPlan:
    """A grouped-GEMV plan: the device descriptor buffer (a torch tensor)
    plus the host launch info, and the tensors it names (kept alive)."""

    def __init__(self, buf, info, keep):
        self.buf = buf
        self.info = info
        self.keep = keep


def ug_gemv_plan_size(count):
    return lib().ug_gemv_plan_size(count)


def ug_gemv_plan_init(problems, device=None):
    """problems: list of dicts with keys x (fp32 [M,K] to quantize in the
    launch) or xq+s (pre-quantized), w, wfmt, beta, K, y, and optionally
    acc, xq/s as outputs when x is given, eps.  Returns a GemvPlan."""
    arr = (GemvProblem * len(problems))()
    keep = []
    for i, p in enumerate(problems):
        x, xq, s, w, y, acc, bias = (p.get(k) for k in ("x", "xq", "s", "w", "y", "acc", "bias"))
        ref = x if x is not None else xq
        M = ref.shape[0]
        K = p.get("K", ref.shape[1])
        wfmt = p["wfmt"]
        N = w.shape[0]
        arr[i] = GemvProblem(
            x=_p(x).value, ldx=_ld(x) if x is not None else 0, eps=p.get("eps", 1e-5),
            xq=_p(xq).value, ldxq=_ld(xq) if xq is not None else 0, s=_p(s).value,
            w=_p(w).value, wfmt=wfmt, ldw=_ld(w), beta=_p(p["beta"]).value,
            bias=_p(bias).value, M=M, N=N, K=K,
            acc=_p(acc).value, ldacc=_ld(acc) if acc is not None else 0,
            y=_p(y).value, ldy=_ld(y) if y is not None else 0)
        keep.append(p)
    size = ug_gemv_plan_size(len(problems))
    dev = device or ref.device
    buf = torch.empty(size, dtype=torch.uint8, device=dev)
    info = GemvPlanInfo()
    _check(lib().ug_gemv_plan_init(ctypes.cast(arr, _vp), len(problems), _p(buf), size,
                                   ctypes.byref(info)), "ug_gemv_plan_init")
    return GemvPlan(buf, info, keep)


def ug_bitlinear_gemv_grouped(plan, stream=None):
    """One launch of every problem of a GemvPlan."""
    _check(lib().ug_bitlinear_gemv_grouped(_p(plan.buf), ctypes.byref(plan.info),
                                           _stream(stream)), "ug_bitlinear_gemv_grouped")


def ug_attention_workspace_size(M, pos0, H, dh):
    return lib().ug_attention_workspace_size(M, pos0, H, dh)


def ug_attention_cached(q, kc, vc, pos0, H, out=None, ws=None, stream=None):
    """Causal attention of q fp32 [M, H*dh] (row m at position pos0 + m)
    over the cache rows kc, vc fp32 [>= pos0 + M, H*dh] -> out fp32
    [M, H*dh]."""
    M, HD = q.shape
    dh = HD // H
    if out is None:
        out = empty_pitched(M, HD, torch.float32, q.device)
    need = ug_attention_workspace_size(M, pos0, H, dh)
    if ws is None:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check(lib().ug_attention_cached(_p(q), _ld(q), _p(kc), _ld(kc), _p(vc), _ld(vc), M, pos0, H,
                                     dh, _p(out), _ld(out), _p(ws),
                                     ws.numel() * ws.element_size(), _stream(stream)),
           "ug_attention_cached")
    return out


def ug_sample_topk(logits, k, temperature, u, tokens=None, want_topk=False, stream=None):
    """Top-k sampling: logits fp32 [B, V], u fp32 [B] uniform draws ->
    tokens int32 [B] (and, with want_topk, the kept indices, logits and
    probabilities [B, k] in rank order)."""
    B, V = logits.shape
    dev = logits.device
    if tokens is None:
        tokens = torch.empty(B, dtype=torch.int32, device=dev)
    idx = val = prob = None
    if want_topk:
        idx = torch.empty((B, k), dtype=torch.int32, device=dev)
        val = torch.empty((B, k), dtype=torch.float32, device=dev)
        prob = torch.empty((B, k), dtype=torch.float32, device=dev)
    _check(lib().ug_sample_topk(_p(logits), _ld(logits), B, V, k, temperature, _p(u), _p(tokens),
                                _p(idx), k if idx is not None else 0, _p(val),
                                k if val is not None else 0, _p(prob),
                                k if prob is not None else 0, _stream(stream)),
           "ug_sample_topk")
    return (tokens, idx, val, prob) if want_topk else tokens


def ug_bitlinear_backward(g, x, W, want=("dx", "dW", "db"), dx=None, dW=None, db=None,
                          ws=None, stream=None):
    """Straight-through backward: g fp32 [M, N], x fp32 [M, K], W fp32
    [N, K] -> dict with dx [M, K], dW [N, K], db [N] (those in `want`)."""
    M, N = g.shape
    K = W.shape[1] if W is not None else x.shape[1]
    dev = g.device
    if "dx" in want and dx is None:
        dx = empty_pitched(M, K, torch.float32, dev)
    if "dW" in want and dW is None:
        dW = empty_pitched(N, K, torch.float32, dev)
    if "db" in want and db is None:
        db = torch.empty(N, dtype=torch.float32, device=dev)
    if ws is None:
        ws = torch.empty(max(16, lib().ug_bitlinear_backward_workspace_size(M, N, K)),
                         dtype=torch.uint8, device=dev)
    _check(lib().ug_bitlinear_backward(
        _p(g), _ld(g), _p(x), _ld(x) if x is not None else 0, _p(W),
        _ld(W) if W is not None else 0, M, N, K,
        _p(dx if "dx" in want else None), _ld(dx) if "dx" in want else 0,
        _p(dW if "dW" in want else None), _ld(dW) if "dW" in want else 0,
        _p(db if "db" in want else None), _p(ws), ws.numel() if ws is not None else 0,
        _stream(stream)), "ug_bitlinear_backward")
    out = {}
    for name, t in (("dx", dx), ("dW", dW), ("db", db)):
        if name in want:
            out[name] = t
    return out


MFMA_PROBE_OPS = {0: 2 * 32 * 32 * 32, 1: 2 * 16 * 16 * 4}  # per instruction


def ug_mfma_rate_probe(kind, blocks, iters, sink, stream=None):
    """Measurement helper (not a step of the forward path): iters x 16
    back-to-back matrix instructions per wave, four waves per block (kind 0:
    int8 32x32x32, kind 1: fp32 16x16x4); sink int32 [4 * blocks] on the
    device.  Returns the operation count, for the caller to divide by the
    time it measures."""
    _check(lib().ug_mfma_rate_probe(kind, blocks, iters, _p(sink), _stream(stream)),
           "ug_mfma_rate_probe")
    return 4 * blocks * iters * 16 * MFMA_PROBE_OPS[kind]


def ug_hbm_read_probe(buf, blocks, sink, walk=1, nbytes=None, stream=None):
    """Measurement helper (not a step of the forward path): reads nbytes
    (default: all) of the device tensor buf once (walk 0: one grid stride;
    walk 1: a contiguous range per block); sink uint32/int32 [4 * blocks]
    on the device, whose XOR is the XOR of every 32-bit word read.  Returns
    the byte count, for the caller to divide by the time it measures."""
    n = buf.numel() * buf.element_size() if nbytes is None else nbytes
    _check(lib().ug_hbm_read_probe(_p(buf), n, blocks, walk, _p(sink), _stream(stream)),
           "ug_hbm_read_probe")
    return n
