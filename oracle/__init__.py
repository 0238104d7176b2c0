"""CPU oracle for the BitLinear forward pass -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls it.

The arithmetic lives in ``ugref.c`` (plain scalar loops, fp32 in the fixed
orders documented there); this module only marshals numpy arrays in and out
through ctypes.  Each function cites the passage of the pages it follows:

* "ultragraph - when the graph is the 1-bit LLM, part 2", section
  "the bytes" -- absmean ternary weights, per-row absmax int8 activations,
  the [-127, 127] range, dequantization by one scalar multiply;
* same page, section "autograd on a byte-graph" -- y = (x_q W_q^T)(s beta);
* same page, section "attention, as graph ops" -- RMSNorm with fp32 gain;
* "ultragraph-1bit 0.12.0" README, sections "A whole ternary GPT" and
  "Layout" -- five ternary values per byte.

The pages give no summation order for beta or for the RMSNorm sum of
squares; this oracle states one (see ugref.c).  Those orders are pinned
bit for bit by hand-worked fixtures (tests/golden/absmean_order.txt,
row_order.txt) on which any other lane map, fold or stage-2 assignment gives
different bits; the true divisions, round-half-even and the (s*beta)
grouping of the rescale are pinned by tests/golden/rounding_cases.txt.
tests/test_oracle_mutants.py plants each of those slips in a copy of
ugref.c and checks that a pin fails.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None

_f32p = ctypes.POINTER(ctypes.c_float)
_i8p = ctypes.POINTER(ctypes.c_int8)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_i64 = ctypes.c_int64
_f32 = ctypes.c_float


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = _build.LIB
    if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
        _build.build()
    _lib = _open(path)
    return _lib


class use_library:
    """Context manager that points every function of this module at another
    build of the oracle for the duration of a with-block (the pin tests use
    it to check that deliberately wrong builds fail them)."""

    def __init__(self, path):
        self.path = path

    def __enter__(self):
        global _lib
        self.prev = _lib
        _lib = _open(self.path)
        return _lib

    def __exit__(self, *exc):
        global _lib
        _lib = self.prev
        return False


def _open(path):
    lib = ctypes.CDLL(path)
    sig = {
        "ugref_quant_act": (None, [_f32p, _i64, _i64, _i64, _f32, _i8p, _i64, _f32p]),
        "ugref_rmsnorm": (None, [_f32p, _i64, _f32p, _i64, _i64, _f32, _f32p, _i64]),
        "ugref_row_sum_squares": (_f32, [_f32p, _i64]),
        "ugref_rmsnorm_quant_act": (None, [_f32p, _i64, _f32p, _i64, _i64, _f32, _f32,
                                           _i8p, _i64, _f32p]),
        "ugref_absmean_sum": (_f32, [_f32p, _i64, _i64, _i64, _f32p]),
        "ugref_quant_weight_absmean": (None, [_f32p, _i64, _i64, _i64, _f32, _i8p, _i64,
                                              _f32p]),
        "ugref_pack_trits": (_i64, [_i8p, _i64, _i64, _i64, _u8p, _i64]),
        "ugref_unpack_trits": (_i64, [_u8p, _i64, _i64, _i64, _i8p, _i64]),
        "ugref_matmul_i32": (None, [_i8p, _i64, _i8p, _i64, _i64, _i64, _i64, _i32p, _i64]),
        "ugref_matmul_i32_pairs": (None, [_i8p, _i64, _i8p, _i64, _i64, _i64p, _i64p, _i64,
                                          _i32p]),
        "ugref_epilogue": (None, [_i32p, _i64, _f32p, _f32, _f32p, _i64, _i64, _f32p, _i64]),
        "ugref_sample_topk": (None, [_f32p, _i64, _i64, _i64, _i64, _f32, _f32p, _i32p, _i32p,
                                     _f32p, ctypes.POINTER(ctypes.c_double)]),
        "ugref_bitlinear_backward": (None, [_f32p, _i64, _f32p, _i64, _f32p, _i64, _i64, _i64,
                                            _i64, _f32p, _i64, _f32p, _i64, _f32p]),
        "ugref_attention": (None, [_f32p, _i64, _f32p, _i64, _f32p, _i64, _i64, _i64, _i64,
                                   _i64, _f32p, _i64]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _c2d(a, dtype):
    a = np.asarray(a)
    if a.dtype != dtype:
        raise TypeError("expected %s, got %s" % (dtype, a.dtype))
    if a.ndim != 2:
        raise ValueError("expected a 2-D array")
    return np.ascontiguousarray(a)


def quant_act(x, eps=1e-5):
    """Per-row absmax int8 quantization ("the bytes": s = max|x|/127 + eps,
    x_q = clip(round(x/s), -127, 127)).  Returns (x_q int8 [M,K], s fp32 [M])."""
    x = _c2d(x, np.float32)
    M, K = x.shape
    xq = np.empty((M, K), np.int8)
    s = np.empty(M, np.float32)
    _load().ugref_quant_act(_ptr(x, ctypes.c_float), K, M, K, float(np.float32(eps)),
                            _ptr(xq, ctypes.c_int8), K, _ptr(s, ctypes.c_float))
    return xq, s


def row_sum_squares(x_row):
    """Sum of squares of one row in the fixed slot order used by rmsnorm()."""
    x = np.ascontiguousarray(np.asarray(x_row, np.float32).reshape(-1))
    return np.float32(_load().ugref_row_sum_squares(_ptr(x, ctypes.c_float), x.size))


def rmsnorm(x, g=None, eps_n=1e-5):
    """RMSNorm with fp32 gain ("attention, as graph ops"):
    x / sqrt(mean(x^2) + eps) * g.  g=None means ones."""
    x = _c2d(x, np.float32)
    M, K = x.shape
    gp = None
    if g is not None:
        g = np.ascontiguousarray(np.asarray(g, np.float32).reshape(K))
        gp = _ptr(g, ctypes.c_float)
    xn = np.empty((M, K), np.float32)
    _load().ugref_rmsnorm(_ptr(x, ctypes.c_float), K, gp, M, K, float(np.float32(eps_n)),
                          _ptr(xn, ctypes.c_float), K)
    return xn


def rmsnorm_quant_act(x, g=None, eps_n=1e-5, eps=1e-5):
    """RMSNorm followed by per-row absmax quantization of its output."""
    x = _c2d(x, np.float32)
    M, K = x.shape
    gp = None
    if g is not None:
        g = np.ascontiguousarray(np.asarray(g, np.float32).reshape(K))
        gp = _ptr(g, ctypes.c_float)
    xq = np.empty((M, K), np.int8)
    s = np.empty(M, np.float32)
    _load().ugref_rmsnorm_quant_act(_ptr(x, ctypes.c_float), K, gp, M, K,
                                    float(np.float32(eps_n)), float(np.float32(eps)),
                                    _ptr(xq, ctypes.c_int8), K, _ptr(s, ctypes.c_float))
    return xq, s


def absmean_sum(W, return_chunks=False):
    """Sum of |W| over the whole tensor in the fixed two-stage order."""
    W = _c2d(W, np.float32)
    N, K = W.shape
    nchunks = -(-(N * K) // 8192)
    S = np.empty(max(nchunks, 1), np.float32)
    T = np.float32(_load().ugref_absmean_sum(_ptr(W, ctypes.c_float), K, N, K,
                                             _ptr(S, ctypes.c_float)))
    return (T, S[:nchunks]) if return_chunks else T


def quant_weight_absmean(W, eps=1e-5):
    """Absmean ternary quantization ("the bytes": beta = mean|W| + eps,
    W_q = clip(round(W/beta), -1, 1)).  Returns (W_q int8 [N,K], beta fp32)."""
    W = _c2d(W, np.float32)
    N, K = W.shape
    wq = np.empty((N, K), np.int8)
    beta = np.empty(1, np.float32)
    _load().ugref_quant_weight_absmean(_ptr(W, ctypes.c_float), K, N, K,
                                       float(np.float32(eps)), _ptr(wq, ctypes.c_int8), K,
                                       _ptr(beta, ctypes.c_float))
    return wq, beta[0]


def packed_pitch(K, align=16):
    """Smallest row pitch in bytes >= ceil(K/5) that is a multiple of align."""
    g = -(-K // 5)
    return -(-g // align) * align


def pack_trits(wq, ldp=None):
    """Five trits per byte (README "A whole ternary GPT", pack.py).
    Returns (packed uint8 [N, ldp], number of entries outside {-1,0,1})."""
    wq = _c2d(wq, np.int8)
    N, K = wq.shape
    if ldp is None:
        ldp = packed_pitch(K)
    packed = np.empty((N, ldp), np.uint8)
    bad = _load().ugref_pack_trits(_ptr(wq, ctypes.c_int8), K, N, K,
                                   _ptr(packed, ctypes.c_uint8), ldp)
    return packed, int(bad)


def unpack_trits(packed, K):
    """Inverse of pack_trits.  Returns (W_q int8 [N,K], number of codes > 242)."""
    packed = _c2d(packed, np.uint8)
    N, ldp = packed.shape
    wq = np.empty((N, K), np.int8)
    bad = _load().ugref_unpack_trits(_ptr(packed, ctypes.c_uint8), ldp, N, K,
                                     _ptr(wq, ctypes.c_int8), K)
    return wq, int(bad)


def matmul_i32(xq, wq):
    """acc = x_q W_q^T in exact integers ("autograd on a byte-graph")."""
    xq = _c2d(xq, np.int8)
    wq = _c2d(wq, np.int8)
    M, K = xq.shape
    N, K2 = wq.shape
    if K != K2:
        raise ValueError("K mismatch")
    acc = np.empty((M, N), np.int32)
    _load().ugref_matmul_i32(_ptr(xq, ctypes.c_int8), K, _ptr(wq, ctypes.c_int8), K,
                             M, N, K, _ptr(acc, ctypes.c_int32), N)
    return acc


def matmul_i32_pairs(xq, wq, mi, ni):
    """acc[mi[p], ni[p]] for a list of index pairs."""
    xq = _c2d(xq, np.int8)
    wq = _c2d(wq, np.int8)
    K = xq.shape[1]
    if wq.shape[1] != K:
        raise ValueError("K mismatch")
    mi = np.ascontiguousarray(np.asarray(mi, np.int64))
    ni = np.ascontiguousarray(np.asarray(ni, np.int64))
    if mi.shape != ni.shape:
        raise ValueError("index shape mismatch")
    out = np.empty(mi.size, np.int32)
    _load().ugref_matmul_i32_pairs(_ptr(xq, ctypes.c_int8), K, _ptr(wq, ctypes.c_int8), K,
                                   K, _ptr(mi, ctypes.c_int64), _ptr(ni, ctypes.c_int64),
                                   mi.size, _ptr(out, ctypes.c_int32))
    return out


def epilogue(acc, s, beta, bias=None):
    """y = fl((float)acc * fl(s * beta)) -- the rescale of
    y = (x_q W_q^T)(s beta) + b ("autograd on a byte-graph"); with a bias
    (fp32 [N]) each output then adds b[n] in one more rounding."""
    acc = _c2d(acc, np.int32)
    M, N = acc.shape
    s = np.ascontiguousarray(np.asarray(s, np.float32).reshape(M))
    bp = None
    if bias is not None:
        bias = np.ascontiguousarray(np.asarray(bias, np.float32).reshape(N))
        bp = _ptr(bias, ctypes.c_float)
    y = np.empty((M, N), np.float32)
    _load().ugref_epilogue(_ptr(acc, ctypes.c_int32), N, _ptr(s, ctypes.c_float),
                           float(np.float32(beta)), bp, M, N, _ptr(y, ctypes.c_float), N)
    return y


def bitlinear(x, W, eps=1e-5, bias=None):
    """The whole forward: quantize x per row and W by absmean, integer
    matmul, rescale (plus the bias, if given).  Returns dict of every
    intermediate."""
    xq, s = quant_act(x, eps)
    wq, beta = quant_weight_absmean(W, eps)
    acc = matmul_i32(xq, wq)
    y = epilogue(acc, s, beta, bias)
    return dict(xq=xq, s=s, wq=wq, beta=beta, acc=acc, y=y)


def attention(q, kc, vc, pos0, H):
    """Causal attention over a key/value cache ("attention, as graph ops":
    softmax(Q K^T / sqrt(d_h) + mask) V per head; README "A whole ternary
    GPT": cached decoding).  q fp32 [M, H*dh] (row m at position pos0 + m),
    kc, vc fp32 [>= pos0 + M, H*dh].  Double precision inside, fp32 out
    [M, H*dh]."""
    q = _c2d(q, np.float32)
    kc = _c2d(kc, np.float32)
    vc = _c2d(vc, np.float32)
    M, HD = q.shape
    if HD % H or kc.shape[1] != HD or vc.shape[1] != HD:
        raise ValueError("head layout mismatch")
    if kc.shape[0] < pos0 + M or vc.shape[0] < pos0 + M:
        raise ValueError("cache shorter than the last query position")
    out = np.empty((M, HD), np.float32)
    _load().ugref_attention(_ptr(q, ctypes.c_float), HD, _ptr(kc, ctypes.c_float), HD,
                            _ptr(vc, ctypes.c_float), HD, M, pos0, H, HD // H,
                            _ptr(out, ctypes.c_float), HD)
    return out


def sample_topk(logits, k, temp, u):
    """Top-k sampling ("a 1-bit llm, from scratch", "the interesting bit";
    README "A whole ternary GPT": temperature and top_k): rank by logit,
    larger first, equal values by lower index; weights exp((l_r - l_1)/T)
    over ranks 1..k; token = the first rank whose cumulative weight exceeds
    u times the total.  logits fp32 [B, V], u [B] in [0, 1).  Returns
    (tokens int32 [B], ranked indices int32 [B, k], their logits fp32
    [B, k], normalized cumulative weights float64 [B, k])."""
    logits = _c2d(logits, np.float32)
    B, V = logits.shape
    if not 1 <= k <= V:
        raise ValueError("k out of range")
    u = np.ascontiguousarray(np.asarray(u, np.float32).reshape(B))
    tok = np.empty(B, np.int32)
    idx = np.empty((B, k), np.int32)
    val = np.empty((B, k), np.float32)
    cdf = np.empty((B, k), np.float64)
    _load().ugref_sample_topk(_ptr(logits, ctypes.c_float), V, B, V, k, float(np.float32(temp)),
                              _ptr(u, ctypes.c_float), _ptr(tok, ctypes.c_int32),
                              _ptr(idx, ctypes.c_int32), _ptr(val, ctypes.c_float),
                              cdf.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    return tok, idx, val, cdf


def bitlinear_backward(g, x, W, want=("dx", "dW", "db")):
    """The straight-through backward of the BitLinear layer ("autograd on a
    byte-graph"): with g = dL/dy [M, N], x [M, K] and the fp32 masters
    W [N, K]: dx = g W, dW = g^T x, db = sum over rows of g.  Double
    precision sums, fp32 results.  Returns a dict of the outputs asked for."""
    g = _c2d(g, np.float32)
    x = _c2d(x, np.float32)
    W = _c2d(W, np.float32)
    M, N = g.shape
    K = x.shape[1]
    if x.shape[0] != M or W.shape != (N, K):
        raise ValueError("shape mismatch")
    out = {}
    dx = np.empty((M, K), np.float32) if "dx" in want else None
    dW = np.empty((N, K), np.float32) if "dW" in want else None
    db = np.empty(N, np.float32) if "db" in want else None
    p = lambda a: _ptr(a, ctypes.c_float) if a is not None else None  # noqa: E731
    _load().ugref_bitlinear_backward(p(g), N, p(x), K, p(W), K, M, N, K, p(dx), K, p(dW), K,
                                     p(db))
    for name, a in (("dx", dx), ("dW", dW), ("db", db)):
        if a is not None:
            out[name] = a
    return out


def num_threads():
    """Threads OpenMP will use for the oracle in this process."""
    v = os.environ.get("OMP_NUM_THREADS")
    if v:
        try:
            return int(v)
        except ValueError:
            pass
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1
