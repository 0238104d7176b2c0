"""The C ABI without a GPU: libug.so loads, exports every symbol include/ug.h
declares, the binding covers the same names, the size queries follow their
documented formulas, and invalid arguments are rejected with the documented
status before anything is launched (no compute call is made here: every
call below fails validation first)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ug.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ug_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def ug():
    from bitlinear_matmul_amd import build, ug as binding
    if not os.path.exists(binding.LIB_PATH):
        build.build()
    try:
        binding.lib()
    except OSError as e:  # HIP runtime library not present
        pytest.skip("cannot load libug.so: %s" % e)
    return binding


def test_header_declares_the_entry_points():
    names = _declared()
    for want in ("ug_quant_act", "ug_rmsnorm_quant_act", "ug_quant_weight_absmean",
                 "ug_quant_weight_absmean_workspace_size", "ug_pack_trits", "ug_unpack_trits",
                 "ug_bitlinear_gemv", "ug_bitlinear_gemm", "ug_bitlinear_gemm_workspace_size",
                 "ug_status_string", "ug_last_hip_error", "ug_version"):
        assert want in names


def test_every_declared_symbol_is_exported(ug):
    h = ctypes.CDLL(ug.LIB_PATH)
    for name in _declared():
        assert hasattr(h, name), name
    assert set(_declared()) == set(ug.SIGNATURES)


def test_version_and_status_strings(ug):
    assert ug.ug_version() == 10000
    for st in range(5):
        assert ug.status_string(st).startswith(["UG_OK", "UG_ERR_INVALID_ARG",
                                                "UG_ERR_UNSUPPORTED", "UG_ERR_WORKSPACE",
                                                "UG_ERR_HIP"][st])
    assert ug.status_string(99) == "unknown ug_status"


def test_workspace_formulas(ug):
    L = ug.lib()
    for N, K in ((512, 128), (6912, 2560), (1, 1), (3, 8193)):
        chunks = -(-(N * K) // 8192)
        assert L.ug_quant_weight_absmean_workspace_size(N, K) == 4 * (-(-chunks // 256) * 256)
    assert L.ug_quant_weight_absmean_workspace_size(0, 5) == 0
    assert L.ug_bitlinear_gemm_workspace_size(16, 100, 37, ug.UG_W_I8) == 0
    assert L.ug_bitlinear_gemm_workspace_size(16, 100, 37, ug.UG_W_PACK5) == 100 * 48
    # problems of at least 512 x 512 add the K-split area in front: 2 KB of
    # tile counters and 256 partial tiles of 256 KB
    split = 2048 + 256 * 256 * 256 * 4
    for M, N, K in ((512, 512, 64), (2048, 2560, 6912), (600, 700, 197), (4096, 6912, 2560)):
        assert L.ug_bitlinear_gemm_workspace_size(M, N, K, ug.UG_W_I8) == split
        dec = N * (-(-K // 16) * 16)
        assert L.ug_bitlinear_gemm_workspace_size(M, N, K, ug.UG_W_PACK5) == split + dec
    assert L.ug_bitlinear_gemm_workspace_size(511, 4096, 64, ug.UG_W_I8) == 0
    assert L.ug_bitlinear_gemm_workspace_size(4096, 511, 64, ug.UG_W_PACK5) == 511 * 64


def test_k_split_ranges_cover_each_tile_once():
    """Host mirror of the K split: block v computes steps
    [s nk / S, (s+1) nk / S) of tile v % T with s = v // T; for every S <= nk
    the ranges of a tile are non-empty and cover [0, nk) once, in order, and
    the partial slots v = s T + t are distinct."""
    for T, nk in ((80, 108), (30, 16), (9, 4), (1, 1), (54, 40)):
        for S in range(1, min(nk, 256 // T) + 1):
            slots = set()
            for t in range(T):
                prev = 0
                for sp in range(S):
                    v = sp * T + t
                    assert v % T == t and v // T == sp
                    ks, ke = sp * nk // S, (sp + 1) * nk // S
                    assert ks == prev and ke > ks
                    prev = ke
                    slots.add(v)
                assert prev == nk
            assert slots == set(range(T * S))


# Fake device addresses: aligned and misaligned.  They are never
# dereferenced because every call below fails validation.
A = ctypes.c_void_p(0x100000)
A2 = ctypes.c_void_p(0x200000)
A3 = ctypes.c_void_p(0x300000)
A4 = ctypes.c_void_p(0x400000)
MIS = ctypes.c_void_p(0x100004)
NULL = ctypes.c_void_p(0)
S = ctypes.c_void_p(0)


def test_quant_act_rejects(ug):
    L = ug.lib()
    E = ug.UG_ERR_INVALID_ARG
    assert L.ug_quant_act(NULL, 128, 4, 128, 1e-5, A2, 128, A3, S) == E
    assert L.ug_quant_act(MIS, 128, 4, 128, 1e-5, A2, 128, A3, S) == E
    assert L.ug_quant_act(A, 128, 0, 128, 1e-5, A2, 128, A3, S) == E
    assert L.ug_quant_act(A, 128, 4, 0, 1e-5, A2, 128, A3, S) == E
    assert L.ug_quant_act(A, 127, 4, 128, 1e-5, A2, 128, A3, S) == E   # ldx < K
    assert L.ug_quant_act(A, 130, 4, 128, 1e-5, A2, 128, A3, S) == E   # ldx % 4
    assert L.ug_quant_act(A, 128, 4, 128, 1e-5, A2, 136, A3, S) == E   # ldq % 16
    assert L.ug_quant_act(A, 128, 4, 128, 0.0, A2, 128, A3, S) == E    # eps <= 0
    assert L.ug_quant_act(A, 128, 4, 128, float("nan"), A2, 128, A3, S) == E
    assert L.ug_quant_act(A, 128, 4, 128, -1e-5, A2, 128, A3, S) == E


def test_rmsnorm_rejects(ug):
    L = ug.lib()
    E = ug.UG_ERR_INVALID_ARG
    assert L.ug_rmsnorm_quant_act(A, 128, MIS, 4, 128, 1e-5, 1e-5, A2, 128, A3, S) == E
    assert L.ug_rmsnorm_quant_act(A, 128, NULL, 4, 128, 0.0, 1e-5, A2, 128, A3, S) == E
    assert L.ug_rmsnorm_quant_act(A, 128, NULL, 4, 128, 1e-5, float("inf"), A2, 128, A3, S) == E
    assert (L.ug_rmsnorm_quant_act(A, 2 ** 24 + 4, NULL, 1, 2 ** 24 + 1, 1e-5, 1e-5, A2,
                                   2 ** 24 + 16, A3, S) == ug.UG_ERR_UNSUPPORTED)


def test_absmean_rejects(ug):
    L = ug.lib()
    need = L.ug_quant_weight_absmean_workspace_size(512, 128)
    E = ug.UG_ERR_INVALID_ARG
    assert L.ug_quant_weight_absmean(NULL, 128, 512, 128, 1e-5, A2, 128, A3, A4, need, S) == E
    assert L.ug_quant_weight_absmean(A, 128, 512, 128, 1e-5, A2, 120, A3, A4, need, S) == E
    assert L.ug_quant_weight_absmean(A, 128, 512, 128, 0.0, A2, 128, A3, A4, need, S) == E
    W = ug.UG_ERR_WORKSPACE
    assert L.ug_quant_weight_absmean(A, 128, 512, 128, 1e-5, A2, 128, A3, NULL, need, S) == W
    assert L.ug_quant_weight_absmean(A, 128, 512, 128, 1e-5, A2, 128, A3, A4, need - 4, S) == W
    assert L.ug_quant_weight_absmean(A, 128, 512, 128, 1e-5, A2, 128, A3, MIS, need, S) == W
    # n = N*K not exactly representable in fp32
    n_bad = (2 ** 24 + 1)
    assert (L.ug_quant_weight_absmean(A, n_bad + 3, 1, n_bad, 1e-5, A2, n_bad + 15, A3, A4,
                                      1 << 30, S) == ug.UG_ERR_UNSUPPORTED)


def test_pack_rejects(ug):
    L = ug.lib()
    E = ug.UG_ERR_INVALID_ARG
    assert L.ug_pack_trits(A, 128, 4, 128, A2, 16, NULL, S) == E      # ldp < ceil(K/5)
    assert L.ug_pack_trits(A, 128, 4, 128, A2, 40, NULL, S) == E      # ldp % 16
    assert L.ug_pack_trits(A, 128, 4, 128, A2, 32, ctypes.c_void_p(0x300002), S) == E
    assert L.ug_pack_trits(A, 100, 4, 128, A2, 32, NULL, S) == E      # ldq < K
    assert L.ug_unpack_trits(A2, 16, 4, 128, A, 128, NULL, S) == E
    assert L.ug_unpack_trits(A2, 32, 0, 128, A, 128, NULL, S) == E


def _gemv(L, **kw):
    a = dict(xq=A, ldx=128, s=A2, w=A3, wfmt=0, ldw=128, beta=A4, M=4, N=64, K=128,
             acc=NULL, ldacc=0, y=ctypes.c_void_p(0x500000), ldy=64, st=S)
    a.update(kw)
    return L.ug_bitlinear_gemv(a["xq"], a["ldx"], a["s"], a["w"], a["wfmt"], a["ldw"], a["beta"],
                               a["M"], a["N"], a["K"], a["acc"], a["ldacc"], a["y"], a["ldy"],
                               a["st"])


def test_gemv_rejects(ug):
    L = ug.lib()
    E = ug.UG_ERR_INVALID_ARG
    assert _gemv(L, y=NULL) == E                       # neither output
    assert _gemv(L, M=65) == E                         # GEMV row limit
    assert _gemv(L, M=0) == E
    assert _gemv(L, wfmt=2) == E                       # unknown format
    assert _gemv(L, ldx=120) == E
    assert _gemv(L, ldx=136) == E                      # pitch % 16
    assert _gemv(L, ldw=64) == E                       # I8 pitch < K
    assert _gemv(L, wfmt=1, ldw=16) == E               # PACK5 pitch < ceil(K/5)
    assert _gemv(L, ldy=62) == E
    assert _gemv(L, acc=ctypes.c_void_p(0x600000), ldacc=30) == E
    assert _gemv(L, s=ctypes.c_void_p(0x100002)) == E   # s needs 4-byte alignment
    assert _gemv(L, K=132105, ldx=132112, ldw=132112) == ug.UG_ERR_UNSUPPORTED


def test_gemm_rejects(ug):
    L = ug.lib()
    E = ug.UG_ERR_INVALID_ARG

    def call(ws=NULL, ws_bytes=0, wfmt=0, ldw=128, y=ctypes.c_void_p(0x500000)):
        return L.ug_bitlinear_gemm(A, 128, A2, A3, wfmt, ldw, A4, 300, 64, 128, NULL, 0, y, 64,
                                   ws, ws_bytes, S)

    assert call(y=NULL) == E
    assert call(wfmt=1, ldw=32) == ug.UG_ERR_WORKSPACE
    assert call(wfmt=1, ldw=32, ws=ctypes.c_void_p(0x700000), ws_bytes=64 * 128 - 1) == \
        ug.UG_ERR_WORKSPACE
