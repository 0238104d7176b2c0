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
    assert ug.ug_version() == 10100
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
    # packed weights are decoded after the 2 KB of counter words
    assert L.ug_bitlinear_gemm_workspace_size(16, 100, 37, ug.UG_W_PACK5) == 2048 + 100 * 48
    # problems of at least 512 x 512 add the K-split area in front: 2 KB of
    # tile counters and 256 partial tiles of 256 KB
    split = 2048 + 256 * 256 * 256 * 4
    for M, N, K in ((512, 512, 64), (2048, 2560, 6912), (600, 700, 197), (4096, 6912, 2560)):
        assert L.ug_bitlinear_gemm_workspace_size(M, N, K, ug.UG_W_I8) == split
        dec = N * (-(-K // 16) * 16)
        assert L.ug_bitlinear_gemm_workspace_size(M, N, K, ug.UG_W_PACK5) == split + dec
    assert L.ug_bitlinear_gemm_workspace_size(511, 4096, 64, ug.UG_W_I8) == 0
    assert L.ug_bitlinear_gemm_workspace_size(4096, 511, 64, ug.UG_W_PACK5) == 2048 + 511 * 64


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


def _share(I, J, P, B=1024):
    """Host mirror of the backward products' plan: tiles beyond the last
    whole round of B blocks (all, if fewer than B) are cut along the
    contraction into S = ceil(B / rem) pieces of 16-deep steps, at most 16
    and each piece at least 8 steps."""
    T = -(-I // 128) * -(-J // 128)
    ns = -(-P // 16)
    rem = T % B
    S = max(1, min(-(-B // rem), ns // 8, 16)) if rem else 1
    npb = -(-(rem * S) // 8) * 8
    return T, ns, rem, S, npb


def test_backward_pieces_cover_each_tile_once():
    """Block b < dp computes tile (b mod 8) dp / 8 + b // 8 whole; block
    dp + b' computes piece v = (b' mod 8) npb / 8 + b' // 8 (if v < rem S):
    steps [k ns / S, (k+1) ns / S) of tile dp + v mod rem, k = v // rem,
    into partial slot v.  Every step of every tile is computed once, the
    slots are distinct, each XCD (block mod 8) gets a contiguous run of
    tiles and of pieces, and the pieces fill about a round."""
    for I, J, P in ((6912, 2560, 2048), (2048, 2560, 6912), (2560, 3840, 48), (48, 3840, 2560),
                    (4096, 4096, 16), (4224, 4096, 96), (96, 4096, 4224), (128, 128, 300),
                    (8192, 4096, 100), (8320, 4096, 40), (16384, 2048, 64), (300, 64, 128),
                    (64, 128, 300), (1, 1, 1), (200, 131, 2100), (128, 128, 65536),
                    (6912, 2048, 2048)):
        T, ns, rem, S, npb = _share(I, J, P)
        dp = T - rem
        assert dp % 1024 == 0 and npb % 8 == 0
        assert rem * S < 2 * 1024 and (rem * S >= 1024 or S == 16 or S == max(1, ns // 8))
        done = set()
        slots = set()
        per_xcd = {x: [] for x in range(8)}
        for b in range(dp + npb):
            if b < dp:
                t = (b % 8) * (dp // 8) + b // 8
                steps = range(ns)
            else:
                v = (b % 8) * (npb // 8) + (b - dp) // 8
                if v >= rem * S:
                    continue
                assert v not in slots
                slots.add(v)
                t, k = dp + v % rem, v // rem
                steps = range(k * ns // S, (k + 1) * ns // S)
                assert len(steps) >= min(8, ns)
            per_xcd[b % 8].append(t)
            for st in steps:
                assert (t, st) not in done
                done.add((t, st))
        assert len(done) == T * ns
        for x, ts in per_xcd.items():     # whole tiles: one contiguous, increasing run
            whole = [t for t in ts if t < dp]
            assert whole == list(range(whole[0], whole[0] + len(whole))) if whole else True


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


def test_absmean_pack5_rejects(ug):
    L = ug.lib()
    need = L.ug_quant_weight_absmean_workspace_size(512, 128)
    E = ug.UG_ERR_INVALID_ARG
    f = L.ug_quant_weight_absmean_pack5
    assert f(NULL, 128, 512, 128, 1e-5, A2, 32, A3, A4, need, S) == E
    assert f(A, 128, 512, 128, 1e-5, A2, 16, A3, A4, need, S) == E      # ldp < ceil(K/5)
    assert f(A, 128, 512, 128, 1e-5, A2, 40, A3, A4, need, S) == E      # ldp % 16
    assert f(A, 126, 512, 128, 1e-5, A2, 32, A3, A4, need, S) == E      # ldw < K
    assert f(A, 128, 512, 128, 0.0, A2, 32, A3, A4, need, S) == E
    W = ug.UG_ERR_WORKSPACE
    assert f(A, 128, 512, 128, 1e-5, A2, 32, A3, NULL, need, S) == W
    assert f(A, 128, 512, 128, 1e-5, A2, 32, A3, A4, need - 4, S) == W


def test_absmean_static_rejects(ug):
    """The allocation-free absmean: the same argument checks, and tensors
    beyond its static scratch (16384 chunks of 8192 elements) are refused
    with UG_ERR_WORKSPACE before anything is looked up or launched."""
    L = ug.lib()
    E = ug.UG_ERR_INVALID_ARG
    assert L.ug_quant_weight_absmean_static(NULL, 128, 512, 128, 1e-5, A2, 128, A3, S) == E
    assert L.ug_quant_weight_absmean_static(A, 128, 512, 128, 0.0, A2, 128, A3, S) == E
    assert L.ug_quant_weight_absmean_static(A, 128, 512, 128, 1e-5, A2, 120, A3, S) == E
    K = 8192
    N = 16384 + 1  # one chunk more than the array holds
    assert (L.ug_quant_weight_absmean_static(A, K, N, K, 1e-5, A2, K, A3, S)
            == ug.UG_ERR_WORKSPACE)
    n_bad = 2 ** 24 + 1
    assert (L.ug_quant_weight_absmean_static(A, n_bad + 3, 1, n_bad, 1e-5, A2, n_bad + 15, A3,
                                             S) == ug.UG_ERR_UNSUPPORTED)


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
    a = dict(xq=A, ldx=128, s=A2, w=A3, wfmt=0, ldw=128, beta=A4, bias=NULL, M=4, N=64, K=128,
             acc=NULL, ldacc=0, y=ctypes.c_void_p(0x500000), ldy=64, st=S)
    a.update(kw)
    return L.ug_bitlinear_gemv(a["xq"], a["ldx"], a["s"], a["w"], a["wfmt"], a["ldw"], a["beta"],
                               a["bias"], a["M"], a["N"], a["K"], a["acc"], a["ldacc"], a["y"],
                               a["ldy"], a["st"])


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
    assert _gemv(L, bias=ctypes.c_void_p(0x600008)) == E   # bias needs 16-byte alignment


def test_gemm_rejects(ug):
    L = ug.lib()
    E = ug.UG_ERR_INVALID_ARG

    def call(ws=NULL, ws_bytes=0, wfmt=0, ldw=128, y=ctypes.c_void_p(0x500000)):
        return L.ug_bitlinear_gemm(A, 128, A2, A3, wfmt, ldw, A4, NULL, 300, 64, 128, NULL, 0, y,
                                   64, ws, ws_bytes, S)

    assert call(y=NULL) == E
    assert call(wfmt=1, ldw=32) == ug.UG_ERR_WORKSPACE
    assert call(wfmt=1, ldw=32, ws=ctypes.c_void_p(0x700000), ws_bytes=64 * 128 - 1) == \
        ug.UG_ERR_WORKSPACE
    # the decoded weights need the counter bytes in front of them too
    assert call(wfmt=1, ldw=32, ws=ctypes.c_void_p(0x700000), ws_bytes=2048 + 64 * 128 - 1) == \
        ug.UG_ERR_WORKSPACE


def test_gemm_tiled_rejects(ug):
    L = ug.lib()
    E = ug.UG_ERR_INVALID_ARG

    def call(tile, splits):
        return L.ug_bitlinear_gemm_tiled(A, 128, A2, A3, 0, 128, A4, NULL, 300, 64, 128, NULL, 0,
                                         NULL, 64, NULL, 0, tile, splits, S)

    assert call(2, -1) == E
    assert call(-2, -1) == E
    assert call(0, 0) == E
    assert call(0, -3) == E
    assert call(0, 1) == E   # still validates the matmul arguments (no output)


def test_grouped_plan_rejects_fused_with_chunked(ug):
    """A group that needs the chunked kernel (x_q rows too long for the
    staging area) cannot also quantize fp32 activations in the launch: the
    plan is refused before anything is copied to the device."""
    L = ug.lib()
    fused = ug.GemvProblem(x=0x100000, ldx=2560, eps=1e-5, xq=0, ldxq=0, s=0, w=0x200000,
                           wfmt=ug.UG_W_PACK5, ldw=512, beta=0x300000, M=16, N=6912, K=2560,
                           acc=0, ldacc=0, y=0x400000, ldy=6912)
    given = ug.GemvProblem(x=0, ldx=0, eps=0.0, xq=0x500000, ldxq=6912, s=0x600000,
                           w=0x700000, wfmt=ug.UG_W_PACK5, ldw=1392, beta=0x800000, M=16,
                           N=2560, K=6912, acc=0, ldacc=0, y=0x900000, ldy=2560)
    arr = (ug.GemvProblem * 2)(fused, given)
    info = ug.GemvPlanInfo()
    size = L.ug_gemv_plan_size(2)
    st = L.ug_gemv_plan_init(ctypes.cast(arr, ctypes.c_void_p), 2, ctypes.c_void_p(0xA00000),
                             size, ctypes.byref(info))
    assert st == ug.UG_ERR_UNSUPPORTED
    # each problem on its own passes validation and planning; without a
    # device the plan copy then fails (with one, the fake address would be
    # handed to a real copy: not done)
    import torch
    if torch.cuda.device_count() > 0:
        return
    for p in (fused, given):
        one = (ug.GemvProblem * 1)(p)
        st = L.ug_gemv_plan_init(ctypes.cast(one, ctypes.c_void_p), 1, ctypes.c_void_p(0xA00000),
                                 L.ug_gemv_plan_size(1), ctypes.byref(info))
        assert st == ug.UG_ERR_HIP


def test_grouped_launch_rejects_bad_variants(ug):
    """ug_bitlinear_gemv_grouped checks the plan's variant before launching:
    the spread staging (bit 13) goes only with the plain stream split of
    five-trit weights and one 16-row block; no other combination is a kernel."""
    L = ug.lib()
    plan = ctypes.create_string_buffer(4096 + 16)
    addr = (ctypes.addressof(plan) + 15) & ~15
    fmt5 = 16 * ug.UG_W_PACK5
    for variant in (8192 + 256 + fmt5 + 1,           # with the fine split
                    8192 + 2048 + fmt5 + 1,          # with the chunked split
                    8192 + 16 * ug.UG_W_I8 + 1,      # one trit per byte
                    8192 + fmt5 + 2, 8192 + fmt5 + 4,  # more than 16 rows
                    16384 + fmt5 + 1):               # no such bit
        info = ug.GemvPlanInfo(count=1, total_items=1, variant=variant, grid=1)
        st = L.ug_bitlinear_gemv_grouped(ctypes.c_void_p(addr), ctypes.byref(info), None)
        assert st == ug.UG_ERR_INVALID_ARG, hex(variant)


def test_attention_rejects_and_sizes(ug):
    L = ug.lib()
    E = ug.UG_ERR_INVALID_ARG
    # workspace: 4 * M * H * ceil((pos0 + M) / 64) * (dh + 4)
    assert L.ug_attention_workspace_size(1, 4095, 20, 128) == 4 * 1 * 20 * 64 * 132
    assert L.ug_attention_workspace_size(300, 0, 3, 64) == 4 * 300 * 3 * 5 * 68
    assert L.ug_attention_workspace_size(1, 0, 1, 48) == 0        # d_h not supported
    need = L.ug_attention_workspace_size(1, 99, 2, 64)

    def call(q=A, ldq=128, M=1, pos0=99, H=2, dh=64, ws=A4, ws_bytes=need, ldk=128):
        return L.ug_attention_cached(q, ldq, A2, ldk, A3, 128, M, pos0, H, dh,
                                     ctypes.c_void_p(0x500000), 128, ws, ws_bytes, S)

    assert call(q=NULL) == E
    assert call(q=MIS) == E
    assert call(dh=48) == E
    assert call(H=0) == E
    assert call(M=0) == E
    assert call(pos0=-1) == E
    assert call(ldq=100) == E            # pitch < H * dh
    assert call(ldk=130) == E            # pitch % 4
    assert call(ws=NULL) == ug.UG_ERR_WORKSPACE
    assert call(ws_bytes=need - 4) == ug.UG_ERR_WORKSPACE
    assert call(pos0=2 ** 24) == ug.UG_ERR_UNSUPPORTED


def test_sample_topk_rejects(ug):
    L = ug.lib()
    E = ug.UG_ERR_INVALID_ARG

    def call(logits=A, ld=4096, B=2, V=4096, k=100, T=1.0, u=A2, tok=A3, idx=NULL, ldi=0):
        return L.ug_sample_topk(logits, ld, B, V, k, T, u, tok, idx, ldi, NULL, 0, NULL, 0, S)

    assert call(logits=MIS) == E
    assert call(tok=NULL) == E
    assert call(k=0) == E
    assert call(k=257, V=4096) == E          # above UG_SAMPLE_MAX_K
    assert call(k=10, V=5, ld=8) == E        # k > V
    assert call(ld=4095) == E                # ld < V
    assert call(ld=4098) == E                # ld % 4
    assert call(T=0.0) == E
    assert call(T=float("inf")) == E
    assert call(idx=A4, ldi=50) == E         # output pitch < k
    assert call(u=ctypes.c_void_p(0x200002)) == E


def test_backward_rejects(ug):
    L = ug.lib()
    E = ug.UG_ERR_INVALID_ARG
    # (no device here: the library assumes 256 CUs, 1024 resident blocks;
    # partial tiles of 64 KB)
    need = L.ug_bitlinear_backward_workspace_size(300, 64, 128)
    # dx: 3 tiles 4 steps deep, not cut; dW: one tile 19 steps deep, cut in
    # 2 pieces (at least 8 steps each)
    assert need == 2 * 65536
    # db's chunk sums alone: dx one tile of 2 steps, dW 3 tiles of 1 step
    assert L.ug_bitlinear_backward_workspace_size(20, 32, 300) == 4 * 1 * 32
    # dx = g W at 2048 x 2560: 320 tiles of 432 steps in 4 pieces each (dW:
    # 1024 whole tiles and 56 in 16 pieces of 8 steps)
    assert L.ug_bitlinear_backward_workspace_size(2048, 6912, 2560) == 1280 * 65536

    def call(g=A, ldg=64, M=300, N=64, K=128, dx=ctypes.c_void_p(0x500000), dW=NULL, db=NULL,
             ws=NULL, ws_bytes=0, ldw=128):
        return L.ug_bitlinear_backward(g, ldg, A2, 128, A3, ldw, M, N, K, dx, 128, dW, 128, db,
                                       ws, ws_bytes, S)

    assert call(g=NULL) == E
    assert call(dx=NULL) == E                       # nothing to compute
    assert call(ldg=62) == E
    assert call(ldw=100) == E                       # W pitch < K (dx needs W)
    assert call(dx=MIS) == E
    assert call(db=ctypes.c_void_p(0x600000)) == ug.UG_ERR_WORKSPACE
    assert call(db=ctypes.c_void_p(0x600000), ws=A4, ws_bytes=need - 4) == ug.UG_ERR_WORKSPACE
    assert call(ws=NULL) == ug.UG_ERR_WORKSPACE
    assert call(M=2 ** 23 + 1) == ug.UG_ERR_UNSUPPORTED


def test_hbm_read_probe_rejects(ug):
    L = ug.lib()
    E, S, NULL = ug.UG_ERR_INVALID_ARG, None, None
    A, B = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x200000)
    assert L.ug_hbm_read_probe(NULL, 1024, 8, 1, B, S) == E                     # no buffer
    assert L.ug_hbm_read_probe(ctypes.c_void_p(0x100008), 1024, 8, 1, B, S) == E  # misaligned
    assert L.ug_hbm_read_probe(A, 0, 8, 1, B, S) == E                           # no bytes
    assert L.ug_hbm_read_probe(A, 1000, 8, 1, B, S) == E                        # not 16-byte words
    assert L.ug_hbm_read_probe(A, 1024, 0, 1, B, S) == E                        # no blocks
    assert L.ug_hbm_read_probe(A, 1024, 65536, 1, B, S) == E
    assert L.ug_hbm_read_probe(A, 1024, 8, 2, B, S) == E                        # no such walk
    assert L.ug_hbm_read_probe(A, 1024, 8, -1, B, S) == E
    assert L.ug_hbm_read_probe(A, 1024, 8, 1, NULL, S) == E                     # no sink
    assert L.ug_hbm_read_probe(A, 1024, 8, 1, ctypes.c_void_p(0x200002), S) == E


def test_mfma_rate_probe_rejects(ug):
    L = ug.lib()
    E = ug.UG_ERR_INVALID_ARG
    assert L.ug_mfma_rate_probe(2, 256, 10, A, S) == E     # no such kind
    assert L.ug_mfma_rate_probe(-1, 256, 10, A, S) == E
    assert L.ug_mfma_rate_probe(0, 0, 10, A, S) == E       # no blocks
    assert L.ug_mfma_rate_probe(1, 256, 0, A, S) == E      # no iterations
    assert L.ug_mfma_rate_probe(0, 256, 10, NULL, S) == E
    assert L.ug_mfma_rate_probe(0, 256, 10, ctypes.c_void_p(0x200002), S) == E
