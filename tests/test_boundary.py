"""The C-ABI library on the host: it loads, exports every entry point the header declares, and its
host-side validation rejects bad arguments before anything is launched (no GPU needed: every call
here returns before the first HIP call)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moesq.h")
LIB = os.path.join(ROOT, "sparse_precision_grouped_amd", "libmoesq.so")

OK, EARG, EUNS, EWS, EPAT, EHIP = 0, -1, -2, -3, -4, -5


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moesq_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(LIB):
        pytest.fail("libmoesq.so is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(LIB)
    lib.moesq_status_str.restype = ctypes.c_char_p
    lib.moesq_workspace_bytes.restype = ctypes.c_size_t
    lib.moesq_workspace_bytes.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
    return lib


def test_header_declares_the_five_calls_and_setup():
    names = _declared()
    for n in ["moesq_quantize_act", "moesq_route_permute", "moesq_grouped_gemm", "moesq_expert_mlp",
              "moesq_unpermute_combine", "moesq_compress_weights", "moesq_unpack_weights",
              "moesq_workspace_bytes", "moesq_status_str", "moesq_version"]:
        assert n in names


def test_library_exports_every_declared_symbol(L):
    for n in _declared():
        assert hasattr(L, n), n


def test_status_strings(L):
    for code in (OK, EARG, EUNS, EWS, EPAT, EHIP):
        assert L.moesq_status_str(code)
    assert L.moesq_version() >= 100


def _p(v):
    return ctypes.c_void_p(v)


FAKE = 0x10000  # never dereferenced: every call below fails validation first


def test_route_validation(L):
    i64, i32, sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    f = L.moesq_route_permute
    f.argtypes = [ctypes.c_void_p] * 2 + [i64, i32, i32] + [ctypes.c_void_p] * 5 + [sz, ctypes.c_void_p]
    args = lambda T=4, k=2, E=8, ids=FAKE, cnt=FAKE: (None, _p(ids), T, k, E, _p(cnt), _p(FAKE), _p(FAKE),  # noqa
                                                      _p(FAKE), None, 0, None)
    assert f(*args(k=9)) == EARG          # k > E
    assert f(*args(k=0)) == EARG
    assert f(*args(E=0)) == EARG
    assert f(*args(ids=0)) == EARG        # null ids
    assert f(*args(cnt=0)) == EARG
    assert f(*args(E=513)) == EUNS        # beyond the routing limit
    # multi-block path needs a workspace
    assert L.moesq_workspace_bytes(1, 65536, 8, 384, 0, 0, 0) > 0
    assert f(*args(T=65536, k=8, E=384)) == EWS
    assert L.moesq_workspace_bytes(1, 16, 8, 128, 0, 0, 0) == 0   # one-workgroup path


def test_route_capacity_validation(L):
    i64, i32, sz, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p
    f = L.moesq_route_capacity
    f.argtypes = [vp, vp, i64, i32, i32, i32, vp, vp, vp, sz, vp]
    call = lambda T=16, k=2, E=8, C=4, ids=FAKE, ws=FAKE, wsb=1 << 20: f(  # noqa: E731
        None, _p(ids) if ids else None, T, k, E, C, _p(FAKE), _p(FAKE), _p(ws) if ws else None, wsb, None)
    assert call(C=0) == EARG
    assert call(k=9) == EARG
    assert call(ids=0) == EARG
    assert call(E=600) == EUNS
    assert call(ws=0) == EWS
    assert call(wsb=16) == EWS
    assert L.moesq_workspace_bytes(5, 16, 2, 8, 0, 0, 0) > 0


def test_quantize_validation(L):
    i64, i32 = ctypes.c_int64, ctypes.c_int32
    f = L.moesq_quantize_act
    vp = ctypes.c_void_p
    f.argtypes = [vp, vp, i32, i64, i32, i64, vp, i32, i64, vp, vp, i32, vp, vp, vp]
    base = dict(x=FAKE, dt=0, T=8, K=64, ld=64, g=None, k=1, rows=8, gamma=FAKE, off=None, E=0, q=FAKE, s=FAKE)

    def call(**kw):
        a = dict(base, **kw)
        return f(None, _p(a["x"]), a["dt"], a["T"], a["K"], a["ld"], _p(a["g"]) if a["g"] else None, a["k"],
                 a["rows"], _p(a["gamma"]) if a["gamma"] else None, _p(a["off"]) if a["off"] else None, a["E"],
                 _p(a["q"]), _p(a["s"]), None)
    assert call(K=48, ld=48) == EARG      # K % 32 != 0
    assert call(dt=7) == EARG             # dtype
    assert call(ld=32) == EARG            # ld_x < K
    assert call(gamma=0) == EARG
    assert call(rows=9) == EARG           # no scatter: rows must equal T
    assert call(g=FAKE, k=2, rows=15) == EARG    # scatter: rows must hold T*k copies
    assert call(g=FAKE, k=513, rows=8 * 513) == EUNS
    assert call(g=FAKE, k=0) == EARG
    assert call(x=FAKE + 4) == EUNS       # misaligned x
    assert call(E=3, rows=8) == EARG      # fixed-capacity rows (no offsets, E > 0) must split into E blocks


def test_route_quantize_validation(L):
    i64, i32, sz, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p
    f = L.moesq_route_quantize
    f.argtypes = [vp, vp, i64, i32, i32, vp, i32, i32, i64, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp, vp]
    base = dict(ids=FAKE, T=16, k=8, E=128, x=FAKE, dt=1, K=2048, ld=2048, gamma=FAKE, cnt=FAKE, ws=None, q=FAKE)

    def call(**kw):
        a = dict(base, **kw)
        p = lambda v: _p(v) if v else None  # noqa: E731
        return f(None, p(a["ids"]), a["T"], a["k"], a["E"], p(a["x"]), a["dt"], a["K"], a["ld"], p(a["gamma"]),
                 p(a["cnt"]), _p(FAKE), _p(FAKE), _p(FAKE), p(a["ws"]), 0, p(a["q"]), _p(FAKE), None, None)
    assert call(k=129) == EARG            # k > E
    assert call(ids=0) == EARG
    assert call(gamma=0) == EARG
    assert call(q=0) == EARG
    assert call(dt=7) == EARG
    assert call(K=48, ld=48) == EARG
    assert call(ld=1024) == EARG
    assert call(E=513) == EUNS
    assert call(x=FAKE + 4) == EUNS
    # beyond the single-launch path the routing workspace is required; within it, it is not
    assert call(T=65536) == EWS
    assert call(T=256, k=9, E=16) == EWS   # T*k > 2048


def test_route_quantize_dyn_validation(L):
    i64, i32, sz, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p
    f = L.moesq_route_quantize_dyn
    f.argtypes = [vp, vp, i64, i32, i32, vp, i32, i32, i64, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp, vp]
    base = dict(ids=FAKE, T=16, k=8, E=128, x=FAKE, dt=1, K=2048, ld=2048, g=FAKE, cnt=FAKE, ws=None, q=FAKE)

    def call(**kw):
        a = dict(base, **kw)
        p = lambda v: _p(v) if v else None  # noqa: E731
        return f(None, p(a["ids"]), a["T"], a["k"], a["E"], p(a["x"]), a["dt"], a["K"], a["ld"], p(a["g"]),
                 p(a["cnt"]), _p(FAKE), _p(FAKE), _p(FAKE), p(a["ws"]), 0, p(a["q"]), _p(FAKE), None, None)
    assert call(g=0) == EARG              # gamma_out is required
    assert call(g=FAKE + 2) == EUNS       # misaligned gamma_out
    assert call(k=129) == EARG
    assert call(ids=0) == EARG
    assert call(q=0) == EARG
    assert call(dt=7) == EARG
    assert call(K=48, ld=48) == EARG
    assert call(E=513) == EUNS
    assert call(T=65536) == EWS


def test_route_quantize_gemm_validation(L):
    class CW(ctypes.Structure):
        _fields_ = [("E", ctypes.c_int32), ("N", ctypes.c_int32), ("K", ctypes.c_int32),
                    ("packed", ctypes.c_void_p), ("mask", ctypes.c_void_p), ("scale", ctypes.c_void_p),
                    ("gscale", ctypes.c_void_p), ("kl", ctypes.c_void_p), ("gscale_split", ctypes.c_int32)]
    i64, i32, sz, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p
    f = L.moesq_route_quantize_gemm
    f.argtypes = [vp, vp, i64, i32, i32, vp, i32, i32, i64, vp, ctypes.POINTER(CW), vp, vp, vp, vp, vp, sz, vp, vp,
                  vp, vp, i32, vp]
    base = dict(ids=FAKE, T=16, k=8, E=128, x=FAKE, dt=1, K=2048, ld=2048, gamma=FAKE, cnt=FAKE, ws=None, q=FAKE,
                y=FAKE, ydt=1, W=(128, 1536, 2048))

    def call(**kw):
        a = dict(base, **kw)
        p = lambda v: _p(v) if v else None  # noqa: E731
        W = CW(*a["W"], FAKE, FAKE, FAKE, FAKE, FAKE, 0)
        return f(None, p(a["ids"]), a["T"], a["k"], a["E"], p(a["x"]), a["dt"], a["K"], a["ld"], p(a["gamma"]),
                 ctypes.byref(W), p(a["cnt"]), _p(FAKE), _p(FAKE), _p(FAKE), p(a["ws"]), 0, p(a["q"]), _p(FAKE), None,
                 p(a["y"]), a["ydt"], None)
    assert call(ydt=5) == EARG
    assert call(W=(64, 1536, 2048)) == EARG   # W->E != E
    assert call(W=(128, 1536, 1024)) == EARG  # W->K != K
    assert call(k=129) == EARG
    assert call(ids=0) == EARG
    assert call(gamma=0) == EARG
    assert call(q=0) == EARG
    assert call(y=0) == EARG
    assert call(cnt=0) == EARG
    assert call(dt=7) == EARG
    assert call(ld=1024) == EARG
    assert call(E=513, W=(513, 1536, 2048)) == EUNS
    assert call(x=FAKE + 4) == EUNS
    assert call(W=(128, 1500, 2048)) == EUNS  # N % 64 != 0
    # beyond the one-launch paths the routing workspace is required
    assert call(T=65536) == EWS


def test_gemm_and_mlp_validation(L):
    class CW(ctypes.Structure):
        _fields_ = [("E", ctypes.c_int32), ("N", ctypes.c_int32), ("K", ctypes.c_int32),
                    ("packed", ctypes.c_void_p), ("mask", ctypes.c_void_p), ("scale", ctypes.c_void_p),
                    ("gscale", ctypes.c_void_p), ("kl", ctypes.c_void_p), ("gscale_split", ctypes.c_int32)]
    vp = ctypes.c_void_p
    g = L.moesq_grouped_gemm
    g.argtypes = [vp, ctypes.POINTER(CW), vp, vp, vp, vp, vp, ctypes.c_int64, vp, ctypes.c_int32, ctypes.c_uint32]
    W = CW(4, 128, 256, FAKE, FAKE, FAKE, FAKE, FAKE)
    call = lambda W, y=FAKE, dt=0: g(None, ctypes.byref(W), _p(FAKE), _p(FAKE), None, _p(FAKE), _p(FAKE), 16, _p(y),  # noqa
                                     dt, 0)
    assert call(W, dt=3) == EARG
    assert call(W, y=0) == EARG
    assert call(CW(4, 128, 240, FAKE, FAKE, FAKE, FAKE, FAKE)) == EARG     # K % 32 != 0
    assert call(CW(4, 128, 96, FAKE, FAKE, FAKE, FAKE, FAKE)) == EUNS      # K % 256 != 0
    assert call(CW(4, 100, 256, FAKE, FAKE, FAKE, FAKE, FAKE)) == EUNS     # N % 64 != 0
    assert call(CW(4, 128, 256, 0, 0, 0, FAKE, 0)) == EARG            # no kernel layout
    assert call(CW(4, 128, 256, FAKE, FAKE, FAKE, FAKE, FAKE, 2)) == EARG  # gscale_split is 0 or 1
    assert call(CW(4, 64, 256, FAKE, FAKE, FAKE, FAKE, FAKE, 1)) == EUNS   # split scales need N % 128 == 0
    m = L.moesq_expert_mlp
    m.argtypes = [vp, ctypes.POINTER(CW), ctypes.POINTER(CW), vp, vp, vp, vp, vp, vp, ctypes.c_int64, vp,
                  ctypes.c_int32, vp, ctypes.c_size_t, ctypes.c_uint32]
    W13 = CW(4, 512, 256, FAKE, FAKE, FAKE, FAKE, FAKE)
    W2 = CW(4, 256, 256, FAKE, FAKE, FAKE, FAKE, FAKE)
    mc = lambda a, b, ws=FAKE, wsb=1 << 30, gh=FAKE, fl=0: m(  # noqa: E731
        None, ctypes.byref(a), ctypes.byref(b), _p(FAKE), _p(FAKE), None, _p(FAKE), _p(gh) if gh else None, _p(FAKE),
        16, _p(FAKE), 0, _p(ws) if ws else None, wsb, fl)
    assert mc(W13, CW(4, 256, 128, FAKE, FAKE, FAKE, FAKE, FAKE)) == EARG   # W2.K != I
    assert mc(W13, CW(3, 256, 256, FAKE, FAKE, FAKE, FAKE, FAKE)) == EARG   # expert count mismatch
    assert mc(W13, W2, ws=0) == EWS
    assert mc(W13, W2, wsb=10) == EWS
    assert mc(W13, W2, gh=0) == EARG                                         # gamma_h is required ...
    CAL, DUMP_G, DUMP_H = 32, 1, 16
    assert mc(W13, W2, gh=0, fl=CAL, wsb=10) == EWS                         # ... except in calibration
    assert mc(W13, W2, gh=0, fl=CAL, ws=0) == EWS
    assert mc(W13, W2, fl=CAL | DUMP_G) == EARG                              # no dumps in calibration
    assert mc(W13, W2, fl=CAL | DUMP_H) == EARG
    # the no-allocation form: batches beyond its static workspace, and the dump / calibration flags
    na = L.moesq_expert_mlp_noalloc
    na.argtypes = [vp, ctypes.POINTER(CW), ctypes.POINTER(CW), vp, vp, vp, vp, vp, vp, ctypes.c_int64, vp,
                   ctypes.c_int32, ctypes.c_uint32]
    K13, K2 = CW(384, 4096, 7168, FAKE, FAKE, FAKE, FAKE, FAKE), CW(384, 7168, 2048, FAKE, FAKE, FAKE, FAKE, FAKE)
    nc = lambda rows, fl=0: na(None, ctypes.byref(K13), ctypes.byref(K2), _p(FAKE), _p(FAKE), None,  # noqa: E731
                               _p(FAKE), _p(FAKE), _p(FAKE), rows, _p(FAKE), 0, fl)
    assert nc(6473) == EWS                      # I = 2048: 6472 rows fit in 32 MiB, 6473 do not
    assert nc(100000) == EWS
    for fl in (DUMP_G, DUMP_H, CAL):
        assert nc(16, fl) == EARG
    assert mc(CW(4, 256, 256, FAKE, FAKE, FAKE, FAKE, FAKE), CW(4, 256, 128, FAKE, FAKE, FAKE, FAKE, FAKE)) == EUNS  # I = 128


def test_prepack_validation_and_size(L):
    class CW(ctypes.Structure):
        _fields_ = [("E", ctypes.c_int32), ("N", ctypes.c_int32), ("K", ctypes.c_int32),
                    ("packed", ctypes.c_void_p), ("mask", ctypes.c_void_p), ("scale", ctypes.c_void_p),
                    ("gscale", ctypes.c_void_p), ("kl", ctypes.c_void_p), ("gscale_split", ctypes.c_int32)]
    vp = ctypes.c_void_p
    L.moesq_kernel_layout_bytes.restype = ctypes.c_size_t
    L.moesq_kernel_layout_bytes.argtypes = [ctypes.c_int32] * 3
    assert L.moesq_kernel_layout_bytes(384, 4096, 7168) == 384 * 4096 * 7168 * 11 // 32
    f = L.moesq_prepack_weights
    f.argtypes = [vp, ctypes.POINTER(CW), vp, ctypes.c_size_t]
    W = CW(2, 64, 512, FAKE, FAKE, FAKE, FAKE, 0)
    need = L.moesq_kernel_layout_bytes(2, 64, 512)
    assert f(None, ctypes.byref(W), None, need) == EARG
    assert f(None, ctypes.byref(W), _p(FAKE), need - 1) == EWS
    assert f(None, ctypes.byref(CW(2, 32, 480, FAKE, FAKE, FAKE, FAKE, 0)), _p(FAKE), 1 << 20) == EUNS
    assert f(None, ctypes.byref(CW(2, 24, 512, FAKE, FAKE, FAKE, FAKE, 0)), _p(FAKE), 1 << 20) == EUNS
    assert f(None, ctypes.byref(CW(2, 32, 512, FAKE, FAKE, FAKE, FAKE, 0)), _p(FAKE), 1 << 20) == EUNS  # N % 64


def test_combine_compress_unpack_validation(L):
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    c = L.moesq_unpermute_combine
    c.argtypes = [vp, vp, i32, vp, vp, i64, i32, i32, vp, i32]
    assert c(None, _p(FAKE), 0, _p(FAKE), _p(FAKE), 4, 0, 64, _p(FAKE), 0) == EARG   # k = 0
    assert c(None, _p(FAKE), 0, _p(FAKE), _p(FAKE), 4, 2, 60, _p(FAKE), 0) == EUNS   # H % 8
    assert c(None, _p(FAKE), 5, _p(FAKE), _p(FAKE), 4, 2, 64, _p(FAKE), 0) == EARG
    k = L.moesq_compress_weights
    k.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    assert k(None, _p(FAKE), 2, 8, 48, _p(FAKE), _p(FAKE), _p(FAKE), _p(FAKE), _p(FAKE), 64, None) == EARG
    assert k(None, _p(FAKE), 2, 8, 64, _p(FAKE), _p(FAKE), _p(FAKE), _p(FAKE), None, 64, None) == EWS
    assert k(None, _p(FAKE), 2, 8, 64, _p(FAKE), _p(FAKE), _p(FAKE), _p(FAKE), _p(FAKE), 4, None) == EWS


def test_workspace_sizes(L):
    ws = lambda kind, T=0, k=0, E=0, K=0, N=0, I=0: L.moesq_workspace_bytes(kind, T, k, E, K, N, I)  # noqa
    a = lambda x: (x + 255) // 256 * 256  # noqa
    rows, I = 1000, 2048
    base = a(rows * I // 2) + a(rows * I // 32) + a(rows * I * 2)
    assert ws(2, rows, 0, 384, 7168, 0, I) == base
    # the dumps: fp32 gate_up [rows][2I], then fp32 h [rows][I], each region 256-byte aligned
    assert ws(3, rows, 0, 384, 7168, 0, I) == base + a(rows * 2 * I * 4) + rows * I * 4
    assert ws(4, E=384) == 384 * 4
    # calibration: amax_h [E] f32, then gamma_h [E] f32 at the next 256-byte boundary
    assert ws(6, E=384) == a(384 * 4) + 384 * 4
    assert ws(6, E=0) == 0
