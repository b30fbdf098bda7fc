"""CPU oracle for the paired-4:8 sparse NVFP4 MoE expert path.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU
baseline leg may import this package; the product path (``sparse_precision_grouped_amd``)
never does, and the two share no code. ``liboracle.so`` is built from ``oracle.cpp`` with
``g++ -O2 -fopenmp -ffp-contract=off`` (no fast-math).

Every function cites the passage of the pages it follows (paper "Hardware-Native Joint
Sparse-Quantization for Trillion-Scale Mixture-of-Experts", arxiv 2610.02241; model card
"Kimi-K2.5-P48NVFP4-MoESQ"). Parity pins for every function live in
``tests/test_oracle_pins.py``; none is marked "parity unpinned".
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

OK, ERR_ARG, ERR_PATTERN = 0, -1, -4


def build(force=False):
    """Compile liboracle.so (the checker itself; building it is not using it)."""
    src = os.path.join(_HERE, "oracle.cpp")
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(src):
        subprocess.check_call(["g++", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
                               "-o", _LIB, src])
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        vp, i64, i32, f32, u8 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_uint8
        L.orc_e2m1_decode.argtypes = [u8]
        L.orc_e2m1_decode.restype = ctypes.c_double
        L.orc_e2m1_encode.argtypes = [f32]
        L.orc_e2m1_encode.restype = u8
        L.orc_e4m3_decode.argtypes = [u8]
        L.orc_e4m3_decode.restype = ctypes.c_double
        L.orc_e4m3_encode.argtypes = [f32]
        L.orc_e4m3_encode.restype = u8
        L.orc_global_scale.argtypes = [f32]
        L.orc_global_scale.restype = f32
        L.orc_amax.argtypes = [vp, i64]
        L.orc_amax.restype = f32
        L.orc_quantize_rows.argtypes = [vp, i64, i32, i64, vp, vp, vp, vp]
        L.orc_quantize_rows.restype = ctypes.c_int
        L.orc_prune_paired48.argtypes = [vp, i64, i32, vp]
        L.orc_pack_pair_bitmask.argtypes = [vp, i64, i32, vp, vp]
        L.orc_pack_pair_bitmask.restype = ctypes.c_int
        L.orc_unpack_pair_bitmask.argtypes = [vp, vp, i64, i32, vp]
        L.orc_unpack_pair_bitmask.restype = ctypes.c_int
        L.orc_compress_weights.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp]
        L.orc_compress_weights.restype = ctypes.c_int
        L.orc_route.argtypes = [vp, i64, i32, i32, vp, vp, vp, vp]
        L.orc_route.restype = ctypes.c_int
        L.orc_dispatch_quantize.argtypes = [vp, i64, i32, vp, i32, vp, i32, vp, vp, vp]
        L.orc_dispatch_quantize.restype = ctypes.c_int
        L.orc_dequant_codes.argtypes = [vp, vp, i64, i32, vp]
        L.orc_grouped_gemm.argtypes = [vp, vp, vp, vp, i32, i32, i32, vp, vp, vp, vp, vp, i64, vp]
        L.orc_grouped_gemm.restype = ctypes.c_int
        L.orc_swiglu.argtypes = [vp, i64, i32, vp]
        L.orc_combine.argtypes = [vp, i32, vp, vp, i64, i32, vp]
        _lib = L
    return _lib


def _p(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


class OracleError(RuntimeError):
    pass


def _check(rc, what):
    if rc != OK:
        raise OracleError("%s failed with status %d" % (what, rc))


# --- codecs (paper Appendix A, Figure 3; Section 3.4, Eq. 5) ---------------------------
def e2m1_decode(code):
    return lib().orc_e2m1_decode(int(code))


def e2m1_encode(r):
    return lib().orc_e2m1_encode(float(r))


def e4m3_decode(code):
    return lib().orc_e4m3_decode(int(code))


def e4m3_encode(u):
    return lib().orc_e4m3_encode(float(u))


def global_scale(amax):
    """Eq. 5 tensor scale gamma = 448 / (amax / 6), fp32; gamma = 1 for amax = 0."""
    return lib().orc_global_scale(float(amax))


def amax(x):
    x = _c(x, np.float32)
    return lib().orc_amax(_p(x), x.size)


def global_scale_of(x):
    return global_scale(amax(x))


# --- quantizer (Eq. 3 + Eq. 5) -----------------------------------------------------------
def quantize_rows(x, gamma, row_group=None):
    """x: [R, C] float32 -> codes [R, C/2] u8, scales [R, C/32] u8 (blocks along C)."""
    x = _c(x, np.float32)
    R, C = x.shape
    gamma = _c(np.atleast_1d(gamma), np.float32)
    rg = None if row_group is None else _c(row_group, np.int32)
    q = np.zeros((R, C // 2), np.uint8)
    s = np.zeros((R, C // 32), np.uint8)
    _check(lib().orc_quantize_rows(_p(x), R, C, C, _p(gamma), _p(rg), _p(q), _p(s)), "quantize_rows")
    return q, s


def dequant(q, s):
    """Exact dequantized values (double) of codes [R, C/2] with block scales [R, C/32]."""
    q = _c(q, np.uint8)
    s = _c(s, np.uint8)
    R, C = q.shape[0], q.shape[1] * 2
    out = np.empty((R, C), np.float64)
    lib().orc_dequant_codes(_p(q), _p(s), R, C, _p(out))
    return out


# --- sparsity and storage (Section 3.2, Appendix A; model card storage layout) ----------
def prune_paired48(w):
    w = _c(w, np.float32)
    out = np.empty_like(w)
    K = w.shape[-1]
    lib().orc_prune_paired48(_p(w), w.size // K, K, _p(out))
    return out


def pack(dense):
    """dense NVFP4 bytes [..., K/2] -> (packed [..., K/4], mask [..., K/16])."""
    dense = _c(dense, np.uint8)
    K = dense.shape[-1] * 2
    rows = dense.size // (K // 2)
    packed = np.zeros(dense.shape[:-1] + (K // 4,), np.uint8)
    mask = np.zeros(dense.shape[:-1] + (K // 16,), np.uint8)
    _check(lib().orc_pack_pair_bitmask(_p(dense), rows, K, _p(packed), _p(mask)), "pack")
    return packed, mask


def unpack(packed, mask):
    packed = _c(packed, np.uint8)
    mask = _c(mask, np.uint8)
    K = packed.shape[-1] * 4
    rows = packed.size // (K // 4)
    dense = np.zeros(packed.shape[:-1] + (K // 2,), np.uint8)
    _check(lib().orc_unpack_pair_bitmask(_p(packed), _p(mask), rows, K, _p(dense)), "unpack")
    return dense


def compress(w):
    """w: [E, N, K] float32 -> dict(packed, mask, scale, gscale)."""
    w = _c(w, np.float32)
    E, N, K = w.shape
    packed = np.zeros((E, N, K // 4), np.uint8)
    mask = np.zeros((E, N, K // 16), np.uint8)
    scale = np.zeros((E, N, K // 32), np.uint8)
    gscale = np.zeros(E, np.float32)
    _check(lib().orc_compress_weights(_p(w), E, N, K, _p(packed), _p(mask), _p(scale), _p(gscale)), "compress")
    return dict(packed=packed, mask=mask, scale=scale, gscale=gscale, E=E, N=N, K=K)


def compress_split(w):
    """A gate_up weight w [E, N, K] whose row halves [0, N/2) and [N/2, N) are separate linears, each
    with its own Eq. 5 tensor scale (the model card's checkpoint keeps gate and up apart): every half
    is compressed as a tensor of its own. -> dict as compress() with gscale [E, 2] and gsplit."""
    w = _c(w, np.float32)
    E, N, K = w.shape
    W = compress(w.reshape(2 * E, N // 2, K))
    return dict(packed=W["packed"].reshape(E, N, K // 4), mask=W["mask"].reshape(E, N, K // 16),
                scale=W["scale"].reshape(E, N, K // 32), gscale=W["gscale"].reshape(E, 2), E=E, N=N, K=K,
                gsplit=True)


def split_halves(W):
    """The two linears of split weights as weights of their own: [gate rows, up rows]."""
    n2 = W["N"] // 2
    return [dict(packed=_c(W["packed"][:, h * n2:(h + 1) * n2], np.uint8),
                 mask=_c(W["mask"][:, h * n2:(h + 1) * n2], np.uint8),
                 scale=_c(W["scale"][:, h * n2:(h + 1) * n2], np.uint8),
                 gscale=_c(W["gscale"][:, h], np.float32), E=W["E"], N=n2, K=W["K"]) for h in (0, 1)]


def dequant_weights(W, e):
    """Dequantized weights of expert e without the tensor scale: e2m1 * e4m3, [N, K] double."""
    dense = unpack(W["packed"][e], W["mask"][e])
    return dequant(dense, W["scale"][e])


# --- routing, dispatch, GEMM, SwiGLU, combine -------------------------------------------
def route(ids, E):
    ids = _c(ids, np.int32)
    T, k = ids.shape
    counts = np.zeros(E, np.int32)
    offsets = np.zeros(E + 1, np.int32)
    sorted_slot = np.zeros(T * k, np.int32)
    slot_pos = np.zeros(T * k, np.int32)
    _check(lib().orc_route(_p(ids), T, k, E, _p(counts), _p(offsets), _p(sorted_slot), _p(slot_pos)), "route")
    return dict(counts=counts, offsets=offsets, sorted_slot=sorted_slot, slot_pos=slot_pos)


def dispatch_quantize(x, sorted_slot, k, offsets, gamma):
    x = _c(x, np.float32)
    T, K = x.shape
    offsets = _c(offsets, np.int32)
    E = offsets.size - 1
    rows = int(offsets[-1])
    q = np.zeros((rows, K // 2), np.uint8)
    s = np.zeros((rows, K // 32), np.uint8)
    gamma = _c(np.broadcast_to(np.asarray(gamma, np.float32), (E,)), np.float32)
    ss = _c(sorted_slot, np.int32)
    _check(lib().orc_dispatch_quantize(_p(x), T, K, _p(ss), k, _p(offsets), E, _p(gamma), _p(q), _p(s)),
           "dispatch_quantize")
    return q, s


def grouped_gemm(W, q, s, gamma_a, offsets, row_list=None):
    """Rows of Y (double) for permuted rows row_list (default: all rows). Split weights (separate gate
    and up linears) are two grouped GEMMs whose outputs sit side by side."""
    if W.get("gsplit"):
        return np.concatenate([grouped_gemm(Wh, q, s, gamma_a, offsets, row_list) for Wh in split_halves(W)], axis=1)
    offsets = _c(offsets, np.int32)
    E = W["E"]
    rows = int(offsets[-1])
    rl = np.arange(rows, dtype=np.int64) if row_list is None else _c(row_list, np.int64)
    y = np.zeros((rl.size, W["N"]), np.float64)
    gamma_a = _c(np.broadcast_to(np.asarray(gamma_a, np.float32), (E,)), np.float32)
    _check(lib().orc_grouped_gemm(_p(W["packed"]), _p(W["mask"]), _p(W["scale"]), _p(W["gscale"]), E, W["N"],
                                  W["K"], _p(_c(q, np.uint8)), _p(_c(s, np.uint8)), _p(gamma_a), _p(offsets),
                                  _p(rl), rl.size, _p(y)), "grouped_gemm")
    return y


def swiglu(y13):
    y13 = _c(y13, np.float64)
    R, I2 = y13.shape
    h = np.empty((R, I2 // 2), np.float64)
    lib().orc_swiglu(_p(y13), R, I2 // 2, _p(h))
    return h


def combine(y, slot_pos, w):
    y = _c(y, np.float64)
    w = _c(w, np.float32)
    T, k = w.shape
    H = y.shape[1]
    out = np.empty((T, H), np.float64)
    lib().orc_combine(_p(y), H, _p(_c(slot_pos, np.int32)), _p(w), T, k, _p(out))
    return out


def expert_of_rows(offsets, rows):
    offsets = np.asarray(offsets)
    return (np.searchsorted(offsets, np.asarray(rows), side="right") - 1).astype(np.int32)


def expert_mlp(W13, W2, q, s, gamma_a, gamma_h, offsets, row_list=None):
    """Routed-expert MLP for permuted rows (paper Appendix D.1 serving path):
    gate_up GEMM -> SwiGLU -> requantize h to NVFP4 in fp32 with the expert's gamma_h
    (32-blocks along I) -> down GEMM. Returns dict with y13, h (double), h codes and y2."""
    offsets = _c(offsets, np.int32)
    rows = int(offsets[-1])
    rl = np.arange(rows, dtype=np.int64) if row_list is None else _c(row_list, np.int64)
    y13 = grouped_gemm(W13, q, s, gamma_a, offsets, rl)
    h = swiglu(y13)
    I = h.shape[1]
    E = W13["E"]
    gamma_h = _c(np.broadcast_to(np.asarray(gamma_h, np.float32), (E,)), np.float32)
    # Decisions on codes are taken in fp32, the kernel's precision.
    hq_rows, hs_rows = quantize_rows(h.astype(np.float32), gamma_h, expert_of_rows(offsets, rl))
    hq = np.zeros((rows, I // 2), np.uint8)
    hs = np.zeros((rows, I // 32), np.uint8)
    hq[rl] = hq_rows
    hs[rl] = hs_rows
    y2 = grouped_gemm(W2, hq, hs, gamma_h, offsets, rl)
    return dict(y13=y13, h=h, hq=hq_rows, hs=hs_rows, y2=y2, rows=rl)


# --- dense NVFP4 control (paper Appendix D.2: the sparse kernel is compared with a dense NVFP4
# grouped GEMM; here the same format without pruning) ----------------------------------------------
def compress_dense(w):
    """Unpruned NVFP4 of fp32 weights [E, N, K]: per expert the Eq. 5 tensor scale over the whole
    [N, K] tensor, then the Eq. 3/5 row quantizer with that scale. Returns codes [E, N, K/2],
    scale [E, N, K/32], gscale [E]."""
    w = _c(w, np.float32)
    E, N, K = w.shape
    codes = np.empty((E, N, K // 2), np.uint8)
    scale = np.empty((E, N, K // 32), np.uint8)
    gscale = np.empty(E, np.float32)
    for e in range(E):
        gscale[e] = global_scale_of(w[e])
        codes[e], scale[e] = quantize_rows(w[e], gscale[e])
    return dict(codes=codes, scale=scale, gscale=gscale, E=E, N=N, K=K)


def dense_grouped_gemm(Wd, q, s, gamma_a, offsets, row_list=None):
    """Rows of Y (double) for the dense control: Y[p] = (deq(q[p], s[p]) / gamma_a[e]) .
    (deq(codes_e, scale_e) / gscale_e)^T for the expert e owning row p; the product by numpy matmul
    in double."""
    offsets = np.asarray(offsets, np.int64)
    E = Wd["E"]
    rows = int(offsets[-1])
    rl = np.arange(rows, dtype=np.int64) if row_list is None else np.asarray(row_list, np.int64)
    gamma_a = np.broadcast_to(np.asarray(gamma_a, np.float32), (E,))
    ex = expert_of_rows(offsets, rl)
    y = np.zeros((rl.size, Wd["N"]), np.float64)
    for e in np.unique(ex):
        sel = np.flatnonzero(ex == e)
        w = dequant(Wd["codes"][e], Wd["scale"][e]) / np.float64(Wd["gscale"][e])
        x = dequant(np.asarray(q)[rl[sel]], np.asarray(s)[rl[sel]]) / np.float64(gamma_a[e])
        y[sel] = x @ w.T
    return y


# --- metrics -------------------------------------------------------------------------------
def rel_frobenius(a, ref):
    """||a - ref||_F / ||ref||_F in double."""
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(a - ref)
    return float(num / den) if den > 0 else float(num)

