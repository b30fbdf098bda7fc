"""Python binding of libmoesq.so: the MoE expert path over paired-4:8 sparse NVFP4 weights on
MI355X (gfx950).

Argument marshalling only: every step runs in the library's HIP kernels. PyTorch supplies device
memory and the current stream. The functions keep the C ABI names (``include/moesq.h``); outputs
that are not passed in are allocated with ``torch.empty`` on the current device.

There is no CPU fallback: if ``libmoesq.so`` is missing, every call raises.
"""
import ctypes
import os

import torch

__all__ = [
    "MoesqError", "Weights", "lib", "moesq_route_permute", "moesq_quantize_act", "moesq_route_quantize",
    "moesq_route_quantize_dyn", "moesq_route_quantize_gemm", "moesq_grouped_gemm",
    "moesq_expert_mlp", "moesq_unpermute_combine", "moesq_compress_weights", "moesq_unpack_weights",
    "moesq_workspace_bytes", "moesq_status_str", "moesq_version", "moesq_global_scale",
    "moesq_prepack_weights", "moesq_kernel_layout_bytes",
    "F32", "BF16", "F_DUMP_GATEUP", "F_FORCE_DECODE", "F_FORCE_PREFILL", "F_CAPACITY", "F_DUMP_H", "F_CALIBRATE",
    "WS_ROUTE", "WS_MLP", "WS_MLP_DUMP", "WS_COMPRESS", "WS_ROUTE_CAPACITY", "WS_MLP_CALIBRATE",
    "moesq_route_capacity", "moesq_calibrate_gamma_h", "moesq_expert_mlp_noalloc", "NOALLOC_SCRATCH_BYTES",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoesq.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_PATTERN, ERR_HIP = 0, -1, -2, -3, -4, -5
F32, BF16 = 0, 1
F_DUMP_GATEUP, F_FORCE_DECODE, F_FORCE_PREFILL, F_CAPACITY, F_DUMP_H, F_CALIBRATE = 1, 2, 4, 8, 16, 32
WS_ROUTE, WS_MLP, WS_MLP_DUMP, WS_COMPRESS, WS_ROUTE_CAPACITY, WS_MLP_CALIBRATE = 1, 2, 3, 4, 5, 6
NOALLOC_SCRATCH_BYTES = 32 << 20   # MOESQ_NOALLOC_SCRATCH_BYTES


class MoesqError(RuntimeError):
    def __init__(self, call, status):
        super().__init__("%s failed: %s (%d)" % (call, moesq_status_str(status), status))
        self.status = status


class _CWeights(ctypes.Structure):
    _fields_ = [("E", ctypes.c_int32), ("N", ctypes.c_int32), ("K", ctypes.c_int32),
                ("packed", ctypes.c_void_p), ("mask", ctypes.c_void_p), ("scale", ctypes.c_void_p),
                ("gscale", ctypes.c_void_p), ("kl", ctypes.c_void_p), ("gscale_split", ctypes.c_int32)]


_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libmoesq.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, u32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32, ctypes.c_size_t
        W = ctypes.POINTER(_CWeights)
        L.moesq_route_permute.argtypes = [vp, vp, i64, i32, i32, vp, vp, vp, vp, vp, sz, vp]
        L.moesq_quantize_act.argtypes = [vp, vp, i32, i64, i32, i64, vp, i32, i64, vp, vp, i32, vp, vp, vp]
        L.moesq_route_capacity.argtypes = [vp, vp, i64, i32, i32, i32, vp, vp, vp, sz, vp]
        L.moesq_route_quantize.argtypes = [vp, vp, i64, i32, i32, vp, i32, i32, i64, vp, vp, vp, vp, vp, vp, sz, vp,
                                           vp, vp, vp]
        L.moesq_grouped_gemm.argtypes = [vp, W, vp, vp, vp, vp, vp, i64, vp, i32, u32]
        L.moesq_route_quantize_dyn.argtypes = [vp, vp, i64, i32, i32, vp, i32, i32, i64, vp, vp, vp, vp, vp, vp, sz,
                                               vp, vp, vp, vp]
        L.moesq_route_quantize_gemm.argtypes = [vp, vp, i64, i32, i32, vp, i32, i32, i64, vp, W, vp, vp, vp,
                                                vp, vp, sz, vp, vp, vp, vp, i32, vp]
        L.moesq_expert_mlp.argtypes = [vp, W, W, vp, vp, vp, vp, vp, vp, i64, vp, i32, vp, sz, u32]
        L.moesq_expert_mlp_noalloc.argtypes = [vp, W, W, vp, vp, vp, vp, vp, vp, i64, vp, i32, u32]
        L.moesq_unpermute_combine.argtypes = [vp, vp, i32, vp, vp, i64, i32, i32, vp, i32]
        L.moesq_compress_weights.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]
        L.moesq_unpack_weights.argtypes = [vp, W, vp, vp]
        L.moesq_global_scale.argtypes = [vp, vp, i32, i64, i32, i64, vp]
        L.moesq_prepack_weights.argtypes = [vp, W, vp, sz]
        L.moesq_kernel_layout_bytes.argtypes = [i32, i32, i32]
        L.moesq_kernel_layout_bytes.restype = sz
        L.moesq_dense_layout_bytes.argtypes = [i32, i32, i32]
        L.moesq_dense_layout_bytes.restype = sz
        L.moesq_prepack_dense_weights.argtypes = [vp, i32, i32, i32, vp, vp, vp, sz]
        L.moesq_dense_grouped_gemm.argtypes = [vp, W, vp, vp, vp, vp, vp, i64, vp, i32, u32]
        L.moesq_workspace_bytes.argtypes = [i32, i64, i32, i32, i32, i32, i32]
        L.moesq_workspace_bytes.restype = sz
        L.moesq_status_str.argtypes = [i32]
        L.moesq_status_str.restype = ctypes.c_char_p
        L.moesq_version.restype = i32
        for name in ("moesq_route_permute", "moesq_route_capacity", "moesq_quantize_act", "moesq_route_quantize", "moesq_route_quantize_dyn", "moesq_route_quantize_gemm", "moesq_grouped_gemm",
                     "moesq_expert_mlp", "moesq_expert_mlp_noalloc",
                     "moesq_unpermute_combine", "moesq_compress_weights", "moesq_unpack_weights", "moesq_global_scale",
                     "moesq_prepack_weights"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def moesq_status_str(status):
    return lib().moesq_status_str(int(status)).decode()


def moesq_version():
    return lib().moesq_version()


def moesq_workspace_bytes(kind, T=0, k=0, E=0, K=0, N=0, I=0):
    return int(lib().moesq_workspace_bytes(kind, T, k, E, K, N, I))


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(call, rc):
    if rc != OK:
        raise MoesqError(call, rc)


def _dtype_code(dt):
    if dt == torch.float32:
        return F32
    if dt == torch.bfloat16:
        return BF16
    raise ValueError("unsupported dtype %s" % dt)


def _dev(t):
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    return t


def _need(t, name, shape, dtype, device=None):
    """A caller-supplied tensor must be a contiguous tensor of the given shape and dtype (the C ABI takes
    bare pointers and cannot check sizes: an undersized buffer would be written out of bounds). Where it
    lives is checked separately (_on_device), after every tensor of a call has passed this check."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s: shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if t.dtype != dtype:
        raise ValueError("%s: dtype %s, expected %s" % (name, t.dtype, dtype))
    if not t.is_contiguous():
        raise ValueError("%s: must be contiguous" % name)


def _need_bytes(t, name, nbytes):
    """A byte buffer (workspace) of at least nbytes, contiguous."""
    if t.numel() * t.element_size() < nbytes:
        raise ValueError("%s: %d bytes, need %d" % (name, t.numel() * t.element_size(), nbytes))
    if not t.is_contiguous():
        raise ValueError("%s: must be contiguous" % name)


def _on_device(**tensors):
    """Every given tensor is a device tensor, all on one device."""
    dev = None
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("%s: expected a device tensor" % name)
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("%s: on %s, expected %s" % (name, t.device, dev))


def _check_codes(q, s, rows, K, xk=None):
    """Expert-sorted activation codes q [rows, K/2] u8, scales s [rows, K/32] u8, optional f16 copy [rows, K]."""
    _need(q, "q", (rows, K // 2), torch.uint8)
    _need(s, "s", (rows, K // 32), torch.uint8)
    _need(xk, "xk", (rows, K), torch.float16)


class Weights:
    """Weights of one projection for E experts (device tensors): pair-bitmask v1 storage
    packed [E,N,K/4] u8, mask [E,N,K/16] u8, scale [E,N,K/32] u8 (UE4M3), gscale [E] f32 (or [E, 2]:
    separate tensor scales of rows [0, N/2) and [N/2, N), a gate_up weight kept as two linears), and
    kl, the same bytes in the GEMM's kernel layout (built by ``prepack``)."""

    def __init__(self, packed, mask, scale, gscale, kl=None):
        E, N, K4 = packed.shape
        self.E, self.N, self.K = E, N, K4 * 4
        assert mask.shape == (E, N, self.K // 16) and scale.shape == (E, N, self.K // 32)
        assert gscale.shape in ((E,), (E, 2)) and gscale.is_contiguous()
        self.gsplit = gscale.dim() == 2
        for t in (packed, mask, scale):
            assert t.dtype == torch.uint8 and t.is_contiguous()
        assert gscale.dtype == torch.float32
        self.packed, self.mask, self.scale, self.gscale, self.kl = packed, mask, scale, gscale, kl

    def prepack(self):
        """Build (or rebuild) the kernel layout from the pair-bitmask storage."""
        nb = moesq_kernel_layout_bytes(self.E, self.N, self.K)
        if self.kl is None or self.kl.numel() < nb:
            self.kl = torch.empty(nb, dtype=torch.uint8, device=self.packed.device)
        c = self.cstruct()
        _check("moesq_prepack_weights", lib().moesq_prepack_weights(_stream(), ctypes.byref(c), _p(self.kl), nb))
        return self

    @classmethod
    def empty(cls, E, N, K, device="cuda"):
        u8 = torch.uint8
        return cls(torch.empty((E, N, K // 4), dtype=u8, device=device),
                   torch.empty((E, N, K // 16), dtype=u8, device=device),
                   torch.empty((E, N, K // 32), dtype=u8, device=device),
                   torch.empty((E,), dtype=torch.float32, device=device))

    def cstruct(self):
        return _CWeights(self.E, self.N, self.K, self.packed.data_ptr(), self.mask.data_ptr(),
                         self.scale.data_ptr(), self.gscale.data_ptr(),
                         None if self.kl is None else self.kl.data_ptr(), int(self.gsplit))

    def nbytes(self):
        return self.packed.numel() + self.mask.numel() + self.scale.numel()


def moesq_route_permute(topk_ids, E, counts=None, offsets=None, sorted_slot=None, slot_pos=None,
                        workspace=None, dev_status=None):
    """Histogram + scan + stable scatter of topk_ids [T, k] (int32). Returns a dict of device tensors."""
    _dev(topk_ids)
    assert topk_ids.dtype == torch.int32 and topk_ids.is_contiguous()
    T, k = topk_ids.shape
    dev = topk_ids.device
    i32 = torch.int32
    counts = torch.empty(E, dtype=i32, device=dev) if counts is None else counts
    offsets = torch.empty(E + 1, dtype=i32, device=dev) if offsets is None else offsets
    sorted_slot = torch.empty(T * k, dtype=i32, device=dev) if sorted_slot is None else sorted_slot
    slot_pos = torch.empty(T * k, dtype=i32, device=dev) if slot_pos is None else slot_pos
    need = moesq_workspace_bytes(WS_ROUTE, T, k, E)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("moesq_route_permute",
           lib().moesq_route_permute(_stream(), _p(topk_ids), T, k, E, _p(counts), _p(offsets), _p(sorted_slot),
                                     _p(slot_pos), _p(workspace), wsb, _p(dev_status)))
    return dict(counts=counts, offsets=offsets, sorted_slot=sorted_slot, slot_pos=slot_pos)


def moesq_route_capacity(topk_ids, E, capacity, counts=None, slot_pos=None, workspace=None, dev_status=None):
    """Slot positions in the fixed-capacity layout (expert e owns rows [e C, (e + 1) C)): returns
    dict(counts [E], slot_pos [T*k]; -1 for slots over the capacity)."""
    _dev(topk_ids)
    assert topk_ids.dtype == torch.int32 and topk_ids.is_contiguous()
    T, k = topk_ids.shape
    dev = topk_ids.device
    counts = torch.empty(E, dtype=torch.int32, device=dev) if counts is None else counts
    slot_pos = torch.empty(T * k, dtype=torch.int32, device=dev) if slot_pos is None else slot_pos
    need = moesq_workspace_bytes(WS_ROUTE_CAPACITY, T, k, E)
    workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev) if workspace is None else workspace
    _check("moesq_route_capacity",
           lib().moesq_route_capacity(_stream(), _p(topk_ids), T, k, E, capacity, _p(counts), _p(slot_pos),
                                      _p(workspace), workspace.numel(), _p(dev_status)))
    return dict(counts=counts, slot_pos=slot_pos)


def moesq_quantize_act(x, gamma, slot_pos=None, k=1, offsets=None, q=None, s=None, rows=None, xk=None,
                       capacity_experts=0):
    """NVFP4-quantize rows of x [T, K] (fp32/bf16). With slot_pos (from moesq_route_permute), token t's
    j-th routed copy goes to permuted row slot_pos[t*k + j] and (with offsets) uses gamma[expert of that
    row]; with ``capacity_experts`` = E (and no offsets) the rows are in the fixed-capacity layout and row
    p uses gamma[p // (rows // E)]. Returns (q [rows,K/2], s [rows,K/32]);
    with ``xk`` (a [rows, K] float16 tensor, or True to allocate one) also writes the GEMM's f16
    operand copy and returns (q, s, xk)."""
    _dev(x)
    T, K = x.shape
    assert x.stride(1) == 1
    if rows is None:
        rows = T if slot_pos is None else slot_pos.numel()
    E = capacity_experts if offsets is None else offsets.numel() - 1
    q = torch.empty((rows, K // 2), dtype=torch.uint8, device=x.device) if q is None else q
    s = torch.empty((rows, K // 32), dtype=torch.uint8, device=x.device) if s is None else s
    want_xk = xk is not None
    if xk is True:
        xk = torch.empty((rows, K), dtype=torch.float16, device=x.device)
    _check("moesq_quantize_act",
           lib().moesq_quantize_act(_stream(), _p(x), _dtype_code(x.dtype), T, K, x.stride(0), _p(slot_pos), k,
                                    rows, _p(gamma), _p(offsets), E, _p(q), _p(s), _p(xk if want_xk else None)))
    return (q, s, xk) if want_xk else (q, s)


def moesq_route_quantize(topk_ids, E, x, gamma, rt=None, q=None, s=None, xk=None, workspace=None,
                         dev_status=None):
    """Routing + scatter quantization in one call (one kernel launch for decode-sized batches).
    topk_ids [T, k] int32, x [T, K] fp32/bf16, gamma [E] fp32. ``rt`` is a dict of routing outputs as
    returned by moesq_route_permute (allocated when None); ``xk`` as in moesq_quantize_act.
    Returns (rt, q, s) or (rt, q, s, xk)."""
    _dev(topk_ids)
    _dev(x)
    assert topk_ids.dtype == torch.int32 and topk_ids.is_contiguous() and x.stride(1) == 1
    T, k = topk_ids.shape
    K = x.shape[1]
    dev = x.device
    i32 = torch.int32
    if rt is None:
        rt = dict(counts=torch.empty(E, dtype=i32, device=dev), offsets=torch.empty(E + 1, dtype=i32, device=dev),
                  sorted_slot=torch.empty(T * k, dtype=i32, device=dev),
                  slot_pos=torch.empty(T * k, dtype=i32, device=dev))
    q = torch.empty((T * k, K // 2), dtype=torch.uint8, device=dev) if q is None else q
    s = torch.empty((T * k, K // 32), dtype=torch.uint8, device=dev) if s is None else s
    want_xk = xk is not None
    if xk is True:
        xk = torch.empty((T * k, K), dtype=torch.float16, device=dev)
    need = moesq_workspace_bytes(WS_ROUTE, T, k, E)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("moesq_route_quantize",
           lib().moesq_route_quantize(_stream(), _p(topk_ids), T, k, E, _p(x), _dtype_code(x.dtype), K, x.stride(0),
                                      _p(gamma), _p(rt["counts"]), _p(rt["offsets"]), _p(rt["sorted_slot"]),
                                      _p(rt["slot_pos"]), _p(workspace), wsb, _p(q), _p(s),
                                      _p(xk if want_xk else None), _p(dev_status)))
    return (rt, q, s, xk) if want_xk else (rt, q, s)


def moesq_route_quantize_dyn(topk_ids, E, x, gamma_out=None, rt=None, q=None, s=None, xk=None, workspace=None,
                             dev_status=None):
    """moesq_route_quantize with the activation tensor scale computed on the device from x (Eq. 5 over
    all of x), written to ``gamma_out`` [E] fp32 (allocated when None). Returns (rt, q, s, gamma_out)
    or (rt, q, s, xk, gamma_out)."""
    _dev(topk_ids)
    _dev(x)
    assert topk_ids.dtype == torch.int32 and topk_ids.is_contiguous() and x.stride(1) == 1
    T, k = topk_ids.shape
    K = x.shape[1]
    dev = x.device
    i32 = torch.int32
    if rt is None:
        rt = dict(counts=torch.empty(E, dtype=i32, device=dev), offsets=torch.empty(E + 1, dtype=i32, device=dev),
                  sorted_slot=torch.empty(T * k, dtype=i32, device=dev),
                  slot_pos=torch.empty(T * k, dtype=i32, device=dev))
    q = torch.empty((T * k, K // 2), dtype=torch.uint8, device=dev) if q is None else q
    s = torch.empty((T * k, K // 32), dtype=torch.uint8, device=dev) if s is None else s
    gamma_out = torch.empty(E, dtype=torch.float32, device=dev) if gamma_out is None else gamma_out
    want_xk = xk is not None
    if xk is True:
        xk = torch.empty((T * k, K), dtype=torch.float16, device=dev)
    need = moesq_workspace_bytes(WS_ROUTE, T, k, E)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("moesq_route_quantize_dyn",
           lib().moesq_route_quantize_dyn(_stream(), _p(topk_ids), T, k, E, _p(x), _dtype_code(x.dtype), K,
                                          x.stride(0), _p(gamma_out), _p(rt["counts"]), _p(rt["offsets"]),
                                          _p(rt["sorted_slot"]), _p(rt["slot_pos"]), _p(workspace), wsb, _p(q),
                                          _p(s), _p(xk if want_xk else None), _p(dev_status)))
    return (rt, q, s, xk, gamma_out) if want_xk else (rt, q, s, gamma_out)


def moesq_route_quantize_gemm(topk_ids, x, gamma_a, W, rt=None, q=None, s=None, xk=None, y=None,
                              y_dtype=torch.bfloat16, workspace=None, dev_status=None):
    """moesq_route_quantize followed by moesq_grouped_gemm in one call (a single launch for small
    decode batches). Arguments as in those two; ``xk`` None (not written), True (allocated) or a
    tensor. Returns (rt, q, s, y) or (rt, q, s, xk, y)."""
    _dev(topk_ids)
    _dev(x)
    assert topk_ids.dtype == torch.int32 and topk_ids.is_contiguous() and x.stride(1) == 1
    T, k = topk_ids.shape
    K, E = x.shape[1], W.E
    dev = x.device
    i32 = torch.int32
    if rt is None:
        rt = dict(counts=torch.empty(E, dtype=i32, device=dev), offsets=torch.empty(E + 1, dtype=i32, device=dev),
                  sorted_slot=torch.empty(T * k, dtype=i32, device=dev),
                  slot_pos=torch.empty(T * k, dtype=i32, device=dev))
    q = torch.empty((T * k, K // 2), dtype=torch.uint8, device=dev) if q is None else q
    s = torch.empty((T * k, K // 32), dtype=torch.uint8, device=dev) if s is None else s
    want_xk = xk is not None
    if xk is True:
        xk = torch.empty((T * k, K), dtype=torch.float16, device=dev)
    if y is None:
        y = torch.empty((T * k, W.N), dtype=y_dtype, device=dev)
    need = moesq_workspace_bytes(WS_ROUTE, T, k, E)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    c = W.cstruct()
    _check("moesq_route_quantize_gemm",
           lib().moesq_route_quantize_gemm(_stream(), _p(topk_ids), T, k, E, _p(x), _dtype_code(x.dtype), K,
                                           x.stride(0), _p(gamma_a), ctypes.byref(c), _p(rt["counts"]),
                                           _p(rt["offsets"]), _p(rt["sorted_slot"]), _p(rt["slot_pos"]),
                                           _p(workspace), wsb, _p(q), _p(s), _p(xk if want_xk else None), _p(y),
                                           _dtype_code(y.dtype), _p(dev_status)))
    return (rt, q, s, xk, y) if want_xk else (rt, q, s, y)


def _check_gemm_io(W, q, s, gamma_a, offsets, xk, flags, y=None, N=None):
    rows = q.shape[0]
    _check_codes(q, s, rows, W.K, xk)
    _need(gamma_a, "gamma_a", (W.E,), torch.float32)
    _need(offsets, "offsets", (W.E,) if flags & F_CAPACITY else (W.E + 1,), torch.int32)
    if y is not None:
        _need(y, "y", (rows, W.N if N is None else N), y.dtype)
    _on_device(q=q, s=s, xk=xk, gamma_a=gamma_a, offsets=offsets, y=y)
    return rows


def moesq_grouped_gemm(W, q, s, gamma_a, offsets, y=None, y_dtype=torch.bfloat16, flags=0, xk=None):
    rows = _check_gemm_io(W, q, s, gamma_a, offsets, xk, flags, y)
    if y is None:
        y = torch.empty((rows, W.N), dtype=y_dtype, device=q.device)
    c = W.cstruct()
    _check("moesq_grouped_gemm",
           lib().moesq_grouped_gemm(_stream(), ctypes.byref(c), _p(q), _p(s), _p(xk), _p(gamma_a), _p(offsets), rows,
                                    _p(y), _dtype_code(y.dtype), flags))
    return y


_DUMPS = F_DUMP_GATEUP | F_DUMP_H


def mlp_workspace(rows, I, dump=False, device="cuda"):
    nb = moesq_workspace_bytes(WS_MLP_DUMP if dump else WS_MLP, rows, 0, 0, 0, 0, I)
    return torch.empty(max(nb, 1), dtype=torch.uint8, device=device)


def _a256(x):
    return (x + 255) // 256 * 256


def mlp_workspace_views(ws, rows, I, dump=False):
    """(h_q [rows, I/2], h_s [rows, I/32], gate_up fp32 [rows, 2I] or None) inside an MLP workspace
    (the f16 copy of h sits between h_s and the gate_up dump)."""
    hq = ws[:rows * (I // 2)].view(rows, I // 2)
    o = _a256(rows * (I // 2))
    hs = ws[o:o + rows * (I // 32)].view(rows, I // 32)
    o += _a256(rows * (I // 32))
    o += _a256(rows * I * 2)
    d = ws[o:o + rows * 2 * I * 4].view(torch.float32).view(rows, 2 * I) if dump else None
    return hq, hs, d


def mlp_hk_view(ws, rows, I):
    """h_k f16 [rows, I] inside an MLP workspace: the down GEMM's operand copy of the requantized h
    (moesq_quantize_act's f16 copy format)."""
    o = _a256(rows * (I // 2)) + _a256(rows * (I // 32))
    return ws[o:o + rows * I * 2].view(torch.float16).view(rows, I)


def mlp_h_views(ws, rows, I):
    """(h_k f16 [rows, I], and the fp32 h [rows, I] that the requantization read, written with F_DUMP_H)
    inside a dump-sized MLP workspace."""
    o = _a256(rows * (I // 2)) + _a256(rows * (I // 32)) + _a256(rows * I * 2) + _a256(rows * 2 * I * 4)
    h = ws[o:o + rows * I * 4].view(torch.float32).view(rows, I)
    return mlp_hk_view(ws, rows, I), h


def moesq_expert_mlp(W13, W2, q, s, gamma_a, gamma_h, offsets, y=None, y_dtype=torch.bfloat16, workspace=None,
                     flags=0, xk=None):
    if flags & F_CALIBRATE:
        raise ValueError("calibration: use moesq_calibrate_gamma_h")
    if not (W13.N % 2 == 0 and W2.K == W13.N // 2 and W2.E == W13.E):
        raise ValueError("W13 [E, 2I, H] and W2 [E, H, I] do not match")
    I = W13.N // 2
    rows = q.shape[0]
    dump = bool(flags & _DUMPS)
    _need(gamma_h, "gamma_h", (W13.E,), torch.float32)
    if workspace is not None:
        _need_bytes(workspace, "workspace",
                    moesq_workspace_bytes(WS_MLP_DUMP if dump else WS_MLP, rows, 0, 0, 0, 0, I))
    _check_gemm_io(W13, q, s, gamma_a, offsets, xk, flags, y, W2.N)
    _on_device(q=q, gamma_h=gamma_h, workspace=workspace)
    if y is None:
        y = torch.empty((rows, W2.N), dtype=y_dtype, device=q.device)
    if workspace is None:
        workspace = mlp_workspace(rows, I, dump, q.device)
    a, b = W13.cstruct(), W2.cstruct()
    _check("moesq_expert_mlp",
           lib().moesq_expert_mlp(_stream(), ctypes.byref(a), ctypes.byref(b), _p(q), _p(s), _p(xk), _p(gamma_a),
                                  _p(gamma_h), _p(offsets), rows, _p(y), _dtype_code(y.dtype), _p(workspace),
                                  workspace.numel(), flags))
    return y, workspace


def moesq_expert_mlp_noalloc(W13, W2, q, s, gamma_a, gamma_h, offsets, y, flags=0, xk=None):
    """moesq_expert_mlp without a workspace argument: the library's static per-GPU scratch array holds the
    intermediate h (for callers that cannot allocate; the caller passes the output y). Calls that may
    overlap on one GPU race on that array."""
    if not (W13.N % 2 == 0 and W2.K == W13.N // 2 and W2.E == W13.E):
        raise ValueError("W13 [E, 2I, H] and W2 [E, H, I] do not match")
    _need(gamma_h, "gamma_h", (W13.E,), torch.float32)
    rows = _check_gemm_io(W13, q, s, gamma_a, offsets, xk, flags, y, W2.N)
    _on_device(q=q, gamma_h=gamma_h, y=y)
    a, b = W13.cstruct(), W2.cstruct()
    _check("moesq_expert_mlp_noalloc",
           lib().moesq_expert_mlp_noalloc(_stream(), ctypes.byref(a), ctypes.byref(b), _p(q), _p(s), _p(xk),
                                          _p(gamma_a), _p(gamma_h), _p(offsets), rows, _p(y), _dtype_code(y.dtype),
                                          flags))
    return y


def moesq_calibrate_gamma_h(W13, W2, q, s, gamma_a, offsets, flags=0, xk=None, workspace=None):
    """The intermediate tensor scales of the routed-expert MLP (moesq_expert_mlp with F_CALIBRATE):
    gate_up + SwiGLU on the given rows, per-expert amax(h) and Eq. 5. Returns (gamma_h [E], amax_h [E])
    as views into the workspace (float32)."""
    E = W13.E
    nb = moesq_workspace_bytes(WS_MLP_CALIBRATE, 0, 0, E)
    if workspace is not None:
        _need_bytes(workspace, "workspace", nb)
    rows = _check_gemm_io(W13, q, s, gamma_a, offsets, xk, flags)
    _on_device(q=q, workspace=workspace)
    if workspace is None:
        workspace = torch.empty(nb, dtype=torch.uint8, device=q.device)
    a, b = W13.cstruct(), W2.cstruct()
    _check("moesq_expert_mlp",
           lib().moesq_expert_mlp(_stream(), ctypes.byref(a), ctypes.byref(b), _p(q), _p(s), _p(xk), _p(gamma_a),
                                  None, _p(offsets), rows, None, F32, _p(workspace), workspace.numel(),
                                  flags | F_CALIBRATE))
    amax = workspace[:4 * E].view(torch.float32)
    o = _a256(4 * E)
    gamma = workspace[o:o + 4 * E].view(torch.float32)
    return gamma, amax


def moesq_unpermute_combine(y_sorted, slot_pos, topk_w, out=None, out_dtype=torch.bfloat16):
    T, k = topk_w.shape
    H = y_sorted.shape[1]
    _need(y_sorted, "y_sorted", (y_sorted.shape[0], H), y_sorted.dtype)
    _need(slot_pos, "slot_pos", (T * k,), torch.int32)
    _need(topk_w, "topk_w", (T, k), torch.float32)
    if out is not None:
        _need(out, "out", (T, H), out.dtype)
    _on_device(y_sorted=y_sorted, slot_pos=slot_pos, topk_w=topk_w, out=out)
    if out is None:
        out = torch.empty((T, H), dtype=out_dtype, device=y_sorted.device)
    _check("moesq_unpermute_combine",
           lib().moesq_unpermute_combine(_stream(), _p(y_sorted), _dtype_code(y_sorted.dtype), _p(slot_pos),
                                         _p(topk_w), T, k, H, _p(out), _dtype_code(out.dtype)))
    return out


def moesq_kernel_layout_bytes(E, N, K):
    return int(lib().moesq_kernel_layout_bytes(E, N, K))


def moesq_prepack_weights(W):
    return W.prepack()


def moesq_compress_weights(w, out=None, workspace=None, dev_status=None, prepack=True, split_halves=False):
    """fp32 weights [E, N, K] -> Weights (paired-4:8 pruning + NVFP4 + pair-bitmask v1), plus the
    kernel layout when ``prepack`` (and K % 256 == 0, N % 64 == 0). ``split_halves``: rows [0, N/2)
    and [N/2, N) are separate linears (gate and up) with their own tensor scale: the [2E, N/2, K]
    view is compressed (same byte layout) and gscale comes back as [E, 2]."""
    _dev(w)
    assert w.dtype == torch.float32 and w.is_contiguous()
    E, N, K = w.shape
    if out is None:
        out = Weights.empty(E, N, K, w.device)
        if split_halves:
            out = Weights(out.packed, out.mask, out.scale, torch.empty((E, 2), dtype=torch.float32, device=w.device))
    assert out.gsplit == split_halves
    Ec, Nc = (2 * E, N // 2) if split_halves else (E, N)
    assert N % 2 == 0 or not split_halves
    need = moesq_workspace_bytes(WS_COMPRESS, 0, 0, Ec)
    workspace = torch.empty(need, dtype=torch.uint8, device=w.device) if workspace is None else workspace
    _check("moesq_compress_weights",
           lib().moesq_compress_weights(_stream(), _p(w), Ec, Nc, K, _p(out.packed), _p(out.mask), _p(out.scale),
                                        _p(out.gscale), _p(workspace), workspace.numel(), _p(dev_status)))
    if prepack and K % 256 == 0 and N % 64 == 0:
        out.prepack()
    return out


def moesq_global_scale(x, out=None):
    """Eq. 5 tensor scale of x [rows, K] (fp32/bf16) computed on the device -> float32 tensor [1]."""
    _dev(x)
    rows, K = x.shape
    assert x.stride(1) == 1
    out = torch.empty(1, dtype=torch.float32, device=x.device) if out is None else out
    _check("moesq_global_scale", lib().moesq_global_scale(_stream(), _p(x), _dtype_code(x.dtype), rows, K,
                                                          x.stride(0), _p(out)))
    return out


def moesq_unpack_weights(W, dense=None, dev_status=None):
    if dense is None:
        dense = torch.empty((W.E, W.N, W.K // 2), dtype=torch.uint8, device=W.packed.device)
    c = W.cstruct()
    _check("moesq_unpack_weights", lib().moesq_unpack_weights(_stream(), ctypes.byref(c), _p(dense), _p(dev_status)))
    return dense


# ---------------------------------------------------------------- dense NVFP4 control ----------
class DenseWeights:
    """Unpruned NVFP4 weights of one projection for E experts (the dense control of the sparse
    kernels): codes [E,N,K/2] u8 (two E2M1 codes per byte, lower K in the low nibble), scale
    [E,N,K/32] u8 (UE4M3), gscale [E] f32, and kl, the dense kernel layout."""

    def __init__(self, codes, scale, gscale, kl=None):
        E, N, K2 = codes.shape
        self.E, self.N, self.K = E, N, K2 * 2
        assert scale.shape == (E, N, self.K // 32) and gscale.shape == (E,)
        self.codes, self.scale, self.gscale, self.kl = codes, scale, gscale, kl

    def prepack(self):
        nb = lib().moesq_dense_layout_bytes(self.E, self.N, self.K)
        if self.kl is None or self.kl.numel() < nb:
            self.kl = torch.empty(nb, dtype=torch.uint8, device=self.codes.device)
        _check("moesq_prepack_dense_weights",
               lib().moesq_prepack_dense_weights(_stream(), self.E, self.N, self.K, _p(self.codes), _p(self.scale),
                                                 _p(self.kl), nb))
        return self

    def cstruct(self):
        return _CWeights(self.E, self.N, self.K, None, None, None, self.gscale.data_ptr(),
                         None if self.kl is None else self.kl.data_ptr())

    def nbytes(self):
        return self.codes.numel() + self.scale.numel()


def compress_dense_weights(w, prepack=True):
    """fp32 weights [E, N, K] -> DenseWeights: per expert the Eq. 5 tensor scale over the whole
    [N, K] tensor, then row-wise NVFP4 quantization with that scale (no pruning)."""
    _dev(w)
    E, N, K = w.shape
    codes = torch.empty((E, N, K // 2), dtype=torch.uint8, device=w.device)
    scale = torch.empty((E, N, K // 32), dtype=torch.uint8, device=w.device)
    gscale = torch.empty((E,), dtype=torch.float32, device=w.device)
    for e in range(E):
        moesq_global_scale(w[e], out=gscale[e:e + 1])
        moesq_quantize_act(w[e], gscale[e:e + 1], q=codes[e], s=scale[e])
    out = DenseWeights(codes, scale, gscale)
    if prepack and K % 256 == 0 and N % 64 == 0:
        out.prepack()
    return out


def moesq_dense_grouped_gemm(W, q, s, gamma_a, offsets, y=None, y_dtype=torch.bfloat16, flags=0, xk=None):
    rows = _check_gemm_io(W, q, s, gamma_a, offsets, xk, flags, y)
    if y is None:
        y = torch.empty((rows, W.N), dtype=y_dtype, device=q.device)
    c = W.cstruct()
    _check("moesq_dense_grouped_gemm",
           lib().moesq_dense_grouped_gemm(_stream(), ctypes.byref(c), _p(q), _p(s), _p(xk), _p(gamma_a), _p(offsets),
                                          rows, _p(y), _dtype_code(y.dtype), flags))
    return y
