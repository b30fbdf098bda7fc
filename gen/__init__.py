"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle checks.

This module draws random numbers only; it holds none of the MoE method's arithmetic.
Host draws come from ``libgen_cpu.so``; device draws (for weight tensors too large to
generate on the host) come from ``libgen_gpu.so``, which computes bit-identical numbers
from the same header (``gen_math.h``).
"""
import ctypes
import os

import numpy as np

from .configs import CONFIGS, Config  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_cpu = None
_gpu = None

# Stream ids: (kind << 48) | detail.
STREAM_WEIGHT = 1 << 48          # | (projection << 32) | expert
STREAM_ACT = 2 << 48             # | tag
STREAM_ROUTER = 3 << 48


def weight_stream(proj, expert):
    return STREAM_WEIGHT | (proj << 32) | expert


def act_stream(tag):
    return STREAM_ACT | tag


def _lib_cpu():
    global _cpu
    if _cpu is None:
        path = os.path.join(_HERE, "libgen_cpu.so")
        if not os.path.exists(path):
            raise RuntimeError("gen/libgen_cpu.so is missing: run __graft_entry__.build()")
        lib = ctypes.CDLL(path)
        u64, i64, i32, dbl = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32, ctypes.c_double
        vp = ctypes.c_void_p
        lib.gen_fill_normal.argtypes = [u64, u64, u64, i64, dbl, vp]
        lib.gen_fill_student_t.argtypes = [u64, u64, u64, i64, i32, dbl, vp]
        lib.gen_fill_uniform.argtypes = [u64, u64, u64, i64, vp]
        lib.gen_route_uniform.argtypes = [u64, i64, i32, i32, vp, vp]
        lib.gen_route_uniform.restype = ctypes.c_int
        lib.gen_route_zipf.argtypes = [u64, i64, i32, i32, dbl, i32, vp, vp]
        lib.gen_route_zipf.restype = ctypes.c_int
        _cpu = lib
    return _cpu


def _lib_gpu():
    global _gpu
    if _gpu is None:
        path = os.path.join(_HERE, "libgen_gpu.so")
        if not os.path.exists(path):
            raise RuntimeError("gen/libgen_gpu.so is missing: run __graft_entry__.build()")
        lib = ctypes.CDLL(path)
        u64, i64, i32, dbl, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32, ctypes.c_double, ctypes.c_void_p
        lib.gen_gpu_fill_normal.argtypes = [vp, u64, u64, u64, i64, dbl, vp]
        lib.gen_gpu_fill_normal.restype = ctypes.c_int
        lib.gen_gpu_fill_student_t.argtypes = [vp, u64, u64, u64, i64, i32, dbl, vp]
        lib.gen_gpu_fill_student_t.restype = ctypes.c_int
        _gpu = lib
    return _gpu


def normal(seed, stream, n, scale=1.0, start=0):
    out = np.empty(n, dtype=np.float32)
    _lib_cpu().gen_fill_normal(seed, stream, start, n, float(scale), out.ctypes.data)
    return out


def student_t(seed, stream, n, nu=4, scale=1.0, start=0):
    out = np.empty(n, dtype=np.float32)
    _lib_cpu().gen_fill_student_t(seed, stream, start, n, nu, float(scale), out.ctypes.data)
    return out


def uniform(seed, stream, n, start=0):
    out = np.empty(n, dtype=np.float64)
    _lib_cpu().gen_fill_uniform(seed, stream, start, n, out.ctypes.data)
    return out


def route_uniform(seed, T, E, k):
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    rc = _lib_cpu().gen_route_uniform(seed, T, E, k, ids.ctypes.data, w.ctypes.data)
    if rc != 0:
        raise ValueError("gen_route_uniform: bad arguments")
    return ids, w


def route_zipf(seed, T, E, k, s=1.1, n_zero=0):
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    rc = _lib_cpu().gen_route_zipf(seed, T, E, k, float(s), n_zero, ids.ctypes.data, w.ctypes.data)
    if rc != 0:
        raise ValueError("gen_route_zipf: bad arguments")
    return ids, w


def gpu_fill_normal(out, seed, stream, scale=1.0, start=0):
    """Fill a contiguous float32 CUDA tensor with the same numbers ``normal`` returns."""
    import torch
    assert out.is_cuda and out.dtype == torch.float32 and out.is_contiguous()
    rc = _lib_gpu().gen_gpu_fill_normal(ctypes.c_void_p(torch.cuda.current_stream().cuda_stream), seed, stream,
                                        start, out.numel(), float(scale), ctypes.c_void_p(out.data_ptr()))
    if rc != 0:
        raise RuntimeError("gen_gpu_fill_normal failed: %d" % rc)
    return out


def gpu_fill_student_t(out, seed, stream, nu=4, scale=1.0, start=0):
    import torch
    assert out.is_cuda and out.dtype == torch.float32 and out.is_contiguous()
    rc = _lib_gpu().gen_gpu_fill_student_t(ctypes.c_void_p(torch.cuda.current_stream().cuda_stream), seed, stream,
                                           start, out.numel(), nu, float(scale), ctypes.c_void_p(out.data_ptr()))
    if rc != 0:
        raise RuntimeError("gen_gpu_fill_student_t failed: %d" % rc)
    return out


def routing(cfg, T=None):
    """Router ids [T, k] and weights [T, k] for a config."""
    T = cfg.T if T is None else T
    if cfg.routing == "uniform":
        return route_uniform(cfg.seed, T, cfg.E, cfg.k)
    return route_zipf(cfg.seed, T, cfg.E, cfg.k, s=cfg.zipf_s, n_zero=cfg.zipf_zero)


def activations(cfg, tag, T, K, start_row=0):
    """Activation rows [T, K] (float32) for a config: N(0,1) or Student-t(nu)."""
    n = T * K
    start = start_row * K
    if cfg.act_dist == "normal":
        x = normal(cfg.seed, act_stream(tag), n, 1.0, start)
    else:
        x = student_t(cfg.seed, act_stream(tag), n, cfg.act_nu, 1.0, start)
    return x.reshape(T, K)


def weights_expert(cfg, proj, expert, N, K):
    """Uncompressed weights of one expert and projection, [N, K] float32 ~ N(0, std^2)."""
    return normal(cfg.seed, weight_stream(proj, expert), N * K, cfg.w_std).reshape(N, K)


def gpu_weights(cfg, proj, E, N, K, out=None):
    """All experts of one projection drawn on the device, [E, N, K] float32."""
    import torch
    if out is None:
        out = torch.empty((E, N, K), dtype=torch.float32, device="cuda")
    for e in range(E):
        gpu_fill_normal(out[e], cfg.seed, weight_stream(proj, e), cfg.w_std)
    return out
