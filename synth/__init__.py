"""Seeded synthetic inputs for the ZeRO-1 shard step (tests and benchmark).

One generator, two implementations with identical bits: ``synth_host.c``
(host, via ctypes) and ``synth_gpu.hip`` (fills device buffers in place). The
value of element ``i`` of a buffer is a pure function of ``(seed, stream, i)``,
so the host can rebuild any sampled element of a device buffer without reading
it back. Nothing here computes any part of the optimizer step.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_HOST_SRC = os.path.join(_HERE, "synth_host.c")
_HOST_LIB = os.path.join(_HERE, "libsynth_host.so")
_GPU_SRC = os.path.join(_HERE, "synth_gpu.hip")
_GPU_LIB = os.path.join(_HERE, "libsynth_gpu.so")

KIND_GRAD, KIND_MASTER, KIND_EXP_AVG, KIND_EXP_AVG_SQ, KIND_INJECT = 0, 1, 2, 3, 4


def stream_id(kind: int, tensor: int, rank: int) -> int:
    """Philox key word 1: kind (4 bits) | tensor (12 bits) | rank (16 bits)."""
    assert 0 <= kind < 16 and 0 <= tensor < 4096 and 0 <= rank < 65536
    return (kind << 28) | (tensor << 16) | rank


def _stale(lib, src):
    return not os.path.exists(lib) or os.path.getmtime(lib) < os.path.getmtime(src)


def build_host(force: bool = False) -> str:
    if force or _stale(_HOST_LIB, _HOST_SRC):
        tmp = _HOST_LIB + ".tmp"
        subprocess.check_call(["gcc", "-O3", "-std=c11", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
                               "-o", tmp, _HOST_SRC, "-lm"])
        os.replace(tmp, _HOST_LIB)
    return _HOST_LIB


def build_gpu(force: bool = False) -> str:
    if force or _stale(_GPU_LIB, _GPU_SRC):
        tmp = _GPU_LIB + ".tmp"
        subprocess.check_call(["hipcc", "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
                               "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                               "-o", tmp, _GPU_SRC])
        os.replace(tmp, _GPU_LIB)
    return _GPU_LIB


_host = None
_gpu = None


def host_lib():
    global _host
    if _host is None:
        L = ctypes.CDLL(build_host() if _stale(_HOST_LIB, _HOST_SRC) else _HOST_LIB)
        vp, i64, u32, dbl, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32, ctypes.c_double, ctypes.c_int32
        L.synth_philox4x32_10.argtypes = [vp, vp, vp]
        L.synth_fill_f32.argtypes = [vp, i64, i64, u32, u32, dbl, i32]
        L.synth_fill_bf16.argtypes = [vp, i64, i64, u32, u32, dbl]
        L.synth_gather_f32.argtypes = [vp, vp, i64, u32, u32, dbl, i32]
        L.synth_gather_bf16.argtypes = [vp, vp, i64, u32, u32, dbl]
        L.synth_raw_blocks.argtypes = [vp, i64, i64, u32, u32]
        for f in ("synth_philox4x32_10", "synth_fill_f32", "synth_fill_bf16", "synth_gather_f32",
                  "synth_gather_bf16", "synth_raw_blocks"):
            getattr(L, f).restype = None
        _host = L
    return _host


def gpu_lib():
    global _gpu
    if _gpu is None:
        if not os.path.exists(_GPU_LIB):
            raise RuntimeError(f"{_GPU_LIB} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(_GPU_LIB)
        vp, i64, u32, dbl, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32, ctypes.c_double, ctypes.c_int32
        L.synth_gpu_fill_f32.argtypes = [vp, i64, i64, u32, u32, dbl, i32, vp]
        L.synth_gpu_fill_bf16.argtypes = [vp, i64, i64, u32, u32, dbl, vp]
        L.synth_gpu_fill_f32.restype = ctypes.c_int
        L.synth_gpu_fill_bf16.restype = ctypes.c_int
        _gpu = L
    return _gpu


# ---------------------------------------------------------------- host side

def philox4x32_10(ctr, key) -> list:
    c = (ctypes.c_uint32 * 4)(*ctr)
    k = (ctypes.c_uint32 * 2)(*key)
    o = (ctypes.c_uint32 * 4)()
    host_lib().synth_philox4x32_10(c, k, o)
    return list(o)


def host_f32(n: int, seed: int, stream: int, std: float, start: int = 0, absval: bool = False) -> np.ndarray:
    out = np.empty(n, np.float32)
    host_lib().synth_fill_f32(out.ctypes.data, n, start, seed, stream, std, int(absval))
    return out


def host_bf16(n: int, seed: int, stream: int, std: float, start: int = 0) -> np.ndarray:
    out = np.empty(n, np.uint16)
    host_lib().synth_fill_bf16(out.ctypes.data, n, start, seed, stream, std)
    return out


def host_f32_at(idx: np.ndarray, seed: int, stream: int, std: float, absval: bool = False) -> np.ndarray:
    idx = np.ascontiguousarray(idx, np.int64)
    out = np.empty(idx.size, np.float32)
    host_lib().synth_gather_f32(out.ctypes.data, idx.ctypes.data, idx.size, seed, stream, std, int(absval))
    return out


def host_bf16_at(idx: np.ndarray, seed: int, stream: int, std: float) -> np.ndarray:
    idx = np.ascontiguousarray(idx, np.int64)
    out = np.empty(idx.size, np.uint16)
    host_lib().synth_gather_bf16(out.ctypes.data, idx.ctypes.data, idx.size, seed, stream, std)
    return out


def raw_blocks(k: int, seed: int, stream: int, start: int = 0) -> np.ndarray:
    out = np.empty((k, 4), np.uint32)
    host_lib().synth_raw_blocks(out.ctypes.data, k, start, seed, stream)
    return out


# ---------------------------------------------------------------- device side

def _stream_handle(torch_stream) -> int:
    return int(torch_stream.cuda_stream)


def device_f32(t, seed: int, stream: int, std: float, start: int = 0, absval: bool = False, torch_stream=None):
    import torch
    assert t.dtype == torch.float32 and t.is_cuda and t.is_contiguous()
    s = torch_stream if torch_stream is not None else torch.cuda.current_stream(t.device)
    rc = gpu_lib().synth_gpu_fill_f32(t.data_ptr(), t.numel(), start, seed, stream, std, int(absval),
                                      _stream_handle(s))
    if rc != 0:
        raise RuntimeError(f"synth_gpu_fill_f32 failed: {rc}")
    return t


def device_bf16(t, seed: int, stream: int, std: float, start: int = 0, torch_stream=None):
    import torch
    assert t.dtype == torch.bfloat16 and t.is_cuda and t.is_contiguous()
    s = torch_stream if torch_stream is not None else torch.cuda.current_stream(t.device)
    rc = gpu_lib().synth_gpu_fill_bf16(t.data_ptr(), t.numel(), start, seed, stream, std, _stream_handle(s))
    if rc != 0:
        raise RuntimeError(f"synth_gpu_fill_bf16 failed: {rc}")
    return t


# ---------------------------------------------------------------- inf injection

def inject_positions(seed: int, run: int, M: int, n: int, rate: float, min_count: int = 1) -> list:
    """Seeded positions (rank, index) of +inf values planted into the M
    replicas of an n-element shard: a Poisson(rate * M * n) count (inverse
    CDF of one uniform), at least min_count, at uniform positions."""
    st = stream_id(KIND_INJECT, 0, run & 0xFFFF)
    blk = raw_blocks(1, seed, st, 0)[0]
    u = (int(blk[0]) | (int(blk[1]) << 32)) / 2.0**64
    lam = rate * M * n
    k, p = 0, math.exp(-lam)
    cdf = p
    while u > cdf and k < 10000:
        k += 1
        p *= lam / k
        cdf += p
    k = max(k, min_count)
    pos = raw_blocks(k, seed, st, 1)
    out = []
    for w in pos:
        x = (int(w[0]) | (int(w[1]) << 32)) % (M * n)
        out.append((x // n, x % n))
    return out
