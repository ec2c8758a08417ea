"""GRINQH decode-stage VMM for AMD Instinct MI355X (gfx950).

Thin ctypes binding over ``libgrinqh.so`` (built from ``csrc/`` by
``python -m decode_stage_gemv_amd.build``).  Every step of the decode path runs
in the library's HIP kernels; this module only checks tensors and passes
device pointers, sizes and the current HIP stream.  PyTorch provides device
memory and streams.  There is no fallback: if the library is missing, every
call raises.

Names follow the C ABI in ``include/grinqh.h``:
``pack``, ``calibrate``, ``assign_bits``, ``vmm``, ``decode_vmm``,
``decode_vmm_noalloc``, ``decode_vmm_accumulate``, ``decode_vmm_lut``, ``prefill``, ``unpack_dense``,
``dense_gemm``, and ``timeline_read`` (measurement aid of the timeline build).
"""
from __future__ import annotations

import ctypes
import os
from typing import Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgrinqh.so")

GROUP = 128
TILE = 1024
MAX_THRESHOLDS = 8
MAX_BITS = 8

OK, EINVAL, EDEVICE, ENOSYS = 0, -1, -2, -3


class GrinqhError(RuntimeError):
    """A library call returned a non-zero status."""

    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn}: status {status}: {message}")
        self.status = status


_lib = None

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int
_sz = ctypes.c_size_t

_SIGNATURES = {
    "grinqh_layout_version": ([], _i32),
    "grinqh_status_string": ([_i32], ctypes.c_char_p),
    "grinqh_last_error": ([], ctypes.c_char_p),
    "grinqh_planes_bytes": ([_i64, _i64, _i32], _i64),
    "grinqh_workspace_bytes": ([_i64, _i64], _i64),
    "grinqh_workspace_init": ([_vp, _sz, _vp], _i32),
    "grinqh_pack": ([_vp, _i64, _i64, _i32, _vp, _vp], _i32),
    "grinqh_calibrate": ([_vp, _i64, _i64, _vp, _i32, _vp, _vp], _i32),
    "grinqh_assign_bits": ([_vp, _i64, _vp, _vp, _i32, _vp, _vp, _vp, _vp], _i32),
    "grinqh_vmm": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i32, _vp, _vp, _sz, _vp], _i32),
    "grinqh_decode_vmm": ([_vp, _vp, _vp, _vp, _i64, _i64, _i32, _vp, _vp, _i32, _vp, _vp, _sz, _vp], _i32),
    "grinqh_decode_vmm_accumulate": ([_vp, _vp, _vp, _vp, _i64, _i64, _i32, _vp, _vp, _i32, _vp, _vp, _vp],
                                     _i32),
    "grinqh_decode_vmm_accumulate_group": ([_i32, _vp, _vp, _vp, _vp, _i64, _vp, _i32, _vp, _vp, _vp, _vp, _vp,
                                            _vp], _i32),
    "grinqh_prefill": ([_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _vp, _vp], _i32),
    "grinqh_lut_entries": ([_i64, _i32], _i64),
    "grinqh_dense_bytes": ([_i64, _i64], _i64),
    "grinqh_unpack_dense": ([_vp, _vp, _vp, _i64, _i64, _i32, _vp, _sz, _vp], _i32),
    "grinqh_dense_gemm": ([_vp, _vp, _i64, _i64, _i64, _vp, _vp], _i32),
    "grinqh_decode_vmm_noalloc": ([_vp, _vp, _vp, _vp, _i64, _i64, _i32, _vp, _vp, _i32, _vp, _vp], _i32),
    "grinqh_decode_vmm_lut": ([_vp, _vp, _vp, _i64, _i64, _i32, _vp, _vp, _i32, _vp, _vp, _vp], _i32),
    "grinqh_timeline_read": ([_vp, _i64], _i32),
}

TIMELINE_LIB_PATH = os.path.join(HERE, "libgrinqh_timeline.so")
TIMELINE_WORKGROUPS = 8192
TIMELINE_SLOTS = 24


def use_library(path: str) -> None:
    """Load the library from `path` instead of ``libgrinqh.so`` (before the
    first call; bench.py uses it for the timeline build, TIMELINE_LIB_PATH)."""
    global LIB_PATH
    if _lib is not None and os.path.abspath(path) != os.path.abspath(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is already loaded")
    LIB_PATH = os.path.abspath(path)


def lib() -> ctypes.CDLL:
    """The loaded library (loaded on first use; raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m decode_stage_gemv_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = res
        _lib = handle
    return _lib


def _check(fn: str, status: int) -> None:
    if status != OK:
        raise GrinqhError(fn, status, lib().grinqh_last_error().decode())


def _stream(stream=None) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _dev(t, name, dtype, shape=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def layout_version() -> int:
    return lib().grinqh_layout_version()


def planes_bytes(K: int, N: int, b_max: int = MAX_BITS) -> int:
    n = lib().grinqh_planes_bytes(K, N, b_max)
    if n < 0:
        raise ValueError(f"no store for K = {K}, N = {N}, b_max = {b_max}")
    return n


def workspace_bytes(K: int, N: int) -> int:
    return lib().grinqh_workspace_bytes(K, N)


def n_groups(K: int) -> int:
    return (K + GROUP - 1) // GROUP


def make_workspace(K: int, N: int, device="cuda", stream=None):
    """Allocate and zero a workspace for K x N layers (one per concurrent stream)."""
    import torch
    nbytes = max(workspace_bytes(K, N), 4)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    _check("grinqh_workspace_init", lib().grinqh_workspace_init(ws.data_ptr(), nbytes, _stream(stream)))
    return ws


def pack(codes, out=None, stream=None, b_max: int = MAX_BITS):
    """b_max-bit codes u8 [K][N] (device) -> bit-plane store u8 [planes_bytes(K, N, b_max)]."""
    import torch
    _dev(codes, "codes", torch.uint8)
    K, N = codes.shape
    nbytes = planes_bytes(K, N, b_max)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=codes.device)
    _dev(out, "planes", torch.uint8, (nbytes,))
    _check("grinqh_pack", lib().grinqh_pack(codes.data_ptr(), K, N, b_max, out.data_ptr(), _stream(stream)))
    return out


def calibrate(calib, P: Sequence[float], out=None, stream=None):
    """fp16 calibration vectors [V][K] and target shares P -> fp32 thresholds [len(P) - 1]."""
    import torch
    _dev(calib, "calib", torch.float16)
    V, K = calib.shape
    n_levels = len(P)
    P_arr = (ctypes.c_double * max(n_levels, 1))(*[float(p) for p in P])
    if out is None:
        out = torch.empty(max(n_levels - 1, 0), dtype=torch.float32, device=calib.device)
    _dev(out, "thresholds", torch.float32, (max(n_levels - 1, 0),))
    _check("grinqh_calibrate", lib().grinqh_calibrate(calib.data_ptr(), V, K, ctypes.cast(P_arr, _vp),
                                                      n_levels, out.data_ptr() if out.numel() else None,
                                                      _stream(stream)))
    return out


def _host_thresholds(thresholds: Sequence[float], levels: Sequence[int]):
    n = len(thresholds)
    if len(levels) != n + 1:
        raise ValueError(f"need len(levels) == len(thresholds) + 1, got {len(levels)} and {n}")
    th = (ctypes.c_float * max(n, 1))(*[float(t) for t in thresholds])
    lv = (ctypes.c_uint8 * (n + 1))(*[int(v) for v in levels])
    return th, lv, n


def assign_bits(x, thresholds: Sequence[float], levels: Sequence[int], bits=None, active_idx=None,
                n_active=None, stream=None):
    """Per-row bit widths, ascending active-row list and its length (all on the device)."""
    import torch
    _dev(x, "x", torch.float16)
    K = x.numel()
    dev = x.device
    bits = torch.empty(K, dtype=torch.uint8, device=dev) if bits is None else bits
    active_idx = torch.empty(K, dtype=torch.int32, device=dev) if active_idx is None else active_idx
    n_active = torch.empty(1, dtype=torch.int32, device=dev) if n_active is None else n_active
    _dev(bits, "bits", torch.uint8, (K,))
    _dev(active_idx, "active_idx", torch.int32, (K,))
    _dev(n_active, "n_active", torch.int32, (1,))
    th, lv, n = _host_thresholds(thresholds, levels)
    _check("grinqh_assign_bits", lib().grinqh_assign_bits(
        x.data_ptr(), K, ctypes.cast(th, _vp), ctypes.cast(lv, _vp), n,
        bits.data_ptr(), active_idx.data_ptr(), n_active.data_ptr(), _stream(stream)))
    return bits, active_idx, n_active


def _check_layer(planes, scales, zeros, x, K, N, b_max):
    import torch
    _dev(planes, "planes", torch.uint8, (planes_bytes(K, N, b_max),))
    _dev(scales, "scales", torch.float16, (n_groups(K), N))
    _dev(zeros, "zeros", torch.float16, (n_groups(K), N))
    _dev(x, "x", torch.float16, (K,))


def vmm(planes, scales, zeros, x, bits, active_idx, n_active, K: int, N: int, workspace,
        out=None, stream=None, b_max: int = MAX_BITS):
    """y fp32 [N] from an explicit assignment (bits, active list, its length).

    active_idx must hold K entries (the kernel clamps the device-side count to
    [0, K] and may read any of them)."""
    import torch
    if not isinstance(active_idx, torch.Tensor) or active_idx.numel() < K:
        raise ValueError(f"active_idx must be a tensor of at least K = {K} entries")
    _check_layer(planes, scales, zeros, x, K, N, b_max)
    _dev(bits, "bits", torch.uint8, (K,))
    _dev(active_idx, "active_idx", torch.int32)
    _dev(n_active, "n_active", torch.int32, (1,))
    _dev(workspace, "workspace", torch.uint8)
    out = torch.empty(N, dtype=torch.float32, device=x.device) if out is None else out
    _dev(out, "y", torch.float32, (N,))
    _check("grinqh_vmm", lib().grinqh_vmm(
        planes.data_ptr(), scales.data_ptr(), zeros.data_ptr(), x.data_ptr(), bits.data_ptr(),
        active_idx.data_ptr(), n_active.data_ptr(), K, N, b_max, out.data_ptr(),
        workspace.data_ptr(), workspace.numel(), _stream(stream)))
    return out


def decode_vmm(planes, scales, zeros, x, K: int, N: int, thresholds: Sequence[float],
               levels: Sequence[int], workspace, out=None, stream=None, b_max: int = MAX_BITS):
    """The fused decode step: assignment and VMM in one launch; returns y fp32 [N]."""
    import torch
    _check_layer(planes, scales, zeros, x, K, N, b_max)
    _dev(workspace, "workspace", torch.uint8)
    out = torch.empty(N, dtype=torch.float32, device=x.device) if out is None else out
    _dev(out, "y", torch.float32, (N,))
    th, lv, n = _host_thresholds(thresholds, levels)
    _check("grinqh_decode_vmm", lib().grinqh_decode_vmm(
        planes.data_ptr(), scales.data_ptr(), zeros.data_ptr(), x.data_ptr(), K, N, b_max,
        ctypes.cast(th, _vp), ctypes.cast(lv, _vp), n, out.data_ptr(),
        workspace.data_ptr(), workspace.numel(), _stream(stream)))
    return out


def decode_vmm_noalloc(planes, scales, zeros, x, K: int, N: int, thresholds: Sequence[float],
                       levels: Sequence[int], out, stream=None, b_max: int = MAX_BITS):
    """grinqh_decode_vmm without a workspace: the library's own device array
    holds the split-K partials (the call allocates nothing; `out` is given)."""
    import torch
    _check_layer(planes, scales, zeros, x, K, N, b_max)
    _dev(out, "y", torch.float32, (N,))
    th, lv, n = _host_thresholds(thresholds, levels)
    _check("grinqh_decode_vmm_noalloc", lib().grinqh_decode_vmm_noalloc(
        planes.data_ptr(), scales.data_ptr(), zeros.data_ptr(), x.data_ptr(), K, N, b_max,
        ctypes.cast(th, _vp), ctypes.cast(lv, _vp), n, out.data_ptr(), _stream(stream)))
    return out


def decode_vmm_accumulate(planes, scales, zeros, x, K: int, N: int, thresholds: Sequence[float],
                          levels: Sequence[int], y, clear=None, stream=None, b_max: int = MAX_BITS):
    """y += the fused decode step's product (fp32 atomics, no workspace); zeroes `clear` if given."""
    import torch
    _check_layer(planes, scales, zeros, x, K, N, b_max)
    _dev(y, "y", torch.float32, (N,))
    if clear is not None:
        _dev(clear, "clear", torch.float32, (N,))
    th, lv, n = _host_thresholds(thresholds, levels)
    _check("grinqh_decode_vmm_accumulate", lib().grinqh_decode_vmm_accumulate(
        planes.data_ptr(), scales.data_ptr(), zeros.data_ptr(), x.data_ptr(), K, N, b_max,
        ctypes.cast(th, _vp), ctypes.cast(lv, _vp), n, y.data_ptr(),
        clear.data_ptr() if clear is not None else None, _stream(stream)))
    return y


MAX_GROUP = 4


def decode_vmm_accumulate_group(members, K: int, stream=None, b_max: int = MAX_BITS):
    """Several independent accumulating decode steps in one launch.

    members: up to MAX_GROUP tuples (planes, scales, zeros, x, N, thresholds,
    levels, y, clear) with clear None or a buffer to zero; every member's y
    gets += x W of its own layer (K rows each).
    """
    import torch
    count = len(members)
    if not 1 <= count <= MAX_GROUP:
        raise ValueError(f"{count} members, expected 1..{MAX_GROUP}")
    arr = lambda vals: (ctypes.c_void_p * count)(*vals)
    keep = []   # host threshold and level arrays must outlive the call
    for (planes, scales, zeros, x, N, thresholds, levels, y, clear) in members:
        _check_layer(planes, scales, zeros, x, K, N, b_max)
        _dev(y, "y", torch.float32, (N,))
        if clear is not None:
            _dev(clear, "clear", torch.float32, (N,))
        keep.append(_host_thresholds(thresholds, levels))
    Ns = (ctypes.c_int64 * count)(*[int(m[4]) for m in members])
    ns = (ctypes.c_int * count)(*[k[2] for k in keep])
    _check("grinqh_decode_vmm_accumulate_group", lib().grinqh_decode_vmm_accumulate_group(
        count, arr([m[0].data_ptr() for m in members]), arr([m[1].data_ptr() for m in members]),
        arr([m[2].data_ptr() for m in members]), arr([m[3].data_ptr() for m in members]), K, Ns, b_max,
        arr([ctypes.cast(k[0], _vp).value for k in keep]), arr([ctypes.cast(k[1], _vp).value for k in keep]), ns,
        arr([m[7].data_ptr() for m in members]),
        arr([m[8].data_ptr() if m[8] is not None else None for m in members]), _stream(stream)))
    return [m[7] for m in members]


def prefill(planes, scales, zeros, X, K: int, N: int, out=None, stream=None, b_max: int = MAX_BITS):
    """Dense prefill of a token batch: Y fp32 [M][N] = X fp16 [M][K] times the full-width weights."""
    import torch
    _dev(X, "X", torch.float16)
    if X.dim() != 2 or X.shape[1] != K:
        raise ValueError(f"X must be [M][{K}], got {tuple(X.shape)}")
    M = X.shape[0]
    _check_layer(planes, scales, zeros, X[0], K, N, b_max)
    out = torch.empty((M, N), dtype=torch.float32, device=X.device) if out is None else out
    _dev(out, "Y", torch.float32, (M, N))
    _check("grinqh_prefill", lib().grinqh_prefill(
        planes.data_ptr(), scales.data_ptr(), zeros.data_ptr(), X.data_ptr(), M, K, N, b_max,
        out.data_ptr(), _stream(stream)))
    return out


def lut_entries(N: int, b_max: int = MAX_BITS) -> int:
    n = lib().grinqh_lut_entries(N, b_max)
    if n < 0:
        raise ValueError(f"no table buffer for N = {N}, b_max = {b_max}")
    return n


def decode_vmm_lut(planes, lut, x, K: int, N: int, thresholds: Sequence[float], levels: Sequence[int], y,
                   clear=None, stream=None, b_max: int = MAX_BITS):
    """y += the decode step with table reconstruction (fp32 atomics); zeroes `clear` if given."""
    import torch
    _dev(planes, "planes", torch.uint8, (planes_bytes(K, N, b_max),))
    _dev(lut, "lut", torch.float16, (lut_entries(N, b_max),))
    _dev(x, "x", torch.float16, (K,))
    _dev(y, "y", torch.float32, (N,))
    if clear is not None:
        _dev(clear, "clear", torch.float32, (N,))
    th, lv, n = _host_thresholds(thresholds, levels)
    _check("grinqh_decode_vmm_lut", lib().grinqh_decode_vmm_lut(
        planes.data_ptr(), lut.data_ptr(), x.data_ptr(), K, N, b_max, ctypes.cast(th, _vp), ctypes.cast(lv, _vp),
        n, y.data_ptr(), clear.data_ptr() if clear is not None else None, _stream(stream)))
    return y


def dense_bytes(K: int, N: int) -> int:
    return lib().grinqh_dense_bytes(K, N)


def unpack_dense(planes, scales, zeros, K: int, N: int, out=None, stream=None, b_max: int = MAX_BITS):
    """The store at full width as dense fp16 weights in B-fragment order (u8 buffer)."""
    import torch
    _dev(planes, "planes", torch.uint8, (planes_bytes(K, N, b_max),))
    _dev(scales, "scales", torch.float16, (n_groups(K), N))
    _dev(zeros, "zeros", torch.float16, (n_groups(K), N))
    nbytes = dense_bytes(K, N)
    out = torch.empty(nbytes, dtype=torch.uint8, device=planes.device) if out is None else out
    _dev(out, "dense", torch.uint8)
    _check("grinqh_unpack_dense", lib().grinqh_unpack_dense(
        planes.data_ptr(), scales.data_ptr(), zeros.data_ptr(), K, N, b_max, out.data_ptr(), out.numel(),
        _stream(stream)))
    return out


def dense_gemm(X, dense, K: int, N: int, out=None, stream=None):
    """Y fp32 [M][N] = X fp16 [M][K] times the unpacked weights in `dense`."""
    import torch
    _dev(X, "X", torch.float16)
    if X.dim() != 2 or X.shape[1] != K:
        raise ValueError(f"X must be [M][{K}], got {tuple(X.shape)}")
    M = X.shape[0]
    _dev(dense, "dense", torch.uint8)
    if dense.numel() < dense_bytes(K, N):
        raise ValueError("dense buffer too small")
    out = torch.empty((M, N), dtype=torch.float32, device=X.device) if out is None else out
    _dev(out, "Y", torch.float32, (M, N))
    _check("grinqh_dense_gemm", lib().grinqh_dense_gemm(X.data_ptr(), dense.data_ptr(), M, K, N, out.data_ptr(),
                                                        _stream(stream)))
    return out


def timeline_read(count: int = TIMELINE_WORKGROUPS * TIMELINE_SLOTS):
    """The timeline build's clock stamps (see grinqh_timeline_read): a numpy
    uint64 array of `count` stamps, workgroup-major, TIMELINE_SLOTS per
    workgroup.  Raises GrinqhError (ENOSYS) with the ordinary library."""
    import numpy as np
    out = np.zeros(count, dtype=np.uint64)
    _check("grinqh_timeline_read", lib().grinqh_timeline_read(out.ctypes.data, count))
    return out
