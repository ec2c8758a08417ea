"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments on the host (these calls return before any HIP call)."""
import ctypes
import os
import re

import pytest

import decode_stage_gemv_amd as g

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "grinqh.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(grinqh_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(g.LIB_PATH):
        pytest.fail("libgrinqh.so is not built (run python -m decode_stage_gemv_amd.build)")
    return g.lib()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) == 21
    for name in names:
        assert hasattr(lib, name), name
        assert name in g._SIGNATURES, name


def test_static_queries(lib):
    assert lib.grinqh_layout_version() == 4
    assert lib.grinqh_status_string(0) == b"ok"
    assert lib.grinqh_status_string(-1) == b"invalid argument"
    assert lib.grinqh_status_string(-2) == b"device error"
    assert lib.grinqh_status_string(-3) == b"not implemented"
    assert lib.grinqh_status_string(7) == b"unknown status"
    assert lib.grinqh_planes_bytes(4096, 14336, 8) == 4096 * 14336
    assert lib.grinqh_planes_bytes(4096, 14336, 6) == 4096 * 14336 * 6 // 8
    assert lib.grinqh_planes_bytes(4096, 14336, 4) == 4096 * 14336 // 2
    assert lib.grinqh_planes_bytes(3, 33, 8) == 3 * 128
    assert lib.grinqh_planes_bytes(3, 33, 1) == 3 * 16
    assert lib.grinqh_planes_bytes(0, 5, 8) == -1
    assert lib.grinqh_planes_bytes(4, 5, 0) == -1
    assert lib.grinqh_planes_bytes(4, 5, 9) == -1
    assert lib.grinqh_workspace_bytes(-1, 5) == -1
    assert lib.grinqh_workspace_bytes(128, 4096) >= 0
    assert lib.grinqh_workspace_bytes(4096, 14336) >= 4 * 14336


FAKE = 0x1000   # never dereferenced: every call below fails validation first


def _err(lib):
    return lib.grinqh_last_error().decode()


def test_pack_validation(lib):
    assert lib.grinqh_pack(None, 4, 4, 8, FAKE, None) == g.EINVAL
    assert lib.grinqh_pack(FAKE, 0, 4, 8, FAKE, None) == g.EINVAL
    assert "positive" in _err(lib)
    assert lib.grinqh_pack(FAKE, 4, -3, 8, FAKE, None) == g.EINVAL
    assert lib.grinqh_pack(FAKE, 4, 4, 0, FAKE, None) == g.EINVAL and "b_max" in _err(lib)
    assert lib.grinqh_pack(FAKE, 4, 4, 9, FAKE, None) == g.EINVAL


def test_assign_validation(lib):
    th = (ctypes.c_float * 4)(0.5, 1.0, 2.0, 4.0)
    lv = (ctypes.c_uint8 * 5)(0, 2, 3, 4, 8)
    args = lambda t, l, n, K=16: lib.grinqh_assign_bits(FAKE, K, ctypes.cast(t, ctypes.c_void_p),
                                                        ctypes.cast(l, ctypes.c_void_p), n, FAKE, FAKE, FAKE, None)
    assert args(th, lv, 9) == g.EINVAL
    assert args(th, lv, -1) == g.EINVAL
    assert args(th, lv, 4, K=0) == g.EINVAL
    bad = (ctypes.c_float * 4)(0.5, 0.25, 2.0, 4.0)
    assert args(bad, lv, 4) == g.EINVAL and "decrease" in _err(lib)
    nan = (ctypes.c_float * 4)(float("nan"), 1.0, 2.0, 4.0)
    assert args(nan, lv, 4) == g.EINVAL
    neg = (ctypes.c_float * 4)(-1.0, 1.0, 2.0, 4.0)
    assert args(neg, lv, 4) == g.EINVAL
    badlv = (ctypes.c_uint8 * 5)(0, 2, 3, 9, 8)
    assert args(th, badlv, 4) == g.EINVAL and "level" in _err(lib)
    assert lib.grinqh_assign_bits(FAKE, 16, ctypes.cast(th, ctypes.c_void_p), ctypes.cast(lv, ctypes.c_void_p),
                                  4, None, FAKE, FAKE, None) == g.EINVAL


def test_vmm_validation(lib):
    need = lib.grinqh_workspace_bytes(4096, 4096)
    assert need > 0
    r = lib.grinqh_vmm(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4096, 4096, 8, FAKE, FAKE, need - 1, None)
    assert r == g.EINVAL and "workspace" in _err(lib)
    r = lib.grinqh_vmm(FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, 4096, 4096, 8, FAKE, FAKE, need, None)
    assert r == g.EINVAL
    r = lib.grinqh_vmm(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4096, 4096, 8, FAKE, FAKE, need, None)
    assert r == g.EINVAL
    r = lib.grinqh_vmm(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4096, 4096, 0, FAKE, FAKE, need, None)
    assert r == g.EINVAL and "b_max" in _err(lib)
    th = (ctypes.c_float * 1)(1.0)
    thp = ctypes.cast(th, ctypes.c_void_p)
    lv = (ctypes.c_uint8 * 2)(0, 12)
    r = lib.grinqh_decode_vmm(FAKE, FAKE, FAKE, FAKE, 4096, 4096, 8, thp,
                              ctypes.cast(lv, ctypes.c_void_p), 1, FAKE, FAKE, need, None)
    assert r == g.EINVAL
    lv8 = (ctypes.c_uint8 * 2)(0, 8)
    r = lib.grinqh_decode_vmm(FAKE, FAKE, FAKE, FAKE, 0, 4096, 8, thp,
                              ctypes.cast(lv8, ctypes.c_void_p), 1, FAKE, FAKE, need, None)
    assert r == g.EINVAL
    # a level above the store's b_max is rejected
    lv6 = (ctypes.c_uint8 * 2)(0, 6)
    r = lib.grinqh_decode_vmm(FAKE, FAKE, FAKE, FAKE, 4096, 4096, 4, thp,
                              ctypes.cast(lv6, ctypes.c_void_p), 1, FAKE, FAKE, need, None)
    assert r == g.EINVAL and "level" in _err(lib)
    r = lib.grinqh_decode_vmm(FAKE, FAKE, FAKE, FAKE, 4096, 4096, 9, thp,
                              ctypes.cast(lv8, ctypes.c_void_p), 1, FAKE, FAKE, need, None)
    assert r == g.EINVAL and "b_max" in _err(lib)


def test_accumulate_validation(lib):
    th = (ctypes.c_float * 1)(1.0)
    lv = (ctypes.c_uint8 * 2)(0, 8)
    thp, lvp = ctypes.cast(th, ctypes.c_void_p), ctypes.cast(lv, ctypes.c_void_p)
    y = 0x100000
    # clear overlapping y is rejected; clear == NULL is allowed (fails later only on bad args)
    r = lib.grinqh_decode_vmm_accumulate(FAKE, FAKE, FAKE, FAKE, 128, 64, 8, thp, lvp, 1, y, y + 128, None)
    assert r == g.EINVAL and "overlap" in _err(lib)
    # so is clear overlapping x (K = 128 halves from FAKE): it is zeroed while x is read
    r = lib.grinqh_decode_vmm_accumulate(FAKE, FAKE, FAKE, FAKE, 128, 64, 8, thp, lvp, 1, y, FAKE + 200, None)
    assert r == g.EINVAL and "overlaps x" in _err(lib)
    r = lib.grinqh_decode_vmm_accumulate(FAKE, FAKE, FAKE, FAKE, 128, 64, 8, thp, lvp, 1, None, None, None)
    assert r == g.EINVAL
    r = lib.grinqh_decode_vmm_accumulate(FAKE, FAKE, FAKE, FAKE, 128, 64, 8, thp, lvp, -2, y, None, None)
    assert r == g.EINVAL
    r = lib.grinqh_decode_vmm_accumulate(FAKE, FAKE, FAKE, FAKE, 128, 64, 6, thp, lvp, 1, y, None, None)
    assert r == g.EINVAL and "level" in _err(lib)


def test_calibrate_validation(lib):
    P = (ctypes.c_double * 3)(0.3, 0.2, 0.5)
    Pp = ctypes.cast(P, ctypes.c_void_p)
    assert lib.grinqh_calibrate(FAKE, 0, 16, Pp, 3, FAKE, None) == g.EINVAL
    assert lib.grinqh_calibrate(FAKE, 4, 16, Pp, 10, FAKE, None) == g.EINVAL
    assert lib.grinqh_calibrate(FAKE, 4, 16, Pp, 0, FAKE, None) == g.EINVAL
    neg = (ctypes.c_double * 3)(0.3, -0.2, 0.5)
    assert lib.grinqh_calibrate(FAKE, 4, 16, ctypes.cast(neg, ctypes.c_void_p), 3, FAKE, None) == g.EINVAL
    # one level: no thresholds to compute, nothing enqueued
    assert lib.grinqh_calibrate(FAKE, 4, 16, Pp, 1, None, None) == g.OK


def test_workspace_init_validation(lib):
    assert lib.grinqh_workspace_init(None, 16, None) == g.EINVAL
    assert lib.grinqh_workspace_init(None, 0, None) == g.OK


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(g, "_lib", None)
    monkeypatch.setattr(g, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        g.lib()


def test_prefill_validation(lib):
    assert lib.grinqh_prefill(None, FAKE, FAKE, FAKE, 4, 128, 64, 8, FAKE, None) == g.EINVAL
    assert lib.grinqh_prefill(FAKE, FAKE, FAKE, FAKE, 0, 128, 64, 8, FAKE, None) == g.EINVAL
    assert "M" in _err(lib)
    assert lib.grinqh_prefill(FAKE, FAKE, FAKE, FAKE, 4, 0, 64, 8, FAKE, None) == g.EINVAL
    assert lib.grinqh_prefill(FAKE, FAKE, FAKE, FAKE, 4, 128, 64, 9, FAKE, None) == g.EINVAL
    assert lib.grinqh_prefill(FAKE, FAKE, FAKE, FAKE, 4, 1 << 21, 64, 8, FAKE, None) == g.EINVAL


def test_unpacked_prefill_validation(lib):
    assert lib.grinqh_dense_bytes(4096, 14336) == 512 * 14336 * 16
    assert lib.grinqh_dense_bytes(9, 33) == 64 * 128 * 2       # rows padded to 64, columns to 128
    assert lib.grinqh_dense_bytes(0, 4) == -1
    need = lib.grinqh_dense_bytes(64, 64)
    assert lib.grinqh_unpack_dense(FAKE, FAKE, FAKE, 64, 64, 8, FAKE, need - 1, None) == g.EINVAL
    assert lib.grinqh_unpack_dense(FAKE, FAKE, FAKE, 64, 64, 8, FAKE + 8, need, None) == g.EINVAL
    assert "aligned" in _err(lib)
    assert lib.grinqh_unpack_dense(FAKE, FAKE, FAKE, 64, 64, 0, FAKE, need, None) == g.EINVAL
    assert lib.grinqh_dense_gemm(FAKE, FAKE, 0, 64, 64, FAKE, None) == g.EINVAL
    assert lib.grinqh_dense_gemm(FAKE, FAKE, 4, 1 << 21, 64, FAKE, None) == g.EINVAL
    assert lib.grinqh_dense_gemm(None, FAKE, 4, 64, 64, FAKE, None) == g.EINVAL
    assert lib.grinqh_dense_gemm(FAKE, FAKE + 8, 4, 64, 64, FAKE, None) == g.EINVAL   # weights read 16 bytes at a time
    assert "aligned" in _err(lib)
    assert lib.grinqh_dense_gemm(FAKE, FAKE, 0, 64, 64, FAKE, None) == g.EINVAL       # an empty batch


def test_lut_validation(lib):
    assert lib.grinqh_lut_entries(14336, 8) == 14336 * 510
    assert lib.grinqh_lut_entries(100, 4) == 100 * 30
    assert lib.grinqh_lut_entries(0, 8) == -1 and lib.grinqh_lut_entries(64, 9) == -1
    th = (ctypes.c_float * 1)(1.0)
    lv = (ctypes.c_uint8 * 2)(0, 8)
    thp, lvp = ctypes.cast(th, ctypes.c_void_p), ctypes.cast(lv, ctypes.c_void_p)
    y = 0x100000
    r = lib.grinqh_decode_vmm_lut(FAKE, None, FAKE, 128, 64, 8, thp, lvp, 1, y, None, None)
    assert r == g.EINVAL
    r = lib.grinqh_decode_vmm_lut(FAKE, FAKE, FAKE, 128, 64, 8, thp, lvp, 1, y, y + 64, None)
    assert r == g.EINVAL and "overlap" in _err(lib)
    r = lib.grinqh_decode_vmm_lut(FAKE, FAKE, FAKE, 128, 64, 8, thp, lvp, 1, y, FAKE - 16, None)
    assert r == g.EINVAL and "overlaps x" in _err(lib)
    r = lib.grinqh_decode_vmm_lut(FAKE, FAKE + 2, FAKE, 128, 64, 8, thp, lvp, 1, y, None, None)
    assert r == g.EINVAL and "aligned" in _err(lib)
    r = lib.grinqh_decode_vmm_lut(FAKE, FAKE, FAKE, 128, 64, 4, thp, lvp, 1, y, None, None)
    assert r == g.EINVAL and "level" in _err(lib)


def test_list_vmm_binding_requires_a_full_length_list():
    """The list entry point's kernel clamps the device-side count to [0, K]
    and may read any of the first K list entries, so the binding refuses a
    list buffer shorter than K before touching the device."""
    import torch
    import decode_stage_gemv_amd as grq
    K, N = 256, 64
    short = torch.zeros(K - 1, dtype=torch.int32)
    with pytest.raises(ValueError, match="active_idx"):
        grq.vmm(None, None, None, None, None, short, None, K, N, None)
    with pytest.raises(ValueError, match="active_idx"):
        grq.vmm(None, None, None, None, None, [0] * K, None, K, N, None)


def test_noalloc_validation(lib):
    """The allocation-free entry point checks its arguments, and rejects a
    layer whose split-K partials exceed its fixed device array, before any
    HIP call (the pointers below are never dereferenced)."""
    th = (ctypes.c_float * 2)(0.5, 1.0)
    lv = (ctypes.c_uint8 * 3)(0, 2, 8)
    p = ctypes.c_void_p(4096)
    f = lib.grinqh_decode_vmm_noalloc
    assert f(None, p, p, p, 256, 256, 8, th, lv, 2, p, None) == g.EINVAL
    assert f(p, p, p, p, 0, 256, 8, th, lv, 2, p, None) == g.EINVAL
    assert f(p, p, p, p, 256, 256, 9, th, lv, 2, p, None) == g.EINVAL
    lv_hi = (ctypes.c_uint8 * 3)(0, 2, 8)
    assert f(p, p, p, p, 256, 256, 4, th, lv_hi, 2, p, None) == g.EINVAL     # level above b_max
    # 65536 x 65536: 64 row splits x 65536 fp32 partials = 16 MiB, more than
    # the array holds next to its tile counters
    assert f(p, p, p, p, 65536, 65536, 8, th, lv, 2, p, None) == g.EINVAL
    assert b"allocation-free" in lib.grinqh_last_error()
    assert g.lib().grinqh_workspace_bytes(65536, 65536) > (16 << 20)
    # 2048 x 300032: few partial bytes (two splits) but more columns than the
    # array's column words cover (262144)
    assert f(p, p, p, p, 2048, 300032, 8, th, lv, 2, p, None) == g.EINVAL
    assert b"padded columns" in lib.grinqh_last_error()


def test_group_validation(lib):
    """The grouped entry point checks the member count, its host arrays, each
    member as the single-layer call would, and clear buffers against every
    member's output, before any HIP call (pointers are never dereferenced)."""
    f = lib.grinqh_decode_vmm_accumulate_group
    P = ctypes.c_void_p

    def arr(*v):
        return (ctypes.c_void_p * len(v))(*v)

    th = (ctypes.c_float * 2)(0.5, 1.0)
    lv = (ctypes.c_uint8 * 3)(0, 2, 8)
    a = 1 << 20
    planes, sc, zr, xx = arr(a, a), arr(a, a), arr(a, a), arr(a, a)
    N = (ctypes.c_int64 * 2)(256, 512)
    ths = arr(ctypes.cast(th, P).value, ctypes.cast(th, P).value)
    lvs = arr(ctypes.cast(lv, P).value, ctypes.cast(lv, P).value)
    ns = (ctypes.c_int * 2)(2, 2)
    y = arr(1 << 24, 2 << 24)
    assert f(0, planes, sc, zr, xx, 256, N, 8, ths, lvs, ns, y, None, None) == g.EINVAL
    assert f(5, planes, sc, zr, xx, 256, N, 8, ths, lvs, ns, y, None, None) == g.EINVAL
    assert f(2, None, sc, zr, xx, 256, N, 8, ths, lvs, ns, y, None, None) == g.EINVAL
    assert f(2, planes, sc, zr, xx, 256, None, 8, ths, lvs, ns, y, None, None) == g.EINVAL
    bad_n = (ctypes.c_int64 * 2)(256, 0)
    assert f(2, planes, sc, zr, xx, 256, bad_n, 8, ths, lvs, ns, y, None, None) == g.EINVAL
    assert b"member 1" in lib.grinqh_last_error()
    lv9 = (ctypes.c_uint8 * 3)(0, 2, 9)
    lvs_bad = arr(ctypes.cast(lv, P).value, ctypes.cast(lv9, P).value)
    assert f(2, planes, sc, zr, xx, 256, N, 8, ths, lvs_bad, ns, y, None, None) == g.EINVAL
    assert b"member 1" in lib.grinqh_last_error()
    # member 0's clear buffer overlapping member 1's y (2 << 24 .. + 2 KiB)
    clear = arr((2 << 24) + 512, None)
    assert f(2, planes, sc, zr, xx, 256, N, 8, ths, lvs, ns, y, clear, None) == g.EINVAL
    assert b"overlaps" in lib.grinqh_last_error()
    # member 1's clear buffer overlapping the members' x (1 << 20 .. + 512 bytes)
    clear = arr(None, a + 256)
    assert f(2, planes, sc, zr, xx, 256, N, 8, ths, lvs, ns, y, clear, None) == g.EINVAL
    assert b"clear overlaps the x" in lib.grinqh_last_error()


def test_timeline_reader_needs_the_timeline_build(lib):
    """The ordinary library has no clock stamps: the reader says so (ENOSYS)
    without touching the device."""
    buf = (ctypes.c_uint64 * 4)()
    assert lib.grinqh_timeline_read(ctypes.addressof(buf), 4) == g.ENOSYS
    assert "without the timeline" in _err(lib)


def test_timeline_build_exports_the_same_symbols_and_checks_arguments():
    """The timeline build exports every declared call too, and its reader
    rejects bad arguments on the host (a zero count copies nothing)."""
    if not os.path.exists(g.TIMELINE_LIB_PATH):
        pytest.fail("libgrinqh_timeline.so is not built (python -m decode_stage_gemv_amd.build --timeline)")
    tl = ctypes.CDLL(g.TIMELINE_LIB_PATH)
    for name in declared_functions():
        assert hasattr(tl, name), name
    tl.grinqh_timeline_read.argtypes = [ctypes.c_void_p, ctypes.c_int64]
    tl.grinqh_timeline_read.restype = ctypes.c_int
    tl.grinqh_last_error.restype = ctypes.c_char_p
    buf = (ctypes.c_uint64 * 4)()
    assert tl.grinqh_timeline_read(None, 4) == g.EINVAL
    assert tl.grinqh_timeline_read(ctypes.addressof(buf), -1) == g.EINVAL
    assert tl.grinqh_timeline_read(ctypes.addressof(buf), g.TIMELINE_WORKGROUPS * g.TIMELINE_SLOTS + 1) == g.EINVAL
    assert tl.grinqh_timeline_read(ctypes.addressof(buf), 0) == g.OK
