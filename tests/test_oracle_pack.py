"""Pins for the oracle's bit-plane store (pack, read-back, bytes touched)."""
import json
import os

import numpy as np
import pytest

import oracle


def _slow_pack(codes):
    """Bit-by-bit packer written from the store's definition, for tiny inputs.

    Row tile of (t, i) starts at t*K*1024 + i*C_t; plane p (code bit 7-p) at
    +p*C_t/8; column 32w + 4m + j of the tile sits in word w at bit 8j + m,
    words little-endian.
    """
    K, N = codes.shape
    Np = -(-N // 128) * 128
    out = bytearray(K * Np)
    t0 = 0
    t = 0
    while t0 < Np:
        ct = min(1024, Np - t0)
        for i in range(K):
            for p in range(8):
                base = t * K * 1024 + i * ct + p * (ct // 8)
                for c in range(ct):
                    col = t0 + c
                    code = int(codes[i, col]) if col < N else 0
                    if (code >> (7 - p)) & 1:
                        w, r = divmod(c, 32)
                        m, j = divmod(r, 4)
                        bitpos = 8 * j + m
                        out[base + 4 * w + bitpos // 8] |= 1 << (bitpos % 8)
        t0 += ct
        t += 1
    return np.frombuffer(bytes(out), dtype=np.uint8)


def test_pack_golden(golden_dir):
    with open(os.path.join(golden_dir, "pack_two_rows.json")) as f:
        g = json.load(f)
    K, N = g["K"], g["N"]
    c = np.arange(N)
    codes = np.stack([c, 255 - c]).astype(np.uint8)
    want = np.frombuffer(bytes.fromhex("".join(g["planes_hex"])), dtype=np.uint8)
    got = oracle.pack(codes)
    assert got.shape == want.shape
    assert np.array_equal(got, want)


@pytest.mark.parametrize("K,N", [(1, 8), (3, 32), (2, 33), (5, 100), (2, 1056), (1, 2100), (4, 1024)])
def test_pack_matches_bitwise_loop(K, N):
    r = np.random.default_rng(K * 1000 + N)
    codes = r.integers(0, 256, size=(K, N), dtype=np.uint8)
    assert np.array_equal(oracle.pack(codes), _slow_pack(codes))


@pytest.mark.parametrize("K,N", [(7, 40), (130, 1090), (3, 3000)])
def test_read_planes_prefix(K, N):
    """The top b planes give q with its low 8 - b bits cleared (nesting)."""
    r = np.random.default_rng(N)
    codes = r.integers(0, 256, size=(K, N), dtype=np.uint8)
    planes = oracle.pack(codes)
    for b in range(9):
        bits = np.full(K, b, np.uint8)
        want = (codes.astype(np.int64) >> (8 - b)) << (8 - b) if b > 0 else np.zeros_like(codes)
        assert np.array_equal(oracle.read_planes(planes, K, N, bits), want.astype(np.uint8))
    mixed = r.integers(0, 9, size=K).astype(np.uint8)
    got = oracle.read_planes(planes, K, N, mixed)
    for i in range(K):
        b = int(mixed[i])
        want = (codes[i].astype(np.int64) >> (8 - b)) << (8 - b) if b else 0 * codes[i]
        assert np.array_equal(got[i], want)


def test_read_touches_only_the_span():
    """Bytes outside the top-b span of each row tile never change the result."""
    K, N = 6, 1100
    r = np.random.default_rng(1)
    codes = r.integers(0, 256, size=(K, N), dtype=np.uint8)
    planes = oracle.pack(codes)
    bits = np.array([0, 1, 3, 8, 2, 5], np.uint8)
    ref = oracle.read_planes(planes, K, N, bits)
    mask = np.zeros(planes.shape, bool)
    for t, (t0, ct) in enumerate(oracle.tiles(N)):
        for i in range(K):
            s = oracle.plane_offset(K, N, t, i, 0)
            mask[s:s + int(bits[i]) * ct // 8] = True
    assert int(mask.sum()) == oracle.span_bytes(K, N, bits)
    assert oracle.span_bytes(K, N, bits) == int(bits.astype(np.int64).sum()) * oracle.padded_cols(N) // 8
    noisy = planes.copy()
    noisy[~mask] = r.integers(0, 256, size=int((~mask).sum()), dtype=np.uint8)
    assert np.array_equal(oracle.read_planes(noisy, K, N, bits), ref)


def test_store_size_and_offsets():
    assert oracle.planes_bytes(4096, 14336) == 4096 * 14336
    assert oracle.planes_bytes(3, 33) == 3 * 128
    assert [ct for _, ct in oracle.tiles(2100)] == [1024, 1024, 128]
    assert [ct for _, ct in oracle.tiles(1400)] == [1024, 384]
    K = 10
    assert oracle.plane_offset(K, 2100, 2, 3, 5) == 2 * K * 1024 + 3 * 128 + 5 * 16
