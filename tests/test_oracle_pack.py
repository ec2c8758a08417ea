"""Pins for the oracle's bit-plane store (pack, read-back, bytes touched)."""
import json
import os

import numpy as np
import pytest

import oracle


def _slow_pack(codes, b_max=8):
    """Bit-by-bit packer written from the store's definition, for tiny inputs.

    Row tile of (t, i) starts at (t*K*1024 + i*C_t) * b_max/8; plane p (code
    bit b_max-1-p) at +p*C_t/8; column 32w + 4m + j of the tile sits in word w
    at bit 8j + m, words little-endian.
    """
    K, N = codes.shape
    Np = -(-N // 128) * 128
    out = bytearray(K * Np * b_max // 8)
    t0 = 0
    t = 0
    while t0 < Np:
        ct = min(1024, Np - t0)
        for i in range(K):
            for p in range(b_max):
                base = (t * K * 1024 + i * ct) * b_max // 8 + p * (ct // 8)
                for c in range(ct):
                    col = t0 + c
                    code = int(codes[i, col]) if col < N else 0
                    if (code >> (b_max - 1 - p)) & 1:
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


# ------------------------------------------------ b_max-bit stores (section 3.3, Appendix C.1)

@pytest.mark.parametrize("b_max", [1, 4, 6, 7])
@pytest.mark.parametrize("K,N", [(1, 8), (2, 33), (3, 1056), (1, 2100)])
def test_pack_bmax_matches_bitwise_loop(K, N, b_max):
    r = np.random.default_rng(K * 1000 + N + b_max)
    codes = r.integers(0, 1 << b_max, size=(K, N), dtype=np.uint8)
    got = oracle.pack(codes, b_max)
    assert got.shape == (oracle.planes_bytes(K, N, b_max),)
    assert np.array_equal(got, _slow_pack(codes, b_max))


@pytest.mark.parametrize("b_max", [4, 6])
def test_bmax_store_is_the_top_planes_of_the_eight_bit_store(b_max):
    """Row tile by row tile, a b_max-bit store equals the first b_max planes of
    the 8-bit store of q 2^(8 - b_max); the 8-bit store's other planes are 0."""
    K, N = 5, 2100
    r = np.random.default_rng(b_max)
    codes = r.integers(0, 1 << b_max, size=(K, N), dtype=np.uint8)
    small = oracle.pack(codes, b_max)
    eight = oracle.pack((codes.astype(np.int64) << (8 - b_max)).astype(np.uint8))
    for t, (t0, ct) in enumerate(oracle.tiles(N)):
        pb = ct // 8
        for i in range(K):
            s0 = oracle.plane_offset(K, N, t, i, 0, b_max)
            e0 = oracle.plane_offset(K, N, t, i, 0)
            assert np.array_equal(small[s0:s0 + b_max * pb], eight[e0:e0 + b_max * pb])
            assert not eight[e0 + b_max * pb:e0 + 8 * pb].any()


@pytest.mark.parametrize("b_max", [4, 6])
def test_read_planes_prefix_bmax(b_max):
    K, N = 9, 1200
    r = np.random.default_rng(10 + b_max)
    codes = r.integers(0, 1 << b_max, size=(K, N), dtype=np.uint8)
    planes = oracle.pack(codes, b_max)
    bits = r.integers(0, b_max + 1, size=K).astype(np.uint8)
    got = oracle.read_planes(planes, K, N, bits, b_max)
    sh = (b_max - bits.astype(np.int64))[:, None]
    want = ((codes.astype(np.int64) >> sh) << sh) * (bits[:, None] > 0)
    assert np.array_equal(got, want.astype(np.uint8))
    with pytest.raises(ValueError):
        oracle.read_planes(planes, K, N, np.full(K, b_max + 1, np.uint8), b_max)


def test_bmax_store_size_and_validation():
    assert oracle.planes_bytes(4096, 14336, 4) == 4096 * 14336 // 2
    assert oracle.planes_bytes(4096, 14336, 6) == 4096 * 14336 * 6 // 8
    assert oracle.planes_bytes(3, 33, 1) == 3 * 128 // 8
    K = 10
    assert oracle.plane_offset(K, 2100, 2, 3, 5, 6) == (2 * K * 1024 + 3 * 128) * 6 // 8 + 5 * 16
    with pytest.raises(ValueError):
        oracle.pack(np.array([[16]], np.uint8), 4)
    with pytest.raises(ValueError):
        oracle.planes_bytes(4, 4, 0)
    with pytest.raises(ValueError):
        oracle.planes_bytes(4, 4, 9)
