"""Pins for the oracle's reconstruction and vector-matrix multiply."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synthetic
from oracle import grinqh_oracle


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def test_vmm_golden_small(golden_dir):
    g = _load(golden_dir, "vmm_small.json")
    y = oracle.vmm(np.array(g["codes"], np.uint8), np.array(g["scales"], np.float16),
                   np.array(g["zeros"], np.float16), np.array(g["x"], np.float16),
                   np.array(g["bits"], np.uint8))
    assert y.tolist() == g["y"]          # every term is exact in fp64


def test_vmm_golden_two_groups(golden_dir):
    g = _load(golden_dir, "vmm_two_groups.json")
    K, N = g["K"], g["N"]
    codes = np.zeros((K, N), np.uint8)
    x = np.zeros(K, np.float16)
    bits = np.zeros(K, np.uint8)
    for i, (b, q, xv) in g["active"].items():
        codes[int(i)] = q
        x[int(i)] = xv
        bits[int(i)] = b
    y = oracle.vmm(codes, np.array(g["scales"], np.float16), np.array(g["zeros"], np.float16), x, bits)
    assert y.tolist() == g["y"]


def test_vmm_golden_bmax4(golden_dir):
    g = _load(golden_dir, "vmm_bmax4.json")
    y = oracle.vmm(np.array(g["codes"], np.uint8), np.array(g["scales"], np.float16),
                   np.array(g["zeros"], np.float16), np.array(g["x"], np.float16),
                   np.array(g["bits"], np.uint8), b_max=g["b_max"])
    assert y.tolist() == g["y"]


def _rand_case(K, N, seed, b_max=8):
    r = np.random.default_rng(seed)
    codes = r.integers(0, 1 << b_max, size=(K, N), dtype=np.uint8)
    G = -(-K // 128)
    scales = (r.random((G, N)) * 0.01 + 1e-4).astype(np.float16)
    zeros = (r.standard_normal((G, N)) * 0.05).astype(np.float16)
    x = (r.standard_normal(K) * 2).astype(np.float16)
    return codes, scales, zeros, x


@pytest.mark.parametrize("K,N", [(256, 256), (300, 70), (1, 5)])
def test_all_eight_bits_is_dense_gemv(K, N):
    """b_i = 8 everywhere: nothing truncated, y = x @ (s q + z) (textbook GEMV)."""
    codes, scales, zeros, x = _rand_case(K, N, K + N)
    g = np.arange(K) // 128
    W = scales[g].astype(np.float64) * codes.astype(np.float64) + zeros[g].astype(np.float64)
    want = x.astype(np.float64) @ W
    got = oracle.vmm(codes, scales, zeros, x, np.full(K, 8, np.uint8))
    scale = np.abs(x.astype(np.float64)) @ np.abs(W)
    assert np.all(np.abs(got - want) <= 1e-12 * scale + 1e-300)


def test_all_zero_bits_is_zero():
    codes, scales, zeros, x = _rand_case(200, 40, 3)
    assert np.array_equal(oracle.vmm(codes, scales, zeros, x, np.zeros(200, np.uint8)), np.zeros(40))


def _fraction_vmm(codes, scales, zeros, x, bits, b_max=8):
    """Exact rational evaluation of section 3.3 with integer bit slicing.

    q_b = q >> (b_max - b) keeps the b most significant of the b_max code
    bits; w_hat = s (q_b << (b_max - b) + phi) + z with phi = 2^(b_max - b - 1)
    for b < b_max, 0 at b = b_max.
    """
    K, N = codes.shape
    y = [Fraction(0)] * N
    for i in range(K):
        b = int(bits[i])
        if b == 0:
            continue
        g = i // 128
        xi = Fraction(float(x[i]))
        for j in range(N):
            qb = int(codes[i, j]) >> (b_max - b)
            phi = (1 << (b_max - 1 - b)) if b < b_max else 0
            w = Fraction(float(scales[g, j])) * ((qb << (b_max - b)) + phi) + Fraction(float(zeros[g, j]))
            y[j] += xi * w
    return y


def _check_exact(codes, scales, zeros, x, bits, b_max=8):
    want = _fraction_vmm(codes, scales, zeros, x, bits, b_max)
    got = oracle.vmm(codes, scales, zeros, x, bits, b_max=b_max)
    mag = oracle.vmm_abs(codes, scales, zeros, x, bits, b_max=b_max)
    for j in range(codes.shape[1]):
        assert abs(Fraction(float(got[j])) - want[j]) <= Fraction(1e-12) * Fraction(float(mag[j])) + Fraction(1e-300)


def test_brute_force_8x8_uniform_bits():
    codes, scales, zeros, x = _rand_case(8, 8, 11)
    for b in range(9):
        _check_exact(codes, scales, zeros, x, np.full(8, b, np.uint8))


def test_brute_force_8x8_random_bits():
    r = np.random.default_rng(12)
    for trial in range(300):
        codes, scales, zeros, x = _rand_case(8, 8, 100 + trial)
        bits = r.integers(0, 9, size=8).astype(np.uint8)
        _check_exact(codes, scales, zeros, x, bits)


def test_brute_force_tie_codes():
    """Codes on truncation boundaries (all-ones / all-zeros low bits)."""
    codes = np.array([[0, 255, 128, 127, 64, 63, 1, 254]] * 8, np.uint8)
    _, scales, zeros, x = _rand_case(8, 8, 5)
    for b in range(9):
        _check_exact(codes, scales, zeros, x, np.full(8, b, np.uint8))


def test_one_hot_input_selects_one_row():
    K, N = 260, 33
    codes, scales, zeros, _ = _rand_case(K, N, 21)
    for i, b in [(0, 8), (129, 3), (259, 1), (77, 5)]:
        x = np.zeros(K, np.float16)
        x[i] = 1.5
        bits = np.zeros(K, np.uint8)
        bits[i] = b
        g = i // 128
        step = 2 ** (8 - b)
        r = (codes[i].astype(np.int64) // step) * step + (step // 2 if b < 8 else 0)
        want = 1.5 * (scales[g].astype(np.float64) * r + zeros[g].astype(np.float64))
        assert np.allclose(oracle.vmm(codes, scales, zeros, x, bits), want, rtol=1e-15, atol=0)


def test_nesting_invariance():
    """Low 8 - b bits of a row's codes are never read: flipping them changes nothing."""
    K, N = 300, 50
    codes, scales, zeros, x = _rand_case(K, N, 31)
    r = np.random.default_rng(32)
    bits = r.integers(0, 9, size=K).astype(np.uint8)
    y0 = oracle.vmm(codes, scales, zeros, x, bits)
    low = ((1 << (8 - bits.astype(np.int64))) - 1)[:, None]
    noise = r.integers(0, 256, size=(K, N))
    flipped = (codes.astype(np.int64) ^ (noise & low)).astype(np.uint8)
    assert np.array_equal(oracle.vmm(flipped, scales, zeros, x, bits), y0)


def test_reconstruction_half_bin_bound():
    """r sits in the middle of the code bin the truncated prefix names."""
    q = np.arange(256)
    for b in range(1, 9):
        r = oracle.reconstruct_level(q, b)
        step = 2 ** (8 - b)
        lo = (q // step) * step
        assert np.all(r >= lo) and np.all(r < lo + step)
        assert np.all(np.abs(r - q) <= (step // 2 if b < 8 else 0))
        if b < 8:
            assert np.all(r - lo == step // 2)


def test_linearity_in_x():
    K, N = 200, 20
    codes, scales, zeros, x = _rand_case(K, N, 41)
    bits = np.random.default_rng(42).integers(0, 9, size=K).astype(np.uint8)
    x2 = (np.random.default_rng(43).standard_normal(K)).astype(np.float16)
    s = (x.astype(np.float64) + x2.astype(np.float64))
    s16 = s.astype(np.float16)
    exact = s16.astype(np.float64) == s       # only where the sum is exact in fp16
    xs = np.where(exact, s16, np.float16(0))
    xa = np.where(exact, x, np.float16(0))
    xb = np.where(exact, x2, np.float16(0))
    ya = oracle.vmm(codes, scales, zeros, xa, bits)
    yb = oracle.vmm(codes, scales, zeros, xb, bits)
    ys = oracle.vmm(codes, scales, zeros, xs, bits)
    mag = oracle.vmm_abs(codes, scales, zeros, xa, bits) + oracle.vmm_abs(codes, scales, zeros, xb, bits)
    assert np.all(np.abs(ys - ya - yb) <= 1e-12 * mag)


def test_vmm_reads_through_the_store():
    """The VMM of codes equals the VMM of what the store returns for each row."""
    lay = synthetic.make_layer(300, 1100, config=0, matrix=5)
    x = lay.x[0]
    th = oracle.calibrate(lay.calib, synthetic.P_TINY)
    bits = oracle.assign(x, th, synthetic.LEVELS_5)
    seen = oracle.read_planes(oracle.pack(lay.codes), 300, 1100, bits)
    y1 = oracle.vmm(lay.codes, lay.scales, lay.zeros, x, bits)
    y2 = oracle.vmm(seen, lay.scales, lay.zeros, x, bits)
    assert np.array_equal(y1, y2)


def test_bytes_read_accounting():
    K, N = 300, 100
    bits = np.zeros(K, np.uint8)
    bits[[0, 5, 290]] = [8, 3, 2]
    br = oracle.bytes_read(bits, K, N)
    assert br["planes"] == 13 * 128 // 8
    assert br["scales"] == 4 * N * 2        # groups 0 and 2 are active, group 1 is not
    assert br["x"] == 2 * K
    assert br["total"] == br["planes"] + br["scales"] + br["x"]
    assert br["avg_bits"] == pytest.approx(13 / 300)


# ------------------------------------------------ the pins catch planted mistakes

def test_planted_mistakes_are_caught(monkeypatch, golden_dir):
    """Plant plausible mistakes in the oracle and check a pin fails for each:
    a dropped or sign-flipped midpoint, an off-by-one width, a dropped zero
    term, a transposed weight operand and a wrong group size."""
    codes, scales, zeros, x = _rand_case(8, 8, 77)
    bits = np.array([1, 2, 3, 4, 5, 6, 7, 8], np.uint8)
    good = grinqh_oracle.reconstruct_level
    good_rows = grinqh_oracle._dequant_rows

    def no_phi(q, b, b_max=8):
        step = float(2 ** (b_max - b))
        return np.floor(np.asarray(q, np.float64) / step) * step

    def minus_phi(q, b, b_max=8):
        return 2 * no_phi(q, b, b_max) - good(q, b, b_max) if 0 < b < b_max else good(q, b, b_max)

    def off_by_one_shift(q, b, b_max=8):
        return good(q, min(b + 1, b_max), b_max)

    for bad in (no_phi, minus_phi, off_by_one_shift):
        monkeypatch.setattr(grinqh_oracle, "reconstruct_level", bad)
        with pytest.raises(AssertionError):
            _check_exact(codes, scales, zeros, x, bits)
    monkeypatch.setattr(grinqh_oracle, "reconstruct_level", good)

    # b_max < 8: a midpoint in 8-bit code units, or one added at b = b_max
    codes4, scales4, zeros4, x4 = _rand_case(8, 8, 78, b_max=4)
    bits4 = np.array([1, 2, 3, 4, 4, 3, 2, 1], np.uint8)

    def eight_bit_phi(q, b, b_max=8):
        return no_phi(q, b, b_max) + (2.0 ** (7 - b) if 0 < b < 8 else 0.0)

    def phi_at_bmax(q, b, b_max=8):
        return no_phi(q, b, b_max) + (2.0 ** (b_max - b - 1) if 0 < b < 8 else 0.0)

    for bad in (no_phi, eight_bit_phi, phi_at_bmax, off_by_one_shift):
        monkeypatch.setattr(grinqh_oracle, "reconstruct_level", bad)
        with pytest.raises(AssertionError):
            _check_exact(codes4, scales4, zeros4, x4, bits4, b_max=4)
        with pytest.raises(AssertionError):
            test_vmm_golden_bmax4(golden_dir)
    monkeypatch.setattr(grinqh_oracle, "reconstruct_level", good)
    _check_exact(codes4, scales4, zeros4, x4, bits4, b_max=4)

    def no_zero_term(codes_, scales_, zeros_, rows, bits_, b_max):
        return good_rows(codes_, scales_, np.zeros_like(zeros_), rows, bits_, b_max)

    def transposed(codes_, scales_, zeros_, rows, bits_, b_max):
        return good_rows(np.ascontiguousarray(codes_.T), scales_, zeros_, rows, bits_, b_max)

    for bad in (no_zero_term, transposed):
        monkeypatch.setattr(grinqh_oracle, "_dequant_rows", bad)
        with pytest.raises(AssertionError):
            _check_exact(codes, scales, zeros, x, bits)
    monkeypatch.setattr(grinqh_oracle, "_dequant_rows", good_rows)
    _check_exact(codes, scales, zeros, x, bits)

    # a wrong group size is caught by the hand-worked two-group golden case
    monkeypatch.setattr(grinqh_oracle, "GROUP", 256)
    with pytest.raises(AssertionError):
        test_vmm_golden_two_groups(golden_dir)
    monkeypatch.setattr(grinqh_oracle, "GROUP", 128)
    test_vmm_golden_two_groups(golden_dir)

# ------------------------------------------------ b_max < 8 (section 3.3: b_max in {4, 6, 8})

SMALL_BMAX = [1, 2, 4, 6, 7]


@pytest.mark.parametrize("b_max", SMALL_BMAX)
def test_brute_force_bmax_uniform_and_random_bits(b_max):
    codes, scales, zeros, x = _rand_case(8, 8, 200 + b_max, b_max)
    for b in range(b_max + 1):
        _check_exact(codes, scales, zeros, x, np.full(8, b, np.uint8), b_max)
    r = np.random.default_rng(b_max)
    for trial in range(60):
        codes, scales, zeros, x = _rand_case(8, 8, 1000 * b_max + trial, b_max)
        _check_exact(codes, scales, zeros, x, r.integers(0, b_max + 1, size=8).astype(np.uint8), b_max)


@pytest.mark.parametrize("b_max", SMALL_BMAX)
def test_bmax_tie_codes(b_max):
    """All-ones, all-zeros and single-bit codes of a b_max-bit integer."""
    top = (1 << b_max) - 1
    row = [0, top, 1 << (b_max - 1), (1 << (b_max - 1)) - 1, 1, top - 1, top >> 1, 0]
    codes = np.array([row] * 8, np.uint8)
    _, scales, zeros, x = _rand_case(8, 8, 6, b_max)
    for b in range(b_max + 1):
        _check_exact(codes, scales, zeros, x, np.full(8, b, np.uint8), b_max)


@pytest.mark.parametrize("b_max", [4, 6])
def test_all_bmax_bits_is_dense_gemv(b_max):
    """b_i = b_max everywhere: nothing truncated, y = x @ (s q + z)."""
    K, N = 300, 70
    codes, scales, zeros, x = _rand_case(K, N, 50 + b_max, b_max)
    g = np.arange(K) // 128
    W = scales[g].astype(np.float64) * codes.astype(np.float64) + zeros[g].astype(np.float64)
    want = x.astype(np.float64) @ W
    got = oracle.vmm(codes, scales, zeros, x, np.full(K, b_max, np.uint8), b_max=b_max)
    scale = np.abs(x.astype(np.float64)) @ np.abs(W)
    assert np.all(np.abs(got - want) <= 1e-12 * scale + 1e-300)


@pytest.mark.parametrize("b_max", [4, 6])
def test_bmax_nesting_and_half_bin(b_max):
    """Low b_max - b code bits are never read, and r is the centre of its bin."""
    K, N = 260, 40
    codes, scales, zeros, x = _rand_case(K, N, 60 + b_max, b_max)
    r = np.random.default_rng(61)
    bits = r.integers(0, b_max + 1, size=K).astype(np.uint8)
    y0 = oracle.vmm(codes, scales, zeros, x, bits, b_max=b_max)
    low = ((1 << (b_max - bits.astype(np.int64))) - 1)[:, None]
    flipped = (codes.astype(np.int64) ^ (r.integers(0, 1 << b_max, size=(K, N)) & low)).astype(np.uint8)
    assert np.array_equal(oracle.vmm(flipped, scales, zeros, x, bits, b_max=b_max), y0)
    q = np.arange(1 << b_max)
    for b in range(1, b_max + 1):
        rr = oracle.reconstruct_level(q, b, b_max)
        step = 2 ** (b_max - b)
        lo = (q // step) * step
        assert np.all(rr - lo == (step // 2 if b < b_max else 0))


def test_bmax_is_the_eight_bit_method_on_shifted_codes():
    """A b_max-bit code q read at width b < b_max rebuilds to the same value as
    the 8-bit code q 2^(8 - b_max) at width b, scaled by 2^(8 - b_max): the
    truncation and the midpoint are both powers of two of the same bin."""
    for b_max in (4, 6):
        q = np.arange(1 << b_max)
        for b in range(1, b_max):
            r_small = oracle.reconstruct_level(q, b, b_max)
            r_eight = oracle.reconstruct_level(q << (8 - b_max), b, 8)
            assert np.array_equal(r_small * 2.0 ** (8 - b_max), r_eight)
        # at b = b_max the widths part: no midpoint at all in the b_max store
        assert np.array_equal(oracle.reconstruct_level(q, b_max, b_max), q.astype(np.float64))


def test_bmax_rejects_widths_above_bmax():
    with pytest.raises(ValueError):
        oracle.reconstruct_level(np.arange(4), 5, 4)
    with pytest.raises(ValueError):
        oracle.reconstruct_level(np.arange(4), 1, 9)
