"""Pins for the oracle's tolerance scales: vmm_abs, vmm_lut_abs, prefill_abs.

Every GPU parity bound is 1e-3 * sum_i |x_i w_hat_ij| + 1e-4 per element, so
the scale itself is pinned here, against things other than the oracle:
hand-worked values in tests/golden/ (the "abs" entries, each derived in the
file's notes from the reconstruction of GRINQH section 3.3), exact rational
brute force with integer bit slicing on tiny inputs, and identities (when
every term x_i w_hat_ij is >= 0 the scale equals the product itself; it
never falls below |y|; it ignores the sign of x and bypassed rows).  The last
test plants plausible mistakes in the scale (a loose per-row bound, the
absolute value taken outside the sum, bypassed rows counted, the untruncated
code, a dropped zero term) and checks that a pin fails for each.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import grinqh_oracle


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def _vmm_golden_args(g):
    return (np.array(g["codes"], np.uint8), np.array(g["scales"], np.float16),
            np.array(g["zeros"], np.float16), np.array(g["x"], np.float16), np.array(g["bits"], np.uint8))


def _two_groups_args(g):
    K, N = g["K"], g["N"]
    codes = np.zeros((K, N), np.uint8)
    x = np.zeros(K, np.float16)
    bits = np.zeros(K, np.uint8)
    for i, (b, q, xv) in g["active"].items():
        codes[int(i)] = q
        x[int(i)] = xv
        bits[int(i)] = b
    return codes, np.array(g["scales"], np.float16), np.array(g["zeros"], np.float16), x, bits


def _lut_golden(golden_dir):
    g = _load(golden_dir, "vmm_lut_small.json")
    tables = [None] + [np.array(g["tables"][str(b)], np.float16) for b in range(1, g["b_max"] + 1)]
    return g, tables


# ------------------------------------------------------------ hand-worked values

def test_vmm_abs_golden(golden_dir):
    g = _load(golden_dir, "vmm_small.json")
    assert oracle.vmm_abs(*_vmm_golden_args(g)).tolist() == g["abs"]
    g4 = _load(golden_dir, "vmm_bmax4.json")
    assert oracle.vmm_abs(*_vmm_golden_args(g4), b_max=g4["b_max"]).tolist() == g4["abs"]
    g2 = _load(golden_dir, "vmm_two_groups.json")
    assert oracle.vmm_abs(*_two_groups_args(g2)).tolist() == g2["abs"]


def test_vmm_lut_abs_golden(golden_dir):
    g, tables = _lut_golden(golden_dir)
    got = oracle.vmm_lut_abs(np.array(g["codes"], np.uint8), tables, np.array(g["x"], np.float16),
                             np.array(g["bits"], np.uint8), g["b_max"])
    assert got.tolist() == g["abs"]


def test_prefill_abs_golden(golden_dir):
    g = _load(golden_dir, "prefill_small.json")
    got = oracle.prefill_abs(np.array(g["codes"], np.uint8), np.array(g["scales"], np.float16),
                             np.array(g["zeros"], np.float16), np.array(g["X"], np.float16), g["b_max"])
    assert got.tolist() == g["abs"]


# ------------------------------------------------------------ exact rational brute force

def _rand_case(K, N, seed, b_max=8):
    r = np.random.default_rng(seed)
    codes = r.integers(0, 1 << b_max, size=(K, N), dtype=np.uint8)
    G = -(-K // 128)
    scales = (r.random((G, N)) * 0.01 + 1e-4).astype(np.float16)
    zeros = (r.standard_normal((G, N)) * 0.05).astype(np.float16)
    x = (r.standard_normal(K) * 2).astype(np.float16)
    return codes, scales, zeros, x


def _fraction_abs(codes, scales, zeros, x, bits, b_max=8):
    """sum over rows with b > 0 of |x_i w_hat_ij|, exactly: the b most
    significant code bits by an integer shift, the midpoint 2^(b_max - b - 1)
    below b_max (section 3.3)."""
    K, N = codes.shape
    out = [Fraction(0)] * N
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
            out[j] += abs(xi * w)
    return out


@pytest.mark.parametrize("b_max", [8, 6, 4, 1])
def test_vmm_abs_exact_rational(b_max):
    r = np.random.default_rng(500 + b_max)
    for trial in range(40):
        codes, scales, zeros, x = _rand_case(8, 8, 600 + 50 * b_max + trial, b_max)
        bits = r.integers(0, b_max + 1, size=8).astype(np.uint8)
        want = _fraction_abs(codes, scales, zeros, x, bits, b_max)
        got = oracle.vmm_abs(codes, scales, zeros, x, bits, b_max=b_max)
        for j in range(8):
            assert abs(Fraction(float(got[j])) - want[j]) <= Fraction(1e-12) * want[j] + Fraction(1e-300)


@pytest.mark.parametrize("b_max", [8, 3])
def test_vmm_lut_abs_exact_rational(b_max):
    r = np.random.default_rng(70 + b_max)
    for trial in range(30):
        K, N = 8, 6
        codes = r.integers(0, 1 << b_max, size=(K, N)).astype(np.uint8)
        tables = [None] + [(r.standard_normal((N, 1 << b)) * 0.05).astype(np.float16) for b in range(1, b_max + 1)]
        x = (r.standard_normal(K) * 2).astype(np.float16)
        bits = r.integers(0, b_max + 1, size=K).astype(np.uint8)
        got = oracle.vmm_lut_abs(codes, tables, x, bits, b_max)
        for j in range(N):
            want = Fraction(0)
            for i in range(K):
                b = int(bits[i])
                if b:
                    want += abs(Fraction(float(x[i])) * Fraction(float(tables[b][j, int(codes[i, j]) >> (b_max - b)])))
            assert abs(Fraction(float(got[j])) - want) <= Fraction(1e-12) * want + Fraction(1e-300)


def test_prefill_abs_exact_rational():
    M, K, N = 3, 8, 5
    r = np.random.default_rng(9)
    codes = r.integers(0, 256, size=(K, N)).astype(np.uint8)
    scales = (r.random((1, N)) * 0.01 + 1e-4).astype(np.float16)
    zeros = (r.standard_normal((1, N)) * 0.05).astype(np.float16)
    X = (r.standard_normal((M, K)) * 2).astype(np.float16)
    got = oracle.prefill_abs(codes, scales, zeros, X)
    for m in range(M):
        for j in range(N):
            want = sum(abs(Fraction(float(X[m, k])) * (Fraction(float(scales[0, j])) * int(codes[k, j])
                                                       + Fraction(float(zeros[0, j])))) for k in range(K))
            assert abs(Fraction(float(got[m, j])) - want) <= Fraction(1e-12) * want


# ------------------------------------------------------------ identities

def test_vmm_abs_equals_vmm_when_every_term_is_nonnegative():
    """x >= 0 and s, z >= 0 make every x_i w_hat_ij >= 0, so the scale is y;
    with every x negative it is -y."""
    K, N = 300, 70
    codes, scales, zeros, x = _rand_case(K, N, 17)
    zeros = np.abs(zeros)
    xp = np.abs(x)
    bits = np.random.default_rng(18).integers(0, 9, size=K).astype(np.uint8)
    y = oracle.vmm(codes, scales, zeros, xp, bits)
    a = oracle.vmm_abs(codes, scales, zeros, xp, bits)
    assert np.all(np.abs(a - y) <= 1e-12 * a)
    yn = oracle.vmm(codes, scales, zeros, -xp, bits)
    assert np.all(np.abs(a + yn) <= 1e-12 * a)
    # and the LUT and prefill scales with non-negative tables / weights
    tables = [None] + [np.abs(np.random.default_rng(b).standard_normal((N, 1 << b)) * 0.05).astype(np.float16)
                       for b in range(1, 9)]
    yl = oracle.vmm_lut(codes, tables, xp, bits)
    al = oracle.vmm_lut_abs(codes, tables, xp, bits)
    assert np.all(np.abs(al - yl) <= 1e-12 * al)
    X = np.stack([xp, xp[::-1]])
    Yp = oracle.prefill(codes, scales, zeros, X)
    Ap = oracle.prefill_abs(codes, scales, zeros, X)
    assert np.all(np.abs(Ap - Yp) <= 1e-12 * Ap)


def test_vmm_abs_bounds_and_symmetries():
    K, N = 260, 40
    codes, scales, zeros, x = _rand_case(K, N, 27)
    bits = np.random.default_rng(28).integers(0, 9, size=K).astype(np.uint8)
    a = oracle.vmm_abs(codes, scales, zeros, x, bits)
    y = oracle.vmm(codes, scales, zeros, x, bits)
    assert np.all(a >= np.abs(y) * (1 - 1e-12))                                 # triangle inequality
    assert np.array_equal(oracle.vmm_abs(codes, scales, zeros, -x, bits), a)    # sign of x
    flip = np.where(np.arange(K) % 3 == 0, -x, x)
    assert np.array_equal(oracle.vmm_abs(codes, scales, zeros, flip, bits), a)  # per-row sign of x
    assert np.array_equal(oracle.vmm_abs(codes, scales, zeros, x, np.zeros(K, np.uint8)), np.zeros(N))
    # a bypassed row's activation does not enter
    x2 = x.copy()
    x2[bits == 0] = np.float16(1000.0)
    assert np.array_equal(oracle.vmm_abs(codes, scales, zeros, x2, bits), a)


# ------------------------------------------------------------ the pins catch planted mistakes

def test_tolerance_planted_mistakes_are_caught(monkeypatch, golden_dir):
    """A looser per-row bound |x| (255 |s| + |z|), |sum| instead of sum |.|,
    bypassed rows counted, the untruncated code, and a dropped zero term each
    fail a pin above."""
    good = grinqh_oracle.vmm_abs

    def loose(codes, scales, zeros, x, bits, chunk=256, b_max=8):
        codes = np.asarray(codes)
        K = codes.shape[0]
        g = np.arange(K) // 128
        top = float((1 << b_max) - 1)
        ax = np.abs(np.asarray(x, np.float16).astype(np.float64)) * (np.asarray(bits) > 0)
        return ax @ (top * np.abs(scales[g].astype(np.float64)) + np.abs(zeros[g].astype(np.float64)))

    def abs_outside(codes, scales, zeros, x, bits, chunk=256, b_max=8):
        return np.abs(grinqh_oracle.vmm(codes, scales, zeros, x, bits, b_max=b_max))

    def bypassed_counted(codes, scales, zeros, x, bits, chunk=256, b_max=8):
        b = np.asarray(bits).copy()
        b[b == 0] = b_max
        return good(codes, scales, zeros, x, b, b_max=b_max)

    def untruncated(codes, scales, zeros, x, bits, chunk=256, b_max=8):
        b = np.where(np.asarray(bits) > 0, b_max, 0).astype(np.uint8)
        return good(codes, scales, zeros, x, b, b_max=b_max)

    def no_zero(codes, scales, zeros, x, bits, chunk=256, b_max=8):
        return good(codes, scales, np.zeros_like(zeros), x, bits, b_max=b_max)

    for bad in (loose, abs_outside, bypassed_counted, untruncated, no_zero):
        monkeypatch.setattr(grinqh_oracle, "vmm_abs", bad)
        monkeypatch.setattr(oracle, "vmm_abs", bad)
        with pytest.raises(AssertionError):
            test_vmm_abs_golden(golden_dir)
        with pytest.raises(AssertionError):
            test_vmm_abs_exact_rational(8)
    monkeypatch.setattr(grinqh_oracle, "vmm_abs", good)
    monkeypatch.setattr(oracle, "vmm_abs", good)
    test_vmm_abs_golden(golden_dir)

    good_lut = grinqh_oracle.vmm_lut_abs

    def lut_abs_outside(codes, lut, x, bits, b_max=8):
        return np.abs(grinqh_oracle.vmm_lut(codes, lut, x, bits, b_max))

    def lut_parent_table(codes, lut, x, bits, b_max=8):
        b = np.where(np.asarray(bits) > 0, b_max, 0).astype(np.uint8)
        return good_lut(codes, lut, x, b, b_max)

    for bad in (lut_abs_outside, lut_parent_table):
        monkeypatch.setattr(oracle, "vmm_lut_abs", bad)
        with pytest.raises(AssertionError):
            test_vmm_lut_abs_golden(golden_dir)
    monkeypatch.setattr(oracle, "vmm_lut_abs", good_lut)

    good_pf = grinqh_oracle.prefill_abs

    def pf_abs_outside(codes, scales, zeros, X, b_max=8):
        return np.abs(grinqh_oracle.prefill(codes, scales, zeros, X, b_max))

    def pf_no_zero(codes, scales, zeros, X, b_max=8):
        return good_pf(codes, scales, np.zeros_like(zeros), X, b_max)

    for bad in (pf_abs_outside, pf_no_zero):
        monkeypatch.setattr(oracle, "prefill_abs", bad)
        with pytest.raises(AssertionError):
            test_prefill_abs_golden(golden_dir)
    monkeypatch.setattr(oracle, "prefill_abs", good_pf)
