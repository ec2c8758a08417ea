"""Pins for the oracle's look-up-table reconstruction (nested non-uniform weights)."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synthetic


def _golden(golden_dir):
    with open(os.path.join(golden_dir, "vmm_lut_small.json")) as f:
        g = json.load(f)
    tables = [None] + [np.array(g["tables"][str(b)], np.float16) for b in range(1, g["b_max"] + 1)]
    return g, tables


def test_lut_golden(golden_dir):
    g, tables = _golden(golden_dir)
    y = oracle.vmm_lut(np.array(g["codes"], np.uint8), tables, np.array(g["x"], np.float16),
                       np.array(g["bits"], np.uint8), g["b_max"])
    assert y.tolist() == g["y"]


def _rand_tables(N, b_max, r):
    return [None] + [(r.standard_normal((N, 1 << b)) * 0.05).astype(np.float16) for b in range(1, b_max + 1)]


@pytest.mark.parametrize("b_max", [8, 4, 1])
def test_lut_exact_rational(b_max):
    r = np.random.default_rng(b_max)
    for trial in range(40):
        K, N = 8, 8
        codes = r.integers(0, 1 << b_max, size=(K, N), dtype=np.uint8)
        tables = _rand_tables(N, b_max, r)
        x = (r.standard_normal(K) * 2).astype(np.float16)
        bits = r.integers(0, b_max + 1, size=K).astype(np.uint8)
        got = oracle.vmm_lut(codes, tables, x, bits, b_max)
        mag = oracle.vmm_lut_abs(codes, tables, x, bits, b_max)
        for j in range(N):
            want = Fraction(0)
            for i in range(K):
                b = int(bits[i])
                if b:
                    want += Fraction(float(x[i])) * Fraction(float(tables[b][j, int(codes[i, j]) >> (b_max - b)]))
            assert abs(Fraction(float(got[j])) - want) <= Fraction(1e-12) * Fraction(float(mag[j])) + Fraction(1e-300)


@pytest.mark.parametrize("b_max", [8, 6])
def test_uniform_midpoint_is_a_special_lut(b_max):
    """Tables s (p 2^(b_max-b) + phi_b) + z reproduce the uniform reconstruction
    (one scale group), which is pinned independently."""
    K, N = 128, 37
    r = np.random.default_rng(11)
    codes = r.integers(0, 1 << b_max, size=(K, N), dtype=np.uint8)
    s = (r.random((1, N)) * 0.01 + 1e-4).astype(np.float16)
    z = (r.standard_normal((1, N)) * 0.05).astype(np.float16)
    x = (r.standard_normal(K) * 2).astype(np.float16)
    bits = r.integers(0, b_max + 1, size=K).astype(np.uint8)
    tables = [None]
    for b in range(1, b_max + 1):
        p = np.arange(1 << b, dtype=np.float64)
        phi = 2.0 ** (b_max - b - 1) if b < b_max else 0.0
        tables.append(s[0].astype(np.float64)[:, None] * (p[None, :] * 2.0 ** (b_max - b) + phi)
                      + z[0].astype(np.float64)[:, None])
    y_lut = oracle.vmm_lut(codes, tables, x, bits, b_max)
    y_uni = oracle.vmm(codes, s, z, x, bits, b_max=b_max)
    mag = oracle.vmm_abs(codes, s, z, x, bits, b_max=b_max)
    assert np.all(np.abs(y_lut - y_uni) <= 1e-12 * mag)


def test_all_bmax_is_dense_gemv_with_parent_table():
    K, N = 200, 30
    codes, tables = synthetic.make_lut_weights(K, N, config=0, matrix=3)
    x = synthetic.make_activations(K, 1, config=0, matrix=3)[0]
    W = tables[8].astype(np.float64)[np.arange(N)[None, :], codes.astype(np.int64)]
    want = x.astype(np.float64) @ W
    got = oracle.vmm_lut(codes, tables, x, np.full(K, 8, np.uint8))
    assert np.all(np.abs(got - want) <= 1e-12 * (np.abs(x.astype(np.float64)) @ np.abs(W)))


def test_lut_zero_bits_onehot_and_nesting():
    K, N = 150, 20
    codes, tables = synthetic.make_lut_weights(K, N, config=0, matrix=4)
    x = synthetic.make_activations(K, 1, config=0, matrix=4)[0]
    assert np.array_equal(oracle.vmm_lut(codes, tables, x, np.zeros(K, np.uint8)), np.zeros(N))
    onehot = np.zeros(K, np.float16)
    onehot[77] = 1.0
    bits = np.zeros(K, np.uint8)
    bits[77] = 3
    want = tables[3].astype(np.float64)[np.arange(N), codes[77].astype(np.int64) >> 5]
    assert np.array_equal(oracle.vmm_lut(codes, tables, onehot, bits), want)
    r = np.random.default_rng(5)
    bits = r.integers(0, 9, size=K).astype(np.uint8)
    low = ((1 << (8 - bits.astype(np.int64))) - 1)[:, None]
    flipped = (codes.astype(np.int64) ^ (r.integers(0, 256, size=(K, N)) & low)).astype(np.uint8)
    assert np.array_equal(oracle.vmm_lut(flipped, tables, x, bits), oracle.vmm_lut(codes, tables, x, bits))


def test_nested_tables_are_centred():
    """The synthetic tables: each coarser entry is the mean of its two children."""
    _, tables = synthetic.make_lut_weights(10, 16, config=0, matrix=5)
    for b in range(1, 8):
        kids = tables[b + 1].astype(np.float64)
        mean = (kids[:, 0::2] + kids[:, 1::2]) / 2
        assert np.all(np.abs(tables[b].astype(np.float64) - mean) <= 2e-3 * np.abs(mean) + 1e-6)


def _variant_y(codes, tables, x, bits, b_max, prefix, table_of):
    """The LUT product with the prefix rule and table choice as parameters."""
    codes = np.asarray(codes, np.int64)
    N = codes.shape[1]
    y = np.zeros(N)
    for i in np.nonzero(np.asarray(bits) > 0)[0]:
        b = int(bits[i])
        y += float(x[i]) * np.asarray(table_of(b), np.float64)[np.arange(N), prefix(codes[i], b)]
    return y


def test_lut_planted_mistakes(golden_dir):
    """Plausible mistakes each miss the hand-worked case: a prefix one bit
    short, a width-blind table (always the parent) and a uniform-style
    midpoint added on top of the centred entry."""
    g, tables = _golden(golden_dir)
    bm = g["b_max"]
    args = (np.array(g["codes"], np.uint8), tables, np.array(g["x"], np.float16), np.array(g["bits"], np.uint8), bm)
    right = _variant_y(*args, lambda q, b: q >> (bm - b), lambda b: tables[b])
    assert right.tolist() == g["y"]
    short = _variant_y(*args, lambda q, b: q >> min(bm - b + 1, bm), lambda b: tables[b])
    blind = _variant_y(*args, lambda q, b: q, lambda b: tables[bm])
    mid = _variant_y(*args, lambda q, b: q >> (bm - b),
                     lambda b: np.asarray(tables[b], np.float64) + (0.5 if b < bm else 0.0))
    for bad in (short, blind, mid):
        assert bad.tolist() != g["y"]
