"""Pins for the oracle's dense prefill product (every row at b_max)."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle


def _case(M, K, N, seed, b_max=8):
    r = np.random.default_rng(seed)
    codes = r.integers(0, 1 << b_max, size=(K, N), dtype=np.uint8)
    G = -(-K // 128)
    scales = (r.random((G, N)) * 0.01 + 1e-4).astype(np.float16)
    zeros = (r.standard_normal((G, N)) * 0.05).astype(np.float16)
    X = (r.standard_normal((M, K)) * 2).astype(np.float16)
    return codes, scales, zeros, X


def test_prefill_golden(golden_dir):
    with open(os.path.join(golden_dir, "prefill_small.json")) as f:
        g = json.load(f)
    Y = oracle.prefill(np.array(g["codes"], np.uint8), np.array(g["scales"], np.float16),
                       np.array(g["zeros"], np.float16), np.array(g["X"], np.float16), g["b_max"])
    assert Y.tolist() == g["Y"]


@pytest.mark.parametrize("b_max", [8, 6, 4])
def test_prefill_exact_rational(b_max):
    """Tiny case against an exact rational evaluation of sum_k X[m][k] (s q + z)."""
    M, K, N = 3, 8, 5
    codes, scales, zeros, X = _case(M, K, N, 7 + b_max, b_max)
    got = oracle.prefill(codes, scales, zeros, X, b_max)
    mag = oracle.prefill_abs(codes, scales, zeros, X, b_max)
    for m in range(M):
        for j in range(N):
            want = sum(Fraction(float(X[m, k])) * (Fraction(float(scales[0, j])) * int(codes[k, j])
                                                   + Fraction(float(zeros[0, j]))) for k in range(K))
            assert abs(Fraction(float(got[m, j])) - want) <= Fraction(1e-12) * Fraction(float(mag[m, j]))


@pytest.mark.parametrize("b_max", [8, 6])
def test_prefill_rows_are_full_width_decode_vmms(b_max):
    """Each output row is the decode VMM of that token with every row at b_max."""
    M, K, N = 4, 300, 70
    codes, scales, zeros, X = _case(M, K, N, 3, b_max)
    Y = oracle.prefill(codes, scales, zeros, X, b_max)
    for m in range(M):
        y = oracle.vmm(codes, scales, zeros, X[m], np.full(K, b_max, np.uint8), b_max=b_max)
        mag = oracle.vmm_abs(codes, scales, zeros, X[m], np.full(K, b_max, np.uint8), b_max=b_max)
        assert np.all(np.abs(Y[m] - y) <= 1e-12 * mag)


def test_prefill_group_indexing():
    """Rows 0..127 use group 0's scale and zero, row 128 and on group 1's."""
    K, N = 130, 3
    codes = np.zeros((K, N), np.uint8)
    codes[127] = [1, 2, 3]
    codes[128] = [4, 5, 6]
    scales = np.array([[1.0, 2.0, 4.0], [0.5, 0.25, 0.125]], np.float16)
    zeros = np.array([[0.0, 0.0, 0.0], [1.0, 1.0, 1.0]], np.float16)
    X = np.zeros((2, K), np.float16)
    X[0, 127] = 1.0
    X[1, 128] = 1.0
    Y = oracle.prefill(codes, scales, zeros, X)
    assert Y[0].tolist() == [1.0, 4.0, 12.0]
    assert Y[1].tolist() == [3.0, 2.25, 1.75]


def test_dense_fp16_is_correctly_rounded():
    """Every entry is the fp16 nearest to the exact s q + z (ties to even):
    the two fp16 neighbours of the result bracket the exact value and the
    result is the closer one."""
    codes, scales, zeros, _ = _case(1, 300, 50, 21)
    exact = oracle.dequant_dense(codes, scales, zeros)
    r = oracle.dequant_dense_fp16(codes, scales, zeros)
    up = np.nextafter(r, np.float16(np.inf)).astype(np.float64)
    dn = np.nextafter(r, np.float16(-np.inf)).astype(np.float64)
    rv = r.astype(np.float64)
    assert np.all(np.abs(rv - exact) <= np.abs(up - exact))
    assert np.all(np.abs(rv - exact) <= np.abs(dn - exact))
    g = np.arange(300) // 128
    assert np.array_equal(rv[5], (scales[g[5]].astype(np.float64) * codes[5] + zeros[g[5]].astype(np.float64)).astype(np.float16).astype(np.float64))
