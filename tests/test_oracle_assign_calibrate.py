"""Pins for the oracle's precision assignment, row selection and calibration.

Everything here runs on the CPU.  Each check rests on something other than the
oracle's own code: hand-worked fixtures, the interval rule as the paper writes
it, NumPy's quantile routine, or closed forms of the input distribution.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import synthetic


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- assignment

def test_assign_golden_ties(golden_dir):
    g = _load(golden_dir, "assign_ties.json")
    x = np.array([c["x"] for c in g["cases"]], dtype=np.float16)
    want = np.array([c["b"] for c in g["cases"]], dtype=np.uint8)
    got = oracle.assign(x, np.array(g["thresholds"], dtype=np.float32), g["levels"])
    assert got.tolist() == want.tolist()


def _interval_rule(x, thresholds, levels):
    """Section 3.1 as written: find k with theta_k <= |x| < theta_{k+1}."""
    bounds = [0.0] + [float(t) for t in thresholds] + [math.inf]
    out = []
    for v in x:
        a = abs(float(np.float32(v)))
        if math.isnan(a):
            out.append(levels[0])
            continue
        k = None
        for j in range(len(bounds) - 1):
            if bounds[j] <= a < bounds[j + 1]:
                k = j  # last matching interval wins when thresholds repeat
        if k is None:          # a == inf
            k = len(bounds) - 2
        out.append(levels[k])
    return np.array(out, dtype=np.uint8)


@pytest.mark.parametrize("seed", range(5))
def test_assign_matches_interval_rule(seed):
    r = np.random.default_rng(seed)
    n = int(r.integers(1, 9))
    th = np.sort(np.abs(r.standard_normal(n) * 2)).astype(np.float16).astype(np.float32)
    if seed == 3:
        th[1:] = th[0]            # repeated thresholds: empty middle bins
    levels = sorted(r.integers(0, 9, size=n + 1).tolist())
    x = (r.standard_normal(4000) * 3).astype(np.float16)
    x[:n] = th.astype(np.float16)          # exact ties
    x[n:2 * n] = -th.astype(np.float16)
    got = oracle.assign(x, th, levels)
    want = _interval_rule(x, th, levels)
    assert np.array_equal(got, want)


def test_assign_degenerate_thresholds():
    x = np.array([0.0, 1e-3, 1.0, -7.0, 60000.0], dtype=np.float16)
    lv = (0, 2, 3, 4, 8)
    assert oracle.assign(x, np.zeros(4, np.float32), lv).tolist() == [8] * 5
    assert oracle.assign(x, np.full(4, np.inf, np.float32), lv).tolist() == [0] * 5
    nan_inf = np.array([np.nan, np.inf, -np.inf], dtype=np.float16)
    assert oracle.assign(nan_inf, np.array([0.5, 1, 2, 4], np.float32), lv).tolist() == [0, 8, 8]
    # n = 0: one level for every row
    assert oracle.assign(x, np.zeros(0, np.float32), (3,)).tolist() == [3] * 5


def test_compact_brute_force():
    r = np.random.default_rng(7)
    for K in (1, 5, 64, 1000):
        bits = r.choice([0, 0, 2, 3, 8], size=K).astype(np.uint8)
        idx, m = oracle.compact(bits)
        want = [i for i in range(K) if bits[i] > 0]
        assert idx.dtype == np.int32 and idx.tolist() == want and m == len(want)
    idx, m = oracle.compact(np.zeros(10, np.uint8))
    assert m == 0 and idx.size == 0


# ---------------------------------------------------------------- calibration

def test_calibrate_golden(golden_dir):
    g = _load(golden_dir, "calibrate_small.json")
    v = np.array(g["vectors"], dtype=np.float16)
    got = oracle.calibrate(v, g["P"])
    assert np.allclose(got, np.array(g["thresholds"], np.float32), rtol=1e-7, atol=0)
    for sp in g["special"]:
        want = np.array([float(t) for t in sp["thresholds"]], np.float32)
        assert np.array_equal(oracle.calibrate(v, sp["P"]), want)


def test_cut_points_sum():
    assert oracle.cut_points((0.25, 0.25, 0.25, 0.15, 0.10)) == [0.25, 0.5, 0.75, 0.9]
    assert oracle.cut_points((1.0,)) == []


@pytest.mark.parametrize("K", [2, 7, 256, 4097])
def test_percentile_matches_numpy_linear(K):
    r = np.random.default_rng(K)
    v = np.abs(r.standard_normal(K)).astype(np.float16).astype(np.float64)
    s = np.sort(v)
    for c in (0.0, 0.1, 0.25, 0.35, 0.5, 0.65, 0.75, 0.9, 0.97, 1.0):
        want = float(np.quantile(v, c, method="linear"))
        assert oracle.empirical_quantile(s, c) == pytest.approx(want, rel=1e-15, abs=0)


def test_calibrate_matches_numpy_mean_of_quantiles():
    lay = synthetic.make_layer(256, 32, config=0, matrix=0)
    P = synthetic.P_TINY
    got = oracle.calibrate(lay.calib, P)
    cuts = np.cumsum(P)[:-1]
    a = np.abs(lay.calib.astype(np.float64))
    want = np.quantile(a, cuts, axis=1, method="linear").mean(axis=1)
    assert np.allclose(got, want.astype(np.float32), rtol=2e-7, atol=0)


def _population_quantile(c, K):
    """Quantile of |x| for the synthetic recipe, from its closed-form CDF.

    |x| = exp(Z) for ordinary channels and 20 exp(Z) for the ceil(1% K)
    outlier channels, Z ~ N(0, 1):  F(t) = (1-f) Phi(ln t) + f Phi(ln t - ln 20).
    Solved by bisection on ln t.
    """
    f = math.ceil(0.01 * K) / K
    Phi = lambda u: 0.5 * (1.0 + math.erf(u / math.sqrt(2.0)))
    F = lambda lt: (1 - f) * Phi(lt) + f * Phi(lt - math.log(20.0))
    lo, hi = -20.0, 20.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if F(mid) < c:
            lo = mid
        else:
            hi = mid
    return math.exp(0.5 * (lo + hi))


def test_calibrate_closed_form_large_K():
    K = 8192
    calib = synthetic.make_calibration(K, config=9, matrix=0)
    P = synthetic.P_LEVELS_5[3]
    got = oracle.calibrate(calib, P)
    for th, c in zip(got, oracle.cut_points(P)):
        assert th == pytest.approx(_population_quantile(c, K), rel=0.01)


@pytest.mark.parametrize("target", [2, 3, 4, 8])
def test_calibration_fidelity(target):
    """Calibrated thresholds hold the target effective bits on fresh tokens.

    The paper reports that measured effective bit widths track the target
    (Appendix D.3, Fig. 6B); here on synthetic tokens from the same recipe.
    """
    K = 4096
    P = synthetic.P_LEVELS_5[target]
    calib = synthetic.make_calibration(K, config=1, matrix=0)
    th = oracle.calibrate(calib, P)
    x = synthetic.make_activations(K, 9, config=1, matrix=0)
    realised = [oracle.assign(x[t], th, synthetic.LEVELS_5).astype(np.float64).mean() for t in range(9)]
    want = sum(p * b for p, b in zip(P, synthetic.LEVELS_5))
    assert abs(float(np.mean(realised)) - want) < 0.1
