"""Checks of the seeded input generator (shapes, determinism, RTN bounds)."""
import math

import numpy as np
import pytest

import synthetic


def test_deterministic_and_role_separated():
    a = synthetic.make_layer(256, 64, config=0, matrix=0)
    b = synthetic.make_layer(256, 64, config=0, matrix=0)
    for f in ("codes", "scales", "zeros", "calib", "x"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    c = synthetic.make_layer(256, 64, config=0, matrix=1)
    assert not np.array_equal(a.codes, c.codes)
    assert not np.array_equal(a.calib[0], a.x[0])


def test_shapes_and_dtypes():
    lay = synthetic.make_layer(300, 70, config=0, matrix=0, n_test=3)
    assert lay.codes.shape == (300, 70) and lay.codes.dtype == np.uint8
    assert lay.scales.shape == (3, 70) and lay.scales.dtype == np.float16
    assert lay.zeros.shape == (3, 70)
    assert lay.calib.shape == (64, 300) and lay.calib.dtype == np.float16
    assert lay.x.shape == (3, 300)


def test_rtn_round_to_nearest_bound():
    r = np.random.default_rng(0)
    w = (r.standard_normal((300, 40)) * 0.02).astype(np.float32)
    q, s, z = synthetic.rtn_quantize(w)
    g = np.arange(300) // 128
    s64 = s[g].astype(np.float64)
    z64 = z[g].astype(np.float64)
    w_hat = s64 * q + z64
    inside = (q > 0) & (q < 255)
    assert np.all(np.abs(w_hat - w)[inside] <= s64[inside] * 0.5 * (1 + 1e-9))
    assert inside.mean() > 0.95
    assert q.min() == 0 and q.max() == 255


@pytest.mark.parametrize("b_max", [4, 6])
def test_rtn_bmax_bound(b_max):
    """At b_max bits the codes span 0 .. 2^b_max - 1 and w_hat is within half a step."""
    r = np.random.default_rng(b_max)
    w = (r.standard_normal((260, 30)) * 0.02).astype(np.float32)
    q, s, z = synthetic.rtn_quantize(w, b_max)
    top = (1 << b_max) - 1
    assert q.min() == 0 and q.max() == top
    g = np.arange(260) // 128
    s64 = s[g].astype(np.float64)
    w_hat = s64 * q + z[g].astype(np.float64)
    inside = (q > 0) & (q < top)
    assert np.all(np.abs(w_hat - w)[inside] <= s64[inside] * 0.5 * (1 + 1e-9))
    lay = synthetic.make_layer(200, 40, config=0, matrix=0, b_max=b_max)
    assert lay.codes.max() <= top


def test_outlier_channels():
    K = 4096
    x = synthetic.make_activations(K, 16, config=1, matrix=0).astype(np.float64)
    rows = synthetic.outlier_rows(K, config=1, matrix=0)
    assert len(rows) == math.ceil(0.01 * K)
    ratio = np.median(np.abs(x[:, rows])) / np.median(np.abs(np.delete(x, rows, axis=1)))
    assert 15 < ratio < 27


@pytest.mark.parametrize("table,levels", [(synthetic.P_LEVELS_5, synthetic.LEVELS_5),
                                          (synthetic.P_LEVELS_4, synthetic.LEVELS_4),
                                          (synthetic.P_BMAX6, synthetic.LEVELS_BMAX6),
                                          (synthetic.P_BMAX4, synthetic.LEVELS_BMAX4)])
def test_precision_tables(table, levels):
    for avg, P in table.items():
        assert sum(P) == pytest.approx(1.0, abs=1e-12)
        assert sum(p * b for p, b in zip(P, levels)) == pytest.approx(avg, abs=1e-12)


def test_torch_rtn_matches_numpy_rule():
    """The device quantiser applies rtn_quantize's rule (evaluated in fp32
    instead of fp64): identical scales and zeros, and codes identical except
    where w sits within fp32 rounding of a decision boundary."""
    torch = pytest.importorskip("torch")
    w = (np.random.default_rng(5).standard_normal((300, 70)) * 0.02).astype(np.float32)
    for b_max in (8, 4):
        c, s, z = synthetic.rtn_quantize(w, b_max)
        ct, st, zt = (t.numpy() for t in synthetic.rtn_quantize_torch(torch.from_numpy(w), b_max))
        assert np.array_equal(st.view(np.uint16), s.view(np.uint16))
        assert np.array_equal(zt.view(np.uint16), z.view(np.uint16))
        diff = ct.astype(np.int16) - c.astype(np.int16)
        assert np.abs(diff).max() <= 1 and np.count_nonzero(diff) <= 2


def test_device_weights_seeded_and_distributed():
    torch = pytest.importorskip("torch")
    a = synthetic.device_weights(256, 128, 3, 4, "cpu")
    b = synthetic.device_weights(256, 128, 3, 4, "cpu")
    c = synthetic.device_weights(256, 128, 3, 5, "cpu")
    assert all(torch.equal(u, v) for u, v in zip(a, b))
    assert not torch.equal(a[0], c[0])
    codes, scales, zeros = a
    g = torch.arange(256) // 128
    w = codes.double() * scales.double()[g] + zeros.double()[g]
    assert abs(w.std().item() - 0.02) < 0.001 and abs(w.mean().item()) < 0.001
    assert codes.min().item() == 0 and codes.max().item() == 255     # every column spans its range


def test_qwen3_stack_listing():
    st = synthetic.qwen3_stack()
    assert len(st) == 252
    assert [m[0] for m in st] == list(range(252))
    assert sum(K * N for _, _, _, K, N in st) == 36 * (2 * 4096 * 4096 + 2 * 4096 * 1024 + 3 * 4096 * 12288)
    assert st[6] == (6, 0, "down", 12288, 4096) and st[-1][1] == 35
