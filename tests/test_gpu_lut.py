"""Parity of grinqh_decode_vmm_lut (table reconstruction) with the fp64 oracle.

Every output element must satisfy |y - y_ref| <= 1e-3 * sum_i |x_i w_ij| + 1e-4
(the table entries are fp16 on both sides, so the only differences are fp32
products and sums).
"""
import functools

import numpy as np
import pytest

import oracle
import synthetic

torch = pytest.importorskip("torch")
import decode_stage_gemv_amd as grq  # noqa: E402

pytestmark = pytest.mark.gpu

REL_TOL = 1e-3
ABS_TOL = 1e-4


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@functools.lru_cache(maxsize=4)
def lut_layer(K, N, cfg, mat, b_max):
    codes, tables = synthetic.make_lut_weights(K, N, config=cfg, matrix=mat, b_max=b_max)
    calib = synthetic.make_calibration(K, config=cfg, matrix=mat)
    x = synthetic.make_activations(K, 2, config=cfg, matrix=mat)
    return codes, tables, calib, x


def _run(K, N, cfg, mat, b_max, P, levels, xi=0, y0=None, cols=None):
    codes, tables, calib, xs = lut_layer(K, N, cfg, mat, b_max)
    x = xs[xi]
    th = oracle.calibrate(calib, P)
    planes = grq.pack(_dev(codes), b_max=b_max)
    lut = _dev(synthetic.lut_flat(tables, N, b_max))
    base = np.zeros(N, np.float32) if y0 is None else y0
    y = _dev(base.copy())
    clear = torch.ones(N, dtype=torch.float32, device="cuda")
    grq.decode_vmm_lut(planes, lut, _dev(x), K, N, th, levels, y, clear, b_max=b_max)
    torch.cuda.synchronize()
    assert torch.count_nonzero(clear).item() == 0
    bits = oracle.assign(x, th, levels)
    got = y.cpu().numpy()
    sel = slice(None) if cols is None else cols
    c_codes = codes if cols is None else codes[:, cols]
    c_tables = tables if cols is None else [None] + [t[cols] for t in tables[1:]]
    ref = oracle.vmm_lut(c_codes, c_tables, x, bits, b_max) + base[sel].astype(np.float64)
    mag = oracle.vmm_lut_abs(c_codes, c_tables, x, bits, b_max) + np.abs(base[sel].astype(np.float64))
    err = np.abs(got[sel].astype(np.float64) - ref)
    bound = REL_TOL * mag + ABS_TOL
    worst = int(np.argmax(err - bound))
    assert np.all(err <= bound), f"col {worst}: gpu {got[sel][worst]} ref {ref[worst]} err {err[worst]}"
    return got


ALL_LEVELS = (0, 1, 2, 3, 4, 5, 6, 7, 8)
P_ALL = (0.1,) * 8 + (0.2,)

CASES = [
    # (K, N, config, matrix, b_max, P, levels)
    (256, 256, 0, 0, 8, synthetic.P_TINY, synthetic.LEVELS_5),
    (300, 70, 5, 0, 8, synthetic.P_TINY, synthetic.LEVELS_5),
    (129, 1100, 5, 1, 8, synthetic.P_LEVELS_5[4], synthetic.LEVELS_5),
    (4097, 1056, 5, 3, 8, synthetic.P_LEVELS_4[1], synthetic.LEVELS_4),
    (4096, 4096, 1, 0, 8, synthetic.P_LEVELS_5[3], synthetic.LEVELS_5),
    (4096, 4096, 1, 0, 8, P_ALL, ALL_LEVELS),        # every width: the largest table set
    (2000, 2080, 5, 4, 4, synthetic.P_BMAX4[3], synthetic.LEVELS_BMAX4),
    (1000, 512, 5, 6, 6, synthetic.P_BMAX6[4], synthetic.LEVELS_BMAX6),
]


@pytest.mark.parametrize("K,N,cfg,mat,b_max,P,levels", CASES)
def test_decode_vmm_lut_parity(K, N, cfg, mat, b_max, P, levels):
    y0 = np.random.default_rng(K + N).standard_normal(N).astype(np.float32)
    _run(K, N, cfg, mat, b_max, P, levels, y0=y0)


def test_lut_all_zero_and_all_full_width():
    K, N = 4096, 1024
    codes, tables, calib, xs = lut_layer(K, N, 2, 1, 8)
    planes = grq.pack(_dev(codes))
    lut = _dev(synthetic.lut_flat(tables, N, 8))
    y = torch.zeros(N, dtype=torch.float32, device="cuda")
    grq.decode_vmm_lut(planes, lut, _dev(xs[0]), K, N, [], (0,), y)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy(), np.zeros(N, np.float32))
    grq.decode_vmm_lut(planes, lut, _dev(xs[0]), K, N, [], (8,), y)
    torch.cuda.synchronize()
    W = tables[8].astype(np.float64)[np.arange(N)[None, :], codes.astype(np.int64)]
    x64 = xs[0].astype(np.float64)
    err = np.abs(y.cpu().numpy() - x64 @ W)
    assert np.all(err <= REL_TOL * (np.abs(x64) @ np.abs(W)) + ABS_TOL)


def test_lut_full_size_all_columns():
    K, N = 4096, 14336
    _run(K, N, 2, 4, 8, synthetic.P_LEVELS_5[3], synthetic.LEVELS_5)


def test_lut_70b_gate_all_columns():
    """8192 x 28672 at levels {0, 2, 4, 8}, every output column: 2048-row
    workgroups with the 8-bit table among the widths in use, two per CU."""
    K, N = 8192, 28672
    _run(K, N, 4, 0, 8, synthetic.P_LEVELS_4[3], synthetic.LEVELS_4)


def test_lut_largest_lds_use():
    """Every width in use with 2048 rows per workgroup (one row split across
    65536 columns): about 143 KB of LDS per workgroup, the most the entry
    point asks for."""
    K, N = 2048, 65536
    r = np.random.default_rng(11)
    cols = np.unique(np.concatenate([r.choice(N, 96, replace=False), [0, 127, 128, 65535]]))
    _run(K, N, 5, 7, 8, P_ALL, ALL_LEVELS, cols=cols)
