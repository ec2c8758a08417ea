"""Parity of the HIP library with the fp64 oracle for stores of b_max < 8 bits.

Section 3.3 of the GRINQH paper evaluates parent models quantised at
b_max in {4, 6, 8}; a b_max-bit store holds b_max planes per row and a row
reads at most b_max of them.  Planes, bits and lists are bit-exact; outputs
meet |y_gpu - y_ref| <= 1e-3 * sum_i |x_i w_hat_ij| + 1e-4 with the oracle's
fp64 sum.
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


@functools.lru_cache(maxsize=6)
def layer(K, N, config, matrix, b_max):
    return synthetic.make_layer(K, N, config=config, matrix=matrix, n_test=2, b_max=b_max)


def _check_y(y_gpu, lay, x, bits, b_max, cols=None, base=None):
    codes, scales, zeros = lay.codes, lay.scales, lay.zeros
    if cols is not None:
        codes, scales, zeros, y_gpu = codes[:, cols], scales[:, cols], zeros[:, cols], y_gpu[cols]
    ref = oracle.vmm(codes, scales, zeros, x, bits, b_max=b_max)
    mag = oracle.vmm_abs(codes, scales, zeros, x, bits, b_max=b_max)
    if base is not None:
        ref = ref + base.astype(np.float64)
        mag = mag + np.abs(base.astype(np.float64))
    err = np.abs(y_gpu.astype(np.float64) - ref)
    bound = REL_TOL * mag + ABS_TOL
    worst = int(np.argmax(err - bound))
    assert np.all(err <= bound), f"col {worst}: gpu {y_gpu[worst]} ref {ref[worst]} err {err[worst]}"


# --------------------------------------------------------------------------- pack

@pytest.mark.parametrize("b_max", [1, 4, 6, 7])
@pytest.mark.parametrize("K,N", [(256, 256), (7, 33), (129, 2100), (300, 70)])
def test_pack_bmax_bit_exact(K, N, b_max):
    codes = np.random.default_rng(K * 7 + N + b_max).integers(0, 1 << b_max, size=(K, N), dtype=np.uint8)
    got = grq.pack(_dev(codes), b_max=b_max).cpu().numpy()
    assert np.array_equal(got, oracle.pack(codes, b_max))


@pytest.mark.parametrize("b_max", [4, 6])
def test_pack_bmax_bit_exact_full_size(b_max):
    lay = layer(4096, 14336, 2, 4, b_max)
    got = grq.pack(_dev(lay.codes), b_max=b_max).cpu().numpy()
    assert np.array_equal(got, oracle.pack(lay.codes, b_max))


# ------------------------------------------------------------------------- VMM

CASES = [
    # (K, N, config, matrix, b_max, P, levels)
    (256, 256, 0, 0, 6, synthetic.P_BMAX6[4], synthetic.LEVELS_BMAX6),
    (256, 256, 0, 0, 4, synthetic.P_BMAX4[3], synthetic.LEVELS_BMAX4),
    (4096, 4096, 1, 0, 6, synthetic.P_BMAX6[3], synthetic.LEVELS_BMAX6),
    (4096, 4096, 1, 0, 4, synthetic.P_BMAX4[2], synthetic.LEVELS_BMAX4),
    (4097, 1056, 5, 3, 6, synthetic.P_BMAX6[4], synthetic.LEVELS_BMAX6),
    (129, 1100, 5, 1, 4, synthetic.P_BMAX4[3], synthetic.LEVELS_BMAX4),
    (300, 70, 5, 0, 7, (0.2, 0.2, 0.2, 0.2, 0.2), (0, 1, 3, 5, 7)),
    (1000, 2080, 5, 4, 1, (0.5, 0.5), (0, 1)),
    (14336, 4096, 2, 6, 6, synthetic.P_BMAX6[4], synthetic.LEVELS_BMAX6),
]


@pytest.mark.parametrize("K,N,cfg,mat,b_max,P,levels", CASES)
def test_decode_vmm_bmax_parity(K, N, cfg, mat, b_max, P, levels):
    lay = layer(K, N, cfg, mat, b_max)
    th = oracle.calibrate(lay.calib, P)
    x = lay.x[0]
    planes = grq.pack(_dev(lay.codes), b_max=b_max)
    sc, zr = _dev(lay.scales), _dev(lay.zeros)
    ws = grq.make_workspace(K, N)
    y = grq.decode_vmm(planes, sc, zr, _dev(x), K, N, th, levels, ws, b_max=b_max)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    bits = oracle.assign(x, th, levels)
    _check_y(y, lay, x, bits, b_max)
    # the two-call path gives the same bits
    b, idx, n = grq.assign_bits(_dev(x), th, levels)
    y2 = grq.vmm(planes, sc, zr, _dev(x), b, idx, n, K, N, ws, b_max=b_max)
    # the accumulating entry point adds the same product into y0
    y0 = np.random.default_rng(K + N).standard_normal(N).astype(np.float32)
    y3 = _dev(y0.copy())
    grq.decode_vmm_accumulate(planes, sc, zr, _dev(x), K, N, th, levels, y3, b_max=b_max)
    torch.cuda.synchronize()
    assert np.array_equal(y2.cpu().numpy().view(np.uint32), y.view(np.uint32))
    _check_y(y3.cpu().numpy(), lay, x, bits, b_max, base=y0)


@pytest.mark.parametrize("b_max", [4, 6])
def test_vmm_bmax_from_oracle_assignment_and_clamp(b_max):
    """Random widths 0..b_max from the oracle; widths above b_max read as b_max."""
    K, N = 4096, 4096
    lay = layer(K, N, 1, 0, b_max)
    x = lay.x[1]
    bits = np.random.default_rng(b_max).integers(0, b_max + 1, size=K).astype(np.uint8)
    idx, n = oracle.compact(bits)
    idx_full = np.zeros(K, np.int32)
    idx_full[:n] = idx
    planes = grq.pack(_dev(lay.codes), b_max=b_max)
    ws = grq.make_workspace(K, N)
    args = (planes, _dev(lay.scales), _dev(lay.zeros), _dev(x))
    tail = (_dev(idx_full), _dev(np.array([n], np.int32)), K, N, ws)
    y = grq.vmm(*args, _dev(bits), *tail, b_max=b_max)
    over = np.where(bits == b_max, np.uint8(8 + b_max), bits).astype(np.uint8)
    y_over = grq.vmm(*args, _dev(over), *tail, b_max=b_max)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    _check_y(y, lay, x, bits, b_max)
    assert np.array_equal(y_over.cpu().numpy().view(np.uint32), y.view(np.uint32))


@pytest.mark.parametrize("b_max", [4, 6])
def test_all_bmax_bits_is_dense_and_zero_bits_is_zero(b_max):
    K, N = 4096, 1024
    lay = layer(K, N, 2, 1, b_max)
    x = lay.x[0]
    planes = grq.pack(_dev(lay.codes), b_max=b_max)
    ws = grq.make_workspace(K, N)
    args = (planes, _dev(lay.scales), _dev(lay.zeros), _dev(x), K, N)
    y = grq.decode_vmm(*args, [], (b_max,), ws, b_max=b_max).cpu().numpy()
    g = np.arange(K) // 128
    dense = x.astype(np.float64) @ (lay.scales[g].astype(np.float64) * lay.codes + lay.zeros[g].astype(np.float64))
    mag = oracle.vmm_abs(lay.codes, lay.scales, lay.zeros, x, np.full(K, b_max, np.uint8), b_max=b_max)
    assert np.all(np.abs(y - dense) <= REL_TOL * mag + ABS_TOL)
    y0 = grq.decode_vmm(*args, [], (0,), ws, b_max=b_max).cpu().numpy()
    assert np.array_equal(y0, np.zeros(N, np.float32))


def test_level_above_bmax_is_rejected():
    lay = layer(256, 256, 0, 0, 4)
    planes = grq.pack(_dev(lay.codes), b_max=4)
    ws = grq.make_workspace(256, 256)
    with pytest.raises(grq.GrinqhError):
        grq.decode_vmm(planes, _dev(lay.scales), _dev(lay.zeros), _dev(lay.x[0]), 256, 256,
                       [1.0], (0, 6), ws, b_max=4)


# ------------------------------------------------- full sizes, every output

FULL = [
    (4096, 14336, 2, 4, 6, synthetic.P_BMAX6[4], synthetic.LEVELS_BMAX6),
    (4096, 14336, 2, 4, 4, synthetic.P_BMAX4[3], synthetic.LEVELS_BMAX4),
    (8192, 28672, 4, 0, 4, synthetic.P_BMAX4[2], synthetic.LEVELS_BMAX4),
]


@pytest.mark.parametrize("K,N,cfg,mat,b_max,P,levels", FULL)
def test_full_size_bmax_all_columns(K, N, cfg, mat, b_max, P, levels):
    lay = layer(K, N, cfg, mat, b_max)
    th = oracle.calibrate(lay.calib, P)
    x = lay.x[0]
    planes = grq.pack(_dev(lay.codes), b_max=b_max)
    y = torch.zeros(N, dtype=torch.float32, device="cuda")
    grq.decode_vmm_accumulate(planes, _dev(lay.scales), _dev(lay.zeros), _dev(x), K, N, th, levels, y,
                              b_max=b_max)
    torch.cuda.synchronize()
    bits = oracle.assign(x, th, levels)
    _check_y(y.cpu().numpy(), lay, x, bits, b_max)
