"""Parity of the HIP library (through its C ABI) with the fp64 oracle.

Bit-exact: packed planes, bit assignments, the active-row list and its
length, calibrated thresholds.  Floating point: every output element within
|y_gpu - y_ref| <= 1e-3 * sum_i |x_i w_hat_ij| + 1e-4 (the sum taken in fp64
by the oracle).
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


@functools.lru_cache(maxsize=8)
def layer(K, N, config=0, matrix=0):
    return synthetic.make_layer(K, N, config=config, matrix=matrix, n_test=2)


def _check_y(y_gpu, codes, scales, zeros, x, bits, cols=None):
    if cols is not None:
        codes, scales, zeros = codes[:, cols], scales[:, cols], zeros[:, cols]
        y_gpu = y_gpu[cols]
    ref = oracle.vmm(codes, scales, zeros, x, bits)
    mag = oracle.vmm_abs(codes, scales, zeros, x, bits)
    err = np.abs(y_gpu.astype(np.float64) - ref)
    bound = REL_TOL * mag + ABS_TOL
    worst = int(np.argmax(err - bound))
    assert np.all(err <= bound), f"col {worst}: gpu {y_gpu[worst]} ref {ref[worst]} err {err[worst]} bound {bound[worst]}"
    return float(np.max(err / (mag + 1e-30)))


def _run_decode(lay, x, th, levels):
    K, N = lay.K, lay.N
    planes = grq.pack(_dev(lay.codes))
    ws = grq.make_workspace(K, N)
    y = grq.decode_vmm(planes, _dev(lay.scales), _dev(lay.zeros), _dev(x), K, N, th, levels, ws)
    torch.cuda.synchronize()
    return y.cpu().numpy(), planes, ws


# --------------------------------------------------------------------------- pack

@pytest.mark.parametrize("K,N", [(256, 256), (300, 70), (130, 1056), (7, 33), (2, 64), (129, 2100), (4096, 1024)])
def test_pack_bit_exact(K, N):
    codes = np.random.default_rng(K * 7 + N).integers(0, 256, size=(K, N), dtype=np.uint8)
    got = grq.pack(_dev(codes)).cpu().numpy()
    assert np.array_equal(got, oracle.pack(codes))


def test_pack_bit_exact_full_size():
    lay = layer(4096, 14336, 2, 4)
    got = grq.pack(_dev(lay.codes)).cpu().numpy()
    assert np.array_equal(got, oracle.pack(lay.codes))


# ------------------------------------------------------------------ calibration

@pytest.mark.parametrize("K,N,cfg,P", [
    (256, 256, 0, synthetic.P_TINY),
    (4096, 64, 1, synthetic.P_LEVELS_5[2]),
    (4096, 64, 1, synthetic.P_LEVELS_5[3]),
    (4096, 64, 1, synthetic.P_LEVELS_5[4]),
    (4096, 64, 1, synthetic.P_LEVELS_5[8]),
    (28672, 64, 4, synthetic.P_LEVELS_4[0.5]),
    (7, 8, 5, (0.3, 0.0, 0.2, 0.5)),
    (1, 8, 5, (0.5, 0.5)),
])
def test_calibrate_bit_exact(K, N, cfg, P):
    calib = synthetic.make_calibration(K, config=cfg, matrix=0)
    want = oracle.calibrate(calib, P)
    got = grq.calibrate(_dev(calib), P).cpu().numpy()
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (got, want)


def test_calibrate_golden_vectors():
    v = np.array([[1.0, -2.0, 3.0, -4.0, 5.0], [0.5, 0.5, 8.0, -1.0, 2.0]], np.float16)
    got = grq.calibrate(_dev(v), (0.3, 0.2, 0.5)).cpu().numpy()
    assert np.array_equal(got, oracle.calibrate(v, (0.3, 0.2, 0.5)))
    assert got.tolist() == pytest.approx([1.4, 2.0], rel=1e-7)


# ------------------------------------------------------------------- assignment

def _assign_both(x, th, levels):
    bits, idx, n = grq.assign_bits(_dev(x), th, levels)
    torch.cuda.synchronize()
    b_ref = oracle.assign(x, np.asarray(th, np.float32), levels)
    i_ref, n_ref = oracle.compact(b_ref)
    n_gpu = int(n.cpu().item())
    assert np.array_equal(bits.cpu().numpy(), b_ref)
    assert n_gpu == n_ref
    assert np.array_equal(idx.cpu().numpy()[:n_gpu], i_ref)
    return b_ref


@pytest.mark.parametrize("K,cfg,P", [(256, 0, synthetic.P_TINY), (4096, 1, synthetic.P_LEVELS_5[3]),
                                     (14336, 2, synthetic.P_LEVELS_5[2]), (20000, 3, synthetic.P_LEVELS_5[4]),
                                     (28672, 4, synthetic.P_LEVELS_4[0.5]), (1, 0, synthetic.P_TINY),
                                     (4097, 1, synthetic.P_LEVELS_5[3]), (32773, 3, synthetic.P_LEVELS_5[4]),
                                     (70001, 2, synthetic.P_LEVELS_5[2]), (4095, 0, synthetic.P_TINY)])
def test_assign_bit_exact(K, cfg, P):
    levels = synthetic.LEVELS_5 if len(P) == 5 else synthetic.LEVELS_4
    th = oracle.calibrate(synthetic.make_calibration(K, config=cfg, matrix=0), P)
    x = synthetic.make_activations(K, 1, config=cfg, matrix=0)[0]
    _assign_both(x, th, levels)


def test_assign_unaligned_input():
    """x starting one element past an 8-byte boundary (the per-element path)."""
    K = 5000
    th = oracle.calibrate(synthetic.make_calibration(K, config=1, matrix=0), synthetic.P_LEVELS_5[3])
    x = synthetic.make_activations(K + 1, 1, config=1, matrix=0)[0]
    full = _dev(x)
    view = full[1:]
    assert view.data_ptr() % 8 != 0
    bits, idx, n = grq.assign_bits(view, th, synthetic.LEVELS_5)
    torch.cuda.synchronize()
    b_ref = oracle.assign(x[1:], np.asarray(th, np.float32), synthetic.LEVELS_5)
    i_ref, n_ref = oracle.compact(b_ref)
    assert np.array_equal(bits.cpu().numpy(), b_ref)
    assert int(n.cpu().item()) == n_ref
    assert np.array_equal(idx.cpu().numpy()[:n_ref], i_ref)


@pytest.mark.parametrize("offset", [1, 4, 8])
def test_assign_misaligned_views(offset):
    """x 2-, 8- and 16-byte aligned views (below 16 the element-wise loads);
    with the 16-byte aligned x, bits starts 3 bytes past an 8-byte boundary."""
    K = 9001
    th = oracle.calibrate(synthetic.make_calibration(K, config=1, matrix=1), synthetic.P_LEVELS_5[3])
    x = synthetic.make_activations(K + offset, 1, config=1, matrix=1)[0]
    view = _dev(x)[offset:]
    bits_out = torch.empty(K + 3, dtype=torch.uint8, device="cuda")[3:] if offset == 8 else None
    bits, idx, n = grq.assign_bits(view, th, synthetic.LEVELS_5, bits=bits_out)
    torch.cuda.synchronize()
    b_ref = oracle.assign(x[offset:], np.asarray(th, np.float32), synthetic.LEVELS_5)
    i_ref, n_ref = oracle.compact(b_ref)
    assert np.array_equal(bits.cpu().numpy(), b_ref)
    assert int(n.cpu().item()) == n_ref
    assert np.array_equal(idx.cpu().numpy()[:n_ref], i_ref)


@pytest.mark.parametrize("K,offset", [(131072, 0), (131073, 0), (200003, 0), (140001, 1)])
def test_assign_long_inputs(K, offset):
    """The largest chunked input (64 chunks) and the single-workgroup path past it."""
    th = oracle.calibrate(synthetic.make_calibration(K, config=2, matrix=0), synthetic.P_LEVELS_5[2])
    x = synthetic.make_activations(K + offset, 1, config=2, matrix=0)[0]
    view = _dev(x)[offset:]
    bits, idx, n = grq.assign_bits(view, th, synthetic.LEVELS_5)
    torch.cuda.synchronize()
    b_ref = oracle.assign(x[offset:], np.asarray(th, np.float32), synthetic.LEVELS_5)
    i_ref, n_ref = oracle.compact(b_ref)
    assert np.array_equal(bits.cpu().numpy(), b_ref)
    assert int(n.cpu().item()) == n_ref
    assert np.array_equal(idx.cpu().numpy()[:n_ref], i_ref)


def test_assign_special_values_in_every_chunk():
    """NaN, infinities, signed zeros, subnormals and exact threshold ties spread
    over several 2048-row chunks, under level tables whose active rows are not
    one interval of |x|: each chunk's count of the rows before it must agree
    with the widths of those rows."""
    K = 11000
    rng = np.random.default_rng(7)
    x = synthetic.make_activations(K, 1, config=7, matrix=1)[0].copy()
    specials = np.array([np.nan, np.inf, -np.inf, 0.0, -0.0, 6e-8, -6e-8, 0.5, -1.0, 2.0, -4.0, 65504.0,
                         -np.nan, 1.0009765625], np.float16)
    pos = rng.choice(K, size=700, replace=False)
    x[pos] = specials[rng.integers(0, len(specials), size=pos.size)]
    th = [0.5, 1.0, 2.0, 4.0]
    for lv in [(0, 2, 3, 4, 8), (2, 0, 8, 0, 3), (0, 3, 0, 5, 0), (1, 1, 1, 1, 1), (0, 0, 0, 0, 0),
               (5, 0, 0, 0, 0), (0, 0, 0, 0, 7), (4, 4, 0, 4, 4)]:
        _assign_both(x, th, lv)
    _assign_both(x, [0.0, 0.5, 0.5, 65504.0, float("inf")], (0, 1, 0, 2, 0, 3))
    _assign_both(x, [0.0, 0.5, 0.5, 65504.0, float("inf")], (3, 1, 0, 2, 0, 0))
    _assign_both(x, [6e-8, 1e-5, 0.25, 0.75, 1.5, 3.0, 70000.0, float("inf")], (0, 1, 0, 1, 0, 1, 0, 1, 0))


@pytest.mark.parametrize("n_th", [0, 1, 2, 3, 5, 6, 7, 8])
def test_assign_every_threshold_count(n_th):
    """One kernel per threshold count: each against the oracle."""
    K = 9000
    x = synthetic.make_activations(K, 1, config=6, matrix=n_th)[0]
    th = sorted(float(v) for v in np.random.default_rng(n_th).uniform(0.2, 8.0, size=n_th))
    levels = tuple(range(n_th + 1)) if n_th < 8 else (0, 1, 2, 3, 4, 5, 6, 7, 8)
    _assign_both(x, th, levels)


def test_assign_edge_cases():
    th = [0.5, 1.0, 2.0, 4.0]
    lv = (0, 2, 3, 4, 8)
    ties = np.array([0.0, 0.25, 0.5, -0.5, 0.75, 1.0, -1.5, 2.0, -3.0, 4.0, -100.0, 65504.0,
                     np.nan, np.inf, -np.inf, -0.0], np.float16)
    b = _assign_both(ties, th, lv)
    assert b[:12].tolist() == [0, 0, 2, 2, 2, 3, 3, 4, 4, 8, 8, 8]
    x = synthetic.make_activations(3000, 1, config=7, matrix=0)[0]
    _assign_both(x, [0.0] * 4, lv)
    _assign_both(x, [float("inf")] * 4, lv)
    _assign_both(x, [], (3,))
    _assign_both(x, [1.0, 1.0, 1.0], (1, 2, 5, 7))
    _assign_both(x, [0.3, 2.5], (2, 0, 8))       # level 0 may sit above 0


# ------------------------------------------------------------------------- VMM

CASES = [
    # (K, N, config, matrix, P, levels)
    (256, 256, 0, 0, synthetic.P_TINY, synthetic.LEVELS_5),
    (4096, 4096, 1, 0, synthetic.P_LEVELS_5[2], synthetic.LEVELS_5),
    (4096, 4096, 1, 0, synthetic.P_LEVELS_5[3], synthetic.LEVELS_5),
    (4096, 4096, 1, 0, synthetic.P_LEVELS_5[4], synthetic.LEVELS_5),
    (4096, 4096, 1, 0, synthetic.P_LEVELS_5[8], synthetic.LEVELS_5),
    (4096, 1024, 2, 1, synthetic.P_LEVELS_5[3], synthetic.LEVELS_5),
    (300, 70, 5, 0, synthetic.P_TINY, synthetic.LEVELS_5),
    (129, 1100, 5, 1, synthetic.P_LEVELS_5[4], synthetic.LEVELS_5),
    (1, 33, 5, 2, (0.0, 1.0), (0, 8)),
    (4097, 1056, 5, 3, synthetic.P_LEVELS_4[1], synthetic.LEVELS_4),
    (1000, 2080, 5, 4, synthetic.P_LEVELS_4[0.5], synthetic.LEVELS_4),
]


@pytest.mark.parametrize("K,N,cfg,mat,P,levels", CASES)
def test_decode_vmm_parity(K, N, cfg, mat, P, levels):
    lay = layer(K, N, cfg, mat)
    th = oracle.calibrate(lay.calib, P)
    x = lay.x[0]
    y, planes, ws = _run_decode(lay, x, th, levels)
    bits = oracle.assign(x, th, levels)
    _check_y(y, lay.codes, lay.scales, lay.zeros, x, bits)
    # the two-call path (assignment, then VMM from the list) gives the same bits
    b, idx, n = grq.assign_bits(_dev(x), th, levels)
    y2 = grq.vmm(planes, _dev(lay.scales), _dev(lay.zeros), _dev(x), b, idx, n, K, N, ws)
    torch.cuda.synchronize()
    assert np.array_equal(y2.cpu().numpy().view(np.uint32), y.view(np.uint32))


def test_vmm_from_oracle_assignment():
    """grinqh_vmm does not need bits produced by grinqh_assign_bits."""
    lay = layer(4096, 4096, 1, 0)
    x = lay.x[1]
    bits = np.random.default_rng(3).integers(0, 9, size=4096).astype(np.uint8)
    idx, n = oracle.compact(bits)
    planes = grq.pack(_dev(lay.codes))
    ws = grq.make_workspace(4096, 4096)
    idx_full = np.zeros(4096, np.int32)
    idx_full[:n] = idx
    y = grq.vmm(planes, _dev(lay.scales), _dev(lay.zeros), _dev(x), _dev(bits), _dev(idx_full),
                _dev(np.array([n], np.int32)), 4096, 4096, ws)
    torch.cuda.synchronize()
    _check_y(y.cpu().numpy(), lay.codes, lay.scales, lay.zeros, x, bits)


def test_vmm_list_subset():
    """Only listed rows contribute, even where bits are non-zero elsewhere."""
    lay = layer(1000, 2080, 5, 4)
    x = lay.x[0]
    bits = np.full(1000, 3, np.uint8)
    listed = np.arange(0, 1000, 7, dtype=np.int32)
    planes = grq.pack(_dev(lay.codes))
    ws = grq.make_workspace(1000, 2080)
    idx_full = np.zeros(1000, np.int32)
    idx_full[:len(listed)] = listed
    y = grq.vmm(planes, _dev(lay.scales), _dev(lay.zeros), _dev(x), _dev(bits), _dev(idx_full),
                _dev(np.array([len(listed)], np.int32)), 1000, 2080, ws)
    torch.cuda.synchronize()
    eff = np.zeros(1000, np.uint8)
    eff[listed] = 3
    _check_y(y.cpu().numpy(), lay.codes, lay.scales, lay.zeros, x, eff)


def test_all_eight_bits_equals_dense_gemv():
    lay = layer(4096, 4096, 1, 0)
    x = lay.x[0]
    y, _, _ = _run_decode(lay, x, [0.0] * 4, synthetic.LEVELS_5)
    bits = np.full(4096, 8, np.uint8)
    _check_y(y, lay.codes, lay.scales, lay.zeros, x, bits)
    g = np.arange(4096) // 128
    dense = x.astype(np.float64) @ (lay.scales[g].astype(np.float64) * lay.codes + lay.zeros[g].astype(np.float64))
    mag = oracle.vmm_abs(lay.codes, lay.scales, lay.zeros, x, bits)
    assert np.all(np.abs(y - dense) <= REL_TOL * mag + ABS_TOL)


def test_all_zero_bits_gives_zero():
    lay = layer(4096, 1024, 2, 1)
    y, _, _ = _run_decode(lay, lay.x[0], [float("inf")] * 4, synthetic.LEVELS_5)
    assert np.array_equal(y, np.zeros(1024, np.float32))


def test_deterministic_repeat():
    lay = layer(4096, 4096, 1, 0)
    th = oracle.calibrate(lay.calib, synthetic.P_LEVELS_5[3])
    planes = grq.pack(_dev(lay.codes))
    ws = grq.make_workspace(4096, 4096)
    args = (planes, _dev(lay.scales), _dev(lay.zeros), _dev(lay.x[0]), 4096, 4096, th, synthetic.LEVELS_5, ws)
    y1 = grq.decode_vmm(*args).cpu().numpy()
    y2 = grq.decode_vmm(*args).cpu().numpy()
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))


@pytest.mark.parametrize("K,N", [(4096, 1024), (6144, 256)])
def test_split_reduction_large_partials(K, N):
    """The split-K reduction with partial sums on both sides of its
    fixed-point range (2^22): column j's scale and zero are multiplied by
    2^(j mod 16) and the activations by 64, so at 4096 x 1024 (64 splits of
    64 rows, the most the fixed-point words take) most partials go as
    integers and some (224 of the 64 x 1024, counted in fp64 when the test
    was written) as floats, in one launch; 6144 x 256 (96 splits) takes the
    partial rows with the same large values.  Within tolerance of the
    oracle, bit-identical on repeat."""
    lay = layer(K, N, 2, 1)
    mult = (2.0 ** (np.arange(N) % 16)).astype(np.float32)
    scales = (lay.scales.astype(np.float32) * mult).astype(np.float16)
    zeros = (lay.zeros.astype(np.float32) * mult).astype(np.float16)
    assert np.all(np.isfinite(scales)) and np.all(np.isfinite(zeros))
    x = (lay.x[0].astype(np.float32) * 64).astype(np.float16)
    assert np.all(np.isfinite(x))
    th = oracle.calibrate(lay.calib, synthetic.P_LEVELS_5[3])
    planes = grq.pack(_dev(lay.codes))
    ws = grq.make_workspace(K, N)
    args = (planes, _dev(scales), _dev(zeros), _dev(x), K, N, th, synthetic.LEVELS_5, ws)
    y1 = grq.decode_vmm(*args).cpu().numpy()
    y2 = grq.decode_vmm(*args).cpu().numpy()
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    bits = oracle.assign(x, th, synthetic.LEVELS_5)
    ref = oracle.vmm(lay.codes, scales, zeros, x, bits)
    assert np.max(np.abs(ref)) > 2.0 ** 24, "no column reaches the float path"
    _check_y(y1, lay.codes, scales, zeros, x, bits)


def test_split_reduction_many_splits():
    """A tall, narrow layer whose split count (256 splits of 64 rows) is past
    the fixed-point reduction's 127: the partial-row path, within tolerance
    and bit-identical on repeat."""
    K, N = 16384, 256
    lay = layer(K, N, 5, 5)
    th = oracle.calibrate(lay.calib, synthetic.P_LEVELS_5[3])
    planes = grq.pack(_dev(lay.codes))
    ws = grq.make_workspace(K, N)
    args = (planes, _dev(lay.scales), _dev(lay.zeros), _dev(lay.x[0]), K, N, th, synthetic.LEVELS_5, ws)
    y1 = grq.decode_vmm(*args).cpu().numpy()
    y2 = grq.decode_vmm(*args).cpu().numpy()
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    bits = oracle.assign(lay.x[0], th, synthetic.LEVELS_5)
    _check_y(y1, lay.codes, lay.scales, lay.zeros, lay.x[0], bits)


# ------------------------------------------------- full sizes, every output

FULL = [
    (4096, 14336, 2, 4, synthetic.P_LEVELS_5[3], synthetic.LEVELS_5),
    (4096, 14336, 2, 4, synthetic.P_LEVELS_5[2], synthetic.LEVELS_5),
    (14336, 4096, 2, 6, synthetic.P_LEVELS_5[4], synthetic.LEVELS_5),
    (8192, 28672, 4, 0, synthetic.P_LEVELS_4[0.5], synthetic.LEVELS_4),
    (28672, 8192, 4, 1, synthetic.P_LEVELS_4[8], synthetic.LEVELS_4),
]


@pytest.mark.parametrize("K,N,cfg,mat,P,levels", FULL)
def test_full_size_all_columns(K, N, cfg, mat, P, levels):
    """Both fused entry points at the benchmark shapes, every output column:
    split-K, and the accumulating one in the decode-loop form the benchmark
    times (add into a zeroed buffer, clear the other)."""
    lay = layer(K, N, cfg, mat)
    th = oracle.calibrate(lay.calib, P)
    x = lay.x[0]
    y, planes, _ = _run_decode(lay, x, th, levels)
    bits = oracle.assign(x, th, levels)
    _check_y(y, lay.codes, lay.scales, lay.zeros, x, bits)
    bufs = [torch.zeros(N, dtype=torch.float32, device="cuda"), torch.ones(N, dtype=torch.float32, device="cuda")]
    grq.decode_vmm_accumulate(planes, _dev(lay.scales), _dev(lay.zeros), _dev(x), K, N, th, levels,
                              bufs[0], bufs[1])
    torch.cuda.synchronize()
    assert torch.count_nonzero(bufs[1]).item() == 0
    _check_y(bufs[0].cpu().numpy(), lay.codes, lay.scales, lay.zeros, x, bits)


EVERY_WIDTH = (0, 1, 2, 3, 4, 5, 6, 7, 8)
P_EVERY_WIDTH = (0.2, 0.1, 0.1, 0.1, 0.1, 0.1, 0.1, 0.1, 0.1)


@pytest.mark.parametrize("K,N,cfg,mat,n_cols", [(1000, 2080, 5, 4, 0), (4096, 4096, 1, 2, 0),
                                                (8192, 17408, 5, 6, 192)])
def test_every_width_in_one_launch(K, N, cfg, mat, n_cols):
    """Levels 0..8 at once (eight thresholds): records of every width, those
    that load planes 0..3 only and those that also load 4..7, in the 8-wave
    geometry and (17 column tiles x 64 groups = 1088 workgroups) the 2-wave
    one, through both fused entry points."""
    lay = layer(K, N, cfg, mat)
    th = oracle.calibrate(lay.calib, P_EVERY_WIDTH)
    x = lay.x[0]
    bits = oracle.assign(x, th, EVERY_WIDTH)
    assert set(np.unique(bits).tolist()) == set(range(9))
    cols = None
    if n_cols:
        r = np.random.default_rng(K + N + 1)
        cols = np.unique(np.concatenate([r.choice(N, n_cols, replace=False), [0, 1023, 1024, N - 1]]))
    y, planes, _ = _run_decode(lay, x, th, EVERY_WIDTH)
    _check_y(y, lay.codes, lay.scales, lay.zeros, x, bits, cols)
    acc = torch.zeros(N, dtype=torch.float32, device="cuda")
    grq.decode_vmm_accumulate(planes, _dev(lay.scales), _dev(lay.zeros), _dev(x), K, N, th, EVERY_WIDTH, acc)
    torch.cuda.synchronize()
    _check_y(acc.cpu().numpy(), lay.codes, lay.scales, lay.zeros, x, bits, cols)


# ------------------------------------------------------ accumulating entry point

@pytest.mark.parametrize("K,N,cfg,mat,P,levels", [CASES[0], CASES[2], CASES[4], CASES[5], CASES[7], CASES[8], CASES[9]])
def test_decode_vmm_accumulate_parity(K, N, cfg, mat, P, levels):
    lay = layer(K, N, cfg, mat)
    th = oracle.calibrate(lay.calib, P)
    x = lay.x[0]
    planes = grq.pack(_dev(lay.codes))
    y0 = np.random.default_rng(K + N).standard_normal(N).astype(np.float32)
    y = _dev(y0.copy())
    clear = torch.ones(N, dtype=torch.float32, device="cuda")
    grq.decode_vmm_accumulate(planes, _dev(lay.scales), _dev(lay.zeros), _dev(x), K, N, th, levels, y, clear)
    torch.cuda.synchronize()
    assert torch.count_nonzero(clear).item() == 0
    bits = oracle.assign(x, th, levels)
    ref = oracle.vmm(lay.codes, lay.scales, lay.zeros, x, bits) + y0.astype(np.float64)
    mag = oracle.vmm_abs(lay.codes, lay.scales, lay.zeros, x, bits) + np.abs(y0.astype(np.float64))
    err = np.abs(y.cpu().numpy().astype(np.float64) - ref)
    assert np.all(err <= REL_TOL * mag + ABS_TOL)


def test_decode_vmm_accumulate_ping_pong():
    """Two buffers alternate: each call adds into one and clears the other."""
    lay = layer(4096, 4096, 1, 0)
    th = oracle.calibrate(lay.calib, synthetic.P_LEVELS_5[3])
    planes = grq.pack(_dev(lay.codes))
    sc, zr = _dev(lay.scales), _dev(lay.zeros)
    bufs = [torch.zeros(4096, dtype=torch.float32, device="cuda") for _ in range(2)]
    for step in range(3):
        x = lay.x[step % 2]
        grq.decode_vmm_accumulate(planes, sc, zr, _dev(x), 4096, 4096, th, synthetic.LEVELS_5,
                                  bufs[step % 2], bufs[(step + 1) % 2])
        torch.cuda.synchronize()
        _check_y(bufs[step % 2].cpu().numpy(), lay.codes, lay.scales, lay.zeros, x,
                 oracle.assign(x, th, synthetic.LEVELS_5))
        assert torch.count_nonzero(bufs[(step + 1) % 2]).item() == 0


# ------------------------------------------------------- every workgroup shape

# Layers whose shapes select each less common workgroup shape of the VMM
# (waves x sub-items x rows): 8 x 1 x 64 with two workgroups per CU (a few
# hundred 128-row units), 4 x 1 x 128 (several small workgroups per CU, the
# rolled record loop), 16 x 4 x 128 (one 512-row item per CU), exact and
# ragged in K and N.
SHAPE_CASES = [
    (2048, 9216, 2, 5, synthetic.P_LEVELS_5[3], synthetic.LEVELS_5),
    (2100, 9000, 5, 6, synthetic.P_LEVELS_5[2], synthetic.LEVELS_5),
    (4096, 24576, 2, 6, synthetic.P_LEVELS_5[3], synthetic.LEVELS_5),
    (4000, 24000, 5, 7, synthetic.P_LEVELS_5[4], synthetic.LEVELS_5),
    (8192, 16384, 2, 7, synthetic.P_LEVELS_5[3], synthetic.LEVELS_5),
    (8000, 16000, 5, 8, synthetic.P_LEVELS_4[1], synthetic.LEVELS_4),
]


@pytest.mark.parametrize("K,N,cfg,mat,P,levels", SHAPE_CASES)
def test_every_workgroup_shape(K, N, cfg, mat, P, levels):
    """All three entry points (split-K fused, list, accumulate) on every
    column, against the oracle; the split-K and list results bit-identical."""
    lay = synthetic.make_layer(K, N, config=cfg, matrix=mat, n_test=1)
    th = oracle.calibrate(lay.calib, P)
    x = lay.x[0]
    y, planes, ws = _run_decode(lay, x, th, levels)
    bits = oracle.assign(x, th, levels)
    _check_y(y, lay.codes, lay.scales, lay.zeros, x, bits)
    b, idx, n = grq.assign_bits(_dev(x), th, levels)
    y2 = grq.vmm(planes, _dev(lay.scales), _dev(lay.zeros), _dev(x), b, idx, n, K, N, ws)
    acc = torch.zeros(N, dtype=torch.float32, device="cuda")
    grq.decode_vmm_accumulate(planes, _dev(lay.scales), _dev(lay.zeros), _dev(x), K, N, th, levels, acc)
    torch.cuda.synchronize()
    assert np.array_equal(y2.cpu().numpy().view(np.uint32), y.view(np.uint32))
    _check_y(acc.cpu().numpy(), lay.codes, lay.scales, lay.zeros, x, bits)


# ------------------------------------------------------- grouped launches

# the group's shape (waves x sub-items x rows) in order: 8x1x64, 8x1x64,
# 4x1x128, 8x1x64, 8x1x64, 16x2x128, 16x4x128, 16x8x128
@pytest.mark.parametrize("K,Ns,b_max", [(4096, (4096, 1024, 1024), 8), (1000, (300, 1100, 70, 2080), 8),
                                        (4096, (12288, 12288), 8), (777, (1056, 513), 6), (64, (33,), 8),
                                        (4096, (8192, 6144), 8), (4096, (16384, 16384), 8),
                                        (8192, (14336, 14336), 8)])
def test_grouped_launch_members(K, Ns, b_max):
    """Every member of a grouped launch against the oracle on every column,
    each with its own store, activation and thresholds; the clear buffers
    zeroed; members that share no shape with the group's choice included."""
    members, refs = [], []
    for i, N in enumerate(Ns):
        lay = synthetic.make_layer(K, N, config=5, matrix=20 + i, n_test=1, b_max=b_max)
        levels = (0, 2, 3, 4, b_max) if b_max > 4 else (0, 1, 2, 3, 4)
        th = oracle.calibrate(lay.calib, synthetic.P_LEVELS_5[3])
        x = lay.x[0]
        y0 = np.random.default_rng(i).standard_normal(N).astype(np.float32)
        y = _dev(y0.copy())
        clear = torch.ones(N, dtype=torch.float32, device="cuda")
        members.append((grq.pack(_dev(lay.codes), b_max=b_max), _dev(lay.scales), _dev(lay.zeros), _dev(x), N, th,
                        levels, y, clear))
        refs.append((lay, x, oracle.assign(x, th, levels), y0))
    grq.decode_vmm_accumulate_group(members, K, b_max=b_max)
    torch.cuda.synchronize()
    for m, (lay, x, bits, y0) in zip(members, refs):
        assert torch.count_nonzero(m[8]).item() == 0
        ref = oracle.vmm(lay.codes, lay.scales, lay.zeros, x, bits, b_max=b_max) + y0.astype(np.float64)
        mag = oracle.vmm_abs(lay.codes, lay.scales, lay.zeros, x, bits, b_max=b_max) + np.abs(y0.astype(np.float64))
        err = np.abs(m[7].cpu().numpy().astype(np.float64) - ref)
        assert np.all(err <= REL_TOL * mag + ABS_TOL)
