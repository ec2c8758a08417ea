"""grinqh_decode_vmm_noalloc (the entry point for callers that cannot
allocate) against grinqh_decode_vmm with a caller workspace, through the C
ABI: bit-identical outputs (the same kernels and the same fixed-order split-K
sum), and within the parity bound of the fp64 oracle.  Several calls in a
row on the one device array, each a different shape (a smaller layer after a
larger one puts its tile counters where the larger one's partial rows were
if the counters did not have a fixed place), and one call replayed from a
captured HIP graph."""
import ctypes

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


def _case(K, N, cfg, mat, P, levels):
    lay = synthetic.make_layer(K, N, config=cfg, matrix=mat, n_test=1)
    th = [float(t) for t in oracle.calibrate(lay.calib, P)]
    return lay, th, levels


def _host(th, levels):
    n = len(th)
    return (ctypes.c_float * max(n, 1))(*th), (ctypes.c_uint8 * (n + 1))(*levels), n


def _run_both(lay, th, levels):
    K, N = lay.K, lay.N
    planes = grq.pack(_dev(lay.codes))
    sc, zr, x = _dev(lay.scales), _dev(lay.zeros), _dev(lay.x[0])
    lib = grq.lib()
    cth, clv, n = _host(th, levels)
    stream = torch.cuda.current_stream().cuda_stream
    y_na = torch.full((N,), float("nan"), dtype=torch.float32, device="cuda")
    st = lib.grinqh_decode_vmm_noalloc(planes.data_ptr(), sc.data_ptr(), zr.data_ptr(), x.data_ptr(), K, N, 8,
                                       cth, clv, n, y_na.data_ptr(), stream)
    assert st == grq.OK, lib.grinqh_last_error()
    ws = grq.make_workspace(K, N)
    y_ws = torch.full((N,), float("nan"), dtype=torch.float32, device="cuda")
    st = lib.grinqh_decode_vmm(planes.data_ptr(), sc.data_ptr(), zr.data_ptr(), x.data_ptr(), K, N, 8,
                               cth, clv, n, y_ws.data_ptr(), ws.data_ptr(), ws.numel(), stream)
    assert st == grq.OK, lib.grinqh_last_error()
    torch.cuda.synchronize()
    return y_na.cpu().numpy(), y_ws.cpu().numpy()


def _check_oracle(y, lay, th, levels):
    x = lay.x[0]
    bits = oracle.assign(x, np.asarray(th, np.float32), levels)
    ref = oracle.vmm(lay.codes, lay.scales, lay.zeros, x, bits)
    mag = oracle.vmm_abs(lay.codes, lay.scales, lay.zeros, x, bits)
    err = np.abs(y.astype(np.float64) - ref)
    assert np.all(err <= REL_TOL * mag + ABS_TOL)


SEQUENCE = [
    (4096, 14336, 2, 4, synthetic.P_LEVELS_5[3], synthetic.LEVELS_5),   # 32 splits x 14 tiles
    (300, 1100, 0, 3, synthetic.P_TINY, synthetic.LEVELS_5),            # smaller, ragged: 5 x 2
    (8192, 28672, 4, 0, synthetic.P_LEVELS_4[0.5], synthetic.LEVELS_4),  # the largest benchmark layer
    (1000, 2080, 5, 4, synthetic.P_TINY, synthetic.LEVELS_5),           # smaller again
]


def test_noalloc_matches_workspace_entry_point_calls_in_a_row():
    for K, N, cfg, mat, P, levels in SEQUENCE:
        lay, th, lv = _case(K, N, cfg, mat, P, levels)
        y_na, y_ws = _run_both(lay, th, lv)
        assert np.array_equal(y_na.view(np.uint32), y_ws.view(np.uint32)), (K, N)
        _check_oracle(y_na, lay, th, lv)


def test_noalloc_in_a_captured_graph():
    """Replays of a graph holding two allocation-free calls of different
    shapes, with eager calls of the workspace entry point between the
    replays; every replay matches the eager result bit for bit."""
    cases = [_case(*SEQUENCE[0]), _case(*SEQUENCE[1])]
    prepared = []
    for lay, th, lv in cases:
        planes = grq.pack(_dev(lay.codes))
        prepared.append((lay, th, lv, planes, _dev(lay.scales), _dev(lay.zeros), _dev(lay.x[0]),
                         torch.zeros(lay.N, dtype=torch.float32, device="cuda")))
    # one eager call first: the first call on a device resolves the array's
    # device address (a runtime query, no allocation)
    lay, th, lv, planes, sc, zr, x, y = prepared[0]
    grq.decode_vmm_noalloc(planes, sc, zr, x, lay.K, lay.N, th, lv, y)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for lay, th, lv, planes, sc, zr, x, y in prepared:
                grq.decode_vmm_noalloc(planes, sc, zr, x, lay.K, lay.N, th, lv, y, stream=s)
    torch.cuda.synchronize()
    eager = []
    for lay, th, lv, planes, sc, zr, x, y in prepared:
        ws = grq.make_workspace(lay.K, lay.N)
        eager.append(grq.decode_vmm(planes, sc, zr, x, lay.K, lay.N, th, lv, ws).cpu().numpy())
    for rep in range(3):
        for _, _, _, _, _, _, _, y in prepared:
            y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for (lay, th, lv, *_, y), want in zip(prepared, eager):
            got = y.cpu().numpy()
            assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), rep
        # eager work between replays
        lay, th, lv, planes, sc, zr, x, _ = prepared[1]
        grq.decode_vmm(planes, sc, zr, x, lay.K, lay.N, th, lv, grq.make_workspace(lay.K, lay.N))
        torch.cuda.synchronize()
