"""The entry points inside a captured HIP graph, the way the benchmark times
them: one capture, several replays with eager work in between, every replay
checked (against the oracle, and bit for bit against the eager call where
the result is deterministic).  Nothing is cleared with a memset node: the
accumulating entry points clear the next output buffer themselves and the
split-K counters reset themselves."""
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


def _check(y, codes, scales, zeros, x, bits):
    ref = oracle.vmm(codes, scales, zeros, x, bits)
    mag = oracle.vmm_abs(codes, scales, zeros, x, bits)
    err = np.abs(y.astype(np.float64) - ref)
    assert np.all(err <= REL_TOL * mag + ABS_TOL)


def test_graph_replays_match_eager_and_oracle():
    K, N = 4096, 4096
    lay = synthetic.make_layer(K, N, config=1, matrix=0, n_test=4)
    P, levels = synthetic.P_LEVELS_5[3], synthetic.LEVELS_5
    th = oracle.calibrate(lay.calib, P)
    planes = grq.pack(_dev(lay.codes))
    sc, zr = _dev(lay.scales), _dev(lay.zeros)
    xs = [_dev(lay.x[i]) for i in range(4)]
    ws = grq.make_workspace(K, N)
    bufs = [torch.zeros(N, dtype=torch.float32, device="cuda") for _ in range(2)]
    y_split = torch.empty(N, dtype=torch.float32, device="cuda")
    y_list = torch.empty(N, dtype=torch.float32, device="cuda")
    bits = torch.empty(K, dtype=torch.uint8, device="cuda")
    idx = torch.empty(K, dtype=torch.int32, device="cuda")
    nact = torch.empty(1, dtype=torch.int32, device="cuda")
    # table path and prefill on small shapes
    Kl, Nl = 1024, 1024
    lcodes, tables = synthetic.make_lut_weights(Kl, Nl, config=5, matrix=8)
    lplanes = grq.pack(_dev(lcodes))
    lut = _dev(synthetic.lut_flat(tables, Nl, 8))
    lcalib = synthetic.make_calibration(Kl, config=5, matrix=8)
    lth = oracle.calibrate(lcalib, P)
    lx = synthetic.make_activations(Kl, 1, config=5, matrix=8)[0]
    lbufs = [torch.zeros(Nl, dtype=torch.float32, device="cuda") for _ in range(2)]
    play = synthetic.make_layer(512, 384, config=5, matrix=9, n_test=1)
    pplanes = grq.pack(_dev(play.codes))
    X = synthetic.make_activations(512, 130, config=5, matrix=9)
    Xd = _dev(X)
    Yp = torch.empty((130, 384), dtype=torch.float32, device="cuda")
    # grouped launches: two members on the same store with their own x
    gy = [torch.zeros(N, dtype=torch.float32, device="cuda") for _ in range(4)]

    def steps():
        for k in range(4):   # decode loop: add into one buffer, clear the other
            grq.decode_vmm_accumulate(planes, sc, zr, xs[k], K, N, th, levels, bufs[k % 2], bufs[(k + 1) % 2])
        grq.decode_vmm(planes, sc, zr, xs[3], K, N, th, levels, ws, out=y_split)
        grq.assign_bits(xs[2], th, levels, bits, idx, nact)
        grq.vmm(planes, sc, zr, xs[2], bits, idx, nact, K, N, ws, out=y_list)
        for k in range(2):
            grq.decode_vmm_lut(lplanes, lut, lxd, Kl, Nl, lth, levels, lbufs[k % 2],
                               lbufs[(k + 1) % 2])
        grq.prefill(pplanes, psc, pzr, Xd, 512, 384, out=Yp)
        for half in range(2):   # add into one pair, clear the other
            a, c = (0, 2) if half == 0 else (2, 0)
            grq.decode_vmm_accumulate_group([(planes, sc, zr, xs[0], N, th, levels, gy[a], gy[c]),
                                             (planes, sc, zr, xs[1], N, th, levels, gy[a + 1], gy[c + 1])], K)

    lxd = _dev(lx)
    psc, pzr = _dev(play.scales), _dev(play.zeros)
    # eager reference of the deterministic results
    steps()
    torch.cuda.synchronize()
    eager_split = y_split.clone()
    eager_list = y_list.clone()
    eager_prefill = Yp.clone()

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            steps()
    torch.cuda.synchronize()

    b3 = oracle.assign(lay.x[3], th, levels)
    b2 = oracle.assign(lay.x[2], th, levels)
    lbits = oracle.assign(lx, lth, levels)
    lref = oracle.vmm_lut(lcodes, tables, lx, lbits)
    lmag = oracle.vmm_lut_abs(lcodes, tables, lx, lbits)
    pref = oracle.prefill(play.codes, play.scales, play.zeros, X)
    pmag = oracle.prefill_abs(play.codes, play.scales, play.zeros, X)
    for rep in range(3):
        # eager work between replays, touching the same buffers
        for t in (bufs + lbufs + gy + [y_split, y_list, Yp]):
            t.fill_(float(rep + 7))
        grq.decode_vmm(planes, sc, zr, xs[0], K, N, th, levels, ws, out=y_split)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        # after the 4-step loop, buffer 1 holds x_3 W and buffer 0 was cleared
        _check(bufs[1].cpu().numpy(), lay.codes, lay.scales, lay.zeros, lay.x[3], b3)
        assert torch.count_nonzero(bufs[0]).item() == 0
        assert torch.equal(y_split, eager_split)
        assert torch.equal(y_list, eager_list)
        _check(y_split.cpu().numpy(), lay.codes, lay.scales, lay.zeros, lay.x[3], b3)
        _check(y_list.cpu().numpy(), lay.codes, lay.scales, lay.zeros, lay.x[2], b2)
        ly = lbufs[1].cpu().numpy().astype(np.float64)
        assert np.all(np.abs(ly - lref) <= REL_TOL * lmag + ABS_TOL)
        assert torch.count_nonzero(lbufs[0]).item() == 0
        assert torch.equal(Yp, eager_prefill)
        _check(gy[2].cpu().numpy(), lay.codes, lay.scales, lay.zeros, lay.x[0], oracle.assign(lay.x[0], th, levels))
        _check(gy[3].cpu().numpy(), lay.codes, lay.scales, lay.zeros, lay.x[1], oracle.assign(lay.x[1], th, levels))
        assert torch.count_nonzero(gy[0]).item() == 0 and torch.count_nonzero(gy[1]).item() == 0
        assert np.all(np.abs(Yp.cpu().numpy().astype(np.float64) - pref) <= REL_TOL * pmag + ABS_TOL)
