"""One token through the 36-layer Qwen3-8B linear stack (252 VMMs in 252
launches or, grouped, in 144; or 144 VMMs with q|k|v and gate|up packed side
by side; the whole 8-plane store resident), in the launch configuration the
stack benchmark times, checked on sampled columns of every VMM against the
fp64 oracle.

Per matrix: the GPU's calibrated thresholds must equal the oracle's bit for
bit, and every sampled output must satisfy
|y - y_ref| <= 1e-3 * sum_i |x_i w_ij| + 1e-4.
"""
import sys

import numpy as np
import pytest

import oracle
import synthetic

torch = pytest.importorskip("torch")
import decode_stage_gemv_amd as grq  # noqa: E402,F401

pytestmark = pytest.mark.gpu

REL_TOL = 1e-3
ABS_TOL = 1e-4


@pytest.mark.parametrize("fused,grouped", [(False, False), (False, True), (True, False)],
                         ids=["per-matrix", "per-matrix-grouped-launches", "fused-projections"])
def test_qwen3_stack_one_token_sampled_columns(fused, grouped):
    import bench
    print(f"building the Qwen3-8B stack (fused={fused}, grouped={grouped})", file=sys.stderr, flush=True)
    st = bench.Stack(keep_cols=6, fused=fused, grouped=grouped)
    assert len(st.mats) == (144 if fused else 252)
    assert st.launches == (252 if not (fused or grouped) else 144)
    st.token(0)                      # adds into output set 0 (zero), clears set 1
    torch.cuda.synchronize()
    bad = []
    for j, m in enumerate(st.mats):
        K = m["K"]
        calib = synthetic.make_calibration(K, synthetic.STACK_CONFIG, m["idx"])
        th = oracle.calibrate(calib, st.P)
        assert np.array_equal(np.asarray(m["thresholds"], np.float32).view(np.uint32),
                              np.asarray(th, np.float32).view(np.uint32)), f"thresholds of matrix {m['idx']}"
        bits = oracle.assign(m["x_host"], th, st.levels)
        codes, scales, zeros = m["host"]
        ref = oracle.vmm(codes, scales, zeros, m["x_host"], bits)
        mag = oracle.vmm_abs(codes, scales, zeros, m["x_host"], bits)
        got = st.ys[0][j].cpu().numpy()[m["cols"]].astype(np.float64)
        err = np.abs(got - ref)
        if not np.all(err <= REL_TOL * mag + ABS_TOL):
            bad.append((m["idx"], m["name"], float(err.max())))
        assert not torch.any(st.ys[1][j]).item(), f"output set 1 of matrix {m['idx']} not cleared"
    assert not bad, f"matrices out of tolerance: {bad[:5]}"
    del st
    torch.cuda.empty_cache()
