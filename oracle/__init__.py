"""fp64 CPU oracle for the GRINQH decode-stage VMM (test infrastructure only).

Only the tests, the smoke check and the CPU-baseline leg of bench.py may
import this package; the HIP library never does.
"""
from .grinqh_oracle import (  # noqa: F401
    B_MAX, GROUP, TILE, WORD, PAD,
    cut_points, empirical_quantile, calibrate,
    assign, compact,
    padded_cols, tiles, planes_bytes, plane_offset, pack, read_planes, span_bytes,
    reconstruct_level, vmm, vmm_abs, decode_step, bytes_read,
    dequant_dense, dequant_dense_fp16, prefill, prefill_abs,
    vmm_lut, vmm_lut_abs,
)
