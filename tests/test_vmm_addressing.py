"""Host model of the VMM kernel's plane-load addressing (csrc/vmm.hip).

The kernel reads plane words with raw buffer loads: a per-workgroup buffer
over its row item's row tiles, a per-lane voffset (row tile start + 4 l, or
an out-of-range value) and a scalar plane offset p * pb.  Only the voffset
is range-checked by the hardware, so every load whose voffset passes must
stay inside the row's own top-b span by construction.  This model restates
that arithmetic (launch shape, buffer base and size, lane offsets, plane
offsets) and checks it for ragged shapes and every b_max.  It uses the
store geometry of the oracle only to name where each row tile starts.
"""
import pytest

import oracle

OUT_OF_RANGE = 0x7FFFFF00
TARGET_CUS = 256


def _launch(K, N):
    Np = oracle.padded_cols(N)
    tiles = (Np + 1023) // 1024
    groups = (K + 127) // 128
    rows = 64 if groups * tiles < TARGET_CUS else 128
    return Np, tiles, rows, (K + rows - 1) // rows


def _check(K, N, b_max):
    Np, tiles, rows, splits = _launch(K, N)
    store = oracle.planes_bytes(K, N, b_max)
    for split in range(splits):
        k0, k1 = split * rows, min(split * rows + rows, K)
        for tile in range(tiles):
            t0 = tile * 1024
            ct = min(1024, Np - t0)
            pb = ct // 8
            rstride = pb * b_max
            off8 = t0 * K + k0 * ct
            assert off8 % 8 == 0
            base = off8 // 8 * b_max
            size = (k1 - k0) * rstride
            assert base + size <= store
            for rq in range(k1 - k0):
                start = oracle.plane_offset(K, N, tile, k0 + rq, 0, b_max)
                assert base + rq * rstride == start
                for lane in range(32):
                    lane_off = 4 * lane if 4 * lane < pb else OUT_OF_RANGE
                    voff = rq * rstride + lane_off
                    if voff >= size:
                        continue           # out of range: the load returns 0
                    for b in range(1, b_max + 1):
                        for p in range(8):
                            addr = base + voff + (p * pb if p < b else 0)
                            assert start <= addr and addr + 4 <= start + b * pb, (K, N, b_max, rq, lane, b, p)


@pytest.mark.parametrize("K,N", [(7, 33), (129, 1100), (300, 70), (130, 1056), (1, 33), (200, 2100)])
@pytest.mark.parametrize("b_max", [1, 4, 6, 8])
def test_every_load_stays_in_its_rows_span(K, N, b_max):
    _check(K, N, b_max)
