"""fp64 CPU oracle for the GRINQH decode-stage vector-matrix multiply.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import or call
this module.  The HIP library never uses it, and it shares no code with the
library (no kernels, headers, tables or helpers).

Source: "GRINQH: Graded Input-based Quantization Hierarchy for Efficient LLM
Generation" (arXiv 2606.23419).  Each function names the section or equation
it follows.  Where the paper is silent the plainest reading is taken; each
such reading is marked "Reading:" below.

Pins: every function here is checked by the CPU tests against something other
than itself: hand-worked examples (tests/golden/), exact rational brute force
on small inputs, closed forms (the dense GEMV at full width, zero at width 0,
a mixture quantile for the thresholds), library routines for special cases
(NumPy's quantile and packbits) and invariants (nesting, half-bin bound,
one-hot rows, linearity).  The paper prints no absolute output of the method,
so none of these pins reproduces a number from the paper itself.

Notation: K input rows (d_in), N output columns (d_out), b_max the bit width
of the stored codes (8 unless a function is told otherwise; section 3.3
evaluates b_max in {4, 6, 8}), groups of 128 rows share one (scale, zero) pair
per column, x is the fp16 activation of the current token.
"""
from __future__ import annotations

import math

import numpy as np

B_MAX = 8
GROUP = 128

# Bit-plane store geometry.  These are this project's choice of the layout the
# paper describes by its properties only (section 3.3 "Storage Layout and
# Weight Loading", Appendix C.1): input-major rows, most significant plane
# first, the top b planes of one row one contiguous span.
TILE = 1024          # output columns per row tile
WORD = 32            # columns per 32-bit plane word
PAD = 128            # N is padded to a multiple of this many columns


# --------------------------------------------------------------------------
# Threshold calibration -- section 3.2 "Threshold Calibration"; Appendix A.1,
# "Implementation via GRINQH", eq. (2).
# --------------------------------------------------------------------------

def cut_points(P) -> list[float]:
    """c_k = sum_{j<k} p_j for k = 1..n, accumulated left to right in fp64.

    theta_k is the c_k-th percentile of |x| (section 3.2).
    """
    cuts = []
    acc = 0.0
    for k in range(1, len(P)):
        acc = acc + float(P[k - 1])
        cuts.append(acc)
    return cuts


def empirical_quantile(values_sorted: np.ndarray, c: float) -> float:
    """Linear-interpolation quantile of an ascending fp64 sample.

    Reading: the paper does not name a percentile estimator; the linear one
    (the default of NumPy and PyTorch) is taken.  Position h = c (K - 1)
    between the order statistics a[floor(h)] and a[floor(h) + 1]:
    Q = a_lo + (h - floor(h)) * (a_hi - a_lo), evaluated in that order.
    """
    K = values_sorted.shape[0]
    h = c * float(K - 1)
    lo = int(math.floor(h))
    lo = min(max(lo, 0), K - 1)
    hi = min(lo + 1, K - 1)
    frac = h - float(lo)
    a_lo = float(values_sorted[lo])
    a_hi = float(values_sorted[hi])
    return a_lo + frac * (a_hi - a_lo)


def calibrate(calib: np.ndarray, P) -> np.ndarray:
    """Per-layer thresholds Theta = (theta_1..theta_n) as fp32.

    For every calibration vector v the c_k-th percentile of |v| is taken, and
    the per-vector values are averaged (section 3.2; Appendix A.1 eq. (2)).

    Readings:
    * One calibration vector is one token's activation over the K inputs.
    * The mean is accumulated vector by vector in fp64 and divided by the
      vector count, then rounded to fp32 (thresholds are compared in fp32).
    * c_k <= 0 gives theta_k = 0 (the theta_0 = 0 boundary of section 3.1:
      nothing lies below it), c_k >= 1 gives theta_k = +inf (the theta_{n+1}
      boundary), so a level with p = 0 is never assigned.
    * Eq. (2) lists theta_1..theta_{n-1}; section 3.1 needs theta_1..theta_n
      for n + 1 levels, which is what is computed here.
    """
    calib = np.asarray(calib)
    V, K = calib.shape
    cuts = cut_points(P)
    out = np.empty(len(cuts), dtype=np.float32)
    sorted_rows = [np.sort(np.abs(calib[v].astype(np.float64))) for v in range(V)]
    for k, c in enumerate(cuts):
        if c <= 0.0:
            out[k] = np.float32(0.0)
            continue
        if c >= 1.0:
            out[k] = np.float32(np.inf)
            continue
        total = 0.0
        for v in range(V):
            total = total + empirical_quantile(sorted_rows[v], c)
        out[k] = np.float32(total / float(V))
    return out


# --------------------------------------------------------------------------
# Dynamic precision assignment -- section 3.1, and active-row selection.
# --------------------------------------------------------------------------

def assign(x: np.ndarray, thresholds: np.ndarray, levels) -> np.ndarray:
    """b_i = b_k when |x_i| lies in [theta_k, theta_{k+1}) (section 3.1).

    With non-decreasing thresholds the bin index is the number of thresholds
    that |x_i| reaches, k_i = #{t : |x_i| >= theta_t}; the comparison is made
    in fp32 (fp16 -> fp32 is exact).  A tie |x_i| = theta_k lands in the upper
    bin, as the half-open interval says.  Reading: NaN compares false
    everywhere and so takes b_0.
    """
    ax = np.abs(np.asarray(x, dtype=np.float16).astype(np.float32))
    th = np.asarray(thresholds, dtype=np.float32)
    k = np.zeros(ax.shape, dtype=np.int64)
    for t in range(th.shape[0]):
        k += (ax >= th[t]).astype(np.int64)
    lv = np.asarray(levels, dtype=np.int64)
    return lv[k].astype(np.uint8)


def compact(bits: np.ndarray):
    """Ascending list of rows with b_i > 0 and its length.

    Rows with b_i = 0 are skipped entirely: the paper treats 0 bits as
    sparsification that bypasses the load (sections 2 and 3).  Reading: the
    list is ascending, so it has exactly one correct value.
    """
    idx = np.nonzero(np.asarray(bits) > 0)[0].astype(np.int32)
    return idx, int(idx.shape[0])


# --------------------------------------------------------------------------
# Bit-plane store -- section 3.3 "Storage Layout and Weight Loading";
# Appendix C.1 "Sparse bit-loading", "Bit-packing", "Grouping".
# --------------------------------------------------------------------------

def padded_cols(N: int) -> int:
    return ((N + PAD - 1) // PAD) * PAD


def tiles(N: int):
    """(start column, width) of each row tile; widths are multiples of 128."""
    Np = padded_cols(N)
    return [(t0, min(TILE, Np - t0)) for t0 in range(0, Np, TILE)]


def _check_bmax(b_max: int) -> int:
    b_max = int(b_max)
    if not 1 <= b_max <= 8:
        raise ValueError(f"b_max = {b_max}, expected 1..8")
    return b_max


def planes_bytes(K: int, N: int, b_max: int = B_MAX) -> int:
    """Store size: b_max planes of N_pad / 8 bytes per row."""
    return K * padded_cols(N) * _check_bmax(b_max) // 8


def plane_offset(K: int, N: int, t: int, i: int, p: int, b_max: int = B_MAX) -> int:
    """Byte offset of plane p (0 = most significant) of row i in tile t.

    Tile t is a block of K row tiles; a row tile holds its b_max planes back
    to back, C_t / 8 bytes each, so planes 0..b-1 form one contiguous span.
    A b_max-bit store is the 8-bit one with fewer planes per row (section 3.3:
    the same format for any maximum width; Appendix C.1: a smaller b_max just
    stops earlier).
    """
    b_max = _check_bmax(b_max)
    t0, ct = tiles(N)[t]
    return (t * K * TILE + i * ct) * b_max // 8 + p * (ct // 8)


def pack(codes: np.ndarray, b_max: int = B_MAX) -> np.ndarray:
    """b_max-bit codes [K][N] -> MSB-first bit planes (the store above).

    Plane p holds bit (b_max - 1 - p) of the code.  Within a plane, 32
    consecutive columns form one little-endian 32-bit word.  Column
    32w + 4m + j (m = 0..7, j = 0..3) of the word sits at bit 8j + m, so byte j
    of a plane word holds the plane bits of columns j, 4+j, ..., 28+j.  (The
    paper groups and permutes packed bits offline so that the kernel rebuilds
    codes with OR and SHIFT only, Appendix C.1 "Grouping"; this is this
    project's permutation for 1-bit planes.)  Padding columns N..N_pad-1 hold
    code 0.  Codes must lie in [0, 2^b_max).
    """
    b_max = _check_bmax(b_max)
    codes = np.asarray(codes, dtype=np.uint8)
    if codes.size and int(codes.max()) >= (1 << b_max):
        raise ValueError(f"a code exceeds {b_max} bits")
    K, N = codes.shape
    Np = padded_cols(N)
    q = np.zeros((K, Np), dtype=np.uint8)
    q[:, :N] = codes
    out = np.zeros(planes_bytes(K, N, b_max), dtype=np.uint8)
    for t, (t0, ct) in enumerate(tiles(N)):
        W = ct // WORD
        sub = q[:, t0:t0 + ct].reshape(K, W, 8, 4)          # [i][w][m][j]
        block = np.empty((K, b_max, ct // 8), dtype=np.uint8)
        for p in range(b_max):
            bit = (sub >> (b_max - 1 - p)) & 1                # plane p = bit b_max-1-p
            bit = np.ascontiguousarray(bit.transpose(0, 1, 3, 2))   # [i][w][j][m]
            by = np.packbits(bit, axis=-1, bitorder="little")       # byte j, bit m
            block[:, p, :] = by.reshape(K, W * 4)
        base = plane_offset(K, N, t, 0, 0, b_max)
        out[base:base + block.size] = block.reshape(-1)
    return out


def read_planes(planes: np.ndarray, K: int, N: int, bits: np.ndarray, b_max: int = B_MAX) -> np.ndarray:
    """Codes as seen through the store: the top b_i planes of row i.

    Returns u8 [K][N] holding q_b * 2^(b_max - b) (the b-bit prefix of the
    code in its original bit positions, low bits zero).  Reads only the planes
    a row needs (section 3.3: load the most significant segments only).
    """
    b_max = _check_bmax(b_max)
    planes = np.asarray(planes, dtype=np.uint8)
    bits = np.asarray(bits)
    out = np.zeros((K, padded_cols(N)), dtype=np.uint8)
    for t, (t0, ct) in enumerate(tiles(N)):
        W = ct // WORD
        for i in range(K):
            b = int(bits[i])
            if b > b_max:
                raise ValueError(f"row {i}: {b} bits from a {b_max}-bit store")
            start = plane_offset(K, N, t, i, 0, b_max)
            span = planes[start:start + b * (ct // 8)]
            acc = np.zeros(ct, dtype=np.uint8)
            for p in range(b):
                by = span[p * (ct // 8):(p + 1) * (ct // 8)].reshape(W, 4, 1)
                bit = np.unpackbits(by, axis=-1, bitorder="little")      # [w][j][m]
                bit = bit.transpose(0, 2, 1).reshape(ct)                 # col 32w+4m+j
                acc |= (bit << (b_max - 1 - p)).astype(np.uint8)
            out[i, t0:t0 + ct] = acc
    return out[:, :N]


def span_bytes(K: int, N: int, bits: np.ndarray) -> int:
    """Bytes a reader of the store touches: b_i * C_t / 8 per (row, tile)."""
    bits = np.asarray(bits, dtype=np.int64)
    return int(sum(int(bits.sum()) * (ct // 8) for _, ct in tiles(N)))


# --------------------------------------------------------------------------
# Truncated reconstruction and the VMM -- section 3.3 "Weight Reconstruction
# and Bias Correction".
# --------------------------------------------------------------------------

def reconstruct_level(q: np.ndarray, b: int, b_max: int = B_MAX) -> np.ndarray:
    """q_b 2^(b_max - b) + phi for b_max-bit codes q at bit width b, as fp64.

    q_b = floor(q / 2^(b_max - b)) is the truncated code and
    phi = 2^(b_max - b - 1) the midpoint correction (section 3.3).  Reading: at
    b = b_max nothing is truncated and phi = 0, so the full code is used as is.
    """
    b_max = _check_bmax(b_max)
    if not 0 <= b <= b_max:
        raise ValueError(f"bit width {b} outside 0..{b_max}")
    step = float(2 ** (b_max - b))
    qb = np.floor(np.asarray(q, dtype=np.float64) / step)
    phi = float(2 ** (b_max - b - 1)) if b < b_max else 0.0
    return qb * step + phi


def _dequant_rows(codes, scales, zeros, rows, bits, b_max):
    """w_hat = s (q_b 2^(b_max-b) + phi) + z for the given rows, fp64 [len(rows)][N]."""
    out = np.empty((len(rows), codes.shape[1]), dtype=np.float64)
    for r, i in enumerate(rows):
        b = int(bits[i])
        g = i // GROUP
        s = scales[g].astype(np.float64)
        z = zeros[g].astype(np.float64)
        out[r] = s * reconstruct_level(codes[i], b, b_max) + z
    return out


def vmm(codes, scales, zeros, x, bits, chunk: int = 256, b_max: int = B_MAX) -> np.ndarray:
    """y_j = sum over rows with b_i > 0 of x_i * w_hat_ij, in fp64.

    Rows with b_i = 0 contribute nothing (bypassed, sections 2 and 3), which
    is the reading taken for "0-bit".  x, s and z enter as their exact fp16
    values; codes are b_max-bit integers.  Returns fp64 [N].
    """
    codes = np.asarray(codes, dtype=np.uint8)
    K, N = codes.shape
    x64 = np.asarray(x, dtype=np.float16).astype(np.float64)
    rows = np.nonzero(np.asarray(bits) > 0)[0]
    y = np.zeros(N, dtype=np.float64)
    for c0 in range(0, len(rows), chunk):
        rr = rows[c0:c0 + chunk]
        w_hat = _dequant_rows(codes, scales, zeros, rr, bits, b_max)
        y += x64[rr] @ w_hat
    return y


def vmm_abs(codes, scales, zeros, x, bits, chunk: int = 256, b_max: int = B_MAX) -> np.ndarray:
    """sum_i |x_i * w_hat_ij| over rows with b_i > 0 (the tolerance scale)."""
    codes = np.asarray(codes, dtype=np.uint8)
    K, N = codes.shape
    x64 = np.abs(np.asarray(x, dtype=np.float16).astype(np.float64))
    rows = np.nonzero(np.asarray(bits) > 0)[0]
    out = np.zeros(N, dtype=np.float64)
    for c0 in range(0, len(rows), chunk):
        rr = rows[c0:c0 + chunk]
        w_hat = _dequant_rows(codes, scales, zeros, rr, bits, b_max)
        out += x64[rr] @ np.abs(w_hat)
    return out


def decode_step(codes, scales, zeros, x, thresholds, levels, b_max: int = B_MAX):
    """One decode-stage VMM: assign, select active rows, multiply."""
    bits = assign(x, thresholds, levels)
    idx, m = compact(bits)
    y = vmm(codes, scales, zeros, x, bits, b_max=b_max)
    return bits, idx, y


# --------------------------------------------------------------------------
# Non-uniform nested weights with look-up tables -- section 3.3 "Storage
# Layout and Weight Loading" (k-means style nested codes: the parent is
# quantised at b_max bits and every prefix of a code names a coarser level)
# and "Weight Reconstruction and Bias Correction" (with LUTs the nested
# levels are already centred, so there is no midpoint term); Appendix E.2
# (any-precision nested weights).
#
# Reading: one table per output column and bit width, as the nested
# k-means formats cited there keep one per output channel; row i at width b
# reads entry (q_ij >> (b_max - b)) of column j's b-bit table.  Tables are
# passed as lut[b] = array [N][2^b] for b = 1..b_max (lut[0] unused).
# --------------------------------------------------------------------------

def vmm_lut(codes, lut, x, bits, b_max: int = B_MAX) -> np.ndarray:
    """y_j = sum over rows with b_i > 0 of x_i * lut[b_i][j][prefix], fp64.

    prefix = floor(q_ij / 2^(b_max - b_i)), the top b_i bits of the code;
    rows with b_i = 0 are bypassed.  Table entries enter as given (fp16
    values are exact in fp64).
    """
    b_max = _check_bmax(b_max)
    codes = np.asarray(codes, dtype=np.int64)
    K, N = codes.shape
    x64 = np.asarray(x, dtype=np.float16).astype(np.float64)
    bits = np.asarray(bits)
    cols = np.arange(N)
    y = np.zeros(N, dtype=np.float64)
    tables = {}   # each width's tables converted to fp64 once
    for i in np.nonzero(bits > 0)[0]:
        b = int(bits[i])
        if b > b_max:
            raise ValueError(f"row {i}: width {b} above b_max = {b_max}")
        prefix = codes[i] // (1 << (b_max - b))
        if b not in tables:
            tables[b] = np.asarray(lut[b], dtype=np.float64)
        y += x64[i] * tables[b][cols, prefix]
    return y


def vmm_lut_abs(codes, lut, x, bits, b_max: int = B_MAX) -> np.ndarray:
    """sum_i |x_i * w_hat_ij| for the LUT reconstruction (tolerance scale)."""
    b_max = _check_bmax(b_max)
    codes = np.asarray(codes, dtype=np.int64)
    K, N = codes.shape
    x64 = np.abs(np.asarray(x, dtype=np.float16).astype(np.float64))
    bits = np.asarray(bits)
    cols = np.arange(N)
    out = np.zeros(N, dtype=np.float64)
    tables = {}   # each width's tables converted to fp64 once
    for i in np.nonzero(bits > 0)[0]:
        b = int(bits[i])
        prefix = codes[i] // (1 << (b_max - b))
        if b not in tables:
            tables[b] = np.asarray(lut[b], dtype=np.float64)
        out += x64[i] * np.abs(tables[b][cols, prefix])
    return out


# --------------------------------------------------------------------------
# Dense prefill -- section 3 (the prefill stage loads weights at a fixed
# precision), section 4 "Prefill vs. Decoding Evaluation" (the kernel unpacks
# the weights at full b_max precision and multiplies densely) and section 5
# "End-to-end Measurements".
# --------------------------------------------------------------------------

def dequant_dense(codes, scales, zeros, b_max: int = B_MAX) -> np.ndarray:
    """W_hat = s q + z for every row at its full width b_max, fp64 [K][N].

    At b = b_max nothing is truncated and phi = 0 (the reading of section 3.3
    used throughout), so the dense weights are the parent model's.
    """
    codes = np.asarray(codes, dtype=np.uint8)
    K = codes.shape[0]
    rows = np.arange(K)
    return _dequant_rows(codes, scales, zeros, rows, np.full(K, _check_bmax(b_max)), b_max)


def dequant_dense_fp16(codes, scales, zeros, b_max: int = B_MAX) -> np.ndarray:
    """The dense weights rounded once to fp16 (round to nearest even).

    s q + z is exact in fp64 for fp16 s, z and an 8-bit q, so this is the
    correctly rounded fp16 value of each weight.
    """
    return dequant_dense(codes, scales, zeros, b_max).astype(np.float16)


def prefill(codes, scales, zeros, X, b_max: int = B_MAX) -> np.ndarray:
    """Y = X W_hat in fp64 for a batch of M token activations X fp16 [M][K]."""
    X64 = np.asarray(X, dtype=np.float16).astype(np.float64)
    return X64 @ dequant_dense(codes, scales, zeros, b_max)


def prefill_abs(codes, scales, zeros, X, b_max: int = B_MAX) -> np.ndarray:
    """|X| |W_hat| (the tolerance scale of the prefill product)."""
    X64 = np.abs(np.asarray(X, dtype=np.float16).astype(np.float64))
    return X64 @ np.abs(dequant_dense(codes, scales, zeros, b_max))


# --------------------------------------------------------------------------
# Bytes accounting.
# --------------------------------------------------------------------------

def bytes_read(bits: np.ndarray, K: int, N: int) -> dict:
    """Algorithmic bytes of one VMM.

    planes: sum_i b_i * N_pad / 8 (only the top b_i planes of active rows);
    scales: 4 N bytes (fp16 s and z) for every group with an active row;
    x: 2 K bytes.  The output (4 N bytes) is reported on its own.
    """
    bits = np.asarray(bits, dtype=np.int64)
    Np = padded_cols(N)
    G = (K + GROUP - 1) // GROUP
    active_groups = sum(1 for g in range(G) if bits[g * GROUP:(g + 1) * GROUP].max(initial=0) > 0)
    planes = int(bits.sum()) * Np // 8
    scales = 4 * N * active_groups
    xb = 2 * K
    return {"planes": planes, "scales": scales, "x": xb, "total": planes + scales + xb,
            "y": 4 * N, "avg_bits": float(bits.sum()) / K}
