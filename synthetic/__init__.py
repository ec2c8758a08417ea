"""Seeded synthetic inputs for the GRINQH decode-stage vector-matrix multiply.

This module only *draws* inputs: weight matrices already quantised to b_max-bit
(8 unless asked otherwise) asymmetric codes with per-(128-row group, column) fp16 scale and zero, fp16
activation vectors, and the precision distributions P that the workloads use.
It holds none of the GRINQH method's arithmetic (no threshold calibration, no
precision assignment, no bit planes, no reconstruction).  Both the fp64 oracle
and the HIP library consume what it returns; neither is imported here.

Recipe (the pages measure on trained Llama-3 / Qwen3 weights and on text
datasets that are not available; these seeded draws stand in for them, keeping
only the model shapes):

* Weights ``W ~ N(0, 0.02^2)`` in fp32, quantised round-to-nearest at 8 bits,
  one (scale, zero) pair per group of 128 input rows and per output column, as
  in the RTN base the paper builds on ("Models and Baselines", section 4, group
  size G = 128).  With L = 2^b_max - 1, ``s = (max - min) / L`` and
  ``z = min`` are rounded round-to-nearest-even to fp16, and codes use those
  rounded values: ``q = clip(rint((w - z) / s), 0, L)`` (``q = 0`` where
  ``s == 0``).  b_max = 4 and 6 quantise the parent model at that width
  directly, as section 3.3 asks of a store with a smaller maximum width.
  The base quantiser is an input recipe: the paper treats the quantisation
  step as independent of GRINQH (Appendix D.1).
* Activations: ``|x_i| = exp(N(0, 1))`` with a random sign; a fixed set of
  ``ceil(0.01 K)`` outlier input channels per matrix is scaled by 20 in every
  vector drawn for that matrix (persistent outlier channels, section 3.1's
  motivation).  Cast to fp16.
* Seeds: ``numpy.random.SeedSequence([config, matrix, role])`` with role 0 for
  W, 1 for the outlier channel set, 2 for calibration vectors, 3 for test
  vectors.
* The 36-layer Qwen3-8B stack (252 matrices, 6.95 G weights) is too large to
  draw on the host in reasonable time, so :func:`device_weights` draws its
  weights on the GPU: the same N(0, 0.02^2) distribution from torch's
  Philox generator seeded by the same (config, matrix, 0) triple, and the
  same rounding rule evaluated in fp32.  Its activations and calibration
  vectors are the NumPy ones above.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

GROUP = 128          # rows per (scale, zero) group
N_CALIB = 64         # calibration vectors per matrix
WEIGHT_STD = 0.02
OUTLIER_FRACTION = 0.01
OUTLIER_SCALE = 20.0

ROLE_W, ROLE_OUTLIERS, ROLE_CALIB, ROLE_TEST = 0, 1, 2, 3

# Precision level sets and target distributions P = (p_0, ..., p_n).  Every P
# below sums to 1 and its weighted average bit width is the key of the entry.
LEVELS_5 = (0, 2, 3, 4, 8)
LEVELS_4 = (0, 2, 4, 8)
# Stores with a smaller maximum width (section 3.3 evaluates b_max in
# {4, 6, 8}; Table 7 runs an effective 4 bits under b_max = 6 and an effective
# 3 bits under b_max = 4), with 2-bit steps as in Figure 2.
LEVELS_BMAX6 = (0, 2, 4, 6)
LEVELS_BMAX4 = (0, 2, 4)

P_LEVELS_5 = {
    2: (0.35, 0.30, 0.20, 0.10, 0.05),
    3: (0.25, 0.20, 0.20, 0.20, 0.15),
    4: (0.15, 0.10, 0.20, 0.30, 0.25),
    8: (0.0, 0.0, 0.0, 0.0, 1.0),
}
# The tiny workload's thresholds are the 25/50/75/90 % quantiles of |x|.
P_TINY = (0.25, 0.25, 0.25, 0.15, 0.10)

P_LEVELS_4 = {
    0.5: (0.88, 0.05, 0.04, 0.03),
    1: (0.75, 0.10, 0.10, 0.05),
    2: (0.50, 0.20, 0.20, 0.10),
    3: (0.30, 0.20, 0.35, 0.15),
    4: (0.15, 0.20, 0.40, 0.25),
    6: (0.10, 0.10, 0.15, 0.65),
    8: (0.0, 0.0, 0.0, 1.0),
}

# Workload shapes (K input rows x N output columns).
LLAMA3_8B_LAYER = {
    "q": (4096, 4096), "k": (4096, 1024), "v": (4096, 1024), "o": (4096, 4096),
    "gate": (4096, 14336), "up": (4096, 14336), "down": (14336, 4096),
}
QWEN3_8B_LAYER = {
    "q": (4096, 4096), "k": (4096, 1024), "v": (4096, 1024), "o": (4096, 4096),
    "gate": (4096, 12288), "up": (4096, 12288), "down": (12288, 4096),
}
QWEN3_8B_LAYERS = 36
STACK_CONFIG = 3     # config index of the Qwen3-8B stack
LLAMA3_70B_MLP = {"gate": (8192, 28672), "down": (28672, 8192)}


P_BMAX6 = {
    3: (0.20, 0.30, 0.30, 0.20),
    4: (0.10, 0.20, 0.30, 0.40),
}
P_BMAX4 = {
    2: (0.25, 0.50, 0.25),
    3: (0.10, 0.30, 0.60),
}

def rng(config: int, matrix: int, role: int) -> np.random.Generator:
    """Independent PCG64 stream for one (config, matrix, role) triple."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([config, matrix, role])))


def n_groups(K: int) -> int:
    return (K + GROUP - 1) // GROUP


def rtn_quantize(w: np.ndarray, b_max: int = 8):
    """Round-to-nearest b_max-bit asymmetric quantisation of fp32 ``w[K][N]``.

    Returns ``(codes u8[K][N], scales f16[G][N], zeros f16[G][N])``.  The last
    group may hold fewer than 128 rows.
    """
    if not 1 <= b_max <= 8:
        raise ValueError(f"b_max = {b_max}, expected 1..8")
    top = float((1 << b_max) - 1)
    K, N = w.shape
    G = n_groups(K)
    codes = np.empty((K, N), dtype=np.uint8)
    scales = np.empty((G, N), dtype=np.float16)
    zeros = np.empty((G, N), dtype=np.float16)
    for g in range(G):
        blk = w[g * GROUP:(g + 1) * GROUP].astype(np.float64)
        lo = blk.min(axis=0)
        hi = blk.max(axis=0)
        s16 = ((hi - lo) / top).astype(np.float16)
        z16 = lo.astype(np.float16)
        s64 = s16.astype(np.float64)
        z64 = z16.astype(np.float64)
        with np.errstate(divide="ignore", invalid="ignore"):
            q = np.rint((blk - z64) / s64)
        q = np.where(s64 == 0.0, 0.0, q)
        codes[g * GROUP:(g + 1) * GROUP] = np.clip(q, 0, top).astype(np.uint8)
        scales[g] = s16
        zeros[g] = z16
    return codes, scales, zeros


def make_weights(K: int, N: int, config: int = 0, matrix: int = 0, b_max: int = 8):
    """Seeded ``W ~ N(0, 0.02^2)`` quantised by :func:`rtn_quantize` at b_max bits."""
    r = rng(config, matrix, ROLE_W)
    codes = np.empty((K, N), dtype=np.uint8)
    G = n_groups(K)
    scales = np.empty((G, N), dtype=np.float16)
    zeros = np.empty((G, N), dtype=np.float16)
    # Draw and quantise one group at a time so large matrices stay small in memory.
    for g in range(G):
        rows = min(GROUP, K - g * GROUP)
        w = r.standard_normal((rows, N), dtype=np.float32) * np.float32(WEIGHT_STD)
        c, s, z = rtn_quantize(w, b_max)
        codes[g * GROUP:g * GROUP + rows] = c
        scales[g] = s[0]
        zeros[g] = z[0]
    return codes, scales, zeros


def outlier_rows(K: int, config: int = 0, matrix: int = 0) -> np.ndarray:
    """Fixed per-matrix set of ceil(1% K) outlier input channels (sorted)."""
    n_out = int(math.ceil(OUTLIER_FRACTION * K))
    r = rng(config, matrix, ROLE_OUTLIERS)
    return np.sort(r.choice(K, size=n_out, replace=False))


def make_activations(K: int, count: int, config: int = 0, matrix: int = 0,
                     role: int = ROLE_TEST) -> np.ndarray:
    """``count`` fp16 activation vectors of length K, shape [count][K]."""
    r = rng(config, matrix, role)
    mag = np.exp(r.standard_normal((count, K)))
    sign = np.where(r.random((count, K)) < 0.5, -1.0, 1.0)
    x = mag * sign
    x[:, outlier_rows(K, config, matrix)] *= OUTLIER_SCALE
    return x.astype(np.float16)


def lut_offsets(N: int, b_max: int = 8) -> list:
    """Start of each width's block in the flat LUT buffer (index b; [0] unused).

    Blocks for b = 1..b_max follow each other; block b holds N tables of 2^b
    fp16 entries (column j's table at j 2^b), so it starts at N (2^b - 2).
    """
    return [0] + [N * ((1 << b) - 2) for b in range(1, b_max + 1)]


def lut_flat(tables, N: int, b_max: int = 8) -> np.ndarray:
    """Per-width tables (tables[b] = fp16 [N][2^b]) -> one flat fp16 buffer."""
    out = np.zeros(N * ((1 << (b_max + 1)) - 2), dtype=np.float16)
    off = lut_offsets(N, b_max)
    for b in range(1, b_max + 1):
        t = np.asarray(tables[b], dtype=np.float16)
        if t.shape != (N, 1 << b):
            raise ValueError(f"table {b} has shape {t.shape}, expected {(N, 1 << b)}")
        out[off[b]:off[b] + N * (1 << b)] = t.reshape(-1)
    return out


def make_lut_weights(K: int, N: int, config: int = 0, matrix: int = 0, b_max: int = 8):
    """Nested non-uniform codes with one table per output column and width.

    Stands in for a k-means style nested quantiser (the pages cite one):
    column j's weights are N(0, sigma_j^2) with sigma_j = 0.02 (0.5 + u_j);
    its b_max-bit centroids sit at the normal quantiles (c + 1/2) / 2^b_max
    times sigma_j, a code is the index of the nearest centroid, and the
    b-bit table entry of prefix p is the mean of the b_max-bit centroids
    whose codes start with p (each coarser level centred on its children).
    Tables are rounded to fp16.  Returns (codes u8 [K][N], tables) with
    tables[b] fp16 [N][2^b] for b = 1..b_max (tables[0] = None).
    """
    from scipy.special import ndtri
    r = rng(config, matrix, ROLE_W)
    sigma = WEIGHT_STD * (0.5 + r.random(N))
    L = 1 << b_max
    base = ndtri((np.arange(L) + 0.5) / L)                     # sorted
    mids = (base[1:] + base[:-1]) / 2.0
    codes = np.empty((K, N), dtype=np.uint8)
    for g0 in range(0, K, GROUP):
        rows = min(GROUP, K - g0)
        z = r.standard_normal((rows, N))                       # w / sigma_j
        codes[g0:g0 + rows] = np.searchsorted(mids, z).astype(np.uint8)
    parent = sigma[:, None] * base[None, :]                    # fp64 [N][L]
    tables = [None] * (b_max + 1)
    for b in range(1, b_max + 1):
        tables[b] = parent.reshape(N, 1 << b, L >> b).mean(axis=2).astype(np.float16)
    return codes, tables


def make_calibration(K: int, config: int = 0, matrix: int = 0, count: int = N_CALIB) -> np.ndarray:
    return make_activations(K, count, config, matrix, ROLE_CALIB)


@dataclass
class Layer:
    """One linear layer's synthetic inputs."""
    K: int
    N: int
    codes: np.ndarray      # u8 [K][N], b_max-bit values
    scales: np.ndarray     # f16 [G][N]
    zeros: np.ndarray      # f16 [G][N]
    calib: np.ndarray      # f16 [N_CALIB][K]
    x: np.ndarray          # f16 [n_test][K]


def make_layer(K: int, N: int, config: int = 0, matrix: int = 0, n_test: int = 1,
               n_calib: int = N_CALIB, b_max: int = 8) -> Layer:
    codes, scales, zeros = make_weights(K, N, config, matrix, b_max)
    calib = make_calibration(K, config, matrix, n_calib)
    x = make_activations(K, n_test, config, matrix, ROLE_TEST)
    return Layer(K, N, codes, scales, zeros, calib, x)


def qwen3_stack():
    """The 252 matrices one token passes through, in order: a list of
    (matrix index, layer, name, K, N) with matrix index = 7 layer + position."""
    out = []
    for layer in range(QWEN3_8B_LAYERS):
        for j, (name, (K, N)) in enumerate(QWEN3_8B_LAYER.items()):
            out.append((len(QWEN3_8B_LAYER) * layer + j, layer, name, K, N))
    return out


def device_weights(K: int, N: int, config: int, matrix: int, device, b_max: int = 8):
    """Seeded ``W ~ N(0, 0.02^2)`` drawn on a torch device and quantised there.

    The rounding rule is :func:`rtn_quantize`'s (fp16 s = (max - min) / L and
    z = min per group and column, q = clip(rint((w - z) / s), 0, L)), evaluated
    in fp32.  Returns torch tensors (codes u8 [K][N], scales f16 [G][N],
    zeros f16 [G][N]) on ``device``.
    """
    import torch
    if not 1 <= b_max <= 8:
        raise ValueError(f"b_max = {b_max}, expected 1..8")
    seed = int(np.random.SeedSequence([config, matrix, ROLE_W]).generate_state(1, np.uint64)[0]) & ((1 << 63) - 1)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    w = torch.randn((K, N), generator=gen, device=device, dtype=torch.float32).mul_(WEIGHT_STD)
    return rtn_quantize_torch(w, b_max)


def rtn_quantize_torch(w, b_max: int = 8):
    """:func:`rtn_quantize` on a torch fp32 tensor ``w[K][N]``, in fp32 on its device."""
    import torch
    top = float((1 << b_max) - 1)
    K, N = w.shape
    G = n_groups(K)
    codes = torch.empty((K, N), dtype=torch.uint8, device=w.device)
    scales = torch.empty((G, N), dtype=torch.float16, device=w.device)
    zeros = torch.empty((G, N), dtype=torch.float16, device=w.device)
    for g in range(G):
        blk = w[g * GROUP:(g + 1) * GROUP]
        lo = blk.amin(dim=0)
        hi = blk.amax(dim=0)
        s16 = ((hi - lo) / top).to(torch.float16)
        z16 = lo.to(torch.float16)
        s32, z32 = s16.float(), z16.float()
        q = torch.round((blk - z32) / s32)
        q = torch.where(s32 == 0.0, torch.zeros_like(q), q)
        codes[g * GROUP:(g + 1) * GROUP] = q.clamp_(0.0, top).to(torch.uint8)
        scales[g] = s16
        zeros[g] = z16
    return codes, scales, zeros
