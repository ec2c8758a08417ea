"""Parity of the dense prefill (grinqh_prefill) with the fp64 oracle.

Every row is read at its full width b_max; the kernel rounds each weight
s q + z to fp16 once and sums in fp32 on the matrix cores, so every output
element must satisfy |Y - Y_ref| <= 1e-3 * sum_k |X[m][k] w[k][n]| + 1e-4
(the weight rounding alone is at most 2^-11 of each term).
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
def layer(K, N, config, matrix, b_max):
    return synthetic.make_layer(K, N, config=config, matrix=matrix, n_test=1, b_max=b_max)


def _tokens(K, M, config, matrix):
    return synthetic.make_activations(K, M, config=config, matrix=matrix)


def _check(Y, lay, X, b_max, rows=None, cols=None):
    codes, scales, zeros = lay.codes, lay.scales, lay.zeros
    if cols is not None:
        codes, scales, zeros, Y = codes[:, cols], scales[:, cols], zeros[:, cols], Y[:, cols]
    if rows is not None:
        X, Y = X[rows], Y[rows]
    ref = oracle.prefill(codes, scales, zeros, X, b_max)
    mag = oracle.prefill_abs(codes, scales, zeros, X, b_max)
    err = np.abs(Y.astype(np.float64) - ref)
    bound = REL_TOL * mag + ABS_TOL
    worst = np.unravel_index(int(np.argmax(err - bound)), err.shape)
    assert np.all(err <= bound), f"at {worst}: gpu {Y[worst]} ref {ref[worst]} err {err[worst]} bound {bound[worst]}"


CASES = [
    # (M, K, N, config, matrix, b_max)
    (1, 256, 256, 0, 0, 8),
    (128, 128, 128, 5, 0, 8),
    (5, 300, 70, 5, 1, 8),          # K not a multiple of 8, N ragged
    (130, 4096, 1100, 5, 2, 8),     # M and N ragged, several tiles
    (33, 4097, 1056, 5, 3, 8),      # K ragged (partial last group, unaligned rows)
    (256, 4096, 4096, 1, 0, 8),
    (200, 1024, 2080, 5, 4, 6),
    (64, 4096, 4096, 1, 0, 4),
    (17, 520, 300, 5, 5, 1),
]


@pytest.mark.parametrize("M,K,N,cfg,mat,b_max", CASES)
def test_prefill_parity(M, K, N, cfg, mat, b_max):
    lay = layer(K, N, cfg, mat, b_max)
    X = _tokens(K, M, cfg, mat)
    planes = grq.pack(_dev(lay.codes), b_max=b_max)
    Y = grq.prefill(planes, _dev(lay.scales), _dev(lay.zeros), _dev(X), K, N, b_max=b_max)
    torch.cuda.synchronize()
    _check(Y.cpu().numpy(), lay, X, b_max)


def test_prefill_single_token_matches_full_width_decode():
    """A batch of one is the decode VMM with every row at b_max."""
    K, N = 4096, 4096
    lay = layer(K, N, 1, 0, 8)
    X = _tokens(K, 1, 1, 0)
    planes = grq.pack(_dev(lay.codes))
    sc, zr = _dev(lay.scales), _dev(lay.zeros)
    Y = grq.prefill(planes, sc, zr, _dev(X), K, N)
    ws = grq.make_workspace(K, N)
    y = grq.decode_vmm(planes, sc, zr, _dev(X[0]), K, N, [], (8,), ws)
    torch.cuda.synchronize()
    mag = oracle.prefill_abs(lay.codes, lay.scales, lay.zeros, X)[0]
    diff = np.abs(Y.cpu().numpy()[0].astype(np.float64) - y.cpu().numpy())
    assert np.all(diff <= 2 * REL_TOL * mag + 2 * ABS_TOL)


def test_prefill_deterministic():
    K, N, M = 4096, 1024, 256
    lay = layer(K, N, 2, 1, 8)
    X = _dev(_tokens(K, M, 2, 1))
    planes = grq.pack(_dev(lay.codes))
    args = (planes, _dev(lay.scales), _dev(lay.zeros), X, K, N)
    y1 = grq.prefill(*args).cpu().numpy()
    y2 = grq.prefill(*args).cpu().numpy()
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))


FULL = [
    (2048, 4096, 14336, 2, 4, 8),
    (512, 14336, 4096, 2, 6, 8),
    (1024, 4096, 14336, 2, 4, 6),
]


@pytest.mark.parametrize("M,K,N,cfg,mat,b_max", FULL)
def test_prefill_full_size_sampled(M, K, N, cfg, mat, b_max):
    lay = layer(K, N, cfg, mat, b_max)
    X = _tokens(K, M, cfg, mat)
    planes = grq.pack(_dev(lay.codes), b_max=b_max)
    Y = grq.prefill(planes, _dev(lay.scales), _dev(lay.zeros), _dev(X), K, N, b_max=b_max)
    torch.cuda.synchronize()
    Y = Y.cpu().numpy()
    r = np.random.default_rng(M + K + N)
    rows = np.unique(np.concatenate([r.choice(M, 24, replace=False), [0, 127, 128, M - 1]]))
    cols = np.unique(np.concatenate([r.choice(N, 160, replace=False), [0, 31, 127, 128, 1023, 1024, N - 1]]))
    _check(Y, lay, X, b_max, rows, cols)


# ------------------------------------------------ unpack once, then a dense GEMM

def _from_fragments(buf, K, N):
    """fp16 [K][N] from the B-fragment order ((k / 8) N_pad + n) 8 + k % 8."""
    Np = -(-N // 128) * 128
    kb = -(-K // 64) * 8
    f = buf.view(np.float16).reshape(kb, Np, 8)
    return f.transpose(0, 2, 1).reshape(kb * 8, Np)[:K, :N], f


@pytest.mark.parametrize("K,N,cfg,mat,b_max", [(256, 256, 0, 0, 8), (300, 70, 5, 1, 8), (4097, 1056, 5, 3, 8),
                                               (1000, 2080, 5, 4, 6), (17, 300, 5, 5, 4)])
def test_unpack_dense_bit_exact(K, N, cfg, mat, b_max):
    lay = layer(K, N, cfg, mat, b_max)
    planes = grq.pack(_dev(lay.codes), b_max=b_max)
    buf = grq.unpack_dense(planes, _dev(lay.scales), _dev(lay.zeros), K, N, b_max=b_max).cpu().numpy()
    W, f = _from_fragments(buf, K, N)
    want = oracle.dequant_dense_fp16(lay.codes, lay.scales, lay.zeros, b_max)
    assert np.array_equal(W.view(np.uint16), want.view(np.uint16))
    Np = -(-N // 128) * 128
    full = f.transpose(0, 2, 1).reshape(-1, Np)
    assert not full[K:].any() and not full[:, N:].any()      # padding is zero


@pytest.mark.parametrize("M,K,N,cfg,mat,b_max", CASES)
def test_unpacked_prefill_parity(M, K, N, cfg, mat, b_max):
    lay = layer(K, N, cfg, mat, b_max)
    X = _tokens(K, M, cfg, mat)
    planes = grq.pack(_dev(lay.codes), b_max=b_max)
    dense = grq.unpack_dense(planes, _dev(lay.scales), _dev(lay.zeros), K, N, b_max=b_max)
    Y = grq.dense_gemm(_dev(X), dense, K, N)
    torch.cuda.synchronize()
    _check(Y.cpu().numpy(), lay, X, b_max)


def test_unpacked_prefill_full_size_sampled():
    M, K, N = 2048, 4096, 14336
    lay = layer(K, N, 2, 4, 8)
    X = _tokens(K, M, 2, 4)
    planes = grq.pack(_dev(lay.codes))
    dense = grq.unpack_dense(planes, _dev(lay.scales), _dev(lay.zeros), K, N)
    Y = grq.dense_gemm(_dev(X), dense, K, N)
    torch.cuda.synchronize()
    Y = Y.cpu().numpy()
    r = np.random.default_rng(99)
    rows = np.unique(np.concatenate([r.choice(M, 24, replace=False), [0, 255, 256, M - 1]]))
    cols = np.unique(np.concatenate([r.choice(N, 160, replace=False), [0, 255, 256, 1023, 1024, N - 1]]))
    _check(Y, lay, X, 8, rows, cols)
