"""Pins of the oracle's GPTQ warm start.

GPTQ (Frantar et al. 2022) quantizes columns in order and feeds each rounding
error into the later columns. The checks below do not reuse its Cholesky
machinery: the continuation after every column against the loss-optimal
continuation written from block inverses of H, Babai's nearest-plane
recursion on the factor of H itself (no inverse), the identity-Hessian case
that reduces to round-to-nearest, and the objective against round-to-nearest.
"""

import numpy as np
import pytest

import oracle
import synthetic
from oracle import GRID_INT2, GRID_TERNARY, GRID_INT3_LOCAL, GRID_INT3

GRIDS = [GRID_INT2, GRID_TERNARY, GRID_INT3_LOCAL, GRID_INT3]


def _values(codes, scales, grid, group):
    c = codes.astype(np.int64)
    v = (c - 1).astype(np.float64) if grid == GRID_TERNARY else \
        oracle.level_value(c, oracle.CODE_BITS[grid]).astype(np.float64)
    return np.repeat(scales.astype(np.float64), group, axis=1) * v


@pytest.mark.parametrize("grid", GRIDS)
def test_identity_hessian_is_round_to_nearest(grid):
    # X = 3 I (K tokens): H is a multiple of I, so no error is fed forward.
    K = 256
    W = synthetic.small_layer(6, K, 4, seed=3)["W"]
    X = 3.0 * np.eye(K)
    s, c, lg, _ = oracle.gptq(W, X, grid)
    s0, c0, l0 = oracle.init_rtn(W, grid)
    np.testing.assert_array_equal(s, s0)
    np.testing.assert_array_equal(c, c0)
    np.testing.assert_array_equal(lg, l0)


@pytest.mark.parametrize("grid", [GRID_INT2, GRID_INT3])
def test_targets_are_the_optimal_continuation(grid):
    # After columns 0..j-1 are fixed at q, the loss over the remaining
    # continuous weights v is minimised by v = w_b + H_bb^-1 H_ba (w_a - q_a);
    # GPTQ must round column j from the first entry of that v.
    M, K, N, group = 3, 24, 40, 8
    rng = np.random.default_rng(9)
    W = rng.normal(0, 0.02, (M, K)).astype(np.float32)
    X = rng.normal(size=(N, K))
    s, c, _, T = oracle.gptq(W, X, grid, group=group)
    H = oracle.gptq_hessian(X)
    Q = _values(c, s, grid, group)
    Wd = W.astype(np.float64)
    for j in range(1, K):
        a, b = slice(0, j), slice(j, K)
        v = Wd[:, b] + np.linalg.solve(H[b, b], H[b, a] @ (Wd[:, a] - Q[:, a]).T).T
        np.testing.assert_allclose(T[:, j], v[:, 0], rtol=1e-9, atol=1e-12)
    np.testing.assert_array_equal(T[:, 0], Wd[:, 0])


def _babai(W, X, grid, group=128):
    # Nearest plane on the factor H = R R^T with R upper (the Cholesky factor
    # of H taken from the last index backwards): column j is rounded from
    # w_j + sum_{i<j} (w_i - q_i) R_ij / R_jj.
    H = oracle.gptq_hessian(X)
    K = H.shape[0]
    J = np.arange(K)[::-1]
    R = np.linalg.cholesky(H[np.ix_(J, J)])[np.ix_(J, J)]
    s, _, _ = oracle.init_rtn(W, grid, group)
    sf = np.repeat(s, group, axis=1)
    Wd = np.asarray(W, dtype=np.float64)
    M = Wd.shape[0]
    d = np.zeros((M, K))
    codes = np.zeros((M, K), dtype=np.int64)
    T = np.zeros((M, K))
    for j in range(K):
        T[:, j] = Wd[:, j] + d[:, :j] @ R[:j, j] / R[j, j]
        codes[:, j], _ = oracle.gsq._nearest_code(T[:, j], sf[:, j], grid)
        q = _values(codes[:, j:j + 1], s[:, j // group:j // group + 1], grid, 1)[:, 0]
        d[:, j] = Wd[:, j] - q
    return codes, T


@pytest.mark.parametrize("grid", GRIDS)
def test_equals_nearest_plane_on_the_factor_of_H(grid):
    M, K, N = 8, 256, 300
    d = synthetic.small_layer(M, K, N, seed=11)
    _, c, _, T = oracle.gptq(d["W"], d["X"], grid)
    cb, Tb = _babai(d["W"], d["X"], grid)
    np.testing.assert_allclose(T, Tb, rtol=1e-8, atol=1e-12)
    np.testing.assert_array_equal(c, cb)


@pytest.mark.parametrize("grid", [GRID_INT2, GRID_INT3])
def test_gptq_lowers_the_objective_against_rtn(grid):
    ratios = []
    for seed in range(4):
        d = synthetic.small_layer(16, 256, 512, seed=20 + seed)
        s, c, _, _ = oracle.gptq(d["W"], d["X"], grid)
        s0, c0, _ = oracle.init_rtn(d["W"], grid)
        ratios.append(oracle.hard_loss(c, s, d["W"], d["X"], grid) /
                      oracle.hard_loss(c0, s0, d["W"], d["X"], grid))
    assert max(ratios) < 1.0


def test_dead_column_and_damping():
    rng = np.random.default_rng(5)
    X = rng.normal(size=(64, 128))
    X[:, 7] = 0.0
    H = oracle.gptq_hessian(X, damp=0.01)
    d = np.diag(X.T @ X).copy()
    d[7] = 1.0
    np.testing.assert_allclose(np.diag(H), d + 0.01 * d.mean(), rtol=1e-14)
    W = rng.normal(0, 0.02, (4, 128)).astype(np.float32)
    s, c, _, T = oracle.gptq(W, X, GRID_INT2)
    assert np.all(np.isfinite(T))
