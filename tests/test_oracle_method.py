"""Pins of the oracle's relaxation, objective, Lion, hardening and packing.

Every check compares the oracle with something it does not compute itself:
closed forms, limits, finite differences, an independent Gram-form objective,
brute-force enumeration, big-integer bit packing, and the numbers the pages
print (tests/golden/paper_numbers.json).
"""

import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import GRID_INT2, GRID_TERNARY, GRID_INT3_LOCAL, GRID_INT3

HERE = os.path.dirname(os.path.abspath(__file__))
GRIDS = [GRID_INT2, GRID_TERNARY, GRID_INT3_LOCAL, GRID_INT3]


def layer(M, K, seed=0, sigma=0.02):
    return np.random.default_rng(seed).normal(0, sigma, (M, K)).astype(np.float32)


def rand_logits(grid, M, K, seed=1, spread=1.5):
    return np.random.default_rng(seed).normal(0, spread, (oracle.N_LOGITS[grid], M, K))


# ----------------------------------------------------------------------------
# Softmax, limits and closed forms
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("grid", [GRID_INT2, GRID_INT3_LOCAL, GRID_INT3])
@pytest.mark.parametrize("tau", [1.0, 0.3, 0.05])
def test_softmax_rows_sum_to_one(grid, tau):
    p = oracle.relax_probs(rand_logits(grid, 4, 256), grid, 0, 0, 3, tau, 1.0)
    np.testing.assert_allclose(p.sum(axis=0), 1.0, rtol=0, atol=1e-12)
    assert np.all(p >= 0)


@pytest.mark.parametrize("grid", GRIDS)
def test_tau_to_zero_gives_argmax_grid_point(grid):
    M, K, tau = 4, 256, 1e-4
    W = layer(M, K)
    s, c0, _ = oracle.init_rtn(W, grid)
    lg = rand_logits(grid, M, K)
    n = oracle.noise(grid, M, K, 7, 1, 5)
    y = lg + n
    w = oracle.relax_fwd(lg, s, W, grid, 7, 1, 5, tau, 1.0, c0)["w_soft"]
    sfull = np.repeat(s.astype(np.float64), 128, axis=1)
    if grid == GRID_TERNARY:
        ok = np.all(np.abs(y) > 1e-2, axis=0)
        hard = (y[0] > 0) * np.where(y[1] > 0, 1.0, -1.0)
    else:
        ys = np.sort(y, axis=0)
        ok = (ys[-1] - ys[-2]) > 1e-2
        k = np.argmax(y, axis=0)
        codes = k if grid in (GRID_INT2, GRID_INT3) else np.clip(c0.astype(np.int64) + k - 2, 0, 7)
        hard = oracle.level_value(codes, oracle.CODE_BITS[grid])
    assert ok.mean() > 0.95
    np.testing.assert_allclose(w[ok], (sfull * hard)[ok], rtol=1e-12, atol=0)


def test_zero_noise_uniform_logits_2bit_is_grid_mean():
    M, K = 3, 256
    W = layer(M, K)
    s, _, _ = oracle.init_rtn(W, GRID_INT2)
    f = oracle.relax_fwd(np.zeros((4, M, K)), s, W, GRID_INT2, 0, 0, 0, 0.37, 0.0)
    # mean of {-3, -1, 1, 3} is 0
    assert np.max(np.abs(f["w_soft"])) < 1e-15
    # and of the eight levels -7..7 of the full 3-bit grid
    s3, _, _ = oracle.init_rtn(W, GRID_INT3)
    f3 = oracle.relax_fwd(np.zeros((8, M, K)), s3, W, GRID_INT3, 0, 0, 0, 0.37, 0.0)
    assert np.max(np.abs(f3["w_soft"])) < 1e-15


def test_full_grid_restricted_to_window_is_local_shift():
    # Noise-free, the full 3-bit relaxation with every level outside c0 +- 2
    # switched off (logit -1e4) is the local-shift relaxation of the same
    # five logits, for warm-start codes away from the edges.
    rng = np.random.default_rng(12)
    K = 128
    c0 = rng.integers(2, 6, size=(1, K)).astype(np.uint8)
    loc = rng.normal(0, 1.5, (5, 1, K))
    full = np.full((8, 1, K), -1e4)
    for d in range(5):
        np.put_along_axis(full, (c0.astype(np.int64) + d - 2)[None], loc[d][None], axis=0)
    s = np.array([[0.013]], dtype=np.float32)
    W = np.zeros((1, K))
    a = oracle.relax_fwd(loc, s, W, GRID_INT3_LOCAL, 0, 0, 0, 0.6, 0.0, c0)["w_soft"]
    b = oracle.relax_fwd(full, s, W, GRID_INT3, 0, 0, 0, 0.6, 0.0)["w_soft"]
    np.testing.assert_allclose(b, a, rtol=1e-13, atol=1e-18)


def test_zero_noise_uniform_logits_local_shift_closed_forms():
    # Candidates clamp(c0 + d, 0, 7), d = -2..2, values 2c - 7:
    # c0 in [2, 5] -> mean q(c0); c0 = 0 -> -29/5; 1 -> -23/5; 6 -> 23/5; 7 -> 29/5.
    expect = {0: -29 / 5, 1: -23 / 5, 2: -3, 3: -1, 4: 1, 5: 3, 6: 23 / 5, 7: 29 / 5}
    K = 128
    codes = np.tile(np.arange(8, dtype=np.uint8), K // 8)[None, :]
    s = np.array([[0.011]], dtype=np.float32)
    f = oracle.relax_fwd(np.zeros((5, 1, K)), s, np.zeros((1, K)), GRID_INT3_LOCAL,
                         0, 0, 0, 2.0, 0.0, codes)
    want = np.array([expect[int(c)] for c in codes[0]]) * float(s[0, 0])
    np.testing.assert_allclose(f["w_soft"][0], want, rtol=1e-14, atol=1e-17)


def test_zero_noise_uniform_logits_ternary_is_zero():
    M, K = 2, 128
    W = layer(M, K)
    s, _, _ = oracle.init_rtn(W, GRID_TERNARY)
    f = oracle.relax_fwd(np.zeros((2, M, K)), s, W, GRID_TERNARY, 0, 0, 0, 0.5, 0.0)
    assert np.max(np.abs(f["w_soft"])) == 0.0


def test_ternary_hard_limit_is_scale_mask_sign():
    M, K = 2, 256
    W = layer(M, K)
    s, _, _ = oracle.init_rtn(W, GRID_TERNARY)
    rng = np.random.default_rng(3)
    lg = rng.choice([-1, 1], size=(2, M, K)) * rng.uniform(0.5, 3.0, size=(2, M, K))
    f = oracle.relax_fwd(lg, s, W, GRID_TERNARY, 0, 0, 0, 1e-4, 0.0)
    mask = lg[0] > 0
    sign = np.where(lg[1] > 0, 1.0, -1.0)
    want = np.repeat(s.astype(np.float64), 128, axis=1) * mask * sign
    np.testing.assert_array_equal(f["w_soft"], want)
    assert np.all(f["w_soft"][~mask] == 0.0)


def test_local_shift_candidates_stay_in_range():
    c0 = np.arange(8, dtype=np.uint8).repeat(3)
    cand = oracle.candidate_codes(GRID_INT3_LOCAL, c0)
    assert cand.shape == (5, c0.size)
    assert np.all(np.abs(cand - c0.astype(np.int64)) <= 2)
    assert cand.min() >= 0 and cand.max() <= 7
    # hardened local-shift codes obey the same bounds for arbitrary logits
    lg = np.random.default_rng(0).normal(size=(5, 1, c0.size))
    hard = oracle.harden(lg, GRID_INT3_LOCAL, c0[None, :])
    assert np.all(np.abs(hard.astype(int) - c0.astype(int)) <= 2)
    assert hard.min() >= 0 and hard.max() <= 7


def test_grid_levels_symmetric():
    for grid in GRIDS:
        v = oracle.grid_levels(grid)
        np.testing.assert_array_equal(np.sort(-v), v)      # symmetric, no zero point offset
    np.testing.assert_array_equal(oracle.grid_levels(GRID_INT2), [-3, -1, 1, 3])
    np.testing.assert_array_equal(oracle.grid_levels(GRID_INT3_LOCAL), np.arange(-7, 8, 2))


# ----------------------------------------------------------------------------
# Gradients: finite differences and invariants
# ----------------------------------------------------------------------------

def _setup_small(grid, M=3, K=16, N=24, group=8, seed=0):
    rng = np.random.default_rng(seed)
    W = rng.normal(0, 0.02, (M, K)).astype(np.float32)
    X = rng.normal(0, 1, (N, K))
    s, c0, _ = oracle.init_rtn(W, grid, group)
    lg = rng.normal(0, 1.0, (oracle.N_LOGITS[grid], M, K))
    return W, X, s.astype(np.float64), c0, lg


def _loss(lg, s, W, X, grid, c0, tau, group, eta=1.0):
    f = oracle.relax_fwd(lg, s, W, grid, 11, 2, 9, tau, eta, c0, group=group)
    return oracle.recon_loss_grad(X, f["dW"])[1]


@pytest.mark.parametrize("grid", GRIDS)
@pytest.mark.parametrize("tau", [1.0, 0.4])
def test_gradients_match_finite_differences(grid, tau):
    group = 8
    W, X, s, c0, lg = _setup_small(grid)
    f = oracle.relax_fwd(lg, s, W, grid, 11, 2, 9, tau, 1.0, c0, group=group)
    _, _, G = oracle.recon_loss_grad(X, f["dW"])
    gl, gs = oracle.relax_bwd(G, lg, s, grid, 11, 2, 9, tau, 1.0, c0, group=group)
    h = 1e-6
    fd = np.zeros_like(gl)
    for idx in np.ndindex(*lg.shape):
        lp, lm = lg.copy(), lg.copy()
        lp[idx] += h
        lm[idx] -= h
        fd[idx] = (_loss(lp, s, W, X, grid, c0, tau, group)
                   - _loss(lm, s, W, X, grid, c0, tau, group)) / (2 * h)
    assert np.max(np.abs(fd - gl)) <= 1e-6 * np.max(np.abs(gl))
    fds = np.zeros_like(gs)
    for idx in np.ndindex(*s.shape):
        hs = 1e-6 * s[idx]
        sp, sm = s.copy(), s.copy()
        sp[idx] += hs
        sm[idx] -= hs
        fds[idx] = (_loss(lg, sp, W, X, grid, c0, tau, group)
                    - _loss(lg, sm, W, X, grid, c0, tau, group)) / (2 * hs)
    assert np.max(np.abs(fds - gs)) <= 1e-6 * np.max(np.abs(gs))


@pytest.mark.parametrize("grid", [GRID_INT2, GRID_INT3_LOCAL, GRID_INT3])
def test_logit_gradients_sum_to_zero(grid):
    # sum_k p_k (v_k - w_hat) = 0, so shifting all logits of a coordinate
    # together leaves the soft weight unchanged.
    W = layer(4, 256)
    s, c0, _ = oracle.init_rtn(W, grid)
    lg = rand_logits(grid, 4, 256)
    G = np.random.default_rng(5).normal(size=(4, 256))
    gl, _ = oracle.relax_bwd(G, lg, s, grid, 1, 0, 2, 0.5, 1.0, c0)
    assert np.max(np.abs(gl.sum(axis=0))) <= 1e-12 * np.max(np.abs(gl))


@pytest.mark.parametrize("grid", GRIDS)
def test_scale_gradient_homogeneity(grid):
    # w_soft is linear in s, so s * dL/ds_g = sum over the group of G * w_soft.
    W = layer(3, 256)
    s, c0, _ = oracle.init_rtn(W, grid)
    lg = rand_logits(grid, 3, 256)
    G = np.random.default_rng(6).normal(size=(3, 256))
    f = oracle.relax_fwd(lg, s, W, grid, 1, 0, 2, 0.8, 1.0, c0)
    _, gs = oracle.relax_bwd(G, lg, s, grid, 1, 0, 2, 0.8, 1.0, c0)
    rhs = (G * f["w_soft"]).reshape(3, 2, 128).sum(axis=2)
    np.testing.assert_allclose(s * gs, rhs, rtol=1e-12, atol=1e-18)


# ----------------------------------------------------------------------------
# Reconstruction objective
# ----------------------------------------------------------------------------

def test_loss_and_gradient_gram_form():
    rng = np.random.default_rng(2)
    X = rng.normal(size=(40, 24))
    D = rng.normal(size=(7, 24)) * 0.01
    RT, loss, G = oracle.recon_loss_grad(X, D)
    H = np.einsum("nk,nj->kj", X, X)             # X^T X formed independently
    assert math.isclose(loss, float(np.einsum("mk,kj,mj->", D, H, D)), rel_tol=1e-12)
    np.testing.assert_allclose(G, 2 * np.einsum("mk,kj->mj", D, H), rtol=1e-12, atol=1e-15)
    # finite differences in dW
    h = 1e-7
    for idx in [(0, 0), (3, 11), (6, 23)]:
        Dp, Dm = D.copy(), D.copy()
        Dp[idx] += h
        Dm[idx] -= h
        fd = (oracle.recon_loss_grad(X, Dp)[1] - oracle.recon_loss_grad(X, Dm)[1]) / (2 * h)
        assert abs(fd - G[idx]) <= 1e-6 * np.abs(G).max()


def test_gram_matrix_by_token_sums():
    # H[i][j] = sum over tokens of x_i * x_j, accumulated one token at a time.
    rng = np.random.default_rng(5)
    X = rng.normal(size=(9, 6))
    H = oracle.gram(X)
    want = np.zeros((6, 6))
    for n in range(9):
        for i in range(6):
            for j in range(6):
                want[i, j] += X[n, i] * X[n, j]
    np.testing.assert_allclose(H, want, rtol=1e-13, atol=1e-13)
    assert np.array_equal(H, H.T)
    assert np.linalg.eigvalsh(H).min() >= -1e-12


def test_gram_bf16_is_rounded_exact_gram():
    rng = np.random.default_rng(6)
    X = rng.normal(size=(64, 32)) * 3.0
    Hb = oracle.gram(X, bf16=True)
    He = oracle.gram(X)
    # every entry is a bf16 value (low 16 bits of the fp32 pattern are zero)
    assert not (Hb.astype(np.float32).view(np.uint32) & 0xFFFF).any()
    # and within half a bf16 ulp (2^-8 relative) of the exact value
    assert np.all(np.abs(Hb - He) <= np.abs(He) * 2.0 ** -8 + 1e-30)


def test_gram_objective_equals_direct_objective():
    # Same objective written two ways: tr(dW X^T X dW^T) and ||X dW^T||^2;
    # the direct form is pinned by finite differences above.
    rng = np.random.default_rng(7)
    X = rng.normal(size=(50, 40))
    D = rng.normal(size=(9, 40)) * 0.01
    _, loss, G = oracle.recon_loss_grad(X, D)
    lg, Gg = oracle.recon_loss_grad_gram(D, oracle.gram(X))
    assert math.isclose(lg, loss, rel_tol=1e-12)
    np.testing.assert_allclose(Gg, G, rtol=1e-11, atol=1e-15)
    # a single nonzero row r: the loss is the quadratic form d_r H d_r^T
    D1 = np.zeros_like(D)
    D1[4] = D[4]
    l1, _ = oracle.recon_loss_grad_gram(D1, oracle.gram(X))
    assert math.isclose(l1, float(np.sum((X @ D[4]) ** 2)), rel_tol=1e-12)


def test_gram_gradient_finite_differences():
    rng = np.random.default_rng(8)
    H = oracle.gram(rng.normal(size=(30, 12)))
    D = rng.normal(size=(4, 12)) * 0.1
    _, G = oracle.recon_loss_grad_gram(D, H)
    h = 1e-6
    for idx in [(0, 0), (2, 7), (3, 11)]:
        Dp, Dm = D.copy(), D.copy()
        Dp[idx] += h
        Dm[idx] -= h
        fd = (oracle.recon_loss_grad_gram(Dp, H)[0] - oracle.recon_loss_grad_gram(Dm, H)[0]) / (2 * h)
        assert abs(fd - G[idx]) <= 1e-7 * np.abs(G).max()


def test_zero_difference_gives_zero_loss_and_gradient():
    X = np.random.default_rng(0).normal(size=(8, 16))
    RT, loss, G = oracle.recon_loss_grad(X, np.zeros((3, 16)))
    assert loss == 0.0 and not G.any() and not RT.any()


def test_grouped_objective_is_sum_of_experts():
    rng = np.random.default_rng(4)
    rows, K = 5, 32
    offs = [0, 7, 7, 19]                          # includes an empty expert
    X = rng.normal(size=(19, K))
    D = rng.normal(size=(3 * rows, K))
    _, loss, G = oracle.recon_loss_grad_grouped(X, offs, D, rows)
    want = 0.0
    for e in range(3):
        Xe = X[offs[e]:offs[e + 1]]
        De = D[e * rows:(e + 1) * rows]
        H = np.einsum("nk,nj->kj", Xe, Xe)
        want += float(np.einsum("mk,kj,mj->", De, H, De))
        np.testing.assert_allclose(G[e * rows:(e + 1) * rows], 2 * De @ H, rtol=1e-12, atol=1e-14)
    assert math.isclose(loss, want, rel_tol=1e-12)


# ----------------------------------------------------------------------------
# Warm start
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("grid", GRIDS)
def test_rtn_codes_are_nearest_levels(grid):
    W = layer(16, 512, seed=8)
    s, c0, lg = oracle.init_rtn(W, grid)
    qmax = oracle.Q_MAX[grid]
    np.testing.assert_array_equal(s, (np.abs(W).reshape(16, 4, 128).max(2) / np.float32(qmax)).astype(np.float32))
    x = W.astype(np.float64) / np.repeat(s, 128, axis=1).astype(np.float64)
    levels = oracle.grid_levels(grid)
    nearest = np.argmin(np.abs(x[..., None] - levels), axis=-1)
    # the max-magnitude weight of each group lands on the outermost level
    np.testing.assert_array_equal(c0, nearest.astype(np.uint8))
    # the initial logits harden back to the warm start
    np.testing.assert_array_equal(oracle.harden(lg, grid, c0), c0)


def test_rtn_zero_group():
    W = np.zeros((1, 128), dtype=np.float32)
    s, c0, _ = oracle.init_rtn(W, GRID_INT2)
    assert s[0, 0] == 0 and np.all(c0 == 2)


# ----------------------------------------------------------------------------
# Brute force on one group of 8 weights
# ----------------------------------------------------------------------------

def _enumerate_all(W, X, s):
    codes = np.array(list(itertools.product(range(4), repeat=8)))    # 65536 x 8
    V = (2 * codes - 3) * float(s) - W.astype(np.float64)[0]
    H = X.T @ X
    losses = np.einsum("ck,kj,cj->c", V, H, V)
    return codes, losses


@pytest.mark.slow
def test_brute_force_one_group():
    hits, better_or_equal_rtn = 0, 0
    seeds = range(6)
    for seed in seeds:
        rng = np.random.default_rng(100 + seed)
        W = rng.normal(0, 0.02, (1, 8)).astype(np.float32)
        X = rng.normal(0, 1, (64, 8))
        s, c0, _ = oracle.init_rtn(W, GRID_INT2, group=8)
        codes, losses = _enumerate_all(W, X, s[0, 0])
        best = int(np.argmin(losses))
        L_star = float(losses[best])
        # the oracle's hard-loss evaluator agrees with the enumeration
        for idx in (best, 0, 12345, 65535):
            got = oracle.hard_loss(codes[idx][None].astype(np.uint8), s, W, X, GRID_INT2, group=8)
            assert math.isclose(got, float(losses[idx]), rel_tol=1e-12)
        out = oracle.quantize_layer(W, X, GRID_INT2, steps=150, seed=seed, lr_logit=3e-2,
                                    lr_scale=0.0, group=8)
        L_gsq = oracle.hard_loss(out["codes"], s, W, X, GRID_INT2, group=8)
        L_rtn = oracle.hard_loss(c0, s, W, X, GRID_INT2, group=8)
        assert L_gsq >= L_star * (1 - 1e-12)
        hits += math.isclose(L_gsq, L_star, rel_tol=1e-9)
        better_or_equal_rtn += L_gsq <= L_rtn * (1 + 1e-12)
    # GSQ never ends worse than its warm start and finds the optimum often.
    assert better_or_equal_rtn == len(seeds)
    assert hits >= len(seeds) // 2


def test_identity_activations_make_rtn_optimal():
    # X = I: the objective separates per coordinate, so for a fixed scale the
    # exact discrete optimum is round-to-nearest.
    rng = np.random.default_rng(9)
    W = rng.normal(0, 0.02, (1, 8)).astype(np.float32)
    X = np.eye(8)
    s, c0, _ = oracle.init_rtn(W, GRID_INT2, group=8)
    codes, losses = _enumerate_all(W, X, s[0, 0])
    np.testing.assert_array_equal(codes[int(np.argmin(losses))], c0[0])


# ----------------------------------------------------------------------------
# Lion
# ----------------------------------------------------------------------------

def test_lion_constant_gradient_closed_form():
    lr = 2.0 ** -10
    g = np.array([0.7, -3.0, 0.0, 1e-30], dtype=np.float64)
    th = np.ones(4, dtype=np.float32)
    m = np.zeros(4, dtype=np.float32)
    for t in range(1, 51):
        th_new, m = oracle.lion(th, g, m, lr, 0.9, 0.99)
        step_sizes = np.abs(th_new.astype(np.float64) - th)
        assert np.all((step_sizes == 0) | (step_sizes == lr))
        th = th_new
        np.testing.assert_array_equal(th, 1.0 - t * lr * np.sign(g))
        np.testing.assert_allclose(m, (1 - 0.99 ** t) * g, rtol=1e-5, atol=0)


def test_lion_weight_decay_closed_form():
    lr, wd = 1e-3, 0.5
    th = np.full(3, 2.0, dtype=np.float32)
    m = np.zeros(3, dtype=np.float32)
    for _ in range(20):
        th, m = oracle.lion(th, np.zeros(3), m, lr, 0.9, 0.99, wd)
    np.testing.assert_allclose(th, 2.0 * (1 - float(np.float32(lr)) * float(np.float32(wd))) ** 20,
                               rtol=1e-6)


def test_lion_sign_uses_interpolated_momentum():
    # c = beta1*m + (1-beta1)*g decides the direction, not g alone.
    th = np.zeros(2, dtype=np.float32)
    m = np.array([1.0, -1.0], dtype=np.float32)
    g = np.array([-5.0, -5.0])          # c = 0.9 - 0.5 > 0 ; -0.9 - 0.5 < 0
    th2, m2 = oracle.lion(th, g, m, 0.25, 0.9, 0.99)
    np.testing.assert_array_equal(th2, [-0.25, 0.25])
    np.testing.assert_allclose(m2, [0.99 - 0.05, -0.99 - 0.05], rtol=1e-6)


# ----------------------------------------------------------------------------
# Hardening, packing and the format numbers the pages print
# ----------------------------------------------------------------------------

def test_harden_rules():
    lg = np.zeros((4, 1, 4))
    lg[:, 0, 1] = [0, 5, 5, 1]            # tie between 1 and 2 -> first index
    lg[:, 0, 2] = [0, 0, 0, 3]
    np.testing.assert_array_equal(oracle.harden(lg, GRID_INT2)[0], [0, 1, 3, 0])
    lt = np.array([[[1.0, 1.0, -0.1, 0.0]], [[1.0, -1.0, 2.0, -0.0]]])
    np.testing.assert_array_equal(oracle.harden(lt, GRID_TERNARY)[0], [2, 0, 1, 2])
    ll = np.zeros((5, 1, 3))
    ll[4, 0, :] = 1.0                     # offset +2
    np.testing.assert_array_equal(oracle.harden(ll, GRID_INT3_LOCAL, np.array([[0, 6, 3]]))[0],
                                  [2, 7, 5])
    lf = np.zeros((8, 1, 3))
    lf[[6, 2], 0, 0] = 1.5                # tie between levels 2 and 6 -> 2
    lf[7, 0, 1] = 0.1
    np.testing.assert_array_equal(oracle.harden(lf, GRID_INT3)[0], [2, 7, 0])


@pytest.mark.parametrize("bits,K", [(2, 128), (3, 128), (2, 384), (3, 256)])
def test_packing_matches_big_integer_stream(bits, K):
    rng = np.random.default_rng(bits * 1000 + K)
    codes = rng.integers(0, 2 ** bits, size=(3, K), dtype=np.uint8)
    packed = oracle.pack_codes(codes, bits)
    assert packed.shape == (3, K * bits // 32) and packed.dtype == np.uint32
    for r in range(3):
        big = sum(int(c) << (bits * j) for j, c in enumerate(codes[r]))
        words = [(big >> (32 * w)) & 0xFFFFFFFF for w in range(K * bits // 32)]
        assert [int(x) for x in packed[r]] == words
    np.testing.assert_array_equal(oracle.unpack_codes(packed, K, bits), codes)


def test_pack_example_by_hand():
    # 2 bits: codes 0,1,2,3 -> 0b11100100 = 0xE4 per byte.
    np.testing.assert_array_equal(oracle.pack_codes(np.tile([0, 1, 2, 3], 16)[None].astype(np.uint8), 2),
                                  [[0xE4E4E4E4] * 4])
    # 3 bits: codes 0..7 fill 24 bits as octal 76543210 = 0xFAC688; then
    # code 0 (bits 24-26), code 1 (bit 27) and the low two bits of code 2
    # (bits 30-31 = 0b10): top byte 0x88 -> word 0x88FAC688; bit 32 (the high
    # bit of code 2 = 0) starts the next word.
    w = oracle.pack_codes(np.tile(np.arange(8), 16)[None].astype(np.uint8), 3)
    assert int(w[0, 0]) == 0x88FAC688
    assert int(w[0, 1]) & 1 == 0


def test_fp16_scales_round_to_nearest_even():
    s = np.array([1.0 + 2 ** -11, 1.0 + 3 * 2 ** -11, 65504.0, 2 ** -25, 0.0], dtype=np.float32)
    bits = oracle.scales_to_f16_bits(s)
    np.testing.assert_array_equal(bits, [0x3C00, 0x3C02, 0x7BFF, 0x0000, 0x0000])


def test_format_numbers_printed_on_the_pages():
    gold = json.load(open(os.path.join(HERE, "golden", "paper_numbers.json")))
    group = gold["group_size"]["value"]
    scale_bits = 16
    assert abs(oracle.CODE_BITS[GRID_INT2] + scale_bits / group - gold["bits_per_param_2bit"]["value"]) <= 0.005
    assert abs(oracle.CODE_BITS[GRID_INT3_LOCAL] + scale_bits / group - gold["bits_per_param_3bit"]["value"]) <= 0.005
    assert abs(math.log2(3) + scale_bits / group - gold["bits_per_param_ternary"]["value"]) <= 0.005
    assert oracle.N_LOGITS[GRID_INT2] == gold["logits_per_coord_2bit"]["value"]
    assert oracle.N_LOGITS[GRID_INT3_LOCAL] == gold["logits_per_coord_local_shift"]["value"]
    assert 2 ** oracle.CODE_BITS[GRID_INT3_LOCAL] == gold["logits_per_coord_full_3bit"]["value"]
    assert list(oracle.LOCAL_OFFSETS) == gold["local_shift_offsets"]["value"]
    assert oracle.N_LOGITS[GRID_TERNARY] / oracle.N_LOGITS[GRID_INT2] == gold["ternary_logit_ratio_to_2bit"]["value"]
    assert oracle.N_LOGITS[GRID_INT3] == gold["logits_per_coord_full_3bit"]["value"]
    # the 2-5x logit memory covers the grids GSQ uses (not the full 3-bit baseline)
    lo, hi = gold["logit_memory_ratio_range"]["value"]
    used = [oracle.N_LOGITS[g] for g in (GRID_INT2, GRID_TERNARY, GRID_INT3_LOCAL)]
    assert min(used) == lo and max(used) == hi


def test_tau_schedule_endpoints():
    tau = oracle.tau_schedule(200, 1.0, 0.05)
    assert tau[0] == np.float32(1.0) and tau[-1] == np.float32(0.05)
    r = tau[1:].astype(np.float64) / tau[:-1]
    np.testing.assert_allclose(r, 0.05 ** (1 / 199), rtol=1e-6)


def test_round_bf16():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -9], dtype=np.float32)
    np.testing.assert_array_equal(oracle.round_bf16(x), [1.0, 1.0, 1.0 + 2 ** -6, -2.5, 1.0])


# ----------------------------------------------------------------------------
# Noise layout and row chunking
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("grid", GRIDS)
def test_noise_layout_per_coordinate(grid):
    # Coordinate (r, j) of rows starting at row0 draws stream elements
    # e = ((row0 + r) * cols + j) * L + k.
    L = oracle.N_LOGITS[grid]
    rows, cols, row0 = 2, 8, 5
    n = oracle.noise(grid, rows, cols, 3, 4, 6, row0)
    inv = oracle.logistic if grid == GRID_TERNARY else oracle.gumbel
    for k in range(L):
        for r in range(rows):
            for j in range(cols):
                e = ((row0 + r) * cols + j) * L + k
                u = oracle.uniform_from_word(oracle.noise_words(3, 4, 6, [e]))
                assert n[k, r, j] == inv(u)[0]


@pytest.mark.parametrize("grid", GRIDS)
def test_row_chunks_agree_with_whole_layer(grid):
    M, K = 6, 256
    W = layer(M, K)
    s, c0, _ = oracle.init_rtn(W, grid)
    lg = rand_logits(grid, M, K)
    G = np.random.default_rng(2).normal(size=(M, K))
    full = oracle.relax_fwd(lg, s, W, grid, 1, 2, 3, 0.6, 1.0, c0)["w_soft"]
    gl, gs = oracle.relax_bwd(G, lg, s, grid, 1, 2, 3, 0.6, 1.0, c0)
    r = slice(2, 5)
    part = oracle.relax_fwd(lg[:, r], s[r], W[r], grid, 1, 2, 3, 0.6, 1.0, c0[r], row0=2)["w_soft"]
    pgl, pgs = oracle.relax_bwd(G[r], lg[:, r], s[r], grid, 1, 2, 3, 0.6, 1.0, c0[r], row0=2)
    np.testing.assert_array_equal(part, full[r])
    np.testing.assert_array_equal(pgl, gl[:, r])
    np.testing.assert_array_equal(pgs, gs[r])


@pytest.mark.parametrize("grid", GRIDS)
def test_step_on_row_blocks_equals_whole_layer_step(grid):
    # Rows are independent in the objective (R[:, r] = X dW[r]^T and G[r] =
    # 2 R[:, r]^T X), so whole steps on row blocks placed with row0 give the
    # rows of the whole-layer step, and their losses sum to its loss.
    M, K, N = 5, 256, 64
    W = layer(M, K)
    X = np.random.default_rng(3).normal(size=(N, K))
    s, c0, lg = oracle.init_rtn(W, grid)

    def fresh(r):
        return {"logits": lg[:, r].copy(), "mom": np.zeros_like(lg[:, r]), "scales": s[r].copy(),
                "scale_mom": np.zeros_like(s[r]), "codes": c0[r].copy()}

    whole = fresh(slice(0, M))
    blocks = [(slice(0, 2), fresh(slice(0, 2))), (slice(2, M), fresh(slice(2, M)))]
    for t, tau in enumerate((1.0, 0.5, 0.2)):
        loss = oracle.step(whole, W, X, grid, t, tau, 7, 1, 5e-2, 1e-4, bf16_dW=True, bf16_RT=True)
        parts = [oracle.step(st, W[r], X, grid, t, tau, 7, 1, 5e-2, 1e-4, bf16_dW=True,
                             bf16_RT=True, row0=r.start) for r, st in blocks]
        assert abs(sum(parts) - loss) <= 1e-12 * loss
    for r, st in blocks:
        for key in ("logits", "mom"):
            np.testing.assert_array_equal(st[key], whole[key][:, r])
        for key in ("scales", "scale_mom"):
            np.testing.assert_array_equal(st[key], whole[key][r])


def test_offset_objective():
    """R = X dW^T + E0: the loss is ||X W_soft^T - Y||^2 for E0 = X W^T - Y
    (computed token by token, independently), zero at the dW that makes the
    output match, the plain objective for E0 = 0, and its gradient matches
    central finite differences."""
    rng = np.random.default_rng(12)
    n, k, m = 30, 16, 5
    X = rng.normal(size=(n, k))
    W = rng.normal(size=(m, k)) * 0.1
    Y = rng.normal(size=(n, m))
    D = rng.normal(size=(m, k)) * 0.01
    E0T = (X @ W.T - Y).T
    RT, loss, G = oracle.recon_loss_grad_offset(X, D, E0T)
    want = sum(float(np.dot(X[t], W[o] + D[o]) - Y[t, o]) ** 2 for t in range(n) for o in range(m))
    assert math.isclose(loss, want, rel_tol=1e-12)
    # the dW that reproduces Y exactly where Y is reachable: Y = X W2^T
    W2 = rng.normal(size=(m, k)) * 0.1
    _, l0, G0 = oracle.recon_loss_grad_offset(X, W2 - W, (X @ W.T - X @ W2.T).T)
    assert l0 <= 1e-20 and np.abs(G0).max() <= 1e-12
    _, lp, Gp = oracle.recon_loss_grad(X, D)
    _, lz, Gz = oracle.recon_loss_grad_offset(X, D, np.zeros((m, n)))
    assert lz == lp and np.array_equal(Gz, Gp)
    h = 1e-7
    for idx in [(0, 0), (2, 9), (4, 15)]:
        Dp, Dm = D.copy(), D.copy()
        Dp[idx] += h
        Dm[idx] -= h
        fd = (oracle.recon_loss_grad_offset(X, Dp, E0T)[1]
              - oracle.recon_loss_grad_offset(X, Dm, E0T)[1]) / (2 * h)
        assert abs(fd - G[idx]) <= 1e-6 * np.abs(G).max()
