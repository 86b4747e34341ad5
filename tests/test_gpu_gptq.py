"""GPU parity of the GPTQ warm start (gsq_init_gptq) with the oracle.

The GPU runs GPTQ's recursion on the factor of H (nearest plane, fp64), the
oracle runs GPTQ's own inverse-Cholesky column loop (fp64): the rounding
decision values agree to about 1e-12 relative, so codes agree except where a
value sits on a rounding boundary. Such a tie may go either way; once a row
has taken a different code its later columns see different errors, so a row
is compared up to its first difference, which must be at a tie.
"""

import numpy as np
import pytest

import oracle
import synthetic
from oracle import gsq as ogsq
from tests.gpu_util import device, to_dev_bf16, bf16_values, f32, report

pytestmark = pytest.mark.gpu

GRIDS = [oracle.GRID_INT2, oracle.GRID_TERNARY, oracle.GRID_INT3_LOCAL, oracle.GRID_INT3]


def _run(d, grid, dev, damp=0.01, M=None):
    import torch
    import post_weight_quantization_philox_amd as g
    W = d["W"] if M is None else d["W"][:M]
    M, K = W.shape
    N = d["X"].shape[0]
    Wd = to_dev_bf16(d["W_bits"][:M], dev) if d["W_bits"] is not None else torch.from_numpy(W).to(dev)
    Xd = to_dev_bf16(d["X_bits"], dev)
    XT = torch.empty((N * K,), dtype=torch.bfloat16, device=dev)
    g.gsq_transpose_tokens(1, [0, N], K, Xd, XT)
    layer = g.GsqLayer.make(grid, M, K, g.DTYPE_BF16 if d["W_bits"] is not None else g.DTYPE_F32)
    nbytes = g.gsq_gptq_workspace_bytes(M, K)
    ws = torch.empty((nbytes,), dtype=torch.uint8, device=dev)
    scales = torch.empty((M, K // 128), dtype=torch.float32, device=dev)
    codes = torch.empty((M, K), dtype=torch.uint8, device=dev)
    logits = torch.empty((oracle.N_LOGITS[grid], M, K), dtype=torch.float32, device=dev)
    info = torch.full((1,), -7, dtype=torch.int32, device=dev)
    g.gsq_init_gptq(layer, Wd, N, XT, damp, 2.0, ws, scales, codes, logits, info)
    torch.cuda.synchronize()
    return W, ws, f32(scales), codes.cpu().numpy(), f32(logits), int(info.item())


def _tie_distance(t, s, grid):
    """Distance of each decision value from the nearest rounding boundary,
    in the units rint works in."""
    _, u = ogsq._nearest_code(t, s, grid)
    u = u.astype(np.float64)
    return np.abs(np.abs(u - np.floor(u)) - 0.5)


def _compare_rows(c_gpu, c_ref, T_ref, scales, grid, tol=1e-5):
    sf = np.repeat(scales, 128, axis=1)
    bad_rows = 0
    for r in range(c_gpu.shape[0]):
        diff = np.nonzero(c_gpu[r] != c_ref[r])[0]
        if diff.size == 0:
            continue
        j = int(diff[0])
        dist = _tie_distance(T_ref[r, j:j + 1], sf[r, j:j + 1], grid)[0]
        assert dist <= tol, f"row {r}: first difference at column {j} is {dist:.3g} from a tie"
        assert abs(int(c_gpu[r, j]) - int(c_ref[r, j])) == 1     # the other side of the tie
        bad_rows += 1
    return bad_rows


@pytest.fixture(scope="module")
def dev():
    return device()


@pytest.mark.parametrize("grid", GRIDS)
@pytest.mark.parametrize("shape", [(64, 512, 256), (37, 384, 192), (40, 128, 192)])
@pytest.mark.parametrize("w_bf16", [True, False])
def test_gptq_parity(dev, grid, shape, w_bf16):
    M, K, N = shape
    d = synthetic.small_layer(M, K, N, seed=M + K, w_bf16=w_bf16)
    W, ws, s, c, lg, info = _run(d, grid, dev)
    assert info == 0
    s_ref, c_ref, lg_ref, T_ref = oracle.gptq(W, d["X"], grid)
    np.testing.assert_array_equal(s.view(np.uint32), s_ref.view(np.uint32))
    bad = _compare_rows(c, c_ref, T_ref, s_ref, grid)
    moved = float(np.mean(c_ref != oracle.init_rtn(W, grid)[1]))
    report(f"gptq grid={grid} {shape} bf16={w_bf16}", rows_split_at_a_tie=bad, codes_moved_vs_rtn=moved)
    assert bad <= max(1, M // 20)
    assert moved > 0.01
    # logits follow the GPU's own codes exactly as the warm start sets them
    np.testing.assert_array_equal(lg.view(np.uint32),
                                  ogsq._logits_from_codes(c, W, grid, 2.0).view(np.uint32))


def test_gptq_more_rows_than_one_pass(dev):
    """More rows than one pass of the group kernel's workgroups covers (256
    workgroups of 32 rows), with a ragged last block: every row against the
    oracle."""
    M, K, N = 8200, 256, 192
    d = synthetic.small_layer(M, K, N, seed=21)
    W, ws, s, c, lg, info = _run(d, oracle.GRID_INT2, dev)
    assert info == 0
    s_ref, c_ref, _, T_ref = oracle.gptq(W, d["X"], oracle.GRID_INT2)
    np.testing.assert_array_equal(s.view(np.uint32), s_ref.view(np.uint32))
    bad = _compare_rows(c, c_ref, T_ref, s_ref, oracle.GRID_INT2)
    report("gptq 8200 rows", rows_split_at_a_tie=bad,
           codes_moved_vs_rtn=float(np.mean(c_ref != oracle.init_rtn(W, 0)[1])))
    assert bad <= max(1, M // 20)


def test_gptq_factor_matches_cholesky(dev):
    """The workspace's intermediates: the fp32 Gram matrix against X^T X, and
    the fp64 factor computed from that fp32 matrix: lower triangle =
    Cholesky of the reversed, damped Gram matrix; upper triangle
    V_ij = R_ij / R_jj with R the factor in the original order."""
    M, K, N = 16, 256, 320
    d = synthetic.small_layer(M, K, N, seed=3)
    _, ws, _, _, _, info = _run(d, oracle.GRID_INT2, dev)
    assert info == 0
    raw = ws.cpu().numpy()
    H32 = raw[:K * K * 4].view(np.float32).reshape(K, K).astype(np.float64)
    X = d["X"].astype(np.float64)
    gam = (N + 2) * 2.0 ** -24 * (np.abs(X).T @ np.abs(X))
    assert np.all(np.abs(H32 - X.T @ X) <= gam)
    h_bytes = (K * K * 4 + 255) // 256 * 256
    A = raw[h_bytes:h_bytes + K * K * 8].view(np.float64).reshape(K, K)
    diag = np.diag(H32).copy()
    diag[diag == 0] = 1.0
    H = H32.copy()
    # damp reaches the kernels as fp32 0.01
    H[np.diag_indices_from(H)] = diag + float(np.float32(0.01)) * float(np.mean(diag))
    J = np.arange(K)[::-1]
    L = np.linalg.cholesky(H[np.ix_(J, J)])
    low = np.tril(np.ones((K, K), dtype=bool))
    np.testing.assert_allclose(A[low], L[low], rtol=0, atol=1e-11 * np.abs(L).max())
    R = L[np.ix_(J, J)]
    up = np.triu(np.ones((K, K), dtype=bool), 1)
    V = R / np.diag(R)[None, :]
    np.testing.assert_allclose(A[up], V[up], rtol=0, atol=1e-11)


def test_gptq_lowers_the_objective(dev):
    M, K, N = 128, 512, 1024
    d = synthetic.small_layer(M, K, N, seed=8)
    for grid in (oracle.GRID_INT2, oracle.GRID_INT3):
        W, _, s, c, _, info = _run(d, grid, dev)
        s0, c0, _ = oracle.init_rtn(W, grid)
        lg = oracle.hard_loss(c, s, W, d["X"], grid)
        l0 = oracle.hard_loss(c0, s0, W, d["X"], grid)
        report(f"gptq objective grid={grid}", rtn=l0, gptq=lg, ratio=lg / l0)
        assert info == 0 and lg < 0.9 * l0


def test_gptq_rank_deficient_without_damping_reports_info(dev):
    # 64 tokens, 256 in-features, no damping: H has rank 64, so a pivot fails.
    d = synthetic.small_layer(8, 256, 64, seed=2)
    _, _, _, c, lg, info = _run(d, oracle.GRID_INT2, dev, damp=0.0)
    assert info > 0
    assert np.all(c <= 3) and np.all(np.isfinite(lg))


def test_gptq_rejects_bad_arguments(dev):
    import torch
    import post_weight_quantization_philox_amd as g
    K, M = 128, 4
    layer = g.GsqLayer.make(g.GRID_INT2, M, K)
    W = torch.zeros((M, K), dtype=torch.bfloat16, device=dev)
    XT = torch.zeros((K * 64,), dtype=torch.bfloat16, device=dev)
    ws = torch.zeros((g.gsq_gptq_workspace_bytes(M, K),), dtype=torch.uint8, device=dev)
    out = [torch.zeros((M, 1), device=dev), torch.zeros((M, K), dtype=torch.uint8, device=dev),
           torch.zeros((4, M, K), device=dev), torch.zeros((1,), dtype=torch.int32, device=dev)]
    for tokens, damp, nbytes in [(63, 0.01, None), (64, -1.0, None), (64, 0.01, 16)]:
        with pytest.raises(g.GsqError):
            g.gsq_init_gptq(layer, W, tokens, XT, damp, 2.0, ws, *out, workspace_bytes=nbytes)
    assert g.gsq_gptq_workspace_bytes(4, 100) == 0


def test_gptq_fullsize_sampled_rows(dev):
    """The 4096x4096 q_proj layer: sampled rows of the GPU's GPTQ codes
    against the oracle run on those rows with the full calibration set."""
    import torch
    from post_weight_quantization_philox_amd.solver import LayerSolver
    data = synthetic.generate("qproj4096_int2", seed=0)
    sol = LayerSolver(to_dev_bf16(data["W_bits"], dev), to_dev_bf16(data["X_bits"], dev),
                      oracle.GRID_INT2, init="gptq")
    torch.cuda.synchronize()
    assert int(sol.gptq_info.item()) == 0
    rows = [0, 1, 2047, 4095]
    c = sol.codes[rows].cpu().numpy()
    s = f32(sol.scales[rows])
    s_ref, c_ref, _, T_ref = oracle.gptq(data["W"][rows], data["X"], oracle.GRID_INT2)
    np.testing.assert_array_equal(s.view(np.uint32), s_ref.view(np.uint32))
    bad = _compare_rows(c, c_ref, T_ref, s_ref, oracle.GRID_INT2)
    report("gptq 4096x4096 sampled rows", rows_split_at_a_tie=bad,
           codes_moved_vs_rtn=float(np.mean(c_ref != oracle.init_rtn(data["W"][rows], 0)[1])))
    assert bad <= 1
