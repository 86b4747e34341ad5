"""Parity of every GPU entry point with the CPU oracle on identical inputs.

Each GPU call is compared with the oracle given that call's exact inputs
(seeded synthetic layers, the same Philox noise, the GPU's own intermediate
tensors where a later call consumes them). Integer results are compared
bit-exactly; floating-point results within the bounds derived in the design
notes (fp32 evaluation of z = (l + eta*g)/tau, bf16 operand rounding).
"""

import numpy as np
import pytest

import oracle
import synthetic
from tests.gpu_util import device, to_dev_bf16, bf16_values, f32, bf16_ulp, report

pytestmark = pytest.mark.gpu

GRIDS = [oracle.GRID_INT2, oracle.GRID_TERNARY, oracle.GRID_INT3_LOCAL, oracle.GRID_INT3]
SHAPES = [(64, 512), (5, 384)]          # several scale groups per row; ragged row count

# Soft weights and logit gradients: 1e-5 of their natural scale (s * q_max,
# and |G| * s * q_max / tau). The fp32 evaluation of y = (l + eta*g)/tau can
# in the worst case reach about 2^-22 * (|l| + |g|) / tau (4e-5 at tau = 0.05);
# measured maxima on these inputs stay below 4e-6 at tau = 0.05, so the
# tolerance is the flat 1e-5 for every tau >= 0.05.
def z_tol(tau, lmax):
    return 1e-5


@pytest.fixture(scope="module")
def dev():
    return device()


def _layer_inputs(grid, M, K, seed, w_bf16=True, spread=1.5):
    d = synthetic.small_layer(M, K, 64, seed=seed, w_bf16=w_bf16)
    W = d["W"]
    s, c0, _ = oracle.init_rtn(W, grid)
    lg = np.random.default_rng(seed + 1).normal(0, spread, (oracle.N_LOGITS[grid], M, K)).astype(np.float32)
    return d, W, s, c0, lg


def _w_dev(d, dev):
    import torch
    if d["W_bits"] is not None:
        return to_dev_bf16(d["W_bits"], dev)
    return torch.from_numpy(d["W"]).to(dev)


# ----------------------------------------------------------------------------
# Noise
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("seed,sid,step,first,count", [
    (0, 0, 0, 0, 4096),
    (0x0123456789ABCDEF, 7, 199, 12345, 3000),
    (42, 0xFFFFFFFF, 0xFFFFFFFF, (1 << 34) + 3, 1000),
])
def test_noise_stream_bit_exact(dev, seed, sid, step, first, count):
    import torch
    import post_weight_quantization_philox_amd as g
    layer = g.GsqLayer.make(g.GRID_INT2, 1, 128, seed=seed, stream=sid)
    out = torch.zeros(count, dtype=torch.int32, device=dev)
    g.gsq_noise_dump(layer, step, first, count, out)
    got = out.cpu().numpy().view(np.uint32)
    ref = oracle.noise_words(seed, sid, step, np.arange(first, first + count, dtype=np.uint64))
    np.testing.assert_array_equal(got, ref)


# ----------------------------------------------------------------------------
# Warm start
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("grid", GRIDS)
@pytest.mark.parametrize("w_bf16", [True, False])
def test_init_rtn_bit_exact(dev, grid, w_bf16):
    import torch
    import post_weight_quantization_philox_amd as g
    M, K = 37, 384
    d = synthetic.small_layer(M, K, 64, seed=3, w_bf16=w_bf16)
    W = d["W"].copy()
    W[1, :128] = 0.0                                   # all-zero group
    qmax = oracle.Q_MAX[grid]
    step_ = 2.0 ** -6
    W[2, :128] = 0.0
    W[2, 0] = qmax * step_                             # maxabs -> exact scale step_
    W[2, 1:16] = np.arange(-7, 8) * step_ * 0.5        # exact ties of w/s at half-integers
    if w_bf16:
        bits = synthetic.bf16_bits(W)
        W = synthetic.bf16_to_f32(bits)
        Wd = to_dev_bf16(bits, dev)
        wdt = g.DTYPE_BF16
    else:
        Wd = torch.from_numpy(W).to(dev)
        wdt = g.DTYPE_F32
    L = oracle.N_LOGITS[grid]
    layer = g.GsqLayer.make(grid, M, K, wdt)
    scales = torch.empty((M, K // 128), dtype=torch.float32, device=dev)
    codes = torch.empty((M, K), dtype=torch.uint8, device=dev)
    logits = torch.empty((L, M, K), dtype=torch.float32, device=dev)
    g.gsq_init_rtn(layer, Wd, scales, codes, logits, 2.0)
    s_ref, c_ref, l_ref = oracle.init_rtn(W, grid)
    np.testing.assert_array_equal(f32(scales).view(np.uint32), s_ref.view(np.uint32))
    np.testing.assert_array_equal(codes.cpu().numpy(), c_ref)
    np.testing.assert_array_equal(f32(logits).view(np.uint32), l_ref.view(np.uint32))


# ----------------------------------------------------------------------------
# Relaxed forward
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("grid", GRIDS)
@pytest.mark.parametrize("tau", [1.0, 0.3, 0.05])
@pytest.mark.parametrize("eta", [1.0, 0.0])
@pytest.mark.parametrize("shape", SHAPES)
def test_relax_fwd(dev, grid, tau, eta, shape):
    import torch
    import post_weight_quantization_philox_amd as g
    M, K = shape
    d, W, s, c0, lg = _layer_inputs(grid, M, K, seed=11, w_bf16=(M != 5))
    layer = g.GsqLayer.make(grid, M, K, g.DTYPE_BF16 if d["W_bits"] is not None else g.DTYPE_F32,
                            seed=77, stream=3)
    step = 17
    dW = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    ws = torch.empty((M, K), dtype=torch.float32, device=dev)
    codes = torch.from_numpy(c0).to(dev)
    g.gsq_relax_fwd(layer, torch.from_numpy(lg).to(dev), torch.from_numpy(s).to(dev),
                    codes, _w_dev(d, dev), step, tau, eta, dW, ws)
    torch.cuda.synchronize()
    ref = oracle.relax_fwd(lg, s, W, grid, 77, 3, step, float(np.float32(tau)), eta, c0)
    nat = np.repeat(s.astype(np.float64), 128, axis=1) * oracle.Q_MAX[grid]
    nat = np.maximum(nat, 1e-30)
    err = np.abs(f32(ws) - ref["w_soft"]) / nat
    tol = z_tol(tau, np.abs(lg).max())
    report(f"relax_fwd grid={grid} tau={tau} eta={eta} {M}x{K}", max_rel=float(err.max()),
           p999=float(np.quantile(err, 0.999)), tol=tol)
    assert err.max() <= tol
    # dW: the bf16 rounding of w_soft - W; within one bf16 ulp of the exact
    # difference plus the w_soft error.
    got = bf16_values(dW).astype(np.float64)
    bound = bf16_ulp(ref["dW"]) + tol * nat
    assert np.all(np.abs(got - ref["dW"]) <= bound)
    exact = np.mean(got == oracle.round_bf16(ref["dW"]).astype(np.float64))
    report("  dW bf16 exact-match fraction", frac=float(exact))
    assert exact > 0.99


# ----------------------------------------------------------------------------
# Relaxed backward and Lion
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("grid", GRIDS)
@pytest.mark.parametrize("tau", [1.0, 0.3, 0.05])
@pytest.mark.parametrize("shape", SHAPES)
def test_relax_bwd_lion(dev, grid, tau, shape):
    import torch
    import post_weight_quantization_philox_amd as g
    M, K = shape
    d, W, s, c0, lg = _layer_inputs(grid, M, K, seed=21)
    rng = np.random.default_rng(5)
    G = (rng.normal(0, 1.0, (M, K)) * 50.0).astype(np.float32)
    L = oracle.N_LOGITS[grid]
    mom = (rng.normal(0, 1.0, (L, M, K)) * 1e-2).astype(np.float32)
    smom = (rng.normal(0, 1.0, s.shape) * 1e-3).astype(np.float32)
    lion = g.GsqLion.make(lr_logit=1e-3, lr_scale=1e-5, beta1=0.9, beta2=0.99, weight_decay=0.0)
    layer = g.GsqLayer.make(grid, M, K, g.DTYPE_BF16, seed=5, stream=9)
    step = 123
    t_lg = torch.from_numpy(lg).to(dev)
    t_mom = torch.from_numpy(mom).to(dev)
    t_s = torch.from_numpy(s).to(dev)
    t_sm = torch.from_numpy(smom).to(dev)
    gl = torch.empty((L, M, K), dtype=torch.float32, device=dev)
    gs = torch.empty(s.shape, dtype=torch.float32, device=dev)
    g.gsq_relax_bwd_lion(layer, torch.from_numpy(G).to(dev), t_lg, t_mom, t_s, t_sm,
                         torch.from_numpy(c0).to(dev), step, tau, 1.0, lion, gl, gs)
    torch.cuda.synchronize()
    tau32 = float(np.float32(tau))
    gl_ref, gs_ref = oracle.relax_bwd(G, lg, s, grid, 5, 9, step, tau32, 1.0, c0)
    # Logit gradient, relative to its natural scale |G| s q_max / tau.
    sfull = np.repeat(s.astype(np.float64), 128, axis=1)
    nat = np.maximum(np.abs(G) * sfull * oracle.Q_MAX[grid] / tau32, 1e-30)
    err = np.abs(f32(gl) - gl_ref) / nat[None]
    tol = z_tol(tau, np.abs(lg).max())
    # Per coordinate, relative to the largest of its L gradients, on the
    # coordinates whose gradient is at least 1e-3 of the natural scale (a
    # saturated softmax makes the rest vanish): reported, the bar being the
    # elementwise one above.
    cmax = np.abs(gl_ref).max(axis=0)
    live = cmax >= 1e-3 * nat
    pc = (np.abs(f32(gl) - gl_ref).max(axis=0) / np.maximum(cmax, 1e-300))[live]
    report(f"grad_logits grid={grid} tau={tau} {M}x{K}", max_rel=float(err.max()), tol=tol,
           per_coord_max=float(pc.max()), per_coord_p999=float(np.quantile(pc, 0.999)),
           per_coord_median=float(np.median(pc)), per_coord_within_1e5=float(np.mean(pc <= 1e-5)),
           live_coords=float(live.mean()))
    assert err.max() <= tol
    # Scale gradient, relative to the group's L1 mass sum |G * w_hat|.
    f = oracle.relax_fwd(lg, s, W, grid, 5, 9, step, tau32, 1.0, c0)
    # Scale gradient: 128-term fp32 sum (worst case 130 * 2^-24 of the L1
    # mass sum |G * w_hat|) plus the w_hat error (tol * q_max per term).
    mass = (np.abs(G) * np.abs(f["w_hat"])).reshape(M, -1, 128).sum(axis=2)
    gabs = np.abs(G).reshape(M, -1, 128).sum(axis=2)
    allowed = 130 * 2.0 ** -24 * mass + tol * oracle.Q_MAX[grid] * gabs
    serr = np.abs(f32(gs) - gs_ref)
    report("  grad_scales", max_rel_mass=float((serr / mass).max()), max_over_bound=float((serr / allowed).max()))
    assert np.all(serr <= allowed)
    # Lion, level 1: the oracle's update fed the GPU's own gradients is
    # bit-exact on the parameters and within one fp32 ulp on the momenta.
    th1, m1 = oracle.lion(lg, f32(gl), mom, 1e-3, 0.9, 0.99, 0.0)
    np.testing.assert_array_equal(f32(t_lg).view(np.uint32), th1.view(np.uint32))
    mscale = 0.99 * np.abs(mom) + 0.01 * np.abs(f32(gl))
    assert np.all(np.abs(f32(t_mom) - m1) <= 2.0 ** -23 * mscale + 1e-38)
    ths, ms = oracle.lion(s, f32(gs), smom, 1e-5, 0.9, 0.99, 0.0)
    np.testing.assert_array_equal(f32(t_s).view(np.uint32), ths.view(np.uint32))
    # Lion, level 2: end to end with the oracle's own gradient; a parameter
    # may move the other way only where c is within the gradient tolerance of 0.
    th2, _ = oracle.lion(lg, gl_ref, mom, 1e-3, 0.9, 0.99, 0.0)
    diff = f32(t_lg) != th2
    c_ref = 0.9 * mom.astype(np.float64) + 0.1 * gl_ref
    ambiguous = np.abs(c_ref) <= 0.1 * tol * nat[None] * 4
    report("  lion end-to-end", mismatches=int(diff.sum()), ambiguous=int(ambiguous.sum()))
    assert np.all(ambiguous[diff])


# ----------------------------------------------------------------------------
# Reconstruction GEMMs
# ----------------------------------------------------------------------------

# 67 experts of 32 rows with 0, 64 or 128 tokens each: more experts than one
# grouped launch takes (64), so each product runs as two launches.
_OFFS67 = [0] + np.cumsum(np.random.default_rng(67).choice([0, 64, 128], 67)).tolist()


@pytest.mark.parametrize("M,N,K,offs", [
    (512, 256, 512, None),            # one linear layer, several tiles
    (300, 192, 384, None),            # ragged rows, partial tiles
    (3 * 256, 320, 256, [0, 128, 128, 320]),   # three experts, one with no tokens
    (67 * 32, _OFFS67[-1], 256, _OFFS67),      # two grouped launches per product
    # Products over more than one round of 256 tiles that do not fill the
    # last round: whole rounds of 256x256 tiles on a column or row block, the
    # rest in 256x128 tiles (ragged where the sizes are).
    (4000, 64, 5120, None),           # G: column block + 128-wide tail
    (5000, 64, 4096, None),           # G: row block + 128-wide ragged tail
    (4000, 5056, 128, None),          # R^T: column block + ragged tail
    (5000, 4096, 128, None),          # R^T: row block + ragged tail
])
def test_recon_loss_grad(dev, M, N, K, offs):
    import torch
    import post_weight_quantization_philox_amd as g
    rng = np.random.default_rng(M + N + K)
    dW_bits = synthetic.bf16_bits((rng.normal(0, 0.01, (M, K))).astype(np.float32))
    X_bits = synthetic.bf16_bits(rng.normal(0, 1, (N, K)).astype(np.float32))
    dW = synthetic.bf16_to_f32(dW_bits).astype(np.float64)
    X = synthetic.bf16_to_f32(X_bits).astype(np.float64)
    if offs is None:
        offs = [0, N]
    E = len(offs) - 1
    rpe = M // E
    tdW = to_dev_bf16(dW_bits, dev)
    tX = to_dev_bf16(X_bits, dev)
    XT = torch.empty((N * K,), dtype=torch.bfloat16, device=dev)
    g.gsq_transpose_tokens(E, offs, K, tX, XT)
    RT = torch.empty((rpe * N,), dtype=torch.bfloat16, device=dev)
    G = torch.full((M, K), float("nan"), dtype=torch.float32, device=dev)
    ws = torch.empty((g.gsq_recon_workspace_bytes(E, offs, rpe, K) // 4,), dtype=torch.float32,
                     device=dev)
    loss = torch.zeros((1,), dtype=torch.float64, device=dev)
    g.gsq_recon_loss_grad(E, offs, rpe, K, tX, XT, tdW, ws, RT, G, loss)
    torch.cuda.synchronize()
    # transpose is exact
    XT_h = bf16_values(XT).astype(np.float64)
    for e in range(E):
        n = offs[e + 1] - offs[e]
        blk = XT_h[K * offs[e]:K * offs[e + 1]].reshape(K, n)
        np.testing.assert_array_equal(blk, X[offs[e]:offs[e + 1]].T)
    RTs, loss_ref, G_ref = oracle.recon_loss_grad_grouped(X, offs, dW, rpe)
    rel = abs(float(loss.item()) - loss_ref) / loss_ref
    report(f"recon loss {M}x{N}x{K} E={E}", rel=rel)
    assert rel <= 1e-5
    RT_h = bf16_values(RT).astype(np.float64)
    Gd = f32(G).astype(np.float64)
    for e in range(E):
        n = offs[e + 1] - offs[e]
        r = slice(e * rpe, (e + 1) * rpe)
        if n == 0:
            assert not Gd[r].any()
            continue
        got_rt = RT_h[rpe * offs[e]:rpe * offs[e + 1]].reshape(rpe, n)
        # R^T: an fp32 dot product of K terms (worst-case error K*2^-24 of the
        # sum of |terms|) rounded once to bf16 (half a bf16 ulp).
        Xe = X[offs[e]:offs[e + 1]]
        gam = (K + 2) * 2.0 ** -24 * (np.abs(dW[r]) @ np.abs(Xe).T)
        assert np.all(np.abs(got_rt - RTs[e]) <= 0.5 * bf16_ulp(RTs[e]) + gam + 1e-30)
        # G from the GPU's own bf16 R^T, exact in fp64, against the same
        # worst-case bound for n tokens.
        Ge = 2.0 * got_rt @ Xe
        bound = (n + 2) * 2.0 ** -24 * (2.0 * np.abs(got_rt) @ np.abs(Xe))
        assert np.all(np.abs(Gd[r] - Ge) <= bound + 1e-30)
        nrm = np.linalg.norm(Gd[r] - Ge) / np.linalg.norm(Ge)
        report(f"  G expert {e}", normwise=float(nrm))
        assert nrm <= 1e-5


@pytest.mark.parametrize("M,N,K", [
    (512, 256, 512),                  # several tiles
    (300, 192, 384),                  # ragged rows, partial tiles
    (4000, 5056, 128),                # R^T: column block + ragged 128-wide tail
    (5000, 4096, 128),                # R^T: row block + ragged tail
])
def test_recon_loss_grad_offset(dev, M, N, K):
    """R = X dW^T + E0 (a layer fitted to a target downstream): E0^T enters
    the first product's epilogue, so R^T, the loss and G follow the oracle's
    offset objective; the offset is read at the right place in split tiles."""
    import torch
    import post_weight_quantization_philox_amd as g
    rng = np.random.default_rng(M + 3 * N + K)
    dW_bits = synthetic.bf16_bits((rng.normal(0, 0.01, (M, K))).astype(np.float32))
    X_bits = synthetic.bf16_bits(rng.normal(0, 1, (N, K)).astype(np.float32))
    E_bits = synthetic.bf16_bits(rng.normal(0, 0.1, (M, N)).astype(np.float32))
    dW = synthetic.bf16_to_f32(dW_bits).astype(np.float64)
    X = synthetic.bf16_to_f32(X_bits).astype(np.float64)
    E0T = synthetic.bf16_to_f32(E_bits).astype(np.float64)
    tX = to_dev_bf16(X_bits, dev)
    XT = torch.empty((N * K,), dtype=torch.bfloat16, device=dev)
    g.gsq_transpose_tokens(1, [0, N], K, tX, XT)
    RT = torch.full((M * N,), float("nan"), dtype=torch.bfloat16, device=dev)
    G = torch.full((M, K), float("nan"), dtype=torch.float32, device=dev)
    ws = torch.empty((g.gsq_recon_workspace_bytes(1, [0, N], M, K) // 4,), dtype=torch.float32,
                     device=dev)
    loss = torch.zeros((1,), dtype=torch.float64, device=dev)
    g.gsq_recon_loss_grad_offset(M, K, N, tX, XT, to_dev_bf16(dW_bits, dev),
                                 to_dev_bf16(E_bits, dev), ws, RT, G, loss)
    torch.cuda.synchronize()
    RT_ref, loss_ref, _ = oracle.recon_loss_grad_offset(X, dW, E0T)
    rel = abs(float(loss.item()) - loss_ref) / loss_ref
    got_rt = bf16_values(RT).astype(np.float64).reshape(M, N)
    # fp32 dot product (worst case (K+2) 2^-24 sum|terms|), one fp32 add of
    # the offset, one rounding to bf16 (half an ulp)
    gam = (K + 2) * 2.0 ** -24 * (np.abs(dW) @ np.abs(X).T) + 2.0 ** -23 * np.abs(RT_ref)
    ok_rt = np.all(np.abs(got_rt - RT_ref) <= 0.5 * bf16_ulp(RT_ref) + gam + 1e-30)
    Ge = 2.0 * got_rt @ X
    bound = (N + 2) * 2.0 ** -24 * (2.0 * np.abs(got_rt) @ np.abs(X))
    Gd = f32(G).astype(np.float64)
    nrm = np.linalg.norm(Gd - Ge) / np.linalg.norm(Ge)
    report(f"recon offset {M}x{N}x{K}", rel_loss=rel, G_normwise=float(nrm))
    assert rel <= 1e-5
    assert ok_rt
    assert np.all(np.abs(Gd - Ge) <= bound + 1e-30)
    assert nrm <= 1e-5


@pytest.mark.parametrize("M,N,K", [
    (512, 256, 512),                  # several tiles
    (300, 192, 384),                  # ragged rows, partial tiles
    (256, 64, 640),                   # few tokens, in-features past two tiles
    (4352, 64, 4096),                 # 17x16 tiles: a row block of whole rounds + a 128-wide tail
])
def test_recon_gram(dev, M, N, K):
    import torch
    import post_weight_quantization_philox_amd as g
    rng = np.random.default_rng(7 * M + N + K)
    dW_bits = synthetic.bf16_bits((rng.normal(0, 0.01, (M, K))).astype(np.float32))
    X_bits = synthetic.bf16_bits(rng.normal(0, 1, (N, K)).astype(np.float32))
    dW = synthetic.bf16_to_f32(dW_bits).astype(np.float64)
    X = synthetic.bf16_to_f32(X_bits).astype(np.float64)
    tdW = to_dev_bf16(dW_bits, dev)
    tX = to_dev_bf16(X_bits, dev)
    XT = torch.empty((N * K,), dtype=torch.bfloat16, device=dev)
    g.gsq_transpose_tokens(1, [0, N], K, tX, XT)
    H = torch.empty((K, K), dtype=torch.bfloat16, device=dev)
    g.gsq_gram(N, K, XT, H)
    G = torch.full((M, K), float("nan"), dtype=torch.float32, device=dev)
    ws = torch.empty((g.gsq_recon_gram_workspace_bytes(M, K) // 4,), dtype=torch.float32, device=dev)
    loss = torch.zeros((1,), dtype=torch.float64, device=dev)
    g.gsq_recon_gram(M, K, H, tdW, ws, G, loss)
    torch.cuda.synchronize()
    # H: an fp32 dot product of N terms rounded once to bf16.
    Hh = bf16_values(H).astype(np.float64)
    H_ref = oracle.gram(X)
    gam = (N + 2) * 2.0 ** -24 * (np.abs(X).T @ np.abs(X))
    assert np.all(np.abs(Hh - H_ref) <= 0.5 * bf16_ulp(H_ref) + gam + 1e-30)
    report(f"gram {N}x{K}", asym=float(np.abs(Hh - Hh.T).max()))
    # G and the loss from the GPU's own bf16 H, exact in fp64, against
    # worst-case fp32 accumulation bounds (K terms per product, then at most
    # 300 terms per fp32 partial of the loss).
    l_ref, G_ref = oracle.recon_loss_grad_gram(dW, Hh)
    Gd = f32(G).astype(np.float64)
    bound = (K + 2) * 2.0 ** -24 * 2.0 * (np.abs(dW) @ np.abs(Hh))
    assert np.all(np.abs(Gd - G_ref) <= bound + 1e-30)
    lb = (K + 2) * 2.0 ** -24 * np.sum(np.abs(dW) * (np.abs(dW) @ np.abs(Hh))) \
        + 300 * 2.0 ** -24 * np.sum(np.abs(dW * G_ref / 2))
    got = float(loss.item())
    assert abs(got - l_ref) <= lb
    # Against the direct form's exact objective: the bf16 rounding of H moves
    # the loss by far less than the 2e-3 allowed for a bf16-GEMM loss.
    _, l_exact, G_exact = oracle.recon_loss_grad(X, dW)
    rel = abs(got - l_exact) / l_exact
    nrm = np.linalg.norm(Gd - G_exact) / np.linalg.norm(G_exact)
    report(f"recon gram {M}x{N}x{K}", rel_vs_direct_exact=rel, G_normwise=float(nrm))
    assert rel <= 2e-3
    assert nrm <= 2.0 ** -8


def test_gram_entry_points_reject_bad_shapes(dev):
    import torch
    import post_weight_quantization_philox_amd as g
    XT = torch.zeros((64 * 128,), dtype=torch.bfloat16, device=dev)
    H = torch.zeros((128, 128), dtype=torch.bfloat16, device=dev)
    for tokens, cols in [(63, 128), (64, 100), (0, 128)]:
        with pytest.raises(g.GsqError):
            g.gsq_gram(tokens, cols, XT, H)
    assert g.gsq_recon_gram_workspace_bytes(10, 100) == 0
    ws = torch.zeros((64,), dtype=torch.float32, device=dev)
    G = torch.zeros((4, 128), dtype=torch.float32, device=dev)
    loss = torch.zeros((1,), dtype=torch.float64, device=dev)
    with pytest.raises(g.GsqError):       # workspace too small
        g.gsq_recon_gram(4, 128, H, H, ws, G, loss, workspace_bytes=4)


# ----------------------------------------------------------------------------
# Hardening and packing
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("grid", GRIDS)
def test_harden_pack_bit_exact(dev, grid):
    import torch
    import post_weight_quantization_philox_amd as g
    M, K = 9, 384
    rng = np.random.default_rng(grid + 40)
    L = oracle.N_LOGITS[grid]
    lg = np.round(rng.normal(0, 1, (L, M, K)) * 2) / 2          # coarse: many exact ties
    lg = lg.astype(np.float32)
    lg[:, 0, :8] = 0.0                                           # all-equal logits
    if grid == oracle.GRID_TERNARY:
        lg[0, 1, :4] = -0.0
    c0 = rng.integers(0, 4 if grid == oracle.GRID_INT2 else 8, (M, K)).astype(np.uint8)
    s = (np.abs(rng.normal(0, 0.01, (M, K // 128))) + 1e-4).astype(np.float32)
    s[0, 0] = 1.0 + 2.0 ** -11                                   # fp16 tie
    layer = g.GsqLayer.make(grid, M, K, g.DTYPE_BF16)
    codes = torch.empty((M, K), dtype=torch.uint8, device=dev)
    bits = oracle.CODE_BITS[grid]
    packed = torch.empty((M, K * bits // 32), dtype=torch.int32, device=dev)
    s16 = torch.empty((M, K // 128), dtype=torch.float16, device=dev)
    g.gsq_harden_pack(layer, torch.from_numpy(lg).to(dev), torch.from_numpy(s).to(dev),
                      torch.from_numpy(c0).to(dev), codes, packed, s16)
    torch.cuda.synchronize()
    c_ref, p_ref, s_ref = oracle.harden_pack(lg, s, grid, c0)
    np.testing.assert_array_equal(codes.cpu().numpy(), c_ref)
    np.testing.assert_array_equal(packed.cpu().numpy().view(np.uint32), p_ref)
    np.testing.assert_array_equal(s16.cpu().numpy().view(np.uint16), s_ref)


# ----------------------------------------------------------------------------
# Fused backward + Lion + next forward
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("grid", GRIDS)
@pytest.mark.parametrize("w_bf16", [True, False])
def test_fused_bwd_fwd_equals_separate_calls(dev, grid, w_bf16):
    import torch
    import post_weight_quantization_philox_amd as g
    M, K = 40, 384
    d, W, s, c0, lg = _layer_inputs(grid, M, K, seed=31, w_bf16=w_bf16)
    rng = np.random.default_rng(8)
    L = oracle.N_LOGITS[grid]
    G = (rng.normal(0, 1.0, (M, K)) * 50.0).astype(np.float32)
    mom = (rng.normal(0, 1.0, (L, M, K)) * 1e-2).astype(np.float32)
    smom = (rng.normal(0, 1.0, s.shape) * 1e-3).astype(np.float32)
    lion = g.GsqLion.make(lr_logit=3e-3, lr_scale=1e-4)
    layer = g.GsqLayer.make(grid, M, K, g.DTYPE_BF16 if w_bf16 else g.DTYPE_F32, seed=3, stream=4)
    Wd = _w_dev(d, dev)
    codes = torch.from_numpy(c0).to(dev)
    outs = []
    for fused in (False, True):
        t = [torch.from_numpy(x).to(dev) for x in (lg, mom, s, smom)]
        dW = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
        Gd = torch.from_numpy(G).to(dev)
        if fused:
            g.gsq_relax_bwd_lion_fwd(layer, Gd, *t, codes, Wd, 41, 0.37, 1.0, lion, 42, 0.31, dW)
        else:
            g.gsq_relax_bwd_lion(layer, Gd, *t, codes, 41, 0.37, 1.0, lion)
            g.gsq_relax_fwd(layer, t[0], t[2], codes, Wd, 42, 0.31, 1.0, dW)
        torch.cuda.synchronize()
        outs.append([x.cpu().numpy() for x in t] + [dW.view(torch.int16).cpu().numpy()])
    for a, b in zip(*outs):
        np.testing.assert_array_equal(a, b)
