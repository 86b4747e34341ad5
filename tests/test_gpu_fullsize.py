"""Parity at the full workload sizes, in the launch configuration bench.py
times, on sampled rows the oracle computes one by one (every kernel of the
step is row-local except the two products, whose sampled rows the oracle forms
from the GPU's own bf16 operands), plus properties that hold at any size.
Also: the step is deterministic (two runs from the same state are identical)."""

import time

import numpy as np
import pytest

import oracle
import synthetic
from tests.gpu_util import device, to_dev_bf16, bf16_values, f32, bf16_ulp, report

pytestmark = pytest.mark.gpu

WORKLOADS = ["linear512_int2", "qproj4096_int2", "downproj4096x14336_ternary",
             "gateproj28672x8192_int3local", "gateproj28672x8192_int3full", "moe64x2048x7168_int2"]


def _sample_rows(M, rpe, seed=0):
    rng = np.random.default_rng(seed)
    rows = {0, 1, M // 2, M - 1, rpe - 1, min(rpe, M - 1)}
    rows |= set(int(r) for r in rng.integers(0, M, 4))
    return sorted(rows)


def _log(msg):
    print(f"[fullsize] {msg}", flush=True)


@pytest.mark.parametrize("name", WORKLOADS)
def test_fullsize_sampled_parity(name):
    import torch
    import post_weight_quantization_philox_amd as g
    from post_weight_quantization_philox_amd.solver import LayerSolver
    dev = device()
    t0 = time.time()
    d = synthetic.generate(name, seed=0)
    wl = d["workload"]
    grid = wl.grid
    _log(f"{name}: inputs drawn in {time.time() - t0:.1f} s")
    Wd = to_dev_bf16(d["W_bits"], dev) if d["W_bits"] is not None else torch.from_numpy(d["W"]).to(dev)
    Xd = to_dev_bf16(d["X_bits"], dev)
    E = wl.experts
    rpe = wl.rows_per_expert or wl.rows
    lion = g.GsqLion.make(lr_logit=wl.lr_logit, lr_scale=1e-5)
    sol = LayerSolver(Wd, Xd, grid, tok_offsets=d["tok_offsets"], rows_per_expert=rpe, seed=0,
                      stream_id=0, lion=lion)
    M, K = sol.rows, sol.cols
    L = oracle.N_LOGITS[grid]
    rows = _sample_rows(M, rpe)
    W = d["W"]
    X = d["X"].astype(np.float64)
    offs = [int(o) for o in d["tok_offsets"]]          # unpadded
    poffs = [int(o) for o in sol.tok_offsets]          # padded to 64 on the device

    # --- warm start: bit-exact on sampled rows ---
    torch.cuda.synchronize()
    s_ref, c_ref, l_ref = oracle.init_rtn(W[rows], grid)
    np.testing.assert_array_equal(f32(sol.scales[rows]).view(np.uint32), s_ref.view(np.uint32))
    np.testing.assert_array_equal(sol.codes[rows].cpu().numpy(), c_ref)
    np.testing.assert_array_equal(f32(sol.logits[:, rows]).view(np.uint32), l_ref.view(np.uint32))
    _log(f"{name}: init ok ({M}x{K}, {L} logits)")

    # --- relaxed forward at step 0 ---
    tau, step = 0.5, 0
    w_soft = torch.empty((M, K), dtype=torch.float32, device=dev)
    sol.relax_fwd(step, tau, 1.0, w_soft)
    torch.cuda.synchronize()
    ws_rows = f32(w_soft[rows])
    dW_rows = bf16_values(sol.dW[rows]).astype(np.float64)
    for j, r in enumerate(rows):
        ref = oracle.relax_fwd(l_ref[:, j:j + 1], s_ref[j:j + 1], W[r:r + 1], grid, 0, 0, step, tau,
                               1.0, c_ref[j:j + 1], row0=r)
        nat = np.repeat(s_ref[j:j + 1].astype(np.float64), 128, axis=1) * oracle.Q_MAX[grid]
        assert np.all(np.abs(ws_rows[j] - ref["w_soft"][0]) <= 1e-5 * np.maximum(nat[0], 1e-30))
        assert np.all(np.abs(dW_rows[j] - ref["dW"][0]) <= bf16_ulp(ref["dW"][0]) + 1e-5 * nat[0])
    _log(f"{name}: relax_fwd ok on rows {rows}")

    # --- objective and gradient ---
    sol.recon()
    torch.cuda.synchronize()
    loss = float(sol.loss.item())
    RT = sol.RT
    G_rows = f32(sol.G[rows]).astype(np.float64)
    exact_rows_loss = gpu_rows_loss = 0.0
    for j, r in enumerate(rows):
        e = r // rpe
        n, pn = offs[e + 1] - offs[e], poffs[e + 1] - poffs[e]
        Xe = X[offs[e]:offs[e + 1]]
        base = rpe * poffs[e] + (r - e * rpe) * pn
        rt = bf16_values(RT[base:base + pn]).astype(np.float64)
        assert not rt[n:].any()                      # padded tokens contribute zero
        rt = rt[:n]
        rt_ref = Xe @ dW_rows[j]                     # exact from the GPU's bf16 operands
        gam = (K + 2) * 2.0 ** -24 * (np.abs(Xe) @ np.abs(dW_rows[j]))
        assert np.all(np.abs(rt - rt_ref) <= 0.5 * bf16_ulp(rt_ref) + gam + 1e-30)
        g_ref = 2.0 * rt @ Xe
        gb = (n + 2) * 2.0 ** -24 * 2.0 * (np.abs(rt) @ np.abs(Xe))
        assert np.all(np.abs(G_rows[j] - g_ref) <= gb + 1e-30)
        ref = oracle.relax_fwd(l_ref[:, j:j + 1], s_ref[j:j + 1], W[r:r + 1], grid, 0, 0, step, tau,
                               1.0, c_ref[j:j + 1], row0=r)
        exact_rows_loss += float(np.sum((Xe @ ref["dW"][0]) ** 2))
        gpu_rows_loss += float(np.sum(rt_ref ** 2))
    # exact-mode loss of the sampled rows (unrounded fp64 dW) against the
    # rows' loss from the GPU's bf16 dW: the rounding may move it by <= 2e-3.
    rel_exact = abs(gpu_rows_loss - exact_rows_loss) / exact_rows_loss
    # whole-layer property: the loss equals the sum of squares of R^T up to
    # R^T's bf16 rounding (the loss is taken before it).
    rt_all = bf16_values(RT).astype(np.float64)
    rel_rt = abs(float(np.sum(rt_all * rt_all)) - loss) / loss
    report(f"{name} recon", loss=loss, rel_vs_exact_rows=rel_exact, rel_vs_sum_RT2=rel_rt)
    assert rel_exact <= 2e-3
    assert rel_rt <= 1e-3
    del rt_all
    _log(f"{name}: recon ok")

    # --- backward + Lion on a copy (debug gradients), then the fused pass ---
    Gh = G_rows
    keep = [x.clone() for x in (sol.logits, sol.mom, sol.scales, sol.scale_mom)]
    gl = torch.empty_like(sol.logits)
    gs = torch.empty_like(sol.scales)
    g.gsq_relax_bwd_lion(sol.layer, sol.G, keep[0], keep[1], keep[2], keep[3], sol.init_codes,
                         step, tau, 1.0, lion, gl, gs)
    torch.cuda.synchronize()
    gl_rows = f32(gl[:, rows])
    gs_rows = f32(gs[rows])
    per_coord = []
    for j, r in enumerate(rows):
        glr, gsr = oracle.relax_bwd(Gh[j:j + 1], l_ref[:, j:j + 1], s_ref[j:j + 1], grid, 0, 0, step,
                                    tau, 1.0, c_ref[j:j + 1], row0=r)
        nat = np.abs(Gh[j]) * np.repeat(s_ref[j].astype(np.float64), 128) * oracle.Q_MAX[grid] / tau
        assert np.all(np.abs(gl_rows[:, j] - glr[:, 0]) <= 1e-5 * nat[None] + 1e-30)
        cmax = np.abs(glr[:, 0]).max(axis=0)
        live = cmax >= 1e-3 * nat
        per_coord.append((np.abs(gl_rows[:, j] - glr[:, 0]).max(axis=0) / np.maximum(cmax, 1e-300))[live])
        f = oracle.relax_fwd(l_ref[:, j:j + 1], s_ref[j:j + 1], W[r:r + 1], grid, 0, 0, step, tau, 1.0,
                             c_ref[j:j + 1], row0=r)
        mass = (np.abs(Gh[j]) * np.abs(f["w_hat"][0])).reshape(-1, 128).sum(1)
        gabs = np.abs(Gh[j]).reshape(-1, 128).sum(1)
        assert np.all(np.abs(gs_rows[j] - gsr[0]) <= 130 * 2.0 ** -24 * mass + 1e-5 * oracle.Q_MAX[grid] * gabs)
    pc = np.concatenate(per_coord)
    report(f"{name} logit gradient per coordinate (|grad| >= 1e-3 of natural scale)",
           max_rel=float(pc.max()), p999=float(np.quantile(pc, 0.999)), median=float(np.median(pc)),
           within_1e5=float(np.mean(pc <= 1e-5)))
    th, _ = oracle.lion(l_ref, gl_rows, np.zeros_like(l_ref), wl.lr_logit, 0.9, 0.99)
    np.testing.assert_array_equal(f32(keep[0][:, rows]).view(np.uint32), th.view(np.uint32))
    _log(f"{name}: relax_bwd_lion ok")
    # the fused pass equals backward + Lion followed by the next forward
    dW_sep = torch.empty_like(sol.dW)
    g.gsq_relax_fwd(sol.layer, keep[0], keep[2], sol.init_codes, sol.W, step + 1, 0.45, 1.0, dW_sep)
    sol.relax_bwd_lion_fwd(step, tau, step + 1, 0.45)
    torch.cuda.synchronize()
    for a, b in zip((sol.logits, sol.mom, sol.scales, sol.scale_mom, sol.dW),
                    (keep[0], keep[1], keep[2], keep[3], dW_sep)):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b)
    _log(f"{name}: fused pass bit-identical")

    # --- harden + pack on sampled rows ---
    codes, packed, s16 = sol.harden()
    torch.cuda.synchronize()
    lg_rows = f32(sol.logits[:, rows])
    c0_rows = sol.codes[rows].cpu().numpy()
    cr, pr, sr = oracle.harden_pack(lg_rows, f32(sol.scales[rows]), grid, c0_rows)
    np.testing.assert_array_equal(codes[rows].cpu().numpy(), cr)
    np.testing.assert_array_equal(packed[rows].cpu().numpy().view(np.uint32), pr)
    np.testing.assert_array_equal(s16[rows].cpu().numpy().view(np.uint16), sr)
    _log(f"{name}: harden_pack ok; {time.time() - t0:.1f} s total")


def test_step_is_deterministic():
    import torch
    import post_weight_quantization_philox_amd as g
    from post_weight_quantization_philox_amd.solver import LayerSolver
    dev = device()
    d = synthetic.generate("qproj4096_int2", seed=0)
    Wd = to_dev_bf16(d["W_bits"], dev)
    Xd = to_dev_bf16(d["X_bits"], dev)
    results = []
    for _ in range(2):
        sol = LayerSolver(Wd, Xd, g.GRID_INT2, seed=3, stream_id=2)
        sol.relax_fwd(0, 1.0)
        for t in range(3):
            sol.step_fused(t, 1.0 - 0.1 * t, 0.9 - 0.1 * t)
        torch.cuda.synchronize()
        results.append([sol.logits.clone(), sol.mom.clone(), sol.scales.clone(), sol.G.clone(),
                        sol.dW.view(torch.int16).clone(), sol.loss.clone()])
        del sol
    for a, b in zip(*results):
        assert torch.equal(a, b)


@pytest.mark.parametrize("name", ["qproj4096_int2", "gateproj28672x8192_int3local"])
def test_fullsize_gram(name):
    """The Gram-form objective at full size: sampled rows of H = X^T X and of
    G = 2 dW H from the GPU's own bf16 operands, and the loss against the
    direct form's GPU loss on the same dW."""
    import torch
    from post_weight_quantization_philox_amd.solver import LayerSolver
    dev = device()
    d = synthetic.generate(name, seed=0)
    wl = d["workload"]
    Wd = to_dev_bf16(d["W_bits"], dev)
    Xd = to_dev_bf16(d["X_bits"], dev)
    X = d["X"].astype(np.float64)
    N = X.shape[0]
    sol = LayerSolver(Wd, Xd, wl.grid, seed=0, stream_id=0, recon="gram")
    M, K = sol.rows, sol.cols
    sol.relax_fwd(0, 0.5)
    sol.recon()
    torch.cuda.synchronize()
    loss_gram = float(sol.loss.item())
    rng = np.random.default_rng(1)
    hrows = sorted({0, K - 1, *(int(r) for r in rng.integers(0, K, 6))})
    H_rows = bf16_values(sol.H[hrows]).astype(np.float64)
    for j, r in enumerate(hrows):
        ref = X.T @ X[:, r]
        gam = (N + 2) * 2.0 ** -24 * (np.abs(X).T @ np.abs(X[:, r]))
        assert np.all(np.abs(H_rows[j] - ref) <= 0.5 * bf16_ulp(ref) + gam + 1e-30)
    _log(f"{name}: gram rows {hrows} ok")
    H = bf16_values(sol.H).astype(np.float64)
    rows = _sample_rows(M, M)
    dW_rows = bf16_values(sol.dW[rows]).astype(np.float64)
    G_rows = f32(sol.G[rows]).astype(np.float64)
    P = dW_rows @ H
    bound = (K + 2) * 2.0 ** -24 * 2.0 * (np.abs(dW_rows) @ np.abs(H))
    assert np.all(np.abs(G_rows - 2.0 * P) <= bound + 1e-30)
    del H
    _log(f"{name}: gram G rows {rows} ok")
    # The direct form on the same dW (GPU): the two roundings of the same
    # objective stay within 2e-3 of the exact value each.
    dsol = LayerSolver(Wd, Xd, wl.grid, seed=0, stream_id=0)
    dsol.dW.copy_(sol.dW)
    dsol.recon()
    torch.cuda.synchronize()
    loss_direct = float(dsol.loss.item())
    rel = abs(loss_gram - loss_direct) / loss_direct
    report(f"{name} gram", loss_gram=loss_gram, loss_direct=loss_direct, rel=rel)
    assert rel <= 4e-3


def test_beyond_32bit_offsets():
    """A 2-bit layer of 33000 x 32768 (1.08e9 coordinates, past 2^30): the
    relax kernels switch to 64-bit element offsets, and the Philox counters
    of the last rows pass 2^32 (stream element i*L). The relaxed forward and
    the fused backward + Lion + next forward on sampled rows against the
    oracle. Inputs are drawn on the device from a seeded generator; the
    sampled rows are copied back."""
    import torch
    import post_weight_quantization_philox_amd as g
    dev = device()
    grid, L = oracle.GRID_INT2, 4
    M, K = 33000, 32768
    assert M * K > 2 ** 30 and (M - 1) * K * L > 2 ** 32
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    W = (torch.randn((M, K), generator=gen, device=dev) * 0.02).to(torch.bfloat16)
    layer = g.GsqLayer.make(grid, M, K, g.DTYPE_BF16, seed=5, stream=1)
    scales = torch.empty((M, K // 128), dtype=torch.float32, device=dev)
    codes = torch.empty((M, K), dtype=torch.uint8, device=dev)
    logits = torch.empty((L, M, K), dtype=torch.float32, device=dev)
    g.gsq_init_rtn(layer, W, scales, codes, logits, 2.0)
    logits.add_(torch.randn((L, M, K), generator=gen, device=dev))
    rows = [0, 16383, 32767, 32768, M - 1]
    Wr = bf16_values(W[rows]).astype(np.float32)
    l0 = f32(logits[:, rows])
    s0 = f32(scales[rows])
    dW = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    g.gsq_relax_fwd(layer, logits, scales, None, W, 3, 0.5, 1.0, dW)
    torch.cuda.synchronize()
    dWr = bf16_values(dW[rows]).astype(np.float64)
    for j, r in enumerate(rows):
        ref = oracle.relax_fwd(l0[:, j:j + 1], s0[j:j + 1], Wr[j:j + 1], grid, 5, 1, 3, 0.5, 1.0,
                               row0=r)
        nat = np.repeat(s0[j].astype(np.float64), 128) * 3
        assert np.all(np.abs(dWr[j] - ref["dW"][0]) <= bf16_ulp(ref["dW"][0]) + 1e-5 * nat)
    _log("beyond 2^30: relax_fwd ok")
    del dW
    G = torch.randn((M, K), generator=gen, device=dev) * 1e3
    mom = torch.zeros((L, M, K), dtype=torch.float32, device=dev)
    smom = torch.zeros((M, K // 128), dtype=torch.float32, device=dev)
    Gr = f32(G[rows]).astype(np.float64)
    lion = g.GsqLion.make(lr_logit=1e-3, lr_scale=1e-5)
    dW2 = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    g.gsq_relax_bwd_lion_fwd(layer, G, logits, mom, scales, smom, None, W, 3, 0.5, 1.0, lion, 4,
                             0.45, dW2)
    torch.cuda.synchronize()
    l1, s1 = f32(logits[:, rows]), f32(scales[rows])
    dW2r = bf16_values(dW2[rows]).astype(np.float64)
    for j, r in enumerate(rows):
        gl, gs = oracle.relax_bwd(Gr[j:j + 1], l0[:, j:j + 1], s0[j:j + 1], grid, 5, 1, 3, 0.5, 1.0,
                                  row0=r)
        th, mm = oracle.lion(l0[:, j:j + 1], gl, np.zeros_like(l0[:, j:j + 1]), 1e-3, 0.9, 0.99)
        nat = np.abs(Gr[j]) * np.repeat(s0[j].astype(np.float64), 128) * 3 / 0.5
        # Lion's sign may differ only where the gradient is within its tolerance of 0
        differ = l1[:, j] != th[:, 0]
        assert np.all(np.abs(gl[:, 0][differ]) <= 1e-5 * np.broadcast_to(nat, gl[:, 0].shape)[differ])
        assert differ.mean() < 1e-3
        ref = oracle.relax_fwd(l1[:, j:j + 1], s1[j:j + 1], Wr[j:j + 1], grid, 5, 1, 4, 0.45, 1.0,
                               row0=r)
        nat2 = np.repeat(s1[j].astype(np.float64), 128) * 3
        assert np.all(np.abs(dW2r[j] - ref["dW"][0]) <= bf16_ulp(ref["dW"][0]) + 1e-5 * nat2)
        gsum_tol = 130 * 2.0 ** -24 * (np.abs(Gr[j]) * 3).reshape(-1, 128).sum(1) + 1e-30
        sn, _ = oracle.lion(s0[j:j + 1], gs, np.zeros_like(s0[j:j + 1]), 1e-5, 0.9, 0.99)
        flips = s1[j] != sn[0]
        assert np.all(np.abs(gs[0][flips]) <= gsum_tol[flips])
    _log("beyond 2^30: fused backward + Lion + next forward ok")


def _trajectory_rows(sol, d, rows, x_of_row, gpu_row_loss, T, lr_logit, lr_scale, sid,
                     init_logit, label, t0, loss_bar=2e-3, groups=None):
    """Run ``T`` annealed steps of ``sol`` (objective, then fused backward +
    Lion + next forward, at the solver's own temperatures) and compare the
    sampled ``rows`` with the oracle's step loop at the oracle's temperatures,
    teacher-forced and free-running. ``x_of_row(r)`` is the calibration block
    row r sees; ``gpu_row_loss()`` reads the sampled rows' losses from the
    GPU's bf16 R^T after a step."""
    from post_weight_quantization_philox_amd.solver import tau_schedule
    grid = d["workload"].grid
    gpu_taus = tau_schedule(T, 1.0, 0.05)
    taus = oracle.tau_schedule(T, 1.0, 0.05)

    def snap():
        return (f32(sol.logits[:, rows]), f32(sol.mom[:, rows]), f32(sol.scales[rows]),
                f32(sol.scale_mom[rows]))

    sol.relax_fwd(0, gpu_taus[0])
    gpu = np.zeros((T, len(rows)))
    states = [snap()]
    for t in range(T):
        sol.step_fused(t, gpu_taus[t], gpu_taus[t + 1] if t + 1 < T else None)
        gpu[t] = gpu_row_loss()
        states.append(snap())
    codes = sol.harden()[0][rows].cpu().numpy()
    _log(f"{label}: {T} GPU steps done; oracle on rows {rows}")
    W = d["W"]
    s, c0, lg = oracle.init_rtn(W[rows], grid, init_logit=init_logit)
    ref = np.zeros_like(gpu)
    c_ref = np.zeros_like(codes)
    rows_state = []
    for j, r in enumerate(rows):
        st = {"logits": lg[:, j:j + 1].copy(), "mom": np.zeros_like(lg[:, j:j + 1]),
              "scales": s[j:j + 1].copy(), "scale_mom": np.zeros_like(s[j:j + 1]),
              "codes": c0[j:j + 1]}
        for t in range(T):
            ref[t, j] = oracle.step(st, W[r:r + 1], x_of_row(r), grid, t, float(taus[t]), 0, sid,
                                    lr_logit, lr_scale, bf16_dW=True, bf16_RT=True, row0=r)
        c_ref[j] = oracle.harden(st["logits"], grid, c0[j:j + 1])[0]
        rows_state.append(st["logits"][:, 0])
    # Teacher-forced: the oracle's step t from the GPU's own state before it,
    # against the GPU's state after it. Lion moves a logit by exactly lr, so
    # a logit differs only where the two took a different sign decision.
    flips, sflips, mom_err = np.zeros(T), np.zeros(T), 0.0
    for t in range(T):
        lg0, m0, s0, sm0 = states[t]
        lg1, m1, s1, sm1 = states[t + 1]
        for j, r in enumerate(rows):
            st = {"logits": lg0[:, j:j + 1].copy(), "mom": m0[:, j:j + 1].copy(),
                  "scales": s0[j:j + 1].copy(), "scale_mom": sm0[j:j + 1].copy(),
                  "codes": c0[j:j + 1]}
            oracle.step(st, W[r:r + 1], x_of_row(r), grid, t, float(taus[t]), 0, sid, lr_logit,
                        lr_scale, bf16_dW=True, bf16_RT=True, row0=r)
            flips[t] += np.count_nonzero(st["logits"][:, 0] != lg1[:, j])
            sflips[t] += np.count_nonzero(st["scales"][0] != s1[j])
            same = st["logits"][:, 0] == lg1[:, j]
            scale_m = max(np.abs(m0[:, j]).max(), np.abs(st["mom"][:, 0]).max()) + 1e-30
            mom_err = max(mom_err, float(np.abs(st["mom"][:, 0] - m1[:, j])[same].max(initial=0.0))
                          / scale_m)
    flips /= lg1[:, 0].size * len(rows)
    sflips /= s1[0].size * len(rows)
    # Free-running: the loss-curve bar applies to the sampled rows' total, as
    # it does to a whole layer's loss. A single row's loss moves more: once
    # Lion's sign has gone the other way on a coordinate where c was within
    # rounding of zero (either way is correct), that logit and its momentum
    # differ from then on, and the effect on the row changes with every
    # step's noise (measured: up to 5e-3 on single rows, below 1e-3 on the
    # total).
    rel_rows = np.abs(gpu - ref) / ref
    rel = np.abs(gpu.sum(axis=1) - ref.sum(axis=1)) / ref.sum(axis=1)
    same_logits = float(np.mean(f32(sol.logits[:, rows]) == np.stack(rows_state, axis=1)))
    agree = float(np.mean(codes == c_ref))
    moved = float(np.mean(c_ref != c0))
    for name, idx in (groups or {}).items():
        ge, gr = gpu[:, idx].sum(axis=1), ref[:, idx].sum(axis=1)
        report(f"  {name}", max_rel_loss=float((np.abs(ge - gr) / gr).max()),
               max_rel_single_row=float(rel_rows[:, idx].max()),
               step_of_max=int(np.argmax(np.abs(ge - gr) / gr)))
    print("[parity]   per-step rel of the total: " + " ".join(f"{v:.1e}" for v in rel), flush=True)
    report(f"{label} trajectory on sampled rows", max_rel_loss=float(rel.max()),
           max_rel_single_row=float(rel_rows.max()), logits_identical=same_logits,
           code_agreement=agree, codes_moved_from_init=moved, max_logit_flips=float(flips.max()),
           max_scale_flips=float(sflips.max()), mom_err=mom_err, seconds=time.time() - t0)
    # Every step matches the oracle up to sign decisions on c within rounding
    # of zero, which are counted and must stay below 1e-4 of the parameters.
    assert flips.max() <= 1e-4 and sflips.max() <= 1e-4
    assert rel.max() <= loss_bar
    # Over the free-running steps those decisions compound (each leaves a
    # logit 2 lr away from the oracle's, and later steps follow from there),
    # most on the ternary layer, whose logits start near the threshold where
    # a code changes.
    assert agree >= 0.995
    assert moved > 0.001


# Warm-start logit and logit learning rate chosen so that hard codes move
# within the steps: a ternary code changes only when a logit crosses 0, so
# the ternary layer starts nearer to it.
@pytest.mark.parametrize("name,init_logit,lr_logit", [("qproj4096_int2", 2.0, 5e-2),
                                                      ("downproj4096x14336_ternary", 0.5, 5e-2),
                                                      ("gateproj28672x8192_int3local", 2.0, 5e-2)])
def test_fullsize_trajectory_sampled_rows(name, init_logit, lr_logit):
    """An annealed solve of the whole layer in the launch configuration the
    bench times (objective, then fused backward + Lion + next forward)
    against the oracle's step loop on sampled rows. Rows are independent in
    the objective (R[:, r] = X dW[r]^T, G[r] = 2 R[:, r]^T X) and each row's
    noise counters follow its place in the layer, so the oracle runs every
    sampled row on its own. Compared: every step teacher-forced (the oracle's
    step from the GPU's state before it against the GPU's state after it),
    and the free-running curves: the sampled rows' loss at every step (the
    GPU's from its bf16 R^T) and the final hard codes."""
    import torch
    import post_weight_quantization_philox_amd as g
    from post_weight_quantization_philox_amd.solver import LayerSolver
    dev = device()
    t0 = time.time()
    d = synthetic.generate(name, seed=0)
    grid = d["workload"].grid
    T, lr_scale, sid = 24, 1e-5, 3
    sol = LayerSolver(to_dev_bf16(d["W_bits"], dev), to_dev_bf16(d["X_bits"], dev), grid, seed=0,
                      stream_id=sid, lion=g.GsqLion.make(lr_logit=lr_logit, lr_scale=lr_scale),
                      init_logit=init_logit)
    M, N = sol.rows, sol.tokens
    rows = _sample_rows(M, M)
    RT = sol.RT.view(M, N)
    X = d["X"].astype(np.float64)

    def gpu_row_loss():
        rt = bf16_values(RT[rows]).astype(np.float64)
        return (rt * rt).sum(axis=1)

    _trajectory_rows(sol, d, rows, lambda r: X, gpu_row_loss, T, lr_logit, lr_scale, sid,
                     init_logit, name, t0)


def test_fullsize_expert_batch_trajectory_sampled_rows():
    """The same annealed comparison on the 64-expert batch (64 x 2048x7168,
    2-bit, routed token counts Zipf(1.1) on [64, 1024]) in the launch
    configuration the bench times (grouped products, fused pass over all
    experts), on sampled rows of the first expert, the last expert and the
    expert with the most tokens. A row of expert e sees only e's tokens."""
    import torch
    import post_weight_quantization_philox_amd as g
    from post_weight_quantization_philox_amd.solver import LayerSolver
    dev = device()
    t0 = time.time()
    name = "moe64x2048x7168_int2"
    d = synthetic.generate(name, seed=0)
    wl = d["workload"]
    E, rpe = wl.experts, wl.rows_per_expert
    T, lr_logit, lr_scale, sid = 24, 5e-2, 1e-5, 3
    offs = [int(o) for o in d["tok_offsets"]]
    counts = np.diff(offs)
    experts = sorted({0, E - 1, int(np.argmax(counts))})
    _log(f"{name}: inputs drawn in {time.time() - t0:.1f} s; experts {experts} with "
         f"{[int(counts[e]) for e in experts]} tokens")
    sol = LayerSolver(to_dev_bf16(d["W_bits"], dev), to_dev_bf16(d["X_bits"], dev), wl.grid,
                      tok_offsets=offs, rows_per_expert=rpe, seed=0, stream_id=sid,
                      lion=g.GsqLion.make(lr_logit=lr_logit, lr_scale=lr_scale))
    poffs = [int(o) for o in sol.tok_offsets]          # padded to 64 on the device
    # 48 rows per expert: a few hundred tokens make each row's loss move more
    # with every legitimate sign difference than a 4096-token row's, so the
    # free-running total needs more rows to stand for the experts' loss.
    rng = np.random.default_rng(1)
    rows = sorted({e * rpe + int(i) for e in experts
                   for i in [0, 1, rpe // 2, rpe - 1, *rng.choice(rpe, 44, replace=False)]})
    X = d["X"].astype(np.float64)
    x_blocks = {e: X[offs[e]:offs[e + 1]] for e in experts}

    def gpu_row_loss():
        out = np.zeros(len(rows))
        for j, r in enumerate(rows):
            e, i = divmod(r, rpe)
            n = poffs[e + 1] - poffs[e]
            blk = sol.RT[rpe * poffs[e]: rpe * poffs[e + 1]].view(rpe, n)
            rt = bf16_values(blk[i]).astype(np.float64)
            out[j] = float((rt * rt).sum())
        return out

    groups = {f"expert {e} ({int(counts[e])} tokens)": [j for j, r in enumerate(rows) if r // rpe == e]
              for e in experts}
    _trajectory_rows(sol, d, rows, lambda r: x_blocks[r // rpe], gpu_row_loss, T, lr_logit,
                     lr_scale, sid, 2.0, name, t0, groups=groups)
