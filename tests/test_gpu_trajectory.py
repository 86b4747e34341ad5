"""End-to-end parity of the annealed solve: the GPU solver (fused backward +
next forward) against the oracle's own step loop on the same seeded layer,
with the oracle rounding dW and R^T to bf16 where the GPU's matrix cores
consume them. Parity is defined on the loss curve and the final hard codes:
Lion's sign can legitimately differ where c is within rounding of zero, and
such a difference then persists, so elementwise equality of the state is not
required."""

import numpy as np
import pytest

import oracle
import synthetic
from tests.gpu_util import device, to_dev_bf16, report

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("grid", [oracle.GRID_INT2, oracle.GRID_TERNARY, oracle.GRID_INT3_LOCAL,
                                  oracle.GRID_INT3])
def test_trajectory_matches_oracle(grid):
    import torch
    import post_weight_quantization_philox_amd as g
    from post_weight_quantization_philox_amd.solver import LayerSolver
    dev = device()
    M, K, N, T = 256, 512, 256, 24
    d = synthetic.small_layer(M, K, N, seed=1, w_bf16=True)
    lr_logit, lr_scale = 1e-1, 1e-5      # large enough that hard codes move in T steps
    solver = LayerSolver(to_dev_bf16(d["W_bits"], dev), to_dev_bf16(d["X_bits"], dev), grid,
                         seed=0, stream_id=5, lion=g.GsqLion.make(lr_logit=lr_logit, lr_scale=lr_scale))
    # The GPU side runs the solver's own annealing schedule, the oracle its own.
    gpu_losses, (codes, packed, s16) = solver.solve(T, 1.0, 0.1, log_every=1)
    taus = oracle.tau_schedule(T, 1.0, 0.1)

    s, c0, lg = oracle.init_rtn(d["W"], grid)
    state = {"logits": lg, "mom": np.zeros_like(lg), "scales": s, "scale_mom": np.zeros_like(s),
             "codes": c0}
    ref_losses = [oracle.step(state, d["W"], d["X"], grid, t, float(taus[t]), 0, 5, lr_logit, lr_scale,
                              bf16_dW=True, bf16_RT=True) for t in range(T)]
    c_ref = oracle.harden(state["logits"], grid, c0)
    rel = np.abs(np.array(gpu_losses) - ref_losses) / np.array(ref_losses)
    agree = np.mean(codes.cpu().numpy() == c_ref)
    same_logits = np.mean(solver.logits.cpu().numpy() == state["logits"])
    moved = np.mean(c_ref != c0)
    report(f"trajectory grid={grid}", max_rel_loss=float(rel.max()), code_agreement=float(agree),
           logits_identical=float(same_logits), codes_moved_from_init=float(moved))
    assert rel.max() <= 2e-3
    assert agree >= 0.999
    assert moved > 0.001              # the comparison covers codes that changed


def test_gram_mode_trajectory_matches_oracle():
    """The Gram-form solve (H = X^T X once, one product per step) against the
    oracle's Gram-form step loop with H rounded to bf16 as the GPU stores it,
    and against the direct-form GPU solve."""
    import torch
    import post_weight_quantization_philox_amd as g
    from post_weight_quantization_philox_amd.solver import LayerSolver
    dev = device()
    grid = oracle.GRID_INT2
    M, K, N, T = 256, 512, 512, 24
    d = synthetic.small_layer(M, K, N, seed=2, w_bf16=True)
    lr_logit, lr_scale = 1e-1, 1e-5
    runs = {}
    for mode in ("gram", "direct"):
        solver = LayerSolver(to_dev_bf16(d["W_bits"], dev), to_dev_bf16(d["X_bits"], dev), grid,
                             seed=0, stream_id=6, recon=mode,
                             lion=g.GsqLion.make(lr_logit=lr_logit, lr_scale=lr_scale))
        losses, hard = solver.solve(T, 1.0, 0.1, log_every=1)
        runs[mode] = (np.array(losses), hard[0].cpu().numpy())
    taus = oracle.tau_schedule(T, 1.0, 0.1)
    s, c0, lg = oracle.init_rtn(d["W"], grid)
    state = {"logits": lg, "mom": np.zeros_like(lg), "scales": s, "scale_mom": np.zeros_like(s),
             "codes": c0}
    H = oracle.gram(d["X"], bf16=True)
    ref = np.array([oracle.step(state, d["W"], None, grid, t, float(taus[t]), 0, 6, lr_logit, lr_scale,
                                bf16_dW=True, H=H) for t in range(T)])
    c_ref = oracle.harden(state["logits"], grid, c0)
    rel = np.abs(runs["gram"][0] - ref) / ref
    rel_modes = np.abs(runs["gram"][0] - runs["direct"][0]) / runs["direct"][0]
    agree = np.mean(runs["gram"][1] == c_ref)
    agree_modes = np.mean(runs["gram"][1] == runs["direct"][1])
    moved = np.mean(c_ref != c0)
    report("trajectory gram", max_rel_loss=float(rel.max()), max_rel_vs_direct=float(rel_modes.max()),
           code_agreement=float(agree), agreement_vs_direct=float(agree_modes),
           codes_moved_from_init=float(moved))
    assert rel.max() <= 2e-3
    # The two forms round different intermediates to bf16 (H here, R^T in the
    # direct form); each stays within 2e-3 of the exact objective, so they
    # stay within 4e-3 of each other, and Lion's sign then differs on a few
    # coordinates.
    assert rel_modes.max() <= 4e-3
    assert agree >= 0.999
    assert agree_modes >= 0.99
    assert moved > 0.001


def test_local_shift_coverage_of_the_full_grid():
    """How often the full 3-bit grid (8 logits) ends within +-2 of the
    warm-start code, the window local shift searches, after a whole annealed
    solve (200 steps, tau 1 -> 0.05) on a synthetic layer; and the hard
    reconstruction error of both against the round-to-nearest start (the
    pages report the +-2 window holding almost every full-grid choice on real
    layers, agihunt.info method paragraph). Logit lr 5e-2 so that codes move
    within 200 steps; scale lr 1e-6: Lion moves a scale by lr every step
    whatever its size, and the 3-bit scales (absmax / 7, about 0.007 here)
    drift too far at 1e-5."""
    import torch
    import post_weight_quantization_philox_amd as g
    from post_weight_quantization_philox_amd.solver import LayerSolver
    dev = device()
    M, K, N, T = 512, 1024, 1024, 200
    d = synthetic.small_layer(M, K, N, seed=4, w_bf16=True)
    W, X = d["W"], d["X"]
    s0, c0, _ = oracle.init_rtn(W, oracle.GRID_INT3)
    rtn = oracle.hard_loss(c0, s0, W, X, oracle.GRID_INT3)
    out = {}
    for grid in (oracle.GRID_INT3, oracle.GRID_INT3_LOCAL):
        sol = LayerSolver(to_dev_bf16(d["W_bits"], dev), to_dev_bf16(d["X_bits"], dev), grid,
                          seed=0, stream_id=9, lion=g.GsqLion.make(lr_logit=5e-2, lr_scale=1e-6))
        _, (codes, _, _) = sol.solve(T, 1.0, 0.05)
        codes = codes.cpu().numpy()
        scales = sol.scales.cpu().numpy()
        out[grid] = (codes, oracle.hard_loss(codes, scales, W, X, grid))
    full = out[oracle.GRID_INT3][0].astype(np.int64)
    within = np.mean(np.abs(full - c0.astype(np.int64)) <= 2)
    moved = np.mean(full != c0)
    report("local-shift coverage", within_pm2=float(within), full_grid_moved=float(moved),
           hard_loss_rtn=rtn, hard_loss_full=out[oracle.GRID_INT3][1],
           hard_loss_local=out[oracle.GRID_INT3_LOCAL][1])
    assert moved > 0.01                  # the solve moved codes, so the window is exercised
    assert within >= 0.99
    assert out[oracle.GRID_INT3][1] < rtn and out[oracle.GRID_INT3_LOCAL][1] < rtn


def test_trajectory_from_gptq_start():
    """GSQ started from the GPU's GPTQ warm start, against the oracle's step
    loop started from the same state (codes, scales and logits copied)."""
    import torch
    import post_weight_quantization_philox_amd as g
    from post_weight_quantization_philox_amd.solver import LayerSolver
    dev = device()
    grid = oracle.GRID_INT3_LOCAL
    M, K, N, T = 256, 512, 512, 24
    d = synthetic.small_layer(M, K, N, seed=3, w_bf16=True)
    lr_logit, lr_scale = 5e-2, 1e-6
    solver = LayerSolver(to_dev_bf16(d["W_bits"], dev), to_dev_bf16(d["X_bits"], dev), grid,
                         seed=0, stream_id=4, init="gptq",
                         lion=g.GsqLion.make(lr_logit=lr_logit, lr_scale=lr_scale))
    torch.cuda.synchronize()
    assert int(solver.gptq_info.item()) == 0
    c0 = solver.codes.cpu().numpy()
    state = {"logits": solver.logits.cpu().numpy(), "mom": np.zeros((5, M, K), np.float32),
             "scales": solver.scales.cpu().numpy(), "scale_mom": np.zeros((M, K // 128), np.float32),
             "codes": c0}
    gpu_losses, hard = solver.solve(T, 1.0, 0.1, log_every=1)
    codes = hard[0].cpu().numpy()
    taus = oracle.tau_schedule(T, 1.0, 0.1)
    ref = [oracle.step(state, d["W"], d["X"], grid, t, float(taus[t]), 0, 4, lr_logit, lr_scale,
                       bf16_dW=True, bf16_RT=True) for t in range(T)]
    c_ref = oracle.harden(state["logits"], grid, c0)
    rel = np.abs(np.array(gpu_losses) - ref) / np.array(ref)
    agree = np.mean(codes == c_ref)
    s_rtn, c_rtn, _ = oracle.init_rtn(d["W"], grid)
    report("trajectory from gptq", max_rel_loss=float(rel.max()), code_agreement=float(agree),
           hard_rtn=oracle.hard_loss(c_rtn, s_rtn, d["W"], d["X"], grid),
           hard_gptq=oracle.hard_loss(c0, s_rtn, d["W"], d["X"], grid),
           hard_after=oracle.hard_loss(c_ref, state["scales"], d["W"], d["X"], grid))
    assert rel.max() <= 2e-3
    assert agree >= 0.999


def test_expert_batch_trajectory_matches_oracle():
    """An annealed solve of an expert batch (grouped products; one expert
    without tokens, one whose tokens the solver pads to 64) against the
    oracle's step loop run expert by expert, each expert's rows placed at
    their rows in the batch for the noise counters. The batch loss is the sum
    of the experts' losses."""
    import torch
    import post_weight_quantization_philox_amd as g
    from post_weight_quantization_philox_amd.solver import LayerSolver
    dev = device()
    grid = oracle.GRID_INT2
    E, rpe, K, T, sid = 5, 128, 256, 24, 9
    counts = [0, 64, 128, 192, 40]
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    rng = np.random.default_rng(11)
    W_bits = synthetic.bf16_bits(rng.normal(0, 0.02, (E * rpe, K)).astype(np.float32))
    X_bits = synthetic.bf16_bits(rng.normal(0, 1, (int(offs[-1]), K)).astype(np.float32))
    W = synthetic.bf16_to_f32(W_bits)
    X = synthetic.bf16_to_f32(X_bits).astype(np.float64)
    lr_logit, lr_scale = 1e-1, 1e-5
    solver = LayerSolver(to_dev_bf16(W_bits, dev), to_dev_bf16(X_bits, dev), grid, tok_offsets=offs,
                         rows_per_expert=rpe, seed=0, stream_id=sid,
                         lion=g.GsqLion.make(lr_logit=lr_logit, lr_scale=lr_scale))
    gpu_losses, hard = solver.solve(T, 1.0, 0.1, log_every=1)
    codes = hard[0].cpu().numpy()
    taus = oracle.tau_schedule(T, 1.0, 0.1)

    s, c0, lg = oracle.init_rtn(W, grid)
    ref = np.zeros(T)
    c_ref = np.zeros_like(codes)
    for e in range(E):
        r = slice(e * rpe, (e + 1) * rpe)
        st = {"logits": lg[:, r].copy(), "mom": np.zeros_like(lg[:, r]), "scales": s[r].copy(),
              "scale_mom": np.zeros_like(s[r]), "codes": c0[r]}
        Xe = X[offs[e]:offs[e + 1]]
        for t in range(T):
            ref[t] += oracle.step(st, W[r], Xe, grid, t, float(taus[t]), 0, sid, lr_logit, lr_scale,
                                  bf16_dW=True, bf16_RT=True, row0=e * rpe)
        c_ref[r] = oracle.harden(st["logits"], grid, c0[r])
    rel = np.abs(np.array(gpu_losses) - ref) / ref
    agree = float(np.mean(codes == c_ref))
    moved = float(np.mean(c_ref != c0))
    idle = float(np.mean(c_ref[:rpe] != c0[:rpe]))
    report("expert batch trajectory", max_rel_loss=float(rel.max()), code_agreement=agree,
           codes_moved_from_init=moved, moved_without_tokens=idle)
    assert rel.max() <= 2e-3
    assert agree >= 0.999
    assert moved > 0.001
    assert idle == 0.0                # no tokens: zero gradient, Lion leaves the logits alone


@pytest.mark.parametrize("grid", [oracle.GRID_INT2, oracle.GRID_INT3_LOCAL])
def test_resume_from_checkpoint_is_bit_identical(grid, tmp_path):
    """A solve stopped after step 9, checkpointed (logits, momenta, scales,
    scale momenta, warm-start codes) and resumed at step 10 in a fresh solver
    of the same layer ends in exactly the state and hard codes of the
    uninterrupted solve: the noise needs no saved generator state."""
    import torch
    import post_weight_quantization_philox_amd as g
    from post_weight_quantization_philox_amd.solver import LayerSolver
    dev = device()
    d = synthetic.small_layer(256, 512, 128, seed=3, w_bf16=True)
    W, X = to_dev_bf16(d["W_bits"], dev), to_dev_bf16(d["X_bits"], dev)
    make = lambda: LayerSolver(W, X, grid, seed=7, stream_id=2,
                               lion=g.GsqLion.make(lr_logit=5e-2, lr_scale=1e-5))
    T = 20
    whole = make()
    log = tmp_path / "solve.jsonl"
    l_whole, (codes_w, packed_w, s16_w) = whole.solve(T, 1.0, 0.1, log_every=1, log_path=str(log))
    import json
    rows = [json.loads(line) for line in log.read_text().splitlines()]
    assert [r["step"] for r in rows] == list(range(T))
    assert [r["loss"] for r in rows] == l_whole
    assert rows[0]["seed"] == 7 and rows[0]["stream"] == 2 and rows[0]["grid"] == grid
    first = make()
    l_first, hard = first.solve(T, 1.0, 0.1, log_every=1, stop=10)
    assert hard is None
    ckpt = first.state()
    del first
    resumed = make()
    resumed.load_state(ckpt)
    l_rest, (codes_r, packed_r, s16_r) = resumed.solve(T, 1.0, 0.1, log_every=1, start=10)
    assert l_first + l_rest == l_whole
    for k in ("logits", "mom", "scales", "scale_mom"):
        assert torch.equal(getattr(whole, k), getattr(resumed, k)), k
    assert torch.equal(codes_w, codes_r) and torch.equal(packed_w, packed_r)
    assert torch.equal(s16_w.view(torch.int16), s16_r.view(torch.int16))
    with pytest.raises(ValueError):
        resumed.solve(T, 1.0, 0.1, start=T)


def test_non_finite_input_stops_the_solve():
    """A NaN among the calibration activations reaches the objective in the
    first step; the solve raises instead of optimising NaNs. (Activations
    enter only arithmetic, never an index, so a NaN cannot misdirect a memory
    access.)"""
    import torch
    import post_weight_quantization_philox_amd as g
    from post_weight_quantization_philox_amd.solver import LayerSolver
    dev = device()
    d = synthetic.small_layer(256, 256, 64, seed=5, w_bf16=True)
    x_bits = d["X_bits"].copy()
    x_bits[3, 17] = 0x7FC0                  # bf16 quiet NaN
    sol = LayerSolver(to_dev_bf16(d["W_bits"], dev), to_dev_bf16(x_bits, dev), g.GRID_INT2,
                      seed=0, stream_id=0)
    with pytest.raises(FloatingPointError, match="step 0"):
        sol.solve(4, 1.0, 0.1, log_every=1)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("lr_logit", [1e-3, 2e-2])
def test_linear512_annealed_solve_matches_oracle(lr_logit):
    """The single 512x512 layer as specified: W fp32 N(0, 0.02^2), 256
    calibration tokens N(0,1) (bf16 in the products), 2-bit grid {-3,-1,1,3},
    group 128, fp32 logits with +2.0 on the round-to-nearest level, tau
    annealed 1.0 -> 0.05 over 200 Lion steps, Philox seed 0; the GPU solve
    (the solver's own schedule) against the oracle's step loop (the oracle's
    schedule) in bf16-mirror mode. At lr 1e-3 no logit can move by the 2.0
    that separates the warm-start level from the others within 200 steps, so
    the codes stay put and only the scales learn; lr 2e-2 is the same solve
    with codes that move. Pinned besides parity: the hardened layer's
    reconstruction error (fp16 scales) stays below round-to-nearest's."""
    import torch
    import post_weight_quantization_philox_amd as g
    from post_weight_quantization_philox_amd.solver import LayerSolver
    dev = device()
    d = synthetic.generate("linear512_int2", seed=0)
    grid, T, lr_scale = oracle.GRID_INT2, 200, 1e-5
    assert d["W_bits"] is None and d["W"].dtype == np.float32     # fp32 weights
    solver = LayerSolver(torch.from_numpy(d["W"]).to(dev), to_dev_bf16(d["X_bits"], dev), grid,
                         seed=0, stream_id=0, lion=g.GsqLion.make(lr_logit=lr_logit, lr_scale=lr_scale))
    gpu_losses, (codes, packed, s16) = solver.solve(T, 1.0, 0.05, log_every=1)
    codes = codes.cpu().numpy()
    s16 = s16.cpu().numpy().view(np.uint16)
    W, X = d["W"], d["X"].astype(np.float64)
    taus = oracle.tau_schedule(T, 1.0, 0.05)
    s, c0, lg = oracle.init_rtn(W, grid)
    state = {"logits": lg, "mom": np.zeros_like(lg), "scales": s, "scale_mom": np.zeros_like(s),
             "codes": c0}
    ref = np.array([oracle.step(state, W, X, grid, t, float(taus[t]), 0, 0, lr_logit, lr_scale,
                                bf16_dW=True, bf16_RT=True) for t in range(T)])
    c_ref, p_ref, s16_ref = oracle.harden_pack(state["logits"], state["scales"], grid)
    rel = np.abs(np.array(gpu_losses) - ref) / ref
    agree = float(np.mean(codes == c_ref))
    moved = float(np.mean(c_ref != c0))
    f16 = lambda b: b.view(np.float16).astype(np.float64)
    hard_rtn = oracle.hard_loss(c0, f16(oracle.scales_to_f16_bits(s)), W, X, grid)
    hard_gpu = oracle.hard_loss(codes, f16(s16), W, X, grid)
    hard_ref = oracle.hard_loss(c_ref, f16(s16_ref), W, X, grid)
    # How far apart the two final logit vectors are where the codes differ
    # (in units of lr): reported. Lion moves every logit by exactly lr per
    # step, so a sign decision taken differently where c was within rounding
    # of zero (R17) leaves the logits 2 lr apart, and over a long free-running
    # solve the two trajectories of such a coordinate drift apart further.
    lg_gpu = solver.logits.cpu().numpy()
    diff = np.argwhere(codes != c_ref)
    gaps = np.array([max(lg_gpu[codes[i, j], i, j] - lg_gpu[c_ref[i, j], i, j],
                         state["logits"][c_ref[i, j], i, j] - state["logits"][codes[i, j], i, j])
                     for i, j in diff]) if len(diff) else np.zeros(0)
    report(f"512x512 solve lr={lr_logit}", max_rel_loss=float(rel.max()), code_agreement=agree,
           codes_moved_from_init=moved, relaxed_loss_first=float(ref[0]),
           relaxed_loss_last=float(ref[-1]), hard_rtn=hard_rtn, hard_gpu=hard_gpu,
           hard_oracle=hard_ref, scales_f16_equal=float(np.mean(s16 == s16_ref)),
           differing_codes=int(len(diff)),
           max_tie_gap_in_lr=float(gaps.max() / lr_logit) if len(gaps) else 0.0,
           median_tie_gap_in_lr=float(np.median(gaps) / lr_logit) if len(gaps) else 0.0)
    assert rel.max() <= 2e-3
    if lr_logit == 1e-3:
        # the configuration as specified: the solves agree on every code
        assert agree >= 0.999
        assert moved == 0.0
    else:
        # 200 free-running steps at 20x the specified lr: sign differences
        # compound and the trajectories of a few coordinates drift apart (up
        # to 172 lr measured, median 38 lr, on 0.13 % of the codes), so the
        # bar is on what the two solves produce: the codes agree on at least
        # 99.8 % and the hardened layers are equally good (the reconstruction
        # errors within the loss-curve bar)
        assert agree >= 0.998
        assert abs(hard_gpu - hard_ref) <= 2e-3 * hard_ref
        assert moved > 0.001
    assert hard_ref < hard_rtn and hard_gpu < hard_rtn
