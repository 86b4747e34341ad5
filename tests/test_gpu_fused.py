"""The second reconstruction product fused with backward + Lion (+ the next
forward) against the two-kernel path on identical inputs: gsq_recon_residual
+ gsq_recon_bwd_lion_fwd must reproduce gsq_recon_loss_grad +
gsq_relax_bwd_lion_fwd (or gsq_relax_bwd_lion on the last step) bit for bit:
R^T, loss, logits, momenta, scales, scale momenta and the next dW. The
two-kernel path is itself compared with the oracle in test_gpu_parity.py and
test_gpu_trajectory.py."""

import numpy as np
import pytest

import oracle
import synthetic
from tests.gpu_util import device, to_dev_bf16, report

pytestmark = pytest.mark.gpu

GRIDS = [oracle.GRID_INT2, oracle.GRID_TERNARY, oracle.GRID_INT3_LOCAL, oracle.GRID_INT3]

# (rows per expert, cols, token counts per expert): a dense layer whose rows
# end inside a 128-row tile; an expert batch with an expert without tokens and
# ragged blocks (padded to 64 by the solver, here given padded); 67 experts
# (two fused launches, the second starting at expert 64).
LAYOUTS = {
    "dense_ragged": (160, 384, [192]),
    "experts5": (256, 256, [64, 0, 320, 128, 64]),
    "experts67": (32, 128, list(np.random.default_rng(67).choice([0, 64, 128], 67))),
}


@pytest.fixture(scope="module")
def dev():
    return device()


def _state(grid, rpe, K, counts, seed, dev, w_bf16=True):
    import torch
    E = len(counts)
    M = E * rpe
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    rng = np.random.default_rng(seed)
    W = rng.normal(0, 0.02, (M, K)).astype(np.float32)
    W_bits = synthetic.bf16_bits(W)
    Wv = synthetic.bf16_to_f32(W_bits)
    s, c0, _ = oracle.init_rtn(Wv, grid)
    L = oracle.N_LOGITS[grid]
    st = {
        "logits": rng.normal(0, 1.5, (L, M, K)).astype(np.float32),
        "mom": (rng.normal(0, 1, (L, M, K)) * 1e-2).astype(np.float32),
        "scales": s,
        "scale_mom": (rng.normal(0, 1, s.shape) * 1e-3).astype(np.float32),
    }
    X_bits = synthetic.bf16_bits(rng.normal(0, 1, (int(offs[-1]), K)).astype(np.float32))
    dW_bits = synthetic.bf16_bits(rng.normal(0, 0.01, (M, K)).astype(np.float32))
    t = {k: torch.from_numpy(v).to(dev) for k, v in st.items()}
    t["codes"] = torch.from_numpy(c0).to(dev)
    t["W"] = to_dev_bf16(W_bits, dev) if w_bf16 else torch.from_numpy(Wv).to(dev)
    t["X"] = to_dev_bf16(X_bits, dev)
    t["dW"] = to_dev_bf16(dW_bits, dev)
    return offs, t


def _both(g, torch, dev, grid, rpe, K, offs, t, with_next, w_bf16=True):
    E = len(offs) - 1
    M = E * rpe
    T = int(offs[-1])
    layer = g.GsqLayer.make(grid, M, K, g.DTYPE_BF16 if w_bf16 else g.DTYPE_F32, seed=11,
                            stream=4)
    lion = g.GsqLion.make(lr_logit=2e-2, lr_scale=1e-5)
    XT = torch.empty((max(1, T * K),), dtype=torch.bfloat16, device=dev)
    g.gsq_transpose_tokens(E, offs, K, t["X"], XT)
    ws_bytes = g.gsq_recon_workspace_bytes(E, offs, rpe, K)
    codes = t["codes"] if grid == oracle.GRID_INT3_LOCAL else None
    step, tau, next_tau = 17, 0.4, 0.35
    out = {}
    for path in ("separate", "fused"):
        c = {k: t[k].clone() for k in ("logits", "mom", "scales", "scale_mom", "dW")}
        RT = torch.full((max(1, rpe * T),), float("nan"), dtype=torch.bfloat16, device=dev)
        ws = torch.empty((ws_bytes // 4,), dtype=torch.float32, device=dev)
        loss = torch.full((2,), float("nan"), dtype=torch.float64, device=dev)
        if path == "separate":
            G = torch.empty((M, K), dtype=torch.float32, device=dev)
            g.gsq_recon_loss_grad(E, offs, rpe, K, t["X"], XT, c["dW"], ws, RT, G, loss)
            if with_next:
                g.gsq_relax_bwd_lion_fwd(layer, G, c["logits"], c["mom"], c["scales"],
                                         c["scale_mom"], codes, t["W"], step, tau, 1.0, lion,
                                         step + 1, next_tau, c["dW"])
            else:
                g.gsq_relax_bwd_lion(layer, G, c["logits"], c["mom"], c["scales"], c["scale_mom"],
                                     codes, step, tau, 1.0, lion)
        else:
            g.gsq_recon_residual(E, offs, rpe, K, t["X"], c["dW"], ws, RT)
            g.gsq_recon_bwd_lion_fwd(layer, E, offs, XT, RT, ws, loss, c["logits"], c["mom"],
                                     c["scales"], c["scale_mom"], codes, t["W"], step, tau, 1.0,
                                     lion, with_next, step + 1, next_tau, c["dW"])
        torch.cuda.synchronize()
        c["RT"], c["loss"] = RT, loss[:1]
        out[path] = c
    return out


@pytest.mark.parametrize("grid", GRIDS)
@pytest.mark.parametrize("layout", list(LAYOUTS))
@pytest.mark.parametrize("with_next", [True, False])
def test_fused_step_bit_identical(dev, grid, layout, with_next):
    import torch
    import post_weight_quantization_philox_amd as g
    rpe, K, counts = LAYOUTS[layout]
    offs, t = _state(grid, rpe, K, counts, seed=grid * 10 + len(counts), dev=dev)
    out = _both(g, torch, dev, grid, rpe, K, offs, t, with_next)
    a, b = out["separate"], out["fused"]
    print(f"[fused] grid={grid} layout={layout} with_next={with_next} loss={a['loss'].item():.6g}",
          flush=True)
    assert np.isfinite(a["loss"].item())
    assert torch.equal(a["loss"], b["loss"])
    assert torch.equal(a["RT"].view(torch.int16), b["RT"].view(torch.int16))
    for k in ("logits", "mom", "scales", "scale_mom"):
        assert torch.equal(a[k], b[k]), k
    assert torch.equal(a["dW"].view(torch.int16), b["dW"].view(torch.int16))
    # the step moved the state (the comparison is not between two no-ops)
    assert not torch.equal(a["logits"], t["logits"])
    if with_next:
        assert not torch.equal(a["dW"].view(torch.int16), t["dW"].view(torch.int16))


def test_fused_step_fp32_weights(dev):
    """fp32 W (the 512x512 layer's dtype) in the fused next forward."""
    import torch
    import post_weight_quantization_philox_amd as g
    rpe, K, counts = 256, 512, [256]
    offs, t = _state(oracle.GRID_INT2, rpe, K, counts, seed=3, dev=dev, w_bf16=False)
    out = _both(g, torch, dev, oracle.GRID_INT2, rpe, K, offs, t, True, w_bf16=False)
    for k in ("logits", "mom", "scales", "scale_mom", "loss"):
        assert torch.equal(out["separate"][k], out["fused"][k]), k
    assert torch.equal(out["separate"]["dW"].view(torch.int16), out["fused"]["dW"].view(torch.int16))


@pytest.mark.parametrize("grid", [oracle.GRID_INT2, oracle.GRID_INT3_LOCAL])
def test_fused_solver_equals_separate_solver(dev, grid):
    """A whole annealed solve of an expert batch with the fused step and with
    the separate calls: identical losses at every step and identical final
    state and hard codes; and the fused solve captured as one HIP graph
    replays it bit for bit (with eager work between replays)."""
    import torch
    import post_weight_quantization_philox_amd as g
    from post_weight_quantization_philox_amd.solver import LayerSolver
    rng = np.random.default_rng(9)
    E, rpe, K, T = 4, 256, 384, 12
    counts = [100, 0, 256, 37]
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    W = to_dev_bf16(synthetic.bf16_bits(rng.normal(0, 0.02, (E * rpe, K)).astype(np.float32)), dev)
    X = to_dev_bf16(synthetic.bf16_bits(rng.normal(0, 1, (int(offs[-1]), K)).astype(np.float32)), dev)
    mk = lambda fuse: LayerSolver(W, X, grid, tok_offsets=offs, rows_per_expert=rpe, seed=2,
                                  stream_id=6, fuse=fuse,
                                  lion=g.GsqLion.make(lr_logit=5e-2, lr_scale=1e-5))
    sep, fus = mk(False), mk(True)
    assert fus.fuse and not sep.fuse
    ls, hs = sep.solve(T, 1.0, 0.05, log_every=1)
    lf, hf = fus.solve(T, 1.0, 0.05, log_every=1)
    assert ls == lf
    for k in ("logits", "mom", "scales", "scale_mom"):
        assert torch.equal(getattr(sep, k), getattr(fus, k)), k
    for a, b in zip(hs, hf):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.float16 else a,
                           b.view(torch.int16) if b.dtype == torch.float16 else b)
    cap = mk(True)
    init = [x.clone() for x in (cap.logits, cap.mom, cap.scales, cap.scale_mom)]
    graph = cap.capture_solve(T, 1.0, 0.05)
    for rep in range(3):
        for dst, src in zip((cap.logits, cap.mom, cap.scales, cap.scale_mom), init):
            dst.copy_(src)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k in ("logits", "mom", "scales", "scale_mom"):
            assert torch.equal(getattr(cap, k), getattr(fus, k)), (rep, k)
        np.testing.assert_array_equal(cap.loss_hist[:, 0].cpu().numpy(), np.array(lf))
    report(f"fused solver grid={grid}", steps=T, last_loss=float(lf[-1]))
