"""The annealed solve captured as one HIP graph: every replay (with eager
work and synchronisations between replays) reproduces the eager solve bit
for bit, for the direct and the Gram-form objective."""

import numpy as np
import pytest

import oracle
import synthetic
from tests.gpu_util import device, to_dev_bf16, report

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("recon", ["direct", "gram"])
def test_graph_replays_equal_eager_solve(recon):
    import torch
    import post_weight_quantization_philox_amd as g
    from post_weight_quantization_philox_amd.solver import LayerSolver
    dev = device()
    M, K, N, T = 256, 512, 320, 24
    d = synthetic.small_layer(M, K, N, seed=6, w_bf16=True)
    mk = lambda: LayerSolver(to_dev_bf16(d["W_bits"], dev), to_dev_bf16(d["X_bits"], dev),
                             oracle.GRID_INT2, seed=1, stream_id=3, recon=recon,
                             lion=g.GsqLion.make(lr_logit=5e-2, lr_scale=1e-6))
    eager = mk()
    losses, _ = eager.solve(T, 1.0, 0.05, log_every=1)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (eager.logits, eager.mom, eager.scales, eager.scale_mom)]
    sol = mk()
    init = [t.clone() for t in (sol.logits, sol.mom, sol.scales, sol.scale_mom)]
    graph = sol.capture_solve(T, 1.0, 0.05)
    for rep in range(3):
        for dst, src in zip((sol.logits, sol.mom, sol.scales, sol.scale_mom), init):
            dst.copy_(src)                          # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip((sol.logits, sol.mom, sol.scales, sol.scale_mom), ref):
            assert torch.equal(a, b), f"replay {rep}"
        hist = sol.loss_hist[:, 0].cpu().numpy()
        np.testing.assert_array_equal(hist, np.array(losses))
        codes = sol.harden()[0]
        torch.cuda.synchronize()
        assert torch.equal(codes, eager.harden()[0])
    report(f"graph solve {recon}", replays=3, last_loss=float(losses[-1]))
