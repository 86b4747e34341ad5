"""Parity on seeded random shapes: grouped products over random expert counts
(up to 70, so some batches take two launches) and random token blocks
(empty ones included), and the relax backward + Lion on random row counts and
group counts (odd numbers of scale groups included), the relaxed forward on
random shapes, the Gram-form product on random layer and token sizes, and
the fused second product against the separate calls on random expert
layouts. Each case runs
the same checks, with the same tolerances, as the fixed-shape tests in
test_gpu_parity.py and test_gpu_fused.py."""

import numpy as np
import pytest

import oracle
from tests import test_gpu_parity as parity
from tests.gpu_util import device

pytestmark = pytest.mark.gpu


def _recon_cases(n, seed=2024):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        # the first case takes more experts than one grouped launch holds
        E = int(rng.integers(65, 71)) if not cases else int(rng.integers(1, 71))
        rpe = int(rng.choice([32, 64, 160, 256, 288]))
        K = int(rng.choice([128, 256, 384, 640]))
        offs = [0] + np.cumsum(rng.choice([0, 64, 128, 192, 320], E)).tolist()
        if offs[-1] == 0:
            continue
        cases.append((E * rpe, int(offs[-1]), K, offs if E > 1 else None))
    return cases


def _bwd_cases(n, seed=2025):
    rng = np.random.default_rng(seed)
    grids = [oracle.GRID_INT2, oracle.GRID_TERNARY, oracle.GRID_INT3_LOCAL, oracle.GRID_INT3]
    return [(grids[i % 4], (int(rng.integers(1, 40)), 128 * int(rng.integers(1, 7))),
             float(rng.choice([1.0, 0.3, 0.05]))) for i in range(n)]


@pytest.fixture(scope="module")
def dev():
    return device()


@pytest.mark.parametrize("M,N,K,offs", _recon_cases(8),
                         ids=lambda v: None if not isinstance(v, list) else f"E{len(v) - 1}")
def test_recon_random_shapes(dev, M, N, K, offs):
    parity.test_recon_loss_grad(dev, M, N, K, offs)


@pytest.mark.parametrize("grid,shape,tau", _bwd_cases(8),
                         ids=lambda v: f"{v[0]}x{v[1]}" if isinstance(v, tuple) else str(v))
def test_relax_bwd_random_shapes(dev, grid, shape, tau):
    parity.test_relax_bwd_lion(dev, grid, tau, shape)


def _fused_cases(n, seed=2026):
    rng = np.random.default_rng(seed)
    grids = [oracle.GRID_INT2, oracle.GRID_TERNARY, oracle.GRID_INT3_LOCAL, oracle.GRID_INT3]
    cases = []
    for i in range(n):
        E = int(rng.integers(65, 71)) if i == 0 else int(rng.integers(1, 40))
        counts = [int(c) for c in rng.choice([0, 64, 128, 192], E)]
        if sum(counts) == 0:
            counts[0] = 64
        cases.append((grids[i % 4], int(rng.choice([32, 64, 160, 256])),
                      int(rng.choice([128, 256, 384])), counts, bool(i % 2 == 0)))
    return cases


@pytest.mark.parametrize("grid,rpe,K,counts,with_next", _fused_cases(6),
                         ids=lambda v: f"E{len(v)}" if isinstance(v, list) else str(v))
def test_fused_step_random_layouts(dev, grid, rpe, K, counts, with_next):
    """The second product fused into backward + Lion (+ next forward) against
    the separate calls, bit for bit, on random expert layouts."""
    import torch
    import post_weight_quantization_philox_amd as g
    from tests import test_gpu_fused as fused
    offs, t = fused._state(grid, rpe, K, counts, seed=len(counts) * 7 + rpe, dev=dev)
    out = fused._both(g, torch, dev, grid, rpe, K, offs, t, with_next)
    a, b = out["separate"], out["fused"]
    assert np.isfinite(a["loss"].item())
    assert torch.equal(a["loss"], b["loss"])
    assert torch.equal(a["RT"].view(torch.int16), b["RT"].view(torch.int16))
    for k in ("logits", "mom", "scales", "scale_mom"):
        assert torch.equal(a[k], b[k]), k
    assert torch.equal(a["dW"].view(torch.int16), b["dW"].view(torch.int16))
    assert not torch.equal(a["logits"], t["logits"])


def _fwd_cases(n, seed=2027):
    rng = np.random.default_rng(seed)
    grids = [oracle.GRID_INT2, oracle.GRID_TERNARY, oracle.GRID_INT3_LOCAL, oracle.GRID_INT3]
    return [(grids[i % 4], float(rng.choice([1.0, 0.3, 0.05])), float(rng.choice([1.0, 0.0])),
             (int(rng.integers(1, 48)), 128 * int(rng.integers(1, 7)))) for i in range(n)]


@pytest.mark.parametrize("grid,tau,eta,shape", _fwd_cases(8),
                         ids=lambda v: f"{v[0]}x{v[1]}" if isinstance(v, tuple) else str(v))
def test_relax_fwd_random_shapes(dev, grid, tau, eta, shape):
    parity.test_relax_fwd(dev, grid, tau, eta, shape)


def _gram_cases(n, seed=2028):
    rng = np.random.default_rng(seed)
    return [(int(rng.integers(1, 600)), 64 * int(rng.integers(1, 9)), 128 * int(rng.integers(1, 9)))
            for _ in range(n)]


@pytest.mark.parametrize("M,N,K", _gram_cases(4))
def test_recon_gram_random_shapes(dev, M, N, K):
    parity.test_recon_gram(dev, M, N, K)
