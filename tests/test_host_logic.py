"""Host-side logic of the product checked on the CPU: the temperature
schedule the solver hands to the kernels (annealing, agihunt.info method
paragraph) against the oracle's schedule."""

import numpy as np
import pytest

import oracle


@pytest.mark.parametrize("T", [1, 2, 24, 200])
@pytest.mark.parametrize("ends", [(1.0, 0.05), (1.0, 0.1)])
def test_solver_tau_schedule_equals_oracle(T, ends):
    pytest.importorskip("torch")
    from post_weight_quantization_philox_amd.solver import tau_schedule
    got = np.asarray(tau_schedule(T, *ends), dtype=np.float64)
    ref = oracle.tau_schedule(T, *ends)
    assert got.shape == ref.shape
    # the solver passes Python floats holding fp32 values: bit-identical to the oracle's fp32
    assert np.array_equal(got.astype(np.float32).view(np.uint32), ref.view(np.uint32))
    assert np.array_equal(got, ref.astype(np.float64))
