"""The allocation-free reconstruction call against the ordinary one: the
same kernels with the loss partials in the library's static device array
instead of a caller workspace, so R^T, G and the loss must be bit-identical.
Two calls in a row (an expert batch, then a smaller dense layer), so the
second runs on the array the first left behind."""

import numpy as np
import pytest

import synthetic
from tests.gpu_util import device, to_dev_bf16, report

pytestmark = pytest.mark.gpu


def _case(dev, counts, rpe, K, seed):
    import torch
    rng = np.random.default_rng(seed)
    E = len(counts)
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    X = to_dev_bf16(synthetic.bf16_bits(rng.normal(0, 1, (int(offs[-1]), K)).astype(np.float32)), dev)
    dW = to_dev_bf16(synthetic.bf16_bits(rng.normal(0, 0.01, (E * rpe, K)).astype(np.float32)), dev)
    XT = torch.empty((max(1, int(offs[-1]) * K),), dtype=torch.bfloat16, device=dev)
    import post_weight_quantization_philox_amd as g
    g.gsq_transpose_tokens(E, offs, K, X, XT)
    return offs, X, XT, dW


def _run(g, torch, dev, offs, rpe, K, X, XT, dW, noalloc):
    E = len(offs) - 1
    T = int(offs[-1])
    RT = torch.full((max(1, rpe * T),), float("nan"), dtype=torch.bfloat16, device=dev)
    G = torch.full((E * rpe, K), float("nan"), dtype=torch.float32, device=dev)
    loss = torch.full((2,), float("nan"), dtype=torch.float64, device=dev)
    if noalloc:
        g.gsq_recon_loss_grad_noalloc(E, offs, rpe, K, X, XT, dW, RT, G, loss)
    else:
        ws = torch.empty((g.gsq_recon_workspace_bytes(E, offs, rpe, K) // 4,), dtype=torch.float32,
                         device=dev)
        g.gsq_recon_loss_grad(E, offs, rpe, K, X, XT, dW, ws, RT, G, loss)
    torch.cuda.synchronize()
    return RT, G, loss


def test_noalloc_matches_workspace_call():
    import torch
    import post_weight_quantization_philox_amd as g
    dev = device()
    # call 1: five experts (one without tokens, ragged blocks); call 2: a
    # smaller dense layer whose partials are fewer than call 1 left behind
    cases = [([64, 0, 320, 128, 576], 512, 512, 1), ([256], 384, 256, 2)]
    for counts, rpe, K, seed in cases:
        offs, X, XT, dW = _case(dev, counts, rpe, K, seed)
        ref = _run(g, torch, dev, offs, rpe, K, X, XT, dW, noalloc=False)
        got = _run(g, torch, dev, offs, rpe, K, X, XT, dW, noalloc=True)
        print(f"[no-alloc] experts={len(counts)} rows/expert={rpe} cols={K} tokens={int(offs[-1])}",
              flush=True)
        assert torch.equal(got[0].view(torch.int16), ref[0].view(torch.int16))
        assert torch.equal(got[1], ref[1])
        assert got[2][0].item() == ref[2][0].item() and np.isfinite(got[2][0].item())
        report(f"no-alloc recon {len(counts)}x{rpe}x{K}", loss=got[2][0].item())
    # too large for the static array: rejected before any launch
    big = np.array([0, 2 * 65536], dtype=np.int64)
    with pytest.raises(g.GsqError, match="GSQ_ERR_SCRATCH"):
        g.gsq_recon_loss_grad_noalloc(1, big, 65536, 128, X, XT, dW, X, X, X)
