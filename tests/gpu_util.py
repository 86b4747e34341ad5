"""Helpers for the GPU parity tests (host-side conversions only)."""

import numpy as np
import pytest


def device():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import post_weight_quantization_philox_amd as g
    g.lib()                       # the HIP library must load: no fallback
    return torch.device("cuda:0")


def to_dev_bf16(bits: np.ndarray, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def bf16_values(t) -> np.ndarray:
    """bf16 device tensor -> fp32 numpy values."""
    import torch
    b = t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def f32(t) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 numbers at |x| (8 significant bits)."""
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


def report(name: str, **vals):
    print(f"[parity] {name}: " + ", ".join(f"{k}={v:.3g}" if isinstance(v, float) else f"{k}={v}"
                                          for k, v in vals.items()), flush=True)
