"""Seeded synthetic workloads: layer weights and calibration activations.

This module only draws inputs. It holds none of the quantization method's
arithmetic and is the one piece both the CPU oracle tests and the GPU path
use. There is no real model or calibration set here; each workload has the
shape, dtype and value distribution of a layer the pages quantize
(Llama-3.1-8B / 70B projections and a mixture-of-experts batch).

Recipe: every array comes from ``numpy.random.default_rng(seed)`` in the order
W, then the workload's extras that shape X (expert token counts), then X, then
extras that modify X (outlier channels). Normals are drawn in fp32, Student-t
in fp64; bf16 inputs are the fp32 draw rounded to nearest even.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

INT2, TERNARY, INT3_LOCAL, INT3 = 0, 1, 2, 3


@dataclass(frozen=True)
class Workload:
    name: str
    rows: int                 # out features (summed over experts for MoE)
    cols: int                 # in features
    tokens: int               # calibration tokens (expected total for MoE)
    grid: int
    w_sigma: float
    w_bf16: bool
    x_kind: str               # "normal", "normal_outliers", "student_t4"
    experts: int = 1
    rows_per_expert: int = 0
    lr_logit: float = 1e-3
    steps: int = 200
    extra: dict = field(default_factory=dict)

    @property
    def coords(self) -> int:
        return self.rows * self.cols


WORKLOADS = {
    # 512x512 linear layer, fp32 weights, 2-bit grid, 256 calibration tokens.
    "linear512_int2": Workload("linear512_int2", 512, 512, 256, INT2, 0.02, False, "normal"),
    # Llama-3.1-8B-shaped q_proj, 2-bit, 4096 tokens with 1 % outlier channels x20.
    "qproj4096_int2": Workload("qproj4096_int2", 4096, 4096, 4096, INT2, 0.02, True,
                               "normal_outliers", extra={"outlier_frac": 0.01, "outlier_gain": 20.0}),
    # 8B-shaped down_proj, ternary (mask + sign), Student-t(4) activations.
    "downproj4096x14336_ternary": Workload("downproj4096x14336_ternary", 4096, 14336, 4096,
                                           TERNARY, 0.015, True, "student_t4"),
    # 70B-shaped gate_proj, 3-bit local shift around the warm-start code.
    "gateproj28672x8192_int3local": Workload("gateproj28672x8192_int3local", 28672, 8192, 8192,
                                             INT3_LOCAL, 0.01, True, "normal"),
    # The same gate_proj with the full 3-bit grid (8 logits): the baseline local shift replaces.
    "gateproj28672x8192_int3full": Workload("gateproj28672x8192_int3full", 28672, 8192, 8192,
                                            INT3, 0.01, True, "normal"),
    # 64 experts of 2048x7168, 2-bit, routed token counts ~ Zipf(1.1) on [64, 1024].
    "moe64x2048x7168_int2": Workload("moe64x2048x7168_int2", 64 * 2048, 7168, 20_900, INT2, 0.02,
                                     True, "normal", experts=64, rows_per_expert=2048,
                                     extra={"zipf_a": 1.1, "n_min": 64, "n_max": 1024}),
}


_CHUNK = 1 << 24


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 array -> bfloat16 bit patterns (uint16), nearest even.

    Works in 32-bit words, in chunks: where b + 0x7FFF + lsb wraps past 2^32
    (only NaN patterns), the kept bits (sum >> 16) mod 2^16 are the same as
    with a wider sum."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    out = np.empty(b.shape, dtype=np.uint16)
    fb, fo = b.reshape(-1), out.reshape(-1)
    for i in range(0, fb.size, _CHUNK):
        c = fb[i:i + _CHUNK]
        fo[i:i + _CHUNK] = (c + np.uint32(0x7FFF) + ((c >> np.uint32(16)) & np.uint32(1))) \
            >> np.uint32(16)
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def expert_token_counts(rng, experts: int, a: float, n_min: int, n_max: int) -> np.ndarray:
    """i.i.d. draws from the pmf proportional to n**-a on {n_min..n_max}."""
    n = np.arange(n_min, n_max + 1)
    p = n.astype(np.float64) ** -a
    return rng.choice(n, size=experts, p=p / p.sum()).astype(np.int64)


def generate(w: Workload | str, seed: int = 0, rows: int | None = None):
    """Draw one workload. Returns a dict with

    * ``W``: fp32 values [rows, cols] (bf16-representable when ``w_bf16``);
    * ``W_bits``: bf16 bits of W (or None for fp32 weights);
    * ``X``: fp32 values [tokens, cols], bf16-representable;
    * ``X_bits``: bf16 bits of X;
    * ``tok_offsets``: int64 [experts + 1] token offsets.

    ``rows`` truncates the layer (the draw of the first rows is unchanged).
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    rng = np.random.default_rng(seed)
    M = w.rows if rows is None else rows
    W = rng.standard_normal((w.rows, w.cols), dtype=np.float32)[:M] * np.float32(w.w_sigma)
    W_bits = None
    if w.w_bf16:
        W_bits = bf16_bits(W)
        W = bf16_to_f32(W_bits)
    if w.experts > 1:
        counts = expert_token_counts(rng, w.experts, w.extra["zipf_a"], w.extra["n_min"],
                                     w.extra["n_max"])
        offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    else:
        offs = np.array([0, w.tokens], dtype=np.int64)
    N = int(offs[-1])
    if w.x_kind == "student_t4":
        X = rng.standard_t(4, size=(N, w.cols)).astype(np.float32)
    else:
        X = rng.standard_normal((N, w.cols), dtype=np.float32)
    if w.x_kind == "normal_outliers":
        n_out = int(round(w.extra["outlier_frac"] * w.cols))
        ch = rng.permutation(w.cols)[:n_out]
        X[:, ch] *= np.float32(w.extra["outlier_gain"])
    X_bits = bf16_bits(X)
    X = bf16_to_f32(X_bits)
    return {"W": W, "W_bits": W_bits, "X": X, "X_bits": X_bits, "tok_offsets": offs,
            "workload": w}


def small_layer(rows: int, cols: int, tokens: int, seed: int = 0, w_sigma: float = 0.02,
                w_bf16: bool = True):
    """A small Gaussian layer and bf16 Gaussian activations for tests."""
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((rows, cols), dtype=np.float32) * np.float32(w_sigma)
    W_bits = None
    if w_bf16:
        W_bits = bf16_bits(W)
        W = bf16_to_f32(W_bits)
    X_bits = bf16_bits(rng.standard_normal((tokens, cols), dtype=np.float32))
    return {"W": W, "W_bits": W_bits, "X": bf16_to_f32(X_bits), "X_bits": X_bits,
            "tok_offsets": np.array([0, tokens], dtype=np.int64)}
