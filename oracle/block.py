"""Plain CPU oracle of a synthetic transformer block (NumPy, fp64): the
forward pass whose intermediate activations are the calibration inputs of
GSQ's staged block schedule.

TEST INFRASTRUCTURE. Only ``tests/`` may import this module. It shares no
code with the GPU library and the GPU library never calls it.

The pages optimise a decoder block in stages: the query and key projections
first, then value and output projections, then the MLP on the block's
output, each stage frozen before the next and its quantized outputs
propagated to the next stage's inputs (agihunt.info, optimizer paragraph on
the staged block schedule). The schedule itself is host sequencing and is
not repeated here; this module holds the block it runs over, so that the
inputs every stage sees can be checked. The block is a Llama-shaped decoder
block with random weights: RMSNorm, causal multi-head attention with grouped
key / value heads (no positional rotation: the schedule, not the model, is
the subject), a residual, RMSNorm, a SwiGLU MLP and a residual.
:func:`block_forward` is exact fp64; :func:`block_forward_mirror` is the same
forward with bfloat16 roundings where the GPU stores an intermediate.
"""

from __future__ import annotations

import numpy as np

from . import gsq


def rmsnorm(x, gamma, eps: float = 1e-5):
    """y = x / sqrt(mean(x^2) + eps) * gamma, per row."""
    x = np.asarray(x, dtype=np.float64)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + eps)
    return x * r * np.asarray(gamma, dtype=np.float64)[None, :]


def softmax_causal(S, scale: float):
    """Row i of softmax(scale * S) over columns 0..i; later columns are 0."""
    S = np.asarray(S, dtype=np.float64) * scale
    n = S.shape[0]
    mask = np.tril(np.ones((n, S.shape[1]), dtype=bool))
    S = np.where(mask, S, -np.inf)
    S = S - S.max(axis=1, keepdims=True)
    P = np.exp(S)
    return P / P.sum(axis=1, keepdims=True)


def silu_mul(gate, up):
    """SwiGLU: silu(gate) * up with silu(z) = z / (1 + exp(-z))."""
    g = np.asarray(gate, dtype=np.float64)
    return g / (1.0 + np.exp(-g)) * np.asarray(up, dtype=np.float64)


def attention(xn, Wq, Wk, Wv, heads: int, kv_heads: int, head_dim: int):
    """Causal attention output before the output projection, [tokens, heads*head_dim]."""
    Q = xn @ np.asarray(Wq, dtype=np.float64).T
    K = xn @ np.asarray(Wk, dtype=np.float64).T
    V = xn @ np.asarray(Wv, dtype=np.float64).T
    group = heads // kv_heads
    out = np.zeros((xn.shape[0], heads * head_dim))
    for h in range(heads):
        g = h // group
        q = Q[:, h * head_dim:(h + 1) * head_dim]
        k = K[:, g * head_dim:(g + 1) * head_dim]
        v = V[:, g * head_dim:(g + 1) * head_dim]
        P = softmax_causal(q @ k.T, 1.0 / np.sqrt(head_dim))
        out[:, h * head_dim:(h + 1) * head_dim] = P @ v
    return out


def block_forward(x, w: dict, cfg: dict):
    """The block's output and the inputs each projection sees:
    ``{"out", "x_attn", "x_o", "h", "x_mlp", "x_down"}`` (``h`` is the
    residual stream after attention)."""
    x = np.asarray(x, dtype=np.float64)
    xa = rmsnorm(x, w["g_attn"])
    ao = attention(xa, w["q"], w["k"], w["v"], cfg["heads"], cfg["kv_heads"], cfg["head_dim"])
    h = x + ao @ np.asarray(w["o"], dtype=np.float64).T
    xm = rmsnorm(h, w["g_mlp"])
    act = silu_mul(xm @ np.asarray(w["gate"], dtype=np.float64).T,
                   xm @ np.asarray(w["up"], dtype=np.float64).T)
    out = h + act @ np.asarray(w["down"], dtype=np.float64).T
    return {"out": out, "x_attn": xa, "x_o": ao, "h": h, "x_mlp": xm, "x_down": act}


def dequantize(codes, scales_f16_bits, grid: int, group: int = 128):
    """Hard weights s * v(code) from stored codes and fp16 scale bits."""
    s = np.asarray(scales_f16_bits, dtype=np.uint16).view(np.float16).astype(np.float64)
    c = np.asarray(codes, dtype=np.int64)
    v = (c - 1).astype(np.float64) if grid == gsq.GRID_TERNARY else \
        gsq.level_value(c, gsq.CODE_BITS[grid]).astype(np.float64)
    return np.repeat(s, group, axis=1) * v


def _rb(x):
    return gsq.round_bf16(np.asarray(x, dtype=np.float64).astype(np.float32)).astype(np.float64)


def block_forward_mirror(x, w: dict, cfg: dict):
    """:func:`block_forward` with every intermediate rounded to bfloat16
    where the GPU stores one (projections, scores, probabilities, attention
    output, residuals, norms, SwiGLU); the arithmetic between roundings stays
    fp64. Weights and x are taken as given (bf16 values)."""
    x = np.asarray(x, dtype=np.float64)
    f = lambda a, W: _rb(a @ np.asarray(W, dtype=np.float64).T)
    xa = _rb(rmsnorm(x, w["g_attn"]))
    Q, K, V = f(xa, w["q"]), f(xa, w["k"]), f(xa, w["v"])
    hd, group = cfg["head_dim"], cfg["heads"] // cfg["kv_heads"]
    ao = np.zeros((x.shape[0], cfg["heads"] * hd))
    for h in range(cfg["heads"]):
        g = h // group
        S = _rb(Q[:, h * hd:(h + 1) * hd] @ K[:, g * hd:(g + 1) * hd].T)
        P = _rb(softmax_causal(S, 1.0 / np.sqrt(hd)))
        ao[:, h * hd:(h + 1) * hd] = _rb(P @ V[:, g * hd:(g + 1) * hd])
    h_ = _rb(x + f(ao, w["o"]))
    xm = _rb(rmsnorm(h_, w["g_mlp"]))
    act = _rb(silu_mul(f(xm, w["gate"]), f(xm, w["up"])))
    out = _rb(h_ + f(act, w["down"]))
    return {"out": out, "x_attn": xa, "x_o": ao, "h": h_, "x_mlp": xm, "x_down": act}


def stage_offset_T(W, x_q, x_fp, resid_q=None, resid_fp=None, mirror: bool = False):
    """Offset of a layer fitted to a full-precision target (the staged
    schedule's value/output and MLP stages, agihunt.info optimizer
    paragraph): E0^T = W (x_q - x_fp)^T + (resid_q - resid_fp)^T, so that
    with R = x_q dW^T + E0 the residual of the layer with weights W + dW is
    x_q (W + dW)^T + resid_q - (x_fp W^T + resid_fp). With ``mirror`` each
    difference, the product and the sum are rounded to bfloat16 where the GPU
    stores them."""
    r = _rb if mirror else (lambda a: np.asarray(a, dtype=np.float64))
    W = np.asarray(W, dtype=np.float64)
    d = r(np.asarray(x_q, dtype=np.float64) - np.asarray(x_fp, dtype=np.float64))
    E = r(W @ d.T)
    if resid_q is not None:
        dr = r(np.asarray(resid_q, dtype=np.float64) - np.asarray(resid_fp, dtype=np.float64))
        E = r(E + dr.T)
    return E

