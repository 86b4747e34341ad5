"""Staged GSQ over one decoder block, driven from the host.

The pages optimise a transformer block in stages rather than all layers at
once: the query and key projections first, then the value and output
projections, then the MLP on the block's output. Each stage is frozen before
the next, and its quantized weights shape the calibration inputs the later
stages see (agihunt.info, optimizer paragraph). This module runs that
schedule on a Llama-shaped decoder block (RMSNorm, causal attention with
grouped key/value heads and no positional rotation, SwiGLU MLP, two
residuals). Every step runs in ``libgsq.so``: the projections and attention
products on the bf16 NT GEMM, normalisation, softmax, SwiGLU, residuals and
dequantisation in their own kernels, and each layer's optimisation in
:class:`~post_weight_quantization_philox_amd.solver.LayerSolver`.

Readings: query and key are quantized together as one row-stacked layer (they
see the same input); the value/output stage quantizes V, then O on the
attention output recomputed with the quantized Q, K and V; gate and up are
quantized together, then down on the SwiGLU activations recomputed with the
quantized gate and up. With ``objective="block"`` (the default) the two
stage-closing projections are fitted to full-precision targets rather than to
their own outputs: O to the full-precision block's attention output, so it
absorbs the error the quantized Q, K and V leave (value/output jointly), and
down to the full-precision block output (the MLP on the block output). Each
is the layer objective with a fixed offset on the residual,
R = X dW^T + E0 (:func:`gsq_recon_loss_grad_offset`): for O,
E0 = (ao_q - ao_fp) W_o^T; for down, E0 = (act_q - act_fp) W_down^T +
(h_q - h_fp), where _q are the block's activations with the quantized earlier
stages and _fp those of the full-precision block. ``objective="layer"`` fits
every layer to its own output.
"""

from __future__ import annotations

import math
import time
from dataclasses import dataclass

import torch

from . import (GsqLion, GsqLayer, DTYPE_BF16, gsq_matmul_nt_bf16, gsq_rmsnorm_bf16,
               gsq_softmax_causal_bf16, gsq_silu_mul_bf16, gsq_add_bf16, gsq_sub_bf16,
               gsq_dequant_bf16, gsq_transpose_tokens)
from .solver import LayerSolver

PROJECTIONS = ("q", "k", "v", "o", "gate", "up", "down")


@dataclass(frozen=True)
class BlockConfig:
    hidden: int
    heads: int
    kv_heads: int
    head_dim: int
    mlp: int
    eps: float = 1e-5

    @property
    def q_dim(self) -> int:
        return self.heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.kv_heads * self.head_dim

    def shapes(self) -> dict:
        """[out, in] of every projection."""
        h = self.hidden
        return {"q": (self.q_dim, h), "k": (self.kv_dim, h), "v": (self.kv_dim, h),
                "o": (h, self.q_dim), "gate": (self.mlp, h), "up": (self.mlp, h),
                "down": (h, self.mlp)}


LLAMA3_8B = BlockConfig(hidden=4096, heads=32, kv_heads=8, head_dim=128, mlp=14336)


def _bf16(shape, dev):
    return torch.empty(shape, dtype=torch.bfloat16, device=dev)


def _linear(x, W):
    """x [n][in] times W [out][in]^T -> [n][out] (bf16)."""
    n, k = x.shape
    out = W.shape[0]
    y = _bf16((n, out), x.device)
    gsq_matmul_nt_bf16(n, out, k, x, k, W, k, y, out)
    return y


def forward(cfg: BlockConfig, w: dict, x: torch.Tensor) -> dict:
    """The block on tokens x [n][hidden] (bf16) with weights ``w`` (bf16
    projections [out][in], fp32 norm gains ``g_attn``, ``g_mlp``). Returns
    the block output and the input each projection sees: ``x_attn`` (q, k,
    v), ``x_o`` (o), ``x_mlp`` (gate, up), ``x_down`` (down); also ``h``,
    the residual stream after attention."""
    n, d = x.shape
    dev = x.device
    xa = _bf16((n, d), dev)
    gsq_rmsnorm_bf16(n, d, x, w["g_attn"], cfg.eps, xa)
    Q, K, V = _linear(xa, w["q"]), _linear(xa, w["k"]), _linear(xa, w["v"])
    VT = _bf16((cfg.kv_dim * n,), dev)
    gsq_transpose_tokens(1, [0, n], cfg.kv_dim, V, VT)
    S = _bf16((n, n), dev)
    P = _bf16((n, n), dev)
    ao = _bf16((n, cfg.q_dim), dev)
    group = cfg.heads // cfg.kv_heads
    hd = cfg.head_dim
    scale = 1.0 / math.sqrt(hd)
    for h in range(cfg.heads):
        g = h // group
        gsq_matmul_nt_bf16(n, n, hd, Q[:, h * hd:], cfg.q_dim, K[:, g * hd:], cfg.kv_dim, S, n)
        gsq_softmax_causal_bf16(n, S, scale, P)
        gsq_matmul_nt_bf16(n, hd, n, P, n, VT[g * hd * n:], n, ao[:, h * hd:], cfg.q_dim)
    hres = _bf16((n, d), dev)
    gsq_add_bf16(n * d, x, _linear(ao, w["o"]), hres)
    xm = _bf16((n, d), dev)
    gsq_rmsnorm_bf16(n, d, hres, w["g_mlp"], cfg.eps, xm)
    act = _bf16((n, cfg.mlp), dev)
    gsq_silu_mul_bf16(n * cfg.mlp, _linear(xm, w["gate"]), _linear(xm, w["up"]), act)
    out = _bf16((n, d), dev)
    gsq_add_bf16(n * d, hres, _linear(act, w["down"]), out)
    return {"out": out, "x_attn": xa, "x_o": ao, "h": hres, "x_mlp": xm, "x_down": act}


def recon_form(recon: str, cols: int, tokens: int) -> str:
    """The reconstruction form a layer uses. ``"auto"`` takes the Gram form
    (H = X^T X once, then one product of 2 rows cols^2 flops per step) where it
    needs fewer flops than the two direct products (4 rows tokens cols), i.e.
    where cols < 2 tokens; both forms compute the same objective."""
    if recon == "auto":
        return "gram" if cols < 2 * tokens else "direct"
    if recon not in ("direct", "gram"):
        raise ValueError(f"recon must be 'direct', 'gram' or 'auto', not {recon!r}")
    return recon


def offset_T(W: torch.Tensor, x_q: torch.Tensor, x_fp: torch.Tensor,
             resid_q: torch.Tensor | None = None, resid_fp: torch.Tensor | None = None):
    """E0^T = W (x_q - x_fp)^T (+ (resid_q - resid_fp)^T), [out][tokens] bf16:
    the offset that makes a layer with input x_q fit the output x_fp W^T
    (+ resid_fp - resid_q) of the full-precision block."""
    n, k = x_q.shape
    out = W.shape[0]
    dev = x_q.device
    d = torch.empty_like(x_q)
    gsq_sub_bf16(n * k, x_q, x_fp, d)
    E = _bf16((out, n), dev)
    gsq_matmul_nt_bf16(out, n, k, W, k, d, k, E, n)
    if resid_q is not None:
        dr = torch.empty_like(resid_q)
        gsq_sub_bf16(n * out, resid_q, resid_fp, dr)
        drT = _bf16((out * n,), dev)
        gsq_transpose_tokens(1, [0, n], out, dr, drT)
        E2 = _bf16((out, n), dev)
        gsq_add_bf16(out * n, E, drT, E2)
        E = E2
    return E


def _quantize(W: torch.Tensor, X: torch.Tensor, grid: int, steps: int, lion: GsqLion,
              tau0: float, tau1: float, init: str, seed: int, stream_id: int, recon: str,
              E0T: torch.Tensor | None = None):
    """One layer's annealed solve; returns the hard weights (bf16), the last
    relaxed loss and the reconstruction form used. With an offset E0T the
    direct form is used (the Gram form would need X^T E0 as well)."""
    form = "direct+offset" if E0T is not None else recon_form(recon, W.shape[1], X.shape[0])
    sol = LayerSolver(W, X, grid, seed=seed, stream_id=stream_id, lion=lion, init=init,
                      recon="direct" if E0T is not None else form, offset_T=E0T)
    losses, (codes, _, s16) = sol.solve(steps, tau0, tau1, log_every=steps)
    Wq = torch.empty_like(W)
    layer = GsqLayer.make(grid, W.shape[0], W.shape[1], DTYPE_BF16)
    gsq_dequant_bf16(layer, codes, s16.view(torch.int16), Wq)
    return Wq, losses[-1], form


def staged_quantize(cfg: BlockConfig, w: dict, x: torch.Tensor, grid: int, steps: int,
                    lion: GsqLion | None = None, tau0: float = 1.0, tau1: float = 0.05,
                    init: str = "rtn", seed: int = 0, recon: str = "direct",
                    objective: str = "block"):
    """The staged schedule. Returns ``(wq, info)``: the weights with every
    projection replaced by its hard quantized version, and per stage the wall
    time, the calibration inputs used, the last relaxed loss, each layer's
    reconstruction form (``recon``: "direct", "gram" or "auto", see
    :func:`recon_form`; "direct+offset" for a layer fitted to a
    full-precision target) and, with ``objective="block"``, the offsets used
    (``offset_T``: O and down)."""
    recon_form(recon, 1, 1)   # reject an unknown form before any work
    if objective not in ("block", "layer"):
        raise ValueError("objective must be 'block' or 'layer'")
    lion = lion or GsqLion.make()
    wq = dict(w)
    info = {}
    fp = forward(cfg, w, x) if objective == "block" else None

    def stage(name, fn):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        out = fn()
        torch.cuda.synchronize()
        info[name] = {"seconds": time.perf_counter() - t0, **out}

    def s1():
        xa = forward(cfg, wq, x)["x_attn"]
        qk = torch.cat([w["q"], w["k"]], dim=0)
        hq, loss, f = _quantize(qk, xa, grid, steps, lion, tau0, tau1, init, seed, 0, recon)
        wq["q"], wq["k"] = hq[:cfg.q_dim].contiguous(), hq[cfg.q_dim:].contiguous()
        return {"x": xa, "loss": loss, "recon": {"q_k": f}}

    def s2():
        xa = forward(cfg, wq, x)["x_attn"]
        wq["v"], lv, fv = _quantize(w["v"], xa, grid, steps, lion, tau0, tau1, init, seed, 1, recon)
        xo = forward(cfg, wq, x)["x_o"]
        e0 = offset_T(w["o"], xo, fp["x_o"]) if fp is not None else None
        wq["o"], lo, fo = _quantize(w["o"], xo, grid, steps, lion, tau0, tau1, init, seed, 2, recon,
                                    e0)
        out = {"x": xo, "loss": lv + lo, "recon": {"v": fv, "o": fo}}
        if e0 is not None:
            out["offset_T"] = e0
        return out

    def s3():
        xm = forward(cfg, wq, x)["x_mlp"]
        gu = torch.cat([w["gate"], w["up"]], dim=0)
        hgu, lgu, fgu = _quantize(gu, xm, grid, steps, lion, tau0, tau1, init, seed, 3, recon)
        wq["gate"], wq["up"] = hgu[:cfg.mlp].contiguous(), hgu[cfg.mlp:].contiguous()
        fq = forward(cfg, wq, x)
        xd = fq["x_down"]
        e0 = (offset_T(w["down"], xd, fp["x_down"], fq["h"], fp["h"]) if fp is not None
              else None)
        wq["down"], ld, fd = _quantize(w["down"], xd, grid, steps, lion, tau0, tau1, init, seed, 4,
                                       recon, e0)
        out = {"x": xd, "loss": lgu + ld, "recon": {"gate_up": fgu, "down": fd}}
        if e0 is not None:
            out["offset_T"] = e0
        return out

    stage("q_k", s1)
    stage("v_o", s2)
    stage("mlp", s3)
    return wq, info
