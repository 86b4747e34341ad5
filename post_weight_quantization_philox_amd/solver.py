"""Per-layer GSQ solve driven from the host: device state plus the call order.

PyTorch only allocates the device tensors and provides the stream; every
arithmetic step runs in ``libgsq.so``. One :class:`LayerSolver` holds the
state of one layer (or one batch of experts) for the whole annealed solve:

* logits and their Lion momentum, planar [L][rows][cols] fp32;
* group scales and their momentum, [rows][cols/128] fp32;
* warm-start codes, [rows][cols] uint8;
* dW (bf16), G (fp32), R^T (bf16) and the loss partial workspace;
* the calibration tokens X (bf16) and their per-expert transpose X^T;
* with ``recon="gram"`` (one dense layer): H = X^T X (bf16, [in][in]) in
  place of R^T, so each step runs one product dW H instead of two.

With ``fuse=True`` each step's second product runs fused with the backward
+ Lion + next forward (:func:`gsq_recon_bwd_lion_fwd`): G is formed and
consumed tile by tile and never stored, with bit-identical results. It moves
8 bytes per weight less, but on the measured layers (the 64-expert batch
included) the separate calls are faster, so ``"auto"`` (the default) keeps
them.

Memory per coordinate: 8L bytes of logits + momentum, 1 (codes), 2 (dW),
4 (G), plus W itself; R^T, X and X^T scale with the token count.
"""

from __future__ import annotations

import json

import math

import numpy as np
import torch

from . import (GRID_INT3_LOCAL, DTYPE_BF16, DTYPE_F32, N_LOGITS, CODE_BITS, GsqLayer,
               GsqLion, gsq_init_rtn, gsq_gptq_workspace_bytes, gsq_init_gptq, gsq_relax_fwd,
               gsq_recon_workspace_bytes, gsq_recon_loss_grad, gsq_recon_loss_grad_offset,
               gsq_transpose_tokens, gsq_gram,
               gsq_recon_gram_workspace_bytes, gsq_recon_gram, gsq_relax_bwd_lion,
               gsq_relax_bwd_lion_fwd, gsq_recon_residual, gsq_recon_bwd_lion_fwd,
               gsq_harden_pack)

TOKEN_ALIGN = 64


def tau_schedule(steps: int, tau0: float = 1.0, tau1: float = 0.05) -> list:
    """Geometric annealing tau_t = tau0 * (tau1/tau0)**(t/(T-1))."""
    if steps == 1:
        return [float(np.float32(tau0))]
    return [float(np.float32(tau0 * (tau1 / tau0) ** (t / (steps - 1)))) for t in range(steps)]


def pad_tokens(X: torch.Tensor, tok_offsets) -> tuple:
    """Pad every expert's token block with zero rows to a multiple of 64.

    A zero token row adds nothing to the reconstruction loss or its gradient,
    so the padded problem has exactly the same loss and G.
    """
    offs = [int(o) for o in tok_offsets]
    counts = [offs[e + 1] - offs[e] for e in range(len(offs) - 1)]
    padded = [int(math.ceil(c / TOKEN_ALIGN) * TOKEN_ALIGN) for c in counts]
    if padded == counts:
        return X.contiguous(), np.asarray(offs, dtype=np.int64)
    new_offs = np.concatenate([[0], np.cumsum(padded)]).astype(np.int64)
    Xp = torch.zeros((int(new_offs[-1]), X.shape[1]), dtype=X.dtype, device=X.device)
    for e, c in enumerate(counts):
        Xp[int(new_offs[e]):int(new_offs[e]) + c] = X[offs[e]:offs[e] + c]
    return Xp, new_offs


class LayerSolver:
    """Device state and step sequence of one layer (or expert batch)."""

    def __init__(self, W: torch.Tensor, X: torch.Tensor, grid: int, tok_offsets=None,
                 rows_per_expert: int | None = None, seed: int = 0, stream_id: int = 0,
                 lion: GsqLion | None = None, init_logit: float = 2.0,
                 recon: str = "direct", init: str = "rtn", damp: float = 0.01,
                 fuse="auto", offset_T=None):
        if not (W.is_cuda and X.is_cuda):
            raise ValueError("W and X must be device tensors")
        if W.dtype not in (torch.bfloat16, torch.float32) or X.dtype != torch.bfloat16:
            raise ValueError("W must be bf16 or fp32 and X bf16")
        dev = W.device
        self.W = W.contiguous()
        self.rows, self.cols = self.W.shape
        self.grid = grid
        self.L = N_LOGITS[grid]
        if tok_offsets is None:
            tok_offsets = [0, X.shape[0]]
        self.n_experts = len(tok_offsets) - 1
        self.rows_per_expert = rows_per_expert or self.rows // self.n_experts
        if self.rows_per_expert * self.n_experts != self.rows:
            raise ValueError("rows must equal n_experts * rows_per_expert")
        if recon not in ("direct", "gram"):
            raise ValueError("recon must be 'direct' or 'gram'")
        if recon == "gram" and self.n_experts != 1:
            raise ValueError("the Gram form is for one dense layer (n_experts = 1)")
        self.recon_mode = recon
        if fuse not in ("auto", True, False):
            raise ValueError("fuse must be 'auto', True or False")
        if fuse is True and recon == "gram":
            raise ValueError("the fused step uses the direct products")
        self.fuse = False if fuse == "auto" else fuse
        self.fuse = self.fuse and recon == "direct"
        # A fixed offset on the residual (R = X dW^T + E0, given as E0^T
        # [rows][tokens] bf16): the layer is fitted to a target downstream of
        # itself. One dense layer, direct form, separate calls.
        self.offset_T = offset_T
        if offset_T is not None:
            if self.n_experts != 1 or recon != "direct" or fuse is True:
                raise ValueError("an offset needs one dense layer in the direct form")
            if tuple(offset_T.shape) != (W.shape[0], X.shape[0]) or X.shape[0] % 64:
                raise ValueError("offset_T must be [rows][tokens] with tokens a multiple of 64")
            self.fuse = False
        self.X, self.tok_offsets = pad_tokens(X, tok_offsets)
        self.tokens = int(self.tok_offsets[-1])
        self.layer = GsqLayer.make(grid, self.rows, self.cols,
                                   DTYPE_BF16 if W.dtype == torch.bfloat16 else DTYPE_F32,
                                   seed=seed, stream=stream_id)
        self.lion = lion or GsqLion.make()
        M, K, L = self.rows, self.cols, self.L
        f32 = dict(dtype=torch.float32, device=dev)
        self.logits = torch.empty((L, M, K), **f32)
        self.mom = torch.zeros((L, M, K), **f32)
        self.scales = torch.empty((M, K // 128), **f32)
        self.scale_mom = torch.zeros((M, K // 128), **f32)
        self.codes = torch.empty((M, K), dtype=torch.uint8, device=dev)
        self.dW = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
        self.G = torch.empty((M, K), **f32)
        self.XT = torch.empty((max(1, self.tokens * K),), dtype=torch.bfloat16, device=dev)
        if recon == "gram":
            self.RT = None
            self.H = torch.empty((K, K), dtype=torch.bfloat16, device=dev)
            ws = gsq_recon_gram_workspace_bytes(M, K)
        else:
            self.RT = torch.empty((max(1, self.rows_per_expert * self.tokens),),
                                  dtype=torch.bfloat16, device=dev)
            self.H = None
            ws = gsq_recon_workspace_bytes(self.n_experts, self.tok_offsets, self.rows_per_expert, K)
        self.workspace = torch.empty((max(ws, 256) // 4,), **f32)
        self.loss = torch.zeros((1,), dtype=torch.float64, device=dev)
        if init not in ("rtn", "gptq"):
            raise ValueError("init must be 'rtn' or 'gptq'")
        if init == "gptq" and (self.n_experts != 1 or self.tokens == 0):
            raise ValueError("the GPTQ warm start is for one dense layer with tokens")
        gsq_transpose_tokens(self.n_experts, self.tok_offsets, K, self.X, self.XT)
        self.gptq_info = None
        if init == "gptq":
            ws = torch.empty((gsq_gptq_workspace_bytes(M, K) + 255) // 256 * 256,
                             dtype=torch.uint8, device=dev)
            self.gptq_info = torch.zeros((1,), dtype=torch.int32, device=dev)
            gsq_init_gptq(self.layer, self.W, self.tokens, self.XT, damp, init_logit, ws,
                          self.scales, self.codes, self.logits, self.gptq_info)
            del ws
            info = int(self.gptq_info.item())
            if info != 0:
                # A non-positive pivot: the factor (and so the warm start) is
                # meaningless; more damping is the usual remedy.
                raise FloatingPointError(
                    f"GPTQ warm start: the damped Gram matrix X^T X + damp I is not positive "
                    f"definite at reversed column {info - 1} (damp={damp})")
        else:
            gsq_init_rtn(self.layer, self.W, self.scales, self.codes, self.logits, init_logit)
        if recon == "gram":
            if self.tokens == 0:
                self.H.zero_()
            else:
                gsq_gram(self.tokens, K, self.XT, self.H)

    @property
    def init_codes(self):
        return self.codes if self.grid == GRID_INT3_LOCAL else None

    def relax_fwd(self, step: int, tau: float, noise_scale: float = 1.0, w_soft_dbg=None):
        gsq_relax_fwd(self.layer, self.logits, self.scales, self.init_codes, self.W, step, tau,
                      noise_scale, self.dW, w_soft_dbg)

    def recon(self, loss_out=None):
        """Objective and gradient of the current dW; the loss goes to
        ``loss_out`` (a 16-byte aligned device fp64 scalar) or ``self.loss``."""
        loss = self.loss if loss_out is None else loss_out
        if self.recon_mode == "gram":
            gsq_recon_gram(self.rows, self.cols, self.H, self.dW, self.workspace, self.G, loss)
        elif self.offset_T is not None:
            gsq_recon_loss_grad_offset(self.rows, self.cols, self.tokens, self.X, self.XT, self.dW,
                                       self.offset_T, self.workspace, self.RT, self.G, loss)
        else:
            gsq_recon_loss_grad(self.n_experts, self.tok_offsets, self.rows_per_expert, self.cols,
                                self.X, self.XT, self.dW, self.workspace, self.RT, self.G, loss)

    def relax_bwd_lion(self, step: int, tau: float, noise_scale: float = 1.0,
                       grad_logits_dbg=None, grad_scales_dbg=None):
        gsq_relax_bwd_lion(self.layer, self.G, self.logits, self.mom, self.scales, self.scale_mom,
                           self.init_codes, step, tau, noise_scale, self.lion, grad_logits_dbg,
                           grad_scales_dbg)

    def relax_bwd_lion_fwd(self, step: int, tau: float, next_step: int, next_tau: float,
                           noise_scale: float = 1.0):
        gsq_relax_bwd_lion_fwd(self.layer, self.G, self.logits, self.mom, self.scales,
                               self.scale_mom, self.init_codes, self.W, step, tau, noise_scale,
                               self.lion, next_step, next_tau, self.dW)

    def step(self, step: int, tau: float, noise_scale: float = 1.0):
        """One relaxed-quantization step: forward, objective, backward + Lion."""
        self.relax_fwd(step, tau, noise_scale)
        self.recon()
        self.relax_bwd_lion(step, tau, noise_scale)

    def recon_residual(self):
        """First product of the objective (R^T and the loss partials), the
        half of :meth:`recon` that :meth:`recon_bwd_lion_fwd` completes."""
        gsq_recon_residual(self.n_experts, self.tok_offsets, self.rows_per_expert, self.cols,
                           self.X, self.dW, self.workspace, self.RT)

    def recon_bwd_lion_fwd(self, step: int, tau: float, next_tau: float | None,
                           noise_scale: float = 1.0, loss_out=None):
        """Second product of the objective fused with backward + Lion of
        ``step`` (+ the forward of ``step + 1`` at ``next_tau``, None on the
        last step); G is never stored. Follows :meth:`recon_residual`."""
        loss = self.loss if loss_out is None else loss_out
        gsq_recon_bwd_lion_fwd(self.layer, self.n_experts, self.tok_offsets, self.XT, self.RT,
                               self.workspace, loss, self.logits, self.mom, self.scales,
                               self.scale_mom, self.init_codes, self.W, step, tau, noise_scale,
                               self.lion, next_tau is not None, step + 1,
                               1.0 if next_tau is None else next_tau, self.dW)

    def step_fused(self, step: int, tau: float, next_tau: float | None,
                   noise_scale: float = 1.0):
        """Objective and backward + Lion of ``step`` (whose dW the previous
        call, or :meth:`relax_fwd`, produced), fused with the forward of
        ``step + 1`` at ``next_tau`` (None on the last step)."""
        if self.fuse:
            self.recon_residual()
            self.recon_bwd_lion_fwd(step, tau, next_tau, noise_scale)
            return
        self.recon()
        if next_tau is None:
            self.relax_bwd_lion(step, tau, noise_scale)
        else:
            self.relax_bwd_lion_fwd(step, tau, step + 1, next_tau, noise_scale)

    def capture_solve(self, steps: int, tau0: float = 1.0, tau1: float = 0.05,
                      noise_scale: float = 1.0):
        """The whole annealed solve (first forward, then every step's
        objective and fused backward + Lion + next forward) captured as one
        HIP graph, so a replay launches it with one call instead of about four
        launches per step. Temperatures are fixed at capture; the loss of step
        t lands in ``self.loss_hist[t, 0]``. Replaying continues from the
        current state (it does not reset it). Returns the graph."""
        taus = tau_schedule(steps, tau0, tau1)
        # one 16-byte slot per step (device tensors are passed 16-byte aligned)
        self.loss_hist = torch.zeros((steps, 2), dtype=torch.float64, device=self.W.device)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self.relax_fwd(0, taus[0], noise_scale)
            for t, tau in enumerate(taus):
                nxt = taus[t + 1] if t + 1 < steps else None
                if self.fuse:
                    self.recon_residual()
                    self.recon_bwd_lion_fwd(t, tau, nxt, noise_scale, self.loss_hist[t])
                    continue
                self.recon(self.loss_hist[t])
                if nxt is not None:
                    self.relax_bwd_lion_fwd(t, tau, t + 1, nxt, noise_scale)
                else:
                    self.relax_bwd_lion(t, tau, noise_scale)
        return graph

    def harden(self):
        """Hard codes (uint8), packed codes (int32 words) and fp16 scales."""
        M, K = self.rows, self.cols
        dev = self.W.device
        codes = torch.empty((M, K), dtype=torch.uint8, device=dev)
        packed = torch.empty((M, K * CODE_BITS[self.grid] // 32), dtype=torch.int32, device=dev)
        s16 = torch.empty((M, K // 128), dtype=torch.float16, device=dev)
        gsq_harden_pack(self.layer, self.logits, self.scales, self.init_codes, codes, packed, s16)
        return codes, packed, s16

    STATE = ("logits", "mom", "scales", "scale_mom", "codes")

    def state(self) -> dict:
        """Device copies of everything a solve carries from step to step:
        logits, Lion momenta, scales, scale momenta and the warm-start codes
        (local shift's centres). With the step index it is a checkpoint: the
        noise is a function of (seed, stream id, step, coordinate), so no
        generator state is needed and a resumed solve replays bit for bit."""
        return {k: getattr(self, k).clone() for k in self.STATE}

    def load_state(self, state: dict):
        """Restore a :meth:`state` taken from a solver of the same layer."""
        for k in self.STATE:
            getattr(self, k).copy_(state[k])

    def solve(self, steps: int, tau0: float = 1.0, tau1: float = 0.05, noise_scale: float = 1.0,
              log_every: int = 0, start: int = 0, stop: int | None = None,
              log_path: str | None = None):
        """The annealed solve over the schedule of ``steps`` temperatures,
        running steps ``start`` .. ``stop - 1`` (default: all). Returns the
        per-step losses (host, every step if ``log_every`` is 1, else only
        those logged) and the hard result, or None for it when the solve
        stops early (take :meth:`state` to resume it with ``start=stop``).
        With ``log_path`` every logged step is also appended there as one
        JSON line: step, tau, loss, layer shape, grid, seed and stream id. A
        logged loss that is not finite raises FloatingPointError."""
        log = open(log_path, "a") if log_path and log_every else None
        try:
            return self._solve(steps, tau0, tau1, noise_scale, log_every, start, stop, log)
        finally:
            if log is not None:
                log.close()

    def _solve(self, steps, tau0, tau1, noise_scale, log_every, start, stop, log):
        losses = []
        taus = tau_schedule(steps, tau0, tau1)
        stop = steps if stop is None else stop
        if not 0 <= start < stop <= steps:
            raise ValueError("need 0 <= start < stop <= steps")
        self.relax_fwd(start, taus[start], noise_scale)
        for t in range(start, stop):
            self.step_fused(t, taus[t], taus[t + 1] if t + 1 < stop else None, noise_scale)
            if log_every and (t % log_every == 0 or t == steps - 1):
                losses.append(float(self.loss.item()))
                if not math.isfinite(losses[-1]):
                    # A non-finite input (weights, activations or state) has
                    # reached the objective: stop instead of optimising NaNs.
                    raise FloatingPointError(f"non-finite loss {losses[-1]} at step {t}")
                if log is not None:
                    log.write(json.dumps({"step": t, "tau": taus[t], "loss": losses[-1],
                                          "rows": self.rows, "cols": self.cols,
                                          "grid": self.grid, "seed": self.layer.seed,
                                          "stream": self.layer.stream}) + "\n")
        return losses, (self.harden() if stop == steps else None)
