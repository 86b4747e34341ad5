"""Plain CPU oracle of the GSQ relaxed-quantization step (NumPy, fp64).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. It shares no code
with the GPU library and the GPU library never calls it.

What it computes, and where the pages say so (all pages are about the paper
"GSQ: Highly-Accurate Low-Precision Scalar Quantization for LLMs via
Gumbel-Softmax Sampling"):

* The grid is a symmetric scalar grid with one scale per group of 128 weights
  and no zero point (agihunt.info summary: idea paragraph, results paragraph,
  takeaway paragraph; thelatestinai.com abstract).
* Each weight coordinate carries learnable logits over the grid levels; a
  Gumbel-Softmax sample gives a soft weighted sum of grid points; as the
  temperature is annealed the sum collapses to a hard choice (agihunt.info,
  method paragraph).
* 2-bit: four uniform levels, four logits per coordinate plus a shared group
  scale. Ternary: two binary choices, a mask and a sign, so half the logits.
  3 bits and more: local shift, only the offsets -2..+2 around the warm-start
  code, five logits instead of eight (agihunt.info, method paragraph;
  atlas.scime.ai summary, Approach section).
* Group scales are learned jointly with the assignments (atlas.scime.ai,
  Summary and Approach; thelatestinai.com abstract).
* The objective is the output reconstruction error on calibration inputs
  (agihunt.info, method paragraph).
* The optimizer is Lion (agihunt.info, optimizer paragraph; atlas.scime.ai,
  Surprising findings).

Readings where the pages are silent are listed in the repository's design
notes; the ones that change numbers are repeated at the function they affect.

Precision: every smooth quantity is computed in fp64. Where a floating-point
value decides an integer (the round-to-nearest warm-start code, the sign taken
by Lion, the fp16 output scale) the decision is taken in fp32, the precision
the GPU kernels use, so that both sides decide identically on identical
inputs. No function here is blocked, fused or reordered beyond the formulas.
"""

from __future__ import annotations

import numpy as np

from .philox import noise_words, uniform_from_word, gumbel, logistic

GRID_INT2 = 0
GRID_TERNARY = 1
GRID_INT3_LOCAL = 2
#: 3 bits with one logit per level of the whole 8-level grid: the baseline that
#: local shift approximates (agihunt.info, method paragraph: eight logits for
#: 3 bits without the shift).
GRID_INT3 = 3

#: logits per coordinate (agihunt.info, method paragraph: 4, 2, 5 and 8).
N_LOGITS = {GRID_INT2: 4, GRID_TERNARY: 2, GRID_INT3_LOCAL: 5, GRID_INT3: 8}
#: largest grid magnitude in units of the scale.
Q_MAX = {GRID_INT2: 3, GRID_TERNARY: 1, GRID_INT3_LOCAL: 7, GRID_INT3: 7}
#: bits per stored code (ternary codes t+1 in {0,1,2} take 2 bits).
CODE_BITS = {GRID_INT2: 2, GRID_TERNARY: 2, GRID_INT3_LOCAL: 3, GRID_INT3: 3}
#: offsets of the local-shift candidates around the warm-start code.
LOCAL_OFFSETS = (-2, -1, 0, 1, 2)


# ----------------------------------------------------------------------------
# Grid
# ----------------------------------------------------------------------------

def level_value(code, bits: int):
    """Value of an unsigned code on the symmetric b-bit grid, in scale units.

    Symmetric with no zero point and spacing 2: q(c) = 2c - (2**b - 1), which
    gives {-3,-1,1,3} for b=2 and the odd integers -7..7 for b=3.
    """
    return 2 * np.asarray(code, dtype=np.int64) - (2 ** bits - 1)


def grid_levels(grid: int) -> np.ndarray:
    """All grid values of a grid, in scale units."""
    if grid == GRID_INT2:
        return level_value(np.arange(4), 2).astype(np.float64)
    if grid in (GRID_INT3_LOCAL, GRID_INT3):
        return level_value(np.arange(8), 3).astype(np.float64)
    if grid == GRID_TERNARY:
        return np.array([-1.0, 0.0, 1.0])
    raise ValueError(f"unknown grid {grid}")


def candidate_codes(grid: int, init_codes: np.ndarray) -> np.ndarray:
    """Codes the L logits of each coordinate stand for, shape [L, ...].

    2-bit: the four codes 0..3 for every coordinate; full 3-bit: the eight
    codes 0..7. Local shift: the warm-start code plus offsets -2..+2, clamped
    to the 8-level range [0, 7] (so edge coordinates carry duplicate
    candidates).
    """
    if grid in (GRID_INT2, GRID_INT3):
        L = N_LOGITS[grid]
        shape = init_codes.shape if init_codes is not None else ()
        return np.broadcast_to(np.arange(L).reshape((L,) + (1,) * len(shape)),
                               (L,) + tuple(shape)).astype(np.int64)
    if grid == GRID_INT3_LOCAL:
        c0 = np.asarray(init_codes, dtype=np.int64)
        return np.stack([np.clip(c0 + d, 0, 7) for d in LOCAL_OFFSETS])
    raise ValueError("candidate codes exist for the 2-bit and local-shift grids")


# ----------------------------------------------------------------------------
# Warm start: round to nearest (the pages start from GPTQ or a GGUF K-Quant;
# the synthetic layers here start from round-to-nearest)
# ----------------------------------------------------------------------------

def init_rtn(W, grid: int, group: int = 128, init_logit: float = 2.0):
    """Absmax group scales, nearest-level codes and the initial logits.

    Returns ``(scales fp32 [M, K/group], codes uint8 [M, K], logits fp32
    [L, M, K])``. Codes are the warm-start code c0 (2-bit, local shift) or
    t0 + 1 with t0 in {-1, 0, 1} (ternary).

    Decisions in fp32: s = maxabs/q_max and x = w/s are correctly rounded fp32
    divisions; u = (x + q_max)*0.5 in fp32; the code is rint(u) (ties to even),
    clamped to the grid. A zero scale gives x = 0.
    Logits: +init_logit on the warm-start level, 0 on the others (local shift:
    the warm-start level is offset 0, logit index 2); ternary sets
    the mask logit to +init_logit if t0 != 0 else -init_logit, and the sign
    logit to +init_logit if w >= 0 else -init_logit.
    """
    w = np.asarray(W, dtype=np.float32)
    M, K = w.shape
    if K % group:
        raise ValueError("cols must be a multiple of the group size")
    qmax = np.float32(Q_MAX[grid])
    amax = np.abs(w).reshape(M, K // group, group).max(axis=2)
    s = (amax / qmax).astype(np.float32)
    codes, _ = _nearest_code(w, np.repeat(s, group, axis=1), grid)
    codes = codes.astype(np.uint8)
    logits = _logits_from_codes(codes, w, grid, init_logit)
    return s, codes, logits


def _logits_from_codes(codes, W, grid: int, init_logit: float):
    """Initial logits of warm-start codes, as :func:`init_rtn` sets them."""
    c = np.asarray(codes, dtype=np.int64)
    L = N_LOGITS[grid]
    il = np.float32(init_logit)
    logits = np.zeros((L,) + c.shape, dtype=np.float32)
    if grid == GRID_TERNARY:
        logits[0] = np.where(c != 1, il, -il)
        logits[1] = np.where(np.asarray(W, dtype=np.float32) >= 0, il, -il)
    elif grid == GRID_INT3_LOCAL:
        logits[2] = il
    else:
        for k in range(L):
            logits[k] = np.where(c == k, il, np.float32(0))
    return logits


def _nearest_code(t, s, grid: int):
    """Round-to-nearest code of target values t (fp64) with scales s, decided
    in fp32 exactly like :func:`init_rtn`: x = fp32(t) / s, then rint."""
    qmax = np.float32(Q_MAX[grid])
    tf = np.asarray(t, dtype=np.float64).astype(np.float32)
    sf = np.asarray(s, dtype=np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        x = np.where(sf > 0, tf / np.where(sf > 0, sf, np.float32(1)), np.float32(0)).astype(np.float32)
    if grid == GRID_TERNARY:
        return (np.clip(np.rint(x), -1, 1).astype(np.int64) + 1), x
    u = ((x + qmax).astype(np.float32) * np.float32(0.5)).astype(np.float32)
    return np.clip(np.rint(u), 0, 2 ** CODE_BITS[grid] - 1).astype(np.int64), u


def gptq_hessian(X, damp: float = 0.01) -> np.ndarray:
    """H = X^T X with GPTQ's damping: lambda = damp * mean(diag H) added to the
    diagonal; a column no token touches (zero diagonal) gets 1 there first,
    so the factorisations exist (its weight does not change the objective)."""
    Xd = np.asarray(X, dtype=np.float64)
    H = Xd.T @ Xd
    d = np.diag(H).copy()
    d[d == 0] = 1.0
    H[np.diag_indices_from(H)] = d
    H[np.diag_indices_from(H)] += damp * float(np.mean(d))
    return H


def gptq(W, X, grid: int, group: int = 128, damp: float = 0.01, init_logit: float = 2.0):
    """GPTQ warm start (Frantar, Ashkboos, Hoefler, Alistarh, "GPTQ: Accurate
    Post-Training Quantization for Generative Pre-trained Transformers", 2022:
    the Cholesky form of its column loop) on the symmetric group grid.

    The pages start GSQ from GPTQ (agihunt.info optimizer paragraph;
    atlas.scime.ai Approach). Group scales are the absmax scales of the
    original weights (GPTQ's static-groups option), so they equal
    :func:`init_rtn`'s. Then, column by column in order: the current column is
    rounded to the nearest grid level (decided in fp32 as in init_rtn); its
    error divided by the diagonal of the upper Cholesky factor U of H^-1
    (H from :func:`gptq_hessian`) is fed into every later column through row
    j of U. Returns ``(scales, codes, logits, targets)`` where targets [M, K]
    are the fp64 values each column was rounded from.
    """
    w = np.array(W, dtype=np.float64)
    M, K = w.shape
    scales, _, _ = init_rtn(W, grid, group, init_logit)
    s_full = np.repeat(scales, group, axis=1)
    H = gptq_hessian(X, damp)
    U = np.linalg.cholesky(np.linalg.inv(H)).T          # H^-1 = U^T U, U upper
    codes = np.zeros((M, K), dtype=np.int64)
    targets = np.zeros((M, K))
    for j in range(K):
        targets[:, j] = w[:, j]
        c, _ = _nearest_code(w[:, j], s_full[:, j], grid)
        codes[:, j] = c
        v = (c - 1).astype(np.float64) if grid == GRID_TERNARY else \
            level_value(c, CODE_BITS[grid]).astype(np.float64)
        q = s_full[:, j].astype(np.float64) * v
        err = (w[:, j] - q) / U[j, j]
        w[:, j + 1:] -= np.outer(err, U[j, j + 1:])
    codes = codes.astype(np.uint8)
    return scales, codes, _logits_from_codes(codes, W, grid, init_logit), targets


# ----------------------------------------------------------------------------
# Noise
# ----------------------------------------------------------------------------

def noise(grid: int, rows: int, cols: int, seed: int, stream: int, step: int,
          row0: int = 0) -> np.ndarray:
    """Noise of every logit of rows [row0, row0+rows), shape [L, rows, cols].

    Coordinate i = (row0 + r)*cols + j draws the L consecutive stream elements
    e = i*L + k, k = 0..L-1. 2-bit and local shift turn each uniform into a
    standard Gumbel; ternary turns each into a standard logistic (one for the
    mask, k = 0, one for the sign, k = 1).
    """
    L = N_LOGITS[grid]
    i = (np.arange(rows, dtype=np.int64)[:, None] + row0) * cols \
        + np.arange(cols, dtype=np.int64)[None, :]
    e = i[None, :, :] * L + np.arange(L, dtype=np.int64)[:, None, None]
    u = uniform_from_word(noise_words(seed, stream, step, e))
    return logistic(u) if grid == GRID_TERNARY else gumbel(u)


# ----------------------------------------------------------------------------
# Relaxation
# ----------------------------------------------------------------------------

def _sigmoid(z):
    return 0.5 * (1.0 + np.tanh(0.5 * z))


def ternary_terms(logits, seed: int, stream: int, step: int, tau: float,
                  noise_scale: float, row0: int = 0):
    """Relaxed mask and sign of the ternary grid, with exact complements.

    z_m = (l_m + eta*n_m)/tau, z_s = (l_s + eta*n_s)/tau; returns
    a = sigmoid(z_m), 1 - a = sigmoid(-z_m), 2b - 1 = tanh(z_s/2) and
    b(1 - b) = sigmoid(z_s)*sigmoid(-z_s) (the same quantities, formed without
    cancellation).
    """
    lg = np.asarray(logits, dtype=np.float64)
    _, rows, cols = lg.shape
    n = noise(GRID_TERNARY, rows, cols, seed, stream, step, row0)
    z = (lg + float(noise_scale) * n) / float(tau)
    return (_sigmoid(z[0]), _sigmoid(-z[0]), np.tanh(0.5 * z[1]),
            _sigmoid(z[1]) * _sigmoid(-z[1]))


def relax_probs(logits, grid: int, seed: int, stream: int, step: int,
                tau: float, noise_scale: float, row0: int = 0):
    """Gumbel-Softmax probabilities at temperature tau.

    2-bit / 3-bit / local shift: p = softmax((l + eta*g)/tau) over the L logits.
    Ternary: a = sigmoid((l_m + eta*n_m)/tau) (mask on),
    b = sigmoid((l_s + eta*n_s)/tau) (sign positive).
    """
    lg = np.asarray(logits, dtype=np.float64)
    L, rows, cols = lg.shape
    n = noise(grid, rows, cols, seed, stream, step, row0)
    z = (lg + float(noise_scale) * n) / float(tau)
    if grid == GRID_TERNARY:
        return _sigmoid(z[0]), _sigmoid(z[1])
    z = z - z.max(axis=0, keepdims=True)
    ez = np.exp(z)
    return ez / ez.sum(axis=0, keepdims=True)


def _values(grid: int, init_codes, shape):
    if grid in (GRID_INT2, GRID_INT3):
        L, bits = N_LOGITS[grid], CODE_BITS[grid]
        return level_value(np.arange(L), bits).astype(np.float64).reshape(L, 1, 1) \
            * np.ones((1,) + tuple(shape))
    return level_value(candidate_codes(grid, init_codes), 3).astype(np.float64)


def relax_fwd(logits, scales, W, grid: int, seed: int, stream: int, step: int,
              tau: float, noise_scale: float = 1.0, init_codes=None,
              row0: int = 0, group: int = 128):
    """Soft weights and the difference to the original layer.

    w_hat = sum_k p_k v_k (2-bit, local shift) or a*(2b - 1) (ternary, the
    relaxed mask times the relaxed sign); w_soft = s_g * w_hat; dW = w_soft - W.
    Returns a dict with ``w_hat``, ``w_soft`` and ``dW`` (fp64, [rows, cols]).
    """
    lg = np.asarray(logits)
    _, rows, cols = lg.shape
    s = np.repeat(np.asarray(scales, dtype=np.float64), group, axis=1)
    if grid == GRID_TERNARY:
        a, _, sgn, _ = ternary_terms(lg, seed, stream, step, tau, noise_scale, row0)
        w_hat = a * sgn
    else:
        p = relax_probs(lg, grid, seed, stream, step, tau, noise_scale, row0)
        w_hat = (p * _values(grid, init_codes, (rows, cols))).sum(axis=0)
    w_soft = s * w_hat
    return {"w_hat": w_hat, "w_soft": w_soft,
            "dW": w_soft - np.asarray(W, dtype=np.float64)}


def relax_bwd(G, logits, scales, grid: int, seed: int, stream: int, step: int,
              tau: float, noise_scale: float = 1.0, init_codes=None,
              row0: int = 0, group: int = 128):
    """Gradients of the loss with respect to the logits and the group scales.

    G is dLoss/dw_soft (equal to dLoss/d(dW), W being constant). With the
    softmax Jacobian dp_j/dz_k = p_j(delta_jk - p_k) and dz/dl = 1/tau:
      2-bit / local shift: dL/dl_k = G * s * p_k * (v_k - w_hat) / tau;
      ternary: dL/dl_m = G * s * a(1-a) * (2b-1) / tau,
               dL/dl_s = G * s * a * 2 b(1-b) / tau;
      scales:  dL/ds_g = sum over the group of G * w_hat.
    Returns ``(grad_logits [L, rows, cols], grad_scales [rows, cols/group])``.
    """
    lg = np.asarray(logits)
    L, rows, cols = lg.shape
    Gd = np.asarray(G, dtype=np.float64)
    s = np.repeat(np.asarray(scales, dtype=np.float64), group, axis=1)
    tau = float(tau)
    if grid == GRID_TERNARY:
        a, abar, sgn, bb = ternary_terms(lg, seed, stream, step, tau,
                                         noise_scale, row0)
        w_hat = a * sgn
        gl = np.stack([Gd * s * a * abar * sgn / tau,
                       Gd * s * a * 2.0 * bb / tau])
    else:
        p = relax_probs(lg, grid, seed, stream, step, tau, noise_scale, row0)
        v = _values(grid, init_codes, (rows, cols))
        w_hat = (p * v).sum(axis=0)
        gl = Gd[None] * s[None] * p * (v - w_hat[None]) / tau
    gs = (Gd * w_hat).reshape(rows, cols // group, group).sum(axis=2)
    return gl, gs


# ----------------------------------------------------------------------------
# Reconstruction objective
# ----------------------------------------------------------------------------

def recon_loss_grad(X, dW):
    """Output reconstruction error of one layer and its gradient.

    R = X dW^T (tokens x out), loss = sum R^2 = ||X W_soft^T - X W^T||_F^2 and
    G = dLoss/d(dW) = 2 R^T X. Plain fp64 matrix products. Returns
    ``(RT [out, tokens], loss, G [out, in])``.
    """
    Xd = np.asarray(X, dtype=np.float64)
    D = np.asarray(dW, dtype=np.float64)
    RT = D @ Xd.T
    return RT, float(np.sum(RT * RT)), 2.0 * (RT @ Xd)


def recon_loss_grad_offset(X, dW, E0T):
    """The reconstruction objective with a fixed offset on the residual.

    R = X dW^T + E0 (E0 fixed, given transposed as ``E0T`` [out, tokens]),
    loss = sum R^2, G = dLoss/d(dW) = 2 R^T X. With E0 = X_q W^T - Y_target
    (the layer's full-precision output on quantized inputs minus the output
    the stage should reproduce) this is ||X_q W_soft^T - Y_target||^2: a
    layer fitted to a target downstream of itself, the block output for the
    MLP and the attention output for the value/output stage (agihunt.info,
    optimizer paragraph on the staged schedule). Returns ``(RT, loss, G)``.
    """
    Xd = np.asarray(X, dtype=np.float64)
    RT = np.asarray(dW, dtype=np.float64) @ Xd.T + np.asarray(E0T, dtype=np.float64)
    return RT, float(np.sum(RT * RT)), 2.0 * (RT @ Xd)


def recon_loss_grad_grouped(X_cat, tok_offsets, dW_cat, rows_per_expert: int):
    """Sum over experts of the per-expert reconstruction objective.

    Expert e owns rows [e*rows_per_expert, (e+1)*rows_per_expert) of dW and
    tokens [tok_offsets[e], tok_offsets[e+1]) of X. Returns ``(RT blocks list,
    loss, G)`` with G stacked like dW.
    """
    D = np.asarray(dW_cat, dtype=np.float64)
    Xd = np.asarray(X_cat, dtype=np.float64)
    E = len(tok_offsets) - 1
    G = np.zeros_like(D)
    loss = 0.0
    RTs = []
    for e in range(E):
        r = slice(e * rows_per_expert, (e + 1) * rows_per_expert)
        RT, l, Ge = recon_loss_grad(Xd[tok_offsets[e]:tok_offsets[e + 1]], D[r])
        RTs.append(RT)
        loss += l
        G[r] = Ge
    return RTs, loss, G


def gram(X, bf16: bool = False) -> np.ndarray:
    """Gram matrix H = X^T X of the calibration tokens ([in, in], fp64).

    The reconstruction objective is a quadratic form in dW: ||X dW^T||_F^2 =
    tr(dW X^T X dW^T), so H holds everything the objective needs from X
    (agihunt.info, method paragraph: the objective is the output
    reconstruction error). With ``bf16`` the result is rounded to bfloat16, as
    the GPU stores it.
    """
    Xd = np.asarray(X, dtype=np.float64)
    H = Xd.T @ Xd
    return round_bf16(H).astype(np.float64) if bf16 else H


def recon_loss_grad_gram(dW, H):
    """The reconstruction objective and its gradient in Gram form.

    With P = dW H: loss = sum(dW * P) = tr(dW H dW^T) and G = 2 P, equal to
    :func:`recon_loss_grad` when H = X^T X. One product of 2*out*in*in flops
    instead of two of 2*out*tokens*in. Returns ``(loss, G)``.
    """
    D = np.asarray(dW, dtype=np.float64)
    P = D @ np.asarray(H, dtype=np.float64)
    return float(np.sum(D * P)), 2.0 * P


def hard_loss(codes, scales, W, X, grid: int, group: int = 128) -> float:
    """Reconstruction error of a hard assignment: ||X (s*v(codes) - W)^T||^2.

    ``codes`` are stored codes (ternary: t + 1).
    """
    c = np.asarray(codes, dtype=np.int64)
    if grid == GRID_TERNARY:
        v = (c - 1).astype(np.float64)
    else:
        v = level_value(c, CODE_BITS[grid]).astype(np.float64)
    s = np.repeat(np.asarray(scales, dtype=np.float64), group, axis=1)
    _, loss, _ = recon_loss_grad(X, s * v - np.asarray(W, dtype=np.float64))
    return loss


# ----------------------------------------------------------------------------
# Lion
# ----------------------------------------------------------------------------

def lion(theta, grad, mom, lr: float, beta1: float, beta2: float,
         weight_decay: float = 0.0):
    """One Lion update (Chen et al., "Symbolic Discovery of Optimization
    Algorithms", 2023), the optimizer the pages choose for the logits.

    c = beta1*m + (1-beta1)*g;  theta <- theta - lr*(sign(c) + wd*theta);
    m <- beta2*m + (1-beta2)*g.

    theta and mom are fp32 state; hyper-parameters are fp32 values. The sign
    decision is taken on c as an fp32 kernel forms it: t = fp32((1-beta1)*g),
    then the exact value beta1*m + t (one fused multiply-add; its rounding
    cannot change the sign). theta and m are then formed in fp64 and stored
    rounded to fp32. Returns ``(theta', m')`` as fp32 arrays.
    """
    th = np.asarray(theta, dtype=np.float32).astype(np.float64)
    m = np.asarray(mom, dtype=np.float32).astype(np.float64)
    g = np.asarray(grad, dtype=np.float64)
    b1 = np.float32(beta1)
    b2 = np.float32(beta2)
    omb1 = np.float32(np.float32(1.0) - b1)
    omb2 = np.float32(np.float32(1.0) - b2)
    t = (float(omb1) * g).astype(np.float32).astype(np.float64)
    c = float(b1) * m + t
    sgn = np.sign(c)
    lr = float(np.float32(lr))
    wd = float(np.float32(weight_decay))
    th_new = th - lr * (sgn + wd * th)
    m_new = float(b2) * m + float(omb2) * g
    return th_new.astype(np.float32), m_new.astype(np.float32)


# ----------------------------------------------------------------------------
# Hardening and packing
# ----------------------------------------------------------------------------

def harden(logits, grid: int, init_codes=None) -> np.ndarray:
    """Noise-free hard codes after annealing (stored form, uint8).

    2-bit / full 3-bit: argmax of the logits (first index on ties). Local
    shift: clamp(c0 + argmax - 2, 0, 7). Ternary: t = [l_m >= 0] * (+1 if
    l_s >= 0 else -1), stored as t + 1.
    """
    lg = np.asarray(logits, dtype=np.float32)
    if grid == GRID_TERNARY:
        t = np.where(lg[0] >= 0, np.where(lg[1] >= 0, 1, -1), 0)
        return (t + 1).astype(np.uint8)
    k = np.argmax(lg, axis=0)
    if grid in (GRID_INT2, GRID_INT3):
        return k.astype(np.uint8)
    c0 = np.asarray(init_codes, dtype=np.int64)
    return np.clip(c0 + k - 2, 0, 7).astype(np.uint8)


def pack_codes(codes, bits: int) -> np.ndarray:
    """Pack each row into a little-endian, LSB-first bit-stream of uint32.

    Code j of a row occupies bits [bits*j, bits*j + bits) of that row's
    stream; the row takes cols*bits/32 words.
    """
    c = np.asarray(codes, dtype=np.uint8)
    M, K = c.shape
    if (K * bits) % 32:
        raise ValueError("row does not fill whole words")
    bitplanes = ((c[:, :, None] >> np.arange(bits, dtype=np.uint8)) & 1).astype(np.uint8)
    stream = bitplanes.reshape(M, K * bits)
    by = np.packbits(stream, axis=1, bitorder="little")
    return by.view("<u4").reshape(M, K * bits // 32).astype(np.uint32)


def unpack_codes(packed, cols: int, bits: int) -> np.ndarray:
    """Inverse of :func:`pack_codes`."""
    p = np.ascontiguousarray(np.asarray(packed, dtype="<u4"))
    M = p.shape[0]
    by = p.view(np.uint8).reshape(M, -1)
    stream = np.unpackbits(by, axis=1, bitorder="little")[:, :cols * bits]
    planes = stream.reshape(M, cols, bits).astype(np.uint8)
    return (planes << np.arange(bits, dtype=np.uint8)).sum(axis=2).astype(np.uint8)


def scales_to_f16_bits(scales) -> np.ndarray:
    """fp32 scales to IEEE half, round to nearest even; returns the bit pattern."""
    return np.asarray(scales, dtype=np.float32).astype(np.float16).view(np.uint16)


def harden_pack(logits, scales, grid: int, init_codes=None):
    """Codes, packed codes and fp16 scales of the hardened layer.

    Rows whose bits do not fill whole 32-bit words (tiny test layers) get no
    packed form (``None``).
    """
    codes = harden(logits, grid, init_codes)
    bits = CODE_BITS[grid]
    packed = pack_codes(codes, bits) if (codes.shape[1] * bits) % 32 == 0 else None
    return codes, packed, scales_to_f16_bits(scales)


# ----------------------------------------------------------------------------
# Temperature schedule and the whole per-layer solve
# ----------------------------------------------------------------------------

def tau_schedule(steps: int, tau0: float = 1.0, tau1: float = 0.05) -> np.ndarray:
    """Geometric annealing tau_t = tau0 * (tau1/tau0)**(t/(T-1)), as fp32."""
    if steps == 1:
        return np.array([tau0], dtype=np.float32)
    t = np.arange(steps, dtype=np.float64) / (steps - 1)
    return (tau0 * (tau1 / tau0) ** t).astype(np.float32)


def round_bf16(x) -> np.ndarray:
    """fp32 value rounded to bfloat16 (nearest, ties to even), returned as fp32."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1)))
         >> np.uint64(16)) << np.uint64(16)
    return r.astype(np.uint32).view(np.float32)


def step(state: dict, W, X, grid: int, t: int, tau: float, seed: int,
         stream: int, lr_logit: float, lr_scale: float, beta1: float = 0.9,
         beta2: float = 0.99, weight_decay: float = 0.0,
         noise_scale: float = 1.0, bf16_dW: bool = False, group: int = 128,
         bf16_RT: bool = False, H=None, row0: int = 0, E0T=None):
    """One full relaxed-quantization step on a whole layer, in place on
    ``state`` (``logits``, ``mom``, ``scales``, ``scale_mom``, ``codes``).
    ``row0`` places the rows given at that row of a larger layer (it only
    moves the noise counters; rows are independent in the objective).

    Forward relaxation, reconstruction loss and gradient, backward to the
    logits and scales, Lion on both. ``bf16_dW`` rounds dW to bfloat16 before
    the products and ``bf16_RT`` rounds R^T to bfloat16 before forming G, as
    a bf16 matrix engine consumes them (the loss stays the exact sum of R^2).
    With a Gram matrix ``H`` (see :func:`gram`) the objective is taken in Gram
    form instead and X is not used; with ``E0T`` the residual carries that
    fixed offset (:func:`recon_loss_grad_offset`). Returns the loss.
    """
    codes = state["codes"] if grid == GRID_INT3_LOCAL else None
    f = relax_fwd(state["logits"], state["scales"], W, grid, seed, stream, t,
                  tau, noise_scale, codes, row0, group)
    dW = round_bf16(f["dW"]).astype(np.float64) if bf16_dW else f["dW"]
    if H is not None:
        loss, G = recon_loss_grad_gram(dW, H)
    else:
        RT, loss, G = (recon_loss_grad(X, dW) if E0T is None
                       else recon_loss_grad_offset(X, dW, E0T))
        if bf16_RT:
            G = 2.0 * (round_bf16(RT).astype(np.float64) @ np.asarray(X, dtype=np.float64))
    gl, gs = relax_bwd(G, state["logits"], state["scales"], grid, seed, stream,
                       t, tau, noise_scale, codes, row0, group)
    state["logits"], state["mom"] = lion(state["logits"], gl, state["mom"],
                                         lr_logit, beta1, beta2, weight_decay)
    state["scales"], state["scale_mom"] = lion(state["scales"], gs,
                                               state["scale_mom"], lr_scale,
                                               beta1, beta2, weight_decay)
    return loss


def quantize_layer(W, X, grid: int, steps: int, seed: int = 0, stream: int = 0,
                   lr_logit: float = 1e-3, lr_scale: float = 1e-5,
                   tau0: float = 1.0, tau1: float = 0.05, init_logit: float = 2.0,
                   beta1: float = 0.9, beta2: float = 0.99,
                   weight_decay: float = 0.0, noise_scale: float = 1.0,
                   bf16_dW: bool = False, group: int = 128):
    """Warm start, ``steps`` annealed relaxation steps, then harden and pack."""
    scales, codes, logits = init_rtn(W, grid, group, init_logit)
    state = {"logits": logits, "mom": np.zeros_like(logits), "scales": scales,
             "scale_mom": np.zeros_like(scales), "codes": codes}
    losses = []
    for t, tau in enumerate(tau_schedule(steps, tau0, tau1)):
        losses.append(step(state, W, X, grid, t, float(tau), seed, stream,
                           lr_logit, lr_scale, beta1, beta2, weight_decay,
                           noise_scale, bf16_dW, group))
    hard, packed, s16 = harden_pack(state["logits"], state["scales"], grid,
                                    state["codes"] if grid == GRID_INT3_LOCAL else None)
    return {"state": state, "losses": np.array(losses), "codes": hard,
            "packed": packed, "scales_f16": s16}
