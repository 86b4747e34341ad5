"""GPU parity of the block forward pieces and the staged schedule.

Each kernel is compared with the oracle on the GPU's own bf16 inputs: fp32
arithmetic against fp64, then one rounding to bf16, so results agree within
one bf16 ulp (exactly for the dequantisation, whose products are exact). The
whole block forward is compared with the oracle's bf16-mirror forward
normwise: a one-ulp difference at any rounding propagates, so the bound is a
few bf16 ulps relative to the tensor's norm.
"""

import numpy as np
import pytest

import oracle
import synthetic
from oracle import block as ob
from tests.gpu_util import device, to_dev_bf16, bf16_values, f32, bf16_ulp, report

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return device()


def _rand_bf16(rng, shape, scale=1.0):
    bits = synthetic.bf16_bits((rng.normal(size=shape) * scale).astype(np.float32))
    return bits, synthetic.bf16_to_f32(bits).astype(np.float64)


def _close_ulp(got, ref, ulps=1):
    assert np.all(np.abs(got - ref) <= ulps * bf16_ulp(ref) + 1e-30)


@pytest.mark.parametrize("I,J,R", [
    (200, 136, 192),       # under half a round: 128-wide tiles throughout
    (4096, 4096, 64),      # exactly one round of 256x256 tiles
    (4000, 5000, 64),      # a column block of whole rounds + a ragged 128-wide tail
    (5000, 4000, 64),      # a row block of whole rounds + a ragged 128-wide tail
])
def test_matmul_nt(dev, I, J, R):
    import torch
    import post_weight_quantization_philox_amd as g
    rng = np.random.default_rng(I + J + R)
    a_bits, A = _rand_bf16(rng, (I, R))
    b_bits, B = _rand_bf16(rng, (J, R))
    C = torch.empty((I, J), dtype=torch.bfloat16, device=dev)
    g.gsq_matmul_nt_bf16(I, J, R, to_dev_bf16(a_bits, dev), R, to_dev_bf16(b_bits, dev), R, C, J)
    torch.cuda.synchronize()
    ref = A @ B.T
    gam = (R + 2) * 2.0 ** -24 * (np.abs(A) @ np.abs(B).T)
    assert np.all(np.abs(bf16_values(C) - ref) <= 0.5 * bf16_ulp(ref) + gam + 1e-30)


def test_matmul_nt_strided_split(dev):
    """Padded leading dimensions on a product split into a row block of whole
    rounds and a 128-wide tail: the tail's operand and output offsets follow
    lda, ldb and ldc, and the padding is neither read into the result nor
    written."""
    import torch
    import post_weight_quantization_philox_amd as g
    rng = np.random.default_rng(11)
    I, J, R, lda, ldb, ldc = 5000, 4000, 64, 72, 80, 4008
    a_bits, A = _rand_bf16(rng, (I, lda))
    b_bits, B = _rand_bf16(rng, (J, ldb))
    C = torch.full((I, ldc), -1.0, dtype=torch.bfloat16, device=dev)
    g.gsq_matmul_nt_bf16(I, J, R, to_dev_bf16(a_bits, dev), lda, to_dev_bf16(b_bits, dev), ldb, C,
                         ldc)
    torch.cuda.synchronize()
    got = bf16_values(C)
    ref = A[:, :R] @ B[:, :R].T
    gam = (R + 2) * 2.0 ** -24 * (np.abs(A[:, :R]) @ np.abs(B[:, :R]).T)
    assert np.all(np.abs(got[:, :J] - ref) <= 0.5 * bf16_ulp(ref) + gam + 1e-30)
    assert np.all(got[:, J:] == -1.0)


def test_rmsnorm_softmax_silu_add(dev):
    import torch
    import post_weight_quantization_philox_amd as g
    rng = np.random.default_rng(1)
    n, d = 64, 384
    xb, x = _rand_bf16(rng, (n, d), 2.0)
    gamma = rng.uniform(0.5, 1.5, d).astype(np.float32)
    y = torch.empty((n, d), dtype=torch.bfloat16, device=dev)
    g.gsq_rmsnorm_bf16(n, d, to_dev_bf16(xb, dev), torch.from_numpy(gamma).to(dev), 1e-5, y)
    sb, S = _rand_bf16(rng, (n, n), 3.0)
    P = torch.empty((n, n), dtype=torch.bfloat16, device=dev)
    g.gsq_softmax_causal_bf16(n, to_dev_bf16(sb, dev), 0.125, P)
    gb, G = _rand_bf16(rng, (n, d), 2.0)
    ub, U = _rand_bf16(rng, (n, d))
    act = torch.empty((n, d), dtype=torch.bfloat16, device=dev)
    g.gsq_silu_mul_bf16(n * d, to_dev_bf16(gb, dev), to_dev_bf16(ub, dev), act)
    s = torch.empty((n, d), dtype=torch.bfloat16, device=dev)
    g.gsq_add_bf16(n * d, to_dev_bf16(xb, dev), to_dev_bf16(gb, dev), s)
    torch.cuda.synchronize()
    _close_ulp(bf16_values(y), ob.rmsnorm(x, gamma.astype(np.float64), 1e-5))
    Pr = ob.softmax_causal(S, 0.125)
    Pg = bf16_values(P)
    assert np.all(np.abs(Pg - Pr) <= bf16_ulp(Pr) + 1e-7)
    assert np.all(Pg[np.triu_indices(n, 1)] == 0)
    _close_ulp(bf16_values(act), ob.silu_mul(G, U))
    _close_ulp(bf16_values(s), x + G)


def test_dequant_bit_exact(dev):
    import torch
    import post_weight_quantization_philox_amd as g
    rng = np.random.default_rng(2)
    M, K = 5, 256
    for grid in (oracle.GRID_INT2, oracle.GRID_TERNARY, oracle.GRID_INT3_LOCAL, oracle.GRID_INT3):
        hi = 3 if grid == oracle.GRID_TERNARY else (4 if grid == oracle.GRID_INT2 else 8)
        codes = rng.integers(0, hi, (M, K)).astype(np.uint8)
        s16 = oracle.scales_to_f16_bits(rng.uniform(1e-3, 0.05, (M, K // 128)).astype(np.float32))
        W = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
        layer = g.GsqLayer.make(grid, M, K)
        g.gsq_dequant_bf16(layer, torch.from_numpy(codes).to(dev),
                           torch.from_numpy(s16.view(np.int16)).to(dev), W)
        torch.cuda.synchronize()
        ref = oracle.round_bf16(ob.dequantize(codes, s16, grid).astype(np.float32))
        np.testing.assert_array_equal(bf16_values(W), ref)


SMALL = dict(hidden=256, heads=2, kv_heads=1, head_dim=128, mlp=512)


def _small_block(dev, n=128, seed=3):
    import torch
    from post_weight_quantization_philox_amd.block import BlockConfig
    cfg = BlockConfig(**SMALL)
    rng = np.random.default_rng(seed)
    w_np, w_dev = {}, {}
    for name, (o, i) in cfg.shapes().items():
        bits, vals = _rand_bf16(rng, (o, i), 1.0 / np.sqrt(i))
        w_np[name], w_dev[name] = vals, to_dev_bf16(bits, dev)
    for name in ("g_attn", "g_mlp"):
        gam = rng.uniform(0.8, 1.2, cfg.hidden).astype(np.float32)
        w_np[name], w_dev[name] = gam.astype(np.float64), torch.from_numpy(gam).to(dev)
    xb, x = _rand_bf16(rng, (n, cfg.hidden))
    return cfg, w_np, w_dev, x, to_dev_bf16(xb, dev)


def _nrm(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def test_block_forward_matches_mirror(dev):
    import torch
    from post_weight_quantization_philox_amd.block import forward
    cfg, w_np, w_dev, x, xd = _small_block(dev)
    out = forward(cfg, w_dev, xd)
    torch.cuda.synchronize()
    ref = ob.block_forward_mirror(x, w_np, SMALL)
    exact = ob.block_forward(x, w_np, SMALL)
    errs = {k: _nrm(bf16_values(out[k]).astype(np.float64), ref[k])
            for k in ("x_attn", "x_o", "h", "x_mlp", "x_down", "out")}
    report("block forward vs bf16 mirror", **errs,
           out_vs_fp64=_nrm(bf16_values(out["out"]).astype(np.float64), exact["out"]))
    for k, e in errs.items():
        assert e <= 4 * 2.0 ** -8, k


@pytest.mark.parametrize("recon,objective", [("direct", "block"), ("gram", "block"),
                                             ("direct", "layer"), ("gram", "layer")])
def test_staged_schedule(dev, recon, objective):
    """The staged schedule on a small block, with the layers on the direct
    products or on the Gram form, each fitted to its own output (``layer``)
    or, for the output and down projections, to the full-precision block
    (``block``): each stage's calibration inputs equal the oracle's mirror
    forward with the GPU's quantized weights of the earlier stages, every
    projection ends quantized (dequantised values on the grid), the offsets
    equal the oracle's, and the quantized block's output error is reported
    against the round-to-nearest block."""
    import torch
    import post_weight_quantization_philox_amd as g
    from post_weight_quantization_philox_amd.block import forward, staged_quantize
    cfg, w_np, w_dev, x, xd = _small_block(dev, seed=4)
    wq, info = staged_quantize(cfg, w_dev, xd, oracle.GRID_INT2, 24,
                               g.GsqLion.make(lr_logit=5e-2, lr_scale=1e-6), recon=recon,
                               objective=objective)
    forms = {k: f for v in info.values() for k, f in v["recon"].items()}
    fitted = {"o", "down"} if objective == "block" else set()
    assert all(f == ("direct+offset" if k in fitted else recon) for k, f in forms.items())
    wq_np = dict(w_np)
    for name in ("q", "k", "v", "o", "gate", "up", "down"):
        wq_np[name] = bf16_values(wq[name]).astype(np.float64)
        # every row is s * {-3,-1,1,3} per group: at most 4 distinct magnitudes... per group
        vals = wq_np[name].reshape(wq_np[name].shape[0], -1, 128)
        assert max(len(np.unique(vals[r, gi])) for r in range(2) for gi in range(vals.shape[1])) <= 4
    # stage inputs: mlp stage's down input from the GPU equals the mirror
    # forward with the GPU's quantized q, k, v, o, gate, up
    wm = dict(wq_np, down=w_np["down"])
    ref = ob.block_forward_mirror(x, wm, SMALL)
    got = bf16_values(info["mlp"]["x"]).astype(np.float64)
    e_in = _nrm(got, ref["x_down"])
    xo_ref = ob.block_forward_mirror(x, dict(wq_np, o=w_np["o"], gate=w_np["gate"], up=w_np["up"],
                                             down=w_np["down"]), SMALL)["x_o"]
    e_xo = _nrm(bf16_values(info["v_o"]["x"]).astype(np.float64), xo_ref)
    # quality against round-to-nearest of every projection (report only: random weights)
    w_rtn = dict(w_np)
    for name in ("q", "k", "v", "o", "gate", "up", "down"):
        s, c, _ = oracle.init_rtn(w_np[name].astype(np.float32), oracle.GRID_INT2)
        w_rtn[name] = ob.dequantize(c, oracle.scales_to_f16_bits(s), oracle.GRID_INT2)
    full = ob.block_forward(x, w_np, SMALL)["out"]
    e_gsq = _nrm(ob.block_forward(x, wq_np, SMALL)["out"], full)
    e_rtn = _nrm(ob.block_forward(x, w_rtn, SMALL)["out"], full)
    extra = {}
    if objective == "block":
        # The offsets against the oracle's, each from the mirror forward with
        # the GPU's quantized earlier stages and the full-precision block.
        fp = ob.block_forward_mirror(x, w_np, SMALL)
        fo = ob.block_forward_mirror(x, dict(wq_np, o=w_np["o"], gate=w_np["gate"],
                                             up=w_np["up"], down=w_np["down"]), SMALL)
        e0o = ob.stage_offset_T(w_np["o"], fo["x_o"], fp["x_o"], mirror=True)
        got_o = bf16_values(info["v_o"]["offset_T"]).astype(np.float64)
        fd = ob.block_forward_mirror(x, dict(wq_np, down=w_np["down"]), SMALL)
        e0d = ob.stage_offset_T(w_np["down"], fd["x_down"], fp["x_down"], fd["h"], fp["h"],
                                mirror=True)
        got_d = bf16_values(info["mlp"]["offset_T"]).astype(np.float64)
        extra = {"offset_o_vs_mirror": _nrm(got_o, e0o), "offset_down_vs_mirror": _nrm(got_d, e0d)}
        # The down stage's objective at the hard result is the block output
        # error: act_q (W_q - W)^T + E0 equals out_q - out_fp.
        act = bf16_values(info["mlp"]["x"]).astype(np.float64)
        R = act @ (wq_np["down"] - w_np["down"]).T + got_d.T
        want = ob.block_forward_mirror(x, wq_np, SMALL)["out"] - fp["out"]
        extra["down_objective_vs_block_error"] = _nrm(R, want)
        # Offsets are differences of near-equal activations, rounded once
        # more than the activations themselves, so the bar is relative to
        # their own (small) norm: 8 bf16 ulps.
        assert extra["offset_o_vs_mirror"] <= 8 * 2.0 ** -8
        assert extra["offset_down_vs_mirror"] <= 8 * 2.0 ** -8
        assert extra["down_objective_vs_block_error"] <= 8 * 2.0 ** -8
    report(f"staged schedule ({recon}, {objective})", x_down_vs_mirror=e_in, x_o_vs_mirror=e_xo,
           out_err_gsq=e_gsq, out_err_rtn=e_rtn, **extra,
           **{f"{k}_s": v["seconds"] for k, v in info.items()})
    assert e_in <= 4 * 2.0 ** -8 and e_xo <= 4 * 2.0 ** -8
