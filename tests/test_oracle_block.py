"""Pins of the block oracle: closed forms and library routines for each
piece, and the block's residual structure."""

import numpy as np

from oracle import block as ob
import oracle


def test_rmsnorm_closed_forms():
    x = np.array([[3.0, 4.0], [1.0, -1.0]])
    y = ob.rmsnorm(x, np.ones(2), eps=0.0)
    np.testing.assert_allclose(y, [[3 / np.sqrt(12.5), 4 / np.sqrt(12.5)], [1.0, -1.0]], rtol=1e-15)
    g = np.array([2.0, 0.5])
    np.testing.assert_allclose(ob.rmsnorm(x, g, eps=0.0), y * g, rtol=1e-15)
    assert np.allclose(np.mean(ob.rmsnorm(np.random.default_rng(0).normal(size=(5, 64)), np.ones(64), 0.0) ** 2, axis=1), 1.0)


def test_softmax_causal_rows():
    rng = np.random.default_rng(1)
    S = rng.normal(size=(6, 6))
    P = ob.softmax_causal(S, 0.7)
    np.testing.assert_allclose(P.sum(axis=1), 1.0, rtol=1e-14)
    assert np.all(np.triu(P, 1) == 0)
    assert P[0, 0] == 1.0
    i = 4
    e = np.exp(0.7 * S[i, :i + 1])
    np.testing.assert_allclose(P[i, :i + 1], e / e.sum(), rtol=1e-14)


def test_silu_mul_closed_form():
    g = np.array([0.0, 1.0, -2.0])
    u = np.array([5.0, 2.0, 3.0])
    np.testing.assert_allclose(ob.silu_mul(g, u), [0.0, 2.0 / (1 + np.exp(-1.0)), -6.0 / (1 + np.exp(2.0))], rtol=1e-15)


def test_attention_single_head_by_hand():
    rng = np.random.default_rng(2)
    n, d = 5, 4
    xn = rng.normal(size=(n, d))
    Wq, Wk, Wv = rng.normal(size=(d, d)), rng.normal(size=(d, d)), rng.normal(size=(d, d))
    out = ob.attention(xn, Wq, Wk, Wv, 1, 1, d)
    Q, K, V = xn @ Wq.T, xn @ Wk.T, xn @ Wv.T
    for i in range(n):
        s = np.array([Q[i] @ K[j] for j in range(i + 1)]) / np.sqrt(d)
        p = np.exp(s - s.max())
        p /= p.sum()
        np.testing.assert_allclose(out[i], p @ V[:i + 1], rtol=1e-12)


def test_grouped_heads_share_key_value():
    # two query heads over one key/value head equal two single-head blocks
    rng = np.random.default_rng(3)
    n, d, hd = 6, 8, 4
    xn = rng.normal(size=(n, d))
    Wq, Wk, Wv = rng.normal(size=(2 * hd, d)), rng.normal(size=(hd, d)), rng.normal(size=(hd, d))
    out = ob.attention(xn, Wq, Wk, Wv, 2, 1, hd)
    for h in range(2):
        one = ob.attention(xn, Wq[h * hd:(h + 1) * hd], Wk, Wv, 1, 1, hd)
        np.testing.assert_allclose(out[:, h * hd:(h + 1) * hd], one, rtol=1e-12)


def test_block_residuals_and_zero_weights():
    rng = np.random.default_rng(4)
    cfg = {"heads": 2, "kv_heads": 1, "head_dim": 4}
    n, d, m = 6, 8, 16
    shp = {"q": (8, d), "k": (4, d), "v": (4, d), "o": (d, 8), "gate": (m, d), "up": (m, d), "down": (d, m)}
    w = {k: rng.normal(size=s) for k, s in shp.items()}
    w["g_attn"], w["g_mlp"] = np.ones(d), np.ones(d)
    x = rng.normal(size=(n, d))
    r = ob.block_forward(x, w, cfg)
    np.testing.assert_allclose(r["out"], x + r["x_o"] @ w["o"].T + r["x_down"] @ w["down"].T, rtol=1e-12)
    w0 = dict(w, o=np.zeros_like(w["o"]), down=np.zeros_like(w["down"]))
    np.testing.assert_allclose(ob.block_forward(x, w0, cfg)["out"], x, rtol=0, atol=0)


def test_dequantize_levels():
    s16 = oracle.scales_to_f16_bits(np.array([[0.5], [0.25]], dtype=np.float32))
    codes = np.tile(np.array([0, 1, 2, 3], dtype=np.uint8), (2, 32))
    Wq = ob.dequantize(codes, s16, oracle.GRID_INT2)
    np.testing.assert_array_equal(Wq[0, :4], [-1.5, -0.5, 0.5, 1.5])
    np.testing.assert_array_equal(Wq[1, :4], [-0.75, -0.25, 0.25, 0.75])
    tc = np.array(([0, 1, 2] * 43)[:128], dtype=np.uint8).reshape(1, 128)
    t = ob.dequantize(tc, s16[:1], oracle.GRID_TERNARY)
    np.testing.assert_array_equal(t[0, :3], [-0.5, 0.0, 0.5])


def _block_case(seed, n=24, d=32, heads=4, kv_heads=2, hd=8, m=48, bf16=True):
    """A small block with grouped heads (2 query heads per key/value head),
    non-unit norm gains and, optionally, bf16-valued weights and tokens."""
    rng = np.random.default_rng(seed)
    cfg = {"heads": heads, "kv_heads": kv_heads, "head_dim": hd}
    shp = {"q": (heads * hd, d), "k": (kv_heads * hd, d), "v": (kv_heads * hd, d),
           "o": (d, heads * hd), "gate": (m, d), "up": (m, d), "down": (d, m)}
    rb = (lambda a: oracle.round_bf16(a.astype(np.float32)).astype(np.float64)) if bf16 else (lambda a: a)
    w = {k: rb(rng.normal(0, 1 / np.sqrt(s[1]), size=s)) for k, s in shp.items()}
    w["g_attn"] = rng.uniform(0.8, 1.2, d)
    w["g_mlp"] = rng.uniform(0.8, 1.2, d)
    return cfg, w, rb(rng.normal(size=(n, d)))


KEYS = ("x_attn", "x_o", "h", "x_mlp", "x_down", "out")


def test_mirror_without_rounding_is_the_forward(monkeypatch):
    """With its bfloat16 roundings switched off, the mirror forward is the
    exact forward: the same heads read the same key/value group, the same
    causal mask, norms, SwiGLU and residuals (a slip in any of them in the
    mirror's own inline attention shows here at fp64 precision)."""
    cfg, w, x = _block_case(5, bf16=False)
    ref = ob.block_forward(x, w, cfg)
    monkeypatch.setattr(ob, "_rb", lambda a: np.asarray(a, dtype=np.float64))
    got = ob.block_forward_mirror(x, w, cfg)
    for k in KEYS:
        np.testing.assert_allclose(got[k], ref[k], rtol=1e-12, atol=1e-12, err_msg=k)


def test_mirror_head_outputs_equal_attention(monkeypatch):
    """Each head of the mirror's attention output equals the pinned
    :func:`attention` of that head alone (rounding off)."""
    cfg, w, x = _block_case(6, bf16=False)
    monkeypatch.setattr(ob, "_rb", lambda a: np.asarray(a, dtype=np.float64))
    ao = ob.block_forward_mirror(x, w, cfg)["x_o"]
    xa = ob.rmsnorm(x, w["g_attn"])
    hd, group = cfg["head_dim"], cfg["heads"] // cfg["kv_heads"]
    for h in range(cfg["heads"]):
        g = h // group
        one = ob.attention(xa, w["q"][h * hd:(h + 1) * hd], w["k"][g * hd:(g + 1) * hd],
                           w["v"][g * hd:(g + 1) * hd], 1, 1, hd)
        np.testing.assert_allclose(ao[:, h * hd:(h + 1) * hd], one, rtol=1e-12, atol=1e-12)


def test_mirror_close_to_exact_forward():
    """With the roundings on, every intermediate of the mirror stays within
    four bfloat16 ulps (2^-6) of the exact forward, normwise."""
    for seed in (7, 8):
        cfg, w, x = _block_case(seed)
        ref = ob.block_forward(x, w, cfg)
        got = ob.block_forward_mirror(x, w, cfg)
        for k in KEYS:
            e = np.linalg.norm(got[k] - ref[k]) / np.linalg.norm(ref[k])
            assert 0 < e <= 2.0 ** -6, (k, e)


def _perturbed(w, seed, scale=0.05):
    rng = np.random.default_rng(seed)
    return {k: (v + scale * np.abs(v).mean() * rng.normal(size=v.shape)
                if k in ("q", "k", "v", "o", "gate", "up", "down") else v) for k, v in w.items()}


def test_output_projection_offset_is_attention_output_error():
    """With the offset, the output projection's objective on the quantized
    attention output is the error of the block's residual stream after
    attention against the full-precision block: ||h_q - h_fp||^2."""
    cfg, w, x = _block_case(10, bf16=False)
    wq = _perturbed(w, 11)
    fp = ob.block_forward(x, w, cfg)
    fq = ob.block_forward(x, dict(wq, o=w["o"]), cfg)        # q, k, v quantized
    E0T = ob.stage_offset_T(w["o"], fq["x_o"], fp["x_o"])
    _, loss, _ = oracle.recon_loss_grad_offset(fq["x_o"], wq["o"] - w["o"], E0T)
    h_q = ob.block_forward(x, wq, cfg)["h"]
    want = float(np.sum((h_q - fp["h"]) ** 2))
    assert abs(loss - want) <= 1e-10 * want


def test_down_projection_offset_is_block_output_error():
    """With the offset, the down projection's objective on the quantized
    SwiGLU activations is the block output error against the full-precision
    block, ||out_q - out_fp||^2 (the MLP fitted on the block output)."""
    cfg, w, x = _block_case(12, bf16=False)
    wq = _perturbed(w, 13)
    fp = ob.block_forward(x, w, cfg)
    fq = ob.block_forward(x, dict(wq, down=w["down"]), cfg)
    E0T = ob.stage_offset_T(w["down"], fq["x_down"], fp["x_down"], fq["h"], fp["h"])
    RT, loss, _ = oracle.recon_loss_grad_offset(fq["x_down"], wq["down"] - w["down"], E0T)
    out_q = ob.block_forward(x, wq, cfg)["out"]
    np.testing.assert_allclose(RT.T, out_q - fp["out"], rtol=1e-9, atol=1e-12)
    assert abs(loss - float(np.sum((out_q - fp["out"]) ** 2))) <= 1e-10 * loss
    # without a quantized earlier stage and with dW = 0 the objective vanishes
    E0_same = ob.stage_offset_T(w["down"], fp["x_down"], fp["x_down"], fp["h"], fp["h"])
    assert not np.any(E0_same)


def test_stage_offset_mirror_rounds_like_the_exact_offset():
    cfg, w, x = _block_case(14)
    wq = _perturbed(w, 15)
    fp = ob.block_forward(x, w, cfg)
    fq = ob.block_forward(x, dict(wq, down=w["down"]), cfg)
    ex = ob.stage_offset_T(w["down"], fq["x_down"], fp["x_down"], fq["h"], fp["h"])
    mi = ob.stage_offset_T(w["down"], fq["x_down"], fp["x_down"], fq["h"], fp["h"], mirror=True)
    assert 0 < np.linalg.norm(mi - ex) / np.linalg.norm(ex) <= 2.0 ** -6
