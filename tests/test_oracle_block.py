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
