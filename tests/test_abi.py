"""The C ABI on the CPU: the library loads, exports every entry point the
header declares, and rejects bad arguments before touching a device (every
call here fails validation, so no kernel is launched)."""

import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

g = pytest.importorskip("post_weight_quantization_philox_amd")

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_GRID, ERR_PARAM = 0, 1, 2, 3, 4, 5
FAKE = 0x10000          # an aligned address that is never dereferenced
FAKE_MISALIGNED = 0x10004


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(g.LIB_PATH):
        pytest.fail("libgsq.so is not built (python -m post_weight_quantization_philox_amd.build)")
    return g.lib()


def header_functions():
    src = open(os.path.join(ROOT, "include", "gsq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gsq_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_entry_point(L):
    declared = header_functions()
    assert len(declared) >= 11
    for name in declared:
        assert hasattr(L, name), name
    assert sorted(g.EXPORTS) == declared


def test_version_and_names(L):
    assert g.gsq_abi_version() == 1
    assert g.gsq_status_str(0) == "GSQ_OK"
    assert g.gsq_status_str(3) == "GSQ_ERR_ALIGN"
    assert [g.gsq_num_logits(k) for k in (0, 1, 2, 7)] == [4, 2, 5, 0]


def _fwd(layer, **kw):
    args = dict(logits=FAKE, scales=FAKE, codes=FAKE, W=FAKE, step=0, tau=1.0, eta=1.0, dW=FAKE,
                dbg=None)
    args.update(kw)
    return g.lib().gsq_relax_fwd(ctypes.byref(layer) if layer is not None else None, args["logits"],
                                 args["scales"], args["codes"], args["W"], args["step"],
                                 args["tau"], args["eta"], args["dW"], args["dbg"], None)


def test_relax_fwd_validation(L):
    lay = g.GsqLayer.make(g.GRID_INT2, 4, 256)
    assert _fwd(None) == ERR_NULL
    assert _fwd(g.GsqLayer.make(9, 4, 256)) == ERR_GRID
    assert _fwd(g.GsqLayer.make(g.GRID_INT2, 4, 200)) == ERR_SHAPE
    assert _fwd(g.GsqLayer.make(g.GRID_INT2, 0, 256)) == ERR_SHAPE
    assert _fwd(g.GsqLayer.make(g.GRID_INT2, 4, 256, group=64)) == ERR_SHAPE
    assert _fwd(g.GsqLayer.make(g.GRID_INT2, 4, 256, w_dtype=5)) == ERR_PARAM
    assert _fwd(lay, logits=None) == ERR_NULL
    assert _fwd(lay, dW=FAKE_MISALIGNED) == ERR_ALIGN
    assert _fwd(lay, dbg=FAKE_MISALIGNED) == ERR_ALIGN
    assert _fwd(lay, tau=0.0) == ERR_PARAM
    assert _fwd(lay, tau=-1.0) == ERR_PARAM
    assert _fwd(lay, tau=float("nan")) == ERR_PARAM
    assert _fwd(lay, tau=float("inf")) == ERR_PARAM
    assert _fwd(lay, eta=1.5) == ERR_PARAM
    assert _fwd(lay, eta=-0.1) == ERR_PARAM
    local = g.GsqLayer.make(g.GRID_INT3_LOCAL, 4, 256)
    assert _fwd(local, codes=None) == ERR_GRID


def test_bwd_lion_validation(L):
    lay = g.GsqLayer.make(g.GRID_TERNARY, 4, 256)
    f = g.lib().gsq_relax_bwd_lion

    def call(lion, gl=None, gs=None, tau=1.0):
        return f(ctypes.byref(lay), FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, tau, 1.0,
                 ctypes.byref(lion) if lion is not None else None, gl, gs, None)

    assert call(None) == ERR_NULL
    assert call(g.GsqLion.make(beta1=1.0)) == ERR_PARAM
    assert call(g.GsqLion.make(beta2=-0.5)) == ERR_PARAM
    assert call(g.GsqLion.make(lr_logit=-1e-3)) == ERR_PARAM
    assert call(g.GsqLion.make(weight_decay=float("nan"))) == ERR_PARAM
    assert call(g.GsqLion.make(), gl=FAKE) == ERR_NULL          # both debug outputs or neither
    assert call(g.GsqLion.make(), tau=0.0) == ERR_PARAM


def test_recon_validation(L):
    f = g.lib().gsq_recon_loss_grad
    offs_bad = np.array([0, 100], dtype=np.int64)        # not a multiple of 64
    offs = np.array([0, 128], dtype=np.int64)
    offs_dec = np.array([0, 128, 64], dtype=np.int64)
    assert f(1, offs_bad.ctypes.data, 64, 256, FAKE, FAKE, FAKE, FAKE, 1 << 20, FAKE, FAKE, FAKE, None) == ERR_SHAPE
    assert f(2, offs_dec.ctypes.data, 64, 256, FAKE, FAKE, FAKE, FAKE, 1 << 20, FAKE, FAKE, FAKE, None) == ERR_SHAPE
    assert f(1, offs.ctypes.data, 64, 200, FAKE, FAKE, FAKE, FAKE, 1 << 20, FAKE, FAKE, FAKE, None) == ERR_SHAPE
    assert f(0, offs.ctypes.data, 64, 256, FAKE, FAKE, FAKE, FAKE, 1 << 20, FAKE, FAKE, FAKE, None) == ERR_SHAPE
    assert f(1, None, 64, 256, FAKE, FAKE, FAKE, FAKE, 1 << 20, FAKE, FAKE, FAKE, None) == ERR_NULL
    assert f(1, offs.ctypes.data, 64, 256, FAKE, FAKE, FAKE, FAKE, 4, FAKE, FAKE, FAKE, None) == ERR_SHAPE
    assert f(1, offs.ctypes.data, 64, 256, FAKE, FAKE, FAKE, FAKE, 1 << 20, FAKE, FAKE_MISALIGNED, FAKE, None) == ERR_ALIGN
    assert f(1, offs.ctypes.data, 64, 256, None, FAKE, FAKE, FAKE, 1 << 20, FAKE, FAKE, FAKE, None) == ERR_NULL
    ws = g.gsq_recon_workspace_bytes(1, offs, 64, 256)
    assert ws >= 4 and ws % 256 == 0
    assert g.gsq_recon_workspace_bytes(1, offs_bad, 64, 256) == 0


def _tiles(n, t):
    return -(-n // t)


def _product_workgroups(I, J):
    """Workgroups of one I x J product (one loss partial each): whole rounds
    of 256 full 256x256 tiles on a column block or a row block, the rest in
    256x128 tiles; under half a round, 256x128 tiles throughout."""
    ti, tj = _tiles(I, 256), _tiles(J, 256)
    T = ti * tj
    if T % 256 == 0:
        return T
    if 2 * T <= 256:
        return ti * _tiles(J, 128)
    n0 = 256 // np.gcd(ti, 256)
    jm = tj // n0 * n0
    if 0 < jm < tj and ti * (tj - jm) * 2 <= 256:
        return ti * jm + ti * _tiles(J - 256 * jm, 128)
    m0 = 256 // np.gcd(tj, 256)
    im = ti // m0 * m0
    if 0 < im < ti and (ti - im) * tj * 2 <= 256:
        return im * tj + (ti - im) * _tiles(J, 128)
    return T


@pytest.mark.parametrize("rows,tokens,want", [
    (4096, 4096, 256),          # one whole round of full tiles
    (1024, 4096, 4 * 32),       # under half a round: 128-wide tiles
    (5000, 4096, 16 * 16 + 4 * 32),    # a row block of whole rounds + tail
    (4000, 5056, 16 * 16 + 16 * 8),    # a column block of whole rounds + ragged tail
    (28672, 8192, 112 * 32),    # 14 whole rounds
    (300, 192, 2 * 2),          # partial tiles, 128 wide
])
def test_workspace_follows_the_launch_plan(L, rows, tokens, want):
    """The recon and Gram workspaces hold one fp32 loss partial per workgroup
    of the product that writes them, as the launch plan splits it."""
    assert _product_workgroups(rows, tokens) == want
    size = lambda n: (n * 4 + 255) // 256 * 256 + 256
    assert g.gsq_recon_workspace_bytes(1, [0, tokens], rows, 256) == size(want)
    # The Gram form's product is rows x cols (cols a multiple of 128).
    if tokens % 128 == 0:
        assert g.gsq_recon_gram_workspace_bytes(rows, tokens) == size(want)


def test_gram_validation(L):
    gr = g.lib().gsq_gram
    assert gr(100, 256, FAKE, FAKE, None) == ERR_SHAPE                 # tokens not a multiple of 64
    assert gr(128, 200, FAKE, FAKE, None) == ERR_SHAPE                 # cols not a multiple of 128
    assert gr(128, 256, None, FAKE, None) == ERR_NULL
    assert gr(128, 256, FAKE, FAKE_MISALIGNED, None) == ERR_ALIGN
    assert gr(64, (1 << 20) + 128, FAKE, FAKE, None) == ERR_SHAPE      # cols^2 > 2^40 coordinates
    rg = g.lib().gsq_recon_gram
    ws = g.gsq_recon_gram_workspace_bytes(300, 256)
    assert ws >= 4 and ws % 256 == 0
    assert g.gsq_recon_gram_workspace_bytes(300, 100) == 0
    assert rg(0, 256, FAKE, FAKE, FAKE, ws, FAKE, FAKE, None) == ERR_SHAPE
    assert rg(300, 256, None, FAKE, FAKE, ws, FAKE, FAKE, None) == ERR_NULL
    assert rg(300, 256, FAKE, FAKE, FAKE, 4, FAKE, FAKE, None) == ERR_SHAPE
    assert rg(300, 256, FAKE, FAKE, FAKE, ws, FAKE_MISALIGNED, FAKE, None) == ERR_ALIGN
    assert rg(1 << 21, 1 << 10, FAKE, FAKE, FAKE, ws, FAKE, FAKE, None) == ERR_SHAPE   # dW over 2 GiB


def test_gptq_validation(L):
    lay = g.GsqLayer.make(g.GRID_INT2, 64, 256)
    f = g.lib().gsq_init_gptq
    ws = g.gsq_gptq_workspace_bytes(64, 256)
    assert ws >= 256 * 256 * 12 + 64 * 256 * 8
    assert g.gsq_gptq_workspace_bytes(64, 100) == 0
    args = lambda **k: [ctypes.byref(k.get("lay", lay)), k.get("W", FAKE), k.get("tokens", 128),
                        k.get("XT", FAKE), ctypes.c_float(k.get("damp", 0.01)), ctypes.c_float(2.0),
                        k.get("ws", FAKE), k.get("nbytes", ws), FAKE, FAKE, FAKE,
                        k.get("info", FAKE), None]
    assert f(*args(tokens=100)) == ERR_SHAPE
    assert f(*args(tokens=0)) == ERR_SHAPE
    assert f(*args(damp=-0.5)) == ERR_PARAM
    assert f(*args(damp=float("nan"))) == ERR_PARAM
    assert f(*args(nbytes=16)) == ERR_SHAPE
    assert f(*args(XT=None)) == ERR_NULL
    assert f(*args(info=None)) == ERR_NULL
    assert f(*args(W=FAKE_MISALIGNED)) == ERR_ALIGN
    assert f(*args(lay=g.GsqLayer.make(7, 64, 256))) == ERR_GRID


def test_harden_and_noise_validation(L):
    lay = g.GsqLayer.make(g.GRID_INT3_LOCAL, 4, 256)
    h = g.lib().gsq_harden_pack
    assert h(ctypes.byref(lay), FAKE, FAKE, None, FAKE, None, None, None) == ERR_GRID
    assert h(ctypes.byref(lay), None, FAKE, FAKE, FAKE, None, None, None) == ERR_NULL
    assert h(ctypes.byref(lay), FAKE, FAKE, FAKE, FAKE_MISALIGNED, None, None, None) == ERR_ALIGN
    assert h(ctypes.byref(lay), FAKE, FAKE, FAKE, None, None, None, None) == OK    # nothing asked
    n = g.lib().gsq_noise_dump
    assert n(ctypes.byref(lay), 0, -1, 4, FAKE, None) == ERR_SHAPE
    assert n(ctypes.byref(lay), 0, 0, 4, None, None) == ERR_NULL
    assert n(ctypes.byref(lay), 0, 0, 4, 0x10002, None) == ERR_ALIGN
    assert n(ctypes.byref(lay), 0, 0, 0, None, None) == OK                          # empty
    i = g.lib().gsq_init_rtn
    assert i(ctypes.byref(lay), FAKE, FAKE, FAKE, FAKE, ctypes.c_float(float("inf")), None) == ERR_PARAM


def test_binding_raises_named_error(L):
    lay = g.GsqLayer.make(g.GRID_INT2, 4, 200)
    with pytest.raises(g.GsqError) as e:
        g.gsq_relax_fwd(lay, FAKE, FAKE, None, FAKE, 0, 1.0, 1.0, FAKE)
    assert e.value.name == "GSQ_ERR_SHAPE"


def test_product_path_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "post_weight_quantization_philox_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, fn)).read()
                assert not re.search(r"^\s*(from|import)\s+oracle\b", text, re.M), fn
                assert "oracle/" not in text, fn


def test_noalloc_validation(L):
    """The allocation-free reconstruction call checks its arguments like the
    workspace call and rejects a problem whose loss partials exceed its
    static array before touching a device."""
    offs = np.array([0, 2 * 65536], dtype=np.int64)
    p = offs.ctypes.data
    f = L.gsq_recon_loss_grad_noalloc
    assert f(1, p, 65536, 128, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 7
    assert g.gsq_status_str(7) == "GSQ_ERR_SCRATCH"
    assert f(1, p, 65536, 128, FAKE, FAKE, None, FAKE, FAKE, FAKE, None) == ERR_NULL
    assert f(1, p, 65536, 200, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == ERR_SHAPE
    assert f(1, p, 65536, 128, FAKE, FAKE, FAKE, FAKE, FAKE_MISALIGNED, FAKE, None) == ERR_ALIGN
