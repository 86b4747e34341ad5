"""GSQ relaxed-quantization step on AMD MI355X (gfx950).

Python binding of ``libgsq.so`` (C ABI in ``include/gsq.h``). Every function
here has the name of the C entry point it calls and only marshals arguments:
torch tensors become device pointers, the current torch stream becomes the
HIP stream, and a non-OK status raises :class:`GsqError`. All work runs in the
library's HIP kernels; there is no fallback path. If ``libgsq.so`` has not been
built, the first call raises.
"""

from __future__ import annotations

import ctypes
import os

__all__ = [
    "GRID_INT2", "GRID_TERNARY", "GRID_INT3_LOCAL", "GRID_INT3", "DTYPE_F32", "DTYPE_BF16",
    "GsqError", "GsqLayer", "GsqLion", "lib", "exported_symbols",
    "gsq_abi_version", "gsq_status_str", "gsq_num_logits", "gsq_init_rtn",
    "gsq_gptq_workspace_bytes", "gsq_init_gptq", "gsq_matmul_nt_bf16", "gsq_rmsnorm_bf16",
    "gsq_softmax_causal_bf16", "gsq_silu_mul_bf16", "gsq_add_bf16", "gsq_sub_bf16",
    "gsq_dequant_bf16", "gsq_recon_loss_grad_offset",
    "gsq_relax_fwd", "gsq_recon_workspace_bytes", "gsq_recon_loss_grad",
    "gsq_recon_loss_grad_noalloc", "gsq_recon_residual", "gsq_recon_bwd_lion_fwd",
    "gsq_transpose_tokens", "gsq_gram",
    "gsq_recon_gram_workspace_bytes", "gsq_recon_gram",
    "gsq_relax_bwd_lion", "gsq_relax_bwd_lion_fwd", "gsq_harden_pack", "gsq_noise_dump",
]

GRID_INT2, GRID_TERNARY, GRID_INT3_LOCAL, GRID_INT3 = 0, 1, 2, 3
DTYPE_F32, DTYPE_BF16 = 0, 1
N_LOGITS = {GRID_INT2: 4, GRID_TERNARY: 2, GRID_INT3_LOCAL: 5, GRID_INT3: 8}
CODE_BITS = {GRID_INT2: 2, GRID_TERNARY: 2, GRID_INT3_LOCAL: 3, GRID_INT3: 3}

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgsq.so")

#: Entry points declared in include/gsq.h.
EXPORTS = ("gsq_abi_version", "gsq_status_str", "gsq_num_logits", "gsq_init_rtn",
           "gsq_gptq_workspace_bytes", "gsq_init_gptq", "gsq_matmul_nt_bf16",
           "gsq_rmsnorm_bf16", "gsq_softmax_causal_bf16", "gsq_silu_mul_bf16", "gsq_add_bf16",
           "gsq_sub_bf16", "gsq_dequant_bf16", "gsq_recon_loss_grad_offset",
           "gsq_relax_fwd", "gsq_recon_workspace_bytes", "gsq_recon_loss_grad",
           "gsq_recon_loss_grad_noalloc", "gsq_recon_residual", "gsq_recon_bwd_lion_fwd",
           "gsq_transpose_tokens",
           "gsq_gram", "gsq_recon_gram_workspace_bytes", "gsq_recon_gram", "gsq_relax_bwd_lion", "gsq_relax_bwd_lion_fwd",
           "gsq_harden_pack", "gsq_noise_dump")


class GsqError(RuntimeError):
    def __init__(self, fn: str, status: int, name: str):
        super().__init__(f"{fn} failed: {name} ({status})")
        self.status = status
        self.name = name


class GsqLayer(ctypes.Structure):
    _fields_ = [("grid", ctypes.c_int32), ("group", ctypes.c_int32),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("w_dtype", ctypes.c_int32), ("stream", ctypes.c_uint32),
                ("seed", ctypes.c_uint64)]

    @classmethod
    def make(cls, grid: int, rows: int, cols: int, w_dtype: int = DTYPE_BF16,
             seed: int = 0, stream: int = 0, group: int = 128) -> "GsqLayer":
        return cls(grid, group, rows, cols, w_dtype, stream & 0xFFFFFFFF,
                   seed & 0xFFFFFFFFFFFFFFFF)


class GsqLion(ctypes.Structure):
    _fields_ = [("lr_logit", ctypes.c_float), ("lr_scale", ctypes.c_float),
                ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("weight_decay", ctypes.c_float)]

    @classmethod
    def make(cls, lr_logit: float = 1e-3, lr_scale: float = 1e-5, beta1: float = 0.9,
             beta2: float = 0.99, weight_decay: float = 0.0) -> "GsqLion":
        return cls(lr_logit, lr_scale, beta1, beta2, weight_decay)


_lib = None
_P = ctypes.c_void_p
_L = ctypes.POINTER(GsqLayer)


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m post_weight_quantization_philox_amd.build` (hipcc, gfx950)")
    l = ctypes.CDLL(LIB_PATH)
    st = ctypes.c_int
    sig = {
        "gsq_abi_version": (ctypes.c_int, []),
        "gsq_status_str": (ctypes.c_char_p, [ctypes.c_int]),
        "gsq_num_logits": (ctypes.c_int, [ctypes.c_int]),
        "gsq_init_rtn": (st, [_L, _P, _P, _P, _P, ctypes.c_float, _P]),
        "gsq_gptq_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int64]),
        "gsq_matmul_nt_bf16": (st, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _P,
                                    ctypes.c_int64, _P, ctypes.c_int64, _P, ctypes.c_int64, _P]),
        "gsq_rmsnorm_bf16": (st, [ctypes.c_int64, ctypes.c_int64, _P, _P, ctypes.c_float, _P, _P]),
        "gsq_softmax_causal_bf16": (st, [ctypes.c_int64, _P, ctypes.c_float, _P, _P]),
        "gsq_silu_mul_bf16": (st, [ctypes.c_int64, _P, _P, _P, _P]),
        "gsq_add_bf16": (st, [ctypes.c_int64, _P, _P, _P, _P]),
        "gsq_sub_bf16": (st, [ctypes.c_int64, _P, _P, _P, _P]),
        "gsq_recon_loss_grad_offset": (st, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _P, _P,
                                            _P, _P, _P, ctypes.c_size_t, _P, _P, _P, _P]),
        "gsq_dequant_bf16": (st, [_L, _P, _P, _P, _P]),
        "gsq_init_gptq": (st, [_L, _P, ctypes.c_int64, _P, ctypes.c_float, ctypes.c_float, _P,
                               ctypes.c_size_t, _P, _P, _P, _P, _P]),
        "gsq_relax_fwd": (st, [_L, _P, _P, _P, _P, ctypes.c_uint32, ctypes.c_float,
                               ctypes.c_float, _P, _P, _P]),
        "gsq_recon_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int32, _P, ctypes.c_int64,
                                                        ctypes.c_int64]),
        "gsq_recon_loss_grad": (st, [ctypes.c_int32, _P, ctypes.c_int64, ctypes.c_int64, _P, _P,
                                     _P, _P, ctypes.c_size_t, _P, _P, _P, _P]),
        "gsq_recon_loss_grad_noalloc": (st, [ctypes.c_int32, _P, ctypes.c_int64, ctypes.c_int64,
                                             _P, _P, _P, _P, _P, _P, _P]),
        "gsq_recon_residual": (st, [ctypes.c_int32, _P, ctypes.c_int64, ctypes.c_int64, _P, _P,
                                    _P, ctypes.c_size_t, _P, _P]),
        "gsq_recon_bwd_lion_fwd": (st, [_L, ctypes.c_int32, _P, _P, _P, _P, ctypes.c_size_t, _P,
                                        _P, _P, _P, _P, _P, _P, ctypes.c_uint32, ctypes.c_float,
                                        ctypes.c_float, ctypes.POINTER(GsqLion), ctypes.c_int32,
                                        ctypes.c_uint32, ctypes.c_float, _P, _P]),
        "gsq_transpose_tokens": (st, [ctypes.c_int32, _P, ctypes.c_int64, _P, _P, _P]),
        "gsq_gram": (st, [ctypes.c_int64, ctypes.c_int64, _P, _P, _P]),
        "gsq_recon_gram_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int64]),
        "gsq_recon_gram": (st, [ctypes.c_int64, ctypes.c_int64, _P, _P, _P, ctypes.c_size_t, _P, _P,
                                _P]),
        "gsq_relax_bwd_lion": (st, [_L, _P, _P, _P, _P, _P, _P, ctypes.c_uint32, ctypes.c_float,
                                    ctypes.c_float, ctypes.POINTER(GsqLion), _P, _P, _P]),
        "gsq_relax_bwd_lion_fwd": (st, [_L, _P, _P, _P, _P, _P, _P, _P, ctypes.c_uint32,
                                        ctypes.c_float, ctypes.c_float, ctypes.POINTER(GsqLion),
                                        ctypes.c_uint32, ctypes.c_float, _P, _P]),
        "gsq_harden_pack": (st, [_L, _P, _P, _P, _P, _P, _P, _P]),
        "gsq_noise_dump": (st, [_L, ctypes.c_uint32, ctypes.c_int64, ctypes.c_int64, _P, _P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(l, name)
        fn.restype = res
        fn.argtypes = args
    _lib = l
    return l


def exported_symbols():
    """Names from EXPORTS that the loaded library defines."""
    l = lib()
    return [n for n in EXPORTS if hasattr(l, n)]


# ----------------------------------------------------------------------------
# Marshalling
# ----------------------------------------------------------------------------

def _ptr(x):
    """Device pointer of a tensor (or an int address, or None)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    if torch.cuda.is_available() and torch.cuda.is_initialized():
        return torch.cuda.current_stream().cuda_stream
    return None


def _check(fn: str, status: int):
    if status != 0:
        raise GsqError(fn, status, lib().gsq_status_str(status).decode())


def _offsets(tok_offsets):
    import numpy as np
    arr = np.ascontiguousarray(np.asarray(tok_offsets, dtype=np.int64))
    return arr, arr.ctypes.data


# ----------------------------------------------------------------------------
# Entry points (same names as the C ABI)
# ----------------------------------------------------------------------------

def gsq_abi_version() -> int:
    return lib().gsq_abi_version()


def gsq_status_str(status: int) -> str:
    return lib().gsq_status_str(status).decode()


def gsq_num_logits(grid: int) -> int:
    return lib().gsq_num_logits(grid)


def gsq_init_rtn(layer: GsqLayer, W, scales, codes, logits, init_logit: float = 2.0,
                 stream=None):
    _check("gsq_init_rtn", lib().gsq_init_rtn(ctypes.byref(layer), _ptr(W), _ptr(scales),
                                              _ptr(codes), _ptr(logits), init_logit,
                                              _stream(stream)))


def gsq_gptq_workspace_bytes(rows: int, cols: int) -> int:
    return lib().gsq_gptq_workspace_bytes(rows, cols)


def gsq_init_gptq(layer: GsqLayer, W, tokens: int, XT, damp: float, init_logit: float, workspace,
                  scales, codes, logits, info, stream=None, workspace_bytes=None):
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("gsq_init_gptq",
           lib().gsq_init_gptq(ctypes.byref(layer), _ptr(W), tokens, _ptr(XT), damp, init_logit,
                               _ptr(workspace), workspace_bytes, _ptr(scales), _ptr(codes),
                               _ptr(logits), _ptr(info), _stream(stream)))


def gsq_matmul_nt_bf16(I: int, J: int, Rd: int, A, lda: int, B, ldb: int, C, ldc: int,
                       stream=None):
    _check("gsq_matmul_nt_bf16", lib().gsq_matmul_nt_bf16(I, J, Rd, _ptr(A), lda, _ptr(B), ldb,
                                                          _ptr(C), ldc, _stream(stream)))


def gsq_rmsnorm_bf16(rows: int, cols: int, x, gamma, eps: float, y, stream=None):
    _check("gsq_rmsnorm_bf16", lib().gsq_rmsnorm_bf16(rows, cols, _ptr(x), _ptr(gamma), eps,
                                                      _ptr(y), _stream(stream)))


def gsq_softmax_causal_bf16(n: int, S, scale: float, P, stream=None):
    _check("gsq_softmax_causal_bf16", lib().gsq_softmax_causal_bf16(n, _ptr(S), scale, _ptr(P),
                                                                    _stream(stream)))


def gsq_silu_mul_bf16(n: int, gate, up, act, stream=None):
    _check("gsq_silu_mul_bf16", lib().gsq_silu_mul_bf16(n, _ptr(gate), _ptr(up), _ptr(act),
                                                        _stream(stream)))


def gsq_add_bf16(n: int, a, b, out, stream=None):
    _check("gsq_add_bf16", lib().gsq_add_bf16(n, _ptr(a), _ptr(b), _ptr(out), _stream(stream)))


def gsq_sub_bf16(n: int, a, b, out, stream=None):
    _check("gsq_sub_bf16", lib().gsq_sub_bf16(n, _ptr(a), _ptr(b), _ptr(out), _stream(stream)))


def gsq_recon_loss_grad_offset(rows: int, cols: int, tokens: int, X, XT, dW_bf16, E0T, workspace,
                               RT, G, loss, stream=None, workspace_bytes=None):
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("gsq_recon_loss_grad_offset",
           lib().gsq_recon_loss_grad_offset(rows, cols, tokens, _ptr(X), _ptr(XT), _ptr(dW_bf16),
                                            _ptr(E0T), _ptr(workspace), workspace_bytes, _ptr(RT),
                                            _ptr(G), _ptr(loss), _stream(stream)))


def gsq_dequant_bf16(layer: GsqLayer, codes, scales_f16, W, stream=None):
    _check("gsq_dequant_bf16", lib().gsq_dequant_bf16(ctypes.byref(layer), _ptr(codes),
                                                      _ptr(scales_f16), _ptr(W), _stream(stream)))


def gsq_relax_fwd(layer: GsqLayer, logits, scales, init_codes, W, step: int, tau: float,
                  noise_scale: float, dW_bf16, w_soft_dbg=None, stream=None):
    _check("gsq_relax_fwd", lib().gsq_relax_fwd(ctypes.byref(layer), _ptr(logits), _ptr(scales),
                                                _ptr(init_codes), _ptr(W), step, tau, noise_scale,
                                                _ptr(dW_bf16), _ptr(w_soft_dbg), _stream(stream)))


def gsq_recon_workspace_bytes(n_experts: int, tok_offsets, rows_per_expert: int, cols: int) -> int:
    arr, p = _offsets(tok_offsets)
    return lib().gsq_recon_workspace_bytes(n_experts, p, rows_per_expert, cols)


def gsq_recon_loss_grad(n_experts: int, tok_offsets, rows_per_expert: int, cols: int, X, XT,
                        dW_bf16, workspace, RT, G, loss, stream=None, workspace_bytes=None):
    arr, p = _offsets(tok_offsets)
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("gsq_recon_loss_grad",
           lib().gsq_recon_loss_grad(n_experts, p, rows_per_expert, cols, _ptr(X), _ptr(XT),
                                     _ptr(dW_bf16), _ptr(workspace), workspace_bytes, _ptr(RT),
                                     _ptr(G), _ptr(loss), _stream(stream)))


def gsq_recon_loss_grad_noalloc(n_experts: int, tok_offsets, rows_per_expert: int, cols: int, X,
                                XT, dW_bf16, RT, G, loss, stream=None):
    arr, p = _offsets(tok_offsets)
    _check("gsq_recon_loss_grad_noalloc",
           lib().gsq_recon_loss_grad_noalloc(n_experts, p, rows_per_expert, cols, _ptr(X),
                                             _ptr(XT), _ptr(dW_bf16), _ptr(RT), _ptr(G),
                                             _ptr(loss), _stream(stream)))


def gsq_recon_residual(n_experts: int, tok_offsets, rows_per_expert: int, cols: int, X, dW_bf16,
                       workspace, RT, stream=None, workspace_bytes=None):
    arr, p = _offsets(tok_offsets)
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("gsq_recon_residual",
           lib().gsq_recon_residual(n_experts, p, rows_per_expert, cols, _ptr(X), _ptr(dW_bf16),
                                    _ptr(workspace), workspace_bytes, _ptr(RT), _stream(stream)))


def gsq_recon_bwd_lion_fwd(layer: GsqLayer, n_experts: int, tok_offsets, XT, RT, workspace, loss,
                           logits, mom, scales, scale_mom, init_codes, W, step: int, tau: float,
                           noise_scale: float, lion: GsqLion, with_next: bool, next_step: int,
                           next_tau: float, dW_bf16, stream=None, workspace_bytes=None):
    arr, p = _offsets(tok_offsets)
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("gsq_recon_bwd_lion_fwd",
           lib().gsq_recon_bwd_lion_fwd(ctypes.byref(layer), n_experts, p, _ptr(XT), _ptr(RT),
                                        _ptr(workspace), workspace_bytes, _ptr(loss), _ptr(logits),
                                        _ptr(mom), _ptr(scales), _ptr(scale_mom), _ptr(init_codes),
                                        _ptr(W), step, tau, noise_scale, ctypes.byref(lion),
                                        1 if with_next else 0, next_step, next_tau, _ptr(dW_bf16),
                                        _stream(stream)))


def gsq_transpose_tokens(n_experts: int, tok_offsets, cols: int, X, XT, stream=None):
    arr, p = _offsets(tok_offsets)
    _check("gsq_transpose_tokens", lib().gsq_transpose_tokens(n_experts, p, cols, _ptr(X),
                                                              _ptr(XT), _stream(stream)))


def gsq_gram(tokens: int, cols: int, XT, H, stream=None):
    _check("gsq_gram", lib().gsq_gram(tokens, cols, _ptr(XT), _ptr(H), _stream(stream)))


def gsq_recon_gram_workspace_bytes(rows: int, cols: int) -> int:
    return lib().gsq_recon_gram_workspace_bytes(rows, cols)


def gsq_recon_gram(rows: int, cols: int, H, dW_bf16, workspace, G, loss, stream=None,
                   workspace_bytes=None):
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("gsq_recon_gram",
           lib().gsq_recon_gram(rows, cols, _ptr(H), _ptr(dW_bf16), _ptr(workspace),
                                workspace_bytes, _ptr(G), _ptr(loss), _stream(stream)))


def gsq_relax_bwd_lion(layer: GsqLayer, G, logits, mom, scales, scale_mom, init_codes,
                       step: int, tau: float, noise_scale: float, lion: GsqLion,
                       grad_logits_dbg=None, grad_scales_dbg=None, stream=None):
    _check("gsq_relax_bwd_lion",
           lib().gsq_relax_bwd_lion(ctypes.byref(layer), _ptr(G), _ptr(logits), _ptr(mom),
                                    _ptr(scales), _ptr(scale_mom), _ptr(init_codes), step, tau,
                                    noise_scale, ctypes.byref(lion), _ptr(grad_logits_dbg),
                                    _ptr(grad_scales_dbg), _stream(stream)))


def gsq_relax_bwd_lion_fwd(layer: GsqLayer, G, logits, mom, scales, scale_mom, init_codes, W,
                           step: int, tau: float, noise_scale: float, lion: GsqLion,
                           next_step: int, next_tau: float, dW_bf16, stream=None):
    _check("gsq_relax_bwd_lion_fwd",
           lib().gsq_relax_bwd_lion_fwd(ctypes.byref(layer), _ptr(G), _ptr(logits), _ptr(mom),
                                        _ptr(scales), _ptr(scale_mom), _ptr(init_codes), _ptr(W),
                                        step, tau, noise_scale, ctypes.byref(lion), next_step,
                                        next_tau, _ptr(dW_bf16), _stream(stream)))


def gsq_harden_pack(layer: GsqLayer, logits, scales, init_codes, codes=None, packed=None,
                    scales_f16=None, stream=None):
    _check("gsq_harden_pack", lib().gsq_harden_pack(ctypes.byref(layer), _ptr(logits),
                                                    _ptr(scales), _ptr(init_codes), _ptr(codes),
                                                    _ptr(packed), _ptr(scales_f16),
                                                    _stream(stream)))


def gsq_noise_dump(layer: GsqLayer, step: int, first: int, count: int, out, stream=None):
    _check("gsq_noise_dump", lib().gsq_noise_dump(ctypes.byref(layer), step, first, count,
                                                  _ptr(out), _stream(stream)))
