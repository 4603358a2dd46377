"""Thin ctypes binding over the C ABI in include/lora_mi355x.h.

Argument marshalling only: tensors become device pointers, the stream becomes
the current torch stream's hipStream_t, status codes become exceptions.  Every
step of the computation runs in the HIP library; there is no fallback.  If the
library has not been built, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblora_mi355x.so")

LORA_F32, LORA_BF16 = 0, 1
LORA_SWIGLU, LORA_GEGLU_TANH, LORA_GEGLU_ERF = 0, 1, 2
LORA_MAX_RANK = 16
DTYPE_CODES = {"f32": LORA_F32, "bf16": LORA_BF16, torch.float32: LORA_F32, torch.bfloat16: LORA_BF16}
ACT_CODES = {"swiglu": LORA_SWIGLU, "geglu_tanh": LORA_GEGLU_TANH, "geglu_erf": LORA_GEGLU_ERF}


class LoraError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"status {status}: {message}")
        self.status = status


class MlpDesc(ctypes.Structure):
    _fields_ = [("n_tokens", ctypes.c_int64), ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("rank", ctypes.c_int32), ("dtype", ctypes.c_int32), ("act", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class QkvDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seq", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("n_q", ctypes.c_int32), ("n_kv", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("rank", ctypes.c_int32), ("dtype", ctypes.c_int32), ("rope_theta", ctypes.c_double)]


class LinearDesc(ctypes.Structure):
    _fields_ = [("n_tokens", ctypes.c_int64), ("in_features", ctypes.c_int32), ("out_features", ctypes.c_int32),
                ("rank", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class Proj(ctypes.Structure):
    _fields_ = [("W", ctypes.c_void_p), ("A", ctypes.c_void_p), ("B", ctypes.c_void_p), ("scale", ctypes.c_float),
                ("bias", ctypes.c_void_p)]


class QkNorm(ctypes.Structure):
    _fields_ = [("q_weight", ctypes.c_void_p), ("k_weight", ctypes.c_void_p), ("eps", ctypes.c_float)]


_P = ctypes.c_void_p
_SIGS = {
    "lora_mlp_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(MlpDesc), ctypes.c_int]),
    "lora_qkv_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(QkvDesc), ctypes.c_int]),
    "lora_mlp_fwd": (ctypes.c_int, [ctypes.POINTER(MlpDesc), _P, ctypes.POINTER(Proj), ctypes.POINTER(Proj),
                                    ctypes.POINTER(Proj), _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "lora_mlp_bwd": (ctypes.c_int, [ctypes.POINTER(MlpDesc), _P, _P, _P, _P, _P, ctypes.POINTER(Proj),
                                    ctypes.POINTER(Proj), ctypes.POINTER(Proj), _P, _P, _P, _P, _P, _P, _P, _P,
                                    ctypes.c_size_t, _P]),
    "lora_qkv_fwd": (ctypes.c_int, [ctypes.POINTER(QkvDesc), _P, ctypes.POINTER(Proj), ctypes.POINTER(Proj),
                                    ctypes.POINTER(Proj), _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "lora_qkv_fwd_noalloc": (ctypes.c_int, [ctypes.POINTER(QkvDesc), _P, ctypes.POINTER(Proj), ctypes.POINTER(Proj),
                                            ctypes.POINTER(Proj), _P, _P, _P, _P, _P]),
    "lora_qkv_fwd_noalloc_max_scratch_bytes": (ctypes.c_size_t, []),
    "lora_qkv_bwd": (ctypes.c_int, [ctypes.POINTER(QkvDesc), _P, _P, _P, _P, _P, ctypes.POINTER(Proj),
                                    ctypes.POINTER(Proj), ctypes.POINTER(Proj), _P, _P, _P, _P, _P, _P, _P, _P,
                                    ctypes.c_size_t, _P]),
    "lora_linear_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(LinearDesc), ctypes.c_int]),
    "lora_linear_fwd": (ctypes.c_int, [ctypes.POINTER(LinearDesc), _P, ctypes.POINTER(Proj), _P, _P, _P,
                                       ctypes.c_size_t, _P]),
    "lora_linear_bwd": (ctypes.c_int, [ctypes.POINTER(LinearDesc), _P, _P, _P, ctypes.POINTER(Proj), _P, _P, _P,
                                       _P, ctypes.c_size_t, _P]),
    "lora_qkv_norm_fwd": (ctypes.c_int, [ctypes.POINTER(QkvDesc), _P, ctypes.POINTER(Proj), ctypes.POINTER(Proj),
                                         ctypes.POINTER(Proj), ctypes.POINTER(QkNorm), _P, _P, _P, _P, _P, _P, _P,
                                         ctypes.c_size_t, _P]),
    "lora_qkv_norm_bwd": (ctypes.c_int, [ctypes.POINTER(QkvDesc), _P, _P, _P, _P, _P, _P, _P, ctypes.POINTER(Proj),
                                         ctypes.POINTER(Proj), ctypes.POINTER(Proj), ctypes.POINTER(QkNorm), _P, _P,
                                         _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "lora_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "lora_last_error_message": (ctypes.c_char_p, []),
    "lora_version": (ctypes.c_char_p, []),
    "lora_timing_enable": (ctypes.c_int, [ctypes.c_int]),
    "lora_timing_reset": (ctypes.c_int, []),
    "lora_timing_query": (ctypes.c_int, [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                                         ctypes.POINTER(ctypes.c_int)]),
    "lora_kernel_names": (ctypes.c_char_p, []),
}

_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library not built: {LIB_PATH} (run __graft_entry__.build())")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


def _check(status: int) -> None:
    if status != 0:
        raise LoraError(status, lib().lora_last_error_message().decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the LoRA library must be contiguous")
    return t.data_ptr()


TORCH_DTYPES = {LORA_F32: torch.float32, LORA_BF16: torch.bfloat16}
_REQUIRE_GPU = True      # the host-only tests turn this off to reach the dtype and size checks


def _need(t: Optional[torch.Tensor], name: str, dtype: torch.dtype, numel: int, optional: bool = False) -> None:
    """Reject, before any device call, a buffer the kernels would read or write
    out of bounds: it must be a contiguous tensor on the GPU, of the dtype the
    descriptor names, with at least `numel` elements."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name}: a tensor is required")
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if _REQUIRE_GPU and not t.is_cuda:
        raise ValueError(f"{name}: must be a GPU tensor (got device {t.device})")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype} does not match the descriptor's {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name}: {t.numel()} elements, the call needs at least {numel}")


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def proj(W: torch.Tensor, A: torch.Tensor, B: torch.Tensor, scale: float,
         bias: Optional[torch.Tensor] = None) -> Proj:
    p = Proj(_ptr(W), _ptr(A), _ptr(B), float(scale), _ptr(bias))
    p.tensors = (W, A, B, bias)        # kept for the size checks of the raw wrappers
    return p


def _need_proj(p: Proj, name: str, dtype: torch.dtype, out_f: int, in_f: int, rank: int,
               bias_ok: bool = True) -> None:
    """W [out, in], A [rank, in], B [out, rank], optional bias [out]."""
    t = getattr(p, "tensors", None)
    if t is None:
        raise ValueError(f"{name}: build the projection with proj() so its tensors can be checked")
    W, A, B, bias = t
    _need(W, name + ".W", dtype, out_f * in_f)
    _need(A, name + ".A", dtype, rank * in_f)
    _need(B, name + ".B", dtype, out_f * rank)
    if bias is not None and not bias_ok:
        raise ValueError(f"{name}: this call takes no bias")
    _need(bias, name + ".bias", dtype, out_f, optional=True)


def _mlp_dims(desc: MlpDesc):
    return int(desc.n_tokens), int(desc.hidden), int(desc.inter), int(desc.rank), TORCH_DTYPES.get(desc.dtype)


def _qkv_dims(desc: QkvDesc):
    N = int(desc.batch) * int(desc.seq)
    Oq, Ok = int(desc.n_q) * int(desc.head_dim), int(desc.n_kv) * int(desc.head_dim)
    return N, int(desc.hidden), Oq, Ok, int(desc.rank), TORCH_DTYPES.get(desc.dtype)


def _lin_dims(desc: LinearDesc):
    return (int(desc.n_tokens), int(desc.in_features), int(desc.out_features), int(desc.rank),
            TORCH_DTYPES.get(desc.dtype))


def _check_dtype(dt) -> torch.dtype:
    if dt is None:
        raise ValueError("descriptor dtype is not one of LORA_F32, LORA_BF16")
    return dt


def _need_ws(ws: Optional[torch.Tensor], need_bytes: int) -> None:
    if need_bytes == 0 and ws is None:
        return
    _need(ws, "workspace", torch.uint8, need_bytes)


def mlp_desc(n_tokens, hidden, inter, rank, dtype, act) -> MlpDesc:
    return MlpDesc(int(n_tokens), int(hidden), int(inter), int(rank), DTYPE_CODES[dtype], ACT_CODES.get(act, act), 0)


def qkv_desc(batch, seq, hidden, n_q, n_kv, head_dim, rank, dtype, theta) -> QkvDesc:
    return QkvDesc(int(batch), int(seq), int(hidden), int(n_q), int(n_kv), int(head_dim), int(rank),
                   DTYPE_CODES[dtype], float(theta))


def linear_desc(n_tokens, in_features, out_features, rank, dtype) -> LinearDesc:
    return LinearDesc(int(n_tokens), int(in_features), int(out_features), int(rank), DTYPE_CODES[dtype])


# ---- raw entry points (same names as the C ABI) ------------------------------

def lora_mlp_workspace_bytes(desc: MlpDesc, pass_: int) -> int:
    return int(lib().lora_mlp_workspace_bytes(ctypes.byref(desc), int(pass_)))


def lora_qkv_workspace_bytes(desc: QkvDesc, pass_: int) -> int:
    return int(lib().lora_qkv_workspace_bytes(ctypes.byref(desc), int(pass_)))


def lora_mlp_fwd(desc, X, gate: Proj, up: Proj, down: Proj, Y, G, U, T, workspace, stream=None):
    N, h, i, r, dt = _mlp_dims(desc)
    dt = _check_dtype(dt)
    _need(X, "X", dt, N * h)
    _need_proj(gate, "gate", dt, i, h, r, bias_ok=False)
    _need_proj(up, "up", dt, i, h, r, bias_ok=False)
    _need_proj(down, "down", dt, h, i, r, bias_ok=False)
    for t, n, m in ((Y, "Y", N * h), (G, "G", N * i), (U, "U", N * i)):
        _need(t, n, dt, m)
    _need(T, "T", torch.float32, 3 * N * r)
    _need(workspace, "workspace", torch.uint8, 1)
    _check(lib().lora_mlp_fwd(ctypes.byref(desc), _ptr(X), ctypes.byref(gate), ctypes.byref(up), ctypes.byref(down),
                              _ptr(Y), _ptr(G), _ptr(U), _ptr(T), _ptr(workspace), workspace.numel(),
                              _stream(stream)))


def lora_mlp_bwd(desc, dY, X, G, U, T, gate: Proj, up: Proj, down: Proj, dX, dA_gate, dB_gate, dA_up, dB_up,
                 dA_down, dB_down, workspace, stream=None):
    N, h, i, r, dt = _mlp_dims(desc)
    dt = _check_dtype(dt)
    for t, n, m in ((dY, "dY", N * h), (X, "X", N * h), (G, "G", N * i), (U, "U", N * i), (dX, "dX", N * h),
                    (dA_gate, "dA_gate", r * h), (dB_gate, "dB_gate", i * r), (dA_up, "dA_up", r * h),
                    (dB_up, "dB_up", i * r), (dA_down, "dA_down", r * i), (dB_down, "dB_down", h * r)):
        _need(t, n, dt, m)
    _need(T, "T", torch.float32, 3 * N * r)
    _need_proj(gate, "gate", dt, i, h, r, bias_ok=False)
    _need_proj(up, "up", dt, i, h, r, bias_ok=False)
    _need_proj(down, "down", dt, h, i, r, bias_ok=False)
    _need(workspace, "workspace", torch.uint8, 1)
    _check(lib().lora_mlp_bwd(ctypes.byref(desc), _ptr(dY), _ptr(X), _ptr(G), _ptr(U), _ptr(T), ctypes.byref(gate),
                              ctypes.byref(up), ctypes.byref(down), _ptr(dX), _ptr(dA_gate), _ptr(dB_gate),
                              _ptr(dA_up), _ptr(dB_up), _ptr(dA_down), _ptr(dB_down), _ptr(workspace),
                              workspace.numel(), _stream(stream)))


def _need_qkv_common(desc, X, q, k, v, T):
    N, h, Oq, Ok, r, dt = _qkv_dims(desc)
    dt = _check_dtype(dt)
    _need(X, "X", dt, N * h)
    _need_proj(q, "q", dt, Oq, h, r)
    _need_proj(k, "k", dt, Ok, h, r)
    _need_proj(v, "v", dt, Ok, h, r)
    _need(T, "T", torch.float32, 3 * N * r)
    return N, h, Oq, Ok, r, dt


def lora_qkv_fwd(desc, X, q: Proj, k: Proj, v: Proj, Q, K, V, T, workspace, stream=None):
    N, h, Oq, Ok, r, dt = _need_qkv_common(desc, X, q, k, v, T)
    for t, n, m in ((Q, "Q", N * Oq), (K, "K", N * Ok), (V, "V", N * Ok)):
        _need(t, n, dt, m)
    _need(workspace, "workspace", torch.uint8, 1)
    _check(lib().lora_qkv_fwd(ctypes.byref(desc), _ptr(X), ctypes.byref(q), ctypes.byref(k), ctypes.byref(v),
                              _ptr(Q), _ptr(K), _ptr(V), _ptr(T), _ptr(workspace), workspace.numel(),
                              _stream(stream)))


def lora_qkv_fwd_noalloc(desc, X, q: Proj, k: Proj, v: Proj, Q, K, V, T, stream=None):
    N, h, Oq, Ok, r, dt = _need_qkv_common(desc, X, q, k, v, T)
    for t, n, m in ((Q, "Q", N * Oq), (K, "K", N * Ok), (V, "V", N * Ok)):
        _need(t, n, dt, m)
    _check(lib().lora_qkv_fwd_noalloc(ctypes.byref(desc), _ptr(X), ctypes.byref(q), ctypes.byref(k),
                                      ctypes.byref(v), _ptr(Q), _ptr(K), _ptr(V), _ptr(T), _stream(stream)))


def lora_qkv_fwd_noalloc_max_scratch_bytes() -> int:
    return int(lib().lora_qkv_fwd_noalloc_max_scratch_bytes())


def _need_qkv_grads(desc, dQ, dK, dV, dX, dA_q, dB_q, dA_k, dB_k, dA_v, dB_v):
    N, h, Oq, Ok, r, dt = _qkv_dims(desc)
    for t, n, m in ((dQ, "dQ", N * Oq), (dK, "dK", N * Ok), (dV, "dV", N * Ok), (dX, "dX", N * h),
                    (dA_q, "dA_q", r * h), (dB_q, "dB_q", Oq * r), (dA_k, "dA_k", r * h), (dB_k, "dB_k", Ok * r),
                    (dA_v, "dA_v", r * h), (dB_v, "dB_v", Ok * r)):
        _need(t, n, dt, m)


def lora_qkv_bwd(desc, dQ, dK, dV, X, T, q: Proj, k: Proj, v: Proj, dX, dA_q, dB_q, dA_k, dB_k, dA_v, dB_v,
                 workspace, stream=None):
    _need_qkv_common(desc, X, q, k, v, T)
    _need_qkv_grads(desc, dQ, dK, dV, dX, dA_q, dB_q, dA_k, dB_k, dA_v, dB_v)
    _need(workspace, "workspace", torch.uint8, 1)
    _check(lib().lora_qkv_bwd(ctypes.byref(desc), _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(X), _ptr(T), ctypes.byref(q),
                              ctypes.byref(k), ctypes.byref(v), _ptr(dX), _ptr(dA_q), _ptr(dB_q), _ptr(dA_k),
                              _ptr(dB_k), _ptr(dA_v), _ptr(dB_v), _ptr(workspace), workspace.numel(),
                              _stream(stream)))


def lora_linear_workspace_bytes(desc: LinearDesc, pass_: int) -> int:
    return int(lib().lora_linear_workspace_bytes(ctypes.byref(desc), int(pass_)))


def lora_linear_fwd(desc, X, p: Proj, Y, T, workspace=None, stream=None):
    N, k, o, r, dt = _lin_dims(desc)
    dt = _check_dtype(dt)
    _need(X, "X", dt, N * k)
    _need_proj(p, "p", dt, o, k, r)
    _need(Y, "Y", dt, N * o)
    _need(T, "T", torch.float32, N * r)
    _need(workspace, "workspace", torch.uint8, 1, optional=True)
    _check(lib().lora_linear_fwd(ctypes.byref(desc), _ptr(X), ctypes.byref(p), _ptr(Y), _ptr(T), _ptr(workspace),
                                 0 if workspace is None else workspace.numel(), _stream(stream)))


def lora_linear_bwd(desc, dY, X, T, p: Proj, dX, dA, dB, workspace, stream=None):
    N, k, o, r, dt = _lin_dims(desc)
    dt = _check_dtype(dt)
    for t, n, m in ((dY, "dY", N * o), (X, "X", N * k), (dX, "dX", N * k), (dA, "dA", r * k), (dB, "dB", o * r)):
        _need(t, n, dt, m)
    _need(T, "T", torch.float32, N * r)
    _need_proj(p, "p", dt, o, k, r)
    _need(workspace, "workspace", torch.uint8, 1)
    _check(lib().lora_linear_bwd(ctypes.byref(desc), _ptr(dY), _ptr(X), _ptr(T), ctypes.byref(p), _ptr(dX), _ptr(dA),
                                 _ptr(dB), _ptr(workspace), workspace.numel(), _stream(stream)))


def qk_norm(q_weight: torch.Tensor, k_weight: torch.Tensor, eps: float) -> QkNorm:
    n = QkNorm(_ptr(q_weight), _ptr(k_weight), float(eps))
    n.tensors = (q_weight, k_weight)
    return n


def _need_norm(desc, norm: QkNorm, Pn, rinv):
    N, h, Oq, Ok, r, dt = _qkv_dims(desc)
    t = getattr(norm, "tensors", None)
    if t is None:
        raise ValueError("norm: build it with qk_norm() so its tensors can be checked")
    _need(t[0], "norm.q_weight", dt, int(desc.head_dim))
    _need(t[1], "norm.k_weight", dt, int(desc.head_dim))
    _need(Pn, "Pn", dt, N * (Oq + Ok))
    _need(rinv, "rinv", torch.float32, N * (int(desc.n_q) + int(desc.n_kv)))


def lora_qkv_norm_fwd(desc, X, q: Proj, k: Proj, v: Proj, norm: QkNorm, Q, K, V, T, Pn, rinv, workspace,
                      stream=None):
    N, h, Oq, Ok, r, dt = _need_qkv_common(desc, X, q, k, v, T)
    for t, n, m in ((Q, "Q", N * Oq), (K, "K", N * Ok), (V, "V", N * Ok)):
        _need(t, n, dt, m)
    _need_norm(desc, norm, Pn, rinv)
    _need(workspace, "workspace", torch.uint8, 1)
    _check(lib().lora_qkv_norm_fwd(ctypes.byref(desc), _ptr(X), ctypes.byref(q), ctypes.byref(k), ctypes.byref(v),
                                   ctypes.byref(norm), _ptr(Q), _ptr(K), _ptr(V), _ptr(T), _ptr(Pn), _ptr(rinv),
                                   _ptr(workspace), workspace.numel(), _stream(stream)))


def lora_qkv_norm_bwd(desc, dQ, dK, dV, X, T, Pn, rinv, q: Proj, k: Proj, v: Proj, norm: QkNorm, dX, dA_q, dB_q,
                      dA_k, dB_k, dA_v, dB_v, workspace, stream=None):
    _need_qkv_common(desc, X, q, k, v, T)
    _need_qkv_grads(desc, dQ, dK, dV, dX, dA_q, dB_q, dA_k, dB_k, dA_v, dB_v)
    _need_norm(desc, norm, Pn, rinv)
    _need(workspace, "workspace", torch.uint8, 1)
    _check(lib().lora_qkv_norm_bwd(ctypes.byref(desc), _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(X), _ptr(T), _ptr(Pn),
                                   _ptr(rinv), ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), ctypes.byref(norm),
                                   _ptr(dX), _ptr(dA_q), _ptr(dB_q), _ptr(dA_k), _ptr(dB_k), _ptr(dA_v), _ptr(dB_v),
                                   _ptr(workspace), workspace.numel(), _stream(stream)))


# ---- timing -------------------------------------------------------------------

def timing_enable(on: bool = True) -> None:
    _check(lib().lora_timing_enable(1 if on else 0))


def timing_reset() -> None:
    _check(lib().lora_timing_reset())


def timing_query(kernel: str):
    """(total milliseconds, launches) of one kernel since the last reset."""
    ms, n = ctypes.c_double(), ctypes.c_int()
    _check(lib().lora_timing_query(kernel.encode(), ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def kernel_names():
    return lib().lora_kernel_names().decode().split(",")


# ---- plumbing: allocate outputs / workspace with torch, then call the ABI -----

def _class_dtype(code: int, X: torch.Tensor) -> torch.dtype:
    """The outputs are allocated in the descriptor's dtype; X must match it."""
    dt = _check_dtype(TORCH_DTYPES.get(code))
    if X.dtype != dt:
        raise ValueError(f"X is {X.dtype} but the call dtype is {dt}")
    return dt


class MLP:
    """LoRA MLP weights on the device plus the buffers one fwd+bwd needs."""

    def __init__(self, t: Dict[str, torch.Tensor], n_tokens, hidden, inter, rank, dtype, act,
                 scales=(2.0, 2.0, 2.0)):
        self.t = t
        self.desc = mlp_desc(n_tokens, hidden, inter, rank, dtype, act)
        self.dtype = _class_dtype(self.desc.dtype, t["X"])
        dev = t["X"].device
        self.N, self.h, self.i, self.r = int(n_tokens), int(hidden), int(inter), int(rank)
        self.gate = proj(t["W_gate"], t["A_gate"], t["B_gate"], scales[0])
        self.up = proj(t["W_up"], t["A_up"], t["B_up"], scales[1])
        self.down = proj(t["W_down"], t["A_down"], t["B_down"], scales[2])
        e = dict(device=dev, dtype=self.dtype)
        self.Y = torch.empty(self.N, self.h, **e)
        self.G = torch.empty(self.N, self.i, **e)
        self.U = torch.empty(self.N, self.i, **e)
        self.T = torch.empty(3, self.N, self.r, device=dev, dtype=torch.float32)
        self.dX = torch.empty(self.N, self.h, **e)
        self.grads = {
            "dA_gate": torch.empty(self.r, self.h, **e), "dB_gate": torch.empty(self.i, self.r, **e),
            "dA_up": torch.empty(self.r, self.h, **e), "dB_up": torch.empty(self.i, self.r, **e),
            "dA_down": torch.empty(self.r, self.i, **e), "dB_down": torch.empty(self.h, self.r, **e),
        }
        self.ws_fwd = torch.empty(max(1, lora_mlp_workspace_bytes(self.desc, 0)), device=dev, dtype=torch.uint8)
        self.ws_bwd = torch.empty(max(1, lora_mlp_workspace_bytes(self.desc, 1)), device=dev, dtype=torch.uint8)

    def forward(self, stream=None):
        lora_mlp_fwd(self.desc, self.t["X"], self.gate, self.up, self.down, self.Y, self.G, self.U, self.T,
                     self.ws_fwd, stream)
        return self.Y

    def backward(self, dY, stream=None):
        g = self.grads
        lora_mlp_bwd(self.desc, dY, self.t["X"], self.G, self.U, self.T, self.gate, self.up, self.down, self.dX,
                     g["dA_gate"], g["dB_gate"], g["dA_up"], g["dB_up"], g["dA_down"], g["dB_down"], self.ws_bwd,
                     stream)
        return self.dX


class QKV:
    """LoRA QKV weights on the device plus the buffers one fwd+bwd needs
    (optional frozen biases under the keys b_q, b_k, b_v; optional q/k norm
    weights under qn_w, kn_w, which select the norm entry points)."""

    def __init__(self, t: Dict[str, torch.Tensor], batch, seq, hidden, n_q, n_kv, head_dim, rank, dtype, theta,
                 scales=(2.0, 2.0, 2.0), norm_eps: float = 1e-6):
        self.t = t
        self.desc = qkv_desc(batch, seq, hidden, n_q, n_kv, head_dim, rank, dtype, theta)
        self.dtype = _class_dtype(self.desc.dtype, t["X"])
        dev = t["X"].device
        self.B, self.S, self.h, self.r, self.d = int(batch), int(seq), int(hidden), int(rank), int(head_dim)
        self.nq, self.nkv = int(n_q), int(n_kv)
        N = self.B * self.S
        self.q = proj(t["W_q"], t["A_q"], t["B_q"], scales[0], t.get("b_q"))
        self.k = proj(t["W_k"], t["A_k"], t["B_k"], scales[1], t.get("b_k"))
        self.v = proj(t["W_v"], t["A_v"], t["B_v"], scales[2], t.get("b_v"))
        e = dict(device=dev, dtype=self.dtype)
        self.Q = torch.empty(self.B, self.nq, self.S, self.d, **e)
        self.K = torch.empty(self.B, self.nkv, self.S, self.d, **e)
        self.V = torch.empty(self.B, self.nkv, self.S, self.d, **e)
        self.T = torch.empty(3, N, self.r, device=dev, dtype=torch.float32)
        self.dX = torch.empty(N, self.h, **e)
        Oq, Ok = self.nq * self.d, self.nkv * self.d
        self.grads = {
            "dA_q": torch.empty(self.r, self.h, **e), "dB_q": torch.empty(Oq, self.r, **e),
            "dA_k": torch.empty(self.r, self.h, **e), "dB_k": torch.empty(Ok, self.r, **e),
            "dA_v": torch.empty(self.r, self.h, **e), "dB_v": torch.empty(Ok, self.r, **e),
        }
        self.ws_fwd = torch.empty(max(1, lora_qkv_workspace_bytes(self.desc, 0)), device=dev, dtype=torch.uint8)
        self.ws_bwd = torch.empty(max(1, lora_qkv_workspace_bytes(self.desc, 1)), device=dev, dtype=torch.uint8)
        self.norm = None
        if "qn_w" in t:
            self.norm = qk_norm(t["qn_w"], t["kn_w"], norm_eps)
            self.Pn = torch.empty(N, Oq + Ok, **e)
            self.rinv = torch.empty(N, self.nq + self.nkv, device=dev, dtype=torch.float32)

    def forward(self, stream=None):
        if self.norm is not None:
            lora_qkv_norm_fwd(self.desc, self.t["X"], self.q, self.k, self.v, self.norm, self.Q, self.K, self.V,
                              self.T, self.Pn, self.rinv, self.ws_fwd, stream)
        else:
            lora_qkv_fwd(self.desc, self.t["X"], self.q, self.k, self.v, self.Q, self.K, self.V, self.T,
                         self.ws_fwd, stream)
        return self.Q, self.K, self.V

    def backward(self, dQ, dK, dV, stream=None):
        g = self.grads
        if self.norm is not None:
            lora_qkv_norm_bwd(self.desc, dQ, dK, dV, self.t["X"], self.T, self.Pn, self.rinv, self.q, self.k, self.v,
                              self.norm, self.dX, g["dA_q"], g["dB_q"], g["dA_k"], g["dB_k"], g["dA_v"], g["dB_v"],
                              self.ws_bwd, stream)
        else:
            lora_qkv_bwd(self.desc, dQ, dK, dV, self.t["X"], self.T, self.q, self.k, self.v, self.dX, g["dA_q"],
                         g["dB_q"], g["dA_k"], g["dB_k"], g["dA_v"], g["dB_v"], self.ws_bwd, stream)
        return self.dX


class Linear:
    """One LoRA linear's weights on the device plus the buffers one fwd+bwd needs
    (optional frozen bias under the key "bias")."""

    def __init__(self, t: Dict[str, torch.Tensor], n_tokens, in_features, out_features, rank, dtype, scale=2.0):
        self.t = t
        self.desc = linear_desc(n_tokens, in_features, out_features, rank, dtype)
        self.dtype = _class_dtype(self.desc.dtype, t["X"])
        dev = t["X"].device
        self.N, self.k, self.o, self.r = int(n_tokens), int(in_features), int(out_features), int(rank)
        self.p = proj(t["W"], t["A"], t["B"], scale, t.get("bias"))
        e = dict(device=dev, dtype=self.dtype)
        self.Y = torch.empty(self.N, self.o, **e)
        self.T = torch.empty(self.N, self.r, device=dev, dtype=torch.float32)
        self.dX = torch.empty(self.N, self.k, **e)
        self.grads = {"dA": torch.empty(self.r, self.k, **e), "dB": torch.empty(self.o, self.r, **e)}
        self.ws_bwd = torch.empty(max(1, lora_linear_workspace_bytes(self.desc, 1)), device=dev, dtype=torch.uint8)
        nf = lora_linear_workspace_bytes(self.desc, 0)
        self.ws_fwd = torch.empty(nf, device=dev, dtype=torch.uint8) if nf else None

    def forward(self, stream=None):
        lora_linear_fwd(self.desc, self.t["X"], self.p, self.Y, self.T, self.ws_fwd, stream)
        return self.Y

    def backward(self, dY, stream=None):
        lora_linear_bwd(self.desc, dY, self.t["X"], self.T, self.p, self.dX, self.grads["dA"], self.grads["dB"],
                        self.ws_bwd, stream)
        return self.dX
