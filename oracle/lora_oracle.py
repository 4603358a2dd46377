"""CPU float64 oracle for the fused LoRA MLP and LoRA QKV projections.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this module.  The product
path (the HIP library and its Python binding) never imports, calls or links
anything here, and this module imports nothing from the product path.

Everything is the plain definition evaluated in float64 with numpy: no
blocking, fusion or reordering beyond what the definitions state.  Matrix
products use ``numpy.matmul`` as a library primitive.  Inputs are the exact
values the device receives (bf16 or fp32 widened to fp64); no intermediate is
rounded.

Sources (the pages' titles and sections):
  * Opake, "Model Patches and Kernels", section "Fused LoRA operations": the
    single LoRA linear ``x @ W.T + x @ A @ B * s`` (opake_lora_w), the fused
    Q+K+V call sharing one input (opake_lora_qkv) and the fused gate+up+down
    call with the activation (opake_lora_mlp); fusion only without active
    LoRA dropout and, for the MLP, without bias.  The fused QKV call may
    carry frozen biases of the base projections (no gradient).
  * Same page, section "Activation functions": SwiGLU ``silu(gate) * up``,
    GeGLU approx ``gelu_tanh(gate) * up``, GeGLU exact (erf).
  * Same page, section "Rotary position embeddings (RoPE)": RoPE on Q and K
    together, GQA with different head counts, following RoFormer.
  * Same page, section "Fused linear cross-entropy", "Key design decisions":
    frozen weights get no weight gradient.
  * Same page, "Model compatibility" and "Fused LoRA operations": Qwen3 /
    Gemma3 attention keeps its per-head q_norm / k_norm RMSNorm (between the
    projection and RoPE) under QKV fusion; RMSNorm is one of the primary
    papers the page's introduction names.
  * Axolotl, "monkeypatch.lora_kernels", section "apply_lora_kernel_patches"
    (note: no dropout, no bias) and section "original_apply_qkv" (input
    hidden_states [batch, seq, hidden] -> (query, key, value)).

Readings where the pages leave a step open (each is also listed with the
design notes):
  * storage follows PEFT / nn.Linear: W [out, in], A [r, in], B [out, r], so
    L(Z) = Z W^T + s (Z A^T) B^T with T = Z A^T [N, r];
  * RoPE pairs column j with column j + d/2 (half split), frequency
    w_j = theta^(-2j/d) for j < d/2, angle = position * w_j computed in
    float64, position = token index within its sequence;
  * Q/K/V are returned head-split as [batch, heads, seq, head_dim];
  * GELU-tanh uses the standard constants sqrt(2/pi) and 0.044715.
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np

__all__ = [
    "silu", "silu_grad", "gelu_tanh", "gelu_tanh_grad", "gelu_erf", "gelu_erf_grad",
    "activation", "lora_linear", "lora_linear_bwd",
    "mlp_fwd", "mlp_bwd",
    "rope_angles", "rope_rotate", "rope_rotate_transpose", "head_split", "head_unsplit",
    "rms_norm", "rms_norm_bwd", "qkv_fwd", "qkv_bwd",
]

_SQRT_2_OVER_PI = math.sqrt(2.0 / math.pi)
_GELU_CUBIC = 0.044715


# ---------------------------------------------------------------------------
# Activations (Opake "Model Patches and Kernels", "Activation functions")
# ---------------------------------------------------------------------------

def _sigmoid(g: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-g))


def silu(g: np.ndarray) -> np.ndarray:
    """SiLU(g) = g * sigmoid(g)."""
    return g * _sigmoid(g)


def silu_grad(g: np.ndarray) -> np.ndarray:
    """d/dg [g sigmoid(g)] = sigmoid(g) * (1 + g (1 - sigmoid(g)))."""
    sg = _sigmoid(g)
    return sg * (1.0 + g * (1.0 - sg))


def gelu_tanh(g: np.ndarray) -> np.ndarray:
    """GELU, tanh approximation: g/2 * (1 + tanh(sqrt(2/pi) (g + 0.044715 g^3)))."""
    return 0.5 * g * (1.0 + np.tanh(_SQRT_2_OVER_PI * (g + _GELU_CUBIC * g ** 3)))


def gelu_tanh_grad(g: np.ndarray) -> np.ndarray:
    """Derivative of gelu_tanh: (1+t)/2 + g/2 (1 - t^2) sqrt(2/pi) (1 + 3*0.044715 g^2)."""
    t = np.tanh(_SQRT_2_OVER_PI * (g + _GELU_CUBIC * g ** 3))
    return 0.5 * (1.0 + t) + 0.5 * g * (1.0 - t * t) * _SQRT_2_OVER_PI * (1.0 + 3.0 * _GELU_CUBIC * g * g)


def _erf(x: np.ndarray) -> np.ndarray:
    return np.vectorize(math.erf, otypes=[np.float64])(x)


def gelu_erf(g: np.ndarray) -> np.ndarray:
    """Exact GELU: g/2 * (1 + erf(g / sqrt(2)))."""
    return 0.5 * g * (1.0 + _erf(g / math.sqrt(2.0)))


def gelu_erf_grad(g: np.ndarray) -> np.ndarray:
    """Phi(g) + g * phi(g), phi the standard normal density."""
    return 0.5 * (1.0 + _erf(g / math.sqrt(2.0))) + g * np.exp(-0.5 * g * g) / math.sqrt(2.0 * math.pi)


_ACTS = {
    "swiglu": (silu, silu_grad),
    "geglu_tanh": (gelu_tanh, gelu_tanh_grad),
    "geglu_erf": (gelu_erf, gelu_erf_grad),
}


def activation(name: str):
    """(phi, phi') of the GLU variant: the gate goes through phi, the up branch is linear."""
    return _ACTS[name]


# ---------------------------------------------------------------------------
# LoRA linear (Opake "Model Patches and Kernels", "Fused LoRA operations")
# ---------------------------------------------------------------------------

def lora_linear(Z: np.ndarray, W: np.ndarray, A: np.ndarray, B: np.ndarray, s: float,
                bias: Optional[np.ndarray] = None):
    """Y = Z W^T + b + s (Z A^T) B^T; returns (Y, T) with T = Z A^T.

    b is the base layer's frozen bias (absent: zero).  It only shifts Y, so
    lora_linear_bwd is the same with or without it.
    """
    T = Z @ A.T
    Y = Z @ W.T + s * (T @ B.T)
    if bias is not None:
        Y = Y + bias[None, :]
    return Y, T


def lora_linear_bwd(dY: np.ndarray, Z: np.ndarray, T: np.ndarray, W: np.ndarray,
                    A: np.ndarray, B: np.ndarray, s: float):
    """Gradients of <dY, lora_linear(Z)> with W frozen (no dW).

    dT = s dY B ; dB = s dY^T T ; dA = dT^T Z ; dZ = dY W + dT A.
    Returns (dZ, dA, dB, dT).
    """
    dT = s * (dY @ B)
    dB = s * (dY.T @ T)
    dA = dT.T @ Z
    dZ = dY @ W + dT @ A
    return dZ, dA, dB, dT


# ---------------------------------------------------------------------------
# LoRA MLP: gate/up -> GLU -> down (opake_lora_mlp)
# ---------------------------------------------------------------------------

def mlp_fwd(p: Dict[str, np.ndarray], act: str, s_gate: float, s_up: float, s_down: float) -> Dict[str, np.ndarray]:
    """Forward of the LoRA MLP.

    G = L_g(X), U = L_u(X), H = phi(G) * U, Y = L_d(H).
    ``p`` holds X and W_*/A_*/B_* for gate, up, down (PEFT storage).
    Returns G, U, H, Y and the rank-r side products T_gate, T_up, T_down.
    """
    phi, _ = activation(act)
    X = p["X"]
    G, Tg = lora_linear(X, p["W_gate"], p["A_gate"], p["B_gate"], s_gate)
    U, Tu = lora_linear(X, p["W_up"], p["A_up"], p["B_up"], s_up)
    H = phi(G) * U
    Y, Td = lora_linear(H, p["W_down"], p["A_down"], p["B_down"], s_down)
    return {"G": G, "U": U, "H": H, "Y": Y, "T_gate": Tg, "T_up": Tu, "T_down": Td}


def mlp_bwd(p: Dict[str, np.ndarray], dY: np.ndarray, act: str,
            s_gate: float, s_up: float, s_down: float) -> Dict[str, np.ndarray]:
    """Backward of the LoRA MLP for the loss <dY, Y>, base weights frozen.

    The forward is re-evaluated from X.  Chain rule through the down
    projection, the GLU (dG = dH * U * phi'(G), dU = dH * phi(G)) and the
    gate/up projections; dX sums both branches.  Returns dX and dA_*/dB_*.
    """
    phi, dphi = activation(act)
    f = mlp_fwd(p, act, s_gate, s_up, s_down)
    dH, dA_d, dB_d, _ = lora_linear_bwd(dY, f["H"], f["T_down"], p["W_down"], p["A_down"], p["B_down"], s_down)
    dG = dH * f["U"] * dphi(f["G"])
    dU = dH * phi(f["G"])
    dXg, dA_g, dB_g, _ = lora_linear_bwd(dG, p["X"], f["T_gate"], p["W_gate"], p["A_gate"], p["B_gate"], s_gate)
    dXu, dA_u, dB_u, _ = lora_linear_bwd(dU, p["X"], f["T_up"], p["W_up"], p["A_up"], p["B_up"], s_up)
    return {"dX": dXg + dXu,
            "dA_gate": dA_g, "dB_gate": dB_g,
            "dA_up": dA_u, "dB_up": dB_u,
            "dA_down": dA_d, "dB_down": dB_d}


# ---------------------------------------------------------------------------
# RoPE and the GQA head split (Opake "Model Patches and Kernels", "RoPE")
# ---------------------------------------------------------------------------

def rope_angles(seq: int, head_dim: int, theta: float) -> np.ndarray:
    """angle[s, j] = s * theta^(-2j/d) for positions s < seq and j < d/2 (float64)."""
    j = np.arange(head_dim // 2, dtype=np.float64)
    inv_freq = theta ** (-2.0 * j / head_dim)
    pos = np.arange(seq, dtype=np.float64)
    return pos[:, None] * inv_freq[None, :]


def rope_rotate(x: np.ndarray, angles: np.ndarray) -> np.ndarray:
    """Rotate pairs (j, j+d/2) of x[..., S, d] by angles[S, d/2].

    y_j = x_j cos a - x_{j+d/2} sin a ;  y_{j+d/2} = x_{j+d/2} cos a + x_j sin a.
    """
    h = x.shape[-1] // 2
    c, s = np.cos(angles), np.sin(angles)
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def rope_rotate_transpose(y: np.ndarray, angles: np.ndarray) -> np.ndarray:
    """Apply R^T (rotation by -a): the adjoint used to pull gradients back through RoPE."""
    h = y.shape[-1] // 2
    c, s = np.cos(angles), np.sin(angles)
    y1, y2 = y[..., :h], y[..., h:]
    return np.concatenate([y1 * c + y2 * s, y2 * c - y1 * s], axis=-1)


def head_split(P: np.ndarray, batch: int, seq: int, heads: int, head_dim: int) -> np.ndarray:
    """[batch*seq, heads*d] (token-major) -> [batch, heads, seq, d]."""
    return P.reshape(batch, seq, heads, head_dim).transpose(0, 2, 1, 3).copy()


def head_unsplit(Q: np.ndarray) -> np.ndarray:
    """[batch, heads, seq, d] -> [batch*seq, heads*d] (inverse of head_split)."""
    b, nh, s, d = Q.shape
    return Q.transpose(0, 2, 1, 3).reshape(b * s, nh * d).copy()


# ---------------------------------------------------------------------------
# Per-head RMSNorm of Q and K (q_norm / k_norm; Zhang & Sennrich's RMSNorm)
# ---------------------------------------------------------------------------

def rms_norm(x: np.ndarray, w: np.ndarray, eps: float):
    """y = x / sqrt(mean(x^2) + eps) * w over the last axis.  Returns (y, rinv)
    with rinv = 1 / sqrt(mean(x^2) + eps) (one value per row)."""
    rinv = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return x * rinv * w, rinv[..., 0]


def rms_norm_bwd(dy: np.ndarray, x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """dx of <dy, rms_norm(x)> for fixed w:
    rinv * (w dy - xhat * mean(w dy xhat)), xhat = x rinv."""
    rinv = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    xhat = x * rinv
    gw = dy * w
    return rinv * (gw - xhat * np.mean(gw * xhat, axis=-1, keepdims=True))


# ---------------------------------------------------------------------------
# LoRA QKV with GQA split and RoPE (opake_lora_qkv; Axolotl original_apply_qkv)
# ---------------------------------------------------------------------------

_QKV = ("q", "k", "v")


_NORM_KEYS = {"q": "qn_w", "k": "kn_w"}


def qkv_fwd(p: Dict[str, np.ndarray], batch: int, seq: int, n_q: int, n_kv: int,
            head_dim: int, theta: float, scales, norm_eps: float = 1e-6) -> Dict[str, np.ndarray]:
    """Q, K, V [B, heads, S, d] from X [B*S, h]: LoRA linear per projection,
    head split, RoPE on Q and K (not V).  Also returns T_q, T_k, T_v.

    Optional frozen biases b_q, b_k, b_v ([out]) are part of the base
    projection, so they are added before the rotation.  qkv_bwd does not read
    them: a frozen bias has no gradient and does not change the others.

    Optional per-head RMSNorm weights qn_w, kn_w ([head_dim], shared by the
    heads of Q resp. K) normalise each head of the projection after the
    split and before the rotation (Qwen3 / Gemma3 q_norm, k_norm); then
    P_q / P_k (the projection before the norm, [B*S, out]) and rinv_q /
    rinv_k ([B*S, heads]) are returned too."""
    X = p["X"]
    heads = {"q": n_q, "k": n_kv, "v": n_kv}
    ang = rope_angles(seq, head_dim, theta)
    out = {}
    for name, s in zip(_QKV, scales):
        P, T = lora_linear(X, p["W_" + name], p["A_" + name], p["B_" + name], s, p.get("b_" + name))
        Z = head_split(P, batch, seq, heads[name], head_dim)
        if _NORM_KEYS.get(name) in p:
            Z, rinv = rms_norm(Z, p[_NORM_KEYS[name]], norm_eps)
            out["P_" + name] = P
            out["rinv_" + name] = head_unsplit(rinv[..., None])
        if name != "v":
            Z = rope_rotate(Z, ang)
        out[name.upper()] = Z
        out["T_" + name] = T
    return out


def qkv_bwd(p: Dict[str, np.ndarray], dQ: np.ndarray, dK: np.ndarray, dV: np.ndarray,
            batch: int, seq: int, n_q: int, n_kv: int, head_dim: int, theta: float,
            scales, norm_eps: float = 1e-6) -> Dict[str, np.ndarray]:
    """Backward of qkv_fwd for the loss <dQ,Q> + <dK,K> + <dV,V>, W frozen.

    dP_q = unsplit(R^T dQ), dP_k = unsplit(R^T dK), dP_v = unsplit(dV); then the
    LoRA linear backward per projection; dX sums the three input gradients.
    With q/k norm weights, R^T dQ is first pulled back through the per-head
    RMSNorm of the (recomputed) projection.
    """
    X = p["X"]
    ang = rope_angles(seq, head_dim, theta)
    grads = {"q": rope_rotate_transpose(dQ, ang), "k": rope_rotate_transpose(dK, ang), "v": dV}
    heads = {"q": n_q, "k": n_kv, "v": n_kv}
    out = {}
    dX = np.zeros_like(X)
    for name, s in zip(_QKV, scales):
        g = grads[name]
        if _NORM_KEYS.get(name) in p:
            P, _ = lora_linear(X, p["W_" + name], p["A_" + name], p["B_" + name], s, p.get("b_" + name))
            Z = head_split(P, batch, seq, heads[name], head_dim)
            g = rms_norm_bwd(g, Z, p[_NORM_KEYS[name]], norm_eps)
        dP = head_unsplit(g)
        T = X @ p["A_" + name].T
        dXp, dA, dB, _ = lora_linear_bwd(dP, X, T, p["W_" + name], p["A_" + name], p["B_" + name], s)
        dX = dX + dXp
        out["dA_" + name] = dA
        out["dB_" + name] = dB
    out["dX"] = dX
    return out
