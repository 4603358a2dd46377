"""Seeded synthetic inputs for the LoRA MLP / QKV projections.

This module is the one thing the HIP path and the CPU oracle share: it draws
the input tensors and nothing else.  It contains none of the method's
arithmetic (no projection, activation, rotation or gradient formula).

Recipe (applied to every tensor):
  1. draw float32 standard normals from ``torch.Generator('cpu')`` seeded with
     ``1000 * seed + tensor_id`` (the ids below are fixed);
  2. multiply by the tensor's standard deviation;
  3. round once to the call dtype (round-to-nearest-even for bfloat16).
The device gets these rounded values; the oracle gets the same values widened
to float64, so both sides see bit-identical inputs.

Distributions follow the benchmark configurations: activations and upstream
gradients ~N(0,1), frozen base weights std 0.02, LoRA A with variance
1/in_dim (std in_dim**-0.5), LoRA B std 0.02 (non-zero, so the adapter path is
visible in every output and gradient), optional frozen base biases std 0.5,
optional q/k RMSNorm weights N(1, 0.2^2).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np
import torch

# Fixed tensor ids for seeding (never renumber: stored expectations and
# cached results depend on them).
MLP_IDS = {
    "X": 0,
    "W_gate": 1, "A_gate": 2, "B_gate": 3,
    "W_up": 4, "A_up": 5, "B_up": 6,
    "W_down": 7, "A_down": 8, "B_down": 9,
    "dY": 10,
}
QKV_IDS = {
    "X": 20,
    "W_q": 21, "A_q": 22, "B_q": 23,
    "W_k": 24, "A_k": 25, "B_k": 26,
    "W_v": 27, "A_v": 28, "B_v": 29,
    "dQ": 30, "dK": 31, "dV": 32,
    "b_q": 33, "b_k": 34, "b_v": 35,
    "qn_w": 36, "kn_w": 37,
}
LINEAR_IDS = {"X": 40, "W": 41, "A": 42, "B": 43, "dY": 44, "bias": 45}

TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


def normal(shape, std: float, seed: int, tensor_id: int, dtype: str, mean: float = 0.0) -> torch.Tensor:
    """Seeded N(mean, std^2) tensor on the CPU, rounded once to ``dtype``."""
    g = torch.Generator("cpu")
    g.manual_seed(1000 * int(seed) + int(tensor_id))
    x = torch.randn(tuple(int(s) for s in shape), generator=g, dtype=torch.float32)
    if std != 1.0:
        x.mul_(float(std))
    if mean != 0.0:
        x.add_(float(mean))
    return x.to(TORCH_DTYPES[dtype])


@dataclasses.dataclass(frozen=True)
class MLPConfig:
    """One LoRA MLP workload: X [n_tokens, hidden], gate/up [hidden->inter], down [inter->hidden]."""
    name: str
    n_tokens: int
    hidden: int
    inter: int
    rank: int
    scale: float
    act: str            # "swiglu" | "geglu_tanh" | "geglu_erf"
    dtype: str          # "f32" | "bf16"
    w_std: float = 0.02
    b_std: float = 0.02
    a_std: Optional[float] = None   # None: (in_dim)**-0.5 per projection

    def a_std_for(self, in_dim: int) -> float:
        return self.a_std if self.a_std is not None else 1.0 / math.sqrt(in_dim)

    def flops(self) -> int:
        """Algorithmic fwd+bwd FLOPs (frozen W: no dW; elementwise work not counted)."""
        N, h, i, r = self.n_tokens, self.hidden, self.inter, self.rank
        return 12 * N * h * i + 18 * N * r * (h + i)

    def flops_fwd(self) -> int:
        """G,U: 2Nhi each + side 2Nhr + fold 2Nri; Y: 2Nih + side 2Nir + fold 2Nrh."""
        N, h, i, r = self.n_tokens, self.hidden, self.inter, self.rank
        return 6 * N * h * i + 6 * N * r * (h + i)

    def flops_bwd(self) -> int:
        N, h, i, r = self.n_tokens, self.hidden, self.inter, self.rank
        return 6 * N * h * i + 12 * N * r * (h + i)


@dataclasses.dataclass(frozen=True)
class QKVConfig:
    """One LoRA QKV workload: X [batch*seq, hidden] -> Q [B,n_q,S,d], K,V [B,n_kv,S,d]."""
    name: str
    batch: int
    seq: int
    hidden: int
    n_q: int
    n_kv: int
    head_dim: int
    rank: int
    scale: float
    theta: float
    dtype: str
    w_std: float = 0.02
    b_std: float = 0.02
    a_std: Optional[float] = None
    bias: bool = False     # frozen base biases b_q, b_k, b_v (std bias_std)
    bias_std: float = 0.5
    qk_norm: bool = False  # per-head RMSNorm weights qn_w, kn_w ~ N(1, norm_std^2)
    norm_std: float = 0.2
    norm_eps: float = 1e-6

    @property
    def n_tokens(self) -> int:
        return self.batch * self.seq

    @property
    def out_dims(self):
        return (self.n_q * self.head_dim, self.n_kv * self.head_dim, self.n_kv * self.head_dim)

    def a_std_for(self, in_dim: int) -> float:
        return self.a_std if self.a_std is not None else 1.0 / math.sqrt(in_dim)

    def flops(self) -> int:
        N, h, r = self.n_tokens, self.hidden, self.rank
        O = sum(self.out_dims)
        return 4 * N * h * O + 6 * N * r * (3 * h + O)

    def flops_fwd(self) -> int:
        N, h, r = self.n_tokens, self.hidden, self.rank
        O = sum(self.out_dims)
        return 2 * N * h * O + 6 * N * h * r + 2 * N * r * O

    def flops_bwd(self) -> int:
        N, h, r = self.n_tokens, self.hidden, self.rank
        O = sum(self.out_dims)
        return 2 * N * h * O + 12 * N * h * r + 4 * N * r * O


@dataclasses.dataclass(frozen=True)
class LinearConfig:
    """One LoRA linear workload: X [n_tokens, in_features] -> Y [n_tokens, out_features]."""
    name: str
    n_tokens: int
    in_features: int
    out_features: int
    rank: int
    scale: float
    dtype: str
    w_std: float = 0.02
    b_std: float = 0.02
    a_std: Optional[float] = None
    bias: bool = False     # frozen base bias (std bias_std)
    bias_std: float = 0.5

    def a_std_for(self, in_dim: int) -> float:
        return self.a_std if self.a_std is not None else 1.0 / math.sqrt(in_dim)

    def flops_fwd(self) -> int:
        N, k, o, r = self.n_tokens, self.in_features, self.out_features, self.rank
        return 2 * N * k * o + 2 * N * k * r + 2 * N * r * o

    def flops_bwd(self) -> int:
        """dX: 2Nok + 2Nrk; dT: 2Nor; dB: 2Nor; dA: 2Nrk."""
        N, k, o, r = self.n_tokens, self.in_features, self.out_features, self.rank
        return 2 * N * k * o + 4 * N * r * k + 4 * N * r * o

    def flops(self) -> int:
        return self.flops_fwd() + self.flops_bwd()


# The benchmark workloads.  C0 takes "A ~ N(0, 1/64)" literally for all
# three adapters (variance 1/64, std 1/8).
C0 = MLPConfig("tiny_mlp_swiglu_f32", 2 * 16, 64, 172, 4, 2.0, "swiglu", "f32", a_std=1.0 / 8.0)
C1 = QKVConfig("qkv_rope_h4096_gqa32x8_d128_bf16", 4, 2048, 4096, 32, 8, 128, 8, 2.0, 1.0e4, "bf16")
C2 = MLPConfig("mlp_swiglu_h4096_i14336_bf16", 4 * 2048, 4096, 14336, 16, 2.0, "swiglu", "bf16")
C3 = MLPConfig("mlp_geglu_tanh_h3072_i24576_bf16", 4 * 2048, 3072, 24576, 16, 2.0, "geglu_tanh", "bf16")
C4_QKV = QKVConfig("qkv_rope_h896_gqa14x2_d64_bf16", 4, 1024, 896, 14, 2, 64, 16, 2.0, 1.0e6, "bf16")
C4_MLP = MLPConfig("mlp_swiglu_h896_i4864_bf16", 4 * 1024, 896, 4864, 16, 2.0, "swiglu", "bf16")

# The attention output projection of the 8B-class model (n_q * head_dim -> hidden).
C_OPROJ = LinearConfig("oproj_h4096_bf16", 4 * 2048, 4096, 4096, 16, 2.0, "bf16")

CONFIGS = {c.name: c for c in (C0, C1, C2, C3, C4_QKV, C4_MLP, C_OPROJ)}


def mlp_inputs(cfg: MLPConfig, seed: int, with_grad: bool = True) -> Dict[str, torch.Tensor]:
    """All MLP tensors (PEFT storage: W [out,in], A [r,in], B [out,r]) on the CPU."""
    N, h, i, r, dt = cfg.n_tokens, cfg.hidden, cfg.inter, cfg.rank, cfg.dtype
    shapes = {
        "X": ((N, h), 1.0),
        "W_gate": ((i, h), cfg.w_std), "A_gate": ((r, h), cfg.a_std_for(h)), "B_gate": ((i, r), cfg.b_std),
        "W_up": ((i, h), cfg.w_std), "A_up": ((r, h), cfg.a_std_for(h)), "B_up": ((i, r), cfg.b_std),
        "W_down": ((h, i), cfg.w_std), "A_down": ((r, i), cfg.a_std_for(i)), "B_down": ((h, r), cfg.b_std),
    }
    if with_grad:
        shapes["dY"] = ((N, h), 1.0)
    return {k: normal(s, std, seed, MLP_IDS[k], dt) for k, (s, std) in shapes.items()}


def qkv_inputs(cfg: QKVConfig, seed: int, with_grad: bool = True) -> Dict[str, torch.Tensor]:
    """All QKV tensors on the CPU; X is [batch*seq, hidden], dQ/dK/dV are [B, heads, S, d]."""
    N, h, r, dt = cfg.n_tokens, cfg.hidden, cfg.rank, cfg.dtype
    Oq, Ok, Ov = cfg.out_dims
    shapes = {
        "X": ((N, h), 1.0),
        "W_q": ((Oq, h), cfg.w_std), "A_q": ((r, h), cfg.a_std_for(h)), "B_q": ((Oq, r), cfg.b_std),
        "W_k": ((Ok, h), cfg.w_std), "A_k": ((r, h), cfg.a_std_for(h)), "B_k": ((Ok, r), cfg.b_std),
        "W_v": ((Ov, h), cfg.w_std), "A_v": ((r, h), cfg.a_std_for(h)), "B_v": ((Ov, r), cfg.b_std),
    }
    if cfg.bias:
        shapes.update({"b_q": ((Oq,), cfg.bias_std), "b_k": ((Ok,), cfg.bias_std), "b_v": ((Ov,), cfg.bias_std)})
    if with_grad:
        B, S, d = cfg.batch, cfg.seq, cfg.head_dim
        shapes["dQ"] = ((B, cfg.n_q, S, d), 1.0)
        shapes["dK"] = ((B, cfg.n_kv, S, d), 1.0)
        shapes["dV"] = ((B, cfg.n_kv, S, d), 1.0)
    out = {k: normal(s, std, seed, QKV_IDS[k], dt) for k, (s, std) in shapes.items()}
    if cfg.qk_norm:
        for k in ("qn_w", "kn_w"):
            out[k] = normal((cfg.head_dim,), cfg.norm_std, seed, QKV_IDS[k], dt, mean=1.0)
    return out


def linear_inputs(cfg: LinearConfig, seed: int, with_grad: bool = True) -> Dict[str, torch.Tensor]:
    """LoRA linear tensors on the CPU: X [N,in], W [out,in], A [r,in], B [out,r], dY [N,out]."""
    N, k, o, r, dt = cfg.n_tokens, cfg.in_features, cfg.out_features, cfg.rank, cfg.dtype
    shapes = {"X": ((N, k), 1.0), "W": ((o, k), cfg.w_std), "A": ((r, k), cfg.a_std_for(k)),
              "B": ((o, r), cfg.b_std)}
    if cfg.bias:
        shapes["bias"] = ((o,), cfg.bias_std)
    if with_grad:
        shapes["dY"] = ((N, o), 1.0)
    return {key: normal(s, std, seed, LINEAR_IDS[key], dt) for key, (s, std) in shapes.items()}


def to_f64(t: Dict[str, torch.Tensor]) -> Dict[str, np.ndarray]:
    """Widen every tensor exactly to a float64 numpy array (the oracle's view)."""
    return {k: v.to(torch.float64).numpy() for k, v in t.items()}
