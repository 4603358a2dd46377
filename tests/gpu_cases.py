"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI
binding on seeded inputs and the CPU oracle on the same values, and compare.

Tolerance (per output tensor): max|gpu - ref| / max|ref| <= 2e-2 in bf16 mode
and <= 1e-5 in fp32 mode.
"""
from __future__ import annotations

import dataclasses
import sys

import numpy as np
import torch

from lora_fine_tuning_mlp_amd import binding as B
from lora_fine_tuning_mlp_amd import synthetic as S
from oracle import lora_oracle as orc

TOL = {"bf16": 2e-2, "f32": 1e-5}


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def rel_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    den = float(np.max(np.abs(ref)))
    num = float(np.max(np.abs(gpu - ref)))
    if den == 0.0:
        return num
    return num / den


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


# ---------------------------------------------------------------------------
# Small parity configurations: several tiles and a ragged tail in every
# dimension the kernels tile (tokens 256, columns 256 or 128, K 64 or 32).
# ---------------------------------------------------------------------------
MLP_CASES = [
    S.C0,
    S.MLPConfig("mlp_bf16_ragged", 600, 384, 640, 16, 2.0, "swiglu", "bf16"),
    S.MLPConfig("mlp_bf16_geglu_unaligned", 300, 196, 300, 5, 2.0, "geglu_tanh", "bf16"),
    S.MLPConfig("mlp_f32_mid", 520, 256, 384, 8, 2.0, "swiglu", "f32"),
    S.MLPConfig("mlp_f32_geglu_ragged", 100, 72, 150, 3, 1.5, "geglu_tanh", "f32"),
    S.MLPConfig("mlp_bf16_long_k", 256, 1024, 512, 16, 2.0, "geglu_tanh", "bf16"),
    S.MLPConfig("mlp_bf16_geglu_erf", 520, 256, 640, 16, 2.0, "geglu_erf", "bf16"),
    S.MLPConfig("mlp_f32_geglu_erf_ragged", 130, 96, 200, 7, 2.0, "geglu_erf", "f32"),
    # few output tiles, long K: the down projection and dX split their K range
    S.MLPConfig("mlp_bf16_splitk", 64, 512, 2048, 16, 2.0, "swiglu", "bf16"),
    S.MLPConfig("mlp_bf16_splitk_cross", 100, 256, 1472, 16, 2.0, "geglu_tanh", "bf16"),
    # more dX tiles than CUs (17 x 17): runs of two column tiles, a last run of
    # one, a ragged last row block and a 64-wide last column tile
    S.MLPConfig("mlp_bf16_dx_runs_ragged", 4200, 4160, 128, 16, 2.0, "swiglu", "bf16"),
    # 17 x 16 dX tiles: the 64-wide last column tile is the second of its run
    S.MLPConfig("mlp_bf16_dx_runs_ragged_tile", 4200, 3904, 128, 16, 2.0, "geglu_tanh", "bf16"),
    # 40 x 7 dX tiles: the separate dT pass runs 7 K splits of 2 chunks over
    # the 14 chunks of [dG | dU], one of them across the dG / dU seam
    S.MLPConfig("mlp_bf16_dt_split_over_seam", 10240, 1792, 448, 16, 2.0, "swiglu", "bf16"),
    # hidden 200 = 3 x 64 + 8: the backward prologue's last 64-column chunk
    # holds 8 columns; rank 8 fills half of each 16-rank B row load
    S.MLPConfig("mlp_bf16_ragged_hidden_r8", 333, 200, 384, 8, 2.0, "swiglu", "bf16"),
]
QKV_CASES = [
    S.QKVConfig("qkv_bf16_d64", 2, 300, 384, 8, 2, 64, 8, 2.0, 1.0e4, "bf16"),
    S.QKVConfig("qkv_bf16_d128", 1, 520, 256, 4, 2, 128, 16, 2.0, 1.0e6, "bf16"),
    S.QKVConfig("qkv_f32_d64", 2, 100, 192, 4, 4, 64, 4, 2.0, 1.0e4, "f32"),
    S.QKVConfig("qkv_bf16_c4heads_ragged", 3, 77, 200, 14, 2, 64, 16, 2.0, 1.0e6, "bf16"),
    S.QKVConfig("qkv_f32_d128", 1, 40, 128, 2, 1, 128, 16, 0.5, 1.0e4, "f32"),
    S.QKVConfig("qkv_bf16_bias_c4heads", 2, 300, 896, 14, 2, 64, 16, 2.0, 1.0e6, "bf16", bias=True),
    S.QKVConfig("qkv_bf16_bias_d128", 1, 260, 256, 4, 2, 128, 8, 2.0, 1.0e4, "bf16", bias=True),
    S.QKVConfig("qkv_f32_bias_d64", 2, 50, 128, 4, 2, 64, 4, 1.5, 1.0e4, "f32", bias=True),
    S.QKVConfig("qkv_bf16_norm_d128", 2, 260, 256, 4, 2, 128, 8, 2.0, 1.0e6, "bf16", qk_norm=True),
    S.QKVConfig("qkv_bf16_norm_bias_d64_odd", 1, 300, 384, 7, 1, 64, 16, 2.0, 1.0e4, "bf16", bias=True,
                qk_norm=True),
    S.QKVConfig("qkv_f32_norm_d64", 2, 70, 128, 4, 2, 64, 4, 1.5, 1.0e4, "f32", qk_norm=True, norm_eps=1e-5),
    S.QKVConfig("qkv_f32_norm_d128", 1, 40, 64, 2, 2, 128, 16, 2.0, 1.0e4, "f32", qk_norm=True, norm_eps=0.5),
    # head_dim 64 on the fast path with one projection per tile (q 512, k 256,
    # v 256 columns) and with q, k and v all in one 256-column tile
    S.QKVConfig("qkv_bf16_d64_one_proj_per_tile", 2, 130, 128, 8, 4, 64, 16, 2.0, 1.0e4, "bf16"),
    S.QKVConfig("qkv_bf16_d64_three_proj_tile", 1, 300, 256, 2, 1, 64, 8, 2.0, 1.0e6, "bf16", bias=True),
    # head_dim 128 with more tiles than CUs (24 x 11): runs of two column
    # tiles, a later tile over q and k (plain loop), a later tile inside v
    # (ping-pong loop), a last run of one 128-wide tile, a ragged row block
    S.QKVConfig("qkv_bf16_d128_runs_ragged", 2, 3022, 128, 15, 3, 128, 16, 2.0, 1.0e4, "bf16", bias=True),
    S.QKVConfig("qkv_bf16_d128_runs_norm", 2, 3022, 128, 15, 3, 128, 8, 2.0, 1.0e6, "bf16", qk_norm=True),
]


LINEAR_CASES = [
    S.LinearConfig("linear_bf16_ragged", 600, 384, 640, 16, 2.0, "bf16"),
    S.LinearConfig("linear_bf16_unaligned", 300, 196, 300, 5, 1.5, "bf16"),
    S.LinearConfig("linear_bf16_long_k", 256, 1024, 512, 8, 2.0, "bf16"),
    S.LinearConfig("linear_f32_mid", 520, 256, 384, 8, 2.0, "f32"),
    S.LinearConfig("linear_f32_ragged", 100, 72, 150, 3, 0.5, "f32"),
    S.LinearConfig("linear_bf16_tiny", 7, 8, 16, 1, 2.0, "bf16"),
    S.LinearConfig("linear_bf16_bias", 520, 512, 384, 16, 2.0, "bf16", bias=True),
    S.LinearConfig("linear_f32_bias_ragged", 90, 40, 70, 4, 2.0, "f32", bias=True),
    S.LinearConfig("linear_bf16_splitk_uneven", 200, 1600, 256, 16, 2.0, "bf16", bias=True),
    # more output tiles than CUs (17 x 16, 17 x 17): runs of two column tiles
    # with a 64-wide last tile inside a run, or a last run of one tile
    S.LinearConfig("linear_bf16_runs_ragged", 4200, 192, 3904, 16, 2.0, "bf16", bias=True),
    S.LinearConfig("linear_bf16_runs_of_one", 4200, 128, 4160, 8, 2.0, "bf16"),
    # 200 outputs = 3 x 64 + 8: a ragged last chunk in the backward prologue
    S.LinearConfig("linear_bf16_ragged_chunk", 333, 256, 200, 16, 2.0, "bf16"),
]


def mlp_scales(cfg):
    return (cfg.scale, cfg.scale, cfg.scale)


def run_mlp_gpu(cfg: S.MLPConfig, t_cpu, dY_cpu=None, scales=None):
    scales = scales or mlp_scales(cfg)
    dev = torch.device("cuda:0")
    t = {k: v.to(dev).contiguous() for k, v in t_cpu.items() if k != "dY"}
    m = B.MLP(t, cfg.n_tokens, cfg.hidden, cfg.inter, cfg.rank, cfg.dtype, cfg.act, scales)
    m.forward()
    dY = (dY_cpu if dY_cpu is not None else t_cpu["dY"]).to(dev).contiguous()
    m.backward(dY)
    torch.cuda.synchronize()
    out = {"Y": to64(m.Y), "G": to64(m.G), "U": to64(m.U),
           "T_gate": to64(m.T[0]), "T_up": to64(m.T[1]), "T_down": to64(m.T[2]), "dX": to64(m.dX)}
    out.update({k: to64(v) for k, v in m.grads.items()})
    return out


def run_mlp_oracle(cfg: S.MLPConfig, t_cpu, dY_cpu=None, scales=None, rows=None):
    """Oracle on all tokens, or on the subset `rows` (outputs are per token;
    with dY zero outside `rows` the adapter gradients are exact too)."""
    scales = scales or mlp_scales(cfg)
    p = S.to_f64({k: v for k, v in t_cpu.items() if k != "dY"})
    dY = (dY_cpu if dY_cpu is not None else t_cpu["dY"]).to(torch.float64).numpy()
    if rows is not None:
        p["X"] = p["X"][rows]
        dY = dY[rows]
    f = orc.mlp_fwd(p, cfg.act, *scales)
    g = orc.mlp_bwd(p, dY, cfg.act, *scales)
    ref = {"Y": f["Y"], "G": f["G"], "U": f["U"], "T_gate": f["T_gate"], "T_up": f["T_up"],
           "T_down": f["T_down"], "dX": g["dX"]}
    for n in ("gate", "up", "down"):
        ref["dA_" + n] = g["dA_" + n]
        ref["dB_" + n] = g["dB_" + n]
    return ref


def run_qkv_gpu(cfg: S.QKVConfig, t_cpu, grads_cpu=None, scales=None):
    scales = scales or (cfg.scale,) * 3
    dev = torch.device("cuda:0")
    t = {k: v.to(dev).contiguous() for k, v in t_cpu.items() if k not in ("dQ", "dK", "dV")}
    m = B.QKV(t, cfg.batch, cfg.seq, cfg.hidden, cfg.n_q, cfg.n_kv, cfg.head_dim, cfg.rank, cfg.dtype, cfg.theta,
              scales, cfg.norm_eps)
    m.forward()
    gc = grads_cpu if grads_cpu is not None else t_cpu
    m.backward(gc["dQ"].to(dev).contiguous(), gc["dK"].to(dev).contiguous(), gc["dV"].to(dev).contiguous())
    torch.cuda.synchronize()
    out = {"Q": to64(m.Q), "K": to64(m.K), "V": to64(m.V), "T_q": to64(m.T[0]), "T_k": to64(m.T[1]),
           "T_v": to64(m.T[2]), "dX": to64(m.dX)}
    if m.norm is not None:
        Oq = cfg.n_q * cfg.head_dim
        out.update({"P_q": to64(m.Pn[:, :Oq]), "P_k": to64(m.Pn[:, Oq:]), "rinv_q": to64(m.rinv[:, :cfg.n_q]),
                    "rinv_k": to64(m.rinv[:, cfg.n_q:])})
    out.update({k: to64(v) for k, v in m.grads.items()})
    return out


def run_qkv_oracle(cfg: S.QKVConfig, t_cpu, grads_cpu=None, scales=None):
    scales = scales or (cfg.scale,) * 3
    p = S.to_f64({k: v for k, v in t_cpu.items() if k not in ("dQ", "dK", "dV")})
    gc = grads_cpu if grads_cpu is not None else t_cpu
    dQ, dK, dV = (gc[k].to(torch.float64).numpy() for k in ("dQ", "dK", "dV"))
    shape = dict(batch=cfg.batch, seq=cfg.seq, n_q=cfg.n_q, n_kv=cfg.n_kv, head_dim=cfg.head_dim, theta=cfg.theta)
    f = orc.qkv_fwd(p, scales=scales, norm_eps=cfg.norm_eps, **shape)
    g = orc.qkv_bwd(p, dQ, dK, dV, scales=scales, norm_eps=cfg.norm_eps, **shape)
    ref = {"Q": f["Q"], "K": f["K"], "V": f["V"], "T_q": f["T_q"], "T_k": f["T_k"], "T_v": f["T_v"],
           "dX": g["dX"]}
    for k in ("P_q", "P_k", "rinv_q", "rinv_k"):
        if k in f:
            ref[k] = f[k]
    for n in "qkv":
        ref["dA_" + n] = g["dA_" + n]
        ref["dB_" + n] = g["dB_" + n]
    return ref


def run_linear_gpu(cfg: S.LinearConfig, t_cpu, dY_cpu=None):
    dev = torch.device("cuda:0")
    t = {k: v.to(dev).contiguous() for k, v in t_cpu.items() if k != "dY"}
    m = B.Linear(t, cfg.n_tokens, cfg.in_features, cfg.out_features, cfg.rank, cfg.dtype, cfg.scale)
    m.forward()
    dY = (dY_cpu if dY_cpu is not None else t_cpu["dY"]).to(dev).contiguous()
    m.backward(dY)
    torch.cuda.synchronize()
    out = {"Y": to64(m.Y), "T": to64(m.T), "dX": to64(m.dX)}
    out.update({k: to64(v) for k, v in m.grads.items()})
    return out


def run_linear_oracle(cfg: S.LinearConfig, t_cpu, dY_cpu=None, rows=None):
    p = S.to_f64({k: v for k, v in t_cpu.items() if k != "dY"})
    dY = (dY_cpu if dY_cpu is not None else t_cpu["dY"]).to(torch.float64).numpy()
    X = p["X"]
    if rows is not None:
        X, dY = X[rows], dY[rows]
    Y, T = orc.lora_linear(X, p["W"], p["A"], p["B"], cfg.scale, p.get("bias"))
    dX, dA, dB, _ = orc.lora_linear_bwd(dY, X, T, p["W"], p["A"], p["B"], cfg.scale)
    return {"Y": Y, "T": T, "dX": dX, "dA": dA, "dB": dB}


def compare(name: str, gpu, ref, tol: float, keys=None):
    """Assert every tensor within tol; returns the per-tensor errors."""
    errs = {}
    bad = []
    for k in keys or ref:
        a, b = gpu[k], ref[k]
        assert a.shape == b.shape, (name, k, a.shape, b.shape)
        if not np.all(np.isfinite(a)):
            bad.append((k, "non-finite"))
            continue
        e = rel_err(a, b)
        errs[k] = e
        if e > tol:
            bad.append((k, e))
    say(f"{name}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert not bad, f"{name}: out of tolerance {tol}: {bad}"
    return errs
