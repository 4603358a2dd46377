"""Pins for the CPU oracle: checks against facts fixed by the pages and the
mathematics, never against the oracle itself.

Every ``check_*`` takes the oracle module as its argument so the same checks
can run against deliberately broken copies (tests/test_oracle_mutations.py)
and show that a planted mistake is caught.

Kinds of pin used here:
  * hand-worked examples under tests/golden/ (derivations written there);
  * closed forms and limits of the activations;
  * library routines for special cases (torch fp64 F.silu / F.gelu, torch
    autograd of the plain definition, complex multiplication for RoPE);
  * identities of the math (LoRA merge W + s B A, B=0 / A=0 / s=0 cases,
    linearity in s, RoPE orthogonality and relative-position property);
  * central finite differences on tiny shapes.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
ACTS = ("swiglu", "geglu_tanh")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    den = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    return float(np.max(np.abs(a - b))) / den if a.size else 0.0


def _rng(seed):
    return np.random.default_rng(seed)


def tiny_mlp(seed=0, N=3, h=8, i=12, r=2, zero=None):
    g = _rng(seed)
    p = {"X": g.standard_normal((N, h))}
    for name, (o, n) in {"gate": (i, h), "up": (i, h), "down": (h, i)}.items():
        p["W_" + name] = g.standard_normal((o, n)) * 0.3
        p["A_" + name] = g.standard_normal((r, n)) * 0.5
        p["B_" + name] = g.standard_normal((o, r)) * 0.5
    if zero:
        for k in list(p):
            if k.startswith(zero):
                p[k] = np.zeros_like(p[k])
    dY = g.standard_normal((N, h))
    return p, dY


def tiny_qkv(seed=0, batch=1, seq=3, h=8, n_q=4, n_kv=2, d=4, r=2, zero=None):
    g = _rng(seed)
    p = {"X": g.standard_normal((batch * seq, h))}
    outs = {"q": n_q * d, "k": n_kv * d, "v": n_kv * d}
    for name, o in outs.items():
        p["W_" + name] = g.standard_normal((o, h)) * 0.3
        p["A_" + name] = g.standard_normal((r, h)) * 0.5
        p["B_" + name] = g.standard_normal((o, r)) * 0.5
    if zero:
        for k in list(p):
            if k.startswith(zero):
                p[k] = np.zeros_like(p[k])
    grads = {"dQ": g.standard_normal((batch, n_q, seq, d)),
             "dK": g.standard_normal((batch, n_kv, seq, d)),
             "dV": g.standard_normal((batch, n_kv, seq, d))}
    return p, grads


MLP_SCALES = (2.0, 1.5, 0.75)
QKV_SCALES = (2.0, 1.25, 0.5)
QKV_SHAPE = dict(batch=1, seq=3, n_q=4, n_kv=2, head_dim=4, theta=10.0)


# ---------------------------------------------------------------------------
# LoRA linear
# ---------------------------------------------------------------------------

def check_lora_linear_worked(orc):
    g = _load("lora_linear_worked.json")
    Z, W, A, B = (np.array(g[k], np.float64) for k in ("Z", "W", "A", "B"))
    dY = np.array(g["dY"], np.float64)
    Y, T = orc.lora_linear(Z, W, A, B, g["s"])
    e = g["expected"]
    assert np.array_equal(T, np.array(e["T"], np.float64)), T
    assert np.allclose(Y, e["Y"], rtol=0, atol=1e-15), Y
    dZ, dA, dB, dT = orc.lora_linear_bwd(dY, Z, T, W, A, B, g["s"])
    for name, v in (("dZ", dZ), ("dA", dA), ("dB", dB), ("dT", dT)):
        assert np.allclose(v, e[name], rtol=0, atol=1e-15), (name, v)


def check_lora_merge_identity(orc):
    """L(Z) = Z (W + s B A)^T and dZ = dY (W + s B A) (textbook LoRA merge)."""
    g = _rng(1)
    for (N, i, o, r, s) in ((5, 7, 9, 3, 2.0), (4, 16, 6, 5, -0.7)):
        Z, W = g.standard_normal((N, i)), g.standard_normal((o, i))
        A, B = g.standard_normal((r, i)), g.standard_normal((o, r))
        dY = g.standard_normal((N, o))
        Weff = W + s * (B @ A)
        Y, T = orc.lora_linear(Z, W, A, B, s)
        assert _rel(Y, Z @ Weff.T) < 1e-12
        dZ, _, _, _ = orc.lora_linear_bwd(dY, Z, T, W, A, B, s)
        assert _rel(dZ, dY @ Weff) < 1e-12


def check_lora_linear_vs_autograd(orc):
    """dA, dB, dZ against torch fp64 autograd of the plain definition."""
    g = _rng(2)
    N, i, o, r, s = 6, 5, 7, 3, 1.7
    Z, W = g.standard_normal((N, i)), g.standard_normal((o, i))
    A, B = g.standard_normal((r, i)), g.standard_normal((o, r))
    dY = g.standard_normal((N, o))
    tZ, tA, tB = (torch.tensor(v, requires_grad=True) for v in (Z, A, B))
    tW = torch.tensor(W)
    Yt = F.linear(tZ, tW) + s * F.linear(F.linear(tZ, tA), tB)
    Yt.backward(torch.tensor(dY))
    Y, T = orc.lora_linear(Z, W, A, B, s)
    dZ, dA, dB, _ = orc.lora_linear_bwd(dY, Z, T, W, A, B, s)
    assert _rel(Y, Yt.detach().numpy()) < 1e-12
    assert _rel(dZ, tZ.grad.numpy()) < 1e-12
    assert _rel(dA, tA.grad.numpy()) < 1e-12
    assert _rel(dB, tB.grad.numpy()) < 1e-12


def check_lora_linear_bias_vs_torch(orc):
    """Frozen base bias: Y against torch F.linear(Z, W, b) plus the adapter;
    gradients against autograd with b a constant (they do not depend on b)."""
    g = _rng(3)
    N, i, o, r, s = 5, 6, 4, 2, 1.25
    Z, W = g.standard_normal((N, i)), g.standard_normal((o, i))
    A, B = g.standard_normal((r, i)), g.standard_normal((o, r))
    b, dY = g.standard_normal(o) * 3.0, g.standard_normal((N, o))
    tZ, tA, tB = (torch.tensor(v, requires_grad=True) for v in (Z, A, B))
    Yt = F.linear(tZ, torch.tensor(W), torch.tensor(b)) + s * F.linear(F.linear(tZ, tA), tB)
    Yt.backward(torch.tensor(dY))
    Y, T = orc.lora_linear(Z, W, A, B, s, b)
    assert _rel(Y, Yt.detach().numpy()) < 1e-12
    Y0, _ = orc.lora_linear(Z, W, A, B, s)
    assert _rel(Y - Y0, np.broadcast_to(b, Y.shape)) < 1e-12
    dZ, dA, dB, _ = orc.lora_linear_bwd(dY, Z, T, W, A, B, s)
    assert _rel(dZ, tZ.grad.numpy()) < 1e-12
    assert _rel(dA, tA.grad.numpy()) < 1e-12
    assert _rel(dB, tB.grad.numpy()) < 1e-12


# ---------------------------------------------------------------------------
# Activations
# ---------------------------------------------------------------------------

def check_activation_closed_forms(orc):
    for act in ("swiglu", "geglu_tanh", "geglu_erf"):
        phi, dphi = orc.activation(act)
        z = np.array([0.0])
        assert phi(z)[0] == 0.0, act
        assert abs(dphi(z)[0] - 0.5) < 1e-15, act
        big = np.array([40.0, -40.0])
        assert abs(phi(big)[0] - 40.0) < 1e-9 and abs(phi(big)[1]) < 1e-9, act
        assert abs(dphi(big)[0] - 1.0) < 1e-9 and abs(dphi(big)[1]) < 1e-9, act
    # sigmoid(ln 3) = 3/4 exactly, so silu(ln 3) = 0.75 ln 3 and
    # silu'(ln 3) = 0.75 (1 + ln 3 / 4).
    phi, dphi = orc.activation("swiglu")
    l3 = np.array([math.log(3.0)])
    assert abs(phi(l3)[0] - 0.75 * math.log(3.0)) < 1e-15
    assert abs(dphi(l3)[0] - 0.75 * (1.0 + math.log(3.0) / 4.0)) < 1e-15


def check_activation_vs_torch(orc):
    """Elementwise against torch fp64 F.silu / F.gelu on a grid in [-20, 20]."""
    grid = np.linspace(-20.0, 20.0, 4001)
    t = torch.tensor(grid, requires_grad=True)
    lib = {"swiglu": lambda x: F.silu(x),
           "geglu_tanh": lambda x: F.gelu(x, approximate="tanh"),
           "geglu_erf": lambda x: F.gelu(x)}
    for act, f in lib.items():
        phi, dphi = orc.activation(act)
        if t.grad is not None:
            t.grad = None
        y = f(t)
        y.sum().backward()
        assert np.max(np.abs(phi(grid) - y.detach().numpy())) < 1e-13, act
        assert np.max(np.abs(dphi(grid) - t.grad.numpy())) < 1e-13, act


# ---------------------------------------------------------------------------
# MLP
# ---------------------------------------------------------------------------

def _torch_mlp(p, act, scales):
    """The LoRA MLP written with torch ops (a separate implementation)."""
    fn = {"swiglu": F.silu, "geglu_tanh": lambda x: F.gelu(x, approximate="tanh")}[act]
    sg, su, sd = scales

    def lin(z, n, s):
        return F.linear(z, p["W_" + n]) + s * F.linear(F.linear(z, p["A_" + n]), p["B_" + n])
    X = p["X"]
    return lin(fn(lin(X, "gate", sg)) * lin(X, "up", su), "down", sd)


def check_mlp_base_path(orc):
    """B = 0 everywhere: the MLP is the plain linear + GLU (torch F.linear / F.silu / F.gelu)."""
    for act in ACTS:
        p, _ = tiny_mlp(3, zero="B_")
        f = orc.mlp_fwd(p, act, *MLP_SCALES)
        tp = {k: torch.tensor(v) for k, v in p.items()}
        fn = {"swiglu": F.silu, "geglu_tanh": lambda x: F.gelu(x, approximate="tanh")}[act]
        G = F.linear(tp["X"], tp["W_gate"])
        U = F.linear(tp["X"], tp["W_up"])
        Y = F.linear(fn(G) * U, tp["W_down"])
        assert _rel(f["G"], G.numpy()) < 1e-13
        assert _rel(f["U"], U.numpy()) < 1e-13
        assert _rel(f["Y"], Y.numpy()) < 1e-13


def check_mlp_adapter_only(orc):
    """W = 0: only the adapter path remains; compare with the torch implementation."""
    for act in ACTS:
        p, _ = tiny_mlp(4, zero="W_")
        tp = {k: torch.tensor(v) for k, v in p.items()}
        Y = _torch_mlp(tp, act, MLP_SCALES).numpy()
        assert np.max(np.abs(Y)) > 1e-3
        assert _rel(orc.mlp_fwd(p, act, *MLP_SCALES)["Y"], Y) < 1e-12


def check_mlp_linear_in_scale(orc):
    """Each projection's output is affine in its scale: L(s) - L(0) = s (L(1) - L(0))."""
    p, _ = tiny_mlp(5)
    for act in ACTS:
        f0 = orc.mlp_fwd(p, act, 0.0, 0.0, 0.0)
        f1 = orc.mlp_fwd(p, act, 1.0, 1.0, 0.0)
        fs = orc.mlp_fwd(p, act, 2.5, 2.5, 0.0)
        for k in ("G", "U"):
            assert _rel(fs[k] - f0[k], 2.5 * (f1[k] - f0[k])) < 1e-12
        d1 = orc.mlp_fwd(p, act, 0.0, 0.0, 1.0)
        ds = orc.mlp_fwd(p, act, 0.0, 0.0, -3.0)
        assert _rel(ds["Y"] - f0["Y"], -3.0 * (d1["Y"] - f0["Y"])) < 1e-12


def check_mlp_exact_zeros(orc):
    """B = 0 => every dA is exactly 0; A = 0 => every dB is exactly 0; s = 0 => both."""
    for act in ACTS:
        p, dY = tiny_mlp(6, zero="B_")
        g = orc.mlp_bwd(p, dY, act, *MLP_SCALES)
        for n in ("gate", "up", "down"):
            assert not np.any(g["dA_" + n]), n
            assert np.any(g["dB_" + n]), n
        p, dY = tiny_mlp(7, zero="A_")
        g = orc.mlp_bwd(p, dY, act, *MLP_SCALES)
        for n in ("gate", "up", "down"):
            assert not np.any(g["dB_" + n]), n
        p, dY = tiny_mlp(8)
        g = orc.mlp_bwd(p, dY, act, 0.0, 0.0, 0.0)
        for n in ("gate", "up", "down"):
            assert not np.any(g["dA_" + n]) and not np.any(g["dB_" + n]), n


def _fd_check(loss, p, analytic, keys, tol=1e-7):
    """Central differences of loss(p) in every entry of p[k] for k in keys."""
    for k in keys:
        base = p[k]
        num = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            x0 = base[idx]
            eps = 1e-6 * max(1.0, abs(x0))
            base[idx] = x0 + eps
            lp = loss(p)
            base[idx] = x0 - eps
            lm = loss(p)
            base[idx] = x0
            num[idx] = (lp - lm) / (2 * eps)
        den = max(1.0, float(np.max(np.abs(analytic[k]))))
        err = float(np.max(np.abs(num - analytic[k]))) / den
        assert err < tol, (k, err)


def check_mlp_finite_differences(orc):
    for act in ACTS:
        p, dY = tiny_mlp(9)
        g = orc.mlp_bwd(p, dY, act, *MLP_SCALES)
        analytic = {"X": g["dX"]}
        for n in ("gate", "up", "down"):
            analytic["A_" + n] = g["dA_" + n]
            analytic["B_" + n] = g["dB_" + n]

        def loss(pp):
            return float(np.sum(dY * orc.mlp_fwd(pp, act, *MLP_SCALES)["Y"]))
        _fd_check(loss, p, analytic, list(analytic))


def check_mlp_vs_autograd(orc):
    for act in ACTS:
        p, dY = tiny_mlp(10, N=5, h=6, i=10, r=3)
        tp = {k: torch.tensor(v, requires_grad=(k[0] in "XAB")) for k, v in p.items()}
        Y = _torch_mlp(tp, act, MLP_SCALES)
        Y.backward(torch.tensor(dY))
        f = orc.mlp_fwd(p, act, *MLP_SCALES)
        g = orc.mlp_bwd(p, dY, act, *MLP_SCALES)
        assert _rel(f["Y"], Y.detach().numpy()) < 1e-12
        assert _rel(g["dX"], tp["X"].grad.numpy()) < 1e-12
        for n in ("gate", "up", "down"):
            assert _rel(g["dA_" + n], tp["A_" + n].grad.numpy()) < 1e-12, n
            assert _rel(g["dB_" + n], tp["B_" + n].grad.numpy()) < 1e-12, n


# ---------------------------------------------------------------------------
# RoPE and head split
# ---------------------------------------------------------------------------

def check_rope_worked(orc):
    g = _load("rope_worked.json")
    d, theta = g["head_dim"], g["theta"]
    ang = orc.rope_angles(3, d, theta)
    x = np.array(g["x"], np.float64)
    for pos, angles in g["angles_by_position"].items():
        pos = int(pos)
        assert np.allclose(ang[pos], angles, rtol=1e-15, atol=0), (pos, ang[pos])
        y = orc.rope_rotate(np.tile(x, (3, 1)), ang)[pos]
        for (a, b), t in zip(g["pairs"], angles):
            ea = x[a] * math.cos(t) - x[b] * math.sin(t)
            eb = x[b] * math.cos(t) + x[a] * math.sin(t)
            assert abs(y[a] - ea) < 1e-15 and abs(y[b] - eb) < 1e-15, (pos, a, b)


def check_rope_invariants(orc):
    g = _rng(11)
    S, d, theta = 37, 8, 1.0e4
    ang = orc.rope_angles(S, d, theta)
    assert np.array_equal(ang[:, 0], np.arange(S, dtype=np.float64))   # j = 0: angle = position
    x = g.standard_normal((2, 3, S, d))
    y = orc.rope_rotate(x, ang)
    assert np.array_equal(y[..., 0, :], x[..., 0, :])                   # position 0 is the identity
    h = d // 2
    nx = x[..., :h] ** 2 + x[..., h:] ** 2
    ny = y[..., :h] ** 2 + y[..., h:] ** 2
    assert np.max(np.abs(nx - ny)) < 1e-13                               # per-pair norms
    assert _rel(orc.rope_rotate_transpose(y, ang), x) < 1e-14             # R^T R = I
    z = g.standard_normal(x.shape)                                       # adjoint: <Rx, z> = <x, R^T z>
    assert abs(np.sum(y * z) - np.sum(x * orc.rope_rotate_transpose(z, ang))) < 1e-11
    # relative position: <R(m) q, R(n) k> depends only on m - n
    q, k = g.standard_normal(d), g.standard_normal(d)
    Q = orc.rope_rotate(np.tile(q, (S, 1)), ang)
    K = orc.rope_rotate(np.tile(k, (S, 1)), ang)
    for (m, n, c) in ((5, 2, 7), (30, 11, 4), (3, 3, 20)):
        assert abs(Q[m] @ K[n] - Q[m + c] @ K[n + c]) < 1e-11


def check_rope_vs_complex(orc):
    """(x_j + i x_{j+d/2}) * exp(i * angle), computed with complex arithmetic."""
    g = _rng(12)
    S, d, theta = 64, 16, 1.0e6
    x = g.standard_normal((2, 5, S, d))
    j = np.arange(d // 2)
    ang = np.arange(S)[:, None] * np.exp(-(2.0 * j / d) * math.log(theta))[None, :]
    assert _rel(orc.rope_angles(S, d, theta), ang) < 1e-13
    z = (x[..., : d // 2] + 1j * x[..., d // 2:]) * np.exp(1j * ang)
    ref = np.concatenate([z.real, z.imag], axis=-1)
    assert _rel(orc.rope_rotate(x, orc.rope_angles(S, d, theta)), ref) < 1e-13


def check_head_split_bruteforce(orc):
    g = _rng(13)
    B, S, nh, d = 2, 3, 4, 6
    P = g.standard_normal((B * S, nh * d))
    Q = orc.head_split(P, B, S, nh, d)
    assert Q.shape == (B, nh, S, d)
    for b in range(B):
        for hd in range(nh):
            for s in range(S):
                for j in range(d):
                    assert Q[b, hd, s, j] == P[b * S + s, hd * d + j]
    assert np.array_equal(orc.head_unsplit(Q), P)


# ---------------------------------------------------------------------------
# QKV
# ---------------------------------------------------------------------------

def _torch_qkv(tp, shape, scales, eps=1e-6):
    """QKV written with torch ops; RoPE as complex multiplication; optional
    q/k norm with torch's F.rms_norm over the head dimension."""
    B, S, nq, nkv, d, theta = (shape[k] for k in ("batch", "seq", "n_q", "n_kv", "head_dim", "theta"))
    j = torch.arange(d // 2, dtype=torch.float64)
    ang = torch.arange(S, dtype=torch.float64)[:, None] * torch.exp(-(2.0 * j / d) * math.log(theta))[None, :]
    rot = torch.polar(torch.ones_like(ang), ang)
    out = {}
    for name, heads, s in zip("qkv", (nq, nkv, nkv), scales):
        P = F.linear(tp["X"], tp["W_" + name], tp.get("b_" + name)) + \
            s * F.linear(F.linear(tp["X"], tp["A_" + name]), tp["B_" + name])
        Z = P.reshape(B, S, heads, d).permute(0, 2, 1, 3)
        wn = tp.get({"q": "qn_w", "k": "kn_w"}.get(name, ""))
        if wn is not None:
            Z = F.rms_norm(Z, (d,), weight=wn, eps=eps)
        if name != "v":
            c = torch.complex(Z[..., : d // 2], Z[..., d // 2:]) * rot
            Z = torch.cat([c.real, c.imag], dim=-1)
        out[name.upper()] = Z
    return out


def check_qkv_base_path(orc):
    """B = 0: Q/K/V are the head-split base projections, Q and K rotated."""
    p, _ = tiny_qkv(14, zero="B_")
    o = orc.qkv_fwd(p, scales=QKV_SCALES, **QKV_SHAPE)
    tp = {k: torch.tensor(v) for k, v in p.items()}
    ref = _torch_qkv(tp, QKV_SHAPE, QKV_SCALES)
    for k in "QKV":
        assert _rel(o[k], ref[k].numpy()) < 1e-13, k


def check_qkv_vs_autograd(orc):
    p, gr = tiny_qkv(15, batch=2, seq=5, h=6, n_q=6, n_kv=2, d=8, r=3)
    shape = dict(batch=2, seq=5, n_q=6, n_kv=2, head_dim=8, theta=50.0)
    tp = {k: torch.tensor(v, requires_grad=(k[0] in "XAB")) for k, v in p.items()}
    ref = _torch_qkv(tp, shape, QKV_SCALES)
    loss = sum((ref[k] * torch.tensor(gr["d" + k])).sum() for k in "QKV")
    loss.backward()
    o = orc.qkv_fwd(p, scales=QKV_SCALES, **shape)
    g = orc.qkv_bwd(p, gr["dQ"], gr["dK"], gr["dV"], scales=QKV_SCALES, **shape)
    for k in "QKV":
        assert _rel(o[k], ref[k].detach().numpy()) < 1e-12, k
    assert _rel(g["dX"], tp["X"].grad.numpy()) < 1e-12
    for n in "qkv":
        assert _rel(g["dA_" + n], tp["A_" + n].grad.numpy()) < 1e-12, n
        assert _rel(g["dB_" + n], tp["B_" + n].grad.numpy()) < 1e-12, n


def check_qkv_bias_vs_autograd(orc):
    """Frozen q/k/v biases go in before RoPE (torch's F.linear bias, then the
    complex rotation); the backward, which ignores them, still matches
    autograd through the biased forward."""
    p, gr = tiny_qkv(19, batch=2, seq=4, h=6, n_q=4, n_kv=2, d=6, r=2)
    shape = dict(batch=2, seq=4, n_q=4, n_kv=2, head_dim=6, theta=30.0)
    g = _rng(20)
    for n, o in (("q", 24), ("k", 12), ("v", 12)):
        p["b_" + n] = g.standard_normal(o) * 2.0
    tp = {k: torch.tensor(v, requires_grad=(k[0] in "XAB")) for k, v in p.items()}
    ref = _torch_qkv(tp, shape, QKV_SCALES)
    loss = sum((ref[k] * torch.tensor(gr["d" + k])).sum() for k in "QKV")
    loss.backward()
    o = orc.qkv_fwd(p, scales=QKV_SCALES, **shape)
    for k in "QKV":
        assert _rel(o[k], ref[k].detach().numpy()) < 1e-12, k
    # V has no rotation: its bias shifts every position by the same vector.
    nob = {k: v for k, v in p.items() if not k.startswith("b_")}
    o0 = orc.qkv_fwd(nob, scales=QKV_SCALES, **shape)
    bv = p["b_v"].reshape(2, 6)[None, :, None, :]
    assert _rel(o["V"] - o0["V"], np.broadcast_to(bv, o["V"].shape)) < 1e-12
    # Q at position 0 is unrotated: its bias shows up unchanged there.
    bq = p["b_q"].reshape(4, 6)[None, :, :]
    assert _rel(o["Q"][:, :, 0] - o0["Q"][:, :, 0], np.broadcast_to(bq, o["Q"][:, :, 0].shape)) < 1e-12
    gq = orc.qkv_bwd(p, gr["dQ"], gr["dK"], gr["dV"], scales=QKV_SCALES, **shape)
    assert _rel(gq["dX"], tp["X"].grad.numpy()) < 1e-12
    for n in "qkv":
        assert _rel(gq["dA_" + n], tp["A_" + n].grad.numpy()) < 1e-12, n
        assert _rel(gq["dB_" + n], tp["B_" + n].grad.numpy()) < 1e-12, n


def check_rms_norm_vs_torch(orc):
    g = _rng(21)
    x, w, dy = g.standard_normal((3, 5, 8)), g.standard_normal(8), g.standard_normal((3, 5, 8))
    for eps in (1e-6, 0.3):
        tx = torch.tensor(x, requires_grad=True)
        y = F.rms_norm(tx, (8,), weight=torch.tensor(w), eps=eps)
        y.backward(torch.tensor(dy))
        yo, rinv = orc.rms_norm(x, w, eps)
        assert _rel(yo, y.detach().numpy()) < 1e-13
        # rinv is the inverse root mean square: rinv^2 (mean x^2 + eps) = 1
        assert np.max(np.abs(rinv ** 2 * (np.mean(x * x, axis=-1) + eps) - 1.0)) < 1e-13
        assert _rel(orc.rms_norm_bwd(dy, x, w, eps), tx.grad.numpy()) < 1e-13


def check_qkv_norm_vs_autograd(orc):
    """q/k norm (F.rms_norm) between the head split and RoPE, forward and
    backward, against torch autograd; with eps = 0 Q is also invariant under
    scaling the whole q projection (W_q, B_q, b_q) by a positive constant."""
    p, gr = tiny_qkv(22, batch=2, seq=4, h=6, n_q=4, n_kv=2, d=8, r=2)
    shape = dict(batch=2, seq=4, n_q=4, n_kv=2, head_dim=8, theta=20.0)
    g = _rng(23)
    p["qn_w"], p["kn_w"] = 1.0 + 0.5 * g.standard_normal(8), 1.0 + 0.5 * g.standard_normal(8)
    p["b_q"] = g.standard_normal(32)
    eps = 1e-5
    tp = {k: torch.tensor(v, requires_grad=(k[0] in "XAB")) for k, v in p.items()}
    ref = _torch_qkv(tp, shape, QKV_SCALES, eps)
    loss = sum((ref[k] * torch.tensor(gr["d" + k])).sum() for k in "QKV")
    loss.backward()
    o = orc.qkv_fwd(p, scales=QKV_SCALES, norm_eps=eps, **shape)
    gq = orc.qkv_bwd(p, gr["dQ"], gr["dK"], gr["dV"], scales=QKV_SCALES, norm_eps=eps, **shape)
    for k in "QKV":
        assert _rel(o[k], ref[k].detach().numpy()) < 1e-12, k
    assert _rel(gq["dX"], tp["X"].grad.numpy()) < 1e-12
    for n in "qkv":
        assert _rel(gq["dA_" + n], tp["A_" + n].grad.numpy()) < 1e-12, n
        assert _rel(gq["dB_" + n], tp["B_" + n].grad.numpy()) < 1e-12, n
    assert o["rinv_q"].shape == (8, 4) and o["rinv_k"].shape == (8, 2) and "rinv_v" not in o
    p0 = dict(p)
    o0 = orc.qkv_fwd(p0, scales=QKV_SCALES, norm_eps=0.0, **shape)
    for k in ("W_q", "B_q", "b_q"):
        p0[k] = p[k] * 3.5
    o1 = orc.qkv_fwd(p0, scales=QKV_SCALES, norm_eps=0.0, **shape)
    assert _rel(o1["Q"], o0["Q"]) < 1e-13
    assert not np.allclose(o1["P_q"], o0["P_q"])


def check_qkv_finite_differences(orc):
    p, gr = tiny_qkv(16)
    g = orc.qkv_bwd(p, gr["dQ"], gr["dK"], gr["dV"], scales=QKV_SCALES, **QKV_SHAPE)
    analytic = {"X": g["dX"]}
    for n in "qkv":
        analytic["A_" + n] = g["dA_" + n]
        analytic["B_" + n] = g["dB_" + n]

    def loss(pp):
        o = orc.qkv_fwd(pp, scales=QKV_SCALES, **QKV_SHAPE)
        return float(sum(np.sum(gr["d" + k] * o[k]) for k in "QKV"))
    _fd_check(loss, p, analytic, list(analytic))


def check_qkv_exact_zeros(orc):
    p, gr = tiny_qkv(17, zero="B_")
    g = orc.qkv_bwd(p, gr["dQ"], gr["dK"], gr["dV"], scales=QKV_SCALES, **QKV_SHAPE)
    for n in "qkv":
        assert not np.any(g["dA_" + n]) and np.any(g["dB_" + n]), n
    p, gr = tiny_qkv(18, zero="A_")
    g = orc.qkv_bwd(p, gr["dQ"], gr["dK"], gr["dV"], scales=QKV_SCALES, **QKV_SHAPE)
    for n in "qkv":
        assert not np.any(g["dB_" + n]), n


ALL_CHECKS = [v for k, v in sorted(globals().items()) if k.startswith("check_")]
