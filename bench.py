"""Benchmark: fused LoRA QKV + MLP forward and backward on one MI355X.

One step = LoRA QKV + RoPE fwd+bwd at 4 x 2048 tokens, h = 4096, 32/8 heads of
128, r = 8, plus LoRA MLP (SwiGLU) fwd+bwd at 8192 tokens, h = 4096,
i = 14336, r = 16, all bf16 with fp32 accumulation, on seeded synthetic
inputs resident in HBM.  Throughput is algorithmic FLOPs (frozen base weights:
no dW; elementwise work not counted) per second.

Prints one JSON line.  Besides the headline value it carries
  legs:          separate legs, outside `value`: one LoRA linear fwd+bwd at
                 the attention output projection's shape (8192 x 4096 -> 4096),
                 the headline QKV shape with per-head q/k RMSNorm, the GeGLU-tanh
                 MLP at 8192 x 3072 -> 24576, and the small-shape regime
                 (4 x 1024 tokens, h 896: MLP i 4864, QKV 14/2 heads of 64), each
                 with its MFMA fraction and its HBM rate on planned bytes;
  roofline:      the dominant kernel's achieved TFLOP/s against the bf16
                 dense MFMA peak, timed live with HIP events around each launch
                 on the stream it runs on;
  cpu_baseline:  the CPU float64 oracle timed on a bounded token sample of the
                 same workload (rank 0, N = 1 only).
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "LoRA MLP+QKV fwd+bwd TFLOP/s and % bf16 MFMA peak, 8192 tokens, h=4096"
PEAK_BF16_TFLOPS = 2500.0          # MI355X dense bf16 MFMA (no sparsity)
PEAK_HBM_GBS = 8000.0


def kernel_flops(qkv, mlp):
    """Algorithmic FLOPs per launch of each kernel at these shapes (no dW,
    rank-r work counted once, elementwise not counted)."""
    N, h, i, r = mlp.n_tokens, mlp.hidden, mlp.inter, mlp.rank
    Nq, hq, rq = qkv.n_tokens, qkv.hidden, qkv.rank
    O = sum(qkv.out_dims)
    return {
        "k_gateup_fwd": 4 * N * h * i + 4 * N * h * r + 4 * N * r * i,
        "k_linear_fwd": 2 * N * i * h + 2 * N * i * r + 2 * N * r * h,
        "k_qkv_fwd": 2 * Nq * hq * O + 6 * Nq * hq * rq + 2 * Nq * rq * O,
        "k_down_bwd": 2 * N * h * i + 8 * N * r * i,
        "k_mlp_dt": 4 * N * i * r,
        "k_mlp_dx_bwd": 4 * N * i * h + 8 * N * r * h,
        "k_proj_dx_bwd": 2 * Nq * O * hq + 12 * Nq * rq * hq,
    }


def linear_kernel_flops(cfg):
    N, k, o, r = cfg.n_tokens, cfg.in_features, cfg.out_features, cfg.rank
    return {"k_linear_fwd": 2 * N * k * o + 2 * N * k * r + 2 * N * r * o,
            "k_proj_dx_bwd": 2 * N * o * k + 4 * N * r * k}


def time_leg(step, steps: int, warmup: int, kflops=None, flush=None):
    """Warm up, then time `steps` calls of `step` with HIP events on the
    current stream (the library's per-launch recorder off); a second pass of
    the same calls with the recorder on gives the per-kernel averages.

    With `flush` (a device tensor larger than the 256 MB MALL and the L2s),
    the tensor is overwritten before every call and each call is timed on
    its own, so every call starts with its inputs in HBM only."""
    import torch
    from lora_fine_tuning_mlp_amd import binding as B

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if flush is None:
        e0.record(stream)
        for _ in range(steps):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
    else:
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a, b in ev:
            flush.fill_(1.0)
            a.record(stream)
            step()
            b.record(stream)
        torch.cuda.synchronize()
        ms = sum(a.elapsed_time(b) for a, b in ev) / steps
    B.timing_reset()
    B.timing_enable(True)
    for _ in range(steps):
        if flush is not None:
            flush.fill_(1.0)
        step()
    torch.cuda.synchronize()
    B.timing_enable(False)
    kernels = {}
    for name in B.kernel_names():
        tot, n = B.timing_query(name)
        if n:
            kernels[name] = {"avg_us": round(1e3 * tot / n, 2), "launches_per_step": n // steps}
            if kflops and name in kflops:
                kernels[name]["tflops"] = round(kflops[name] / (1e-3 * tot / n) / 1e12, 1)
    return ms, kernels


def copy_probe(mib: int) -> None:
    """A plain device copy of `mib` MiB: calibrates rocprofv3's byte counters."""
    if mib:
        import torch
        a = torch.empty(mib * (1 << 20) // 4, device="cuda:0", dtype=torch.float32).fill_(1.0)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()


def mall_flush_buffer():
    """A 1 GiB device buffer; overwriting it evicts the MALL (256 MB) and the L2s."""
    import torch
    return torch.empty(1 << 28, device="cuda:0", dtype=torch.float32)


def bench_linear(cfg, steps: int, warmup: int):
    """One LoRA linear (fwd+bwd) on its own, after the headline step: the
    attention output projection of the same model.  Not part of `value`."""
    import torch
    from lora_fine_tuning_mlp_amd import binding as B
    from lora_fine_tuning_mlp_amd import synthetic as S

    dev = torch.device("cuda:0")
    t = {k: v.to(dev) for k, v in S.linear_inputs(cfg, 0).items()}
    lin = B.Linear({k: v for k, v in t.items() if k != "dY"}, cfg.n_tokens, cfg.in_features, cfg.out_features,
                   cfg.rank, cfg.dtype, cfg.scale)
    dY = t["dY"]

    def step():
        lin.forward()
        lin.backward(dY)

    ms, kernels = time_leg(step, steps, warmup, linear_kernel_flops(cfg))
    leg = {"workload": cfg.name, "tokens": cfg.n_tokens, "in": cfg.in_features, "out": cfg.out_features,
           "rank": cfg.rank, "ms_per_step": round(ms, 4), "tflops": round(cfg.flops() / (ms * 1e-3) / 1e12, 2),
           "kernels": kernels}
    return with_rooflines(leg, cfg.flops(), linear_planned_bytes(cfg))


def mlp_planned_bytes(cfg) -> int:
    """HBM bytes one fused MLP fwd+bwd must move as planned: X twice, the
    three base weights twice, Y, dY and dX, and the [N, i] intermediates
    G, U (saved), H (forward workspace) and dG, dU (backward workspace), each
    written once and read once."""
    N, h, i = cfg.n_tokens, cfg.hidden, cfg.inter
    e = 2 if cfg.dtype == "bf16" else 4
    return e * (5 * N * h + 6 * h * i + 10 * N * i)


def qkv_planned_bytes(cfg) -> int:
    """HBM bytes of one fused QKV fwd+bwd as planned: X twice, dX, the base
    weights twice, Q/K/V written, dQ/dK/dV read, and the token-major
    gradient dP [N, O] (inverse RoPE applied) written and read back."""
    N, h = cfg.n_tokens, cfg.hidden
    O = sum(cfg.out_dims)
    e = 2 if cfg.dtype == "bf16" else 4
    return e * (3 * N * h + 2 * O * h + 4 * N * O)


def linear_planned_bytes(cfg) -> int:
    """HBM bytes of one LoRA linear fwd+bwd: Z twice, dZ, W twice, Y, dY."""
    N, k, o = cfg.n_tokens, cfg.in_features, cfg.out_features
    e = 2 if cfg.dtype == "bf16" else 4
    return e * (3 * N * k + 2 * k * o + 2 * N * o)


def with_rooflines(leg: dict, flops: int, planned_bytes: int) -> dict:
    """Add the MFMA fraction and the achieved HBM rate on planned bytes."""
    sec = leg["ms_per_step"] * 1e-3
    leg["frac_peak"] = round(flops / sec / 1e12 / PEAK_BF16_TFLOPS, 4)
    leg["planned_bytes"] = planned_bytes
    leg["hbm_gbs"] = round(planned_bytes / sec / 1e9, 1)
    leg["hbm_frac"] = round(planned_bytes / sec / 1e9 / PEAK_HBM_GBS, 4)
    return leg


def qkv_kernel_flops(cfg):
    N, h, r = cfg.n_tokens, cfg.hidden, cfg.rank
    O = sum(cfg.out_dims)
    return {"k_qkv_fwd": 2 * N * h * O + 6 * N * h * r + 2 * N * r * O,
            "k_proj_dx_bwd": 2 * N * O * h + 12 * N * r * h}


def mlp_kernel_flops(cfg):
    N, h, i, r = cfg.n_tokens, cfg.hidden, cfg.inter, cfg.rank
    return {"k_gateup_fwd": 4 * N * h * i + 4 * N * h * r + 4 * N * r * i,
            "k_linear_fwd": 2 * N * i * h + 2 * N * i * r + 2 * N * r * h,
            "k_down_bwd": 2 * N * h * i + 8 * N * r * i,
            "k_mlp_dt": 4 * N * i * r,
            "k_mlp_dx_bwd": 4 * N * i * h + 8 * N * r * h}


def bench_mlp(cfg, steps: int, warmup: int, flush=None):
    """LoRA MLP fwd+bwd at `cfg` on its own (GeGLU-tanh at h 3072, and the
    small-shape regime).  Not part of `value`.  `flush`: see time_leg."""
    import torch
    from lora_fine_tuning_mlp_amd import binding as B
    from lora_fine_tuning_mlp_amd import synthetic as S

    dev = torch.device("cuda:0")
    t = {k: v.to(dev) for k, v in S.mlp_inputs(cfg, 0).items()}
    m = B.MLP({k: v for k, v in t.items() if k != "dY"}, cfg.n_tokens, cfg.hidden, cfg.inter, cfg.rank, cfg.dtype,
              cfg.act, (cfg.scale,) * 3)
    dY = t["dY"]

    def step():
        m.forward()
        m.backward(dY)

    ms, kernels = time_leg(step, steps, warmup, mlp_kernel_flops(cfg), flush)
    leg = {"workload": cfg.name, "tokens": cfg.n_tokens, "hidden": cfg.hidden, "inter": cfg.inter,
           "rank": cfg.rank, "act": cfg.act, "ms_per_step": round(ms, 4),
           "tflops": round(cfg.flops() / (ms * 1e-3) / 1e12, 2), "kernels": kernels}
    return with_rooflines(leg, cfg.flops(), mlp_planned_bytes(cfg))


def bench_qkv(cfg, steps: int, warmup: int, flush=None):
    """LoRA QKV fwd+bwd at `cfg` (used for the q/k-norm variant of the
    headline QKV shape, and the small-shape regime).  Not part of `value`.
    `flush`: see time_leg."""
    import torch
    from lora_fine_tuning_mlp_amd import binding as B
    from lora_fine_tuning_mlp_amd import synthetic as S

    dev = torch.device("cuda:0")
    t = {k: v.to(dev) for k, v in S.qkv_inputs(cfg, 0).items()}
    m = B.QKV({k: v for k, v in t.items() if k not in ("dQ", "dK", "dV")}, cfg.batch, cfg.seq, cfg.hidden, cfg.n_q,
              cfg.n_kv, cfg.head_dim, cfg.rank, cfg.dtype, cfg.theta, (cfg.scale,) * 3, cfg.norm_eps)
    dQ, dK, dV = t["dQ"], t["dK"], t["dV"]

    def step():
        m.forward()
        m.backward(dQ, dK, dV)

    ms, kernels = time_leg(step, steps, warmup, qkv_kernel_flops(cfg), flush)
    leg = {"workload": cfg.name, "tokens": cfg.n_tokens, "qk_norm": cfg.qk_norm, "bias": cfg.bias,
           "ms_per_step": round(ms, 4), "tflops": round(cfg.flops() / (ms * 1e-3) / 1e12, 2), "kernels": kernels}
    return with_rooflines(leg, cfg.flops(), qkv_planned_bytes(cfg))


def _unfused_mlp(t, act: str, s: float):
    """The same LoRA MLP as separate torch ops (hipBLASLt GEMMs + elementwise
    kernels, autograd for the backward, W frozen): what a caller runs when
    the fused call is skipped."""
    import torch
    import torch.nn.functional as F

    phi = {"swiglu": F.silu, "geglu_tanh": lambda g: F.gelu(g, approximate="tanh"), "geglu_erf": F.gelu}[act]
    X = t["X"].detach().requires_grad_(True)
    ad = {k: t[k].detach().requires_grad_(True) for k in t if k[0] in "AB" and "_" in k}

    def lin(Z, n):
        return F.linear(Z, t["W_" + n]) + s * F.linear(F.linear(Z, ad["A_" + n]), ad["B_" + n])

    def step():
        Y = lin(phi(lin(X, "gate")) * lin(X, "up"), "down")
        Y.backward(t["dY"])
        return Y
    return step


def _unfused_qkv(t, cfg):
    """LoRA QKV + head split + RoPE as separate torch ops with autograd."""
    import math
    import torch
    import torch.nn.functional as F

    B, S, d = cfg.batch, cfg.seq, cfg.head_dim
    dev = t["X"].device
    j = torch.arange(d // 2, device=dev, dtype=torch.float64)
    ang = torch.arange(S, device=dev, dtype=torch.float64)[:, None] * torch.exp(-(2.0 * j / d) * math.log(cfg.theta))
    cos, sin = ang.cos().to(t["X"].dtype), ang.sin().to(t["X"].dtype)
    X = t["X"].detach().requires_grad_(True)
    ad = {k: t[k].detach().requires_grad_(True) for k in t if k[:2] in ("A_", "B_")}

    def proj(n, heads):
        P = F.linear(X, t["W_" + n]) + cfg.scale * F.linear(F.linear(X, ad["A_" + n]), ad["B_" + n])
        return P.view(B, S, heads, d).transpose(1, 2)

    def rope(Z):
        x1, x2 = Z[..., : d // 2], Z[..., d // 2:]
        return torch.cat([x1 * cos - x2 * sin, x2 * cos + x1 * sin], dim=-1)

    def step():
        Q, K, V = rope(proj("q", cfg.n_q)), rope(proj("k", cfg.n_kv)), proj("v", cfg.n_kv)
        torch.autograd.backward([Q, K, V], [t["dQ"], t["dK"], t["dV"]])
    return step


def crossover(steps: int, warmup: int):
    """Fused calls against the unfused torch sequence over a ladder of token
    counts at two model widths: where does fusion start to pay?"""
    import torch
    from lora_fine_tuning_mlp_amd import binding as B
    from lora_fine_tuning_mlp_amd import synthetic as S

    dev = torch.device("cuda:0")

    def event_ms(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    rows = []
    for base, tokens in ((S.C4_MLP, (16, 64, 256, 1024, 4096)), (S.C2, (64, 256, 1024, 4096, 8192))):
        for n in tokens:
            cfg = dataclasses.replace(base, name=f"{base.name}_n{n}", n_tokens=n)
            t = {k: v.to(dev) for k, v in S.mlp_inputs(cfg, 0).items()}
            m = B.MLP({k: v for k, v in t.items() if k != "dY"}, n, cfg.hidden, cfg.inter, cfg.rank, cfg.dtype,
                      cfg.act, (cfg.scale,) * 3)
            fused = event_ms(lambda: (m.forward(), m.backward(t["dY"])))
            unfused = event_ms(_unfused_mlp(t, cfg.act, cfg.scale))
            rows.append({"op": "mlp", "hidden": cfg.hidden, "inter": cfg.inter, "tokens": n,
                         "fused_ms": round(fused, 4), "unfused_ms": round(unfused, 4),
                         "speedup": round(unfused / fused, 3)})
            print(f"[crossover] {rows[-1]}", file=sys.stderr, flush=True)
            del m, t
    for base, seqs in ((S.C4_QKV, (4, 16, 64, 256, 1024)), (S.C1, (16, 64, 256, 1024, 2048))):
        for sq in seqs:
            cfg = dataclasses.replace(base, name=f"{base.name}_s{sq}", seq=sq)
            t = {k: v.to(dev) for k, v in S.qkv_inputs(cfg, 0).items()}
            m = B.QKV({k: v for k, v in t.items() if k not in ("dQ", "dK", "dV")}, cfg.batch, sq, cfg.hidden,
                      cfg.n_q, cfg.n_kv, cfg.head_dim, cfg.rank, cfg.dtype, cfg.theta, (cfg.scale,) * 3)
            fused = event_ms(lambda: (m.forward(), m.backward(t["dQ"], t["dK"], t["dV"])))
            unfused = event_ms(_unfused_qkv(t, cfg))
            rows.append({"op": "qkv", "hidden": cfg.hidden, "heads": f"{cfg.n_q}/{cfg.n_kv}x{cfg.head_dim}",
                         "tokens": cfg.n_tokens, "fused_ms": round(fused, 4), "unfused_ms": round(unfused, 4),
                         "speedup": round(unfused / fused, 3)})
            print(f"[crossover] {rows[-1]}", file=sys.stderr, flush=True)
            del m, t
    return rows


def step_distribution(qkv, mlp, dqkv, dY, steps: int, stream):
    """Per-step timings from events recorded between the four calls of each
    step (QKV fwd, QKV bwd, MLP fwd, MLP bwd): median, min and p90 of the
    whole step, and the median of each call."""
    import numpy as np
    import torch

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    torch.cuda.synchronize()
    for e in ev:
        e[0].record(stream)
        qkv.forward()
        e[1].record(stream)
        qkv.backward(*dqkv)
        e[2].record(stream)
        mlp.forward()
        e[3].record(stream)
        mlp.backward(dY)
        e[4].record(stream)
    torch.cuda.synchronize()
    t = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(4)] for e in ev])   # [steps][4] ms
    whole = t.sum(axis=1)
    r4 = lambda x: round(float(x), 4)
    return {"median": r4(np.median(whole)), "min": r4(whole.min()), "p90": r4(np.percentile(whole, 90)),
            "qkv_fwd_median": r4(np.median(t[:, 0])), "qkv_bwd_median": r4(np.median(t[:, 1])),
            "mlp_fwd_median": r4(np.median(t[:, 2])), "mlp_bwd_median": r4(np.median(t[:, 3])),
            "fwd_median": r4(np.median(t[:, 0] + t[:, 2])), "bwd_median": r4(np.median(t[:, 1] + t[:, 3])),
            "steps": steps}


def stored_traffic(kernel: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current sources (else None)."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
    except ValueError:
        return None
    from lora_fine_tuning_mlp_amd.profiling import source_hash
    ent = d.get(kernel)
    if not ent or ent.get("source_hash") != source_hash():
        return None
    return ent.get("bytes_per_launch")


def cpu_baseline(qkv_cfg, mlp_cfg, tokens: int, reps: int = 1):
    """Time the CPU oracle (as it stands) on `tokens` tokens of each workload,
    `reps` times over.  The QKV sample keeps the workload's sequence length
    (batches of seq) when `tokens` is a multiple of it, else it is one
    sequence of `tokens`."""
    import dataclasses
    import numpy as np
    from threadpoolctl import threadpool_info
    from lora_fine_tuning_mlp_amd import synthetic as S
    from oracle import lora_oracle as orc

    mlp_s = dataclasses.replace(mlp_cfg, n_tokens=tokens)
    if tokens % qkv_cfg.seq == 0:
        qkv_s = dataclasses.replace(qkv_cfg, batch=tokens // qkv_cfg.seq)
    else:
        qkv_s = dataclasses.replace(qkv_cfg, batch=1, seq=tokens)
    tm = S.mlp_inputs(mlp_s, 0)
    tq = S.qkv_inputs(qkv_s, 0)
    pm = S.to_f64({k: v for k, v in tm.items() if k != "dY"})
    dY = tm["dY"].double().numpy()
    pq = S.to_f64({k: v for k, v in tq.items() if k not in ("dQ", "dK", "dV")})
    dQ, dK, dV = (tq[k].double().numpy() for k in ("dQ", "dK", "dV"))
    shape = dict(batch=qkv_s.batch, seq=qkv_s.seq, n_q=qkv_s.n_q, n_kv=qkv_s.n_kv, head_dim=qkv_s.head_dim, theta=qkv_s.theta)
    sc = (qkv_s.scale,) * 3
    t0 = time.perf_counter()
    for _ in range(reps):
        orc.qkv_fwd(pq, scales=sc, **shape)
        orc.qkv_bwd(pq, dQ, dK, dV, scales=sc, **shape)
        orc.mlp_fwd(pm, mlp_s.act, mlp_s.scale, mlp_s.scale, mlp_s.scale)
        orc.mlp_bwd(pm, dY, mlp_s.act, mlp_s.scale, mlp_s.scale, mlp_s.scale)
    dt = time.perf_counter() - t0
    flops = reps * (qkv_s.flops() + mlp_s.flops())
    threads = max([d.get("num_threads", 1) for d in threadpool_info() if d.get("user_api") == "blas"] or [1])
    # The tiny fp32 MLP (2 x 16 tokens, h 64) on one thread, as a fixed reference point.
    from threadpoolctl import threadpool_limits
    t0c = S.mlp_inputs(S.C0, 0)
    pc = S.to_f64({k: v for k, v in t0c.items() if k != "dY"})
    dYc = t0c["dY"].double().numpy()
    with threadpool_limits(limits=1):
        c0t = time.perf_counter()
        for _ in range(20):
            orc.mlp_fwd(pc, S.C0.act, S.C0.scale, S.C0.scale, S.C0.scale)
            orc.mlp_bwd(pc, dYc, S.C0.act, S.C0.scale, S.C0.scale, S.C0.scale)
        c0_s = (time.perf_counter() - c0t) / 20
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{tokens} tokens of each workload (QKV as {qkv_s.batch} x {qkv_s.seq}; MLP {tokens} rows): "
                  f"fwd+bwd of both in float64 numpy, {reps} time(s), {dt:.2f} s wall",
        "seconds": dt,
        "cpu_model": model,
        "tiny_mlp_1thread_ms": round(1e3 * c0_s, 3),
    }


LEG_NAMES = ("oproj", "qkv_qknorm", "mlp_geglu_h3072", "small_mlp_h896", "small_qkv_h896",
             "small_mlp_h896_cold", "small_qkv_h896_cold")


def run_legs(names, steps: int, warmup: int):
    """The separate legs (outside `value`).  The large ones run steps / 2
    calls; the small-shape ones run `steps` calls twice: as a loop of calls
    whose inputs stay in the MALL between calls, and ("_cold") with the MALL
    and L2s flushed before every call."""
    from lora_fine_tuning_mlp_amd import synthetic as S

    ls, lw = max(1, steps // 2), max(1, warmup)
    flush = mall_flush_buffer() if any(n.endswith("_cold") for n in names) else None
    make = {
        "oproj": lambda: bench_linear(S.C_OPROJ, ls, lw),
        "qkv_qknorm": lambda: bench_qkv(dataclasses.replace(S.C1, name=S.C1.name + "_qknorm", qk_norm=True), ls, lw),
        "mlp_geglu_h3072": lambda: bench_mlp(S.C3, ls, lw),
        "small_mlp_h896": lambda: bench_mlp(S.C4_MLP, steps, lw),
        "small_qkv_h896": lambda: bench_qkv(S.C4_QKV, steps, lw),
        "small_mlp_h896_cold": lambda: bench_mlp(S.C4_MLP, steps, lw, flush),
        "small_qkv_h896_cold": lambda: bench_qkv(S.C4_QKV, steps, lw, flush),
    }
    out = {}
    for n in names:
        print(f"[bench] leg {n}", file=sys.stderr, flush=True)
        out[n] = make[n]()
        if n.endswith("_cold"):
            out[n]["mall"] = "flushed before every call (1 GiB overwrite), each call timed on its own"
        elif n.startswith("small_"):
            out[n]["mall"] = "not flushed: a loop of calls on the same inputs (working set < 256 MB MALL)"
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-tokens", type=int, default=8192, help="token sample for the CPU oracle baseline")
    ap.add_argument("--cpu-reps", type=int, default=2, help="repetitions of the CPU oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-legs", action="store_true",
                    help="skip the separate o_proj linear and q/k-norm QKV legs (outside the headline value)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run a plain device copy of this size (calibrates rocprofv3 byte counters)")
    ap.add_argument("--crossover", action="store_true",
                    help="instead of the headline step: fused vs unfused (torch) timings over token counts")
    ap.add_argument("--leg", choices=LEG_NAMES, action="append",
                    help="instead of the headline step: run only this separate leg (repeatable) and print its JSON")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); this build has no "
              f"multi-GPU path: the projections are data-parallel over tokens and would shard as described in the "
              f"design notes.", file=sys.stderr)
        sys.exit(2)

    import torch
    from lora_fine_tuning_mlp_amd import binding as B
    from lora_fine_tuning_mlp_amd import synthetic as S

    qkv_cfg, mlp_cfg = S.C1, S.C2
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.leg:
        legs = run_legs(args.leg, args.steps, args.warmup)
        copy_probe(args.copy_probe_mib)
        print(json.dumps({"legs": legs, "dtype": "bf16", "data": "synthetic"}), flush=True)
        return
    if args.crossover:
        rows = crossover(max(3, args.steps), max(2, args.warmup))
        print(json.dumps({"crossover": rows, "unit": "ms per fwd+bwd", "dtype": "bf16", "data": "synthetic"}),
              flush=True)
        return
    print(f"[bench] generating inputs ({qkv_cfg.name}, {mlp_cfg.name})", file=sys.stderr, flush=True)
    tq = {k: v.to(dev) for k, v in S.qkv_inputs(qkv_cfg, 0).items()}
    tm = {k: v.to(dev) for k, v in S.mlp_inputs(mlp_cfg, 0).items()}
    qkv = B.QKV({k: v for k, v in tq.items() if k not in ("dQ", "dK", "dV")}, qkv_cfg.batch, qkv_cfg.seq,
                qkv_cfg.hidden, qkv_cfg.n_q, qkv_cfg.n_kv, qkv_cfg.head_dim, qkv_cfg.rank, qkv_cfg.dtype,
                qkv_cfg.theta, (qkv_cfg.scale,) * 3)
    mlp = B.MLP({k: v for k, v in tm.items() if k != "dY"}, mlp_cfg.n_tokens, mlp_cfg.hidden, mlp_cfg.inter,
                mlp_cfg.rank, mlp_cfg.dtype, mlp_cfg.act, (mlp_cfg.scale,) * 3)
    dQ, dK, dV, dY = tq["dQ"], tq["dK"], tq["dV"], tm["dY"]

    def step():
        qkv.forward()
        qkv.backward(dQ, dK, dV)
        mlp.forward()
        mlp.backward(dY)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: HIP events on the library's stream around the K steps,
    # with the library's per-launch recorder off.
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    total_ms = e0.elapsed_time(e1)
    ms_per_step = total_ms / args.steps
    flops_step = qkv_cfg.flops() + mlp_cfg.flops()
    value = flops_step / (ms_per_step * 1e-3) / 1e12

    # Per-kernel pass: the same K steps again, with HIP events recorded around
    # every launch on the stream it runs on (the roofline's kernel timing).
    B.timing_reset()
    B.timing_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    B.timing_enable(False)
    per_kernel = {}
    for name in B.kernel_names():
        ms, n = B.timing_query(name)
        if n:
            per_kernel[name] = {"total_ms": ms, "launches": n, "avg_us": 1e3 * ms / n}
    kf = kernel_flops(qkv_cfg, mlp_cfg)
    dominant = max((k for k in per_kernel if k in kf), key=lambda k: per_kernel[k]["total_ms"])
    avg_s = per_kernel[dominant]["avg_us"] * 1e-6
    achieved = kf[dominant] / avg_s / 1e12
    for k in per_kernel:
        if k in kf:
            pk = per_kernel[k]
            pk["tflops"] = kf[k] / (pk["avg_us"] * 1e-6) / 1e12
            pk["frac_peak"] = pk["tflops"] / PEAK_BF16_TFLOPS
    traffic = stored_traffic(dominant)
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic, "kernel": dominant,
                "flops_per_launch": kf[dominant], "avg_launch_us": round(per_kernel[dominant]["avg_us"], 2),
                "timing": "per-launch HIP events on the launch stream, second pass of the same steps"}

    # Distribution pass (after the timed region, same work): events between
    # the four calls of every step give per-step median / min / p90 and the
    # forward and backward medians of each op.
    dist = step_distribution(qkv, mlp, (dQ, dK, dV), dY, args.steps, stream)

    legs = None
    if not args.no_legs:
        print("[bench] separate legs: o_proj, q/k-norm QKV, GeGLU MLP at h 3072, small shapes", file=sys.stderr,
              flush=True)
        legs = run_legs(LEG_NAMES, args.steps, args.warmup)

    copy_probe(args.copy_probe_mib)

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded normals: X, dY ~N(0,1); W std 0.02; A var 1/in; B std 0.02)",
        "config": {"workload": "lora_qkv_rope_c1 + lora_mlp_swiglu_c2 fwd+bwd", "tokens": mlp_cfg.n_tokens,
                   "hidden": mlp_cfg.hidden, "inter": mlp_cfg.inter, "mlp_rank": mlp_cfg.rank,
                   "qkv_heads": f"{qkv_cfg.n_q}/{qkv_cfg.n_kv}x{qkv_cfg.head_dim}", "qkv_rank": qkv_cfg.rank,
                   "rope_theta": qkv_cfg.theta, "flops_per_step": flops_step},
        "frac_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "step_ms": dist,
        "roofline": roofline,
        "kernels": {k: {kk: (round(vv, 3) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in per_kernel.items()},
        "legs": legs,
    }
    if not args.no_cpu_baseline:
        print(f"[bench] cpu oracle on {args.cpu_tokens} tokens", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(qkv_cfg, mlp_cfg, args.cpu_tokens, args.cpu_reps)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
