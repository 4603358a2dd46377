"""GPU parity of the HIP path (through the C ABI) against the CPU oracle on
seeded inputs: element by element on multi-tile shapes with ragged tails,
plus the exact special cases and run-to-run determinism."""
import dataclasses

import numpy as np
import pytest
import torch

from lora_fine_tuning_mlp_amd import synthetic as S
from lora_fine_tuning_mlp_amd import binding as B_
from oracle import lora_oracle as orc
from tests import gpu_cases as gc

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from lora_fine_tuning_mlp_amd import binding
    binding.lib()   # fails loudly when the HIP library is missing


@pytest.mark.parametrize("cfg", gc.MLP_CASES, ids=lambda c: c.name)
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_mlp_parity(cfg, seed):
    gc.say(f"mlp parity {cfg.name} seed={seed}")
    t = S.mlp_inputs(cfg, seed)
    gc.compare(f"{cfg.name}/s{seed}", gc.run_mlp_gpu(cfg, t), gc.run_mlp_oracle(cfg, t), gc.TOL[cfg.dtype])


@pytest.mark.parametrize("cfg", gc.QKV_CASES, ids=lambda c: c.name)
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_qkv_parity(cfg, seed):
    gc.say(f"qkv parity {cfg.name} seed={seed}")
    t = S.qkv_inputs(cfg, seed)
    gc.compare(f"{cfg.name}/s{seed}", gc.run_qkv_gpu(cfg, t), gc.run_qkv_oracle(cfg, t), gc.TOL[cfg.dtype])


def test_c0_all_seeds():
    for seed in (0, 1, 2):
        t = S.mlp_inputs(S.C0, seed)
        gc.compare(f"C0/s{seed}", gc.run_mlp_gpu(S.C0, t), gc.run_mlp_oracle(S.C0, t), gc.TOL["f32"])


@pytest.mark.parametrize("cfg", [gc.MLP_CASES[1], gc.MLP_CASES[3]], ids=lambda c: c.name)
def test_mlp_special_cases(cfg):
    """B = 0 => dA exactly 0;  A = 0 => dB exactly 0;  W = 0 => adapter-only path."""
    t = S.mlp_inputs(cfg, 5)
    tb = dict(t)
    for n in ("gate", "up", "down"):
        tb["B_" + n] = torch.zeros_like(t["B_" + n])
    out = gc.run_mlp_gpu(cfg, tb)
    for n in ("gate", "up", "down"):
        assert not np.any(out["dA_" + n]), n
    gc.compare(f"{cfg.name}/B0", out, gc.run_mlp_oracle(cfg, tb), gc.TOL[cfg.dtype])
    ta = dict(t)
    for n in ("gate", "up", "down"):
        ta["A_" + n] = torch.zeros_like(t["A_" + n])
    out = gc.run_mlp_gpu(cfg, ta)
    for n in ("gate", "up", "down"):
        assert not np.any(out["dB_" + n]), n
    tw = dict(t)
    for n in ("gate", "up", "down"):
        tw["W_" + n] = torch.zeros_like(t["W_" + n])
    gc.compare(f"{cfg.name}/W0", gc.run_mlp_gpu(cfg, tw), gc.run_mlp_oracle(cfg, tw), gc.TOL[cfg.dtype])


@pytest.mark.parametrize("cfg", [gc.QKV_CASES[0], gc.QKV_CASES[2]], ids=lambda c: c.name)
def test_qkv_special_cases(cfg):
    t = S.qkv_inputs(cfg, 6)
    tb = dict(t)
    for n in "qkv":
        tb["B_" + n] = torch.zeros_like(t["B_" + n])
    out = gc.run_qkv_gpu(cfg, tb)
    for n in "qkv":
        assert not np.any(out["dA_" + n]), n
    gc.compare(f"{cfg.name}/B0", out, gc.run_qkv_oracle(cfg, tb), gc.TOL[cfg.dtype])
    ta = dict(t)
    for n in "qkv":
        ta["A_" + n] = torch.zeros_like(t["A_" + n])
    out = gc.run_qkv_gpu(cfg, ta)
    for n in "qkv":
        assert not np.any(out["dB_" + n]), n
    tw = dict(t)
    for n in "qkv":
        tw["W_" + n] = torch.zeros_like(t["W_" + n])
    gc.compare(f"{cfg.name}/W0", gc.run_qkv_gpu(cfg, tw), gc.run_qkv_oracle(cfg, tw), gc.TOL[cfg.dtype])


@pytest.mark.parametrize("cfg", gc.LINEAR_CASES, ids=lambda c: c.name)
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_linear_parity(cfg, seed):
    gc.say(f"linear parity {cfg.name} seed={seed}")
    t = S.linear_inputs(cfg, seed)
    gc.compare(f"{cfg.name}/s{seed}", gc.run_linear_gpu(cfg, t), gc.run_linear_oracle(cfg, t), gc.TOL[cfg.dtype])


@pytest.mark.parametrize("cfg", [gc.LINEAR_CASES[0], gc.LINEAR_CASES[3]], ids=lambda c: c.name)
def test_linear_special_cases(cfg):
    """B = 0 => dA exactly 0 and Y = X W^T;  A = 0 => dB and T exactly 0;  W = 0 => adapter only."""
    t = S.linear_inputs(cfg, 5)
    tb = dict(t, B=torch.zeros_like(t["B"]))
    out = gc.run_linear_gpu(cfg, tb)
    assert not np.any(out["dA"])
    gc.compare(f"{cfg.name}/B0", out, gc.run_linear_oracle(cfg, tb), gc.TOL[cfg.dtype])
    ta = dict(t, A=torch.zeros_like(t["A"]))
    out = gc.run_linear_gpu(cfg, ta)
    assert not np.any(out["dB"]) and not np.any(out["T"])
    tw = dict(t, W=torch.zeros_like(t["W"]))
    gc.compare(f"{cfg.name}/W0", gc.run_linear_gpu(cfg, tw), gc.run_linear_oracle(cfg, tw), gc.TOL[cfg.dtype])


def test_linear_matches_mlp_down_projection():
    """The MLP's down projection and a lone LoRA linear on the same H compute the
    same Y: run the MLP, feed its hidden activations to the linear entry point."""
    cfg = gc.MLP_CASES[1]
    t = S.mlp_inputs(cfg, 4)
    dev = torch.device("cuda:0")
    td = {k: v.to(dev).contiguous() for k, v in t.items() if k != "dY"}
    m = B_.MLP(td, cfg.n_tokens, cfg.hidden, cfg.inter, cfg.rank, cfg.dtype, cfg.act, gc.mlp_scales(cfg))
    m.forward()
    p = S.to_f64({k: v for k, v in t.items() if k != "dY"})
    f = orc.mlp_fwd(p, cfg.act, *gc.mlp_scales(cfg))
    H = torch.from_numpy(f["H"]).to(S.TORCH_DTYPES[cfg.dtype]).to(dev).contiguous()
    lin = B_.Linear({"X": H, "W": td["W_down"], "A": td["A_down"], "B": td["B_down"]}, cfg.n_tokens, cfg.inter,
                    cfg.hidden, cfg.rank, cfg.dtype, cfg.scale)
    lin.forward()
    torch.cuda.synchronize()
    assert gc.rel_err(gc.to64(lin.Y), f["Y"]) <= gc.TOL[cfg.dtype]
    assert gc.rel_err(gc.to64(m.Y), f["Y"]) <= gc.TOL[cfg.dtype]


def test_zero_scale_is_the_base_projection():
    """s = 0: Y is the plain base projection and every adapter gradient
    (dT = s dY B, dB = s dY^T T, dA = dT^T Z) is exactly zero."""
    cfg = gc.MLP_CASES[1]
    t = S.mlp_inputs(cfg, 8)
    out = gc.run_mlp_gpu(cfg, t, scales=(0.0, 0.0, 0.0))
    for n in ("gate", "up", "down"):
        assert not np.any(out["dA_" + n]) and not np.any(out["dB_" + n]), n
    gc.compare(f"{cfg.name}/s0", out, gc.run_mlp_oracle(cfg, t, scales=(0.0, 0.0, 0.0)), gc.TOL[cfg.dtype])
    qc = gc.QKV_CASES[0]
    tq = S.qkv_inputs(qc, 8)
    out = gc.run_qkv_gpu(qc, tq, scales=(0.0, 0.0, 0.0))
    for n in "qkv":
        assert not np.any(out["dA_" + n]) and not np.any(out["dB_" + n]), n
    gc.compare(f"{qc.name}/s0", out, gc.run_qkv_oracle(qc, tq, scales=(0.0, 0.0, 0.0)), gc.TOL[qc.dtype])
    lc = dataclasses.replace(gc.LINEAR_CASES[0], scale=0.0)
    tl = S.linear_inputs(lc, 8)
    out = gc.run_linear_gpu(lc, tl)
    assert not np.any(out["dA"]) and not np.any(out["dB"])
    gc.compare(f"{lc.name}/s0", out, gc.run_linear_oracle(lc, tl), gc.TOL[lc.dtype])


def test_empty_batch_gradients_are_zero():
    """No tokens: forward writes nothing, the adapter gradients are empty sums
    (exactly zero), even where the outputs held NaN before the call."""
    dev = torch.device("cuda:0")
    cfg = S.MLPConfig("mlp_empty", 0, 128, 192, 8, 2.0, "swiglu", "bf16")
    t = {k: v.to(dev) for k, v in S.mlp_inputs(cfg, 0).items()}
    m = B_.MLP({k: v for k, v in t.items() if k != "dY"}, 0, 128, 192, 8, "bf16", "swiglu")
    for g in m.grads.values():
        g.fill_(float("nan"))
    m.forward()
    m.backward(t["dY"])
    torch.cuda.synchronize()
    for k, g in m.grads.items():
        assert torch.count_nonzero(g).item() == 0, k
    qc = S.QKVConfig("qkv_empty", 0, 16, 128, 4, 2, 64, 8, 2.0, 1.0e4, "bf16")
    tq = {k: v.to(dev) for k, v in S.qkv_inputs(qc, 0).items()}
    mq = B_.QKV({k: v for k, v in tq.items() if k not in ("dQ", "dK", "dV")}, 0, 16, 128, 4, 2, 64, 8, "bf16", 1.0e4)
    for g in mq.grads.values():
        g.fill_(float("nan"))
    mq.forward()
    mq.backward(tq["dQ"], tq["dK"], tq["dV"])
    torch.cuda.synchronize()
    for k, g in mq.grads.items():
        assert torch.count_nonzero(g).item() == 0, k
    lc = S.LinearConfig("linear_empty", 0, 64, 96, 4, 2.0, "f32")
    tl = {k: v.to(dev) for k, v in S.linear_inputs(lc, 0).items()}
    ml = B_.Linear({k: v for k, v in tl.items() if k != "dY"}, 0, 64, 96, 4, "f32")
    for g in ml.grads.values():
        g.fill_(float("nan"))
    ml.forward()
    ml.backward(tl["dY"])
    torch.cuda.synchronize()
    for k, g in ml.grads.items():
        assert torch.count_nonzero(g).item() == 0, k


def test_rope_position_zero_identity_on_device():
    """At position 0 RoPE is the identity: Q[:, :, 0] equals the unrotated projection."""
    cfg = gc.QKV_CASES[2]
    t = S.qkv_inputs(cfg, 7)
    out = gc.run_qkv_gpu(cfg, t)
    ref = gc.run_qkv_oracle(cfg, t)
    assert gc.rel_err(out["Q"][:, :, 0], ref["Q"][:, :, 0]) <= gc.TOL["f32"]


def test_determinism():
    mlp = {c.name: c for c in gc.MLP_CASES}
    lin = {c.name: c for c in gc.LINEAR_CASES}
    for cfg in (gc.MLP_CASES[1], gc.QKV_CASES[0], gc.LINEAR_CASES[0], mlp["mlp_bf16_splitk_cross"],
                mlp["mlp_bf16_dx_runs_ragged"], lin["linear_bf16_splitk_uneven"], lin["linear_bf16_runs_ragged"],
                [c for c in gc.QKV_CASES if c.name == "qkv_bf16_d128_runs_ragged"][0]):
        if isinstance(cfg, S.MLPConfig):
            t = S.mlp_inputs(cfg, 3)
            a, b = gc.run_mlp_gpu(cfg, t), gc.run_mlp_gpu(cfg, t)
        elif isinstance(cfg, S.LinearConfig):
            t = S.linear_inputs(cfg, 3)
            a, b = gc.run_linear_gpu(cfg, t), gc.run_linear_gpu(cfg, t)
        else:
            t = S.qkv_inputs(cfg, 3)
            a, b = gc.run_qkv_gpu(cfg, t), gc.run_qkv_gpu(cfg, t)
        for k in a:
            assert np.array_equal(a[k], b[k]), (cfg.name, k)
