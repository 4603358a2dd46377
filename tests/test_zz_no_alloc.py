"""The allocation-free QKV forward (lora_qkv_fwd_noalloc, scratch in a static
device array) gives exactly what lora_qkv_fwd gives with a caller workspace,
on two calls in a row, the second one smaller (the array keeps the first
call's table, which the second must not read)."""
import numpy as np
import pytest
import torch

from lora_fine_tuning_mlp_amd import binding as B
from lora_fine_tuning_mlp_amd import synthetic as S
from tests import gpu_cases as gc

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    B.lib()


def _noalloc_outputs(m: B.QKV, cfg: S.QKVConfig):
    e = dict(device=m.Q.device, dtype=m.Q.dtype)
    Q, K, V = torch.empty_like(m.Q), torch.empty_like(m.K), torch.empty_like(m.V)
    T = torch.empty_like(m.T)
    for x in (Q, K, V, T):
        x.fill_(float("nan"))
    B.lora_qkv_fwd_noalloc(m.desc, m.t["X"], m.q, m.k, m.v, Q, K, V, T)
    return Q, K, V, T


CALLS = [S.QKVConfig("qkv_bf16_noalloc_big", 2, 600, 256, 4, 2, 128, 16, 2.0, 1.0e4, "bf16", bias=True),
         S.QKVConfig("qkv_bf16_noalloc_small", 1, 77, 128, 4, 1, 64, 8, 2.0, 1.0e6, "bf16")]


def test_noalloc_matches_workspace_entry_point_twice():
    dev = torch.device("cuda:0")
    for i, cfg in enumerate(CALLS):
        gc.say(f"noalloc call {i}: {cfg.name}")
        t = {k: v.to(dev).contiguous() for k, v in S.qkv_inputs(cfg, 3 + i).items() if k not in ("dQ", "dK", "dV")}
        m = B.QKV(t, cfg.batch, cfg.seq, cfg.hidden, cfg.n_q, cfg.n_kv, cfg.head_dim, cfg.rank, cfg.dtype,
                  cfg.theta, (cfg.scale,) * 3)
        m.forward()
        got = _noalloc_outputs(m, cfg)
        torch.cuda.synchronize()
        for name, a, b in zip(("Q", "K", "V", "T"), got, (m.Q, m.K, m.V, m.T)):
            assert torch.equal(a, b), f"call {i}: {name} differs from lora_qkv_fwd"
        # and both match the oracle (the tolerance of the call dtype)
        ref = gc.run_qkv_oracle(cfg, S.qkv_inputs(cfg, 3 + i))
        for name, a in zip(("Q", "K", "V"), got[:3]):
            assert gc.rel_err(gc.to64(a), ref[name]) <= gc.TOL[cfg.dtype], name


def test_noalloc_rejects_shapes_beyond_its_scratch():
    cap = B.lora_qkv_fwd_noalloc_max_scratch_bytes()
    seq = cap // (64 * 4) + 8                  # cos + sin tables of seq x 64 floats exceed the array
    cfg = S.QKVConfig("qkv_noalloc_too_long", 1, seq, 128, 2, 1, 128, 4, 2.0, 1.0e4, "bf16")
    assert B.lora_qkv_workspace_bytes(B.qkv_desc(1, seq, 128, 2, 1, 128, 4, "bf16", 1e4), 0) > cap
    dev = torch.device("cuda:0")
    t = {k: v.to(dev).contiguous() for k, v in S.qkv_inputs(cfg, 0).items() if k not in ("dQ", "dK", "dV")}
    m = B.QKV(t, cfg.batch, cfg.seq, cfg.hidden, cfg.n_q, cfg.n_kv, cfg.head_dim, cfg.rank, cfg.dtype, cfg.theta)
    with pytest.raises(B.LoraError) as ei:
        B.lora_qkv_fwd_noalloc(m.desc, m.t["X"], m.q, m.k, m.v, m.Q, m.K, m.V, m.T)
    assert ei.value.status == 4 and "static buffer" in str(ei.value)
