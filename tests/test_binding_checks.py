"""The Python binding rejects, before any library call, buffers the kernels
would read or write out of bounds: host tensors, a dtype other than the
descriptor's, too few elements, projections it cannot size-check.  Host only."""
import pytest
import torch

from lora_fine_tuning_mlp_amd import binding as B


class _NoLib:
    def __getattr__(self, name):
        raise AssertionError(f"library function {name} reached although validation should have failed")


@pytest.fixture(autouse=True)
def _no_library_calls(monkeypatch):
    monkeypatch.setattr(B, "lib", lambda: _NoLib())


N, H, I, R = 32, 64, 96, 4


def _mlp_tensors(dtype=torch.bfloat16):
    e = dict(dtype=dtype)
    t = {"X": torch.zeros(N, H, **e), "Y": torch.zeros(N, H, **e), "G": torch.zeros(N, I, **e),
         "U": torch.zeros(N, I, **e), "T": torch.zeros(3, N, R), "ws": torch.zeros(1024, dtype=torch.uint8)}
    projs = {n: B.proj(torch.zeros(o, i, **e), torch.zeros(R, i, **e), torch.zeros(o, R, **e), 2.0)
             for n, o, i in (("gate", I, H), ("up", I, H), ("down", H, I))}
    return t, projs


def _fwd(t, projs, dtype="bf16"):
    desc = B.mlp_desc(N, H, I, R, dtype, "swiglu")
    B.lora_mlp_fwd(desc, t["X"], projs["gate"], projs["up"], projs["down"], t["Y"], t["G"], t["U"], t["T"], t["ws"])


def test_host_tensors_are_rejected():
    t, projs = _mlp_tensors()
    with pytest.raises(ValueError, match="GPU tensor"):
        _fwd(t, projs)


def test_dtype_must_match_the_descriptor(monkeypatch):
    monkeypatch.setattr(B, "_REQUIRE_GPU", False)
    t, projs = _mlp_tensors(torch.bfloat16)
    with pytest.raises(ValueError, match="dtype"):
        _fwd(t, projs, dtype="f32")
    t["T"] = torch.zeros(3, N, R, dtype=torch.bfloat16)          # T is float32 whatever the call dtype
    with pytest.raises(ValueError, match="T: dtype"):
        _fwd(t, projs)


def test_undersized_buffers_are_rejected(monkeypatch):
    monkeypatch.setattr(B, "_REQUIRE_GPU", False)
    t, projs = _mlp_tensors()
    t["U"] = torch.zeros(N - 1, I, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="U: .* at least"):
        _fwd(t, projs)
    t, projs = _mlp_tensors()
    projs["down"] = B.proj(torch.zeros(H, I - 1, dtype=torch.bfloat16), torch.zeros(R, I, dtype=torch.bfloat16),
                           torch.zeros(H, R, dtype=torch.bfloat16), 2.0)
    with pytest.raises(ValueError, match="down.W"):
        _fwd(t, projs)


def test_mlp_projection_bias_is_refused(monkeypatch):
    monkeypatch.setattr(B, "_REQUIRE_GPU", False)
    t, projs = _mlp_tensors()
    e = dict(dtype=torch.bfloat16)
    projs["up"] = B.proj(torch.zeros(I, H, **e), torch.zeros(R, H, **e), torch.zeros(I, R, **e), 2.0,
                         torch.zeros(I, **e))
    with pytest.raises(ValueError, match="no bias"):
        _fwd(t, projs)


def test_raw_proj_structs_cannot_be_checked(monkeypatch):
    monkeypatch.setattr(B, "_REQUIRE_GPU", False)
    t, projs = _mlp_tensors()
    projs["gate"] = B.Proj(0x1000, 0x1000, 0x1000, 2.0)
    with pytest.raises(ValueError, match="proj\\(\\)"):
        _fwd(t, projs)


def test_linear_and_qkv_checks(monkeypatch):
    monkeypatch.setattr(B, "_REQUIRE_GPU", False)
    e = dict(dtype=torch.float32)
    d = B.linear_desc(N, H, I, R, "f32")
    p = B.proj(torch.zeros(I, H, **e), torch.zeros(R, H, **e), torch.zeros(I, R, **e), 2.0)
    with pytest.raises(ValueError, match="Y"):
        B.lora_linear_fwd(d, torch.zeros(N, H, **e), p, torch.zeros(N, I - 1, **e), torch.zeros(N, R))
    q = B.qkv_desc(2, 16, H, 4, 2, 64, R, "bf16", 1e4)
    b = dict(dtype=torch.bfloat16)
    pq = B.proj(torch.zeros(256, H, **b), torch.zeros(R, H, **b), torch.zeros(256, R, **b), 2.0)
    pk = B.proj(torch.zeros(128, H, **b), torch.zeros(R, H, **b), torch.zeros(128, R, **b), 2.0)
    Q, K, V = torch.zeros(2, 4, 16, 64, **b), torch.zeros(2, 2, 16, 64, **b), torch.zeros(2, 2, 16, 32, **b)
    with pytest.raises(ValueError, match="V"):
        B.lora_qkv_fwd(q, torch.zeros(32, H, **b), pq, pk, pk, Q, K, V, torch.zeros(3, 32, R),
                       torch.zeros(64, dtype=torch.uint8))


def test_classes_refuse_x_in_another_dtype():
    t, projs = _mlp_tensors(torch.bfloat16)
    tt = {"X": t["X"]}
    with pytest.raises(ValueError, match="call dtype"):
        B.MLP(tt, N, H, I, R, "f32", "swiglu")
