"""Host-side checks of the C ABI (no GPU): the library loads, exports every
function include/lora_mi355x.h declares, and rejects bad arguments with the
documented status codes before touching the device."""
import ctypes
import os
import re

import pytest

from lora_fine_tuning_mlp_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lora_mi355x.h")

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH), reason="library not built")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(lora_[a-z0-9_]+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("lora_mlp_fwd", "lora_mlp_bwd", "lora_qkv_fwd", "lora_qkv_bwd", "lora_linear_fwd", "lora_linear_bwd",
              "lora_mlp_workspace_bytes", "lora_qkv_workspace_bytes", "lora_linear_workspace_bytes",
              "lora_status_string"):
        assert n in names


def test_every_declared_symbol_is_exported():
    h = ctypes.CDLL(B.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(h, n)]
    assert not missing, missing


def test_status_strings():
    lib = B.lib()
    assert lib.lora_status_string(0) == b"ok"
    for code in range(1, 6):
        assert lib.lora_status_string(code) not in (b"ok", b"unknown status")
    assert lib.lora_version().startswith(b"lora_mi355x")


def _mlp(**kw):
    d = dict(n_tokens=64, hidden=128, inter=256, rank=8, dtype="bf16", act="swiglu")
    d.update(kw)
    return B.mlp_desc(**d)


def _qkv(**kw):
    d = dict(batch=2, seq=32, hidden=128, n_q=4, n_kv=2, head_dim=64, rank=8, dtype="bf16", theta=1e4)
    d.update(kw)
    return B.qkv_desc(**d)


def test_workspace_queries():
    for p in (0, 1):
        assert B.lora_mlp_workspace_bytes(_mlp(), p) > 0
        assert B.lora_qkv_workspace_bytes(_qkv(), p) > 0
    # forward needs H [N, i] in the call dtype at least
    assert B.lora_mlp_workspace_bytes(_mlp(), 0) >= 64 * 256 * 2
    # invalid descriptors report 0
    assert B.lora_mlp_workspace_bytes(_mlp(rank=0), 0) == 0
    assert B.lora_qkv_workspace_bytes(_qkv(head_dim=48), 1) == 0
    assert B.lora_mlp_workspace_bytes(_mlp(), 2) == 0


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation first


def _call_mlp_fwd(desc, ws_bytes, null_x=False):
    lib = B.lib()
    pr = B.Proj(FAKE.value, FAKE.value, FAKE.value, 2.0)
    X = None if null_x else FAKE
    return lib.lora_mlp_fwd(ctypes.byref(desc) if desc is not None else None, X, ctypes.byref(pr), ctypes.byref(pr),
                            ctypes.byref(pr), FAKE, FAKE, FAKE, FAKE, FAKE, ws_bytes, None)


def test_mlp_validation_codes():
    lib = B.lib()
    assert _call_mlp_fwd(None, 1 << 40) == 1
    assert _call_mlp_fwd(_mlp(), 1 << 40, null_x=True) == 1
    assert _call_mlp_fwd(_mlp(n_tokens=-8), 1 << 40) == 2
    assert _call_mlp_fwd(_mlp(hidden=-4), 1 << 40) == 2
    assert _call_mlp_fwd(_mlp(rank=B.LORA_MAX_RANK + 1), 1 << 40) == 3
    bad_dtype = _mlp()
    bad_dtype.dtype = 7
    assert _call_mlp_fwd(bad_dtype, 1 << 40) == 3
    bad_act = _mlp()
    bad_act.act = 3
    assert _call_mlp_fwd(bad_act, 1 << 40) == 3
    need = B.lora_mlp_workspace_bytes(_mlp(), 0)
    assert _call_mlp_fwd(_mlp(), need - 1) == 4
    assert b"workspace" in lib.lora_last_error_message()
    # the fused MLP is bias-free: a projection carrying a bias is refused
    pb = B.Proj(FAKE.value, FAKE.value, FAKE.value, 2.0, FAKE.value)
    pr = B.Proj(FAKE.value, FAKE.value, FAKE.value, 2.0)
    assert lib.lora_mlp_fwd(ctypes.byref(_mlp()), FAKE, ctypes.byref(pr), ctypes.byref(pb), ctypes.byref(pr), FAKE,
                            FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == 3
    assert b"bias" in lib.lora_last_error_message()


def _call_qkv_bwd(desc, ws_bytes):
    lib = B.lib()
    pr = B.Proj(FAKE.value, FAKE.value, FAKE.value, 2.0)
    f = FAKE
    return lib.lora_qkv_bwd(ctypes.byref(desc), f, f, f, f, f, ctypes.byref(pr), ctypes.byref(pr), ctypes.byref(pr),
                            f, f, f, f, f, f, f, f, ws_bytes, None)


def test_qkv_validation_codes():
    assert _call_qkv_bwd(_qkv(head_dim=63), 1 << 40) == 2        # odd head_dim
    assert _call_qkv_bwd(_qkv(n_q=6, n_kv=4), 1 << 40) == 2      # n_q % n_kv != 0
    assert _call_qkv_bwd(_qkv(theta=0.0), 1 << 40) == 2
    assert _call_qkv_bwd(_qkv(head_dim=96), 1 << 40) == 3        # unsupported head_dim
    assert _call_qkv_bwd(_qkv(rank=32), 1 << 40) == 3
    need = B.lora_qkv_workspace_bytes(_qkv(), 1)
    assert _call_qkv_bwd(_qkv(), need - 256) == 4


def _lin(**kw):
    d = dict(n_tokens=64, in_features=128, out_features=96, rank=8, dtype="bf16")
    d.update(kw)
    return B.linear_desc(**d)


def test_linear_workspace_queries():
    assert B.lora_linear_workspace_bytes(_lin(), 0) == 0          # one tile, short K: no split
    # one output tile with a long K range: the forward splits K and needs workspace
    long_k = _lin(n_tokens=64, in_features=4096, out_features=256)
    assert B.lora_linear_workspace_bytes(long_k, 0) > 4 * 256 * 256 * 4
    assert B.lora_linear_workspace_bytes(_lin(n_tokens=64, in_features=4096, out_features=256, dtype="f32"), 0) == 0
    need = B.lora_linear_workspace_bytes(_lin(), 1)
    # at least the per-row-block dA partials [ceil(N/256)][in][16] and dB partials in float32
    assert need >= (128 + 96) * 16 * 4
    assert B.lora_linear_workspace_bytes(_lin(rank=0), 1) == 0
    assert B.lora_linear_workspace_bytes(_lin(), 3) == 0


def _call_linear_bwd(desc, ws_bytes, ws=FAKE):
    lib = B.lib()
    pr = B.Proj(FAKE.value, FAKE.value, FAKE.value, 2.0)
    f = FAKE
    return lib.lora_linear_bwd(ctypes.byref(desc) if desc is not None else None, f, f, f, ctypes.byref(pr), f, f, f,
                               ws, ws_bytes, None)


def test_linear_validation_codes():
    lib = B.lib()
    assert _call_linear_bwd(None, 1 << 40) == 1
    assert _call_linear_bwd(_lin(out_features=0), 1 << 40) == 2
    assert _call_linear_bwd(_lin(rank=B.LORA_MAX_RANK + 1), 1 << 40) == 3
    bad = _lin()
    bad.dtype = 9
    assert _call_linear_bwd(bad, 1 << 40) == 3
    need = B.lora_linear_workspace_bytes(_lin(), 1)
    assert _call_linear_bwd(_lin(), need - 1) == 4
    assert _call_linear_bwd(_lin(), need, ws=None) == 4
    pr = B.Proj(None, FAKE.value, FAKE.value, 2.0)
    assert lib.lora_linear_fwd(ctypes.byref(_lin()), FAKE, ctypes.byref(pr), FAKE, FAKE, None, 0, None) == 1


def test_qkv_norm_validation_codes():
    lib = B.lib()
    pr = B.Proj(FAKE.value, FAKE.value, FAKE.value, 2.0)
    f = FAKE
    ws = B.lora_qkv_workspace_bytes(_qkv(), 0)

    def fwd(norm, Pn=FAKE, rinv=FAKE):
        return lib.lora_qkv_norm_fwd(ctypes.byref(_qkv()), f, ctypes.byref(pr), ctypes.byref(pr), ctypes.byref(pr),
                                     ctypes.byref(norm) if norm is not None else None, f, f, f, f, Pn, rinv, f, ws,
                                     None)
    assert fwd(None) == 1
    assert fwd(B.QkNorm(None, FAKE.value, 1e-6)) == 1
    assert fwd(B.QkNorm(FAKE.value, FAKE.value, 1e-6), Pn=None) == 1
    assert fwd(B.QkNorm(FAKE.value, FAKE.value, -1.0)) == 2
    assert fwd(B.QkNorm(FAKE.value, 0x1002, 1e-6)) == 3          # misaligned weight
    assert b"aligned" in lib.lora_last_error_message()


def test_empty_batch_forward_is_a_no_op():
    """n_tokens = 0 (or batch = 0) is a valid call: the forward has nothing to
    write and needs no workspace, so it returns OK without touching memory."""
    lib = B.lib()
    pr = B.Proj(FAKE.value, FAKE.value, FAKE.value, 2.0)
    f = FAKE
    d = _mlp(n_tokens=0)
    assert B.lora_mlp_workspace_bytes(d, 0) == 0
    assert lib.lora_mlp_fwd(ctypes.byref(d), f, ctypes.byref(pr), ctypes.byref(pr), ctypes.byref(pr), f, f, f, f,
                            None, 0, None) == 0
    dl = _lin(n_tokens=0)
    assert lib.lora_linear_fwd(ctypes.byref(dl), f, ctypes.byref(pr), f, f, None, 0, None) == 0
    dq = _qkv(batch=0)
    ws = B.lora_qkv_workspace_bytes(dq, 0)
    assert lib.lora_qkv_fwd(ctypes.byref(dq), f, ctypes.byref(pr), ctypes.byref(pr), ctypes.byref(pr), f, f, f, f,
                            f, ws, None) == 0
    assert _call_mlp_fwd(_mlp(n_tokens=-1), 1 << 40) == 2


def test_kernel_names_listed():
    names = B.kernel_names()
    for k in ("k_gateup_fwd", "k_linear_fwd", "k_qkv_fwd", "k_down_bwd", "k_mlp_dx_bwd", "k_proj_dx_bwd",
              "k_qk_norm_bwd"):
        assert k in names


def test_noalloc_qkv_forward_is_exported_and_bounded():
    """The allocation-free QKV forward reports its fixed scratch size and
    refuses, before any device call, a shape whose RoPE table exceeds it."""
    lib = B.lib()
    cap = B.lora_qkv_fwd_noalloc_max_scratch_bytes()
    assert cap == 4 << 20
    pr = B.Proj(FAKE.value, FAKE.value, FAKE.value, 2.0)
    f = FAKE
    too_long = _qkv(batch=1, seq=cap // (64 * 4) + 8, head_dim=128)
    assert B.lora_qkv_workspace_bytes(too_long, 0) > cap
    assert lib.lora_qkv_fwd_noalloc(ctypes.byref(too_long), f, ctypes.byref(pr), ctypes.byref(pr), ctypes.byref(pr),
                                    f, f, f, f, None) == 4
    assert b"static buffer" in lib.lora_last_error_message()
    assert lib.lora_qkv_fwd_noalloc(ctypes.byref(_qkv(batch=0)), f, ctypes.byref(pr), ctypes.byref(pr),
                                    ctypes.byref(pr), f, f, f, f, None) == 0
