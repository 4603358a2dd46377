"""Plant plausible mistakes in a copy of the oracle (on the CPU) and show that
at least one pin catches each.  The real oracle is never modified."""
import os
import types

import pytest

from tests import oracle_pins

SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "lora_oracle.py")

# (description, text in the oracle, replacement)
MUTATIONS = [
    ("adapter term dropped", "Y = Z @ W.T + s * (T @ B.T)", "Y = Z @ W.T"),
    ("scale applied twice", "Y = Z @ W.T + s * (T @ B.T)", "Y = Z @ W.T + s * s * (T @ B.T)"),
    ("side product uses W", "T = Z @ A.T\n    Y", "T = Z @ W[: A.shape[0]].T\n    Y"),
    ("dT missing scale", "dT = s * (dY @ B)", "dT = dY @ B"),
    ("dB missing scale", "dB = s * (dY.T @ T)", "dB = dY.T @ T"),
    ("dA halved", "dA = dT.T @ Z", "dA = dT.T @ Z * 0.5"),
    ("dA drops dT", "dA = dT.T @ Z", "dA = (dY @ B).T @ Z"),
    ("dZ drops adapter", "dZ = dY @ W + dT @ A", "dZ = dY @ W"),
    ("silu' drops term", "return sg * (1.0 + g * (1.0 - sg))", "return sg"),
    ("silu is sigmoid", "return g * _sigmoid(g)", "return _sigmoid(g)"),
    ("gelu_tanh cubic sign", "(g + _GELU_CUBIC * g ** 3)))", "(g - _GELU_CUBIC * g ** 3)))"),
    ("gelu_tanh' drops 1-t^2", "0.5 * g * (1.0 - t * t) * _SQRT_2_OVER_PI", "0.5 * g * _SQRT_2_OVER_PI"),
    ("GLU backward drops U", "dG = dH * f[\"U\"] * dphi(f[\"G\"])", "dG = dH * dphi(f[\"G\"])"),
    ("GLU backward swaps phi", "dU = dH * phi(f[\"G\"])", "dU = dH * dphi(f[\"G\"])"),
    ("dX drops up branch", "return {\"dX\": dXg + dXu,", "return {\"dX\": dXg,"),
    ("rope frequency exponent", "inv_freq = theta ** (-2.0 * j / head_dim)", "inv_freq = theta ** (-1.0 * j / head_dim)"),
    ("rope sign", "x1 * c - x2 * s, x2 * c + x1 * s", "x1 * c + x2 * s, x2 * c - x1 * s"),
    ("rope adjacent pairs", "x1, x2 = x[..., :h], x[..., h:]", "x1, x2 = x[..., 0::2], x[..., 1::2]"),
    ("rope transpose not inverted", "y1 * c + y2 * s, y2 * c - y1 * s", "y1 * c - y2 * s, y2 * c + y1 * s"),
    ("head split order", ".transpose(0, 2, 1, 3).copy()\n\n\ndef head_unsplit", ".transpose(0, 2, 1, 3)[:, ::-1].copy()\n\n\ndef head_unsplit"),
    ("rope on V", "if name != \"v\":\n            Z = rope_rotate", "if True:\n            Z = rope_rotate"),
    ("no RoPE adjoint in backward", "grads = {\"q\": rope_rotate_transpose(dQ, ang)", "grads = {\"q\": dQ"),
    ("rms eps outside sqrt", "1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)\n    return",
     "1.0 / (np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) + eps)\n    return"),
    ("rms norm drops weight", "return x * rinv * w, rinv[..., 0]", "return x * rinv, rinv[..., 0]"),
    ("rms backward drops mean term", "return rinv * (gw - xhat * np.mean(gw * xhat, axis=-1, keepdims=True))",
     "return rinv * gw"),
    ("qk norm after RoPE",
     ("            Z, rinv = rms_norm(Z, p[_NORM_KEYS[name]], norm_eps)\n",
      "        out[name.upper()] = Z\n"),
     ("            _, rinv = rms_norm(Z, p[_NORM_KEYS[name]], norm_eps)\n",
      "        if _NORM_KEYS.get(name) in p:\n"
      "            Z, _ = rms_norm(Z, p[_NORM_KEYS[name]], norm_eps)\n"
      "        out[name.upper()] = Z\n")),
    ("gelu_erf' drops density", " + g * np.exp(-0.5 * g * g) / math.sqrt(2.0 * math.pi)", ""),
    ("gelu_erf without 1/sqrt2", "_erf(g / math.sqrt(2.0)))\n\n\ndef gelu_erf_grad", "_erf(g))\n\n\ndef gelu_erf_grad"),
    ("bias dropped", "Y = Y + bias[None, :]", "Y = Y"),
    ("bias scaled with adapter", "Y = Y + bias[None, :]", "Y = Y + s * bias[None, :]"),
    ("qkv bias after RoPE",
     ("p[\"B_\" + name], s, p.get(\"b_\" + name))\n        Z = head_split(P, batch, seq, heads[name], head_dim)\n",
      "        out[name.upper()] = Z\n"),
     ("p[\"B_\" + name], s)\n        Z = head_split(P, batch, seq, heads[name], head_dim)\n",
      "        if p.get(\"b_\" + name) is not None:\n"
      "            Z = Z + head_split(np.broadcast_to(p[\"b_\" + name], P.shape), batch, seq, heads[name], head_dim)\n"
      "        out[name.upper()] = Z\n")),
]


def _mutant(old, new):
    """A copy of the oracle with `old` replaced by `new` (or, for tuples, each
    old[i] by new[i]); every anchor must occur exactly once."""
    src = open(SRC_PATH).read()
    olds, news = (old, new) if isinstance(old, tuple) else ((old,), (new,))
    for o, n in zip(olds, news):
        assert src.count(o) == 1, f"mutation anchor not unique/found: {o!r}"
        src = src.replace(o, n)
    mod = types.ModuleType("lora_oracle_mutant")
    exec(compile(src, "lora_oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("desc,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(desc, old, new):
    mod = _mutant(old, new)
    caught = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            check(mod)
        except Exception:  # an assertion or a shape error both count as caught
            caught.append(check.__name__)
    assert caught, f"no pin caught: {desc}"
