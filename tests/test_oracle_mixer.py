"""Pins of the mixer oracle (oracle/mixer.py) against references that do not depend on it.

The pages print no worked numbers for the mixer, so every pin is a library routine, a
closed form or an identity the definitions fix:
* the causal convolution equals numpy.convolve with the reversed taps, channel by channel;
  a unit tap on the last position is the identity and a unit tap on the first a delay of
  three tokens;
* SiLU, sigmoid and log-sigmoid satisfy their odd-part identities
  (silu(x) - silu(-x) = x, sigmoid(x) + sigmoid(-x) = 1, logsig(x) - logsig(-x) = x),
  exp(logsig) = sigmoid, and logsig stays finite far into both tails;
* L2 normalisation gives unit rows and is scale invariant; the RMS output has unit RMS
  before the gate and is scale invariant;
* planted mistakes (taps reversed, a missing SiLU, the wrong norm axis, the gate dropped)
  fail these pins."""
import numpy as np
import pytest

import oracle
from oracle import mixer as M


def rng_inputs(seed, B=2, T=11, H=3, dk=8, dv=6):
    r = np.random.default_rng(seed)
    x = dict(xq=r.standard_normal((B, T, H, dk)), xk=r.standard_normal((B, T, H, dk)),
             xv=r.standard_normal((B, T, H, dv)), xb=2 * r.standard_normal((B, T, H, dk)),
             xw=2 * r.standard_normal((B, T, H, dv)), xa=3 * r.standard_normal((B, T, H, dk)),
             conv_q=r.standard_normal((H * dk, 4)), conv_k=r.standard_normal((H * dk, 4)),
             conv_v=r.standard_normal((H * dv, 4)))
    return x


def check_conv(conv):
    r = np.random.default_rng(1)
    B, T, H, d = 2, 9, 2, 5
    x = r.standard_normal((B, T, H, d))
    taps = r.standard_normal((H * d, 4))
    y = conv(x, taps)
    for b in range(B):
        for h in range(H):
            for c in range(d):
                ref = np.convolve(x[b, :, h, c], taps[h * d + c][::-1])[:T]
                np.testing.assert_allclose(y[b, :, h, c], ref, rtol=0, atol=1e-13)
    ident = np.zeros((H * d, 4)); ident[:, 3] = 1.0
    np.testing.assert_array_equal(conv(x, ident), x)
    delay = np.zeros((H * d, 4)); delay[:, 0] = 1.0
    yd = conv(x, delay)
    np.testing.assert_array_equal(yd[:, 3:], x[:, :-3])
    np.testing.assert_array_equal(yd[:, :3], 0.0)


def check_activations(silu, sigmoid, log_sigmoid):
    x = np.linspace(-30, 30, 601)
    np.testing.assert_allclose(silu(x) - silu(-x), x, rtol=0, atol=1e-12)
    assert silu(np.zeros(3)).tolist() == [0.0, 0.0, 0.0]
    np.testing.assert_allclose(sigmoid(x) + sigmoid(-x), 1.0, rtol=0, atol=1e-15)
    assert sigmoid(np.zeros(1))[0] == 0.5
    np.testing.assert_allclose(log_sigmoid(x) - log_sigmoid(-x), x, rtol=0, atol=1e-12)
    np.testing.assert_allclose(np.exp(log_sigmoid(x)), sigmoid(x), rtol=1e-14, atol=0)
    np.testing.assert_allclose(log_sigmoid(np.zeros(1)), [-np.log(2.0)], rtol=1e-15)
    far = log_sigmoid(np.array([-800.0, 800.0]))
    assert np.isfinite(far).all() and far[0] == -800.0 and far[1] == 0.0
    assert np.all(np.diff(sigmoid(x)) >= 0)


def check_prep(prep):
    x = rng_inputs(2)
    out = prep(**x, eps=0.0)
    # unit rows
    np.testing.assert_allclose(np.linalg.norm(out["q"], axis=-1), 1.0, rtol=1e-13)
    np.testing.assert_allclose(np.linalg.norm(out["k"], axis=-1), 1.0, rtol=1e-13)
    # eps enters inside the square root
    oe = prep(**x, eps=0.25)
    u = M.silu(M.causal_conv(x["xk"], x["conv_k"]))
    n2 = (u * u).sum(-1)
    np.testing.assert_allclose(np.linalg.norm(oe["k"], axis=-1) ** 2, n2 / (n2 + 0.25), rtol=1e-12)
    # gates and decay are the activations of their logits, token by token
    np.testing.assert_allclose(out["b"] + M.sigmoid(-x["xb"]), 1.0, atol=1e-15)
    np.testing.assert_allclose(out["log_alpha"] - M.log_sigmoid(-x["xa"]), x["xa"], atol=1e-12)
    assert (out["log_alpha"] <= 0).all()
    # identity taps: q is the normalised SiLU of the projection itself; scale invariance
    ident = np.zeros_like(x["conv_q"]); ident[:, 3] = 1.0
    x2 = dict(x, conv_q=ident, conv_k=ident * 2.5)
    o2 = prep(**x2, eps=0.0)
    u = M.silu(x["xq"])
    np.testing.assert_allclose(o2["q"] * np.linalg.norm(u, axis=-1, keepdims=True), u, atol=1e-12)
    # the value path has no normalisation: a unit delay shifts v by three tokens
    delay = np.zeros_like(x["conv_v"]); delay[:, 0] = 1.0
    o3 = prep(**dict(x, conv_v=delay))
    np.testing.assert_allclose(o3["v"][:, 3:], M.silu(x["xv"][:, :-3]), atol=1e-15)
    np.testing.assert_array_equal(o3["v"][:, :3], 0.0)


def check_out(out_fn):
    r = np.random.default_rng(3)
    o = r.standard_normal((2, 7, 3, 6)) * 5.0
    z = r.standard_normal((2, 7, 3, 6))
    gamma = r.uniform(0.5, 1.5, 6)
    y = out_fn(o, z, gamma, eps=0.0)
    pre = y / (gamma * M.silu(z))
    np.testing.assert_allclose(np.sqrt((pre ** 2).mean(-1)), 1.0, rtol=1e-12)
    np.testing.assert_allclose(out_fn(3.0 * o, z, gamma, eps=0.0), y, rtol=1e-12)
    # sign and direction follow o
    assert np.all(np.sign(pre) == np.sign(o))
    # eps: a zero row stays finite and zero
    yz = out_fn(np.zeros((1, 1, 1, 6)), np.ones((1, 1, 1, 6)), np.ones(6), eps=1e-6)
    assert np.all(yz == 0.0)


def test_causal_conv_equals_numpy_convolve():
    check_conv(M.causal_conv)


def test_activation_identities():
    check_activations(M.silu, M.sigmoid, M.log_sigmoid)


def test_mixer_prep_properties():
    check_prep(oracle.mixer_prep)


def test_mixer_out_properties():
    check_out(oracle.mixer_out)


# ---- planted mistakes must fail a pin ----

def _reversed_taps_conv(x, taps):
    return M.causal_conv(x, np.asarray(taps)[:, ::-1])


def _sigmoid_as_silu(x):
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x)) * 0.0 + 1.0 / (1.0 + np.exp(-x)) * (1.0 + 1e-3 * x)


def _prep_without_silu(xq, xk, xv, xb, xw, xa, conv_q, conv_k, conv_v, eps=1e-6):
    out = M.mixer_prep(xq, xk, xv, xb, xw, xa, conv_q, conv_k, conv_v, eps)
    out["v"] = M.causal_conv(xv, conv_v)
    return out


def _prep_norm_wrong_axis(xq, xk, xv, xb, xw, xa, conv_q, conv_k, conv_v, eps=1e-6):
    out = M.mixer_prep(xq, xk, xv, xb, xw, xa, conv_q, conv_k, conv_v, eps)
    u = M.silu(M.causal_conv(xq, conv_q))
    out["q"] = u / np.sqrt((u * u).sum(-2, keepdims=True) + eps)
    return out


def _out_without_gate(o, z, gamma, eps=1e-6):
    o = np.asarray(o, dtype=np.float64)
    return o / np.sqrt((o * o).mean(-1, keepdims=True) + eps) * np.asarray(gamma)


def _out_norm_over_heads(o, z, gamma, eps=1e-6):
    o = np.asarray(o, dtype=np.float64)
    return o / np.sqrt((o * o).mean(-2, keepdims=True) + eps) * gamma * M.silu(z)


@pytest.mark.parametrize("check,mutant", [
    (check_conv, _reversed_taps_conv),
    (lambda f: check_activations(lambda x: np.asarray(x) * f(x), f, M.log_sigmoid), _sigmoid_as_silu),
    (check_prep, _prep_without_silu),
    (check_prep, _prep_norm_wrong_axis),
    (check_out, _out_without_gate),
    (check_out, _out_norm_over_heads),
])
def test_planted_mistakes_fail_a_pin(check, mutant):
    with pytest.raises(AssertionError):
        check(mutant)
