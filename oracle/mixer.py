"""fp64 CPU oracle of the mixer around the GDN-2 recurrence -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import this
module.  It shares no code with the HIP library and never imports it.  Plain numpy in
float64; every step is the textbook definition written out.

What is computed (page "Why NVIDIA Gated DeltaNet-2 separates erase and write gates",
axbrief.com, the section on the layer's architecture, and section "Gated Delta Rule-2" for
the gates):

* query and key path: linear projection, short causal convolution, SiLU, L2 normalisation;
* value path: linear projection, short convolution, SiLU;
* erase gate b and write gate w: sigmoid of a projection of the token;
* the layer output: RMS normalisation of the recurrence output and a SiLU output gate.

The projections are matrix products outside this module: its inputs are their outputs.
Readings where the pages are silent (each listed with the design notes):

* the short convolution has 4 taps (the pages: a small filter over 3 to 4 tokens), is
  depthwise (one filter per channel of every head), and tap j of channel c multiplies the
  input at token t - 3 + j; tokens before the start of the sequence are zero;
* L2 normalisation divides by sqrt(sum of squares + eps) over the head's dk channels;
* the decay takes the same sigmoid form as the two gates: log alpha = log sigmoid(a);
* the output is o / sqrt(mean(o^2) + eps) * gamma * SiLU(z), the mean over the head's dv
  channels, gamma one weight per channel shared by the heads, z an output-gate projection.

Parity status: pinned by tests/test_oracle_mixer.py (numpy.convolve for the convolution,
the odd-part identities of SiLU, sigmoid and log-sigmoid, unit norms, scale invariance and
the no-op cases of every step).
"""
from __future__ import annotations

import numpy as np

CONV_TAPS = 4


def _f64(x):
    if hasattr(x, "detach"):
        x = x.detach().cpu().double().numpy()
    return np.asarray(x, dtype=np.float64)


def sigmoid(x):
    """1 / (1 + e^-x), evaluated without overflow on either side."""
    x = _f64(x)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    e = np.exp(x[~pos])
    out[~pos] = e / (1.0 + e)
    return out


def log_sigmoid(x):
    """log(1 / (1 + e^-x)) = min(x, 0) - log(1 + e^-|x|)."""
    x = _f64(x)
    return np.minimum(x, 0.0) - np.log1p(np.exp(-np.abs(x)))


def silu(x):
    x = _f64(x)
    return x * sigmoid(x)


def causal_conv(x, taps):
    """Depthwise causal convolution along tokens.

    x [B,T,H,d], taps [H*d, W]: y[b,t,h,c] = sum_j taps[h*d + c, j] * x[b, t - W + 1 + j, h, c],
    with x = 0 before token 0."""
    x, taps = _f64(x), _f64(taps)
    B, T, H, d = x.shape
    W = taps.shape[1]
    tw = taps.reshape(H, d, W)
    y = np.zeros_like(x)
    for t in range(T):
        for j in range(W):
            s = t - W + 1 + j
            if s >= 0:
                y[:, t] += tw[None, :, :, j] * x[:, s]
    return y


def l2_normalize(u, eps):
    u = _f64(u)
    return u / np.sqrt((u * u).sum(-1, keepdims=True) + eps)


def mixer_prep(xq, xk, xv, xb, xw, xa, conv_q, conv_k, conv_v, eps=1e-6):
    """The recurrence's inputs from the projections' outputs.

    xq, xk, xb, xa [B,T,H,dk]; xv, xw [B,T,H,dv]; conv_q, conv_k [H*dk, 4]; conv_v [H*dv, 4].
    Returns q, k, v, b, w, log_alpha (fp64)."""
    q = l2_normalize(silu(causal_conv(xq, conv_q)), eps)
    k = l2_normalize(silu(causal_conv(xk, conv_k)), eps)
    v = silu(causal_conv(xv, conv_v))
    return dict(q=q, k=k, v=v, b=sigmoid(xb), w=sigmoid(xw), log_alpha=log_sigmoid(xa))


def mixer_out(o, z, gamma, eps=1e-6):
    """Layer output from the recurrence output o [B,T,H,dv], the gate projection z [B,T,H,dv]
    and the norm weight gamma [dv]."""
    o, z, gamma = _f64(o), _f64(z), _f64(gamma)
    rms = np.sqrt((o * o).mean(-1, keepdims=True) + eps)
    return o / rms * gamma * silu(z)
