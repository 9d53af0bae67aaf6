"""Plain fp64 front and back operations of the decode layer (test infrastructure
only; see the package docstring).

vLLM KdaSplit page, kernel body: before the recurrent update each of the three
sections (q, k, v) of a token's projected input x [3 * H * D] goes through a
causal depthwise convolution of 4 taps whose first three inputs are the conv
state [3 * H * D, 3] of the request's slot (oldest first) and whose fourth is x,
with per-section, per-tap, per-channel weights [3, 4, H * D] and an optional bias;
then SiLU (y * sigmoid(y)); q and k of each head are L2-normalised with 1e-6
inside the square root; beta = sigmoid(raw beta). The conv state of the slot
becomes its last two entries and x. After the update, the gated RMSNorm of each
head: o * rsqrt(mean(o^2) + eps) * w[channel] * sigmoid(gate). A row whose slot is
<= 0 is padding: zero outputs, nothing written. The decay (gate) stage of that
page is not modelled here; the query scale is applied by the decode step.
"""

import numpy as np


def _sig(x):
    return 1.0 / (1.0 + np.exp(-x))


def conv_silu_step(x, w, bias, conv_state, slots):
    """x [N, C] (C = 3 H D); w [3, 4, C / 3]; bias [C] or None; conv_state [P, C, 3];
    slots [N]. Returns (y [N, C] after SiLU, new conv_state)."""
    x = np.asarray(x, np.float64)
    st = np.asarray(conv_state, np.float64).copy()
    N, C = x.shape
    dim = C // 3
    wc = np.concatenate([np.asarray(w, np.float64)[s].T for s in range(3)], axis=0)  # [C, 4]
    y = np.zeros((N, C))
    for b in range(N):
        slot = int(slots[b])
        if slot <= 0:
            continue
        window = np.concatenate([st[slot], x[b][:, None]], axis=1)  # [C, 4]: oldest .. newest
        acc = np.sum(window * wc, axis=1)
        if bias is not None:
            acc = acc + np.asarray(bias, np.float64)
        y[b] = acc * _sig(acc)
        st[slot] = window[:, 1:]
    return y, st


def decode_prologue(x, w, bias, conv_state, slots, beta_raw, H, D):
    """The front operations for one decode token per request.

    Returns (q, k, v [N, H, D], beta [N, H], new conv_state); q and k unit-norm
    per head (up to the 1e-6), padding rows all zero."""
    y, st = conv_silu_step(x, w, bias, conv_state, slots)
    N = y.shape[0]
    dim = H * D
    q = y[:, :dim].reshape(N, H, D)
    k = y[:, dim:2 * dim].reshape(N, H, D)
    v = y[:, 2 * dim:].reshape(N, H, D)
    q = q / np.sqrt(np.sum(q * q, axis=-1, keepdims=True) + 1e-6)
    k = k / np.sqrt(np.sum(k * k, axis=-1, keepdims=True) + 1e-6)
    beta = _sig(np.asarray(beta_raw, np.float64))
    pad = np.asarray(slots) <= 0
    beta[pad] = 0.0
    return q, k, v, beta, st


def gated_rmsnorm(o, gate, w, eps):
    """o [N, H, D]; gate [N, H * D] (raw); w [D]. Returns [N, H, D]."""
    o = np.asarray(o, np.float64)
    N, H, D = o.shape
    rstd = 1.0 / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    return o * rstd * np.asarray(w, np.float64)[None, None, :] * _sig(np.asarray(gate, np.float64).reshape(N, H, D))
