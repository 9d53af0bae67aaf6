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
page is ``oracle/gate.py``; the query scale is applied by the decode step.

For T > 1 tokens per request (speculative verify, the page's class docstring and
the kernel body's ``tokens`` branch) the conv page of slot[b, 0] holds T + 2
columns per channel; token t convolves the sequence (page columns a - 1, a,
a + 1, then x_0 .. x_{T-1}) at positions t .. t + 3, with a = accepted[b], and
the page becomes (column a, column a + 1, x_0, .., x_{T-1}).
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


def _sections(y, H, D):
    N = y.shape[0]
    dim = H * D
    return (y[:, :dim].reshape(N, H, D), y[:, dim:2 * dim].reshape(N, H, D), y[:, 2 * dim:].reshape(N, H, D))


def decode_prologue_verify(x, w, bias, conv_state, slots, accepted, beta_raw, H, D, T):
    """Front operations for T tokens per request (speculative verify).

    x [N * T, 3 H D] (rows b * T + t); w [3, 4, H D]; bias [3 H D] or None;
    conv_state [P, 3 H D, T + 2]; slots [N, C] (C >= T): the conv page is
    slot[b, 0], the recurrent state's source slot[b, accepted[b] - 1];
    accepted [N]; beta_raw [N * T, H].

    A request is padding (zero outputs, conv state untouched) when accepted[b] is
    outside [1, T] (its taps would leave the page) or its source or conv slot is
    not positive, or the conv slot is outside the pool. Returns (q, k, v
    [N * T, H, D], beta [N * T, H], new conv_state)."""
    x = np.asarray(x, np.float64)
    st = np.asarray(conv_state, np.float64).copy()
    P, C, W = st.shape
    assert W == T + 2
    N = x.shape[0] // T
    dim = C // 3
    wc = np.concatenate([np.asarray(w, np.float64)[s].T for s in range(3)], axis=0)  # [C, 4]
    y = np.zeros((N * T, C))
    active = np.zeros(N * T, bool)
    for b in range(N):
        acc = int(accepted[b])
        if not 1 <= acc <= T:
            continue
        src, cslot = int(slots[b, acc - 1]), int(slots[b, 0])
        if src <= 0 or cslot <= 0 or cslot >= P:
            continue
        page = st[cslot]
        seq = np.concatenate([page[:, acc - 1:acc + 2], x[b * T:(b + 1) * T].T], axis=1)  # [C, 3 + T]
        for t in range(T):
            a = np.sum(seq[:, t:t + 4] * wc, axis=1)
            if bias is not None:
                a = a + np.asarray(bias, np.float64)
            y[b * T + t] = a * _sig(a)
            active[b * T + t] = True
        st[cslot] = np.concatenate([page[:, acc:acc + 2], x[b * T:(b + 1) * T].T], axis=1)
    q, k, v = _sections(y, H, D)
    q = q / np.sqrt(np.sum(q * q, axis=-1, keepdims=True) + 1e-6)
    k = k / np.sqrt(np.sum(k * k, axis=-1, keepdims=True) + 1e-6)
    beta = _sig(np.asarray(beta_raw, np.float64))
    beta[~active] = 0.0
    return q, k, v, beta, st
