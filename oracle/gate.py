"""The per-key-channel decay ("gate") stage of the KDA decode layer, as the vLLM
KdaSplit page's gate projection computes it (method ``gate_warp`` and its
``multicast``). TEST INFRASTRUCTURE ONLY (see the package docstring).

For token t, head h and key channel ("feature") f of the recurrent state, with
the gate activation f_a [T, R] (bf16, R = 128), the projection weight
F_B [H * K, R] (bf16), a_log [H], dt_bias [H * K] (float32) and a scalar
lower_bound:

    raw      = sum_c f_a[t, c] * F_B[h K + f, c]      float32, in the order ``mode`` fixes
    raw_g    = bf16(raw)                              round to nearest even
    pre      = exp(a_log[h]) * (raw_g + dt_bias[h K + f])
    gate     = sigmoid(pre)
    log_dec  = lower_bound * gate                     (the decay is exp(log_dec))

The page keeps the projection in IEEE float32 and names three reduction orders
(``gate_mode``): 0 = one chain of eight 16-column MMA blocks, 1 = four chains of
two blocks summed as 0 + (((c0 + c1) + c2) + c3), 2 = sixteen partials of eight
FMAs (columns 8 i .. 8 i + 7, in column order) summed in a butterfly
(p[i] += p[i + 2^s] for s = 3, 2, 1, 0). The page does not say in which order an
MMA block adds its 16 products; the reading taken here is the IEEE one of the
other mode: fused multiply-adds in column order, so every mode is a fixed
sequence of correctly rounded float32 operations, which this oracle reproduces
exactly (``fma32``). raw_g is therefore exact (a rounding decision taken in the
same precision on both sides); the transcendental tail is in float64 here.
"""

from __future__ import annotations

import numpy as np

R = 128  # projection rank (columns of f_a and F_B) on the page


def _f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def fma32(a, b, c):
    """Correctly rounded float32 a * b + c (round to nearest even) for float32
    inputs, elementwise. The float32 product is exact in float64; the float64 sum
    s and its error e (TwoSum) give the exact result s + e, which is rounded to
    float32 once: rounding s alone differs only when s lies exactly halfway
    between two float32 numbers and e is not zero (then e decides)."""
    a, b, c = (np.asarray(x, np.float32).astype(np.float64) for x in (a, b, c))
    p = a * b  # exact: 24 + 24 significant bits
    s = p + c
    bb = s - p
    e = (p - (s - bb)) + (c - bb)
    r = s.astype(np.float32)
    rd = r.astype(np.float64)
    # neighbour of r on s's side
    toward = np.where(s > rd, np.float32(np.inf), np.float32(-np.inf)).astype(np.float32)
    nb = np.nextafter(r, toward).astype(np.float64)
    tie = (s != rd) & (np.abs(s - rd) == np.abs(nb - s)) & (e != 0)
    # at a tie s rounded to r (even); the exact value lies beyond s toward nb iff e
    # has the sign of (nb - s)
    beyond = tie & (np.sign(e) == np.sign(nb - s))
    r = np.where(beyond, nb.astype(np.float32), r)
    return np.asarray(r, np.float32)


def add32(a, b):
    """Correctly rounded float32 a + b."""
    return fma32(a, np.float32(1.0), b)


def round_bf16(x):
    """Round float32 values to bfloat16 (nearest even); returned as float64."""
    f = np.ascontiguousarray(np.asarray(x, np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _chain(x, w, cols):
    """float32 FMA chain from 0 over columns ``cols`` of x [..., R] * w [..., R]."""
    acc = np.zeros(np.broadcast_shapes(x.shape[:-1], w.shape[:-1]), np.float32)
    for c in cols:
        acc = fma32(x[..., c], w[..., c], acc)
    return acc


def projection(f_a, f_b, mode):
    """raw [T, F] = f_a [T, R] . f_b [F, R]^T in float32, reduction order ``mode``."""
    x = _f32(f_a)[:, None, :]  # [T, 1, R]
    w = _f32(f_b)[None, :, :]  # [1, F, R]
    if mode == 0:
        return _chain(x, w, range(R))
    if mode == 1:
        p = [_chain(x, w, range(32 * j, 32 * j + 32)) for j in range(4)]
        return add32(np.float32(0.0), add32(add32(add32(p[0], p[1]), p[2]), p[3]))
    if mode == 2:
        p = [_chain(x, w, range(8 * i, 8 * i + 8)) for i in range(16)]
        for s in (3, 2, 1, 0):
            for i in range(1 << s):
                p[i] = add32(p[i], p[i | (1 << s)])
        return p[0]
    raise ValueError(f"unknown gate mode {mode}")


def kda_gate(f_a, f_b, a_log, dt_bias, lower_bound, H, K, mode):
    """Per-key-channel log-decays of the KDA decode layer.

    f_a [T, 128]; f_b [H * K, 128]; a_log [H]; dt_bias [H * K]; lower_bound a
    scalar. Returns (raw_g [T, H, K] (bf16 values), log_decay [T, H, K]), float64.
    """
    T = np.asarray(f_a).shape[0]
    raw_g = round_bf16(projection(f_a, f_b, mode)).reshape(T, H, K)
    a = np.asarray(a_log, np.float64).reshape(1, H, 1)
    dt = np.asarray(dt_bias, np.float64).reshape(1, H, K)
    pre = np.exp(a) * (raw_g + dt)
    gate = 1.0 / (1.0 + np.exp(-pre))
    return raw_g, float(lower_bound) * gate
