"""Plain fp64 implementations of the gated delta rule (see the package docstring).

TEST INFRASTRUCTURE ONLY: never imported by the product path.

Notation, per sequence and head: q_t, k_t in R^K, v_t in R^V, beta_t in (0, 1),
a_t <= 0 the raw per-token log-gate, s the query scale. The state S is V x K
(rows = value channels, columns = key channels), the layout of the recurrent
state pool on the vLLM KdaSplit page (class docstring: state [slot, head, value,
key]). The chunk kernels of the WarpDrive page carry h = S^T (K x V).

Readings where the pages are silent (each listed in the design notes):
* the gate argument is the raw per-token log-gate a_t; the chunk form uses its
  inclusive cumulative sum restarted at every chunk start;
* chunks are [64c, min(64c + 64, T)) counted from each sequence's start; a short
  last chunk uses g at its last valid row as g_last;
* the WY matrix A of recompute_w_u is (I + StrictLower(diag(beta) K K^T * E))^-1
  with E_ij = exp(g_i - g_j);
* the scale multiplies q only.
"""

from __future__ import annotations

import numpy as np

CHUNK = 64


def _as64(x):
    return np.asarray(x, dtype=np.float64)


def recurrent_fwd(q, k, v, a, beta, scale=1.0, S0=None):
    """Per-token gated delta rule: the definition the chunked form must reproduce.

    Follows the step order of the vLLM KdaSplit page, method ``update`` (decay the
    state rows, dot each row with k, v_new = (v - dot) * beta, rank-one update of
    the rows with k, dot the updated rows with the query), with a scalar decay per
    token and head instead of that page's per-key-channel decays:

        S <- exp(a_t) S
        delta = beta_t (v_t - S k_t)
        S <- S + delta k_t^T
        o_t = S (s q_t)

    q, k: [T, H, K]; v: [T, H, V]; a, beta: [T, H]; S0: [H, V, K] or None (zeros).
    Returns (o [T, H, V], S_T [H, V, K]).
    """
    q, k, v, a, beta = map(_as64, (q, k, v, a, beta))
    T, H, K = q.shape
    V = v.shape[-1]
    S = np.zeros((H, V, K)) if S0 is None else _as64(S0).copy()
    o = np.zeros((T, H, V))
    for t in range(T):
        S *= np.exp(a[t])[:, None, None]
        dot = np.einsum("hvk,hk->hv", S, k[t])
        delta = beta[t][:, None] * (v[t] - dot)
        S += delta[:, :, None] * k[t][:, None, :]
        o[t] = np.einsum("hvk,hk->hv", S, scale * q[t])
    return o, S


def unit_lower_inverse(L):
    """(I + L)^-1 for strictly lower-triangular L, by forward substitution.

    Row i of (I + L) A = I gives A[i, :i] = -L[i, :i] A[:i, :i], A[i, i] = 1.
    L: [..., n, n]. Returns A of the same shape.
    """
    L = _as64(L)
    n = L.shape[-1]
    A = np.zeros_like(L)
    idx = np.arange(n)
    A[..., idx, idx] = 1.0
    for i in range(1, n):
        A[..., i, :i] = -np.einsum("...m,...mj->...j", L[..., i, :i], A[..., :i, :i])
    return A


def chunked_fwd(q, k, v, a, beta, scale=1.0, S0=None, chunk=CHUNK, return_stages=False):
    """Chunked WY form of the gated delta rule (WarpDrive page, kernels 5, 3, 4 and
    its "Pipeline" paragraph: recompute_w_u, then chunk_fwd_h, then chunk_fwd_o).

    For each chunk of n <= 64 rows, with h the K x V state entering the chunk:

    * g = inclusive cumulative sum of a over the chunk; g_L = g at its last row;
    * L_ij = beta_i (k_i . k_j) exp(g_i - g_j) for j < i, else 0 (exp taken only
      where j < i); A = (I + L)^-1 (the chunk's WY matrix);
    * recompute_w_u: u = A diag(beta) V, w = A diag(beta exp(g)) K;
    * chunk_fwd_h (its five steps): keep h_n = h; v_new = u - w h;
      v_gated = diag(exp(g_L - g)) v_new; h <- exp(g_L) h; h <- h + K^T v_gated;
    * chunk_fwd_o: inter = s diag(exp(g)) Q h_n; P = s (Q K^T) * E * M with
      E_ij = exp(g_i - g_j), M_ij = [i >= j] (the inclusive causal mask);
      intra = P v_new; o = inter + intra.

    Shapes as ``recurrent_fwd``. Returns (o, S_T) and, with ``return_stages``, a
    list of per-chunk dicts holding g, A, u, w, h (entering state, K x V), v_new, P.
    """
    q, k, v, a, beta = map(_as64, (q, k, v, a, beta))
    T, H, K = q.shape
    V = v.shape[-1]
    h = np.zeros((H, K, V)) if S0 is None else _as64(S0).transpose(0, 2, 1).copy()
    o = np.zeros((T, H, V))
    stages = []
    for c0 in range(0, T, chunk):
        n = min(chunk, T - c0)
        rows = slice(c0, c0 + n)
        Q = q[rows].transpose(1, 0, 2)  # [H, n, K]
        Kc = k[rows].transpose(1, 0, 2)  # [H, n, K]
        Vc = v[rows].transpose(1, 0, 2)  # [H, n, V]
        b = beta[rows].T  # [H, n]
        g = np.cumsum(a[rows].T, axis=1)  # [H, n]
        gL = g[:, -1]
        diff = g[:, :, None] - g[:, None, :]  # g_i - g_j
        strict = np.tril(np.ones((n, n), dtype=bool), -1)
        incl = np.tril(np.ones((n, n), dtype=bool), 0)
        E_strict = np.where(strict, np.exp(np.where(strict, diff, 0.0)), 0.0)
        E_incl = np.where(incl, np.exp(np.where(incl, diff, 0.0)), 0.0)

        L = b[:, :, None] * (Kc @ Kc.transpose(0, 2, 1)) * E_strict
        A = unit_lower_inverse(L)
        u = A @ (b[:, :, None] * Vc)
        w = A @ ((b * np.exp(g))[:, :, None] * Kc)

        h_n = h
        v_new = u - w @ h_n
        P = scale * (Q @ Kc.transpose(0, 2, 1)) * E_incl
        o_c = scale * np.exp(g)[:, :, None] * (Q @ h_n) + P @ v_new
        o[rows] = o_c.transpose(1, 0, 2)
        v_gated = np.exp(gL[:, None] - g)[:, :, None] * v_new
        h = np.exp(gL)[:, None, None] * h_n + Kc.transpose(0, 2, 1) @ v_gated
        if return_stages:
            stages.append(dict(g=g, A=A, u=u, w=w, h=h_n, v_new=v_new, P=P))
    S_T = h.transpose(0, 2, 1).copy()
    if return_stages:
        return o, S_T, stages
    return o, S_T


def _varlen(fn, q, k, v, a, beta, cu_seqlens, scale, S0):
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    N = len(cu) - 1
    H, V, K = q.shape[1], v.shape[-1], q.shape[-1]
    o = np.zeros((q.shape[0], H, V))
    ST = np.zeros((N, H, V, K))
    for s in range(N):
        r = slice(int(cu[s]), int(cu[s + 1]))
        init = None if S0 is None else S0[s]
        if cu[s + 1] == cu[s]:
            ST[s] = np.zeros((H, V, K)) if init is None else _as64(init)
            continue
        o[r], ST[s] = fn(q[r], k[r], v[r], a[r], beta[r], scale=scale, S0=init)
    return o, ST


def recurrent_fwd_varlen(q, k, v, a, beta, cu_seqlens, scale=1.0, S0=None):
    """``recurrent_fwd`` applied to each sequence [cu[s], cu[s+1]) of a packed
    stream independently. S0: [N, H, V, K] or None. Returns (o, S_T [N, H, V, K]).
    An empty sequence passes its initial state through."""
    return _varlen(recurrent_fwd, q, k, v, a, beta, cu_seqlens, scale, S0)


def chunked_fwd_varlen(q, k, v, a, beta, cu_seqlens, scale=1.0, S0=None):
    """``chunked_fwd`` per sequence of a packed stream; the chunk grid restarts at
    every sequence start."""
    return _varlen(chunked_fwd, q, k, v, a, beta, cu_seqlens, scale, S0)


def decode_step(q, k, v, a, beta, pool, slots, scale=1.0):
    """One recurrent step for N requests over a slot-indexed state pool.

    vLLM KdaSplit page, class docstring: the state pool is [slot, head, value,
    key]; a row whose slot is <= 0 is padding, which is never written and whose
    output is zero (the kernel body's padding branch). For every other row b and
    head h the state pool[slots[b], h] takes one step of ``recurrent_fwd``.

    q, k: [N, H, K]; v: [N, H, V]; a, beta: [N, H]; pool: [P, H, V, K]; slots: [N].
    Returns (o [N, H, V], new_pool); the input pool is not modified.
    """
    q, k, v, a, beta = map(_as64, (q, k, v, a, beta))
    pool = _as64(pool).copy()
    N, H, _ = q.shape
    o = np.zeros((N, H, v.shape[-1]))
    for b in range(N):
        slot = int(slots[b])
        if slot <= 0:
            continue
        ob, S = recurrent_fwd(q[b:b + 1], k[b:b + 1], v[b:b + 1], a[b:b + 1],
                              beta[b:b + 1], scale=scale, S0=pool[slot])
        o[b] = ob[0]
        pool[slot] = S
    return o, pool


def decode_verify(q, k, v, a, beta, pool, slots, accepted, scale=1.0):
    """Speculative-verify decode: T tokens per request over a slot-indexed pool.

    vLLM KdaSplit page, class docstring (``tokens`` q > 1): request b's T tokens
    (rows b * T + t) run in order; its state comes from pool[slots[b, accepted[b]
    - 1]], and the state after token t goes to pool[slots[b, t]] when that slot is
    > 0. A request whose source slot is <= 0 (or whose accepted count is outside
    [1, slot columns], a reading where the page is silent) is padding: its outputs
    are zero and nothing is written. Each token is one step of ``recurrent_fwd``.

    q, k: [N, T, H, K]; v: [N, T, H, V]; a, beta: [N, T, H]; pool: [P, H, V, K];
    slots: [N, C] with C >= T; accepted: [N]. Returns (o [N, T, H, V], new_pool);
    the input pool is not modified.
    """
    q, k, v, a, beta = map(_as64, (q, k, v, a, beta))
    pool = _as64(pool).copy()
    N, T, H, _ = q.shape
    o = np.zeros((N, T, H, v.shape[-1]))
    cols = slots.shape[1]
    for b in range(N):
        acc = int(accepted[b])
        if not 1 <= acc <= cols:
            continue
        src = int(slots[b, acc - 1])
        if src <= 0:
            continue
        S = pool[src].copy()
        for t in range(T):
            ot, S = recurrent_fwd(q[b, t:t + 1], k[b, t:t + 1], v[b, t:t + 1], a[b, t:t + 1],
                                  beta[b, t:t + 1], scale=scale, S0=S)
            o[b, t] = ot[0]
            dst = int(slots[b, t])
            if dst > 0:
                pool[dst] = S
    return o, pool


def recurrent_fwd_kda(q, k, v, g, beta, scale=1.0, S0=None):
    """Delta rule with a decay per key channel (the vLLM KdaSplit page, method
    ``update``: every state element of key column e is multiplied by that column's
    decay, then the same delta-rule write and query dot as ``recurrent_fwd``):

        S <- S diag(exp(g_t))          (g_t in R^K, the per-channel log-decay)
        delta = beta_t (v_t - S k_t);  S <- S + delta k_t^T;  o_t = S (s q_t)

    q, k, g: [T, H, K]; v: [T, H, V]; beta: [T, H]; S0: [H, V, K] or None.
    Returns (o [T, H, V], S_T [H, V, K]).
    """
    q, k, v, g, beta = map(_as64, (q, k, v, g, beta))
    T, H, K = q.shape
    V = v.shape[-1]
    S = np.zeros((H, V, K)) if S0 is None else _as64(S0).copy()
    o = np.zeros((T, H, V))
    for t in range(T):
        S *= np.exp(g[t])[:, None, :]
        dot = np.einsum("hvk,hk->hv", S, k[t])
        delta = beta[t][:, None] * (v[t] - dot)
        S += delta[:, :, None] * k[t][:, None, :]
        o[t] = np.einsum("hvk,hk->hv", S, scale * q[t])
    return o, S


def decode_step_kda(q, k, v, g, beta, pool, slots, scale=1.0):
    """``decode_step`` with a per-key-channel log-decay g [N, H, K]: one step of
    ``recurrent_fwd_kda`` per active row over the slot-indexed pool (slot <= 0 is
    padding: zero output, nothing written)."""
    q, k, v, g, beta = map(_as64, (q, k, v, g, beta))
    pool = _as64(pool).copy()
    N, H, _ = q.shape
    o = np.zeros((N, H, v.shape[-1]))
    for b in range(N):
        slot = int(slots[b])
        if slot <= 0:
            continue
        ob, S = recurrent_fwd_kda(q[b:b + 1], k[b:b + 1], v[b:b + 1], g[b:b + 1], beta[b:b + 1],
                                  scale=scale, S0=pool[slot])
        o[b] = ob[0]
        pool[slot] = S
    return o, pool
