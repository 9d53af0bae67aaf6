"""Thin torch-facing wrappers over the C ABI (argument marshalling only).

Torch supplies device memory and the current stream; every step of the
computation runs in the HIP kernels of libgdn.so.
"""

from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import torch

from . import _lib

__all__ = ["chunk_fwd", "chunk_fwd_noalloc", "chunk_fwd_plan", "recurrent_step", "workspace_bytes", "GdnError"]

GdnError = _lib.GdnError

_DTYPES = {torch.bfloat16: _lib.GDN_BF16, torch.float32: _lib.GDN_F32}


def _dt(t: torch.dtype) -> int:
    if t not in _DTYPES:
        raise TypeError(f"unsupported dtype {t}; use torch.bfloat16 or torch.float32")
    return _DTYPES[t]


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _shape(t: Optional[torch.Tensor], shape, name: str):
    """Rejects a tensor whose shape is not ``shape``: the C ABI takes sizes, not
    shapes, so a wrong-sized buffer would otherwise be read or written out of bounds."""
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _need(t: torch.Tensor, name: str, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def workspace_bytes(n_seqs: int, total_tokens: int, H: int, K: int, V: int, in_dtype=torch.bfloat16) -> int:
    """Device workspace bytes ``chunk_fwd`` needs (see gdn_chunk_fwd_workspace_bytes)."""
    return int(_lib.lib().gdn_chunk_fwd_workspace_bytes(n_seqs, total_tokens, H, K, V, _dt(in_dtype)))


def chunk_fwd_plan(n_seqs: int, total_tokens: int, max_len: int, H: int, K: int, V: int, in_dtype=torch.bfloat16):
    """Segment plan and workspace offsets of ``chunk_fwd`` for these sizes (see
    gdn_chunk_fwd_plan): ((segments, chunks of segment 0, chunks of segments
    1 .. n - 2), {name: byte offset} for "af", "pf", "gx", "seg_sum", "seg_state")."""
    plan = (ctypes.c_int32 * 3)()
    offs = (ctypes.c_int64 * 5)()
    _lib.check(_lib.lib().gdn_chunk_fwd_plan(n_seqs, total_tokens, max_len, H, K, V, _dt(in_dtype), plan, offs),
               "gdn_chunk_fwd_plan")
    return tuple(plan), dict(zip(("af", "pf", "gx", "seg_sum", "seg_state"), tuple(offs)))


def chunk_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor, *,
              scale: Optional[float] = None, cu_seqlens: Optional[Sequence[int]] = None,
              cu_seqlens_dev: Optional[torch.Tensor] = None, h0: Optional[torch.Tensor] = None,
              output_final_state: bool = True, ht: Optional[torch.Tensor] = None,
              state_pool: Optional[torch.Tensor] = None, state_slots: Optional[torch.Tensor] = None,
              out_dtype: Optional[torch.dtype] = None, out: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None, stream=None, events: Optional[Sequence[int]] = None):
    """Chunked gated delta rule forward (gdn_chunk_fwd).

    q, k: [B, T, H, K] (B equal-length sequences) or [Ttot, H, K] with
    ``cu_seqlens`` (host sequence offsets, length N + 1); v: [..., H, V];
    g, beta: [..., H] float32 (g is the raw per-token log-gate). ``h0``:
    [N, H, V, K] float32. Returns (o, ht): o shaped like v in ``out_dtype``
    (default: q's dtype); ht [N, H, V, K] float32 or None. With ``state_pool``
    ([P, H, V, K]) and ``state_slots`` ([N] int32) the initial and final states
    live in the pool (updated in place) and ht is None. ``events``: three
    hipEvent_t handles recorded around the prep and scan kernels
    (gdn_chunk_fwd_profiled).
    """
    return _chunk_call(q, k, v, g, beta, scale, cu_seqlens, cu_seqlens_dev, h0, output_final_state, ht, state_pool,
                       state_slots, out_dtype, out, workspace, stream, events, noalloc=False, kda=False)


def chunk_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor, *,
                      out: torch.Tensor, scale: Optional[float] = None, cu_seqlens: Optional[Sequence[int]] = None,
                      cu_seqlens_dev: Optional[torch.Tensor] = None, h0: Optional[torch.Tensor] = None,
                      ht: Optional[torch.Tensor] = None, state_pool: Optional[torch.Tensor] = None,
                      state_slots: Optional[torch.Tensor] = None, stream=None):
    """``chunk_fwd`` through gdn_chunk_fwd_noalloc: no workspace argument and no
    device allocation, here or in the library (whose workspace is its own device
    array of GDN_NOALLOC_WORKSPACE_BYTES). ``out`` must be given (its dtype is
    the output dtype); the final state is stored only into a given ``ht`` (or
    the pool); packed calls need ``cu_seqlens_dev`` as well as ``cu_seqlens``.
    Returns (out, ht)."""
    if out is None:
        raise ValueError("chunk_fwd_noalloc needs out")
    if cu_seqlens is not None and cu_seqlens_dev is None:
        raise ValueError("chunk_fwd_noalloc needs cu_seqlens_dev with cu_seqlens")
    return _chunk_call(q, k, v, g, beta, scale, cu_seqlens, cu_seqlens_dev, h0, False, ht, state_pool, state_slots,
                       out.dtype, out, None, stream, None, noalloc=True, kda=False)


def _chunk_call(q, k, v, g, beta, scale, cu_seqlens, cu_seqlens_dev, h0, output_final_state, ht, state_pool,
                state_slots, out_dtype, out, workspace, stream, events, noalloc, kda):
    H, K = q.shape[-2], q.shape[-1]
    V = v.shape[-1]
    if q.dim() == 4:
        if cu_seqlens is not None:
            raise ValueError("cu_seqlens needs packed [Ttot, H, K] inputs")
        n_seqs, total = q.shape[0], q.shape[0] * q.shape[1]
    elif q.dim() == 3:
        total = q.shape[0]
        n_seqs = 1 if cu_seqlens is None else len(cu_seqlens) - 1
    else:
        raise ValueError("q must be [B, T, H, K] or [Ttot, H, K]")
    g_shape = q.shape if kda else q.shape[:-1]
    if k.shape != q.shape or v.shape[:-1] != q.shape[:-1] or g.shape != g_shape or beta.shape != q.shape[:-1]:
        raise ValueError("inconsistent shapes of q, k, v, g, beta")
    if cu_seqlens is not None and n_seqs < 1:
        raise ValueError("cu_seqlens needs at least two offsets")
    state = (n_seqs, H, V, K)
    _shape(out, v.shape, "out")
    if state_pool is not None:
        if h0 is not None or ht is not None:
            raise ValueError("h0 and ht must be None when state_pool is given")
        if state_slots is None:
            raise ValueError("state_pool needs state_slots")
        if state_pool.dim() != 4 or tuple(state_pool.shape[1:]) != (H, V, K):
            raise ValueError(f"state_pool must have shape (P, {H}, {V}, {K}), got {tuple(state_pool.shape)}")
        _shape(state_slots, (n_seqs,), "state_slots")
    else:
        _shape(h0, state, "h0")
        _shape(ht, state, "ht")
    if cu_seqlens_dev is not None:
        _shape(cu_seqlens_dev, (n_seqs + 1,), "cu_seqlens_dev")
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, q.dtype)
    for name, t in (("g", g), ("beta", beta)):
        _need(t, name, torch.float32)
    in_dt = q.dtype
    out_dtype = out_dtype or in_dt
    if out is None:
        out = torch.empty(v.shape, dtype=out_dtype, device=v.device)
    _need(out, "out", out_dtype)

    cu_host = cu_dev = None
    if cu_seqlens is not None:
        host = torch.as_tensor(list(cu_seqlens) if not torch.is_tensor(cu_seqlens) else cu_seqlens,
                               dtype=torch.int32).cpu().contiguous()
        cu_host = host
        cu_dev = cu_seqlens_dev if cu_seqlens_dev is not None else host.to(q.device)
        _need(cu_dev, "cu_seqlens_dev", torch.int32)

    if state_pool is not None:
        _need(state_pool, "state_pool", torch.float32)
        _need(state_slots, "state_slots", torch.int32)
        ht = None
        pool_slots = state_pool.shape[0]
    else:
        pool_slots = 0
        if h0 is not None:
            _need(h0, "h0", torch.float32)
        if output_final_state and ht is None:
            ht = torch.empty((n_seqs, H, V, K), dtype=torch.float32, device=q.device)
        if ht is not None:
            _need(ht, "ht", torch.float32)

    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(out), n_seqs, total, H, K, V,
            float(K ** -0.5 if scale is None else scale), _dt(in_dt), _dt(out_dtype),
            _ptr(cu_dev), None if cu_host is None else cu_host.data_ptr(),
            _ptr(h0), _ptr(ht), _ptr(state_pool), pool_slots, _ptr(state_slots))
    L = _lib.lib()
    if noalloc:
        _lib.check(L.gdn_chunk_fwd_noalloc(*args, _stream(stream)), "gdn_chunk_fwd_noalloc")
        return out, ht
    if kda:
        need, fn, fn_prof, name = (int(L.gdn_chunk_fwd_kda_workspace_bytes(n_seqs, total, H, K)), L.gdn_chunk_fwd_kda,
                                   L.gdn_chunk_fwd_kda_profiled, "gdn_chunk_fwd_kda")
    else:
        need, fn, fn_prof, name = (workspace_bytes(n_seqs, total, H, K, V, in_dt), L.gdn_chunk_fwd,
                                   L.gdn_chunk_fwd_profiled, "gdn_chunk_fwd")
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    args = args + (_ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    st = fn(*args) if events is None else fn_prof(*args, (ctypes.c_void_p * 3)(*events))
    _lib.check(st, name)
    return out, ht


def recurrent_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
                   state_pool: torch.Tensor, slots: torch.Tensor, *, scale: Optional[float] = None,
                   out_dtype: Optional[torch.dtype] = None, out: Optional[torch.Tensor] = None, stream=None):
    """One decode step (gdn_recurrent_step): q, k [N, H, K]; v [N, H, V]; g, beta
    [N, H] float32; state_pool [P, H, V, K] float32 updated in place; slots [N]
    int32 (<= 0: padding). Returns o [N, H, V]."""
    N, H, K = q.shape
    V = v.shape[-1]
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, q.dtype)
    for name, t in (("g", g), ("beta", beta), ("state_pool", state_pool)):
        _need(t, name, torch.float32)
    _need(slots, "slots", torch.int32)
    if k.shape != q.shape or v.shape[:2] != (N, H) or g.shape != (N, H) or beta.shape != (N, H):
        raise ValueError("inconsistent shapes of q, k, v, g, beta")
    if state_pool.dim() != 4 or tuple(state_pool.shape[1:]) != (H, V, K) or slots.shape != (N,):
        raise ValueError("state_pool must be [P, H, V, K] and slots [N]")
    out_dtype = out_dtype or q.dtype
    if out is None:
        out = torch.empty((N, H, V), dtype=out_dtype, device=q.device)
    _need(out, "out", out_dtype)
    st = _lib.lib().gdn_recurrent_step(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_pool), state_pool.shape[0], _ptr(slots),
        _ptr(out), N, H, K, V, float(K ** -0.5 if scale is None else scale), _dt(q.dtype), _dt(out_dtype),
        _stream(stream))
    _lib.check(st, "gdn_recurrent_step")
    return out



def recurrent_verify(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
                     state_pool: torch.Tensor, slots: torch.Tensor, accepted: torch.Tensor, *,
                     scale: Optional[float] = None, out_dtype: Optional[torch.dtype] = None,
                     out: Optional[torch.Tensor] = None, stream=None):
    """Speculative-verify decode (gdn_recurrent_verify): q, k [N, T, H, K]; v
    [N, T, H, V]; g, beta [N, T, H] float32; state_pool [P, H, V, K] float32,
    written in place at the per-token slots; slots [N, C] int32 (C >= T);
    accepted [N] int32. Returns o [N, T, H, V]."""
    N, T, H, K = q.shape
    V = v.shape[-1]
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, q.dtype)
    for name, t in (("g", g), ("beta", beta), ("state_pool", state_pool)):
        _need(t, name, torch.float32)
    _need(slots, "slots", torch.int32)
    _need(accepted, "accepted", torch.int32)
    if k.shape != q.shape or v.shape[:3] != (N, T, H) or g.shape != (N, T, H) or beta.shape != (N, T, H):
        raise ValueError("inconsistent shapes of q, k, v, g, beta")
    if state_pool.dim() != 4 or tuple(state_pool.shape[1:]) != (H, V, K):
        raise ValueError("state_pool must be [P, H, V, K]")
    if slots.dim() != 2 or slots.shape[0] != N or accepted.shape != (N,):
        raise ValueError("slots must be [N, C] and accepted [N]")
    out_dtype = out_dtype or q.dtype
    if out is None:
        out = torch.empty((N, T, H, V), dtype=out_dtype, device=q.device)
    _need(out, "out", out_dtype)
    st = _lib.lib().gdn_recurrent_verify(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_pool), state_pool.shape[0], _ptr(slots),
        slots.shape[1], _ptr(accepted), _ptr(out), N, T, H, K, V, float(K ** -0.5 if scale is None else scale),
        _dt(q.dtype), _dt(out_dtype), _stream(stream))
    _lib.check(st, "gdn_recurrent_verify")
    return out


def kda_gate(f_a: torch.Tensor, f_b: torch.Tensor, a_log: torch.Tensor, dt_bias: torch.Tensor,
             lower_bound: float, H: int, *, mode: int = 0, with_raw: bool = False, out: Optional[torch.Tensor] = None,
             stream=None):
    """Per-key-channel log-decays of the KDA decode layer (gdn_kda_gate): f_a bf16
    [N, 128]; f_b bf16 [H * K, 128]; a_log float32 [H]; dt_bias float32 [H * K].
    Returns g float32 [N, H, K] (and the bf16 projection [N, H, K] with
    ``with_raw``)."""
    N = f_a.shape[0]
    if f_a.dim() != 2 or f_a.shape[1] != 128:
        raise ValueError("f_a must be [N, 128]")
    if f_b.dim() != 2 or f_b.shape[1] != 128 or f_b.shape[0] % H:
        raise ValueError("f_b must be [H * K, 128]")
    K = f_b.shape[0] // H
    _shape(a_log, (H,), "a_log")
    _shape(dt_bias, (H * K,), "dt_bias")
    _shape(out, (N, H, K), "out")
    _need(f_a, "f_a", torch.bfloat16)
    _need(f_b, "f_b", torch.bfloat16)
    _need(a_log, "a_log", torch.float32)
    _need(dt_bias, "dt_bias", torch.float32)
    if out is None:
        out = torch.empty((N, H, K), dtype=torch.float32, device=f_a.device)
    _need(out, "out", torch.float32)
    raw = torch.empty((N, H, K), dtype=torch.bfloat16, device=f_a.device) if with_raw else None
    st = _lib.lib().gdn_kda_gate(_ptr(f_a), _ptr(f_b), _ptr(a_log), _ptr(dt_bias), float(lower_bound), int(mode),
                                 _ptr(out), _ptr(raw), N, H, K, _stream(stream))
    _lib.check(st, "gdn_kda_gate")
    return (out, raw) if with_raw else out


def fp8_quant(x: torch.Tensor, group: int = 128, *, codes: Optional[torch.Tensor] = None,
              scales: Optional[torch.Tensor] = None, stream=None):
    """FP8 group quantisation (gdn_fp8_quant): x float32 [..., C] with C a multiple
    of ``group`` (64 or 128). Returns (codes uint8 [..., C] holding E4M3 values,
    scales float32 [..., C / group])."""
    _need(x, "x", torch.float32)
    C = x.shape[-1]
    rows = x.numel() // C if C else 0
    if codes is None:
        codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((*x.shape[:-1], C // group), dtype=torch.float32, device=x.device)
    _need(codes, "codes", torch.uint8)
    _need(scales, "scales", torch.float32)
    st = _lib.lib().gdn_fp8_quant(_ptr(x), _ptr(codes), _ptr(scales), rows, C, group, _stream(stream))
    _lib.check(st, "gdn_fp8_quant")
    return codes, scales


def recurrent_step_kda(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
                       state_pool: torch.Tensor, slots: torch.Tensor, *, scale: Optional[float] = None,
                       out_dtype: Optional[torch.dtype] = None, out: Optional[torch.Tensor] = None, stream=None):
    """One decode step with a decay per key channel (gdn_recurrent_step_kda): as
    ``recurrent_step`` but g is [N, H, K] float32 (per-channel log-decays)."""
    N, H, K = q.shape
    V = v.shape[-1]
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, q.dtype)
    for name, t in (("g", g), ("beta", beta), ("state_pool", state_pool)):
        _need(t, name, torch.float32)
    _need(slots, "slots", torch.int32)
    if k.shape != q.shape or v.shape[:2] != (N, H) or g.shape != (N, H, K) or beta.shape != (N, H):
        raise ValueError("inconsistent shapes of q, k, v, g, beta")
    if state_pool.dim() != 4 or tuple(state_pool.shape[1:]) != (H, V, K) or slots.shape != (N,):
        raise ValueError("state_pool must be [P, H, V, K] and slots [N]")
    out_dtype = out_dtype or q.dtype
    if out is None:
        out = torch.empty((N, H, V), dtype=out_dtype, device=q.device)
    _need(out, "out", out_dtype)
    st = _lib.lib().gdn_recurrent_step_kda(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_pool), state_pool.shape[0], _ptr(slots),
        _ptr(out), N, H, K, V, float(K ** -0.5 if scale is None else scale), _dt(q.dtype), _dt(out_dtype),
        _stream(stream))
    _lib.check(st, "gdn_recurrent_step_kda")
    return out


def decode_prologue(x: torch.Tensor, conv_w: torch.Tensor, conv_bias: Optional[torch.Tensor],
                    conv_state: torch.Tensor, slots: torch.Tensor, beta_raw: torch.Tensor, H: int, *,
                    stream=None):
    """Front operations of a decode layer (gdn_decode_prologue): x bf16 [N, 3 H D],
    conv_w float32 [3, 4, H D], conv_bias float32 [3 H D] or None, conv_state bf16
    [P, 3 H D, 3] (updated in place), slots int32 [N], beta_raw float32 [N, H].
    Returns (q, k, v float32 [N, H, D], beta float32 [N, H])."""
    _need(x, "x", torch.bfloat16)
    _need(conv_w, "conv_w", torch.float32)
    _need(conv_state, "conv_state", torch.bfloat16)
    _need(slots, "slots", torch.int32)
    _need(beta_raw, "beta_raw", torch.float32)
    N, C = x.shape
    if C % (3 * H):
        raise ValueError("x must be [N, 3 H D]")
    D = C // (3 * H)
    if conv_w.shape != (3, 4, H * D) or conv_state.dim() != 3 or tuple(conv_state.shape[1:]) != (C, 3):
        raise ValueError("conv_w must be [3, 4, H D] and conv_state [P, 3 H D, 3]")
    if slots.shape != (N,) or beta_raw.shape != (N, H):
        raise ValueError("slots must be [N] and beta_raw [N, H]")
    if conv_bias is not None:
        _need(conv_bias, "conv_bias", torch.float32)
        if conv_bias.shape != (C,):
            raise ValueError("conv_bias must be [3 H D]")
    q, k, v = (torch.empty((N, H, D), dtype=torch.float32, device=x.device) for _ in range(3))
    beta = torch.empty((N, H), dtype=torch.float32, device=x.device)
    st = _lib.lib().gdn_decode_prologue(
        _ptr(x), _ptr(conv_w), _ptr(conv_bias), _ptr(conv_state), conv_state.shape[0], _ptr(slots),
        _ptr(beta_raw), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), N, H, D, _stream(stream))
    _lib.check(st, "gdn_decode_prologue")
    return q, k, v, beta


def decode_prologue_verify(x: torch.Tensor, conv_w: torch.Tensor, conv_bias: Optional[torch.Tensor],
                           conv_state: torch.Tensor, slots: torch.Tensor, accepted: torch.Tensor,
                           beta_raw: torch.Tensor, H: int, T: int, *, stream=None):
    """Front operations for T tokens per request (gdn_decode_prologue_verify): x
    bf16 [N T, 3 H D]; conv_state bf16 [P, 3 H D, T + 2] (updated in place);
    slots int32 [N, C >= T]; accepted int32 [N]; beta_raw float32 [N T, H].
    Returns (q, k, v float32 [N T, H, D], beta float32 [N T, H])."""
    if x.dim() != 2 or x.shape[0] % T or x.shape[1] % (3 * H):
        raise ValueError("x must be [N T, 3 H D]")
    NT, C = x.shape
    N, D = NT // T, C // (3 * H)
    if conv_w.shape != (3, 4, H * D) or conv_state.dim() != 3 or tuple(conv_state.shape[1:]) != (C, T + 2):
        raise ValueError("conv_w must be [3, 4, H D] and conv_state [P, 3 H D, T + 2]")
    if slots.dim() != 2 or slots.shape[0] != N or accepted.shape != (N,) or beta_raw.shape != (NT, H):
        raise ValueError("slots must be [N, C], accepted [N] and beta_raw [N T, H]")
    _need(x, "x", torch.bfloat16)
    _need(conv_w, "conv_w", torch.float32)
    _need(conv_state, "conv_state", torch.bfloat16)
    _need(slots, "slots", torch.int32)
    _need(accepted, "accepted", torch.int32)
    _need(beta_raw, "beta_raw", torch.float32)
    if conv_bias is not None:
        _need(conv_bias, "conv_bias", torch.float32)
        _shape(conv_bias, (C,), "conv_bias")
    q, k, v = (torch.empty((NT, H, D), dtype=torch.float32, device=x.device) for _ in range(3))
    beta = torch.empty((NT, H), dtype=torch.float32, device=x.device)
    st = _lib.lib().gdn_decode_prologue_verify(
        _ptr(x), _ptr(conv_w), _ptr(conv_bias), _ptr(conv_state), conv_state.shape[0], _ptr(slots), slots.shape[1],
        _ptr(accepted), _ptr(beta_raw), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), N, T, H, D, _stream(stream))
    _lib.check(st, "gdn_decode_prologue_verify")
    return q, k, v, beta


def decode_layer(x: torch.Tensor, conv_w: torch.Tensor, conv_bias: Optional[torch.Tensor], conv_state: torch.Tensor,
                 slots: torch.Tensor, beta_raw: torch.Tensor, g: torch.Tensor, state_pool: torch.Tensor, H: int, *,
                 gate: Optional[torch.Tensor] = None, norm_w: Optional[torch.Tensor] = None, eps: float = 1e-6,
                 scale: Optional[float] = None, out_dtype: torch.dtype = torch.bfloat16,
                 out: Optional[torch.Tensor] = None, stream=None):
    """The decode layer in one launch (gdn_decode_layer): front operations, the
    delta-rule update (g [N, H] scalar or [N, H, D] per-channel log-decays) and,
    with norm_w, the gated RMSNorm. Returns out [N, H, D]."""
    if x.dim() != 2 or x.shape[1] % (3 * H):
        raise ValueError("x must be [N, 3 H D]")
    N, C = x.shape
    D = C // (3 * H)
    if conv_w.shape != (3, 4, H * D) or conv_state.dim() != 3 or tuple(conv_state.shape[1:]) != (C, 3):
        raise ValueError("conv_w must be [3, 4, H D] and conv_state [P, 3 H D, 3]")
    if state_pool.dim() != 4 or tuple(state_pool.shape[1:]) != (H, D, D):
        raise ValueError("state_pool must be [P, H, D, D]")
    kda = g.dim() == 3
    _shape(g, (N, H, D) if kda else (N, H), "g")
    _shape(slots, (N,), "slots")
    _shape(beta_raw, (N, H), "beta_raw")
    _shape(out, (N, H, D), "out")
    if norm_w is not None:
        _shape(norm_w, (D,), "norm_w")
        _shape(gate, (N, H * D), "gate")
    _need(x, "x", torch.bfloat16)
    _need(conv_w, "conv_w", torch.float32)
    _need(conv_state, "conv_state", torch.bfloat16)
    _need(slots, "slots", torch.int32)
    _need(beta_raw, "beta_raw", torch.float32)
    _need(g, "g", torch.float32)
    _need(state_pool, "state_pool", torch.float32)
    if conv_bias is not None:
        _need(conv_bias, "conv_bias", torch.float32)
        _shape(conv_bias, (C,), "conv_bias")
    if norm_w is not None:
        _need(norm_w, "norm_w", torch.float32)
        _need(gate, "gate", torch.bfloat16)
    if out is None:
        out = torch.empty((N, H, D), dtype=out_dtype, device=x.device)
    _need(out, "out", out_dtype)
    st = _lib.lib().gdn_decode_layer(
        _ptr(x), _ptr(conv_w), _ptr(conv_bias), _ptr(conv_state), conv_state.shape[0], _ptr(slots), _ptr(beta_raw),
        _ptr(g), int(kda), _ptr(state_pool), state_pool.shape[0], _ptr(gate), _ptr(norm_w), float(eps), _ptr(out),
        _dt(out.dtype), N, H, D, float(D ** -0.5 if scale is None else scale), _stream(stream))
    _lib.check(st, "gdn_decode_layer")
    return out


def gated_rmsnorm(o: torch.Tensor, gate: torch.Tensor, norm_w: torch.Tensor, eps: float = 1e-6, *,
                  out_dtype: torch.dtype = torch.bfloat16, out: Optional[torch.Tensor] = None, stream=None):
    """Gated RMSNorm of decode outputs (gdn_gated_rmsnorm): o float32 [N, H, D],
    gate bf16 [N, H D], norm_w float32 [D]. Returns [N, H, D] in out_dtype."""
    _need(o, "o", torch.float32)
    _need(gate, "gate", torch.bfloat16)
    _need(norm_w, "norm_w", torch.float32)
    N, H, D = o.shape
    if gate.shape != (N, H * D) or norm_w.shape != (D,):
        raise ValueError("gate must be [N, H D] and norm_w [D]")
    if out is None:
        out = torch.empty((N, H, D), dtype=out_dtype, device=o.device)
    _need(out, "out", out_dtype)
    st = _lib.lib().gdn_gated_rmsnorm(_ptr(o), _ptr(gate), _ptr(norm_w), float(eps), _ptr(out), N, H, D,
                                      _dt(out_dtype), _stream(stream))
    _lib.check(st, "gdn_gated_rmsnorm")
    return out


def chunk_fwd_kda(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor, *,
                  scale: Optional[float] = None, cu_seqlens: Optional[Sequence[int]] = None,
                  cu_seqlens_dev: Optional[torch.Tensor] = None, h0: Optional[torch.Tensor] = None,
                  output_final_state: bool = True, ht: Optional[torch.Tensor] = None,
                  state_pool: Optional[torch.Tensor] = None, state_slots: Optional[torch.Tensor] = None,
                  out_dtype: Optional[torch.dtype] = None, out: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None, stream=None, events: Optional[Sequence[int]] = None):
    """Chunked forward with a decay per key channel (gdn_chunk_fwd_kda): as
    ``chunk_fwd`` (B equal-length sequences [B, T, ...] or a packed stream with
    ``cu_seqlens``; h0 / ht or a state pool) but g is float32 [..., H, K], the
    per-token, per-channel log-decays. Returns (o, ht)."""
    return _chunk_call(q, k, v, g, beta, scale, cu_seqlens, cu_seqlens_dev, h0, output_final_state, ht, state_pool,
                       state_slots, out_dtype, out, workspace, stream, events, noalloc=False, kda=True)
