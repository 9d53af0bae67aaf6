"""Seeded synthetic inputs for the chunked gated delta rule and its decode step.

This module draws random inputs and nothing else: it holds none of the method's
arithmetic, so the GPU path and the CPU oracle can both be fed from it without
sharing any computation.

Recipe (shapes and distributions of the workloads the WarpDrive page and the
vLLM KdaSplit page describe; neither page measures on a public dataset):

* q, k ~ N(0, 1), each per-(token, head) vector scaled to unit L2 norm, then
  rounded to the input dtype (round-to-nearest-even);
* v ~ N(0, 1), rounded to the input dtype;
* beta = sigmoid(N(0, 1)), float32;
* raw per-token log-gate a = -softplus(N(0, 1) + shift), float32, shift = 2 for the
  standard "short memory" gate (mean per-token decay about 0.16) and -4 for the
  "long memory" gate that stresses the carry across chunks;
* initial states and pools ~ N(0, 0.1^2), float32, in [.., H, V, K] layout;
* decode layer front and back (``layer_inputs``): projected inputs x, raw gates
  and conv states ~ N(0, 1) rounded to bf16; conv weights ~ U(-1/2, 1/2) (the
  usual 1/sqrt(taps) bound for 4 taps) and biases ~ U(-1/2, 1/2) in float32; raw
  beta ~ N(0, 1); norm weights 1 + N(0, 0.1^2).

All values are returned as float64 numpy arrays that are exactly representable in
the stated storage dtype, plus the storage dtype itself, so the oracle consumes
exactly the values the kernels read.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "round_to_bf16",
    "round_to_f32",
    "ChunkInputs",
    "DecodeInputs",
    "chunk_inputs",
    "varlen_lengths",
    "decode_inputs",
    "LayerInputs",
    "layer_inputs",
    "GateInputs",
    "gate_inputs",
    "LayerVerifyInputs",
    "layer_verify_inputs",
]


def round_to_f32(x: np.ndarray) -> np.ndarray:
    """Round to float32 (RNE) and return as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round to bfloat16 (round-to-nearest-even via float32) and return as float64."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = (u.astype(np.uint32) << 16).view(np.float32)
    return out.astype(np.float64)


def _round(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_to_bf16(x)
    if dtype == "f32":
        return round_to_f32(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def _unit_rows(rng: np.random.Generator, shape) -> np.ndarray:
    x = rng.standard_normal(shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _softplus(x):
    return np.logaddexp(0.0, x)


@dataclass
class ChunkInputs:
    """Inputs of one chunked forward call. Token-major packed layout.

    q, k: [Ttot, H, K]; v: [Ttot, H, V]; a, beta: [Ttot, H]; cu_seqlens: [N+1]
    (int64, host); h0: [N, H, V, K] or None; pool/slots: optional state pool
    [P, H, V, K] with per-sequence slot ids [N] (slot <= 0: zero initial state,
    final state not stored).
    """

    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    a: np.ndarray
    beta: np.ndarray
    cu_seqlens: np.ndarray
    dtype: str
    h0: np.ndarray | None = None
    pool: np.ndarray | None = None
    slots: np.ndarray | None = None
    equal_length: bool = True
    meta: dict = field(default_factory=dict)

    @property
    def n_seqs(self) -> int:
        return len(self.cu_seqlens) - 1

    @property
    def total_tokens(self) -> int:
        return int(self.cu_seqlens[-1])


def varlen_lengths(n: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """Sequence lengths uniform on [lo, hi] (inclusive), seeded."""
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi + 1, n)


def chunk_inputs(
    lengths,
    H: int,
    K: int,
    V: int,
    dtype: str = "bf16",
    seed: int = 0,
    gate_shift: float = 2.0,
    h0_std: float | None = None,
    pool_slots: int | None = None,
    slot_ids=None,
) -> ChunkInputs:
    """Draw inputs for sequences of the given lengths packed into one token stream.

    ``lengths`` may be an int list; all-equal lengths mark the call as equal-length
    (no cu_seqlens needed by the kernels). ``h0_std`` draws a dense initial state;
    ``pool_slots`` draws a state pool of that many slots (slot 0 reserved) and uses
    ``slot_ids`` (default 1..N) as the per-sequence slots.
    """
    lengths = np.asarray(lengths, dtype=np.int64)
    n = len(lengths)
    rng = np.random.default_rng(seed)
    cu = np.zeros(n + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lengths)
    T = int(cu[-1])
    q = _round(_unit_rows(rng, (T, H, K)), dtype)
    k = _round(_unit_rows(rng, (T, H, K)), dtype)
    v = _round(rng.standard_normal((T, H, V)), dtype)
    beta = round_to_f32(_sigmoid(rng.standard_normal((T, H))))
    a = round_to_f32(-_softplus(rng.standard_normal((T, H)) + gate_shift))
    h0 = None
    if h0_std is not None:
        h0 = round_to_f32(rng.normal(0.0, h0_std, (n, H, V, K)))
    pool = slots = None
    if pool_slots is not None:
        pool = round_to_f32(rng.normal(0.0, 0.1, (pool_slots, H, V, K)))
        slots = (np.arange(1, n + 1) if slot_ids is None else np.asarray(slot_ids)).astype(np.int32)
    equal = bool(n > 0 and np.all(lengths == lengths[0]))
    return ChunkInputs(q, k, v, a, beta, cu, dtype, h0=h0, pool=pool, slots=slots,
                       equal_length=equal, meta=dict(seed=seed, gate_shift=gate_shift))


@dataclass
class DecodeInputs:
    """Inputs of one decode step: q, k [N, H, K]; v [N, H, V]; a, beta [N, H];
    pool [P, H, V, K]; slots [N] (int32; <= 0 marks a padding row)."""

    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    a: np.ndarray
    beta: np.ndarray
    pool: np.ndarray
    slots: np.ndarray
    dtype: str


def decode_inputs(
    N: int,
    H: int,
    K: int,
    V: int,
    pool_slots: int,
    dtype: str = "bf16",
    seed: int = 0,
    n_padding: int = 0,
    gate_shift: float = 2.0,
) -> DecodeInputs:
    """Draw one decode step over a slot pool. Active rows get distinct slots drawn
    without replacement from 1..pool_slots-1; ``n_padding`` rows at random positions
    get slot 0 or -1."""
    rng = np.random.default_rng(seed)
    q = _round(_unit_rows(rng, (N, H, K)), dtype)
    k = _round(_unit_rows(rng, (N, H, K)), dtype)
    v = _round(rng.standard_normal((N, H, V)), dtype)
    beta = round_to_f32(_sigmoid(rng.standard_normal((N, H))))
    a = round_to_f32(-_softplus(rng.standard_normal((N, H)) + gate_shift))
    pool = round_to_f32(rng.normal(0.0, 0.1, (pool_slots, H, V, K)))
    n_active = N - n_padding
    if n_active > pool_slots - 1:
        raise ValueError("more active rows than usable pool slots")
    active = rng.choice(np.arange(1, pool_slots), n_active, replace=False)
    slots = np.zeros(N, dtype=np.int32)
    pad_pos = rng.choice(N, n_padding, replace=False) if n_padding else np.zeros(0, np.int64)
    mask = np.ones(N, bool)
    mask[pad_pos] = False
    slots[mask] = active
    slots[pad_pos] = rng.choice(np.array([0, -1]), len(pad_pos))
    return DecodeInputs(q, k, v, a, beta, pool, slots, dtype)


@dataclass
class VerifyInputs:
    q: np.ndarray          # [N, T, H, K]
    k: np.ndarray
    v: np.ndarray          # [N, T, H, V]
    a: np.ndarray          # [N, T, H]
    beta: np.ndarray
    pool: np.ndarray       # [P, H, V, K]
    slots: np.ndarray      # [N, C] int32
    accepted: np.ndarray   # [N] int32
    dtype: str


def verify_inputs(
    N: int,
    T: int,
    H: int,
    K: int,
    V: int,
    pool_slots: int,
    dtype: str = "bf16",
    seed: int = 0,
    cols: int = 0,
    n_padding: int = 0,
    n_nowrite: int = 0,
    gate_shift: float = 2.0,
) -> VerifyInputs:
    """Draw one speculative-verify decode call: N requests of T tokens, a slot
    table [N, C] (C = cols or T) whose positive entries are distinct slots drawn
    from 1..pool_slots-1, and accepted counts uniform in [1, C]. ``n_padding``
    requests get a source slot (column accepted - 1) of 0 or -1; ``n_nowrite``
    other table entries of active requests (never their source) get 0 or -1."""
    rng = np.random.default_rng(seed)
    C = cols or T
    if C < T:
        raise ValueError("the slot table needs at least T columns")
    q = _round(_unit_rows(rng, (N, T, H, K)), dtype)
    k = _round(_unit_rows(rng, (N, T, H, K)), dtype)
    v = _round(rng.standard_normal((N, T, H, V)), dtype)
    beta = round_to_f32(_sigmoid(rng.standard_normal((N, T, H))))
    a = round_to_f32(-_softplus(rng.standard_normal((N, T, H)) + gate_shift))
    pool = round_to_f32(rng.normal(0.0, 0.1, (pool_slots, H, V, K)))
    if N * C > pool_slots - 1:
        raise ValueError("more table entries than usable pool slots")
    slots = rng.choice(np.arange(1, pool_slots), N * C, replace=False).astype(np.int32).reshape(N, C)
    accepted = rng.integers(1, C + 1, N).astype(np.int32)
    pad = rng.choice(N, n_padding, replace=False) if n_padding else np.zeros(0, np.int64)
    for b in pad:
        slots[b, accepted[b] - 1] = rng.choice([0, -1])
    active = np.setdiff1d(np.arange(N), pad)
    cand = [(b, c) for b in active for c in range(C) if c != accepted[b] - 1]
    if n_nowrite:
        for i in rng.choice(len(cand), n_nowrite, replace=False):
            b, c = cand[i]
            slots[b, c] = rng.choice([0, -1])
    return VerifyInputs(q, k, v, a, beta, pool, slots, accepted, dtype)


def channel_log_decay(shape, seed, shift=2.0):
    """Per-key-channel log-decays -softplus(N(0, 1) + shift), float32 (the scalar
    gate's distribution, drawn independently for every channel)."""
    rng = np.random.default_rng(seed)
    return round_to_f32(-_softplus(rng.standard_normal(shape) + shift))


@dataclass
class LayerInputs:
    x: np.ndarray           # [N, 3 H D] bf16 values
    conv_w: np.ndarray      # [3, 4, H D] float32
    conv_bias: np.ndarray   # [3 H D] float32
    conv_state: np.ndarray  # [pool_slots, 3 H D, 3] bf16 values
    slots: np.ndarray       # [N] int32; <= 0 padding
    beta_raw: np.ndarray    # [N, H] float32
    gate: np.ndarray        # [N, H D] bf16 values
    norm_w: np.ndarray      # [D] float32
    H: int
    D: int


def layer_inputs(N: int, H: int, D: int, pool_slots: int, seed: int = 0, n_padding: int = 0) -> LayerInputs:
    """Draw one decode token per request for the layer's front and back operations.
    Slots are drawn as in ``decode_inputs``: distinct active slots in
    1..pool_slots-1, ``n_padding`` rows at random positions with slot 0 or -1."""
    rng = np.random.default_rng(seed)
    dim = H * D
    x = round_to_bf16(rng.standard_normal((N, 3 * dim)))
    conv_w = round_to_f32(rng.uniform(-0.5, 0.5, (3, 4, dim)))
    conv_bias = round_to_f32(rng.uniform(-0.5, 0.5, 3 * dim))
    conv_state = round_to_bf16(rng.standard_normal((pool_slots, 3 * dim, 3)))
    beta_raw = round_to_f32(rng.standard_normal((N, H)))
    gate = round_to_bf16(rng.standard_normal((N, dim)))
    norm_w = round_to_f32(1.0 + 0.1 * rng.standard_normal(D))
    n_active = N - n_padding
    if n_active > pool_slots - 1:
        raise ValueError("more active rows than usable pool slots")
    slots = np.zeros(N, dtype=np.int32)
    pad_pos = rng.choice(N, n_padding, replace=False) if n_padding else np.zeros(0, np.int64)
    mask = np.ones(N, bool)
    mask[pad_pos] = False
    slots[mask] = rng.choice(np.arange(1, pool_slots), n_active, replace=False)
    slots[pad_pos] = rng.choice(np.array([0, -1]), len(pad_pos))
    return LayerInputs(x, conv_w, conv_bias, conv_state, slots, beta_raw, gate, norm_w, H, D)


@dataclass
class GateInputs:
    f_a: np.ndarray      # [N, 128] bf16 values
    f_b: np.ndarray      # [H * K, 128] bf16 values
    a_log: np.ndarray    # [H] float32
    dt_bias: np.ndarray  # [H * K] float32
    lower_bound: float


def gate_inputs(N: int, H: int, K: int, seed: int = 0, lower_bound: float = -5.0) -> GateInputs:
    """Inputs of the KDA gate stage: activations f_a ~ N(0, 1) and projection
    weights F_B ~ N(0, 1 / 128) (unit-variance projections), both rounded to bf16;
    a_log ~ U(-2, 1/2) and dt_bias ~ N(0, 1) in float32."""
    rng = np.random.default_rng(seed)
    f_a = round_to_bf16(rng.standard_normal((N, 128)))
    f_b = round_to_bf16(rng.standard_normal((H * K, 128)) / np.sqrt(128.0))
    a_log = round_to_f32(rng.uniform(-2.0, 0.5, H))
    dt = round_to_f32(rng.standard_normal(H * K))
    return GateInputs(f_a, f_b, a_log, dt, float(np.float32(lower_bound)))


@dataclass
class LayerVerifyInputs:
    x: np.ndarray           # [N * T, 3 H D] bf16 values
    conv_w: np.ndarray      # [3, 4, H D] float32
    conv_bias: np.ndarray   # [3 H D] float32
    conv_state: np.ndarray  # [P, 3 H D, T + 2] bf16 values
    slots: np.ndarray       # [N, T] int32: conv page slot[b, 0], state source slot[b, accepted - 1]
    accepted: np.ndarray    # [N] int32
    beta_raw: np.ndarray    # [N * T, H] float32
    gate: np.ndarray        # [N * T, H D] bf16 values
    norm_w: np.ndarray      # [D] float32
    a: np.ndarray           # [N * T, H] float32 raw log-gates of the recurrent step
    pool: np.ndarray        # [P, H, D, D] float32 recurrent states
    H: int
    D: int
    T: int


def layer_verify_inputs(N: int, T: int, H: int, D: int, pool_slots: int, seed: int = 0,
                        n_padding: int = 0) -> LayerVerifyInputs:
    """One speculative-verify call of a decode layer: T tokens per request, the
    distributions of ``layer_inputs`` for the front and back operations and of
    ``verify_inputs`` for the recurrent step; one slot table [N, T] of distinct
    positive slots serves the conv pages (column 0) and the recurrent states;
    accepted counts uniform in [1, T]; ``n_padding`` requests get a source slot
    (column accepted - 1) of 0 or -1."""
    rng = np.random.default_rng(seed)
    dim = H * D
    x = round_to_bf16(rng.standard_normal((N * T, 3 * dim)))
    conv_w = round_to_f32(rng.uniform(-0.5, 0.5, (3, 4, dim)))
    conv_bias = round_to_f32(rng.uniform(-0.5, 0.5, 3 * dim))
    conv_state = round_to_bf16(rng.standard_normal((pool_slots, 3 * dim, T + 2)))
    beta_raw = round_to_f32(rng.standard_normal((N * T, H)))
    gate = round_to_bf16(rng.standard_normal((N * T, dim)))
    norm_w = round_to_f32(1.0 + 0.1 * rng.standard_normal(D))
    a = round_to_f32(-_softplus(rng.standard_normal((N * T, H)) + 2.0))
    pool = round_to_f32(rng.normal(0.0, 0.1, (pool_slots, H, D, D)))
    if N * T > pool_slots - 1:
        raise ValueError("more table entries than usable pool slots")
    slots = rng.choice(np.arange(1, pool_slots), N * T, replace=False).astype(np.int32).reshape(N, T)
    accepted = rng.integers(1, T + 1, N).astype(np.int32)
    for b in (rng.choice(N, n_padding, replace=False) if n_padding else []):
        if accepted[b] == 1:  # keep the conv slot (column 0) positive where it is not the source
            accepted[b] = min(2, T)
        slots[b, accepted[b] - 1] = rng.choice([0, -1])
    return LayerVerifyInputs(x, conv_w, conv_bias, conv_state, slots, accepted, beta_raw, gate, norm_w, a, pool,
                             H, D, T)
