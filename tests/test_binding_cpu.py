"""CPU checks of the torch binding's argument validation: buffers whose shape
does not match the call are rejected with ValueError before anything reaches the
C ABI (which takes sizes, not shapes, and so could not catch them). No GPU and
no device tensors are needed: the shape checks run first."""

import pytest
import torch

from linear_attention_sequence_recompute_amd import api

B, T, H, K, V = 2, 70, 3, 64, 64


def _inputs(packed=False):
    lead = (B * T,) if packed else (B, T)
    q = torch.zeros(*lead, H, K, dtype=torch.bfloat16)
    return (q, q.clone(), torch.zeros(*lead, H, V, dtype=torch.bfloat16), torch.zeros(*lead, H),
            torch.zeros(*lead, H))


def _state(n=B):
    return torch.zeros(n, H, V, K)


@pytest.mark.parametrize("kw,msg", [
    (dict(out=torch.zeros(B, T, H, V + 1)), "out must have shape"),
    (dict(h0=_state(B + 1)), "h0 must have shape"),
    (dict(h0=torch.zeros(B, H, K, V + 16)), "h0 must have shape"),
    (dict(ht=_state(1)), "ht must have shape"),
    (dict(state_pool=torch.zeros(4, H, V, K + 64), state_slots=torch.zeros(B, dtype=torch.int32)),
     "state_pool must have shape"),
    (dict(state_pool=torch.zeros(4, H, V, K), state_slots=torch.zeros(B + 1, dtype=torch.int32)),
     "state_slots must have shape"),
    (dict(state_pool=torch.zeros(4, H, V, K)), "state_pool needs state_slots"),
    (dict(state_pool=torch.zeros(4, H, V, K), state_slots=torch.zeros(B, dtype=torch.int32), h0=_state()),
     "must be None when state_pool"),
])
def test_chunk_fwd_rejects_wrong_shapes(kw, msg):
    with pytest.raises(ValueError, match=msg):
        api.chunk_fwd(*_inputs(), **kw)


def test_chunk_fwd_packed_rejects_wrong_shapes():
    cu = [0, 30, B * T]
    with pytest.raises(ValueError, match="h0 must have shape"):
        api.chunk_fwd(*_inputs(packed=True), cu_seqlens=cu, h0=_state(3))
    with pytest.raises(ValueError, match="cu_seqlens_dev must have shape"):
        api.chunk_fwd(*_inputs(packed=True), cu_seqlens=cu, cu_seqlens_dev=torch.zeros(4, dtype=torch.int32))
    with pytest.raises(ValueError, match="out must have shape"):
        api.chunk_fwd(*_inputs(packed=True), cu_seqlens=cu, out=torch.zeros(B * T - 1, H, V))


def test_chunk_fwd_shapes_pass_to_device_checks():
    """Correct shapes on CPU tensors get past the shape checks and stop at the
    device check (the binding never hands host memory to the library)."""
    with pytest.raises(ValueError, match="must be a device tensor"):
        api.chunk_fwd(*_inputs(), h0=_state(), ht=_state())


@pytest.mark.parametrize("kw,msg", [
    (dict(out=torch.zeros(B, T, H, V - 16)), "out must have shape"),
    (dict(h0=_state(B + 1)), "h0 must have shape"),
    (dict(ht=torch.zeros(B, H, K, V + 64)), "ht must have shape"),
])
def test_chunk_fwd_kda_rejects_wrong_shapes(kw, msg):
    q, k, v, _, beta = _inputs()
    g = torch.zeros(B, T, H, K)
    with pytest.raises(ValueError, match=msg):
        api.chunk_fwd_kda(q, k, v, g, beta, **kw)
