"""gdn_chunk_fwd_noalloc (through the C ABI) against gdn_chunk_fwd: two calls in a
row on one GPU, the second smaller, each bit-identical to the workspace entry
point's results (same kernels, same launches), the second also against the
oracle. The library's device array keeps the first call's contents, so the
second call also shows that stale contents do not leak into results."""

import numpy as np
import pytest
import torch

import oracle
from linear_attention_sequence_recompute_amd import _lib, api
from linear_attention_sequence_recompute_amd.workloads import chunk_inputs
from tests.gpu_util import dev, host, max_err_over_rms

pytestmark = pytest.mark.gpu


def _tensors(ci, B=None):
    dt = torch.bfloat16
    q, k, v = dev(ci.q, dt), dev(ci.k, dt), dev(ci.v, dt)
    g, b = dev(ci.a), dev(ci.beta)
    if B:
        q, k, v = (x.view(B, -1, *x.shape[1:]) for x in (q, k, v))
        g, b = (x.view(B, -1, x.shape[-1]) for x in (g, b))
    return q, k, v, g, b


def test_noalloc_two_calls_match_the_workspace_entry_point():
    assert torch.cuda.is_available()
    # call 1: B=1, H=16, T=4096, K=V=128 (the chunk workload; chunk-parallel form), dense h0/ht
    ci = chunk_inputs([4096], 16, 128, 128, dtype="bf16", seed=2, h0_std=0.1)
    assert api.workspace_bytes(1, 4096, 16, 128, 128) <= _lib.GDN_NOALLOC_WORKSPACE_BYTES
    q, k, v, g, b = _tensors(ci, B=1)
    h0 = dev(ci.h0)
    o_ref, ht_ref = api.chunk_fwd(q, k, v, g, b, scale=128 ** -0.5, h0=h0, out_dtype=torch.float32)
    o = torch.full_like(o_ref, float("nan"))
    ht = torch.full_like(ht_ref, float("nan"))
    api.chunk_fwd_noalloc(q, k, v, g, b, out=o, scale=128 ** -0.5, h0=h0, ht=ht)
    torch.cuda.synchronize()
    print("[noalloc call 1] B=1 H=16 T=4096 K=V=128", flush=True)
    assert torch.equal(o, o_ref) and torch.equal(ht, ht_ref)

    # call 2, smaller: packed sequences (one empty, ragged tails), H=4, K=V=64,
    # states in a pool with a padding slot, bf16 output
    lengths = [300, 77, 0, 129]
    ci = chunk_inputs(lengths, 4, 64, 64, dtype="bf16", seed=7, pool_slots=6, slot_ids=[2, 5, 1, 0])
    q, k, v, g, b = _tensors(ci)
    cu = ci.cu_seqlens.tolist()
    cu_dev = dev(ci.cu_seqlens, torch.int32)
    slots = dev(ci.slots, torch.int32)
    pool0 = dev(ci.pool)
    pool_ref = pool0.clone()
    o_ref, _ = api.chunk_fwd(q, k, v, g, b, scale=0.125, cu_seqlens=cu, cu_seqlens_dev=cu_dev, state_pool=pool_ref,
                             state_slots=slots, out_dtype=torch.bfloat16)
    pool = pool0.clone()
    o = torch.empty_like(o_ref)
    api.chunk_fwd_noalloc(q, k, v, g, b, out=o, scale=0.125, cu_seqlens=cu, cu_seqlens_dev=cu_dev, state_pool=pool,
                          state_slots=slots)
    torch.cuda.synchronize()
    print("[noalloc call 2] packed [300, 77, 0, 129] H=4 K=V=64 pool", flush=True)
    assert torch.equal(o, o_ref) and torch.equal(pool, pool_ref)
    # and against the oracle (bf16 output: the tolerance plus the output's own rounding)
    oh = host(o)
    for s in range(len(lengths)):
        r = slice(cu[s], cu[s + 1])
        S0 = ci.pool[ci.slots[s]] if ci.slots[s] > 0 else None
        if cu[s + 1] > cu[s]:
            o_or, S_or = oracle.chunked_fwd(ci.q[r], ci.k[r], ci.v[r], ci.a[r], ci.beta[r], scale=0.125, S0=S0)
            err = np.max(np.abs(oh[r] - o_or) - 2.0 ** -8 * np.abs(o_or)) / np.sqrt(np.mean(o_or ** 2))
            assert err <= 2e-3, f"sequence {s}: {err:.3e}"
            if ci.slots[s] > 0:
                assert max_err_over_rms(host(pool[ci.slots[s]]), S_or) <= 2e-3
    for slot in (0, 3, 4):  # padding and unused slots untouched
        assert torch.equal(pool[slot], pool0[slot])
