"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Tolerances (stated per the target): float32 outputs and final states within
max|err| <= 2e-3 * RMS(reference) for bf16 inputs and <= 1e-4 * RMS(reference)
for float32 inputs; bf16 outputs equal round-to-nearest-even of the float32
output of the same call, bit for bit. Integer work (schedules, slots, padding,
untouched pool pages) is checked exactly.
"""

import os

import numpy as np
import pytest
import torch

import oracle
from linear_attention_sequence_recompute_amd import api
from linear_attention_sequence_recompute_amd.workloads import (channel_log_decay, chunk_inputs, decode_inputs,
                                                              layer_inputs, round_to_f32, varlen_lengths,
                                                              verify_inputs)
from tests.gpu_util import TORCH_DT, bf16_rne, dev, host, max_err_over_rms

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-3, "f32": 1e-4}


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    yield


def _print(*a):
    print(*a, flush=True)


# --------------------------------------------------------------------- chunk

def run_chunk(ci, scale, out_dtype, use_pool=False, pool_dev=None):
    dt = TORCH_DT[ci.dtype]
    q, k, v = dev(ci.q, dt), dev(ci.k, dt), dev(ci.v, dt)
    g, b = dev(ci.a), dev(ci.beta)
    kw = {}
    if not ci.equal_length:
        kw["cu_seqlens"] = ci.cu_seqlens.tolist()
    elif ci.n_seqs > 1:
        T = ci.total_tokens // ci.n_seqs
        q, k, v = (x.view(ci.n_seqs, T, *x.shape[1:]) for x in (q, k, v))
        g, b = (x.view(ci.n_seqs, T, -1) for x in (g, b))
    if use_pool:
        kw["state_pool"] = pool_dev
        kw["state_slots"] = dev(ci.slots, torch.int32)
    elif ci.h0 is not None:
        kw["h0"] = dev(ci.h0)
    o, ht = api.chunk_fwd(q, k, v, g, b, scale=scale, out_dtype=TORCH_DT[out_dtype], **kw)
    torch.cuda.synchronize()
    return o.reshape(ci.total_tokens, *o.shape[-2:]), ht


def oracle_chunk(ci, scale, heads=None, seqs=None):
    """Oracle outputs for the chosen heads of the chosen sequences (all by default)."""
    heads = slice(None) if heads is None else heads
    cu = ci.cu_seqlens
    seqs = range(ci.n_seqs) if seqs is None else seqs
    res = {}
    for s in seqs:
        r = slice(int(cu[s]), int(cu[s + 1]))
        if ci.h0 is not None:
            S0 = ci.h0[s][heads]
        elif ci.pool is not None and ci.slots[s] > 0:
            S0 = ci.pool[ci.slots[s]][heads]
        else:
            S0 = None
        if cu[s + 1] == cu[s]:
            res[s] = (np.zeros((0,)), S0)
            continue
        o, S = oracle.chunked_fwd(ci.q[r][:, heads], ci.k[r][:, heads], ci.v[r][:, heads], ci.a[r][:, heads],
                                  ci.beta[r][:, heads], scale=scale, S0=S0)
        res[s] = (o, S)
    return res


def check_chunk(ci, scale, heads=None, seqs=None, label=""):
    """f32 output vs oracle; bf16 output == RNE(f32 output); final states."""
    tol = TOL[ci.dtype]
    o32, ht = run_chunk(ci, scale, "f32")
    o16, ht2 = run_chunk(ci, scale, "bf16")
    assert torch.equal(o16, bf16_rne(o32)), f"{label}: bf16 output is not RNE of the f32 output"
    if ht is not None:
        assert torch.equal(ht, ht2), f"{label}: final state depends on the output dtype"
    ref = oracle_chunk(ci, scale, heads, seqs)
    o32h = host(o32)
    hsel = slice(None) if heads is None else heads
    worst_o = worst_s = 0.0
    for s, (o_ref, S_ref) in ref.items():
        r = slice(int(ci.cu_seqlens[s]), int(ci.cu_seqlens[s + 1]))
        if o_ref.size:
            e = max_err_over_rms(o32h[r][:, hsel], o_ref)
            worst_o = max(worst_o, e)
        if ht is not None:
            S_gpu = host(ht[s])[hsel]
            S_exp = np.zeros_like(S_gpu) if S_ref is None else S_ref
            e = max_err_over_rms(S_gpu, S_exp) if np.any(S_exp) else float(np.max(np.abs(S_gpu)))
            worst_s = max(worst_s, e)
    _print(f"[chunk {label}] max|do|/rms={worst_o:.3e} max|dS|/rms={worst_s:.3e} tol={tol}")
    assert worst_o <= tol, f"{label}: output error {worst_o:.3e} > {tol}"
    assert worst_s <= tol, f"{label}: state error {worst_s:.3e} > {tol}"
    return o32, ht


def test_tiny_fp32_mode():
    """B=1, H=1, T=256 (4 chunks), K=V=64, float32 inputs and outputs, h0 = 0."""
    ci = chunk_inputs([256], 1, 64, 64, dtype="f32", seed=1)
    for scale in (1.0, 0.125):
        check_chunk(ci, scale, label=f"tiny-f32 s={scale}")


@pytest.mark.parametrize("K,V", [(128, 128), (64, 64), (128, 64), (64, 128)])
@pytest.mark.parametrize("T", [293, 64, 1])
def test_ragged_small(K, V, T):
    """Several chunks plus a ragged tail; all head sizes; nonzero initial state."""
    ci = chunk_inputs([T], 3, K, V, dtype="bf16", seed=T + K + V, h0_std=0.1)
    check_chunk(ci, K ** -0.5, label=f"ragged K={K} V={V} T={T}")


@pytest.mark.parametrize("shift", [2.0, -4.0])
def test_gates(shift):
    """Short-memory (config) and long-memory gates, which stress the carry."""
    ci = chunk_inputs([640], 4, 128, 128, dtype="bf16", seed=10, gate_shift=shift, h0_std=0.1)
    check_chunk(ci, 128 ** -0.5, label=f"gate shift={shift}")


def test_fp32_mode_long_memory():
    ci = chunk_inputs([300], 2, 128, 128, dtype="f32", seed=12, gate_shift=-4.0, h0_std=0.1)
    check_chunk(ci, 0.3, label="f32 long memory")


@pytest.mark.parametrize("K,V", [(128, 64), (64, 128)])
def test_fp32_mode_mixed_head_sizes(K, V):
    """float32 inputs with K != V: several chunks, a ragged tail, long memory."""
    ci = chunk_inputs([200], 2, K, V, dtype="f32", seed=40 + K + V, gate_shift=-4.0, h0_std=0.1)
    check_chunk(ci, K ** -0.5, label=f"f32 K={K} V={V}")


@pytest.mark.parametrize("K,V", [(128, 128), (64, 64), (128, 64), (64, 128)])
def test_many_pairs_all_head_sizes(K, V):
    """80 (sequence, head) pairs: more scan workgroups than compute units (several
    rounds of workgroups), every head size, nonzero initial states."""
    ci = chunk_inputs([130] * 5, 16, K, V, dtype="bf16", seed=50 + K + V, h0_std=0.1)
    check_chunk(ci, K ** -0.5, label=f"80 pairs K={K} V={V}")


def test_odd_batch_and_heads():
    """3 sequences x 5 heads = 15 (sequence, head) pairs: the launch pads the pairs
    to a multiple of 8 (one per XCD) and the padding workgroups must do nothing."""
    ci = chunk_inputs([130] * 3, 5, 128, 128, dtype="bf16", seed=41, h0_std=0.1)
    check_chunk(ci, 128 ** -0.5, label="B=3 H=5")


def test_two_chain_workgroups_odd_pairs():
    """7 sequences x 5 heads = 35 pairs: 280 single-slice workgroups would exceed
    the 256 compute units, so the scan runs two slices per workgroup; the pairs
    are padded to 40 and the padding workgroups must do nothing."""
    ci = chunk_inputs([130] * 7, 5, 128, 128, dtype="bf16", seed=42, h0_std=0.1)
    check_chunk(ci, 128 ** -0.5, label="B=7 H=5 (two slices per workgroup)")


def test_two_chain_varlen_edges():
    """Empty, single-token, chunk-multiple and ragged sequences with 40 heads (two
    slices per scan workgroup), long-memory gates, dense h0/ht; every sequence
    and head checked."""
    lengths = [0, 1, 64, 65, 0, 130, 127, 3]
    ci = chunk_inputs(lengths, 40, 128, 128, dtype="bf16", seed=43, gate_shift=-4.0, h0_std=0.1)
    check_chunk(ci, 0.2, label="varlen edges, 40 heads")


# The chunk-parallel form (segments of chunks, their affine state maps, then all
# segments at once) runs for bf16 inputs when few (sequence, head) pairs would
# leave most compute units idle: at most 16 pairs at V = 128 and at least 16
# chunks. Long-memory gates make the segment maps far from zero.

@pytest.mark.parametrize("K,V", [(128, 128), (64, 64), (128, 64), (64, 128)])
def test_segmented_ragged_long_memory(K, V):
    """T = 1500 (23 full chunks and a ragged one), 3 heads, h0 != 0."""
    ci = chunk_inputs([1500], 3, K, V, dtype="bf16", seed=60 + K + V, gate_shift=-4.0, h0_std=0.1)
    check_chunk(ci, K ** -0.5, label=f"segmented K={K} V={V}")


def test_segmented_varlen_pool():
    """Packed sequences of very different lengths (one segment or several, an
    empty one) with states in a pool, one slot padding (<= 0)."""
    lengths = [3000, 100, 0, 1500, 1280, 37]
    ci = chunk_inputs(lengths, 2, 128, 128, dtype="bf16", seed=61, gate_shift=-4.0, pool_slots=8,
                      slot_ids=[3, 1, 7, 0, 5, 2])
    pool0 = dev(ci.pool)
    scale = 128 ** -0.5
    pool32 = pool0.clone()
    o32, _ = run_chunk(ci, scale, "f32", use_pool=True, pool_dev=pool32)
    pool16 = pool0.clone()
    o16, _ = run_chunk(ci, scale, "bf16", use_pool=True, pool_dev=pool16)
    assert torch.equal(o16, bf16_rne(o32))
    assert torch.equal(pool16, pool32)
    for s in (0, 4, 6):  # unused slots and the padding sequence's: untouched
        assert torch.equal(pool32[s], pool0[s]), f"slot {s} was written"
    ref = oracle_chunk(ci, scale)
    o_h = host(o32)
    for s in range(len(lengths)):
        r = slice(int(ci.cu_seqlens[s]), int(ci.cu_seqlens[s + 1]))
        o_ref, S_ref = ref[s]
        if o_ref.size:
            eo = max_err_over_rms(o_h[r], o_ref)
            _print(f"[segmented varlen seq {s} len {lengths[s]}] max|do|/rms={eo:.3e}")
            assert eo <= TOL["bf16"]
        if ci.slots[s] > 0:
            got = host(pool32[ci.slots[s]])
            if S_ref is None:
                S_ref = np.zeros_like(got)
            es = max_err_over_rms(got, S_ref) if np.any(S_ref) else float(np.max(np.abs(got)))
            assert es <= TOL["bf16"], f"seq {s}: state error {es:.3e}"


def test_segmented_in_place_state():
    """ht aliasing h0 in the chunk-parallel form: only the last segment writes
    the final state, after every segment's initial state was taken."""
    ci = chunk_inputs([2048, 2048], 2, 128, 128, dtype="bf16", seed=62, gate_shift=-4.0, h0_std=0.1)
    dt = torch.bfloat16
    q, k, v = (dev(x, dt).view(2, 2048, 2, -1) for x in (ci.q, ci.k, ci.v))
    g, b = dev(ci.a).view(2, 2048, 2), dev(ci.beta).view(2, 2048, 2)
    h0 = dev(ci.h0)
    o1, ht1 = api.chunk_fwd(q, k, v, g, b, scale=0.1, h0=h0, out_dtype=torch.float32)
    state = h0.clone()
    o2, _ = api.chunk_fwd(q, k, v, g, b, scale=0.1, h0=state, ht=state, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o2, o1) and torch.equal(state, ht1)
    ref = oracle_chunk(ci, 0.1)
    for s in range(2):
        assert max_err_over_rms(host(o1[s]), ref[s][0]) <= TOL["bf16"]
        assert max_err_over_rms(host(ht1[s]), ref[s][1]) <= TOL["bf16"]


# Intermediates: prep's workspace outputs and the chunk-parallel form's segment
# states and maps, read back through gdn_chunk_fwd_plan's offsets, against the
# oracle's stages, so that a regression shows in the stage that caused it.

_TILES = ((0, 0), (1, 0), (2, 0), (2, 1), (3, 0), (3, 1))


def _kappa(g, e):
    return 4 * g + e if e < 4 else 12 + 4 * g + e


def _bf16_planes(raw, shape):
    """hi + lo of bfloat16 plane pairs: raw bytes -> float64 [..., 64 lanes, 8]."""
    x = np.frombuffer(raw.tobytes(), dtype=np.uint16).reshape(*shape, 2, 64, 8)
    f = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return f[..., 0, :, :] + f[..., 1, :, :]


def _f32_planes(raw, shape):
    """float32 fragments stored as two planes (elements 0-3, then 4-7) -> [..., 64 lanes, 8]."""
    x = np.frombuffer(raw.tobytes(), dtype=np.float32).reshape(*shape, 2, 64, 4).astype(np.float64)
    return np.concatenate([x[..., 0, :, :], x[..., 1, :, :]], axis=-1)


def _tile_set(raw, n_ch, dtype):
    """A' or P of each (chunk, head) from its six A-operand tiles, [n_ch, 64, 64]."""
    planes = _bf16_planes if dtype == "bf16" else _f32_planes
    val = planes(raw[:n_ch * 12288], (n_ch, 6))
    out = np.zeros((n_ch, 64, 64))
    for t, (rt, ks) in enumerate(_TILES):
        for g in range(4):
            for e in range(8):
                out[:, 16 * rt:16 * rt + 16, 32 * ks + _kappa(g, e)] = val[:, t, 16 * g:16 * g + 16, e]
    return out


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prep_intermediates_match_oracle_stages(dtype):
    """recompute_w_u's outputs in the workspace (WarpDrive page, kernel 5):
    A' = A diag(beta) and P = s (Q K^T) * E * M as A-operand tiles (bf16 inputs:
    high + low bfloat16 planes; fp32 inputs: float32), and the gate vectors g,
    e^g, e^{g_last - g}, against the oracle's per-chunk stages; two sequences of
    300 tokens (a ragged chunk of 44 rows: its rows and columns past the end are
    zero, its gate rows repeat the last), 4 heads, every (chunk, head)."""
    B, T, H, K, V = 2, 300, 4, 128, 128
    ci = chunk_inputs([T] * B, H, K, V, dtype=dtype, seed=71, gate_shift=-2.0, h0_std=0.1)
    dt = TORCH_DT[dtype]
    q, k, v = (dev(x, dt).view(B, T, H, -1) for x in (ci.q, ci.k, ci.v))
    g, b = dev(ci.a).view(B, T, H), dev(ci.beta).view(B, T, H)
    ws = torch.zeros(api.workspace_bytes(B, B * T, H, K, V, in_dtype=dt), dtype=torch.uint8, device="cuda")
    api.chunk_fwd(q, k, v, g, b, scale=0.2, h0=dev(ci.h0), out_dtype=torch.float32, workspace=ws)
    torch.cuda.synchronize()
    (n_seg, _, _), off = api.chunk_fwd_plan(B, B * T, T, H, K, V, in_dtype=dt)
    raw = ws.cpu().numpy()
    ncs = (T + 63) // 64
    n_ch = B * ncs * H
    ap = _tile_set(raw[off["af"]:], n_ch, dtype)
    pp = _tile_set(raw[off["pf"]:], n_ch, dtype)
    gx = np.frombuffer(raw[off["gx"]:off["gx"] + n_ch * 768].tobytes(), dtype=np.float32).reshape(n_ch, 3, 64)
    worst = {"A'": 0.0, "P": 0.0, "g": 0.0, "e^g": 0.0, "e^{gL-g}": 0.0}
    for s in range(B):
        r = slice(s * T, (s + 1) * T)
        _, _, stages = oracle.chunked_fwd(ci.q[r], ci.k[r], ci.v[r], ci.a[r], ci.beta[r], scale=0.2,
                                          S0=ci.h0[s], return_stages=True)
        for j, st in enumerate(stages):
            n = st["g"].shape[1]
            bta = ci.beta[r][64 * j:64 * j + n].T  # [H, n]
            for h in range(H):
                ch = (s * ncs + j) * H + h
                a_ref = st["A"][h] * bta[h][None, :]
                p_ref = st["P"][h]
                for name, got, ref in (("A'", ap[ch], a_ref), ("P", pp[ch], p_ref)):
                    full = np.zeros((64, 64))
                    full[:n, :n] = ref
                    worst[name] = max(worst[name], float(np.max(np.abs(got - full)) / np.max(np.abs(ref))))
                gv = st["g"][h]
                g_full = np.concatenate([gv, np.full(64 - n, gv[-1])])
                worst["g"] = max(worst["g"], float(np.max(np.abs(gx[ch, 0] - g_full) / (1 + np.abs(g_full)))))
                for name, row, ref in (("e^g", 1, np.exp(g_full)), ("e^{gL-g}", 2, np.exp(g_full[-1] - g_full))):
                    worst[name] = max(worst[name], float(np.max(np.abs(gx[ch, row] - ref) / ref)))
    _print(f"[prep intermediates {dtype}] " + " ".join(f"{k} {v:.2e}" for k, v in worst.items()),
           f"(plan {n_seg} segments)")
    assert worst["A'"] <= 2e-4 and worst["P"] <= 2e-4, worst
    # g: 64 float32 additions (|error| <= 64 * 2^-24 |g|); the exponentials add that
    # absolute error of their argument as relative error
    assert worst["g"] <= 1e-5 and worst["e^g"] <= 1e-4 and worst["e^{gL-g}"] <= 1e-4, worst


def test_segment_states_and_maps_match_oracle():
    """The chunk-parallel form's intermediates in the workspace: segment 0's final
    state, and for each segment j = 1 .. n - 2 its affine map h -> M_j h + c_j:
    c_j is the segment's final state from zero, M_j its final state from the
    identity with V = 0 (the map's linear part), both from the oracle run on the
    segment's chunks. B = 1, T = 1600 (25 chunks), H = 4: six segments of
    4 + 5 x 4 + 1 chunks, four maps; long-memory gates."""
    B, T, H, K, V = 1, 1600, 4, 128, 128
    (n_seg, L0, L1), off = api.chunk_fwd_plan(B, T, T, H, K, V)
    assert n_seg >= 3, "this shape is meant to take the chunk-parallel form"
    ci = chunk_inputs([T], H, K, V, dtype="bf16", seed=72, gate_shift=-4.0, h0_std=0.1)
    dt = torch.bfloat16
    q, k, v = (dev(x, dt).view(B, T, H, -1) for x in (ci.q, ci.k, ci.v))
    g, b = dev(ci.a).view(B, T, H), dev(ci.beta).view(B, T, H)
    ws = torch.zeros(api.workspace_bytes(B, T, H, K, V), dtype=torch.uint8, device="cuda")
    api.chunk_fwd(q, k, v, g, b, scale=K ** -0.5, h0=dev(ci.h0), out_dtype=torch.float32, workspace=ws)
    torch.cuda.synchronize()
    raw = ws.cpu().numpy()
    page = (V + K) * K * 4
    st0 = np.frombuffer(raw[off["seg_state"]:off["seg_state"] + H * V * K * 4].tobytes(), dtype=np.float32)
    st0 = st0.reshape(H, V, K)

    def oracle_state(c0, c1, S0, zero_v=False):
        r = slice(64 * c0, 64 * c1)
        vv = np.zeros_like(ci.v[r]) if zero_v else ci.v[r]
        _, S = oracle.chunked_fwd(ci.q[r], ci.k[r], vv, ci.a[r], ci.beta[r], scale=K ** -0.5, S0=S0)
        return S  # [H, V, K]

    e0 = max_err_over_rms(st0, oracle_state(0, L0, ci.h0[0]))
    worst_c = worst_m = worst_mt = 0.0
    eye = np.broadcast_to(np.eye(K), (H, V, K)).copy()
    nkb = K // 32
    for j in range(1, n_seg - 1):
        c0, c1 = L0 + (j - 1) * L1, L0 + j * L1
        c_ref = oracle_state(c0, c1, None)
        m_ref = oracle_state(c0, c1, eye, zero_v=True).transpose(0, 2, 1)  # M_j = (final state)^T
        for h in range(H):
            base = off["seg_sum"] + (h * (n_seg - 2) + j - 1) * page
            c_got = np.frombuffer(raw[base:base + V * K * 4].tobytes(), dtype=np.float32).reshape(V, K)
            worst_c = max(worst_c, max_err_over_rms(c_got, c_ref[h]))
            frag = _bf16_planes(raw[base + V * K * 4:base + page], (nkb, 2 * nkb))  # [kb, t, lane, e]
            m_got = np.zeros((K, K))
            for kb in range(nkb):
                for t in range(2 * nkb):
                    for lane in range(64):
                        gg, c = lane >> 4, lane & 15
                        row = 32 * (t // 2) + 8 * (c // 4) + 4 * (t % 2) + c % 4
                        m_got[row, 32 * kb + 8 * gg:32 * kb + 8 * gg + 8] = frag[kb, t, lane]
            worst_m = max(worst_m, max_err_over_rms(m_got, m_ref[h]))
            worst_mt = max(worst_mt, max_err_over_rms(m_got, m_ref[h].T))  # printed: tells a transposed map
    _print(f"[segment intermediates: {n_seg} segments of {L0} + {L1} x {n_seg - 2} + rest] "
           f"state 0 {e0:.3e} c {worst_c:.3e} M {worst_m:.3e} (against M^T {worst_mt:.3e})")
    tol = TOL["bf16"]
    assert e0 <= tol and worst_c <= tol and worst_m <= tol


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shift", [4.0, 8.0])
def test_fast_gates_ragged_chunks(dtype, shift):
    """Gates that forget within a few tokens (mean log-gate about -4 and -8) with
    sequence lengths that end mid-chunk (498 = 7 x 64 + 50, and 50): the final
    state is then made almost entirely of the last rows' writes, scaled by
    e^{g_last - g}, which is exactly 1 at the last row, so the chunk's g_last and
    the sums of the rows past its end must equal the last row's sum exactly."""
    for lengths in ([498, 498], [50]):
        ci = chunk_inputs(lengths, 3, 128, 128, dtype=dtype, seed=7000, h0_std=0.1, gate_shift=shift)
        check_chunk(ci, 128 ** -0.5, label=f"fast gates {dtype} shift={shift} lengths={lengths}")


@pytest.mark.parametrize("B,T,H", [(1, 32768, 1), (1, 16384, 2)])
def test_chunk_parallel_at_the_segment_limit(B, T, H):
    """Very long sequences with few pairs take the most segments the form allows
    (eight: segment 0, six maps, the last segment folding all six), each of
    tens of chunks; long-memory gates, so that the state the folds carry
    matters to the end; outputs and final states in full against the oracle."""
    (n_seg, L0, L1), _ = api.chunk_fwd_plan(B, B * T, T, H, 128, 128)
    assert n_seg == 8, (n_seg, L0, L1)
    ci = chunk_inputs([T] * B, H, 128, 128, dtype="bf16", seed=7700 + T + H, h0_std=0.1, gate_shift=-4.0)
    check_chunk(ci, 128 ** -0.5, label=f"B={B} T={T} H={H}, {n_seg} segments of {L0} + {L1} x {n_seg - 2} + rest")


def _random_chunk_case(seed):
    """Sizes of one seeded random chunk-path case: 1-4 sequences of equal or mixed
    lengths (empty and one-token sequences among them), 1-5 heads, every head-size
    pair, bf16 or fp32, with or without an initial state, three gate regimes."""
    rng = np.random.default_rng(5000 + seed)
    n = int(rng.integers(1, 5))
    K, V = [(128, 128), (64, 64), (128, 64), (64, 128)][int(rng.integers(4))]
    H = int(rng.integers(1, 6))
    dtype = "bf16" if rng.random() < 0.75 else "f32"
    if rng.random() < 0.3:
        lengths = [int(rng.integers(1, 1400))] * n
    else:
        lengths = [int(x) for x in rng.integers(0, 1700, n)]
        if n > 1 and rng.random() < 0.3:
            lengths[int(rng.integers(n))] = int(rng.choice([0, 1, 64, 65]))
    h0 = 0.1 if rng.random() < 0.5 else None
    shift = float(rng.choice([2.0, -2.0, -4.0]))
    return lengths, H, K, V, dtype, h0, shift


def test_chunk_random_shapes():
    """Sixteen seeded random cases of the chunk path against the oracle (every
    (sequence, head) pair, outputs and final states), so that shapes no fixed test
    names are covered too; the cases that have few pairs and long sequences take
    the chunk-parallel form, and at least some do."""
    took_segments = 0
    for seed in range(16):
        lengths, H, K, V, dtype, h0, shift = _random_chunk_case(seed)
        ci = chunk_inputs(lengths, H, K, V, dtype=dtype, seed=7000 + seed, h0_std=h0, gate_shift=shift)
        (n_seg, _, _), _ = api.chunk_fwd_plan(len(lengths), sum(lengths), max(lengths), H, K, V,
                                              in_dtype=TORCH_DT[dtype])
        took_segments += n_seg > 1
        label = f"random {seed}: lengths {lengths} H={H} K={K} V={V} {dtype} h0={h0 is not None} " \
                f"shift={shift} segments={n_seg}"
        _print(label)
        check_chunk(ci, K ** -0.5, label=label)
    assert took_segments >= 2, "the sweep should reach the chunk-parallel form"


def test_config_h16_t4096_full():
    """B=1, H=16, T=4096, K=V=128, bf16: every output and the final state."""
    ci = chunk_inputs([4096], 16, 128, 128, dtype="bf16", seed=2)
    check_chunk(ci, 128 ** -0.5, label="H16 T4096")


def test_config_batched_long_full():
    """B=4, H=32, T=8192, K=V=128, bf16, h0 ~ N(0, 0.1^2): the launch the long
    configuration times; every (sequence, head) pair, every output and every
    final state against the oracle."""
    ci = chunk_inputs([8192] * 4, 32, 128, 128, dtype="bf16", seed=3, h0_std=0.1)
    check_chunk(ci, 128 ** -0.5, label="B4 H32 T8192")


def test_varlen_pool_full():
    """16 packed sequences, lengths uniform in [100, 6000] (not chunk-aligned),
    initial states read from and final states written back to a state pool;
    every (sequence, head) pair checked."""
    lengths = varlen_lengths(16, 100, 6000, seed=4)
    ci = chunk_inputs(lengths, 16, 128, 128, dtype="bf16", seed=4, pool_slots=17)
    pool0 = dev(ci.pool)
    scale = 128 ** -0.5
    pool32 = pool0.clone()
    o32, _ = run_chunk(ci, scale, "f32", use_pool=True, pool_dev=pool32)
    pool16 = pool0.clone()
    o16, _ = run_chunk(ci, scale, "bf16", use_pool=True, pool_dev=pool16)
    assert torch.equal(o16, bf16_rne(o32))
    assert torch.equal(pool16, pool32)
    # slot 0 is reserved and untouched
    assert torch.equal(pool32[0], pool0[0])
    ref = oracle_chunk(ci, scale)
    o_h = host(o32)
    worst_o = worst_s = 0.0
    for s in range(len(lengths)):
        r = slice(int(ci.cu_seqlens[s]), int(ci.cu_seqlens[s + 1]))
        o_ref, S_ref = ref[s]
        worst_o = max(worst_o, max_err_over_rms(o_h[r], o_ref))
        worst_s = max(worst_s, max_err_over_rms(host(pool32[ci.slots[s]]), S_ref))
    _print(f"[varlen 16 seqs, all pairs] max|do|/rms={worst_o:.3e} max|dS|/rms={worst_s:.3e}")
    assert worst_o <= TOL["bf16"] and worst_s <= TOL["bf16"]


def test_varlen_edge_lengths_dense_states():
    """Empty sequences, single tokens, exact chunk multiples and ragged tails in
    one packed call, with dense h0/ht; every sequence checked."""
    lengths = [0, 1, 64, 65, 0, 130, 127, 3]
    ci = chunk_inputs(lengths, 3, 128, 128, dtype="bf16", seed=21, h0_std=0.1)
    check_chunk(ci, 0.2, label="varlen edges")


def test_many_short_sequences():
    """700 packed sequences of 0-90 tokens (the chunk schedule walks the sequences
    256 at a time, carrying the chunk count across its passes), 2 heads, dense
    h0/ht; every sequence checked."""
    lengths = [int(x) for x in np.random.default_rng(23).integers(0, 91, 700)]
    ci = chunk_inputs(lengths, 2, 64, 64, dtype="bf16", seed=24, h0_std=0.1)
    check_chunk(ci, 0.2, label="700 short sequences")


def test_pool_padding_slots():
    """Sequences whose slot is <= 0 start from zero and write nothing back."""
    lengths = [100, 70, 200]
    ci = chunk_inputs(lengths, 2, 64, 64, dtype="bf16", seed=22, pool_slots=6, slot_ids=[3, 0, -1])
    pool0 = dev(ci.pool)
    pool = pool0.clone()
    o, _ = run_chunk(ci, 0.5, "f32", use_pool=True, pool_dev=pool)
    for s in range(6):
        if s != 3:
            assert torch.equal(pool[s], pool0[s]), f"slot {s} was written"
    ref = oracle_chunk(ci, 0.5)
    o_h = host(o)
    for s in range(3):
        r = slice(int(ci.cu_seqlens[s]), int(ci.cu_seqlens[s + 1]))
        assert max_err_over_rms(o_h[r], ref[s][0]) <= TOL["bf16"]
    assert max_err_over_rms(host(pool[3]), ref[0][1]) <= TOL["bf16"]


def test_in_place_state_alias_and_determinism():
    ci = chunk_inputs([200, 200], 2, 128, 128, dtype="bf16", seed=23, h0_std=0.1)
    dt = torch.bfloat16
    q, k, v = (dev(x, dt).view(2, 200, 2, -1) for x in (ci.q, ci.k, ci.v))
    g, b = dev(ci.a).view(2, 200, 2), dev(ci.beta).view(2, 200, 2)
    h0 = dev(ci.h0)
    o1, ht1 = api.chunk_fwd(q, k, v, g, b, scale=0.1, h0=h0, out_dtype=torch.float32)
    o2, ht2 = api.chunk_fwd(q, k, v, g, b, scale=0.1, h0=h0, out_dtype=torch.float32)
    assert torch.equal(o1, o2) and torch.equal(ht1, ht2)
    state = h0.clone()
    o3, _ = api.chunk_fwd(q, k, v, g, b, scale=0.1, h0=state, ht=state, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o3, o1) and torch.equal(state, ht1)


def test_decode_steps_match_chunked_prefill_on_gpu():
    """T decode steps on one slot and one chunked call over the same tokens agree
    (both against each other and the oracle)."""
    T, H, K, V = 70, 2, 128, 128
    ci = chunk_inputs([T], H, K, V, dtype="bf16", seed=24, h0_std=0.1)
    o_c, ht = run_chunk(ci, 0.25, "f32")
    pool = torch.zeros(3, H, V, K, device="cuda")
    pool[1] = dev(ci.h0[0])
    slots = torch.tensor([1], dtype=torch.int32, device="cuda")
    outs = []
    for t in range(T):
        sl = slice(t, t + 1)
        outs.append(api.recurrent_step(dev(ci.q[sl], torch.bfloat16), dev(ci.k[sl], torch.bfloat16),
                                       dev(ci.v[sl], torch.bfloat16), dev(ci.a[sl]), dev(ci.beta[sl]), pool,
                                       slots, scale=0.25, out_dtype=torch.float32))
    o_d = torch.cat(outs)
    torch.cuda.synchronize()
    assert max_err_over_rms(host(o_d), host(o_c)) <= TOL["bf16"]
    assert max_err_over_rms(host(pool[1]), host(ht[0])) <= TOL["bf16"]


# -------------------------------------------------------------------- decode

def run_decode(di, scale, out_dtype, pool_dev):
    dt = TORCH_DT[di.dtype]
    o = api.recurrent_step(dev(di.q, dt), dev(di.k, dt), dev(di.v, dt), dev(di.a), dev(di.beta), pool_dev,
                           dev(di.slots, torch.int32), scale=scale, out_dtype=TORCH_DT[out_dtype])
    torch.cuda.synchronize()
    return o


def check_decode(di, scale, label):
    tol = TOL[di.dtype]
    pool0 = dev(di.pool)
    p32 = pool0.clone()
    o32 = run_decode(di, scale, "f32", p32)
    p16 = pool0.clone()
    o16 = run_decode(di, scale, "bf16", p16)
    assert torch.equal(o16, bf16_rne(o32)), f"{label}: bf16 output is not RNE of the f32 output"
    assert torch.equal(p16, p32)
    o_ref, pool_ref = oracle.decode_step(di.q, di.k, di.v, di.a, di.beta, di.pool, di.slots, scale=scale)
    pad = di.slots <= 0
    o_h = host(o32)
    assert np.all(o_h[pad] == 0) and not np.any(np.signbit(o_h[pad])), f"{label}: padding rows not +0"
    active = di.slots[~pad]
    eo = max_err_over_rms(o_h[~pad], o_ref[~pad])
    es = max_err_over_rms(host(p32[active.tolist()]), pool_ref[active])
    untouched = np.setdiff1d(np.arange(di.pool.shape[0]), active)
    assert torch.equal(p32[untouched.tolist()], pool0[untouched.tolist()]), f"{label}: untouched slots changed"
    _print(f"[decode {label}] max|do|/rms={eo:.3e} max|dS|/rms={es:.3e} tol={tol}")
    assert eo <= tol and es <= tol


@pytest.mark.parametrize("K,V", [(128, 128), (64, 64), (128, 64), (64, 128)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_small(K, V, dtype):
    di = decode_inputs(N=40, H=3, K=K, V=V, pool_slots=64, dtype=dtype, seed=K + V, n_padding=6)
    check_decode(di, K ** -0.5, f"K={K} V={V} {dtype}")


def test_decode_config_full():
    """N=256 requests, H=32, K=V=128, pool of 512 slots (1 GiB), 32 padding rows."""
    di = decode_inputs(N=256, H=32, K=128, V=128, pool_slots=512, dtype="bf16", seed=5, n_padding=32)
    check_decode(di, 128 ** -0.5, "N256 H32 pool512")


def test_decode_out_of_range_slot_is_padding():
    di = decode_inputs(N=8, H=2, K=64, V=64, pool_slots=16, dtype="bf16", seed=31)
    di.slots[3] = 16  # == pool_slots: out of range
    di.slots[5] = 10 ** 6
    pool0 = dev(di.pool)
    pool = pool0.clone()
    o = run_decode(di, 0.5, "f32", pool)
    assert torch.all(o[3] == 0) and torch.all(o[5] == 0)
    keep = [s for s in range(16) if s not in set(di.slots[[0, 1, 2, 4, 6, 7]].tolist())]
    assert torch.equal(pool[keep], pool0[keep])


def test_decode_random_shapes():
    """Twelve seeded random decode steps against the oracle (scalar gates; with
    per-channel decays for every other case): 1-300 requests with some padding
    rows, 1-6 heads, every head-size pair, bf16 and fp32, pools a little or much
    larger than the batch, gates from long memory to forgetting within a token."""
    for seed in range(12):
        rng = np.random.default_rng(9000 + seed)
        N = int(rng.integers(1, 301))
        H = int(rng.integers(1, 7))
        K, V = [(128, 128), (64, 64), (128, 64), (64, 128)][int(rng.integers(4))]
        dtype = "bf16" if rng.random() < 0.7 else "f32"
        n_pad = int(rng.integers(0, N // 4 + 1))
        pool = N - n_pad + 1 + int(rng.integers(0, 2 * N + 2))
        shift = float(rng.choice([-4.0, 2.0, 8.0]))
        di = decode_inputs(N=N, H=H, K=K, V=V, pool_slots=pool, dtype=dtype, seed=9100 + seed, n_padding=n_pad,
                           gate_shift=shift)
        label = f"random {seed}: N={N} H={H} K={K} V={V} {dtype} pad={n_pad} pool={pool} shift={shift}"
        check_decode(di, K ** -0.5, label)
        if seed % 2:
            g = channel_log_decay((N, H, K), 9200 + seed, shift)
            check_decode_kda(di, g, K ** -0.5, label)


# --------------------------------------------- per-key-channel decay (KDA)

def check_decode_kda(di, g, scale, label):
    tol = TOL[di.dtype]
    dt = TORCH_DT[di.dtype]
    pool0 = dev(di.pool)
    outs = {}
    for od in ("f32", "bf16"):
        pool = pool0.clone()
        o = api.recurrent_step_kda(dev(di.q, dt), dev(di.k, dt), dev(di.v, dt), dev(g), dev(di.beta), pool,
                                   dev(di.slots, torch.int32), scale=scale, out_dtype=TORCH_DT[od])
        torch.cuda.synchronize()
        outs[od] = (o, pool)
    (o32, p32), (o16, p16) = outs["f32"], outs["bf16"]
    assert torch.equal(o16, bf16_rne(o32)) and torch.equal(p16, p32)
    o_ref, pool_ref = oracle.decode_step_kda(di.q, di.k, di.v, g, di.beta, di.pool, di.slots, scale=scale)
    act = [b for b in range(len(di.slots)) if di.slots[b] > 0]
    pad = [b for b in range(len(di.slots)) if di.slots[b] <= 0]
    eo = max_err_over_rms(host(o32)[act], o_ref[act])
    used = {int(di.slots[b]) for b in act}
    es = max(max_err_over_rms(host(p32[s]), pool_ref[s]) for s in used)
    for b in pad:
        assert bool((o32[b].view(torch.int32) == 0).all()), f"{label}: padding row {b} output is not +0"
    for s in range(di.pool.shape[0]):
        if s not in used:
            assert torch.equal(p32[s], pool0[s]), f"{label}: slot {s} was written"
    _print(f"[decode kda {label}] max|do|/rms={eo:.3e} max|dS|/rms={es:.3e} tol={tol}")
    assert eo <= tol and es <= tol


@pytest.mark.parametrize("K,V", [(128, 128), (64, 64), (128, 64), (64, 128)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_kda_small(K, V, dtype):
    di = decode_inputs(N=24, H=3, K=K, V=V, pool_slots=40, dtype=dtype, seed=80 + K + V, n_padding=4)
    g = channel_log_decay((24, 3, K), seed=81 + K, shift=-2.0)
    check_decode_kda(di, g, K ** -0.5, f"K={K} V={V} {dtype}")


def test_decode_kda_config_full():
    """N=256 requests, H=32, K=V=128, 512-slot pool, 32 padding rows."""
    di = decode_inputs(N=256, H=32, K=128, V=128, pool_slots=512, dtype="bf16", seed=5, n_padding=32)
    g = channel_log_decay((256, 32, 128), seed=82)
    check_decode_kda(di, g, 128 ** -0.5, "N256 H32")


def test_decode_kda_uniform_channels_equal_the_scalar_step():
    """A decay vector with every channel equal to the scalar gate gives the scalar
    kernel's results bit for bit (the same multiply per state element)."""
    di = decode_inputs(N=40, H=4, K=128, V=128, pool_slots=64, dtype="bf16", seed=83, n_padding=5)
    g = np.repeat(di.a[:, :, None], 128, axis=2).astype(np.float32)
    dt = torch.bfloat16
    p1, p2 = dev(di.pool), dev(di.pool)
    o1 = api.recurrent_step(dev(di.q, dt), dev(di.k, dt), dev(di.v, dt), dev(di.a), dev(di.beta), p1,
                            dev(di.slots, torch.int32), out_dtype=torch.float32)
    o2 = api.recurrent_step_kda(dev(di.q, dt), dev(di.k, dt), dev(di.v, dt), dev(g), dev(di.beta), p2,
                                dev(di.slots, torch.int32), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(p1, p2)


# ----------------------------------------------------- speculative verify

def run_verify(vi, scale, out_dtype, pool_dev):
    dt = TORCH_DT[vi.dtype]
    o = api.recurrent_verify(dev(vi.q, dt), dev(vi.k, dt), dev(vi.v, dt), dev(vi.a), dev(vi.beta), pool_dev,
                             dev(vi.slots, torch.int32), dev(vi.accepted, torch.int32), scale=scale,
                             out_dtype=TORCH_DT[out_dtype])
    torch.cuda.synchronize()
    return o


def check_verify(vi, scale, label):
    """f32 outputs and written states vs the oracle; padding requests +0; slots
    not written bit-identical; bf16 outputs == RNE(f32 outputs)."""
    tol = TOL[vi.dtype]
    pool0 = dev(vi.pool)
    p32 = pool0.clone()
    o32 = run_verify(vi, scale, "f32", p32)
    p16 = pool0.clone()
    o16 = run_verify(vi, scale, "bf16", p16)
    assert torch.equal(o16, bf16_rne(o32)), f"{label}: bf16 output is not RNE of the f32 output"
    assert torch.equal(p16, p32), f"{label}: written states depend on the output dtype"
    o_ref, pool_ref = oracle.decode_verify(vi.q, vi.k, vi.v, vi.a, vi.beta, vi.pool, vi.slots, vi.accepted,
                                           scale=scale)
    N, T = vi.q.shape[:2]
    cols = vi.slots.shape[1]
    o_h = host(o32)
    active, written = [], set()
    for b in range(N):
        acc = int(vi.accepted[b])
        src = int(vi.slots[b, acc - 1]) if 1 <= acc <= cols else 0
        if src <= 0:
            assert bool((o32[b].view(torch.int32) == 0).all()), f"{label}: padding request {b} output is not +0"
            continue
        active.append(b)
        written.update(int(x) for x in vi.slots[b, :T] if x > 0)
    eo = max_err_over_rms(o_h[active], o_ref[active])
    pool_h = host(p32)
    es = max(max_err_over_rms(pool_h[s], pool_ref[s]) for s in written) if written else 0.0
    for s in range(vi.pool.shape[0]):
        if s not in written:
            assert torch.equal(p32[s], pool0[s]), f"{label}: slot {s} was written"
    _print(f"[verify {label}] max|do|/rms={eo:.3e} max|dS|/rms={es:.3e} tol={tol}")
    assert eo <= tol and es <= tol


@pytest.mark.parametrize("K,V", [(128, 128), (64, 64), (128, 64), (64, 128)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("T", [1, 3, 8])
def test_verify_small(K, V, dtype, T):
    """Speculative verify: 6 requests (one padding), T tokens each, a slot table
    wider than T with some non-positive entries (not written), long-memory gates."""
    vi = verify_inputs(N=6, T=T, H=2, K=K, V=V, pool_slots=64, dtype=dtype, seed=70 + T + K + V, cols=T + 2,
                       n_padding=1, n_nowrite=2, gate_shift=-4.0)
    check_verify(vi, K ** -0.5, f"K={K} V={V} {dtype} T={T}")


def test_verify_random_shapes():
    """Ten seeded random speculative-verify calls against the oracle: 1-40
    requests of 1-8 tokens, slot tables up to three columns wider than T with
    padding requests and entries that are not written, 1-4 heads, every
    head-size pair, bf16 and fp32, three gate regimes."""
    for seed in range(10):
        rng = np.random.default_rng(9300 + seed)
        N = int(rng.integers(1, 41))
        T = int(rng.integers(1, 9))
        C = T + int(rng.integers(0, 4))
        H = int(rng.integers(1, 5))
        K, V = [(128, 128), (64, 64), (128, 64), (64, 128)][int(rng.integers(4))]
        dtype = "bf16" if rng.random() < 0.7 else "f32"
        n_pad = int(rng.integers(0, N // 3 + 1))
        n_nowrite = int(rng.integers(0, 4)) if (N - n_pad) * (C - 1) >= 3 else 0
        shift = float(rng.choice([-4.0, 2.0, 8.0]))
        vi = verify_inputs(N=N, T=T, H=H, K=K, V=V, pool_slots=N * C + 1 + int(rng.integers(0, 20)), dtype=dtype,
                           seed=9400 + seed, cols=C, n_padding=n_pad, n_nowrite=n_nowrite, gate_shift=shift)
        check_verify(vi, K ** -0.5, f"random {seed}: N={N} T={T} C={C} H={H} K={K} V={V} {dtype} pad={n_pad} "
                                    f"nowrite={n_nowrite} shift={shift}")


def test_verify_config_full():
    """96 requests x 4 tokens, H=32, K=V=128, 512-slot pool (the timed shape), 8
    padding requests and 16 unwritten table entries; every output and state."""
    vi = verify_inputs(N=96, T=4, H=32, K=128, V=128, pool_slots=512, dtype="bf16", seed=7, n_padding=8,
                       n_nowrite=16)
    check_verify(vi, 128 ** -0.5, "N96 T4 H32")


# ------------------------------------------------------- fp8 quantisation

def _fp8_input(rows, cols, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((rows, cols)) * np.exp2(rng.integers(-20, 20, (rows, 1)))).astype(np.float32)
    x[::7, : cols // 2] = 0.0                       # all-zero groups
    x[1::5, 3] = -0.0                               # negative zeros
    x[rows // 2, 5] = np.float32(1e-40)             # a float32 subnormal
    return x


@pytest.mark.parametrize("group", [64, 128])
@pytest.mark.parametrize("rows,cols", [(1, 128), (37, 384), (300, 1024)])
def test_fp8_quant_bit_exact(group, rows, cols):
    """Codes and scales equal the oracle's bit for bit (several workgroups and a
    ragged last one, zero groups, signed zeros, subnormal inputs)."""
    x = _fp8_input(rows, cols, seed=rows + cols + group)
    codes, scales = api.fp8_quant(dev(x), group)
    torch.cuda.synchronize()
    c_ref, s_ref = oracle.fp8_quant(x, group)
    np.testing.assert_array_equal(codes.cpu().numpy(), c_ref)
    np.testing.assert_array_equal(scales.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))


def test_fp8_quant_every_code_and_tie():
    """Groups whose absmax is 448 have scale 1, so the quotients are the inputs:
    every finite E4M3 value and every midpoint between neighbours (ties, which
    round to the even code) goes through the conversion and must give the
    oracle's code."""
    finite = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    vals = np.sort(oracle.e4m3_decode(finite)).astype(np.float64)
    mids = (vals[:-1] + vals[1:]) / 2
    body = np.concatenate([vals, mids]).astype(np.float32)
    groups = -(-len(body) // 127)
    x = np.zeros((groups, 128), np.float32)
    x[:, 0] = 448.0
    x[:, 1:].flat[:len(body)] = body
    codes, scales = api.fp8_quant(dev(x.reshape(1, -1)), 128)
    torch.cuda.synchronize()
    c_ref, s_ref = oracle.fp8_quant(x.reshape(1, -1), 128)
    assert np.all(s_ref == 1.0)
    np.testing.assert_array_equal(codes.cpu().numpy(), c_ref)


def test_fp8_quant_config_sampled():
    """The timed shape, [16384, 4096] float32 with groups of 128: 512 sampled rows
    bit-exact against the oracle."""
    rows, cols = 16384, 4096
    xd = torch.randn(rows, cols, device="cuda") * torch.exp2(torch.randint(-8, 8, (rows, 1), device="cuda").float())
    codes, scales = api.fp8_quant(xd, 128)
    torch.cuda.synchronize()
    pick = np.random.default_rng(5).choice(rows, 512, replace=False)
    x = xd[torch.from_numpy(pick).cuda()].cpu().numpy()
    c_ref, s_ref = oracle.fp8_quant(x, 128)
    np.testing.assert_array_equal(codes[torch.from_numpy(pick).cuda()].cpu().numpy(), c_ref)
    np.testing.assert_array_equal(scales[torch.from_numpy(pick).cuda()].cpu().numpy().view(np.uint32),
                                  s_ref.view(np.uint32))


# ------------------------------------- chunk form with a decay per key channel

def run_chunk_kda(ci, g, B, T, scale, out_dtype, h0=None, ht=None):
    dt = TORCH_DT[ci.dtype]
    H, K = ci.q.shape[1:]
    V = ci.v.shape[-1]
    q, k = dev(ci.q, dt).view(B, T, H, K), dev(ci.k, dt).view(B, T, H, K)
    v = dev(ci.v, dt).view(B, T, H, V)
    o, ht = api.chunk_fwd_kda(q, k, v, dev(g).view(B, T, H, K), dev(ci.beta).view(B, T, H), scale=scale, h0=h0,
                              ht=ht, out_dtype=TORCH_DT[out_dtype])
    torch.cuda.synchronize()
    return o, ht


def check_chunk_kda(B, T, H, K, V, dtype, seed, shift, label, heads=None, forget=0):
    ci = chunk_inputs([T] * B, H, K, V, dtype=dtype, seed=seed, h0_std=0.1)
    g = channel_log_decay((B * T, H, K), seed + 1, shift)
    if forget:  # `forget` random (token, head, channel) entries forget everything: log-decay -inf
        rng = np.random.default_rng(seed + 2)
        idx = rng.choice(g.size, forget, replace=False)
        g.reshape(-1)[idx] = -np.inf
    scale = K ** -0.5
    h0 = dev(ci.h0)
    o32, ht32 = run_chunk_kda(ci, g, B, T, scale, "f32", h0)
    o16, ht16 = run_chunk_kda(ci, g, B, T, scale, "bf16", h0)
    assert torch.equal(o16, bf16_rne(o32)), f"{label}: bf16 output is not RNE of the f32 output"
    assert torch.equal(ht16, ht32)
    heads = list(range(H)) if heads is None else heads
    eo = es = 0.0
    for b in range(B):
        sl = slice(b * T, (b + 1) * T)
        o_ref, s_ref = oracle.recurrent_fwd_kda(ci.q[sl][:, heads], ci.k[sl][:, heads], ci.v[sl][:, heads],
                                                g[sl][:, heads], ci.beta[sl][:, heads], scale=scale,
                                                S0=ci.h0[b][heads])
        eo = max(eo, max_err_over_rms(host(o32[b])[:, heads], o_ref))
        es = max(es, max_err_over_rms(host(ht32[b])[heads], s_ref))
    tol = TOL[dtype]
    _print(f"[chunk kda {label}] max|do|/rms={eo:.3e} max|dS|/rms={es:.3e} tol={tol}")
    assert eo <= tol and es <= tol


@pytest.mark.parametrize("K,V", [(128, 128), (64, 64), (128, 64), (64, 128)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_chunk_kda_small(K, V, dtype):
    """Two sequences of 150 tokens (two full chunks and a ragged one), three heads."""
    check_chunk_kda(2, 150, 3, K, V, dtype, seed=90 + K + V, shift=2.0, label=f"K={K} V={V} {dtype}")


def test_chunk_kda_random_packed():
    """Eight seeded random packed calls of the per-channel chunk form against the
    oracle: 1-4 sequences of mixed lengths (empty and one-token ones among them)
    with dense initial states, 1-4 heads, every head-size pair, bf16 and fp32,
    decays from long memory to forgetting within a token."""
    for seed in range(8):
        rng = np.random.default_rng(9500 + seed)
        n = int(rng.integers(1, 5))
        lengths = [int(x) for x in rng.integers(0, 600, n)]
        if n > 1:
            lengths[int(rng.integers(n))] = int(rng.choice([0, 1, 64, 65]))
        H = int(rng.integers(1, 5))
        K, V = [(128, 128), (64, 64), (128, 64), (64, 128)][int(rng.integers(4))]
        dtype = "bf16" if rng.random() < 0.6 else "f32"
        shift = float(rng.choice([-4.0, 2.0, 8.0]))
        ci = chunk_inputs(lengths, H, K, V, dtype=dtype, seed=9600 + seed, h0_std=0.1)
        T = sum(lengths)
        g = channel_log_decay((T, H, K), 9700 + seed, shift)
        dt = TORCH_DT[dtype]
        q, k, v = (dev(x, dt) for x in (ci.q, ci.k, ci.v))
        outs = {}
        for od in ("f32", "bf16"):
            o, ht = api.chunk_fwd_kda(q, k, v, dev(g), dev(ci.beta), scale=K ** -0.5, cu_seqlens=ci.cu_seqlens.tolist(),
                                      h0=dev(ci.h0), out_dtype=TORCH_DT[od])
            torch.cuda.synchronize()
            outs[od] = (o, ht)
        (o32, ht32), (o16, ht16) = outs["f32"], outs["bf16"]
        assert torch.equal(o16, bf16_rne(o32)) and torch.equal(ht16, ht32)
        o_h, ht_h = host(o32), host(ht32)
        eo = es = 0.0
        for si in range(n):
            r = slice(int(ci.cu_seqlens[si]), int(ci.cu_seqlens[si + 1]))
            if r.stop == r.start:
                assert np.array_equal(ht_h[si], ci.h0[si]), "an empty sequence passes its state through"
                continue
            o_ref, s_ref = oracle.recurrent_fwd_kda(ci.q[r], ci.k[r], ci.v[r], g[r], ci.beta[r], scale=K ** -0.5,
                                                    S0=ci.h0[si])
            eo = max(eo, max_err_over_rms(o_h[r], o_ref))
            es = max(es, max_err_over_rms(ht_h[si], s_ref))
        tol = TOL[dtype]
        _print(f"[chunk kda random {seed}: lengths {lengths} H={H} K={K} V={V} {dtype} shift={shift}] "
               f"max|do|/rms={eo:.3e} max|dS|/rms={es:.3e} tol={tol}")
        assert eo <= tol and es <= tol


def test_chunk_kda_long_memory():
    """Slow per-channel decays (shift -4): the carry across chunks dominates."""
    check_chunk_kda(1, 300, 2, 128, 128, "bf16", seed=97, shift=-4.0, label="long memory")


def test_chunk_kda_config_full():
    """B=1, H=16, T=4096, K=V=128 (the chunk workload's shape), every head against the oracle."""
    check_chunk_kda(1, 4096, 16, 128, 128, "bf16", seed=98, shift=2.0, label="H16 T4096")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_chunk_kda_fully_forgetting_channels(dtype):
    """Some (token, head, channel) log-decays are -inf (that channel's memory is
    wiped): outputs and states stay finite and match the definition, where
    exp(-inf) = 0; rows past the ragged end read such a value too."""
    check_chunk_kda(2, 150, 3, 128, 128, dtype, seed=120, shift=-4.0, label=f"-inf decays {dtype}", forget=200)


def test_chunk_kda_uniform_channels_equal_the_scalar_gate():
    """Every key channel given the token's scalar log-gate: the per-channel chunk
    form computes the scalar rule, checked against the scalar oracle and against
    the scalar chunk path on the same inputs."""
    B, T, H, K, V = 2, 200, 2, 128, 128
    ci = chunk_inputs([T] * B, H, K, V, dtype="bf16", seed=101, h0_std=0.1)
    g = np.repeat(ci.a[:, :, None], K, axis=2)
    h0 = dev(ci.h0)
    o_k, ht_k = run_chunk_kda(ci, g, B, T, K ** -0.5, "f32", h0)
    o_s, ht_s = run_chunk(ci, K ** -0.5, "f32")
    eo = es = 0.0
    for b in range(B):
        sl = slice(b * T, (b + 1) * T)
        o_ref, s_ref = oracle.recurrent_fwd(ci.q[sl], ci.k[sl], ci.v[sl], ci.a[sl], ci.beta[sl], scale=K ** -0.5,
                                            S0=ci.h0[b])
        eo = max(eo, max_err_over_rms(host(o_k[b]), o_ref))
        es = max(es, max_err_over_rms(host(ht_k[b]), s_ref))
    e_cross = max_err_over_rms(host(o_k).reshape(B * T, H, V), host(o_s))
    _print(f"[chunk kda uniform] vs scalar oracle o={eo:.2e} S={es:.2e}; vs scalar chunk path {e_cross:.2e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"] and e_cross <= TOL["bf16"]
    assert max_err_over_rms(host(ht_k), host(ht_s)) <= TOL["bf16"]


def test_chunk_kda_empty_and_in_place():
    ci = chunk_inputs([1, 1], 2, 64, 64, dtype="bf16", seed=99, h0_std=0.1)
    h0 = dev(ci.h0)
    g = channel_log_decay((2, 2, 64), 100)
    empty = ci.q[:0]
    o, ht = api.chunk_fwd_kda(dev(empty, torch.bfloat16).view(2, 0, 2, 64), dev(empty, torch.bfloat16).view(2, 0, 2, 64),
                              dev(ci.v[:0], torch.bfloat16).view(2, 0, 2, 64), dev(g[:0]).view(2, 0, 2, 64),
                              dev(ci.beta[:0]).view(2, 0, 2), h0=h0)
    torch.cuda.synchronize()
    assert o.numel() == 0 and torch.equal(ht, h0)  # T == 0 passes the initial state through
    o1, ht1 = run_chunk_kda(ci, g, 2, 1, 0.5, "f32", h0)
    state = h0.clone()
    o2, ht2 = run_chunk_kda(ci, g, 2, 1, 0.5, "f32", state, ht=state)  # in place
    assert torch.equal(o1, o2) and torch.equal(ht1, state)


# ------------------------------------------ decode layer front and back operations
#
# Tolerances: q, k, v, beta and the normalised output are float32 results of a
# few float32 operations on exactly representable inputs, so they are held to
# max|err| <= 1e-5 * RMS(reference); the conv state is bf16 values moved, so it is
# compared bit for bit; a bf16 output equals RNE of the float32 output of the
# same call.

LAYER_TOL = 1e-5


def run_prologue(li, state_dev, bias=True):
    return api.decode_prologue(dev(li.x, torch.bfloat16), dev(li.conv_w), dev(li.conv_bias) if bias else None,
                               state_dev, dev(li.slots, torch.int32), dev(li.beta_raw), li.H)


def check_prologue(li, label, bias=True):
    state0 = dev(li.conv_state, torch.bfloat16)
    state = state0.clone()
    q, k, v, beta = run_prologue(li, state, bias)
    torch.cuda.synchronize()
    rq, rk, rv, rb, rst = oracle.decode_prologue(li.x, li.conv_w, li.conv_bias if bias else None, li.conv_state,
                                                 li.slots, li.beta_raw, li.H, li.D)
    act = li.slots > 0
    errs = [max_err_over_rms(host(t)[act], r[act]) for t, r in ((q, rq), (k, rk), (v, rv), (beta, rb))]
    for t in (q, k, v, beta):
        assert bool((t[torch.from_numpy(~act).cuda()].view(torch.int32) == 0).all()), f"{label}: padding not +0"
    assert np.array_equal(host(state), rst), f"{label}: conv state differs"
    _print(f"[prologue {label}] max err/rms q,k,v,beta = " + " ".join(f"{e:.2e}" for e in errs))
    assert max(errs) <= LAYER_TOL


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("bias", [True, False])
def test_decode_prologue_small(D, bias):
    li = layer_inputs(N=37, H=3, D=D, pool_slots=48, seed=D + bias, n_padding=5)
    check_prologue(li, f"D={D} bias={bias}", bias)


def test_decode_prologue_config_full():
    """N=256 requests, H=32 heads of 128 channels, a pool of 512 conv states, 32 padding rows."""
    li = layer_inputs(N=256, H=32, D=128, pool_slots=512, seed=9, n_padding=32)
    check_prologue(li, "N256 H32 D128")


def test_decode_prologue_consecutive_tokens_shift_the_state():
    """Four tokens in a row through one slot: the state after them holds the last
    three inputs, and every token's outputs match the oracle's running state."""
    li = layer_inputs(N=4, H=2, D=64, pool_slots=8, seed=77)
    state = dev(li.conv_state, torch.bfloat16)
    st_ref = li.conv_state
    for t in range(4):
        x_t, b_t, slot = li.x[t:t + 1], li.beta_raw[t:t + 1], np.array([3], np.int32)
        q, k, v, beta = api.decode_prologue(dev(x_t, torch.bfloat16), dev(li.conv_w), dev(li.conv_bias), state,
                                            dev(slot, torch.int32), dev(b_t), li.H)
        torch.cuda.synchronize()
        rq, rk, rv, rb, st_ref = oracle.decode_prologue(x_t, li.conv_w, li.conv_bias, st_ref, slot, b_t, li.H,
                                                        li.D)
        for t_, r in ((q, rq), (k, rk), (v, rv), (beta, rb)):
            assert max_err_over_rms(host(t_), r) <= LAYER_TOL
    assert np.array_equal(host(state), st_ref)
    assert np.array_equal(host(state)[3], li.x[1:4].T)


@pytest.mark.parametrize("D", [64, 128])
def test_gated_rmsnorm(D):
    N, H = 29, 5
    rng = np.random.default_rng(D)
    o = rng.standard_normal((N, H, D)).astype(np.float32).astype(np.float64)
    o[3] *= 1e-3  # a small-norm row
    li = layer_inputs(N=N, H=H, D=D, pool_slots=N + 1, seed=D)
    o_d = dev(o)
    outs = {od: api.gated_rmsnorm(o_d, dev(li.gate, torch.bfloat16), dev(li.norm_w), 1e-6,
                                  out_dtype=TORCH_DT[od]) for od in ("f32", "bf16")}
    torch.cuda.synchronize()
    ref = oracle.gated_rmsnorm(o, li.gate, li.norm_w, 1e-6)
    err = max_err_over_rms(host(outs["f32"]), ref)
    _print(f"[gated rmsnorm D={D}] max err/rms={err:.2e}")
    assert err <= LAYER_TOL
    assert torch.equal(outs["bf16"], bf16_rne(outs["f32"]))


def test_decode_layer_composition():
    """Front operations, the recurrent decode step and the gated RMSNorm in a row,
    against the oracle's three steps: N=64 requests, H=4 heads of 128 channels."""
    N, H, D, P = 64, 4, 128, 80
    li = layer_inputs(N=N, H=H, D=D, pool_slots=P, seed=123, n_padding=6)
    rng = np.random.default_rng(124)
    a = round_to_f32(-np.log1p(np.exp(rng.standard_normal((N, H)) + 2.0)))
    pool0 = round_to_f32(rng.normal(0.0, 0.1, (P, H, D, D)))
    conv = dev(li.conv_state, torch.bfloat16)
    pool = dev(pool0)
    slots = dev(li.slots, torch.int32)
    q, k, v, beta = run_prologue(li, conv)
    o = api.recurrent_step(q, k, v, dev(a), beta, pool, slots, scale=D ** -0.5, out_dtype=torch.float32)
    out = api.gated_rmsnorm(o, dev(li.gate, torch.bfloat16), dev(li.norm_w), 1e-6, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rq, rk, rv, rb, _ = oracle.decode_prologue(li.x, li.conv_w, li.conv_bias, li.conv_state, li.slots,
                                               li.beta_raw, H, D)
    ro, rpool = oracle.decode_step(rq, rk, rv, a, rb, pool0, li.slots, scale=D ** -0.5)
    ref = oracle.gated_rmsnorm(ro, li.gate, li.norm_w, 1e-6)
    act = li.slots > 0
    e_out = max_err_over_rms(host(out)[act], ref[act])
    e_st = max_err_over_rms(host(pool)[li.slots[act]], rpool[li.slots[act]])
    _print(f"[decode layer] max err/rms out={e_out:.2e} state={e_st:.2e}")
    assert e_out <= TOL["f32"] and e_st <= TOL["f32"]


def test_graph_capture_replays_match_eager():
    """A chunked call and a decode step captured in one HIP graph: three replays,
    with eager work between them, give the eager results bit for bit (the chunked
    call is idempotent; the decode step advances the pool like eager steps)."""
    T, H, K, V = 300, 4, 128, 128
    ci = chunk_inputs([T], H, K, V, dtype="bf16", seed=42, h0_std=0.1)
    dt = torch.bfloat16
    q, k, v = (dev(x, dt).view(1, T, H, -1) for x in (ci.q, ci.k, ci.v))
    g, b = dev(ci.a).view(1, T, H), dev(ci.beta).view(1, T, H)
    h0 = dev(ci.h0)
    o = torch.empty(1, T, H, V, dtype=torch.float32, device="cuda")
    ht = torch.empty(1, H, V, K, dtype=torch.float32, device="cuda")
    ws = torch.empty(api.workspace_bytes(1, T, H, K, V), dtype=torch.uint8, device="cuda")
    di = decode_inputs(N=16, H=H, K=K, V=V, pool_slots=24, dtype="bf16", seed=43, n_padding=3)
    dq, dk, dv = (dev(x, dt) for x in (di.q, di.k, di.v))
    dg, dbeta = dev(di.a), dev(di.beta)
    slots = dev(di.slots, torch.int32)
    pool0 = dev(di.pool)
    do = torch.empty(16, H, V, dtype=torch.float32, device="cuda")

    def calls(pool):
        api.chunk_fwd(q, k, v, g, b, scale=0.2, h0=h0, ht=ht, out=o, out_dtype=torch.float32, workspace=ws)
        api.recurrent_step(dq, dk, dv, dg, dbeta, pool, slots, scale=0.3, out=do, out_dtype=torch.float32)

    # eager: one chunked call; three decode steps in sequence
    pool_e = pool0.clone()
    calls(pool_e)
    torch.cuda.synchronize()
    o_ref, ht_ref = o.clone(), ht.clone()
    do_ref, pool_ref = [do.clone()], [pool_e.clone()]
    for _ in range(2):
        calls(pool_e)
        torch.cuda.synchronize()
        do_ref.append(do.clone())
        pool_ref.append(pool_e.clone())

    pool_g = pool0.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture, on the capture's stream kind
        calls(pool0.clone())
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls(pool_g)
    for rep in range(3):
        o.fill_(float("nan"))
        ht.fill_(float("nan"))
        ws.fill_(0xFF)
        do.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(ht, ht_ref), f"replay {rep}: chunked call differs"
        assert torch.equal(do, do_ref[rep]) and torch.equal(pool_g, pool_ref[rep]), f"replay {rep}: decode differs"
    _print("[graph] 3 replays equal to eager")


# ------------------------------------------ gate stage of the KDA decode layer
#
# The bf16 projection is a rounding decision taken in float32 in the order the
# gate mode fixes, on both sides: bit-exact. The log-decays go through
# transcendentals (float32 on the GPU, float64 in the oracle): within
# 2e-6 * |lower_bound|.

def _gate_dev(gi):
    return (dev(gi.f_a, torch.bfloat16), dev(gi.f_b, torch.bfloat16), dev(gi.a_log), dev(gi.dt_bias))


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("N,H,K", [(1, 3, 128), (13, 2, 64), (300, 5, 128)])
def test_kda_gate(mode, N, H, K):
    from linear_attention_sequence_recompute_amd.workloads import gate_inputs
    gi = gate_inputs(N, H, K, seed=200 + N + H + K + mode)
    g, raw = api.kda_gate(*_gate_dev(gi), gi.lower_bound, H, mode=mode, with_raw=True)
    torch.cuda.synchronize()
    raw_ref, g_ref = oracle.kda_gate(gi.f_a, gi.f_b, gi.a_log, gi.dt_bias, gi.lower_bound, H, K, mode)
    np.testing.assert_array_equal(host(raw), raw_ref)
    err = float(np.max(np.abs(host(g) - g_ref)))
    _print(f"[kda gate mode={mode} N={N} H={H} K={K}] max|dg|={err:.2e}")
    assert err <= 2e-6 * abs(gi.lower_bound)


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_kda_gate_orders_golden(mode):
    """The hand-derived fixture where the three orders round differently."""
    import json
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "gate_orders.json")))
    f_a = np.zeros((1, 128))
    for c, x in gold["f_a"].items():
        f_a[0, int(c)] = x
    K = 64
    f_b = np.zeros((K, 128))  # features 2.. are zero rows
    for f, row in enumerate(gold["f_b"]):
        for c, x in row.items():
            f_b[f, int(c)] = x
    g, raw = api.kda_gate(dev(f_a, torch.bfloat16), dev(f_b, torch.bfloat16), dev(np.zeros(1)), dev(np.zeros(K)),
                          -1.0, 1, mode=mode, with_raw=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(raw)[0, 0, :2], gold["raw_g"][str(mode)])


def test_kda_gate_then_decode_step():
    """gate -> decode step with per-channel decays, against the oracle's chain."""
    from linear_attention_sequence_recompute_amd.workloads import gate_inputs
    N, H, K = 64, 4, 128
    gi = gate_inputs(N, H, K, seed=210)
    di = decode_inputs(N, H, K, K, 80, dtype="bf16", seed=211, n_padding=5)
    g = api.kda_gate(*_gate_dev(gi), gi.lower_bound, H, mode=1)
    pool = dev(di.pool)
    o = api.recurrent_step_kda(dev(di.q, torch.bfloat16), dev(di.k, torch.bfloat16), dev(di.v, torch.bfloat16), g,
                               dev(di.beta), pool, dev(di.slots, torch.int32), scale=K ** -0.5,
                               out_dtype=torch.float32)
    torch.cuda.synchronize()
    _, g_ref = oracle.kda_gate(gi.f_a, gi.f_b, gi.a_log, gi.dt_bias, gi.lower_bound, H, K, 1)
    o_ref, pool_ref = oracle.decode_step_kda(di.q, di.k, di.v, g_ref, di.beta, di.pool, di.slots, scale=K ** -0.5)
    eo, ep = max_err_over_rms(host(o), o_ref), max_err_over_rms(host(pool), pool_ref)
    _print(f"[gate -> decode kda] o {eo:.2e} pool {ep:.2e}")
    assert eo <= 1e-4 and ep <= 1e-4


# -------------------------------------- decode layer front for speculative verify

def check_prologue_verify(li, label):
    state = dev(li.conv_state, torch.bfloat16)
    q, k, v, beta = api.decode_prologue_verify(dev(li.x, torch.bfloat16), dev(li.conv_w), dev(li.conv_bias), state,
                                               dev(li.slots, torch.int32), dev(li.accepted, torch.int32),
                                               dev(li.beta_raw), li.H, li.T)
    torch.cuda.synchronize()
    rq, rk, rv, rb, rst = oracle.decode_prologue_verify(li.x, li.conv_w, li.conv_bias, li.conv_state, li.slots,
                                                        li.accepted, li.beta_raw, li.H, li.D, li.T)
    act = rb[:, 0] != 0
    errs = [max_err_over_rms(host(t)[act], r[act]) for t, r in ((q, rq), (k, rk), (v, rv), (beta, rb))]
    for t in (q, k, v, beta):
        assert bool((t[torch.from_numpy(~act).cuda()].view(torch.int32) == 0).all()), f"{label}: padding not +0"
    assert np.array_equal(host(state), rst), f"{label}: conv state differs"
    _print(f"[prologue verify {label}] max err/rms q,k,v,beta = " + " ".join(f"{e:.2e}" for e in errs))
    assert max(errs) <= LAYER_TOL


@pytest.mark.parametrize("D,T", [(64, 2), (128, 4), (128, 8), (64, 1)])
def test_decode_prologue_verify(D, T):
    from linear_attention_sequence_recompute_amd.workloads import layer_verify_inputs
    li = layer_verify_inputs(N=13, T=T, H=3, D=D, pool_slots=13 * T + 9, seed=300 + D + T, n_padding=3)
    check_prologue_verify(li, f"D={D} T={T}")


def test_decode_layer_verify_composition():
    """Verify-mode front (T = 4), the speculative-verify decode and the gated
    RMSNorm in a row, against the oracle's three steps: N=24 requests, H=4 heads
    of 128 channels, 3 padding requests."""
    from linear_attention_sequence_recompute_amd.workloads import layer_verify_inputs
    N, T, H, D = 24, 4, 4, 128
    P = N * T + 5
    li = layer_verify_inputs(N=N, T=T, H=H, D=D, pool_slots=P, seed=321, n_padding=3)
    conv = dev(li.conv_state, torch.bfloat16)
    pool = dev(li.pool)
    slots, acc = dev(li.slots, torch.int32), dev(li.accepted, torch.int32)
    q, k, v, beta = api.decode_prologue_verify(dev(li.x, torch.bfloat16), dev(li.conv_w), dev(li.conv_bias), conv,
                                               slots, acc, dev(li.beta_raw), H, T)
    o = api.recurrent_verify(q.view(N, T, H, D), k.view(N, T, H, D), v.view(N, T, H, D), dev(li.a).view(N, T, H),
                             beta.view(N, T, H), pool, slots, acc, scale=D ** -0.5, out_dtype=torch.float32)
    out = api.gated_rmsnorm(o.view(N * T, H, D), dev(li.gate, torch.bfloat16), dev(li.norm_w), 1e-6,
                            out_dtype=torch.float32)
    torch.cuda.synchronize()
    rq, rk, rv, rb, _ = oracle.decode_prologue_verify(li.x, li.conv_w, li.conv_bias, li.conv_state, li.slots,
                                                      li.accepted, li.beta_raw, H, D, T)
    ro, rpool = oracle.decode_verify(rq.reshape(N, T, H, D), rk.reshape(N, T, H, D), rv.reshape(N, T, H, D),
                                     li.a.reshape(N, T, H), rb.reshape(N, T, H), li.pool, li.slots, li.accepted,
                                     scale=D ** -0.5)
    ref = oracle.gated_rmsnorm(ro.reshape(N * T, H, D), li.gate, li.norm_w, 1e-6)
    act = rb[:, 0] != 0
    e_out = max_err_over_rms(host(out)[act], ref[act])
    e_st = max_err_over_rms(host(pool), rpool)
    _print(f"[decode layer verify] max err/rms out={e_out:.2e} pool={e_st:.2e}")
    assert e_out <= TOL["f32"] and e_st <= TOL["f32"]
    assert bool((out[torch.from_numpy(~act).cuda()] == 0).all())


# ---------------------------------------------------- the decode layer in one launch

def _layer_fused_case(N, H, D, P, seed, kda, norm, n_padding, out_dtype="f32"):
    li = layer_inputs(N=N, H=H, D=D, pool_slots=P, seed=seed, n_padding=n_padding)
    rng = np.random.default_rng(seed + 1)
    if kda:
        g = channel_log_decay((N, H, D), seed + 2)
    else:
        g = round_to_f32(-np.log1p(np.exp(rng.standard_normal((N, H)) + 2.0)))
    pool0 = round_to_f32(rng.normal(0.0, 0.1, (P, H, D, D)))
    conv = dev(li.conv_state, torch.bfloat16)
    pool = dev(pool0)
    out = api.decode_layer(dev(li.x, torch.bfloat16), dev(li.conv_w), dev(li.conv_bias), conv,
                           dev(li.slots, torch.int32), dev(li.beta_raw), dev(g), pool, H,
                           gate=dev(li.gate, torch.bfloat16) if norm else None, norm_w=dev(li.norm_w) if norm else None,
                           out_dtype=TORCH_DT[out_dtype])
    torch.cuda.synchronize()
    rq, rk, rv, rb, rst = oracle.decode_prologue(li.x, li.conv_w, li.conv_bias, li.conv_state, li.slots,
                                                 li.beta_raw, H, D)
    step = oracle.decode_step_kda if kda else oracle.decode_step
    ro, rpool = step(rq, rk, rv, g, rb, pool0, li.slots, scale=D ** -0.5)
    ref = oracle.gated_rmsnorm(ro, li.gate, li.norm_w, 1e-6) if norm else ro
    act = li.slots > 0
    e_out = max_err_over_rms(host(out)[act], ref[act])
    e_st = max_err_over_rms(host(pool)[li.slots[act]], rpool[li.slots[act]])
    return li, out, conv, pool, pool0, rst, e_out, e_st, act


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("kda", [False, True])
@pytest.mark.parametrize("norm", [False, True])
def test_decode_layer_fused(D, kda, norm):
    li, out, conv, pool, pool0, rst, e_out, e_st, act = _layer_fused_case(40, 3, D, 52, 400 + D + 2 * kda + norm, kda,
                                                                          norm, n_padding=5)
    _print(f"[decode layer fused D={D} kda={kda} norm={norm}] out {e_out:.2e} state {e_st:.2e}")
    assert e_out <= TOL["f32"] and e_st <= TOL["f32"]
    assert np.array_equal(host(conv), rst), "conv state differs"
    assert bool((out[torch.from_numpy(~act).cuda()].view(torch.int32) == 0).all()), "padding rows not +0"
    unused = np.setdiff1d(np.arange(pool.shape[0]), li.slots[act])
    assert torch.equal(pool[torch.from_numpy(unused).cuda()], dev(pool0)[torch.from_numpy(unused).cuda()])


def test_decode_layer_fused_random():
    """Eight seeded random calls of the fused decode layer against the oracle's
    front, step and gated RMSNorm: 1-200 requests with padding rows, 1-6 heads of
    64 or 128, pools a little or much larger than the batch, scalar gates or
    per-channel decays, with and without the norm; the conv state bit for bit."""
    for seed in range(8):
        rng = np.random.default_rng(9800 + seed)
        N = int(rng.integers(1, 201))
        H = int(rng.integers(1, 7))
        D = int(rng.choice([64, 128]))
        n_pad = int(rng.integers(0, N // 4 + 1))
        P = N + 1 + int(rng.integers(0, N + 8))
        kda, norm = bool(rng.random() < 0.5), bool(rng.random() < 0.5)
        li, out, conv, pool, pool0, rst, e_out, e_st, act = _layer_fused_case(N, H, D, P, 9900 + seed, kda, norm,
                                                                              n_padding=n_pad)
        _print(f"[decode layer fused random {seed}: N={N} H={H} D={D} P={P} pad={n_pad} kda={kda} norm={norm}] "
               f"out {e_out:.2e} state {e_st:.2e}")
        assert e_out <= TOL["f32"] and e_st <= TOL["f32"]
        assert np.array_equal(host(conv), rst), "conv state differs"
        assert bool((out[torch.from_numpy(~act).cuda()].view(torch.int32) == 0).all()), "padding rows not +0"


def test_decode_layer_fused_config_full():
    """N=256 requests, H=32 heads of 128, pool of 512 slots, 32 padding rows, per-channel
    decays, gated RMSNorm, bf16 output (= RNE of the float32 output of the same call)."""
    li, out, conv, pool, pool0, rst, e_out, e_st, act = _layer_fused_case(256, 32, 128, 512, 450, True, True, 32)
    _print(f"[decode layer fused N256 H32] out {e_out:.2e} state {e_st:.2e}")
    assert e_out <= TOL["f32"] and e_st <= TOL["f32"]
    assert np.array_equal(host(conv), rst)


def test_chunk_kda_varlen_pool():
    """Packed sequences of very different lengths (empty, one token, chunk
    multiples, ragged tails) with per-channel decays and states in a pool (one
    padding slot): every sequence against the per-token definition; unused and
    padding slots untouched; bf16 output = RNE of the float32 output."""
    lengths = [300, 0, 1, 64, 65, 130, 7]
    H, K, V = 3, 128, 64
    ci = chunk_inputs(lengths, H, K, V, dtype="bf16", seed=130, pool_slots=10, slot_ids=[4, 2, 0, 7, 1, 9, 5])
    g = channel_log_decay((ci.total_tokens, H, K), 131, -1.0)
    dt = torch.bfloat16
    q, k, v = dev(ci.q, dt), dev(ci.k, dt), dev(ci.v, dt)
    cu = ci.cu_seqlens.tolist()
    pool0 = dev(ci.pool)
    outs = {}
    for od in ("f32", "bf16"):
        pool = pool0.clone()
        o, ht = api.chunk_fwd_kda(q, k, v, dev(g), dev(ci.beta), scale=K ** -0.5, cu_seqlens=cu, state_pool=pool,
                                  state_slots=dev(ci.slots, torch.int32), out_dtype=TORCH_DT[od])
        torch.cuda.synchronize()
        assert ht is None
        outs[od] = (o, pool)
    assert torch.equal(outs["bf16"][0], bf16_rne(outs["f32"][0]))
    assert torch.equal(outs["bf16"][1], outs["f32"][1])
    o, pool = outs["f32"]
    for sl in (0, 3, 6, 8):  # unused and the padding sequence's: untouched
        assert torch.equal(pool[sl], pool0[sl]), f"slot {sl} was written"
    oh = host(o)
    eo = es = 0.0
    for s in range(len(lengths)):
        r = slice(cu[s], cu[s + 1])
        S0 = ci.pool[ci.slots[s]] if ci.slots[s] > 0 else None
        o_ref, S_ref = oracle.recurrent_fwd_kda(ci.q[r], ci.k[r], ci.v[r], g[r], ci.beta[r], scale=K ** -0.5, S0=S0)
        if lengths[s]:
            eo = max(eo, max_err_over_rms(oh[r], o_ref))
        if ci.slots[s] > 0:
            es = max(es, max_err_over_rms(host(pool[ci.slots[s]]), S_ref))
    _print(f"[chunk kda varlen pool] max|do|/rms={eo:.3e} max|dS|/rms={es:.3e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


def test_chunk_kda_varlen_dense_states_f32():
    """Packed float32 inputs with dense h0 / ht updated in place (ht = h0)."""
    lengths = [150, 64, 1, 200]
    H, K, V = 2, 64, 128
    ci = chunk_inputs(lengths, H, K, V, dtype="f32", seed=140, h0_std=0.1)
    g = channel_log_decay((ci.total_tokens, H, K), 141, -2.0)
    cu = ci.cu_seqlens.tolist()
    state = dev(ci.h0)
    o, ht = api.chunk_fwd_kda(dev(ci.q), dev(ci.k), dev(ci.v), dev(g), dev(ci.beta), scale=0.3, cu_seqlens=cu,
                              h0=state, ht=state, out_dtype=torch.float32)
    torch.cuda.synchronize()
    eo = es = 0.0
    for s in range(len(lengths)):
        r = slice(cu[s], cu[s + 1])
        o_ref, S_ref = oracle.recurrent_fwd_kda(ci.q[r], ci.k[r], ci.v[r], g[r], ci.beta[r], scale=0.3, S0=ci.h0[s])
        eo = max(eo, max_err_over_rms(host(o)[r], o_ref))
        es = max(es, max_err_over_rms(host(state[s]), S_ref))
    _print(f"[chunk kda varlen f32 in place] max|do|/rms={eo:.3e} max|dS|/rms={es:.3e}")
    assert eo <= TOL["f32"] and es <= TOL["f32"]


@pytest.mark.parametrize("nbytes", [16, 16 * 8191, 16 * 8192 * 3 + 16 * 77, 1 << 24])
def test_probes_move_every_byte(nbytes):
    """The streaming probes cover the whole buffer with their per-workgroup
    regions (sizes below, at and past one region per workgroup, ragged): the
    copy reproduces the source, the write fills every element with its pattern,
    the read's partial sums add up to the source's sum."""
    lib = api._lib.lib()
    n = nbytes // 16
    src = torch.arange(4 * n, dtype=torch.float32, device="cuda").remainder_(97.0)
    dst = torch.full_like(src, -1.0)
    sink = torch.zeros(8192, dtype=torch.float32, device="cuda")
    assert lib.gdn_probe_copy(src.data_ptr(), dst.data_ptr(), nbytes, None) == 0
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    assert lib.gdn_probe_write(dst.data_ptr(), nbytes, None) == 0
    torch.cuda.synchronize()
    assert torch.equal(dst.view(n, 4), torch.tensor([1.0, 2.0, 3.0, 4.0], device="cuda").expand(n, 4))
    assert lib.gdn_probe_read(src.data_ptr(), sink.data_ptr(), nbytes, None) == 0
    torch.cuda.synchronize()
    assert float(sink.double().sum()) == pytest.approx(float(src.double().sum()), rel=1e-6)

