"""CPU checks of the C ABI: the library loads, exports every symbol include/gdn.h
declares, and its host-side validation rejects bad arguments before launching
anything (no call here reaches a kernel launch, so no GPU is needed)."""

import ctypes
import os
import re

import numpy as np
import pytest

from linear_attention_sequence_recompute_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libgdn.so not built")

BF16, F32 = _lib.GDN_BF16, _lib.GDN_F32
FAKE = 1 << 20  # an aligned non-null address; never dereferenced by the failing calls below


def declared_functions(headers=None):
    names = []
    for h in headers or HEADERS:
        names += re.findall(r"^\S[^()#]*?\b(gdn_\w+)\s*\(", open(h).read(), re.M)
    return names


def test_header_declares_the_boundary():
    assert set(declared_functions([HEADER])) == {"gdn_chunk_fwd_workspace_bytes", "gdn_chunk_fwd_plan", "gdn_chunk_fwd",
                                         "gdn_chunk_fwd_profiled", "gdn_chunk_fwd_noalloc", "gdn_recurrent_step",
                                         "gdn_recurrent_step_kda",
                                         "gdn_recurrent_verify", "gdn_kda_gate", "gdn_fp8_quant", "gdn_decode_prologue", "gdn_decode_prologue_verify", "gdn_decode_layer",
                                         "gdn_gated_rmsnorm", "gdn_chunk_fwd_kda_workspace_bytes",
                                         "gdn_chunk_fwd_kda", "gdn_chunk_fwd_kda_profiled", "gdn_status_string"}


def test_library_exports_every_declared_symbol():
    raw = ctypes.CDLL(_lib.LIB_PATH)
    for name in declared_functions():
        assert hasattr(raw, name), name
    assert set(_lib.SIGNATURES) == set(declared_functions())


def test_status_strings():
    for st in (0, -1, -2, -3, -4):
        assert _lib.status_string(st).startswith("GDN_")
    assert _lib.status_string(-99) == "GDN_UNKNOWN_STATUS"


def test_workspace_bytes():
    L = _lib.lib()
    assert L.gdn_chunk_fwd_workspace_bytes(1, 4096, 16, 96, 128, BF16) == 0
    assert L.gdn_chunk_fwd_workspace_bytes(1, 4096, 0, 128, 128, BF16) == 0
    assert L.gdn_chunk_fwd_workspace_bytes(1, 4096, 16, 128, 128, 7) == 0
    b1 = L.gdn_chunk_fwd_workspace_bytes(1, 4096, 16, 128, 128, BF16)
    b2 = L.gdn_chunk_fwd_workspace_bytes(1, 4096, 16, 128, 128, F32)
    b3 = L.gdn_chunk_fwd_workspace_bytes(16, 60217, 16, 128, 128, BF16)
    assert 0 < b2 < b1 and b3 > b2
    # A' and P (the 6 nonzero hi/lo fragment tiles, 12 KiB each) plus three 64-float gate vectors per (chunk, head)
    per = b2 / ((4096 // 64 + 1) * 16)
    assert 24 * 1024 + 768 <= per < 26 * 1024
    # bf16 with 16 (sequence, head) pairs: room for the chunk-parallel form with 4
    # segments: 3 segment maps ([V + K][K] f32) and a copy of the initial state ([V][K] f32) per pair
    assert b1 - b2 == 16 * (3 * 256 * 128 + 128 * 128) * 4
    # 256 pairs fill the GPU without segments: no such room
    per3 = b3 / ((60217 // 64 + 16) * 16)
    assert 24 * 1024 + 768 <= per3 < 26 * 1024


def _chunk(**kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, o=FAKE, n_seqs=1, total=256, H=2, K=64, V=64,
                scale=1.0, in_dt=BF16, out_dt=BF16, cu=None, cu_host=None, h0=None, ht=None, pool=None,
                pool_slots=0, slots=None, ws=FAKE, ws_bytes=0, stream=None)
    args.update(kw)
    a = args
    return _lib.lib().gdn_chunk_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["o"], a["n_seqs"], a["total"],
                                    a["H"], a["K"], a["V"], a["scale"], a["in_dt"], a["out_dt"], a["cu"],
                                    a["cu_host"], a["h0"], a["ht"], a["pool"], a["pool_slots"], a["slots"],
                                    a["ws"], a["ws_bytes"], a["stream"])


def test_chunk_fwd_validation():
    E = _lib
    assert _chunk(K=96) == E.GDN_EUNSUPPORTED
    assert _chunk(V=32) == E.GDN_EUNSUPPORTED
    assert _chunk(in_dt=5) == E.GDN_EUNSUPPORTED
    assert _chunk(H=0) == E.GDN_EINVAL
    assert _chunk(total=-1) == E.GDN_EINVAL
    assert _chunk(n_seqs=3, total=256) == E.GDN_EINVAL  # not divisible into equal lengths
    assert _chunk(q=None) == E.GDN_EINVAL
    assert _chunk(q=FAKE + 2) == E.GDN_EINVAL  # misaligned
    assert _chunk(h0=FAKE + 4) == E.GDN_EINVAL
    assert _chunk(pool=FAKE, pool_slots=4, slots=None) == E.GDN_EINVAL
    assert _chunk(pool=FAKE, pool_slots=4, slots=FAKE, h0=FAKE) == E.GDN_EINVAL
    assert _chunk(slots=FAKE) == E.GDN_EINVAL
    assert _chunk(ws_bytes=10) == E.GDN_EWORKSPACE
    assert _chunk(ws=None, ws_bytes=1 << 40) == E.GDN_EWORKSPACE
    assert _chunk(ws=FAKE + 16, ws_bytes=1 << 40) == E.GDN_EWORKSPACE
    # empty call is a no-op success
    assert _chunk(n_seqs=0, total=0) == E.GDN_OK


def test_chunk_fwd_profiled_needs_events():
    L = _lib.lib()
    args = [FAKE] * 6 + [1, 256, 2, 64, 64, 1.0, BF16, BF16, None, None, None, None, None, 0, None, FAKE, 1 << 40, None]
    assert L.gdn_chunk_fwd_profiled(*args, None) == _lib.GDN_EINVAL
    ev = (ctypes.c_void_p * 3)(FAKE, None, FAKE)
    assert L.gdn_chunk_fwd_profiled(*args, ev) == _lib.GDN_EINVAL


def test_chunk_fwd_cu_seqlens_validation():
    E = _lib
    good = np.array([0, 100, 100, 256], dtype=np.int32)
    ptr = good.ctypes.data
    assert _chunk(n_seqs=3, cu=FAKE, cu_host=None) == E.GDN_EINVAL
    assert _chunk(n_seqs=3, cu=None, cu_host=ptr) == E.GDN_EINVAL
    bad_end = np.array([0, 100, 100, 255], dtype=np.int32)
    assert _chunk(n_seqs=3, cu=FAKE, cu_host=bad_end.ctypes.data) == E.GDN_EINVAL
    bad_start = np.array([1, 100, 100, 256], dtype=np.int32)
    assert _chunk(n_seqs=3, cu=FAKE, cu_host=bad_start.ctypes.data) == E.GDN_EINVAL
    decreasing = np.array([0, 100, 90, 256], dtype=np.int32)
    assert _chunk(n_seqs=3, cu=FAKE, cu_host=decreasing.ctypes.data) == E.GDN_EINVAL
    # a consistent schedule gets as far as the workspace check
    assert _chunk(n_seqs=3, cu=FAKE, cu_host=ptr, ws_bytes=0) == E.GDN_EWORKSPACE


def _step(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, pool=FAKE, pool_slots=8, slots=FAKE, o=FAKE, N=4, H=2,
             K=128, V=128, scale=1.0, in_dt=BF16, out_dt=BF16, stream=None)
    a.update(kw)
    return _lib.lib().gdn_recurrent_step(a["q"], a["k"], a["v"], a["g"], a["beta"], a["pool"], a["pool_slots"],
                                         a["slots"], a["o"], a["N"], a["H"], a["K"], a["V"], a["scale"],
                                         a["in_dt"], a["out_dt"], a["stream"])


def test_recurrent_step_validation():
    E = _lib
    assert _step(K=32) == E.GDN_EUNSUPPORTED
    assert _step(out_dt=3) == E.GDN_EUNSUPPORTED
    assert _step(H=0) == E.GDN_EINVAL
    assert _step(N=-1) == E.GDN_EINVAL
    assert _step(N=0) == E.GDN_OK
    assert _step(pool=None) == E.GDN_EINVAL
    assert _step(slots=None) == E.GDN_EINVAL
    assert _step(pool_slots=0) == E.GDN_EINVAL
    assert _step(pool=FAKE + 4) == E.GDN_EINVAL
    assert _step(q=FAKE + 1) == E.GDN_EINVAL


def test_recurrent_step_grid_limit():
    # one workgroup per 16 state rows of each (request, head) must fit a 1-D grid
    assert _step(N=1 << 20, H=4096, V=128) == _lib.GDN_EINVAL


def _verify(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, pool=FAKE, pool_slots=64, slots=FAKE, cols=4,
             accepted=FAKE, o=FAKE, N=4, T=4, H=2, K=128, V=128, scale=1.0, in_dt=BF16, out_dt=BF16, stream=None)
    a.update(kw)
    return _lib.lib().gdn_recurrent_verify(a["q"], a["k"], a["v"], a["g"], a["beta"], a["pool"], a["pool_slots"],
                                           a["slots"], a["cols"], a["accepted"], a["o"], a["N"], a["T"], a["H"],
                                           a["K"], a["V"], a["scale"], a["in_dt"], a["out_dt"], a["stream"])


def test_recurrent_verify_validation():
    E = _lib
    assert _verify(K=32) == E.GDN_EUNSUPPORTED
    assert _verify(in_dt=4) == E.GDN_EUNSUPPORTED
    assert _verify(T=0) == E.GDN_EINVAL
    assert _verify(T=9, cols=9) == E.GDN_EINVAL
    assert _verify(cols=3) == E.GDN_EINVAL  # fewer slot columns than tokens
    assert _verify(N=-1) == E.GDN_EINVAL
    assert _verify(H=0) == E.GDN_EINVAL
    assert _verify(N=0) == E.GDN_OK
    assert _verify(accepted=None) == E.GDN_EINVAL
    assert _verify(slots=None) == E.GDN_EINVAL
    assert _verify(pool_slots=0) == E.GDN_EINVAL
    assert _verify(accepted=FAKE + 2) == E.GDN_EINVAL
    assert _verify(q=FAKE + 1) == E.GDN_EINVAL
    assert _verify(N=1 << 20, H=4096) == E.GDN_EINVAL  # grid limit


def _fp8(**kw):
    a = dict(x=FAKE, codes=FAKE, scales=FAKE, rows=4, cols=256, group=128, stream=None)
    a.update(kw)
    return _lib.lib().gdn_fp8_quant(a["x"], a["codes"], a["scales"], a["rows"], a["cols"], a["group"], a["stream"])


def test_fp8_quant_validation():
    E = _lib
    assert _fp8(group=32) == E.GDN_EUNSUPPORTED
    assert _fp8(cols=200) == E.GDN_EINVAL       # not a multiple of the group
    assert _fp8(rows=-1) == E.GDN_EINVAL
    assert _fp8(rows=0) == E.GDN_OK
    assert _fp8(x=None) == E.GDN_EINVAL
    assert _fp8(x=FAKE + 4) == E.GDN_EINVAL     # x must be 16-byte aligned
    assert _fp8(codes=FAKE + 2) == E.GDN_EINVAL
    assert _fp8(rows=1 << 40, cols=1 << 20) == E.GDN_EINVAL  # grid limit


def test_recurrent_step_kda_validation():
    E = _lib
    args = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, pool=FAKE, pool_slots=8, slots=FAKE, o=FAKE, N=4, H=2,
                K=128, V=128, scale=1.0, in_dt=BF16, out_dt=BF16, stream=None)

    def call(**kw):
        a = dict(args, **kw)
        return _lib.lib().gdn_recurrent_step_kda(a["q"], a["k"], a["v"], a["g"], a["beta"], a["pool"],
                                                 a["pool_slots"], a["slots"], a["o"], a["N"], a["H"], a["K"],
                                                 a["V"], a["scale"], a["in_dt"], a["out_dt"], a["stream"])
    assert call(K=96) == E.GDN_EUNSUPPORTED
    assert call(N=0) == E.GDN_OK
    assert call(g=None) == E.GDN_EINVAL
    assert call(g=FAKE + 4) == E.GDN_EINVAL   # the per-channel decays are read as float4
    assert call(pool=FAKE + 4) == E.GDN_EINVAL


def test_decode_prologue_validation():
    E = _lib
    args = dict(x=FAKE, w=FAKE, bias=None, state=FAKE, pool_slots=8, slots=FAKE, beta_raw=FAKE, q=FAKE, k=FAKE,
                v=FAKE, beta=FAKE, N=4, H=2, D=128, stream=None)

    def call(**kw):
        a = dict(args, **kw)
        return _lib.lib().gdn_decode_prologue(a["x"], a["w"], a["bias"], a["state"], a["pool_slots"], a["slots"],
                                              a["beta_raw"], a["q"], a["k"], a["v"], a["beta"], a["N"], a["H"],
                                              a["D"], a["stream"])
    assert call(D=96) == E.GDN_EUNSUPPORTED
    assert call(N=0) == E.GDN_OK
    assert call(N=-1) == E.GDN_EINVAL
    assert call(H=0) == E.GDN_EINVAL
    assert call(state=None) == E.GDN_EINVAL
    assert call(beta=None) == E.GDN_EINVAL
    assert call(pool_slots=0) == E.GDN_EINVAL
    assert call(x=FAKE + 2) == E.GDN_EINVAL      # pairs of bf16 channels: 4-byte aligned
    assert call(state=FAKE + 2) == E.GDN_EINVAL
    assert call(q=FAKE + 4) == E.GDN_EINVAL      # float2 pairs: 8-byte aligned
    assert call(bias=FAKE + 4) == E.GDN_EINVAL
    assert call(N=1 << 20, H=4096) == E.GDN_EINVAL  # grid limit


def test_gated_rmsnorm_validation():
    E = _lib
    args = dict(o=FAKE, gate=FAKE, w=FAKE, eps=1e-6, out=FAKE, N=4, H=2, D=64, out_dt=BF16, stream=None)

    def call(**kw):
        a = dict(args, **kw)
        return _lib.lib().gdn_gated_rmsnorm(a["o"], a["gate"], a["w"], a["eps"], a["out"], a["N"], a["H"], a["D"],
                                            a["out_dt"], a["stream"])
    assert call(D=32) == E.GDN_EUNSUPPORTED
    assert call(out_dt=4) == E.GDN_EUNSUPPORTED
    assert call(N=0) == E.GDN_OK
    assert call(eps=-1.0) == E.GDN_EINVAL
    assert call(eps=float("nan")) == E.GDN_EINVAL
    assert call(gate=None) == E.GDN_EINVAL
    assert call(o=FAKE + 4) == E.GDN_EINVAL
    assert call(gate=FAKE + 2) == E.GDN_EINVAL
    assert call(out=FAKE + 2) == E.GDN_EINVAL
    assert call(out=FAKE + 4, out_dt=_lib.GDN_F32) == E.GDN_EINVAL
    assert call(N=1 << 20, H=4096) == E.GDN_EINVAL


def test_chunk_fwd_kda_validation():
    E = _lib
    L = _lib.lib()
    # chunk operands for floor(T / 64) + n_seqs chunks, then the packed schedule (16 B per chunk, 4 B per offset)
    ops = (64 + 1) * 16 * (2 * 4096 + 3 * 64 * 128 + 128) * 4
    assert L.gdn_chunk_fwd_kda_workspace_bytes(1, 4096, 16, 128) == (ops + 255) // 256 * 256 + 65 * 16 + 2 * 4
    assert L.gdn_chunk_fwd_kda_workspace_bytes(1, 100, 2, 96) == 0
    assert L.gdn_chunk_fwd_kda_workspace_bytes(-1, 100, 2, 64) == 0
    args = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, o=FAKE, n=2, total=200, H=2, K=128, V=128, scale=1.0,
                in_dt=BF16, out_dt=BF16, cu=None, cu_host=None, h0=None, ht=None, pool=None, pool_slots=0,
                slots=None, ws=FAKE, ws_bytes=1 << 40, stream=None)

    def call(**kw):
        a = dict(args, **kw)
        return L.gdn_chunk_fwd_kda(a["q"], a["k"], a["v"], a["g"], a["beta"], a["o"], a["n"], a["total"], a["H"],
                                   a["K"], a["V"], a["scale"], a["in_dt"], a["out_dt"], a["cu"], a["cu_host"], a["h0"],
                                   a["ht"], a["pool"], a["pool_slots"], a["slots"], a["ws"], a["ws_bytes"],
                                   a["stream"])
    assert call(K=96) == E.GDN_EUNSUPPORTED
    assert call(V=40) == E.GDN_EUNSUPPORTED
    assert call(V=512) == E.GDN_EUNSUPPORTED
    assert call(in_dt=4) == E.GDN_EUNSUPPORTED
    assert call(n=0, total=0) == E.GDN_OK
    assert call(n=-1) == E.GDN_EINVAL
    assert call(total=201) == E.GDN_EINVAL         # not a multiple of n_seqs without offsets
    assert call(H=0) == E.GDN_EINVAL
    assert call(scale=float("inf")) == E.GDN_EINVAL
    assert call(q=None) == E.GDN_EINVAL
    assert call(q=FAKE + 1) == E.GDN_EINVAL
    assert call(k=FAKE + 8) == E.GDN_EINVAL      # q, k, g read four channels at a time: 16-byte aligned
    assert call(g=FAKE + 4) == E.GDN_EINVAL
    assert call(h0=FAKE + 2) == E.GDN_EINVAL
    assert call(pool=FAKE, pool_slots=4, slots=FAKE, h0=FAKE) == E.GDN_EINVAL  # a pool excludes h0 / ht
    assert call(pool=FAKE, pool_slots=4, slots=None) == E.GDN_EINVAL
    assert call(slots=FAKE) == E.GDN_EINVAL                                    # slots without a pool
    bad = (ctypes.c_int32 * 3)(0, 120, 100)
    assert call(cu=FAKE, cu_host=ctypes.addressof(bad)) == E.GDN_EINVAL        # decreasing offsets
    assert call(cu=FAKE, cu_host=None) == E.GDN_EINVAL
    assert call(ws=None) == E.GDN_EWORKSPACE
    assert call(ws_bytes=1024) == E.GDN_EWORKSPACE
    assert call(ws=FAKE + 16) == E.GDN_EWORKSPACE


def test_probe_validation():
    """The measurement probes reject bad arguments before launching."""
    L = _lib.lib()
    EINVAL = _lib.GDN_EINVAL
    assert L.gdn_probe_mfma_bf16(None, 2048, 10, None) == EINVAL
    assert L.gdn_probe_mfma_bf16(FAKE, 2046, 10, None) == EINVAL  # not a multiple of 4
    assert L.gdn_probe_mfma_bf16(FAKE, 2048, 0, None) == EINVAL
    assert L.gdn_probe_copy(FAKE, None, 1 << 20, None) == EINVAL
    assert L.gdn_probe_copy(FAKE, FAKE + 8, 1 << 20, None) == EINVAL  # misaligned
    assert L.gdn_probe_copy(FAKE, FAKE, 1000, None) == EINVAL  # not a multiple of 16
    assert L.gdn_probe_read(FAKE, FAKE, 0, None) == EINVAL
    assert L.gdn_probe_write(None, 1 << 20, None) == EINVAL
    assert L.gdn_probe_write(FAKE, 24, None) == EINVAL


def _noalloc(**kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, o=FAKE, n_seqs=1, total=256, H=2, K=64, V=64,
                scale=1.0, in_dt=BF16, out_dt=BF16, cu=None, cu_host=None, h0=None, ht=None, pool=None,
                pool_slots=0, slots=None, stream=None)
    args.update(kw)
    a = args
    return _lib.lib().gdn_chunk_fwd_noalloc(a["q"], a["k"], a["v"], a["g"], a["beta"], a["o"], a["n_seqs"],
                                            a["total"], a["H"], a["K"], a["V"], a["scale"], a["in_dt"], a["out_dt"],
                                            a["cu"], a["cu_host"], a["h0"], a["ht"], a["pool"], a["pool_slots"],
                                            a["slots"], a["stream"])


def test_noalloc_rejects_before_touching_the_device():
    """Sizes whose workspace exceeds the library's device array are refused with
    GDN_EWORKSPACE, and invalid arguments with the same status as gdn_chunk_fwd,
    both before the array's device address is asked for (no GPU here)."""
    L = _lib.lib()
    big = dict(n_seqs=4, total=4 * 8192, H=32, K=128, V=128)
    assert L.gdn_chunk_fwd_workspace_bytes(4, 4 * 8192, 32, 128, 128, BF16) > _lib.GDN_NOALLOC_WORKSPACE_BYTES
    assert _noalloc(**big) == _lib.GDN_EWORKSPACE
    assert _noalloc(K=96) == _lib.GDN_EUNSUPPORTED
    assert _noalloc(H=0) == _lib.GDN_EINVAL
    assert _noalloc(q=None) == _lib.GDN_EINVAL
    assert _noalloc(in_dt=7) == _lib.GDN_EUNSUPPORTED


def test_kda_gate_validation():
    L = _lib.lib()
    EINVAL, EUNS = _lib.GDN_EINVAL, _lib.GDN_EUNSUPPORTED
    call = lambda **kw: L.gdn_kda_gate(kw.get("fa", FAKE), kw.get("fb", FAKE), kw.get("al", FAKE), kw.get("dt", FAKE),
                                       kw.get("lb", -5.0), kw.get("mode", 0), kw.get("g", FAKE), kw.get("raw", None),
                                       kw.get("N", 4), kw.get("H", 2), kw.get("K", 128), None)
    assert call(K=96) == EUNS
    assert call(mode=3) == EINVAL and call(mode=-1) == EINVAL
    assert call(H=0) == EINVAL and call(N=-1) == EINVAL
    assert call(lb=float("inf")) == EINVAL and call(lb=float("nan")) == EINVAL
    assert call(fa=None) == EINVAL and call(g=None) == EINVAL
    assert call(fa=FAKE + 8) == EINVAL and call(raw=FAKE + 1) == EINVAL
    assert call(N=2 ** 31 - 1, H=65535) == EINVAL  # the 1-D grid would exceed 2^31 - 1 workgroups
    assert call(N=0) == _lib.GDN_OK


def test_decode_prologue_verify_validation():
    L = _lib.lib()
    EINVAL, EUNS = _lib.GDN_EINVAL, _lib.GDN_EUNSUPPORTED

    def call(**kw):
        a = dict(x=FAKE, w=FAKE, bias=None, st=FAKE, pool=8, slots=FAKE, cols=4, acc=FAKE, braw=FAKE, q=FAKE, k=FAKE,
                 v=FAKE, beta=FAKE, N=2, T=4, H=2, D=128)
        a.update(kw)
        return L.gdn_decode_prologue_verify(a["x"], a["w"], a["bias"], a["st"], a["pool"], a["slots"], a["cols"],
                                            a["acc"], a["braw"], a["q"], a["k"], a["v"], a["beta"], a["N"], a["T"],
                                            a["H"], a["D"], None)
    assert call(D=96) == EUNS
    assert call(T=0) == EINVAL and call(T=9) == EINVAL and call(cols=3) == EINVAL
    assert call(acc=None) == EINVAL and call(pool=0) == EINVAL
    assert call(q=FAKE + 4) == EINVAL and call(st=FAKE + 1) == EINVAL
    assert call(N=0) == _lib.GDN_OK


def test_decode_layer_validation():
    L = _lib.lib()
    EINVAL, EUNS = _lib.GDN_EINVAL, _lib.GDN_EUNSUPPORTED

    def call(**kw):
        a = dict(x=FAKE, w=FAKE, bias=None, st=FAKE, cs=8, slots=FAKE, braw=FAKE, g=FAKE, kda=0, pool=FAKE, ps=8,
                 gate=FAKE, nw=FAKE, eps=1e-6, out=FAKE, od=BF16, N=2, H=2, D=128)
        a.update(kw)
        return L.gdn_decode_layer(a["x"], a["w"], a["bias"], a["st"], a["cs"], a["slots"], a["braw"], a["g"], a["kda"],
                                  a["pool"], a["ps"], a["gate"], a["nw"], a["eps"], a["out"], a["od"], a["N"], a["H"],
                                  a["D"], 1.0, None)
    assert call(D=96) == EUNS and call(od=7) == EUNS
    assert call(H=0) == EINVAL and call(eps=-1.0) == EINVAL and call(eps=float("nan")) == EINVAL
    assert call(gate=None) == EINVAL and call(pool=None) == EINVAL and call(cs=0) == EINVAL
    assert call(kda=1, g=FAKE + 4) == EINVAL and call(pool=FAKE + 4) == EINVAL
    assert call(N=0) == _lib.GDN_OK


def test_chunk_fwd_plan():
    """gdn_chunk_fwd_plan: the segment plan the host takes (64 chunks for 16 pairs in five
    segments, 13 + 13 x 3 + 12; one pass for many pairs and for float32 inputs) and
    workspace offsets consistent with gdn_chunk_fwd_workspace_bytes; invalid sizes and
    null outputs rejected. Host only."""
    plan = (ctypes.c_int32 * 3)()
    offs = (ctypes.c_int64 * 5)()
    L = _lib.lib()

    def call(n_seqs=1, total=4096, max_len=4096, H=16, K=128, V=128, dt=_lib.GDN_BF16, p=plan, o=offs):
        return L.gdn_chunk_fwd_plan(n_seqs, total, max_len, H, K, V, dt, p, o)

    assert call() == _lib.GDN_OK
    assert tuple(plan) == (5, 13, 13)
    nch = (4096 // 64 + 1) * 16  # chunk slots: total / 64 + n_seqs, per head
    af, pf, gx, seg_sum, seg_state = tuple(offs)
    assert af == 0 and pf == nch * 12288 and gx == 2 * nch * 12288 and seg_sum > gx + nch * 768
    assert seg_state - seg_sum == 16 * 3 * (128 + 128) * 128 * 4  # 16 pairs x 3 maps
    assert seg_state + 16 * 128 * 128 * 4 <= L.gdn_chunk_fwd_workspace_bytes(1, 4096, 16, 128, 128, _lib.GDN_BF16)
    assert call(n_seqs=4, total=4 * 8192, max_len=8192, H=32) == _lib.GDN_OK and tuple(plan) == (1, 0, 0)
    assert call(dt=_lib.GDN_F32) == _lib.GDN_OK and tuple(plan) == (1, 0, 0)
    assert call(total=64 * 11, max_len=64 * 11) == _lib.GDN_OK and tuple(plan) == (1, 0, 0)  # too short to split
    EINVAL = _lib.GDN_EINVAL
    assert call(max_len=4097) == EINVAL
    assert call(n_seqs=-1) == EINVAL
    assert call(H=0) == EINVAL
    assert call(H=65536) == EINVAL  # the limits of gdn_chunk_fwd
    assert call(total=2**31 - 1, max_len=4096) == EINVAL
    assert call(n_seqs=2**23, total=2**24, max_len=16, H=64) == EINVAL
    assert call(n_seqs=1, total=2**30, max_len=2**30, H=256) == EINVAL  # (chunk, head) count beyond prep's grid
    assert call(p=None) == EINVAL and call(o=None) == EINVAL
    assert call(K=96) == _lib.GDN_EUNSUPPORTED
