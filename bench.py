#!/usr/bin/env python3
"""Throughput of the gated delta rule on one MI355X.

A step is one chunked forward pass (gdn_chunk_fwd: the prep kernel for
recompute_w_u, then chunk_fwd_h fused with chunk_fwd_o, which at this shape runs
in the chunk-parallel form: segment 0's scan beside the later segments' state
maps, then the scan of the later segments) over one batch of
B=1, H=16, T=4096, K=V=128 bf16 inputs, already resident in device memory.
`value` is tokens over the wall time of the K timed steps (back to back, between
device synchronisations). Beside it, per call, HIP events recorded by the
library on its stream give the prep and h + o durations twice: warm (calls back
to back) and cold (a 512 MiB fill before each call evicts L2 and the 256 MiB
infinity cache), each as mean, median, p10 and p90.

The other chunk workloads (tiny float32; B=4 H=32 T=8192 with h0; 16 packed
sequences with a state pool) are timed the same way under "configs". The decode
step (gdn_recurrent_step, N=256 requests, H=32, K=V=128, a 512-slot float32
state pool) and the other kernels of the library are timed beside them, and
measurement probes give the peaks this GPU reaches (a bf16 MFMA loop, a 2 GiB
streaming copy and read) next to the published ones.

Prints one JSON line on stdout (everything else goes to stderr).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
       python bench.py --only chunk|chunk1|chunk3|chunk4|decode|kda|verify|fp8|layer|gate|chunk_kda|peaks|copy
                       --steps K
       (profiling runs)
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E, published
PEAK_FP32_TFLOPS = 157.3   # MI355X fp32, vector and dense MFMA alike, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic.json")
CSRC = os.path.join(ROOT, "linear_attention_sequence_recompute_amd", "csrc")

# chunk workload: B=1, H=16, T=4096, K=V=128, C=64
B, H, T, K, V, C = 1, 16, 4096, 128, 128, 64
# decode workload: N=256 requests, H=32, K=V=128, pool of 512 slots
DN, DH, DK, DV, DSLOTS = 256, 32, 128, 128, 512
# speculative-verify decode: 96 requests x 4 tokens over the same pool shape
VN, VT = 96, 4
# fp8 group quantisation: a [16384, 4096] float32 activation matrix, groups of 128
QR, QC, QG = 16384, 4096, 128


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_digest() -> str:
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def chunk_flops(lengths, H, K, V):
    """Algorithmic FLOPs of one call (the dense per-chunk tiles, as the WarpDrive
    page lists the products) over sequences of the given lengths. A chunk of n
    tokens (n = 64 but for a sequence's ragged last chunk) counts, per head,
    h: 2nKV (w h) + 2nKV (k^T v_gated); o: 2nKV (q h) + 2n^2 K (q k^T) + 2n^2 V
    (P v_new); prep: 2n^2 K (k k^T) + n^3 / 3 (solve) + 2n^2 V (u) + 2n^2 K (w).
    Returns (h + o, full forward)."""
    ho = full = 0
    for L in lengths:
        for c0 in range(0, int(L), C):
            n = min(C, int(L) - c0)
            h = 4 * n * K * V
            o = 2 * n * K * V + 2 * n * n * K + 2 * n * n * V
            prep = 2 * n * n * K + n ** 3 // 3 + 2 * n * n * V + 2 * n * n * K
            ho += H * (h + o)
            full += H * (h + o + prep)
    return ho, full


def decode_bytes(n_active: int) -> int:
    """Algorithmic HBM bytes of one decode step: each active (request, head) state
    page is read and written once; q, k, v, o in bf16; g, beta in fp32."""
    per = 2 * DV * DK * 4 + (2 * DK + DV) * 2 + 2 * 4 + DV * 2
    return n_active * DH * per


class HipEvents:
    """hipEvent_t handles from the HIP runtime torch loaded."""

    def __init__(self):
        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                m = re.search(r"(\S*libamdhip64\.so\S*)", line)
                if m:
                    path = m.group(1)
                    break
        self.hip = ctypes.CDLL(path or "libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        evs = []
        for _ in range(n):
            e = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
            evs.append(e.value)
        return evs

    def record(self, ev, stream):
        assert self.hip.hipEventRecord(ev, stream) == 0

    def ms(self, a, b):
        self.hip.hipEventSynchronize(b)
        out = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(out), a, b) == 0
        return float(out.value)

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(e)


def stats(xs):
    xs = sorted(xs)
    n = len(xs)
    return dict(mean=sum(xs) / n, median=xs[n // 2], p10=xs[int(0.1 * (n - 1))], p90=xs[int(0.9 * (n - 1))])


def traffic_for(*kernels: str):
    """HBM bytes per call of the named kernels (summed) from the committed PMC
    counter runs, or None when the kernels changed since the counters were
    taken or one of them was not recorded."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_digest") != source_digest():
        return None
    total = 0
    for kernel in kernels:
        k = rec.get("kernels", {}).get(kernel)
        if k is None or k.get("bytes_per_launch") is None:
            return None
        total += k["bytes_per_launch"]
    return total


# Chunk workloads: (label, lengths, H, K, V, input dtype, seed, h0 std, pool slots).
# Equal lengths run as [B, T, ...] tensors; unequal ones packed with cu_seqlens.
CHUNK_CONFIGS = {
    "chunk1": ("tiny chunked forward, B=1 H=1 T=256 K=V=64, float32 q/k/v/o, h0 = 0", [256], 1, 64, 64, "f32", 1,
               None, None),
    "chunk": ("chunked GatedDeltaNet forward, B=1 H=16 T=4096 K=V=128 C=64, bf16 q/k/v, fp32 beta/g, o bf16 + "
              "final state fp32", [T] * B, H, K, V, "bf16", 2, None, None),
    "chunk3": ("long/batched chunked forward, B=4 H=32 T=8192 K=V=128, bf16 q/k/v/o, h0 ~ N(0, 0.1^2) fp32, "
               "final state fp32", [8192] * 4, 32, 128, 128, "bf16", 3, 0.1, None),
    "chunk4": ("variable-length packed prefill, 16 sequences of uniform [100, 6000] tokens (60217 in all), H=16 "
               "K=V=128, bf16 q/k/v/o, states read from and written to a 17-slot fp32 pool", "varlen", 16, 128, 128,
               "bf16", 4, None, 17),
}


def chunk_workload(name):
    from linear_attention_sequence_recompute_amd.workloads import chunk_inputs, varlen_lengths

    label, lengths, h, k, v, dtype, seed, h0_std, pool = CHUNK_CONFIGS[name]
    if lengths == "varlen":
        lengths = [int(x) for x in varlen_lengths(16, 100, 6000, seed=4)]
    ci = chunk_inputs(lengths, h, k, v, dtype=dtype, seed=seed, h0_std=h0_std, pool_slots=pool)
    return label, ci


def bench_chunk(torch, api, hev, steps, warmup, name="chunk", flush_bytes=512 << 20, before=None):
    """Warm wall time of `steps` back-to-back calls, then per-call events warm and
    cold (caches flushed before every call). `before` (optional) runs once with
    the inputs resident, before the warmup; its result is returned as _before."""
    label, ci = chunk_workload(name)
    dev = torch.device("cuda")
    dt = torch.bfloat16 if ci.dtype == "bf16" else torch.float32
    Hh, Kk = ci.q.shape[1:]
    Vv = ci.v.shape[-1]
    lengths = np.diff(ci.cu_seqlens).tolist()
    n = ci.n_seqs

    def t(x, d):
        x = torch.from_numpy(np.ascontiguousarray(x)).to(d).to(dev)
        return x.view(n, -1, *x.shape[1:]) if ci.equal_length else x

    q, k, v = (t(x, dt) for x in (ci.q, ci.k, ci.v))
    g, b = t(ci.a, torch.float32), t(ci.beta, torch.float32)
    o = torch.empty(v.shape, dtype=dt, device=dev)
    kw = {}
    if ci.pool is not None:
        kw["state_pool"] = torch.from_numpy(ci.pool).float().to(dev)
        kw["state_slots"] = torch.from_numpy(ci.slots).int().to(dev)
    else:
        kw["ht"] = torch.empty(n, Hh, Vv, Kk, dtype=torch.float32, device=dev)
        if ci.h0 is not None:
            kw["h0"] = torch.from_numpy(ci.h0).float().to(dev)
    if not ci.equal_length:
        kw["cu_seqlens"] = ci.cu_seqlens.tolist()
        kw["cu_seqlens_dev"] = torch.from_numpy(ci.cu_seqlens).int().to(dev)
    del ci
    ws = torch.empty(api.workspace_bytes(n, int(sum(lengths)), Hh, Kk, Vv, dt), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    scale = Kk ** -0.5

    def step(evs=None):
        api.chunk_fwd(q, k, v, g, b, scale=scale, out=o, workspace=ws, stream=stream, events=evs, **kw)

    # work to run with the inputs resident, right before the warmup
    before_res = before() if before is not None else None
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    # the timed steps: plain calls (events between the two kernels cost about
    # 10 us per call, so per-kernel durations come from the next loops)
    t0 = time.perf_counter()
    for i in range(steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # per-part durations: as many calls again, with HIP events the library
    # records on the launch stream before prep, between the kernels and after scan
    evs = [hev.create(3) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    warm = dict(prep_us=stats([1e3 * hev.ms(e[0], e[1]) for e in evs]),
                h_o_us=stats([1e3 * hev.ms(e[1], e[2]) for e in evs]),
                call_us=stats([1e3 * hev.ms(e[0], e[2]) for e in evs]))

    # the same with L2 and the 256 MiB infinity cache flushed before every call
    flush = torch.empty(flush_bytes, dtype=torch.uint8, device=dev)
    cp, cs, cc = [], [], []
    for i in range(steps):
        flush.fill_(i & 0xFF)
        step(evs[i])
        torch.cuda.synchronize()
        cp.append(1e3 * hev.ms(evs[i][0], evs[i][1]))
        cs.append(1e3 * hev.ms(evs[i][1], evs[i][2]))
        cc.append(1e3 * hev.ms(evs[i][0], evs[i][2]))
    for e in evs:
        hev.destroy(e)
    del flush
    cold = dict(prep_us=stats(cp), h_o_us=stats(cs), call_us=stats(cc))
    return dict(label=label, lengths=lengths, H=Hh, K=Kk, V=Vv, dtype=dt, wall_s=wall, warm=warm, cold=cold,
                _before=before_res)


def chunk_entry(res, steps, peaks):
    """JSON entry of a chunk workload: tokens/s (warm wall time, warm and cold
    events), per-part times and the h + o roofline against the bf16 MFMA peak
    (float32 inputs run on the fp32 MFMA and are priced against its peak)."""
    tokens = int(sum(res["lengths"]))
    f_ho, f_full = chunk_flops(res["lengths"], res["H"], res["K"], res["V"])
    bf16 = res["dtype"] is not None and str(res["dtype"]).endswith("bfloat16")
    peak = PEAK_BF16_TFLOPS if bf16 else PEAK_FP32_TFLOPS
    ho_w, ho_c = res["warm"]["h_o_us"]["mean"], res["cold"]["h_o_us"]["mean"]
    ach_w, ach_c = f_ho / ho_w / 1e6, f_ho / ho_c / 1e6
    ms = 1e3 * res["wall_s"] / steps
    entry = {
        "workload": res["label"],
        "value": tokens / (ms / 1e3), "unit": "tokens/s", "ms_per_step": ms,
        "value_cold": tokens / (res["cold"]["call_us"]["mean"] / 1e6),
        "timing_us": {"warm": res["warm"], "cold": res["cold"]},
        "roofline": {"bound": "mfma", "achieved": ach_w, "peak": peak, "unit": "TFLOP/s", "frac": ach_w / peak,
                     "cold_achieved": ach_c, "cold_frac": ach_c / peak, "flops_per_launch": f_ho,
                     "avg_launch_us": ho_w},
        "full_fwd_tflops": f_full / (ms / 1e3) / 1e12,
    }
    if bf16 and peaks and peaks.get("mfma_bf16_tflops"):
        entry["roofline"]["frac_of_measured_peak"] = ach_w / peaks["mfma_bf16_tflops"]
    return entry


def kda_chunk_flops():
    """Algorithmic flops per call of the chunk form with per-channel decays at the
    chunk workload's shape. Scan, per (chunk, head, value column): (K o e^G) h,
    (s q o e^G) h and (K o e^{G_last - G})^T D, 64 K multiply-adds each, and
    A' R and P D, 64 * 64 each. Prep, per (chunk, head): 2080 token pairs x K
    channels (one exponent, three multiply-adds), the substitution 64 * 2016
    multiply-adds, and the three scaled operands (64 K, two exponents)."""
    nch = B * (T // C) * H
    scan = nch * V * 2 * (3 * C * K + 2 * C * C)
    prep = nch * (2080 * K * 7 + 2 * C * 2016 + C * K * 5)
    return scan, prep


def bench_chunk_kda(torch, api, hev, steps, warmup):
    """The chunk form with a decay per key channel at the chunk workload's shape:
    B=1, H=16, T=4096, K=V=128, bf16 in and out, per-channel log-decays."""
    from linear_attention_sequence_recompute_amd.workloads import channel_log_decay, chunk_inputs

    ci = chunk_inputs([T] * B, H, K, V, dtype="bf16", seed=2)
    dev = torch.device("cuda")

    def t(x, dt):
        return torch.from_numpy(x).to(dt).to(dev).view(B, T, *x.shape[1:])

    q, k, v = (t(x, torch.bfloat16) for x in (ci.q, ci.k, ci.v))
    g = t(channel_log_decay((B * T, H, K), 3), torch.float32)
    b = t(ci.beta, torch.float32)
    o = torch.empty(B, T, H, V, dtype=torch.bfloat16, device=dev)
    ht = torch.empty(B, H, V, K, dtype=torch.float32, device=dev)
    ws = torch.empty(int(api._lib.lib().gdn_chunk_fwd_kda_workspace_bytes(B, T, H, K)), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream()

    def step(evs=None):
        api.chunk_fwd_kda(q, k, v, g, b, scale=K ** -0.5, out=o, ht=ht, workspace=ws, stream=stream, events=evs)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    evs = [hev.create(3) for _ in range(steps)]
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    prep = [hev.ms(e[0], e[1]) for e in evs]
    scan = [hev.ms(e[1], e[2]) for e in evs]
    for e in evs:
        hev.destroy(e)
    return dict(wall_s=wall, prep_ms=stats(prep), scan_ms=stats(scan))


def bench_decode(torch, api, hev, steps, warmup):
    from linear_attention_sequence_recompute_amd.workloads import decode_inputs

    di = decode_inputs(DN, DH, DK, DV, DSLOTS, dtype="bf16", seed=5, n_padding=0)
    dev = torch.device("cuda")
    q, k, v = (torch.from_numpy(x).to(torch.bfloat16).to(dev) for x in (di.q, di.k, di.v))
    g, b = (torch.from_numpy(x).float().to(dev) for x in (di.a, di.beta))
    pool = torch.from_numpy(di.pool).float().to(dev)
    slots = torch.from_numpy(di.slots).int().to(dev)
    o = torch.empty(DN, DH, DV, dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    scale = DK ** -0.5

    def step():
        api.recurrent_step(q, k, v, g, b, pool, slots, scale=scale, out=o, stream=stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [hev.create(2) for _ in range(steps)]
    s = stream.cuda_stream
    t0 = time.perf_counter()
    for i in range(steps):
        hev.record(evs[i][0], s)
        step()
        hev.record(evs[i][1], s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = [hev.ms(e[0], e[1]) for e in evs]
    for e in evs:
        hev.destroy(e)
    return dict(wall_s=wall, kernel_ms=stats(ms), n_active=int((di.slots > 0).sum()), _inputs=di)


def bench_decode_kda(torch, api, hev, steps, warmup):
    """The decode workload with a log-decay per key channel (g [N, H, K])."""
    from linear_attention_sequence_recompute_amd.workloads import channel_log_decay, decode_inputs

    di = decode_inputs(DN, DH, DK, DV, DSLOTS, dtype="bf16", seed=5, n_padding=0)
    dev = torch.device("cuda")
    q, k, v = (torch.from_numpy(x).to(torch.bfloat16).to(dev) for x in (di.q, di.k, di.v))
    g = torch.from_numpy(channel_log_decay((DN, DH, DK), seed=6)).float().to(dev)
    b = torch.from_numpy(di.beta).float().to(dev)
    pool = torch.from_numpy(di.pool).float().to(dev)
    slots = torch.from_numpy(di.slots).int().to(dev)
    o = torch.empty(DN, DH, DV, dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        api.recurrent_step_kda(q, k, v, g, b, pool, slots, scale=DK ** -0.5, out=o, stream=stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [hev.create(2) for _ in range(steps)]
    s = stream.cuda_stream
    for i in range(steps):
        hev.record(evs[i][0], s)
        step()
        hev.record(evs[i][1], s)
    torch.cuda.synchronize()
    ms = [hev.ms(e[0], e[1]) for e in evs]
    for e in evs:
        hev.destroy(e)
    return dict(kernel_ms=stats(ms), n_active=int((di.slots > 0).sum()))


def verify_bytes(n_active: int, T: int) -> int:
    """Algorithmic HBM bytes of one verify call: per active (request, head) the
    source state is read once and T states are written; q, k, v, o in bf16 and
    g, beta in fp32 for each token."""
    per = (1 + T) * DV * DK * 4 + T * ((2 * DK + DV) * 2 + 2 * 4 + DV * 2)
    return n_active * DH * per


def bench_verify(torch, api, hev, steps, warmup):
    """Speculative-verify decode: VN requests x VT tokens over the decode pool."""
    from linear_attention_sequence_recompute_amd.workloads import verify_inputs

    vi = verify_inputs(VN, VT, DH, DK, DV, DSLOTS, dtype="bf16", seed=8)
    dev = torch.device("cuda")
    q, k, v = (torch.from_numpy(x).to(torch.bfloat16).to(dev) for x in (vi.q, vi.k, vi.v))
    g, b = (torch.from_numpy(x).float().to(dev) for x in (vi.a, vi.beta))
    pool = torch.from_numpy(vi.pool).float().to(dev)
    slots = torch.from_numpy(vi.slots).int().to(dev)
    accepted = torch.from_numpy(vi.accepted).int().to(dev)
    o = torch.empty(VN, VT, DH, DV, dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        api.recurrent_verify(q, k, v, g, b, pool, slots, accepted, scale=DK ** -0.5, out=o, stream=stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [hev.create(2) for _ in range(steps)]
    s = stream.cuda_stream
    for i in range(steps):
        hev.record(evs[i][0], s)
        step()
        hev.record(evs[i][1], s)
    torch.cuda.synchronize()
    ms = [hev.ms(e[0], e[1]) for e in evs]
    for e in evs:
        hev.destroy(e)
    return dict(kernel_ms=stats(ms), n_active=VN)


def bench_fp8(torch, api, hev, steps, warmup):
    """fp8 group quantisation of a [QR, QC] float32 activation matrix, groups of QG."""
    dev = torch.device("cuda")
    g = torch.Generator(device=dev).manual_seed(9)
    x = torch.randn(QR, QC, device=dev, generator=g)
    codes = torch.empty(QR, QC, dtype=torch.uint8, device=dev)
    scales = torch.empty(QR, QC // QG, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        api.fp8_quant(x, QG, codes=codes, scales=scales, stream=stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [hev.create(2) for _ in range(steps)]
    s = stream.cuda_stream
    for i in range(steps):
        hev.record(evs[i][0], s)
        step()
        hev.record(evs[i][1], s)
    torch.cuda.synchronize()
    ms = [hev.ms(e[0], e[1]) for e in evs]
    for e in evs:
        hev.destroy(e)
    return dict(kernel_ms=stats(ms))


def bench_gate(torch, api, hev, steps, warmup):
    """The KDA gate stage for N=DN tokens, H=DH heads, K=DK channels, each mode."""
    from linear_attention_sequence_recompute_amd.workloads import gate_inputs

    gi = gate_inputs(DN, DH, DK, seed=14)
    dev = torch.device("cuda")
    t = lambda x, d: torch.from_numpy(x).to(d).to(dev)
    f_a, f_b, a_log, dt = t(gi.f_a, torch.bfloat16), t(gi.f_b, torch.bfloat16), t(gi.a_log, torch.float32), \
        t(gi.dt_bias, torch.float32)
    g = torch.empty(DN, DH, DK, device=dev)
    stream = torch.cuda.current_stream()
    s = stream.cuda_stream
    out = {}
    for mode in (0, 1, 2):
        def step():
            api.kda_gate(f_a, f_b, a_log, dt, gi.lower_bound, DH, mode=mode, out=g, stream=stream)
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        evs = [hev.create(2) for _ in range(steps)]
        for i in range(steps):
            hev.record(evs[i][0], s)
            step()
            hev.record(evs[i][1], s)
        torch.cuda.synchronize()
        out[f"mode{mode}_ms"] = stats([hev.ms(e[0], e[1]) for e in evs])
        for e in evs:
            hev.destroy(e)
    return out


def layer_bytes():
    """Algorithmic bytes of the decode layer's front and back operations at
    N=DN requests, H=DH heads of DK channels (all active): each input and output
    element moved once, the conv state read and written once."""
    dim = DH * DK
    pro = (DN * 3 * dim * 2 + 2 * DN * 3 * dim * 3 * 2 + (3 * 4 * dim + 3 * dim) * 4 + DN * DH * 4
           + DN * 3 * dim * 4 + DN * DH * 4)
    rms = DN * dim * 4 + DN * dim * 2 + DK * 4 + DN * dim * 2
    return pro, rms


def bench_layer(torch, api, hev, steps, warmup):
    """Decode layer front (conv + SiLU + norms + beta) and back (gated RMSNorm)
    operations for N=DN requests, H=DH heads of DK channels, a conv-state pool of
    DSLOTS slots."""
    dev = torch.device("cuda")
    g = torch.Generator(device=dev).manual_seed(13)
    dim = DH * DK
    x = torch.randn(DN, 3 * dim, device=dev, generator=g).to(torch.bfloat16)
    w = torch.rand(3, 4, dim, device=dev, generator=g) - 0.5
    bias = torch.rand(3 * dim, device=dev, generator=g) - 0.5
    conv = torch.randn(DSLOTS, 3 * dim, 3, device=dev, generator=g).to(torch.bfloat16)
    slots = (torch.randperm(DSLOTS - 1, device=dev, generator=g)[:DN] + 1).to(torch.int32)
    braw = torch.randn(DN, DH, device=dev, generator=g)
    o = torch.randn(DN, DH, DK, device=dev, generator=g)
    gate = torch.randn(DN, dim, device=dev, generator=g).to(torch.bfloat16)
    nw = torch.ones(DK, device=dev)
    out = torch.empty(DN, DH, DK, dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()

    def pro():
        api.decode_prologue(x, w, bias, conv, slots, braw, DH, stream=stream)

    def rms():
        api.gated_rmsnorm(o, gate, nw, 1e-6, out=out, stream=stream)

    for _ in range(warmup):
        pro()
        rms()
    torch.cuda.synchronize()
    evs = [hev.create(4) for _ in range(steps)]
    s = stream.cuda_stream
    for i in range(steps):
        hev.record(evs[i][0], s)
        pro()
        hev.record(evs[i][1], s)
        hev.record(evs[i][2], s)
        rms()
        hev.record(evs[i][3], s)
    torch.cuda.synchronize()
    ms_p = [hev.ms(e[0], e[1]) for e in evs]
    ms_r = [hev.ms(e[2], e[3]) for e in evs]
    for e in evs:
        hev.destroy(e)
    # the whole layer: separate launches (front, decode step, RMSNorm) against
    # the fused one, on the same inputs and a pool of DSLOTS states
    pool = torch.randn(DSLOTS, DH, DK, DK, device=dev, generator=g) * 0.1
    lg = -torch.nn.functional.softplus(torch.randn(DN, DH, device=dev, generator=g) + 2.0)
    out32 = torch.empty(DN, DH, DK, dtype=torch.float32, device=dev)

    def separate():
        q, k, v, beta = api.decode_prologue(x, w, bias, conv, slots, braw, DH, stream=stream)
        api.recurrent_step(q, k, v, lg, beta, pool, slots, scale=DK ** -0.5, out=out32, stream=stream)
        api.gated_rmsnorm(out32, gate, nw, 1e-6, out=out, stream=stream)

    def fused():
        api.decode_layer(x, w, bias, conv, slots, braw, lg, pool, DH, gate=gate, norm_w=nw, out=out, stream=stream)

    # the layer with per-key-channel decays from the gate's projection: the gate
    # stage, then the fused layer on its decays
    f_a = torch.randn(DN, 128, device=dev, generator=g).to(torch.bfloat16)
    f_b = (torch.randn(DH * DK, 128, device=dev, generator=g) * 128 ** -0.5).to(torch.bfloat16)
    a_log = torch.rand(DH, device=dev, generator=g) * 2.5 - 2.0
    dt = torch.randn(DH * DK, device=dev, generator=g)
    g_kda = torch.empty(DN, DH, DK, device=dev)

    def gate_then_fused():
        api.kda_gate(f_a, f_b, a_log, dt, -5.0, DH, mode=1, out=g_kda, stream=stream)
        api.decode_layer(x, w, bias, conv, slots, braw, g_kda, pool, DH, gate=gate, norm_w=nw, out=out, stream=stream)


    res = {}
    for name, fn in (("separate", separate), ("fused", fused), ("kda_gate_then_fused", gate_then_fused)):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        evs = [hev.create(2) for _ in range(steps)]
        for i in range(steps):
            hev.record(evs[i][0], s)
            fn()
            hev.record(evs[i][1], s)
        torch.cuda.synchronize()
        res[name] = stats([hev.ms(e[0], e[1]) for e in evs])
        for e in evs:
            hev.destroy(e)
    return dict(prologue_ms=stats(ms_p), rmsnorm_ms=stats(ms_r), layer_separate_ms=res["separate"],
                layer_fused_ms=res["fused"], layer_kda_gate_then_fused_ms=res["kda_gate_then_fused"])


def bench_copy(torch, steps, nbytes=1 << 30):
    """A plain device copy of known size: the calibration kernel for PMC byte
    counters (FETCH_SIZE and WRITE_SIZE of this launch should read nbytes each)."""
    x = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    x.fill_(1)
    y = torch.empty_like(x)
    for _ in range(steps):
        y.copy_(x)
    torch.cuda.synchronize()
    return nbytes


def bench_peaks(torch, api, hev, reps=5, nbytes=2 << 30):
    """The peaks this GPU reaches, from the library's measurement probes: a bf16
    MFMA loop over every SIMD (2 waves each, 8 independent accumulators per
    wave), a streaming copy, read and write of 2 GiB each."""
    L = api._lib.lib()
    stream = torch.cuda.current_stream().cuda_stream
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    waves, iters = cus * 4 * 2, 4096
    sink = torch.empty(max(waves * 64, 8192), dtype=torch.float32, device="cuda")
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        evs = [hev.create(2) for _ in range(reps)]
        for e in evs:
            hev.record(e[0], stream)
            fn()
            hev.record(e[1], stream)
        torch.cuda.synchronize()
        ms = [hev.ms(e[0], e[1]) for e in evs]
        for e in evs:
            hev.destroy(e)
        return stats(ms)["median"] / 1e3

    def ok(st):
        assert st == 0, api._lib.status_string(st)

    t_mfma = timed(lambda: ok(L.gdn_probe_mfma_bf16(sink.data_ptr(), waves, iters, stream)))
    t_copy = timed(lambda: ok(L.gdn_probe_copy(src.data_ptr(), dst.data_ptr(), nbytes, stream)))
    t_read = timed(lambda: ok(L.gdn_probe_read(src.data_ptr(), sink.data_ptr(), nbytes, stream)))
    t_write = timed(lambda: ok(L.gdn_probe_write(dst.data_ptr(), nbytes, stream)))
    del src, dst
    flops = waves * iters * 8 * 16384
    return {"mfma_bf16_tflops": flops / t_mfma / 1e12, "copy_gbs": 2 * nbytes / t_copy / 1e9,
            "read_gbs": nbytes / t_read / 1e9, "write_gbs": nbytes / t_write / 1e9,
            "probes": f"bf16 MFMA loop: {waves} waves x {iters} x 8 v_mfma_f32_16x16x32_bf16; copy, read and write "
                      f"of {nbytes >> 30} GiB (copy counts bytes read + written); median of {reps}"}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(min_seconds=10.0, decode_in=None):
    """The fp64 oracle on the host cores, each leg on a bounded sample:
    the chunked WY form (O2) over repeated full passes of the B=1, H=16, T=4096
    workload until min_seconds have elapsed (the headline value); the naive
    per-token recurrence (O1) over the tiny workload (repeated for a second) and
    one full pass of the H=16, T=4096 workload; the decode step (O3) over the
    N=256, H=32 decode workload once (GB/s of the same algorithmic bytes as the
    GPU's)."""
    import oracle
    from linear_attention_sequence_recompute_amd.workloads import chunk_inputs

    affinity = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    ci = chunk_inputs([T], H, K, V, dtype="bf16", seed=2)
    n_tok = passes = 0
    t0 = time.perf_counter()
    while True:
        oracle.chunked_fwd(ci.q, ci.k, ci.v, ci.a, ci.beta, scale=K ** -0.5)
        n_tok += T
        passes += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    dt = time.perf_counter() - t0
    extra = {}
    t1 = time.perf_counter()
    oracle.recurrent_fwd(ci.q, ci.k, ci.v, ci.a, ci.beta, scale=K ** -0.5)
    extra["o1_naive_h16_t4096_tokens_per_s"] = T / (time.perf_counter() - t1)
    tiny = chunk_inputs([256], 1, 64, 64, dtype="f32", seed=1)
    n1 = 0
    t1 = time.perf_counter()
    while time.perf_counter() - t1 < 1.0:
        oracle.recurrent_fwd(tiny.q, tiny.k, tiny.v, tiny.a, tiny.beta, scale=1.0)
        n1 += 256
    extra["o1_naive_tiny_tokens_per_s"] = n1 / (time.perf_counter() - t1)
    if decode_in is not None:
        di = decode_in
        t1 = time.perf_counter()
        oracle.decode_step(di.q, di.k, di.v, di.a, di.beta, di.pool, di.slots, scale=DK ** -0.5)
        dt3 = time.perf_counter() - t1
        extra["o3_decode_gbs"] = decode_bytes(int((di.slots > 0).sum())) / dt3 / 1e9
        extra["o3_decode_s"] = dt3
    return dict(value=n_tok / dt, unit="tokens/s", cores=int(threads), kind="oracle",
                sample=f"{passes} full passes of the B=1 H=16 T=4096 K=V=128 workload through the fp64 chunked "
                       f"oracle (numpy, {threads} BLAS threads) in {dt:.1f} s; O1 and O3 legs as in 'extra'",
                cpu_model=cpu_model(), affinity_cores=affinity, blas_threads=int(threads), extra=extra)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", choices=["all", "chunk", "chunk1", "chunk3", "chunk4", "decode", "kda", "verify", "fp8",
                                       "layer", "gate", "chunk_kda", "peaks", "copy"], default="all")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the chunked forward and the decode step need no "
              f"communication, and the library runs each call on a single MI355X (asked for --gpus "
              f"{args.gpus}, WORLD_SIZE={world}).", file=sys.stderr)
        sys.exit(2)

    import torch

    from linear_attention_sequence_recompute_amd import api

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    hev = HipEvents()

    if args.only == "copy":
        n = bench_copy(torch, args.steps)
        log(f"copied {n} bytes x {args.steps}")
        return
    only = args.only
    res = {}

    def run(name, fn, msg):
        if only in ("all", name):
            log(msg + " ...")
            res[name] = fn()
            log(json.dumps({k: v for k, v in res[name].items() if not k.startswith("_")}, default=str))

    run("peaks", lambda: bench_peaks(torch, api, hev), "measured peaks: bf16 MFMA loop, 2 GiB copy and read")

    def other_chunks():
        for name in ("chunk1", "chunk3", "chunk4"):
            run(name, lambda name=name: bench_chunk(torch, api, hev, args.steps, args.warmup, name),
                f"{name}: {CHUNK_CONFIGS[name][0]}")

    # In the full run the other chunk workloads are measured between building the
    # headline's inputs and its warmup steps, so that the headline's timed calls
    # follow sustained chunk work, as they would in a prefill loop, rather than
    # the idle host time of building the inputs (the GPU takes some 30 ms of this
    # load to reach its working clock: the first 50 calls after a second idle
    # average about 80 us, later ones 67 us).
    run("chunk", lambda: bench_chunk(torch, api, hev, args.steps, args.warmup, "chunk",
                                     before=other_chunks if only == "all" else None),
        f"chunk: {CHUNK_CONFIGS['chunk'][0]}")
    if only != "all":
        other_chunks()
    run("decode", lambda: bench_decode(torch, api, hev, args.steps, args.warmup), "decode: N=256 H=32 K=V=128 pool=512")
    run("kda", lambda: bench_decode_kda(torch, api, hev, args.steps, args.warmup),
        "decode with per-key-channel decay: N=256 H=32 K=V=128 pool=512")
    run("verify", lambda: bench_verify(torch, api, hev, args.steps, args.warmup),
        f"verify decode: N={VN} T={VT} H=32 K=V=128 pool=512")
    run("fp8", lambda: bench_fp8(torch, api, hev, args.steps, args.warmup), f"fp8 quant: [{QR}, {QC}] float32, "
        f"groups of {QG}")
    run("layer", lambda: bench_layer(torch, api, hev, args.steps, args.warmup),
        f"decode layer front/back: N={DN} H={DH} D={DK} conv pool={DSLOTS}")
    run("gate", lambda: bench_gate(torch, api, hev, args.steps, args.warmup),
        f"KDA gate stage: N={DN} H={DH} K={DK}, rank 128, modes 0-2")
    run("chunk_kda", lambda: bench_chunk_kda(torch, api, hev, args.steps, args.warmup),
        "chunk form with per-channel decays: B=1 H=16 T=4096 K=V=128 bf16")
    if only != "all":
        return

    peaks = res["peaks"]
    head = chunk_entry(res["chunk"], args.steps, peaks)
    head["roofline"]["kernel"] = ("chunk_fwd_h fused with chunk_fwd_o: seg0_kernel (segment 0's scan beside the "
                                  "maps of segments 1-3) + scan_kernel (segments 1-4); the chunk-parallel form at "
                                  "this shape, 5 segments of 4 x 13 + 12 chunks")
    head["roofline"]["traffic"] = traffic_for("seg0_kernel", "scan_kernel")
    res_d = res["decode"]
    dec_s = res_d["kernel_ms"]["mean"] / 1e3
    dec_b = decode_bytes(res_d["n_active"])
    dec_gbs = dec_b / dec_s / 1e9

    def hbm_roofline(achieved_gbs, kernel_traffic, nbytes, write_bytes=None):
        """HBM roofline entry; with the bytes written known, also the ceiling the
        measured streaming read and write rates give for that read/write mix
        (read bytes at the read rate, then written bytes at the write rate)."""
        r = {"bound": "hbm", "achieved": achieved_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
             "frac": achieved_gbs / PEAK_HBM_GBS, "frac_of_measured_copy": achieved_gbs / peaks["copy_gbs"],
             "traffic": kernel_traffic, "bytes_per_launch": nbytes}
        if write_bytes is not None:
            rd = nbytes - write_bytes
            mix = nbytes / (rd / peaks["read_gbs"] + write_bytes / peaks["write_gbs"])
            r.update(write_bytes=write_bytes, measured_mix_ceiling_gbs=mix, frac_of_measured_mix=achieved_gbs / mix)
        return r

    out = {
        "metric": "GDN fwd tokens/s + % bf16 MFMA peak (H16,K=V=128,T4096); decode GB/s % peak",
        "value": head["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": head["workload"], "global_batch": B, "seq_len": T, "heads": H, "head_dim": K,
                   "chunk": C, "parallelism": "single GPU"},
        "value_cold": head["value_cold"],
        "timing_us": head["timing_us"],
        "roofline": head["roofline"],
        "full_fwd_tflops": head["full_fwd_tflops"],
        "measured_peaks": peaks,
        "configs": {"tiny_f32": chunk_entry(res["chunk1"], args.steps, peaks),
                    "batched_long": chunk_entry(res["chunk3"], args.steps, peaks),
                    "varlen_pool": chunk_entry(res["chunk4"], args.steps, peaks)},
        "decode": {"workload": "recurrent decode step, N=256 requests (all active), H=32, K=V=128, "
                               "pool [512, 32, 128, 128] fp32, bf16 q/k/v/o",
                   "value": dec_gbs, "unit": "GB/s", "avg_launch_us": dec_s * 1e6,
                   "timing_us": {k: v * 1e3 for k, v in res_d["kernel_ms"].items()},
                   "roofline": hbm_roofline(dec_gbs, traffic_for("recurrent_step_kernel"), dec_b,
                                            res_d["n_active"] * DH * (DV * DK * 4 + DV * 2))},
    }
    res_k = res["kda"]
    kda_s = res_k["kernel_ms"]["mean"] / 1e3
    kda_b = decode_bytes(res_k["n_active"]) + res_k["n_active"] * DH * (DK - 1) * 4  # g per key channel
    out["decode_kda"] = {
        "workload": "recurrent decode step with a log-decay per key channel, N=256 requests (all active), H=32, "
                    "K=V=128, pool [512, 32, 128, 128] fp32, bf16 q/k/v/o",
        "value": kda_b / kda_s / 1e9, "unit": "GB/s", "avg_launch_us": kda_s * 1e6,
        "roofline": hbm_roofline(kda_b / kda_s / 1e9, traffic_for("recurrent_step_kernel_kda"), kda_b)}
    res_v = res["verify"]
    ver_s = res_v["kernel_ms"]["mean"] / 1e3
    ver_b = verify_bytes(res_v["n_active"], VT)
    out["decode_verify"] = {
        "workload": f"speculative-verify decode, {VN} requests x {VT} tokens, H=32, K=V=128, pool [512, 32, 128, 128] "
                    "fp32 (source read once, a state written per token), bf16 q/k/v/o",
        "value": ver_b / ver_s / 1e9, "unit": "GB/s", "avg_launch_us": ver_s * 1e6,
        "tokens_per_s": VN * VT / ver_s,
        "roofline": hbm_roofline(ver_b / ver_s / 1e9, traffic_for("recurrent_verify_kernel"), ver_b,
                                 res_v["n_active"] * DH * VT * (DV * DK * 4 + DV * 2))}
    q_s = res["fp8"]["kernel_ms"]["mean"] / 1e3
    q_b = QR * QC * (4 + 1) + QR * (QC // QG) * 4
    out["fp8_quant"] = {
        "workload": f"fp8 group quantisation, [{QR}, {QC}] float32 activations, groups of {QG}, E4M3 codes + "
                    "float32 scales",
        "value": q_b / q_s / 1e9, "unit": "GB/s", "avg_launch_us": q_s * 1e6,
        "roofline": hbm_roofline(q_b / q_s / 1e9, traffic_for("fp8_quant_kernel"), q_b)}
    lp_b, lr_b = layer_bytes()
    res_l = res["layer"]
    lp_s, lr_s = res_l["prologue_ms"]["mean"] / 1e3, res_l["rmsnorm_ms"]["mean"] / 1e3
    out["decode_layer"] = {
        "workload": f"decode layer front (4-tap conv over a bf16 conv-state pool of {DSLOTS} slots, SiLU, q/k L2 "
                    f"norm, sigmoid beta) and back (gated RMSNorm, bf16 out), N={DN} requests, H={DH}, D={DK}",
        "prologue": {"avg_launch_us": lp_s * 1e6, "bytes_per_launch": lp_b,
                     "roofline": hbm_roofline(lp_b / lp_s / 1e9, traffic_for("decode_prologue_kernel"), lp_b)},
        "gated_rmsnorm": {"avg_launch_us": lr_s * 1e6, "bytes_per_launch": lr_b,
                          "roofline": hbm_roofline(lr_b / lr_s / 1e9, traffic_for("gated_rmsnorm_kernel"), lr_b)}}
    lf_s = res_l["layer_fused_ms"]["mean"] / 1e3
    # the fused layer's algorithmic bytes: the decode step's (q, k, v not read) plus the front's x, conv state read and
    # written, weights, beta_raw and the RMSNorm's gate and weights
    lf_b = dec_b - DN * DH * (2 * DK + DV) * 2 + DN * 3 * DH * DK * 2 + 2 * DN * 3 * DH * DK * 3 * 2 \
        + (3 * 4 * DH * DK + 3 * DH * DK) * 4 + DN * DH * 4 + DN * DH * DK * 2 + DK * 4
    out["decode_layer"]["layer"] = {
        "workload": f"the whole decode layer (front, decode step with a scalar gate, gated RMSNorm), N={DN} H={DH} "
                    f"D={DK}, state pool {DSLOTS} slots",
        "separate_launches_us": res_l["layer_separate_ms"]["mean"] * 1e3,
        "fused_us": lf_s * 1e6, "bytes_per_launch": lf_b,
        "roofline": hbm_roofline(lf_b / lf_s / 1e9, traffic_for("decode_layer_kernel"), lf_b)}
    out["decode_layer"]["layer_kda_gate"] = {
        "workload": f"the decode layer with per-key-channel decays from the gate's rank-128 projection (mode 1): "
                    f"the gate stage, then the fused layer on its decays, N={DN} H={DH} D={DK}, state pool {DSLOTS} "
                    f"slots",
        "gate_stage_then_fused_us": res_l["layer_kda_gate_then_fused_ms"]["mean"] * 1e3}
    gate_flops = 2 * DN * DH * DK * 128
    out["kda_gate"] = {
        "workload": f"KDA gate stage (low-rank projection f_a . F_B, bf16 rounding, decays), N={DN} tokens, H={DH}, "
                    f"K={DK}, rank 128; the projection as exact IEEE float32 FMA chains",
        "modes_us": {m: res["gate"][f"mode{m}_ms"]["mean"] * 1e3 for m in (0, 1, 2)},
        "roofline": {"bound": "alu", "achieved": gate_flops / (res["gate"]["mode0_ms"]["mean"] / 1e3) / 1e12,
                     "peak": PEAK_FP32_TFLOPS, "unit": "TFLOP/s",
                     "frac": gate_flops / (res["gate"]["mode0_ms"]["mean"] / 1e3) / 1e12 / PEAK_FP32_TFLOPS,
                     "flops_per_launch": gate_flops, "note": "mode 0; the fp32 vector peak counts packed FMAs, "
                                                             "which IEEE-ordered scalar chains cannot use"}}
    res_ck = res["chunk_kda"]
    ck_scan_f, ck_prep_f = kda_chunk_flops()
    ck_scan_s, ck_prep_s = res_ck["scan_ms"]["mean"] / 1e3, res_ck["prep_ms"]["mean"] / 1e3
    ck_ms = 1e3 * res_ck["wall_s"] / args.steps
    out["chunk_kda"] = {
        "workload": "chunk form of the delta rule with a log-decay per key channel, B=1 H=16 T=4096 K=V=128 C=64, "
                    "bf16 q/k/v/o, fp32 g [T, H, K] and beta, fp32 final state",
        "value": B * T / (ck_ms / 1e3), "unit": "tokens/s", "ms_per_call": ck_ms,
        "kernels_us": {"prep": ck_prep_s * 1e6, "scan": ck_scan_s * 1e6},
        "roofline": {"bound": "mfma", "kernel": "kda_scan_split_kernel (split-bf16 MFMA)",
                     "achieved": ck_scan_f / ck_scan_s / 1e12, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": ck_scan_f / ck_scan_s / 1e12 / PEAK_BF16_TFLOPS,
                     "traffic": traffic_for("kda_scan_split_kernel"), "flops_per_launch": ck_scan_f,
                     "avg_launch_us": ck_scan_s * 1e6,
                     "note": "128 workgroups of 64 dependent chunk steps; a step is bound by delivering its "
                             "~130 KB of operand fragments per workgroup through the CU's vector memory path"},
        "prep_roofline": {"bound": "alu", "achieved": ck_prep_f / ck_prep_s / 1e12, "peak": PEAK_FP32_TFLOPS,
                          "unit": "TFLOP/s", "frac": ck_prep_f / ck_prep_s / 1e12 / PEAK_FP32_TFLOPS,
                          "traffic": traffic_for("kda_prep_split_kernel"), "flops_per_launch": ck_prep_f}}
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds, res_d.get("_inputs"))
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
