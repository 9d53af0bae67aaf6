#!/usr/bin/env python3
"""Throughput of the gated delta rule on one MI355X.

A step is one chunked forward pass (gdn_chunk_fwd: the prep kernel for
recompute_w_u, then chunk_fwd_h fused with chunk_fwd_o, which at this shape runs
in the chunk-parallel form: summary kernel, then scan kernel) over
one batch of B=1, H=16, T=4096, K=V=128 bf16 inputs, already resident in device
memory. The decode step (gdn_recurrent_step, N=256 requests,
H=32, K=V=128, a 512-slot float32 state pool) is timed beside it in the same run
and reported under "decode".

Prints one JSON line on stdout (everything else goes to stderr). The K timed
steps are plain calls. Per-kernel durations come from K further calls of
gdn_chunk_fwd_profiled, which records HIP events on the library's stream around
each launch (recording them inside the timed steps would add about 10 us per
call); the roofline of the dominant part, chunk_fwd_h + chunk_fwd_o (the span of
the summary and scan kernels), is its algorithmic FLOPs per call over that
duration.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
       python bench.py --only chunk|decode|kda|verify|fp8|layer|chunk_kda|copy --steps K   (profiling runs)
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


def chunk_flops():
    """Algorithmic FLOPs per launch (dense per-chunk tiles, as the WarpDrive page
    lists the products). Returns (h + o, full forward)."""
    n_ch = B * H * (T // C)
    h = 2 * C * K * V + 2 * C * K * V            # w h, k^T v_gated
    o = 2 * C * K * V + 2 * C * C * K + 2 * C * C * V  # q h, q k^T, P v_new
    prep = 2 * C * C * K + C ** 3 // 3 + 2 * C * C * V + 2 * C * C * K  # k k^T, solve, u, w
    return n_ch * (h + o), n_ch * (h + o + prep)


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


def bench_chunk(torch, api, hev, steps, warmup, flush_bytes=512 << 20):
    from linear_attention_sequence_recompute_amd.workloads import chunk_inputs

    ci = chunk_inputs([T] * B, H, K, V, dtype="bf16", seed=2)
    dev = torch.device("cuda")

    def t(x, dt):
        return torch.from_numpy(x).to(dt).to(dev).view(B, T, *x.shape[1:])

    q, k, v = (t(x, torch.bfloat16) for x in (ci.q, ci.k, ci.v))
    g, b = t(ci.a, torch.float32), t(ci.beta, torch.float32)
    o = torch.empty(B, T, H, V, dtype=torch.bfloat16, device=dev)
    ht = torch.empty(B, H, V, K, dtype=torch.float32, device=dev)
    ws = torch.empty(api.workspace_bytes(B, B * T, H, K, V), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    scale = K ** -0.5

    def step(evs=None):
        api.chunk_fwd(q, k, v, g, b, scale=scale, out=o, ht=ht, workspace=ws, stream=stream, events=evs)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    # the timed steps: plain calls (events between the two kernels cost about
    # 10 us per call, so per-kernel durations come from the next loop)
    t0 = time.perf_counter()
    for i in range(steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # per-kernel durations: as many calls again, with HIP events the library
    # records on the launch stream before prep, between the kernels and after scan
    evs = [hev.create(3) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    prep = [hev.ms(e[0], e[1]) for e in evs]
    scan = [hev.ms(e[1], e[2]) for e in evs]
    whole = [hev.ms(e[0], e[2]) for e in evs]

    # the same with L2 and the 256 MiB infinity cache flushed before every step
    flush = torch.empty(flush_bytes, dtype=torch.uint8, device=dev)
    cold_prep, cold_scan = [], []
    for i in range(steps):
        flush.fill_(i & 0xFF)
        step(evs[i])
        torch.cuda.synchronize()
        cold_prep.append(hev.ms(evs[i][0], evs[i][1]))
        cold_scan.append(hev.ms(evs[i][1], evs[i][2]))
    for e in evs:
        hev.destroy(e)
    del flush
    return dict(wall_s=wall, prep_ms=stats(prep), scan_ms=stats(scan), call_ms=stats(whole),
                cold_prep_ms=stats(cold_prep), cold_scan_ms=stats(cold_scan))


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
    return dict(wall_s=wall, kernel_ms=stats(ms), n_active=int((di.slots > 0).sum()))


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
    return dict(prologue_ms=stats(ms_p), rmsnorm_ms=stats(ms_r))


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


def cpu_baseline(min_seconds=10.0):
    """The fp64 oracle (chunked WY form) on the host cores, over repeated passes
    of the same B=1, H=16, T=4096 workload until min_seconds have elapsed."""
    import numpy as np  # noqa: F401

    import oracle
    from linear_attention_sequence_recompute_amd.workloads import chunk_inputs

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    ci = chunk_inputs([T], H, K, V, dtype="bf16", seed=2)
    n_tok = 0
    t0 = time.perf_counter()
    passes = 0
    while True:
        oracle.chunked_fwd(ci.q, ci.k, ci.v, ci.a, ci.beta, scale=K ** -0.5)
        n_tok += T
        passes += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    dt = time.perf_counter() - t0
    return dict(value=n_tok / dt, unit="tokens/s", cores=int(threads), kind="oracle",
                sample=f"{passes} full passes of the B=1 H=16 T=4096 K=V=128 workload through the fp64 chunked "
                       f"oracle (numpy, {threads} BLAS threads) in {dt:.1f} s")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", choices=["all", "chunk", "decode", "kda", "verify", "fp8", "layer", "chunk_kda", "copy"], default="all")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the chunked forward and the decode step need no "
              f"communication, and this build runs on a single MI355X (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE={world}).", file=sys.stderr)
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
    res_c = res_d = None
    if args.only in ("all", "chunk"):
        log("chunk: B=1 H=16 T=4096 K=V=128 bf16 ...")
        res_c = bench_chunk(torch, api, hev, args.steps, args.warmup)
        log(json.dumps(res_c))
    if args.only in ("all", "decode"):
        log("decode: N=256 H=32 K=V=128 pool=512 ...")
        res_d = bench_decode(torch, api, hev, args.steps, args.warmup)
        log(json.dumps(res_d))
    res_k = None
    if args.only in ("all", "kda"):
        log("decode with per-key-channel decay: N=256 H=32 K=V=128 pool=512 ...")
        res_k = bench_decode_kda(torch, api, hev, args.steps, args.warmup)
        log(json.dumps(res_k))
    res_v = None
    if args.only in ("all", "verify"):
        log(f"verify decode: N={VN} T={VT} H=32 K=V=128 pool=512 ...")
        res_v = bench_verify(torch, api, hev, args.steps, args.warmup)
        log(json.dumps(res_v))
    res_q = None
    if args.only in ("all", "fp8"):
        log(f"fp8 quant: [{QR}, {QC}] float32, groups of {QG} ...")
        res_q = bench_fp8(torch, api, hev, args.steps, args.warmup)
        log(json.dumps(res_q))
    res_l = None
    if args.only in ("all", "layer"):
        log(f"decode layer front/back: N={DN} H={DH} D={DK} conv pool={DSLOTS} ...")
        res_l = bench_layer(torch, api, hev, args.steps, args.warmup)
        log(json.dumps(res_l))
    res_ck = None
    if args.only in ("all", "chunk_kda"):
        log("chunk form with per-channel decays: B=1 H=16 T=4096 K=V=128 bf16 ...")
        res_ck = bench_chunk_kda(torch, api, hev, args.steps, args.warmup)
        log(json.dumps(res_ck))
    if args.only != "all":
        return

    flops_ho, flops_full = chunk_flops()
    tokens = B * T
    ms_per_step = 1e3 * res_c["wall_s"] / args.steps
    scan_s = res_c["scan_ms"]["mean"] / 1e3
    achieved = flops_ho / scan_s / 1e12
    dec_s = res_d["kernel_ms"]["mean"] / 1e3
    dec_b = decode_bytes(res_d["n_active"])
    dec_gbs = dec_b / dec_s / 1e9
    out = {
        "metric": "GDN fwd tokens/s + % bf16 MFMA peak (H16,K=V=128,T4096); decode GB/s % peak",
        "value": tokens / (ms_per_step / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "chunked GatedDeltaNet forward, B=1 H=16 T=4096 K=V=128 C=64, bf16 q/k/v, "
                               "fp32 beta/g, o bf16 + final state fp32",
                   "global_batch": B, "seq_len": T, "heads": H, "head_dim": K, "chunk": C,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma",
                     "kernel": "chunk_fwd_h fused with chunk_fwd_o: summary_kernel + scan_kernel "
                               "(chunk-parallel form, 4 segments of 16 chunks)",
                     "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": traffic_for("summary_kernel", "scan_kernel"),
                     "flops_per_launch": flops_ho, "avg_launch_us": scan_s * 1e6},
        "kernels_us": {"prep": res_c["prep_ms"]["mean"] * 1e3, "h_o": res_c["scan_ms"]["mean"] * 1e3,
                       "call": res_c["call_ms"]["mean"] * 1e3,
                       "cold_prep": res_c["cold_prep_ms"]["mean"] * 1e3,
                       "cold_h_o": res_c["cold_scan_ms"]["mean"] * 1e3},
        "full_fwd_tflops": flops_full / (ms_per_step / 1e3) / 1e12,
        "decode": {"workload": "recurrent decode step, N=256 requests (all active), H=32, K=V=128, "
                               "pool [512, 32, 128, 128] fp32, bf16 q/k/v/o",
                   "value": dec_gbs, "unit": "GB/s", "avg_launch_us": dec_s * 1e6,
                   "roofline": {"bound": "hbm", "achieved": dec_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                "frac": dec_gbs / PEAK_HBM_GBS, "traffic": traffic_for("recurrent_step_kernel"),
                                "bytes_per_launch": dec_b}},
    }
    kda_s = res_k["kernel_ms"]["mean"] / 1e3
    kda_b = decode_bytes(res_k["n_active"]) + res_k["n_active"] * DH * (DK - 1) * 4  # g per key channel
    out["decode_kda"] = {
        "workload": "recurrent decode step with a log-decay per key channel, N=256 requests (all active), H=32, "
                    "K=V=128, pool [512, 32, 128, 128] fp32, bf16 q/k/v/o",
        "value": kda_b / kda_s / 1e9, "unit": "GB/s", "avg_launch_us": kda_s * 1e6,
        "roofline": {"bound": "hbm", "achieved": kda_b / kda_s / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": kda_b / kda_s / 1e9 / PEAK_HBM_GBS, "traffic": traffic_for("recurrent_step_kernel_kda"),
                     "bytes_per_launch": kda_b}}
    ver_s = res_v["kernel_ms"]["mean"] / 1e3
    ver_b = verify_bytes(res_v["n_active"], VT)
    out["decode_verify"] = {
        "workload": f"speculative-verify decode, {VN} requests x {VT} tokens, H=32, K=V=128, pool [512, 32, 128, 128] "
                    "fp32 (source read once, a state written per token), bf16 q/k/v/o",
        "value": ver_b / ver_s / 1e9, "unit": "GB/s", "avg_launch_us": ver_s * 1e6,
        "tokens_per_s": VN * VT / ver_s,
        "roofline": {"bound": "hbm", "achieved": ver_b / ver_s / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": ver_b / ver_s / 1e9 / PEAK_HBM_GBS, "traffic": traffic_for("recurrent_verify_kernel"),
                     "bytes_per_launch": ver_b}}
    q_s = res_q["kernel_ms"]["mean"] / 1e3
    q_b = QR * QC * (4 + 1) + QR * (QC // QG) * 4
    out["fp8_quant"] = {
        "workload": f"fp8 group quantisation, [{QR}, {QC}] float32 activations, groups of {QG}, E4M3 codes + "
                    "float32 scales",
        "value": q_b / q_s / 1e9, "unit": "GB/s", "avg_launch_us": q_s * 1e6,
        "roofline": {"bound": "hbm", "achieved": q_b / q_s / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": q_b / q_s / 1e9 / PEAK_HBM_GBS, "traffic": traffic_for("fp8_quant_kernel"),
                     "bytes_per_launch": q_b}}
    lp_b, lr_b = layer_bytes()
    lp_s, lr_s = res_l["prologue_ms"]["mean"] / 1e3, res_l["rmsnorm_ms"]["mean"] / 1e3
    out["decode_layer"] = {
        "workload": f"decode layer front (4-tap conv over a bf16 conv-state pool of {DSLOTS} slots, SiLU, q/k L2 "
                    f"norm, sigmoid beta) and back (gated RMSNorm, bf16 out), N={DN} requests, H={DH}, D={DK}",
        "prologue": {"avg_launch_us": lp_s * 1e6, "bytes_per_launch": lp_b,
                     "roofline": {"bound": "hbm", "achieved": lp_b / lp_s / 1e9, "peak": PEAK_HBM_GBS,
                                  "unit": "GB/s", "frac": lp_b / lp_s / 1e9 / PEAK_HBM_GBS,
                                  "traffic": traffic_for("decode_prologue_kernel")}},
        "gated_rmsnorm": {"avg_launch_us": lr_s * 1e6, "bytes_per_launch": lr_b,
                          "roofline": {"bound": "hbm", "achieved": lr_b / lr_s / 1e9, "peak": PEAK_HBM_GBS,
                                       "unit": "GB/s", "frac": lr_b / lr_s / 1e9 / PEAK_HBM_GBS,
                                       "traffic": traffic_for("gated_rmsnorm_kernel")}}}
    ck_scan_f, ck_prep_f = kda_chunk_flops()
    ck_scan_s, ck_prep_s = res_ck["scan_ms"]["mean"] / 1e3, res_ck["prep_ms"]["mean"] / 1e3
    ck_ms = 1e3 * res_ck["wall_s"] / args.steps
    out["chunk_kda"] = {
        "workload": "chunk form of the delta rule with a log-decay per key channel, B=1 H=16 T=4096 K=V=128 C=64, "
                    "bf16 q/k/v/o, fp32 g [T, H, K] and beta, fp32 final state",
        "value": B * T / (ck_ms / 1e3), "unit": "tokens/s", "ms_per_call": ck_ms,
        "kernels_us": {"prep": ck_prep_s * 1e6, "scan": ck_scan_s * 1e6},
        "roofline": {"bound": "mfma", "kernel": "kda_scan_kernel (fp32 MFMA)", "achieved": ck_scan_f / ck_scan_s / 1e12,
                     "peak": PEAK_FP32_TFLOPS, "unit": "TFLOP/s",
                     "frac": ck_scan_f / ck_scan_s / 1e12 / PEAK_FP32_TFLOPS,
                     "traffic": traffic_for("kda_scan_kernel"), "flops_per_launch": ck_scan_f,
                     "avg_launch_us": ck_scan_s * 1e6},
        "prep_roofline": {"bound": "alu", "achieved": ck_prep_f / ck_prep_s / 1e12, "peak": PEAK_FP32_TFLOPS,
                          "unit": "TFLOP/s", "frac": ck_prep_f / ck_prep_s / 1e12 / PEAK_FP32_TFLOPS,
                          "traffic": traffic_for("kda_prep_kernel"), "flops_per_launch": ck_prep_f}}
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
