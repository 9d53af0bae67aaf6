"""Host logic of bench.py (no GPU): the algorithmic FLOP and byte counts the
roofline figures divide by, the traffic record's digest check, the JSON entry
of a chunk workload, and the refusal of more than one GPU."""

import json
import os
import subprocess
import sys

import pytest

import bench


def test_chunk_flops_of_the_timed_shape():
    """B=1 H=16 T=4096 K=V=128: 64 chunks x 16 heads, each 4nKV (h) + 2nKV +
    2n^2 K + 2n^2 V (o) at n = 64, i.e. 8,388,608 FLOPs per (chunk, head)."""
    ho, full = bench.chunk_flops([4096], 16, 128, 128)
    assert ho == 64 * 16 * 8_388_608 == 8_589_934_592
    prep = 2 * 64 * 64 * 128 + 64 ** 3 // 3 + 2 * 64 * 64 * 128 + 2 * 64 * 64 * 128
    assert full == ho + 64 * 16 * prep


def test_chunk_flops_ragged_and_packed():
    """A ragged last chunk counts its own n; packed sequences add up; an empty
    sequence counts nothing."""
    one = bench.chunk_flops([50], 1, 64, 32)[0]
    assert one == 4 * 50 * 64 * 32 + 2 * 50 * 64 * 32 + 2 * 50 * 50 * 64 + 2 * 50 * 50 * 32
    assert bench.chunk_flops([64, 50, 0], 1, 64, 32)[0] == bench.chunk_flops([64], 1, 64, 32)[0] + one


def test_decode_and_verify_bytes():
    """Per active (request, head): the state page read and written (verify: read
    once, written per token), q, k, v, o in bf16, g and beta in float32."""
    page = 128 * 128 * 4
    per_token_io = (2 * 128 + 128) * 2 + 2 * 4 + 128 * 2
    assert bench.decode_bytes(256) == 256 * 32 * (2 * page + per_token_io) == 1_082_195_968
    assert bench.verify_bytes(96, 4) == 96 * 32 * (5 * page + 4 * per_token_io)


def test_traffic_is_reported_only_for_the_profiled_sources(tmp_path, monkeypatch):
    rec = {"source_digest": bench.source_digest(),
           "kernels": {"a": {"bytes_per_launch": 100}, "b": {"bytes_per_launch": 23}, "c": {"bytes_per_launch": None}}}
    f = tmp_path / "t.json"
    f.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.traffic_for("a", "b") == 123
    assert bench.traffic_for("a", "missing") is None and bench.traffic_for("c") is None
    rec["source_digest"] = "0" * 16
    f.write_text(json.dumps(rec))
    assert bench.traffic_for("a") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "absent.json"))
    assert bench.traffic_for("a") is None


def test_chunk_entry():
    """tokens/s from the wall time of the timed steps; the roofline from the
    warm h + o events against the dtype's peak."""
    t = {k: {"mean": v} for k, v in (("prep_us", 20.0), ("h_o_us", 50.0), ("call_us", 70.0))}
    res = {"label": "x", "lengths": [4096], "H": 16, "K": 128, "V": 128, "dtype": "torch.bfloat16",
           "warm": t, "cold": {**t, "call_us": {"mean": 100.0}, "h_o_us": {"mean": 60.0}}, "wall_s": 20 * 68e-6}
    e = bench.chunk_entry(res, 20, {"mfma_bf16_tflops": 2000.0})
    assert e["ms_per_step"] == pytest.approx(0.068)
    assert e["value"] == pytest.approx(4096 / 68e-6)
    assert e["value_cold"] == pytest.approx(4096 / 100e-6)
    r = e["roofline"]
    assert r["achieved"] == pytest.approx(8_589_934_592 / 50e-6 / 1e12)
    assert r["frac"] == pytest.approx(r["achieved"] / 2500.0) and r["peak"] == 2500.0
    assert r["frac_of_measured_peak"] == pytest.approx(r["achieved"] / 2000.0)
    e32 = bench.chunk_entry({**res, "dtype": "torch.float32"}, 20, None)
    assert e32["roofline"]["peak"] == bench.PEAK_FP32_TFLOPS


def test_more_than_one_gpu_is_refused():
    """--gpus N > 1 exits with status 2 and says why, before touching any GPU."""
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
