"""Pins of the KDA gate stage oracle (vLLM KdaSplit page, method gate_warp).

The float32 arithmetic is checked against exact rational arithmetic (a
correctly rounded result found by brute force over the neighbouring float32
values), the reduction orders against hand-derived values where they round
differently (tests/golden/gate_orders.json), the bf16 rounding against
hand-derived ties, and the decay against its limits and closed forms; planted
mistakes each fail a pin.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import gate as gate_mod
from oracle import kda_gate

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "gate_orders.json")


def _rne32_exact(v: Fraction) -> np.float32:
    """The float32 nearest to the rational v (ties to even), by brute force over
    the neighbours of a candidate."""
    c = np.float32(float(v))
    cands = [c, np.nextafter(c, np.float32(np.inf)), np.nextafter(c, np.float32(-np.inf))]
    best = min(cands, key=lambda r: (abs(Fraction(float(r)) - v), int(np.float32(r).view(np.uint32)) & 1))
    return np.float32(best)


def test_fma32_correctly_rounded_random():
    rng = np.random.default_rng(1)
    n = 3000
    a = rng.standard_normal(n).astype(np.float32)
    b = (rng.standard_normal(n) * np.exp2(rng.integers(-20, 20, n))).astype(np.float32)
    c = (rng.standard_normal(n) * np.exp2(rng.integers(-40, 40, n))).astype(np.float32)
    r = gate_mod.fma32(a, b, c)
    for i in range(n):
        ex = Fraction(float(a[i])) * Fraction(float(b[i])) + Fraction(float(c[i]))
        assert r[i] == _rne32_exact(ex), i


def test_fma32_ties_decided_by_the_low_bits():
    """Cases where the float64 sum is exactly a float32 midpoint but the exact
    result is not (or is): the low part decides."""
    one = np.float32(1.0)
    u = np.float32(2.0 ** -24)  # half a float32 ulp at 1
    tiny = np.float32(2.0 ** -80)
    cases = [
        (u, one, one + np.float32(2.0 ** -23) * 0),          # 1 + 2^-24: tie -> 1 (even)
        (u + np.float32(2.0 ** -47), one, one),               # just above the tie -> 1 + 2^-23
        (u, np.float32(1.0) + np.float32(2.0 ** -23), one),   # product 2^-24 (1 + 2^-23): above the tie
        (tiny, tiny, one),                                    # negligible product
        (np.float32(3.0), np.float32(-1.0), np.float32(3.0)),  # exact zero
    ]
    for a, b, c in cases:
        ex = Fraction(float(a)) * Fraction(float(b)) + Fraction(float(c))
        assert gate_mod.fma32(a, b, c) == _rne32_exact(ex), (a, b, c)
    # where one float64 sum rounded to float32 is wrong (double rounding): a b =
    # -2^-16 (1 - 2^-46), c = 256 + 2^-15; the exact sum 256 + 2^-16 + 2^-62 lies
    # above the float32 midpoint 256 + 2^-16, which is the float64 sum
    a = np.float32(-(2.0 ** -16) * (1 + 2.0 ** -23))
    b = np.float32(1 - 2.0 ** -23)
    c = np.float32(256 + 2.0 ** -15)
    ex = Fraction(float(a)) * Fraction(float(b)) + Fraction(float(c))
    assert ex == 256 + Fraction(1, 2 ** 16) + Fraction(1, 2 ** 62)
    assert np.float32(np.float64(a) * np.float64(b) + np.float64(c)) == np.float32(256.0)  # the wrong answer
    assert gate_mod.fma32(a, b, c) == np.float32(256 + 2.0 ** -15)


def _golden():
    g = json.load(open(GOLDEN))
    f_a = np.zeros((1, 128))
    for c, x in g["f_a"].items():
        f_a[0, int(c)] = x
    f_b = np.zeros((len(g["f_b"]), 128))
    for f, row in enumerate(g["f_b"]):
        for c, x in row.items():
            f_b[f, int(c)] = x
    return g, f_a, f_b


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_reduction_orders_golden(mode):
    g, f_a, f_b = _golden()
    raw_g, ld = kda_gate(f_a, f_b, [0.0], [0.0, 0.0], -1.0, 1, 2, mode)
    np.testing.assert_array_equal(raw_g[0, 0], g["raw_g"][str(mode)])
    # a_log = 0, dt = 0, lower_bound = -1: log-decay = -sigmoid(raw_g)
    np.testing.assert_allclose(ld[0, 0], -1.0 / (1.0 + np.exp(-raw_g[0, 0])), rtol=1e-15)


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_projection_close_to_the_exact_dot_product(mode):
    rng = np.random.default_rng(2 + mode)
    from linear_attention_sequence_recompute_amd.workloads import round_to_bf16
    f_a = round_to_bf16(rng.standard_normal((3, 128)))
    f_b = round_to_bf16(rng.standard_normal((5, 128)) * 0.1)
    raw = gate_mod.projection(f_a, f_b, mode).astype(np.float64)
    exact = f_a @ f_b.T  # float64: 8-bit significands, exact to far below float32
    bound = 128 * 2.0 ** -24 * (np.abs(f_a) @ np.abs(f_b).T)
    assert np.all(np.abs(raw - exact) <= bound)


def test_round_bf16_ties_to_even():
    x = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -23, -(1 + 2 ** -8), 2.0 ** -130], np.float32)
    np.testing.assert_array_equal(gate_mod.round_bf16(x), [1.0, 1 + 2 ** -6, 1 + 2 ** -7, -1.0, 2.0 ** -130])


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_decay_limits_and_closed_forms(mode):
    rng = np.random.default_rng(7)
    H, K = 2, 4
    f_a = np.round(rng.standard_normal((3, 128)) * 8) / 8
    # F_B = 0: raw_g = 0, log-decay = lower_bound * sigmoid(e^{a} dt)
    a_log = np.array([np.log(2.0), -1.0])
    dt = rng.standard_normal(H * K)
    raw_g, ld = kda_gate(f_a, np.zeros((H * K, 128)), a_log, dt, -3.0, H, K, mode)
    assert np.all(raw_g == 0)
    pre = np.exp(a_log)[:, None] * dt.reshape(H, K)
    np.testing.assert_allclose(ld, np.broadcast_to(-3.0 / (1 + np.exp(-pre)), ld.shape), rtol=1e-14)
    # gate -> 0: no decay (log-decay -> 0); gate -> 1: log-decay -> lower_bound
    _, ld0 = kda_gate(f_a, np.zeros((H * K, 128)), [0.0, 0.0], np.full(H * K, -60.0), -3.0, H, K, mode)
    _, ld1 = kda_gate(f_a, np.zeros((H * K, 128)), [0.0, 0.0], np.full(H * K, 60.0), -3.0, H, K, mode)
    assert np.all(np.abs(ld0) < 1e-25) and np.all(np.abs(ld1 + 3.0) < 1e-25)
    # a_log enters through exp: a_log = log 2, raw_g + dt = 1/2 gives pre = 1
    _, ldh = kda_gate(f_a, np.zeros((H * K, 128)), [np.log(2.0)] * H, np.full(H * K, 0.5), -1.0, H, K, mode)
    np.testing.assert_allclose(ldh, -1.0 / (1.0 + np.exp(-1.0)), rtol=1e-14)


def test_head_and_feature_layout():
    """Row h K + f of F_B and entry h K + f of dt_bias belong to head h, feature f;
    a_log[h] to head h."""
    H, K = 3, 2
    f_a = np.zeros((1, 128))
    f_a[0, 5] = 1.0
    f_b = np.zeros((H * K, 128))
    for r in range(H * K):
        f_b[r, 5] = r + 1.0  # raw_g = r + 1 exactly
    raw_g, ld = kda_gate(f_a, f_b, [0.0, np.log(0.5), np.log(0.25)], np.zeros(H * K), -1.0, H, K, 2)
    np.testing.assert_array_equal(raw_g[0], np.arange(1.0, H * K + 1).reshape(H, K))
    pre = np.array([[1, 2], [3 * 0.5, 4 * 0.5], [5 * 0.25, 6 * 0.25]])
    np.testing.assert_allclose(ld[0], -1.0 / (1.0 + np.exp(-pre)), rtol=1e-14)


# --------------------------------------------------------------- planted mistakes

def _run_pins(monkeypatch_fn):
    failures = 0
    for fn in (lambda: [test_reduction_orders_golden(m) for m in (0, 1, 2)],
               lambda: [test_decay_limits_and_closed_forms(m) for m in (0, 1, 2)],
               test_head_and_feature_layout, test_round_bf16_ties_to_even,
               test_fma32_ties_decided_by_the_low_bits):
        try:
            fn()
        except AssertionError:
            failures += 1
    return failures


@pytest.mark.parametrize("mistake", ["no_bf16", "mode2_as_mode0", "a_log_not_exp", "no_dt", "sigmoid_dropped",
                                     "float64_sum", "heads_transposed"])
def test_planted_mistakes_are_caught(monkeypatch, mistake):
    orig_kda, orig_proj, orig_fma = gate_mod.kda_gate, gate_mod.projection, gate_mod.fma32

    def kda_variant(f_a, f_b, a_log, dt_bias, lower_bound, H, K, mode):
        T = np.asarray(f_a).shape[0]
        raw = gate_mod.projection(f_a, f_b, 0 if (mistake == "mode2_as_mode0" and mode == 2) else mode)
        raw_g = raw.astype(np.float64) if mistake == "no_bf16" else gate_mod.round_bf16(raw)
        raw_g = raw_g.reshape(T, H, K)
        if mistake == "heads_transposed":
            raw_g = raw_g.reshape(T, K, H).transpose(0, 2, 1) if H != K else raw_g.transpose(0, 2, 1)
        a = np.asarray(a_log, np.float64).reshape(1, H, 1)
        dt = np.asarray(dt_bias, np.float64).reshape(1, H, K)
        scale = a if mistake == "a_log_not_exp" else np.exp(a)
        pre = scale * (raw_g + (0.0 if mistake == "no_dt" else dt))
        gate = pre if mistake == "sigmoid_dropped" else 1.0 / (1.0 + np.exp(-pre))
        return raw_g, float(lower_bound) * gate

    if mistake == "float64_sum":
        def fma_variant(a, b, c):  # one float64 sum rounded to float32 (double rounding)
            return (np.asarray(a, np.float32).astype(np.float64) * np.asarray(b, np.float32).astype(np.float64)
                    + np.asarray(c, np.float32).astype(np.float64)).astype(np.float32)
        monkeypatch.setattr(gate_mod, "fma32", fma_variant)
    else:
        monkeypatch.setattr(gate_mod, "kda_gate", kda_variant)
        monkeypatch.setattr(__import__(__name__), "kda_gate", kda_variant, raising=False)
        globals()["kda_gate"] = kda_variant
    try:
        assert _run_pins(None) > 0, f"planted mistake {mistake} passed every pin"
    finally:
        globals()["kda_gate"] = orig_kda
        gate_mod.projection, gate_mod.fma32 = orig_proj, orig_fma
