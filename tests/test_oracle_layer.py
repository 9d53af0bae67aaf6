"""Pins of the decode layer's front and back operations (KdaSplit kernel body).

The convolution is checked against numpy's convolve over a token sequence (a
library routine), the state shift against the inputs it must hold, the norms
against closed forms; planted mistakes each fail a pin.
"""

import numpy as np
import pytest

from oracle import conv_silu_step, decode_prologue, gated_rmsnorm
from oracle import layer as layer_mod


def _silu(y):
    return y / (1.0 + np.exp(-y))


def check_conv(fn):
    rng = np.random.default_rng(0)
    H, D, T = 2, 4, 9
    C = 3 * H * D
    w = rng.standard_normal((3, 4, H * D))
    bias = rng.standard_normal(C)
    xs = rng.standard_normal((T, C))
    st = np.zeros((3, C, 3))
    ys = []
    for t in range(T):
        y, st = fn(xs[t:t + 1], w, bias, st, np.array([2]))
        ys.append(y[0])
    ys = np.array(ys)
    wc = np.concatenate([w[s].T for s in range(3)], axis=0)  # [C, 4], tap 3 multiplies the newest input
    for c in range(C):
        ref = np.convolve(xs[:, c], wc[c, ::-1])[:T] + bias[c]  # causal, zero history
        np.testing.assert_allclose(ys[:, c], _silu(ref), rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(st[2], xs[-3:].T)   # the slot holds the last three inputs, oldest first
    np.testing.assert_array_equal(st[1], 0.0)         # other slots untouched
    # padding row: zero output, state untouched
    y, st2 = fn(xs[:1], w, bias, st, np.array([0]))
    assert np.all(y == 0) and np.array_equal(st2, st)


def test_conv_matches_numpy_convolve():
    check_conv(conv_silu_step)


def check_prologue(fn):
    rng = np.random.default_rng(1)
    H, D, N = 3, 8, 5
    C = 3 * H * D
    x = rng.standard_normal((N, C)) * 3
    w = rng.standard_normal((3, 4, H * D))
    st = rng.standard_normal((7, C, 3))
    slots = np.array([1, 0, 3, 6, -1])
    q, k, v, beta, _ = fn(x, w, None, st, slots, rng.standard_normal((N, H)), H, D)
    for b in (0, 2, 3):
        nq, nk = np.sum(q[b] ** 2, -1), np.sum(k[b] ** 2, -1)   # per head
        assert np.all(np.abs(nq - 1) < 1e-3) and np.all(np.abs(nk - 1) < 1e-3)
        assert np.all((beta[b] > 0) & (beta[b] < 1))
    for b in (1, 4):
        assert np.all(q[b] == 0) and np.all(k[b] == 0) and np.all(v[b] == 0) and np.all(beta[b] == 0)
    # identity convolution (only the newest tap, weight 1): v = silu(x) exactly; beta = 1/2 at raw 0
    wid = np.zeros((3, 4, H * D))
    wid[:, 3, :] = 1.0
    q2, _, v2, b2, _ = fn(x, wid, None, st, slots, np.zeros((N, H)), H, D)
    np.testing.assert_allclose(v2[0].ravel(), _silu(x[0, 2 * H * D:]), rtol=1e-14)
    assert np.all(b2[[0, 2, 3]] == 0.5)
    # a tiny q head: the 1e-6 under the root sets its norm, sum / (sum + 1e-6)
    xs = x.copy()
    xs[0, :D] = 1e-4
    q3, _, _, _, _ = fn(xs, wid, None, st, slots, np.zeros((N, H)), H, D)
    y = _silu(1e-4)
    np.testing.assert_allclose(np.sum(q3[0, 0] ** 2), D * y * y / (D * y * y + 1e-6), rtol=1e-9)


def test_prologue_norms():
    check_prologue(decode_prologue)


def _prologue_mutant(mutation):
    def fn(x, w, bias, conv_state, slots, beta_raw, H, D):
        y, st = conv_silu_step(x, w, bias, conv_state, slots)
        N = y.shape[0]
        q = y[:, :H * D].reshape(N, H, D)
        k = y[:, H * D:2 * H * D].reshape(N, H, D)
        v = y[:, 2 * H * D:].reshape(N, H, D)
        if mutation == "norm_over_all_heads":
            q = q / np.sqrt(np.sum(q * q, axis=(1, 2), keepdims=True) + 1e-6)
            k = k / np.sqrt(np.sum(k * k, axis=(1, 2), keepdims=True) + 1e-6)
        else:  # eps_outside_root
            q = q / (np.sqrt(np.sum(q * q, axis=-1, keepdims=True)) + 1e-6)
            k = k / (np.sqrt(np.sum(k * k, axis=-1, keepdims=True)) + 1e-6)
        beta = 1.0 / (1.0 + np.exp(-np.asarray(beta_raw, np.float64)))
        beta[np.asarray(slots) <= 0] = 0.0
        return q, k, v, beta, st
    return fn


@pytest.mark.parametrize("mutation", ["norm_over_all_heads", "eps_outside_root"])
def test_prologue_pins_catch_mistakes(mutation):
    with pytest.raises(AssertionError):
        check_prologue(_prologue_mutant(mutation))


def check_rmsnorm(fn):
    rng = np.random.default_rng(2)
    o = rng.standard_normal((4, 2, 16))
    out = fn(o, np.full((4, 32), 40.0), np.ones(16), 1e-6)   # sigmoid(40) = 1 - 4e-18
    np.testing.assert_allclose(np.sqrt(np.mean(out ** 2, -1)), 1.0, rtol=1e-5)
    c = np.full((1, 1, 16), 3.0)                               # constant vector: 3 / sqrt(9 + eps)
    w = rng.uniform(0.5, 2, 16)
    g = rng.standard_normal((1, 16))
    ref = 3.0 / np.sqrt(9.0 + 1e-2) * w / (1 + np.exp(-g[0]))
    np.testing.assert_allclose(fn(c, g, w, 1e-2)[0, 0], ref, rtol=1e-12)


def test_gated_rmsnorm_closed_forms():
    check_rmsnorm(gated_rmsnorm)


def _conv_mutant(mutation):
    def fn(x, w, bias, conv_state, slots):
        st = np.asarray(conv_state, np.float64).copy()
        N, C = x.shape
        wc = np.concatenate([np.asarray(w)[s].T for s in range(3)], axis=0)
        if mutation == "taps_reversed":
            wc = wc[:, ::-1]
        y = np.zeros((N, C))
        for b in range(N):
            slot = int(slots[b])
            if slot <= 0:
                continue
            window = np.concatenate([st[slot], x[b][:, None]], axis=1)
            acc = np.sum(window * wc, axis=1) + (bias if bias is not None else 0)
            y[b] = _silu(acc)
            st[slot] = window[:, :3] if mutation == "shift_keeps_oldest" else window[:, 1:]
        return y, st
    return fn


@pytest.mark.parametrize("mutation", ["taps_reversed", "shift_keeps_oldest"])
def test_conv_pins_catch_mistakes(mutation):
    check_conv(_conv_mutant(None))
    with pytest.raises(AssertionError):
        check_conv(_conv_mutant(mutation))


def test_rmsnorm_pins_catch_missing_eps_and_gate():
    with pytest.raises(AssertionError):
        check_rmsnorm(lambda o, g, w, eps: layer_mod.gated_rmsnorm(o, g, w, 0.0))
    with pytest.raises(AssertionError):
        check_rmsnorm(lambda o, g, w, eps: layer_mod.gated_rmsnorm(o, np.full_like(np.asarray(g, float), 40.0), w,
                                                                   eps))


# ------------------------------------------------ multi-token (verify) conv front

from oracle import decode_prologue_verify  # noqa: E402
from oracle import layer as _layer  # noqa: E402


def test_verify_front_one_token_is_the_decode_front():
    rng = np.random.default_rng(5)
    H, D, N, P = 2, 4, 5, 7
    C = 3 * H * D
    x = rng.standard_normal((N, C))
    w = rng.standard_normal((3, 4, H * D))
    bias = rng.standard_normal(C)
    st = rng.standard_normal((P, C, 3))
    slots = np.array([3, 0, 5, 1, 6])
    braw = rng.standard_normal((N, H))
    ref = decode_prologue(x, w, bias, st, slots, braw, H, D)
    got = decode_prologue_verify(x, w, bias, st, slots[:, None], np.ones(N, int), braw, H, D, 1)
    for a, b in zip(got, ref):
        np.testing.assert_allclose(a, b, rtol=1e-14, atol=1e-14)


def _spec_stream(fn, seed=11):
    """Calls of T = 4 drafts with random accepted counts on one conv slot: every
    call's outputs equal the causal convolution (numpy's convolve) over the
    stream of accepted inputs followed by the call's drafts; the page after a call
    is (column a, column a + 1, drafts)."""
    rng = np.random.default_rng(seed)
    H, D, T, P = 1, 2, 4, 3
    C = 3 * H * D
    w = rng.standard_normal((3, 4, H * D))
    wc = np.concatenate([w[s].T for s in range(3)], axis=0)
    hist = rng.standard_normal((3, C))  # the accepted stream so far (oldest first)
    st = np.zeros((P, C, T + 2))
    st[2, :, :3] = hist.T
    stream = list(hist)
    acc = 1
    for call in range(6):
        x = rng.standard_normal((T, C))
        slots = np.array([[2, 1, 2, 1]])
        q, k, v, beta, st2 = fn(x, w, None, st, slots, np.array([acc]), np.zeros((T, H)), H, D, T)
        y = np.concatenate([q, k, v], axis=0)  # normalised: compare v (raw SiLU) and q, k directions
        seq = np.array(stream + list(x))  # accepted stream, then the drafts
        for c in range(C):
            ref = np.convolve(seq[:, c], wc[c, ::-1])[:len(seq)]
            conv = ref[len(stream):]
            silu = conv / (1 + np.exp(-conv))
            if c >= 2 * H * D:  # v section: raw
                np.testing.assert_allclose(v[:, 0, c - 2 * H * D], silu, rtol=1e-12, atol=1e-12)
        np.testing.assert_array_equal(st2[2][:, :2], st[2][:, acc:acc + 2])
        np.testing.assert_array_equal(st2[2][:, 2:], x.T)
        np.testing.assert_array_equal(st2[1], st[1])
        m = int(rng.integers(1, T + 1))  # drafts accepted
        stream += list(x[:m])
        acc, st = m, st2


def test_verify_front_follows_the_accepted_stream():
    _spec_stream(decode_prologue_verify)


def test_verify_front_padding():
    rng = np.random.default_rng(6)
    H, D, T, P = 1, 2, 3, 4
    C = 3 * H * D
    st = rng.standard_normal((P, C, T + 2))
    x = rng.standard_normal((4 * T, C))
    slots = np.array([[1, 2, 3], [0, 2, 3], [2, 0, 3], [3, 1, 2]])
    accepted = np.array([0, 1, 2, 4])  # 0 and T + 1 out of range; row 1's conv slot 0; row 2's source slot 0
    q, k, v, beta, st2 = decode_prologue_verify(x, rng.standard_normal((3, 4, H * D)), None, st, slots, accepted,
                                                np.ones((4 * T, H)), H, D, T)
    assert np.all(q == 0) and np.all(v == 0) and np.all(beta == 0)
    np.testing.assert_array_equal(st2, st)


@pytest.mark.parametrize("mutation", ["taps_from_a", "rewrite_keeps_a_minus_1", "conv_slot_from_source"])
def test_verify_front_pins_catch_mistakes(mutation):
    def mutant(x, w, bias, conv_state, slots, accepted, beta_raw, H, D, T):
        x = np.asarray(x, np.float64)
        st = np.asarray(conv_state, np.float64).copy()
        N, C = x.shape[0] // T, st.shape[1]
        wc = np.concatenate([np.asarray(w, np.float64)[s].T for s in range(3)], axis=0)
        y = np.zeros((N * T, C))
        for b in range(N):
            a = int(accepted[b])
            cs = int(slots[b, a - 1]) if mutation == "conv_slot_from_source" else int(slots[b, 0])
            page = st[cs]
            o = a if mutation == "taps_from_a" else a - 1
            seq = np.concatenate([page[:, o:o + 3], x[b * T:(b + 1) * T].T], axis=1)
            for t in range(T):
                z = np.sum(seq[:, t:t + 4] * wc, axis=1)
                y[b * T + t] = z * _layer._sig(z)
            r = a - 1 if mutation == "rewrite_keeps_a_minus_1" else a
            st[cs] = np.concatenate([page[:, r:r + 2], x[b * T:(b + 1) * T].T], axis=1)
        q, k, v = _layer._sections(y, H, D)
        return q, k, v, np.zeros((N * T, H)), st
    with pytest.raises(AssertionError):
        _spec_stream(mutant)
