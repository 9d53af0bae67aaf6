"""Pins of the fp8 group-quantisation oracle (WarpDrive page, kernel 1).

The E4M3 encoding is checked against torch's float8_e4m3fn conversion (a library
routine implementing the same format and rounding) and against examples derived
by hand from the format; the group quantisation against invariants that follow
from its definition. Planted mistakes each fail at least one pin.
"""

import numpy as np
import pytest
import torch

from oracle import e4m3_decode, e4m3_encode, fp8_quant
from oracle import fp8 as fp8mod


def torch_e4m3(y):
    return torch.from_numpy(np.asarray(y, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _sweep():
    rng = np.random.default_rng(0)
    finite = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    vals = e4m3_decode(finite).astype(np.float32)                      # every code's value
    mids = ((vals[:-1].astype(np.float64) + vals[1:]) / 2).astype(np.float32)  # ties (exact in fp32)
    mags = np.exp2(rng.uniform(-12, np.log2(448.0), 20000)).astype(np.float32)
    rand = np.concatenate([mags, -mags])
    y = np.concatenate([vals, mids, rand, np.float32([0.0, -0.0, 448.0, -448.0, 2.0 ** -9, 2.0 ** -10])])
    return np.clip(y, -448, 448).astype(np.float32)


def check_encoder(enc):
    y = _sweep()
    np.testing.assert_array_equal(enc(y), torch_e4m3(y))
    # hand-derived from the format (sign, 4-bit exponent with bias 7, 3-bit mantissa)
    hand = {1.0: 0x38, 448.0: 0x7E, -448.0: 0xFE, 2.0 ** -9: 0x01, 2.0 ** -6: 0x08, 0.0: 0x00,
            1.0625: 0x38,   # halfway between 1 (m=0) and 1.125 (m=1): to the even mantissa 0
            1.1875: 0x3A,   # halfway between 1.125 (m=1) and 1.25 (m=2): to 2
            -3.0: 0xC4, 0.5: 0x30, 240.0: 0x77, 2.0 ** -10: 0x00, 3 * 2.0 ** -10: 0x02}
    for x, code in hand.items():
        assert int(enc(np.float32([x]))[0]) == code, (x, hex(code))


def test_e4m3_encode_matches_library_and_hand_examples():
    check_encoder(e4m3_encode)


def test_e4m3_round_trip():
    finite = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    np.testing.assert_array_equal(e4m3_encode(e4m3_decode(finite).astype(np.float32)), finite)


def check_quant(fn):
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((6, 512)) * np.exp2(rng.integers(-8, 8, (6, 1)))).astype(np.float32)
    x[2, 128:256] = 0.0              # an all-zero group
    x[3, 0:128] *= 1e-6              # a tiny group (subnormal-range quotients do not occur: it scales)
    for group in (64, 128):
        codes, scales = fn(x, group)
        xg = x.reshape(6, -1, group)
        cg = codes.reshape(6, -1, group)
        absmax = np.abs(xg).max(-1)
        np.testing.assert_array_equal(scales, (absmax / np.float32(448.0)).astype(np.float32))
        for r in range(6):
            for gi in range(xg.shape[1]):
                if absmax[r, gi] == 0:
                    assert np.all(cg[r, gi] == 0) and scales[r, gi] == 0
                    continue
                i = int(np.argmax(np.abs(xg[r, gi])))
                assert cg[r, gi, i] == (0xFE if xg[r, gi, i] < 0 else 0x7E)   # the max element is +-448
                deq = e4m3_decode(cg[r, gi]) * float(scales[r, gi])
                err = np.abs(deq - xg[r, gi])
                # half a unit in the last place of E4M3: 2^-4 of the value, 2^-10 x scale near zero
                bound = np.maximum(np.abs(xg[r, gi]) * 2.0 ** -4, 2.0 ** -10 * float(scales[r, gi])) * (1 + 1e-6)
                assert np.all(err <= bound)
        # groups are independent
        x2 = x.copy()
        x2[0, :group] *= 3.0
        c2, s2 = fn(x2, group)
        np.testing.assert_array_equal(c2[:, group:], codes[:, group:])
        np.testing.assert_array_equal(s2[0, 1:], scales[0, 1:])


def test_fp8_quant_invariants():
    check_quant(fp8_quant)


# ------------------------------------------------------------ planted mistakes

def _encode_half_up(y):
    a = np.abs(np.asarray(y, np.float32)).astype(np.float64)
    out = []
    for v, s in zip(a.ravel(), np.signbit(np.asarray(y, np.float32)).ravel()):
        if v < 2.0 ** -6:
            c = int(np.floor(v * 2 ** 9 + 0.5))
        else:
            e = int(np.floor(np.log2(v)))
            m = int(np.floor((v / 2.0 ** e - 1) * 8 + 0.5))
            if m == 8:
                m, e = 0, e + 1
            c = ((e + 7) << 3) | m
        out.append(c | (0x80 if s else 0))
    return np.array(out, np.uint8).reshape(np.shape(y))


def _encode_bias8(y):
    c = e4m3_encode(y).astype(np.int64)
    ef = (c >> 3) & 0xF
    return ((c & 0x87) | (np.minimum(ef + 1, 15) << 3)).astype(np.uint8)


@pytest.mark.parametrize("enc", [_encode_half_up, _encode_bias8])
def test_encoder_pins_catch_mistakes(enc):
    with pytest.raises(AssertionError):
        check_encoder(enc)


def _quant_mutant(mutation):
    def fn(x, group):
        xg = np.asarray(x, np.float32).reshape(*x.shape[:-1], -1, group)
        absmax = np.abs(xg).max(-1)
        div = np.float32(240.0 if mutation == "fnuz_max" else 448.0)
        scale = (absmax / div).astype(np.float32)
        with np.errstate(divide="ignore", invalid="ignore"):
            y = np.where(scale[..., None] > 0, xg / scale[..., None], 0).astype(np.float32)
        if mutation == "global_scale":
            gmax = np.abs(xg).max()
            scale = np.full_like(scale, gmax / np.float32(448.0))
            y = (xg / scale[..., None]).astype(np.float32)
        y = np.clip(y, -448, 448).astype(np.float32)
        return fp8mod.e4m3_encode(y).reshape(x.shape), scale
    return fn


@pytest.mark.parametrize("mutation", ["fnuz_max", "global_scale"])
def test_quant_pins_catch_mistakes(mutation):
    with pytest.raises(AssertionError):
        check_quant(_quant_mutant(mutation))
