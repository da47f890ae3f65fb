"""Pins of the oracle's MXFP8 decoder (OCP Microscaling: FP8 E4M3 elements, E8M0 scales of 32-element
blocks) and of the input generator's MXFP8 quantiser.  The values pinned are the format's defining
ones: largest normal 448 = 1.75 * 2^8, smallest subnormal 2^-9, the NaN codes 0x7F / 0xFF (no
infinities), scale codes worth 2^(s-127) with 255 NaN."""
import numpy as np
import pytest

import datagen
import oracle

# (code, value): sign, the subnormal grid, the first normal binade, 1.0, the largest finite values
E4M3_TABLE = [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x02, 2.0 ** -8), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
    (0x09, 1.125 * 2.0 ** -6), (0x30, 0.5), (0x38, 1.0), (0x39, 1.125), (0x3F, 1.875), (0x40, 2.0),
    (0x77, 240.0), (0x78, 256.0), (0x7E, 448.0), (0x81, -(2.0 ** -9)), (0xB8, -1.0), (0xC4, -3.0),
    (0xFE, -448.0),
]


@pytest.mark.parametrize("code,value", E4M3_TABLE)
def test_e4m3_defining_values(code, value):
    assert oracle.e4m3_value(np.array([code], np.uint8))[0] == value


def test_e4m3_nan_codes_and_signed_zero():
    v = oracle.e4m3_value(np.arange(256, dtype=np.uint8))
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF]) and int(np.isnan(v).sum()) == 2
    assert v[0x80] == 0.0 and np.signbit(v[0x80])


def test_e4m3_grid():
    """The 126 positive finite codes decode to strictly increasing values, 2^-9 .. 448, and inside
    [2^E, 2^(E+1)) they step by 2^(E-3) (by 2^-9 below 2^-6)."""
    v = oracle.e4m3_value(np.arange(1, 0x7F, dtype=np.uint8))
    assert np.all(np.diff(v) > 0)
    assert v[0] == 2.0 ** -9 and v[-1] == 448.0
    E = np.floor(np.log2(np.maximum(v, 2.0 ** -6)))
    step = np.exp2(E - 3)
    assert np.all(np.diff(v) <= step[1:] + 0.0)
    assert np.all(np.mod(v, step) == 0)
    neg = oracle.e4m3_value(np.arange(0x81, 0xFF, dtype=np.uint8))
    assert np.array_equal(neg, -v)


def test_e8m0_values():
    s = oracle.e8m0_value(np.array([0, 1, 126, 127, 128, 254, 255], np.uint8))
    assert s[0] == 2.0 ** -127 and s[1] == 2.0 ** -126 and s[2] == 0.5 and s[3] == 1.0 and s[4] == 2.0
    assert s[5] == 2.0 ** 127 and np.isnan(s[6])


def test_block_scaling():
    """Element i of a row takes scale i // 32."""
    codes = np.full((2, 128), 0x38, np.uint8)  # 1.0
    codes[1, 5] = 0xC4                          # -3.0
    scales = np.array([[127, 128, 126, 130], [0, 254, 127, 127]], np.uint8)
    x = oracle.mxfp8_decode(codes, scales)
    assert np.array_equal(x[0], np.repeat([1.0, 2.0, 0.5, 8.0], 32))
    assert x[1, 5] == -3.0 * 2.0 ** -127 and x[1, 0] == 2.0 ** -127 and x[1, 40] == 2.0 ** 127
    assert np.all(x[1, 64:] == 1.0)


def test_quantiser_round_trip():
    """Every finite E4M3 value encodes back to its own code, and quantising N(0, 1) rows errs by at
    most half a grid step: |x - y| <= max(|x| 2^-4, 2^(X-10)) with 2^X the block's scale."""
    v = oracle.e4m3_value(np.arange(256, dtype=np.uint8))
    fin = np.isfinite(v)
    assert np.array_equal(datagen._e4m3_encode(v[fin]), np.arange(256, dtype=np.uint8)[fin])
    x = np.random.default_rng(7).standard_normal((64, 128)) * np.exp2(np.random.default_rng(8).integers(-20, 20, (64, 1)))
    codes, scales = datagen.mxfp8_quantize(x)
    y = oracle.mxfp8_decode(codes, scales)
    X = np.repeat(scales.astype(np.float64) - 127, 32, axis=-1)
    assert np.all(np.abs(y - x) <= np.maximum(np.abs(x) * 2.0 ** -4, np.exp2(X - 10)))
    assert np.all(np.abs(x / np.exp2(X)) <= 448.0)  # no block saturates


def test_mxfp8_prefill_inputs_decode_near_bf16():
    d = datagen.mxfp8_prefill_inputs(11, 1, 40, 2, 64, 128, 0.02)
    for name, s in (("q", "qs"), ("k", "ks"), ("v", "vs")):
        x = datagen.to_f64(d[name])
        y = oracle.mxfp8_decode(d[name + "8"], d[s])
        assert y.shape == x.shape and d[s].shape == x.shape[:-1] + (x.shape[-1] // 32,)
        assert np.all(np.abs(y - x) <= np.abs(x).max() * 2.0 ** -4)
