"""Pins of the FP8 row oracle (``oracle.fp8``) against things other than itself
(CPU only):

* a library routine: PyTorch's own float8_e4m3fn casts, for the decoding of all
  256 codes and for the rounding of 200k float32 values in [-448, 448] (ties to
  even included, since exact midpoints are drawn on purpose);
* closed forms: every finite code re-encodes to itself; exact midpoints between
  neighbouring values go to the even mantissa; a row whose largest magnitude is
  448 gets scale 1; a zero row gets scale 0 and zero codes; scaling a row by a
  power of two scales its scale and keeps its codes; the largest element of a
  row is coded +-448;
* the rounding error bound: |dequantized - x| <= scale * max(|x / scale| / 16, 2^-10);
* planted mistakes (the FNUZ exponent bias, rounding half away from zero, no
  clamp before rounding, a wrong amax divisor, a dropped sign of zero) are each
  caught by one of these pins.
"""

import numpy as np
import pytest
import torch

from oracle import fp8


def _torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def _torch_encode(y):
    return torch.from_numpy(np.asarray(y, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _values(seed, n=200_000):
    rng = np.random.default_rng(seed)
    y = rng.standard_normal(n) * 10.0 ** rng.uniform(-4.5, 2.7, n)
    y = np.clip(y, -448, 448).astype(np.float32)
    # exact midpoints between neighbouring finite values, both signs
    vals = np.unique(np.abs(fp8.decode(np.arange(0, 0x7F, dtype=np.uint8))))
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    return np.concatenate([y, mids, -mids, np.float32([0.0, -0.0, 448.0, -448.0])]).astype(np.float32)


def test_decode_matches_library():
    c = np.arange(256, dtype=np.uint8)
    d, t = fp8.decode(c), _torch_decode(c)
    assert np.array_equal(np.isnan(d), np.isnan(t))
    ok = ~np.isnan(t)
    assert np.array_equal(d[ok], t[ok])
    assert np.array_equal(np.signbit(d[ok]), np.signbit(t[ok]))


@pytest.mark.parametrize("seed", [0, 1])
def test_encode_matches_library(seed):
    y = _values(seed)
    assert np.array_equal(fp8.encode(y), _torch_encode(y))


def test_codes_reencode_to_themselves():
    c = np.array([i for i in range(256) if (i & 0x7F) != 0x7F], np.uint8)
    assert np.array_equal(fp8.encode(fp8.decode(c).astype(np.float32)), c)


def test_midpoints_go_to_even_mantissa():
    c = np.arange(0, 0x7E, dtype=np.uint8)            # c and c + 1 are neighbours
    mid = ((fp8.decode(c) + fp8.decode(c + 1)) / 2).astype(np.float32)
    got = fp8.encode(mid)
    even = np.where(c % 2 == 0, c, c + 1).astype(np.uint8)
    assert np.array_equal(got, even)


def test_quantize_closed_forms():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((6, 512)).astype(np.float32)
    x[0] *= np.float32(440.0 / np.abs(x[0]).max())   # all below 448 ...
    x[0, 7] = -448.0                                   # ... but one: amax exactly 448 -> scale 1
    x[1] = 0.0
    x[2] = -0.0
    codes, scale = fp8.quantize_rows(x)
    assert scale[0] == np.float32(1.0)
    assert np.array_equal(codes[0], fp8.encode(x[0]))
    assert scale[1] == 0 and scale[2] == 0 and not codes[1:3].any()
    # a power-of-two factor moves the scale and keeps the codes
    c2, s2 = fp8.quantize_rows(x[3:] * np.float32(2.0 ** -9))
    assert np.array_equal(c2, codes[3:])
    assert np.array_equal(s2, scale[3:] * np.float32(2.0 ** -9))
    # the largest magnitude of each row is coded +-448
    for r in range(3, 6):
        j = int(np.argmax(np.abs(x[r])))
        assert codes[r, j] & 0x7F == 0x7E


@pytest.mark.parametrize("dtype", [np.float16, np.float32])
def test_quantize_error_bound(dtype):
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((64, 512)) * 10.0 ** rng.uniform(-3, 3, (64, 1))).astype(dtype)
    codes, scale = fp8.quantize_rows(x)
    back = fp8.dequantize_rows(codes, scale)
    xf = x.astype(np.float64)
    y = np.abs(xf) / scale.astype(np.float64)[:, None]
    bound = scale.astype(np.float64)[:, None] * np.maximum(y / 16.0, 2.0 ** -10) * (1 + 1e-6)
    assert np.all(np.abs(back - xf) <= bound)


# --------------------------------------------------------------------------- planted mistakes

def _pins():
    return [test_decode_matches_library, lambda: test_encode_matches_library(0),
            test_codes_reencode_to_themselves, test_midpoints_go_to_even_mantissa,
            test_quantize_closed_forms, lambda: test_quantize_error_bound(np.float32)]


def _some_pin_fails():
    for pin in _pins():
        try:
            pin()
        except (AssertionError, ValueError):
            return True
    return False


def _fnuz_bias(monkeypatch):
    orig = fp8.decode
    monkeypatch.setattr(fp8, "decode", lambda c: orig(c) / 2.0)


def _half_away(monkeypatch):
    monkeypatch.setattr(fp8, "_round_half_even", lambda a: np.floor(np.abs(a) + 0.5) * np.sign(a))


def _no_clamp(monkeypatch):
    monkeypatch.setattr(fp8, "_clamp", lambda y: y)


def _wrong_divisor(monkeypatch):
    monkeypatch.setattr(fp8, "E4M3_MAX", 240.0)


def _unsigned_zero(monkeypatch):
    monkeypatch.setattr(fp8, "_sign_bit", lambda y: np.asarray(y) < 0)


@pytest.mark.parametrize("plant", [_fnuz_bias, _half_away, _no_clamp, _wrong_divisor, _unsigned_zero],
                         ids=lambda f: f.__name__.strip("_"))
def test_planted_mistake_is_caught(plant, monkeypatch):
    assert not _some_pin_fails()
    plant(monkeypatch)
    assert _some_pin_fails()
