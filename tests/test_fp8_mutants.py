"""Plant plausible mistakes in the FP8 oracle and check that the pins catch
each one."""

import numpy as np
import pytest

import test_fp8_oracle as pins
from oracle import fp8

ORIG_ENC, ORIG_DEC = fp8.e4m3_encode, fp8.e4m3_decode


def enc_ties_away(y):
    y = np.asarray(y, dtype=np.float32)
    c = ORIG_ENC(y)
    # move every exact midpoint to the code farther from zero
    v = ORIG_DEC(c)
    other = ORIG_DEC(np.where(np.abs(v) < np.abs(y), c + 1, c - 1).astype(np.uint8))
    mid = np.abs(np.abs(y) - np.abs(v)) == np.abs(np.abs(y) - np.abs(other))
    return np.where(mid & (np.abs(other) > np.abs(v)), np.where(np.abs(v) < np.abs(y), c + 1, c - 1),
                    c).astype(np.uint8)


def enc_truncate(y):
    y = np.asarray(y, dtype=np.float32)
    c = ORIG_ENC(y)
    over = np.abs(ORIG_DEC(c)) > np.abs(y)
    return np.where(over & ((c & 0x7F) > 0), c - 1, c).astype(np.uint8)


def dec_bias8(c):
    return ORIG_DEC(c) / 2.0


def enc_no_saturation(y):
    y = np.asarray(y, dtype=np.float32)
    return np.where(np.abs(y) >= 464.0, fp8.NAN_CODE, ORIG_ENC(y)).astype(np.uint8)


def dec_subnormal_step(c):
    c = np.asarray(c, dtype=np.uint8)
    v = ORIG_DEC(c)
    return np.where(((c >> 3) & 15) == 0, v * 2.0, v)


def quantize_multiplies(x, scale):
    return ORIG_ENC(np.asarray(x, dtype=np.float32) * np.float32(scale))


MUTANTS = {
    "ties_away": ("e4m3_encode", enc_ties_away),
    "truncate": ("e4m3_encode", enc_truncate),
    "bias8": ("e4m3_decode", dec_bias8),
    "no_saturation": ("e4m3_encode", enc_no_saturation),
    "subnormal_step": ("e4m3_decode", dec_subnormal_step),
    "scale_multiplies": ("quantize", quantize_multiplies),
}

PINS = [pins.test_decode_matches_torch_for_every_code, pins.test_every_finite_code_round_trips,
        pins.test_encode_matches_torch_below_the_overflow_midpoint,
        pins.test_ties_go_to_the_even_code, pins.test_saturation_and_specials,
        pins.test_brute_force_nearest, pins.test_quantize_is_one_fp32_product_then_round,
        pins.test_fp8_cache_write_round_trip]


def failures():
    n = 0
    for pin in PINS:
        try:
            pin()
        except Exception:
            n += 1
    return n


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(monkeypatch, name):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(fp8, attr, fn)
    assert failures() > 0, name


def test_unmutated_oracle_passes():
    assert failures() == 0
