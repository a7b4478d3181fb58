"""Plant plausible mistakes in the INT8 oracle and check that the pins catch
each one."""

import numpy as np
import pytest

import test_int8_oracle as pins
from oracle import int8

ORIG_ENC, ORIG_DEC, ORIG_Q = int8.i8_encode, int8.i8_decode, int8.quantize


def enc_ties_away(y):
    y = np.asarray(y, dtype=np.float32).astype(np.float64)
    a = np.minimum(np.abs(np.nan_to_num(y)), 127.0)
    k = np.floor(a + 0.5).astype(np.int64)
    k = np.where(np.signbit(y), -k, k)
    return (k & 0xFF).astype(np.uint8)


def enc_truncate(y):
    y = np.asarray(y, dtype=np.float32).astype(np.float64)
    k = np.trunc(np.clip(np.nan_to_num(y), -127, 127)).astype(np.int64)
    return (k & 0xFF).astype(np.uint8)


def enc_clamp_128(y):
    y = np.asarray(y, dtype=np.float32).astype(np.float64)
    k = np.clip(np.rint(np.nan_to_num(y)), -128, 127).astype(np.int64)
    return (k & 0xFF).astype(np.uint8)


def enc_nan_max(y):
    y = np.asarray(y, dtype=np.float32)
    return np.where(np.isnan(y), np.uint8(127), ORIG_ENC(y)).astype(np.uint8)


def dec_unsigned(c):
    return np.asarray(c, dtype=np.uint8).astype(np.float64)


def quantize_multiplies(x, scale):
    return ORIG_ENC(np.asarray(x, dtype=np.float32) * np.float32(scale))


MUTANTS = {
    "ties_away": ("i8_encode", enc_ties_away),
    "truncate": ("i8_encode", enc_truncate),
    "clamp_128": ("i8_encode", enc_clamp_128),
    "nan_max": ("i8_encode", enc_nan_max),
    "unsigned_decode": ("i8_decode", dec_unsigned),
    "scale_multiplies": ("quantize", quantize_multiplies),
}

PINS = [pins.test_decode_is_twos_complement, pins.test_every_code_but_minus_128_round_trips,
        pins.test_encode_matches_torch_round_on_every_bf16_pattern,
        pins.test_ties_go_to_the_even_integer, pins.test_saturation_and_specials,
        pins.test_brute_force_nearest, pins.test_quantize_is_one_fp32_product_then_round,
        pins.test_int8_cache_write_round_trip]


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
    monkeypatch.setattr(int8, attr, fn)
    assert failures() > 0, name


def test_unmutated_oracle_passes():
    assert failures() == 0
