"""Pins of the FP8 (OCP E4M3) oracle: the format's definition, PyTorch's own
float8_e4m3fn cast where it is defined (a library special case), exhaustive
round trips, ties and saturation."""

import numpy as np
import pytest
import torch

from oracle import fp8


def torch_codes(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_matches_torch_for_every_code():
    c = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(c).view(torch.float8_e4m3fn).double().numpy()
    got = fp8.e4m3_decode(c)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])


def test_every_finite_code_round_trips():
    c = np.array([x for x in range(256) if x not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(fp8.e4m3_encode(fp8.e4m3_decode(c).astype(np.float32)), c)


def test_encode_matches_torch_below_the_overflow_midpoint():
    # every bf16 bit pattern whose value is finite and below 464 in magnitude
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    x = bits.view(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) < 464.0)]
    assert np.array_equal(fp8.e4m3_encode(x), torch_codes(x))
    rng = np.random.default_rng(0)
    y = (rng.standard_normal(200000) * np.exp2(rng.integers(-12, 9, 200000))).astype(np.float32)
    y = y[np.abs(y) < 464.0]
    assert np.array_equal(fp8.e4m3_encode(y), torch_codes(y))


def test_ties_go_to_the_even_code():
    v = fp8.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    mids = ((v[:-1] + v[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (v[:-1] + v[1:]) / 2)   # exact midpoints
    codes = fp8.e4m3_encode(mids).astype(int)
    lo = np.arange(0, 0x7E)
    assert np.array_equal(codes, np.where(lo % 2 == 0, lo, lo + 1))


def test_saturation_and_specials():
    enc = fp8.e4m3_encode
    assert enc([448.0, 463.9, 464.0, 1e30, np.inf]).tolist() == [0x7E] * 5
    assert enc([-448.0, -1e30, -np.inf]).tolist() == [0xFE] * 3
    assert enc([np.nan])[0] == fp8.NAN_CODE
    assert enc([0.0, -0.0]).tolist() == [0x00, 0x80]
    assert enc([2.0 ** -10, 2.0 ** -10 * 1.0001]).tolist() == [0x00, 0x01]   # half the least subnormal


def test_brute_force_nearest():
    v = fp8.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    rng = np.random.default_rng(1)
    x = rng.uniform(0, 460, 5000).astype(np.float32)
    for xi, c in zip(x, fp8.e4m3_encode(x)):
        d = np.abs(v - float(xi))
        best = np.flatnonzero(d == d.min())
        assert c in best and (len(best) == 1 or c % 2 == 0)


def test_quantize_is_one_fp32_product_then_round():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(10000).astype(np.float32)
    for scale in (1.0, 0.037, 3.5, 1 / 448):
        inv = np.float32(1.0 / scale)
        assert np.array_equal(fp8.quantize(x, scale), fp8.e4m3_encode(x * inv))
    # error of the round trip: at most half a code step, relative 2^-4
    y = fp8.dequantize(fp8.quantize(x, 0.05), 0.05)
    inside = np.abs(x) / 0.05 >= 2.0 ** -6
    assert np.all(np.abs(y - x)[inside] <= 2.0 ** -4 * np.abs(x)[inside] * (1 + 1e-6))


def test_fp8_cache_write_round_trip():
    rng = np.random.default_rng(3)
    T, H_kv, D, N, BS = 5, 2, 16, 6, 4
    k = rng.standard_normal((T, H_kv, D)).astype(np.float32)
    v = rng.standard_normal((T, H_kv, D)).astype(np.float32)
    kc = np.full((N, H_kv, BS, D), 0x7F, np.uint8)
    vc = kc.copy()
    slots = np.array([0, 7, -1, 22, 13])
    k2, v2 = fp8.reshape_and_cache_fp8(k, v, kc, vc, slots, 0.02, 0.03)
    for i, s in enumerate(slots):
        if s < 0:
            continue
        assert np.array_equal(k2[s // BS, :, s % BS], fp8.quantize(k[i], 0.02))
        assert np.array_equal(v2[s // BS, :, s % BS], fp8.quantize(v[i], 0.03))
    written = {(s // BS, s % BS) for s in slots if s >= 0}
    for b in range(N):
        for o in range(BS):
            if (b, o) not in written:
                assert np.all(k2[b, :, o] == 0x7F) and np.all(v2[b, :, o] == 0x7F)
